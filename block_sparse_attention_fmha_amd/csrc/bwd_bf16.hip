// bf16 attention backward for gfx950: dQ, dK, dV recomputed from the saved LSE.
//
// The fuzz tester of "Enable 2CTA for SM100 block-sparse backward" drives the backward
// with (q, k, v, out, dout, lse) and separate transposed block-sparse lists; its
// relative-bias backward passes the gradient through unchanged. "Optimize Flash Dynamic
// Mask Attention Kernel Configurations" keeps a seq-k-parallel backward with a
// deterministic grid. Math (per (b, h)):
//   P = exp(S - LSE), dV = P^T dO, dP = dO V^T, D_i = sum_d dO_id O_id,
//   dS = P (dP - D) [x (1 - tanh^2) under softcap], dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels, no atomics (every gradient element has one writer and a fixed
// summation order, so results are bitwise reproducible):
//   1. preprocess: D = rowsum(dO * O) with DPP row reductions;
//   2. dK/dV pass: a workgroup owns 128 keys (32 per wave, K and V of those keys held in
//      VGPRs as MFMA B operands) and walks 64-query tiles of Q / dO staged in LDS;
//      S = Q K^T and dP = dO V^T come out with ONE KEY PER LANE and 8 consecutive queries
//      per register group, which is exactly the B operand of dV^T += dO^T P and
//      dK^T += Q^T dS; dO^T / Q^T operands come from transposed LDS reads;
//   3. dQ pass: a workgroup owns 128 queries (Q and dO fragments in VGPRs) and walks
//      64-key tiles of K / V in LDS, mirroring the forward: S^T = K Q^T, dP^T = V dO^T,
//      dQ^T += K^T dS^T with K^T from transposed LDS reads.
// The dQ pass recomputes S and dP (7 matrix products instead of 5): that is the price
// of determinism without atomics.
//
// LDS tiles are row-major with the XOR chunk swizzle of SwizzledTile so that the same
// tile serves 16-byte MFMA row reads and transposed reads without bank conflicts.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kThreads = 256;
constexpr int kBQ = 64;      // queries per dK/dV step
constexpr int kBK = 128;     // keys per dK/dV workgroup
constexpr int kQM = 128;     // queries per dQ workgroup
constexpr int kKN = 64;      // keys per dQ step

// ------------------------------------------------------------------------------- preprocess
template <int DV>
__global__ __launch_bounds__(kThreads)
void bwd_preprocess_kernel(const BwdParams bp) {
  constexpr int LPK = DV / 8;
  constexpr int ROWS = kThreads / LPK;
  const AttnParams& p = bp.a;
  const int64_t r = (int64_t)blockIdx.x * ROWS + threadIdx.x / LPK;
  const int dl = threadIdx.x % LPK;
  const int64_t total = (int64_t)p.B * p.H * p.Nq;
  const bool in = r < total;
  float x = 0.0f;
  int b = 0, h = 0, i = 0;
  if (in) {
    i = (int)(r % p.Nq);
    const int64_t bh = r / p.Nq;
    h = (int)(bh % p.H);
    b = (int)(bh / p.H);
    const __bf16* Og = (const __bf16*)p.o + b * p.os_b + h * p.os_h + (int64_t)i * p.os_s + 8 * dl;
    const __bf16* Dg = (const __bf16*)bp.dout + b * bp.dos_b + h * bp.dos_h + (int64_t)i * bp.dos_s + 8 * dl;
    float of[8], df[8];
    bf16x8_to_f32(*(const u32x4*)Og, of);
    bf16x8_to_f32(*(const u32x4*)Dg, df);
#pragma unroll
    for (int e = 0; e < 8; ++e) x = __builtin_fmaf(of[e], df[e], x);
  }
  x = group_sum<LPK>(x);
  if (in && dl == 0) bp.dsum[r] = x;
}

// Log2-domain probability of the recomputed score, its softcap derivative factor, and
// the mask. `raw` is <q, k>; lse2 = LSE * log2(e) (+inf for empty / out-of-range rows).
template <bool SOFTCAP, bool BIAS>
__device__ __forceinline__ float recompute_p(float raw, const AttnParams& p, int i, int j, float lse2,
                                             float& dcap) {
  if constexpr (SOFTCAP || BIAS) {
    float x = raw * p.scale;
    dcap = 1.0f;
    if constexpr (SOFTCAP) {
      const float e = fast_exp2(x * (2.0f * kLog2e / p.softcap));
      const float th = 1.0f - 2.0f * fast_rcp(e + 1.0f);
      x = p.softcap * th;
      dcap = 1.0f - th * th;
    }
    float u = x * kLog2e;
    if constexpr (BIAS) u += p.bias_log2 * (float)abs(i - j);
    return fast_exp2(u - lse2);
  } else {
    dcap = 1.0f;
    return fast_exp2(__builtin_fmaf(raw, p.scale_log2, -lse2));
  }
}

// ------------------------------------------------------------------------------- dK / dV
template <int DQK, int DV>
struct DkdvSmem {
  static constexpr int QB = kBQ * DQK * 2;
  static constexpr int OB = kBQ * DV * 2;
  static constexpr int STAGE = QB + OB + 2 * kBQ * 4;   // Q, dO, lse2, D
  static constexpr int BYTES = 2 * STAGE;
};

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dkdv_kernel(const BwdParams bp) {
  using SM = DkdvSmem<DQK, DV>;
  using TQ = SwizzledTile<DQK>;
  using TO = SwizzledTile<DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, bp.grid_padded_kv);
  if (bid >= bp.total_work_kv) return;
  const int bh = bid / bp.n_kv_tiles;
  const int kt = bid - bh * bp.n_kv_tiles;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int k0 = kt * kBK;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
  const int Nq = p.Nq, Nk = p.Nk, delta = Nk - Nq;
  const int kw = k0 + 32 * w;
  const int key = kw + lq;

  const __bf16* Qg = (const __bf16*)p.q + b * p.qs_b + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + h * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + h * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + b * bp.dos_b + h * bp.dos_h;
  const float* LSEg = p.lse + ((int64_t)b * p.H + h) * Nq;
  const float* Dg = bp.dsum + ((int64_t)b * p.H + h) * Nq;

  // ---- query-step sequence
  const int mk = p.mask.kind;
  int count, s_lo = 0, sub = 1, npart = 0, ncols = 0;
  const int* pidx = nullptr;
  const int* fidx = nullptr;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nq;
    if (mk == kMaskCausal || mk == kMaskWindow) lo = max(0, k0 - delta);
    if (mk == kMaskPrefix) lo = (k0 < p.mask.prefix) ? 0 : max(0, k0 - delta);
    if (mk == kMaskWindow) hi = min(Nq, k0 + kBK - 1 - delta + p.mask.window + 1);
    lo = min(lo, Nq);
    s_lo = lo / kBQ;
    count = max(0, (hi + kBQ - 1) / kBQ - s_lo);
  } else {
    const int ks = k0 / p.lists.tile_rows;
    const int hm = (p.lists.heads == 1) ? 0 : h;
    const int row = (b * p.lists.heads + hm) * p.lists.n_rows + ks;
    ncols = p.lists.n_cols;
    npart = clamp_count(p.lists.pcnt[row], ncols);
    const int nfull = clamp_count(p.lists.fcnt[row], ncols);
    pidx = p.lists.pidx + (int64_t)row * ncols;
    fidx = p.lists.fidx + (int64_t)row * ncols;
    sub = p.lists.tile_cols / kBQ;
    count = (npart + nfull) * sub;
  }
  auto step_at = [&](int it, int& i0, bool& partial) {
    if constexpr (!LISTS) {
      i0 = (s_lo + it) * kBQ;
      partial = false;
    } else {
      const int e = it / sub, s = it - e * sub;
      int qt;
      if (e < npart) { qt = list_entry(pidx, e, ncols); partial = true; }
      else { qt = list_entry(fidx, e - npart, ncols); partial = false; }
      i0 = qt * sub * kBQ + s * kBQ;
    }
  };

  // ---- K and V of this lane's key as B operands (k-slot = head dim)
  bf16x8 kf[DQK / 16], vf[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    kf[ks] = (key < Nk) ? *(const bf16x8*)(Kg + (int64_t)key * p.ks_s + 16 * ks + 8 * g) : bf16x8{};
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    vf[ks] = (key < Nk) ? *(const bf16x8*)(Vg + (int64_t)key * p.vs_s + 16 * ks + 8 * g) : bf16x8{};

  // ---- staging of one Q / dO tile (+ lse2, D)
  constexpr int QCH = kBQ * DQK / 8 / kThreads;
  constexpr int OCH = kBQ * DV / 8 / kThreads;
  u32x4 qreg[QCH], oreg[OCH];
  float lreg = 0.0f, dreg = 0.0f;
  auto load_step = [&](int i0) {
#pragma unroll
    for (int c2 = 0; c2 < QCH; ++c2) {
      const int c = tid + kThreads * c2;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      const int i = i0 + row;
      qreg[c2] = (i < Nq) ? *(const u32x4*)(Qg + (int64_t)i * p.qs_s + col * 8) : u32x4{};
    }
#pragma unroll
    for (int c2 = 0; c2 < OCH; ++c2) {
      const int c = tid + kThreads * c2;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      const int i = i0 + row;
      oreg[c2] = (i < Nq) ? *(const u32x4*)(DOg + (int64_t)i * bp.dos_s + col * 8) : u32x4{};
    }
    if (tid < kBQ) {
      const int i = i0 + tid;
      const float ls = (i < Nq) ? LSEg[i] : kNegInf;
      lreg = (ls == kNegInf) ? __builtin_huge_valf() : ls * kLog2e;
      dreg = (i < Nq) ? Dg[i] : 0.0f;
    }
  };
  auto store_step = [&](int buf) {
    char* Ql = smem + buf * SM::STAGE;
    char* Ol = Ql + SM::QB;
    float* Ll = (float*)(Ol + SM::OB);
#pragma unroll
    for (int c2 = 0; c2 < QCH; ++c2) {
      const int c = tid + kThreads * c2;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      *(u32x4*)(Ql + TQ::off(row, col * 8)) = qreg[c2];
    }
#pragma unroll
    for (int c2 = 0; c2 < OCH; ++c2) {
      const int c = tid + kThreads * c2;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      *(u32x4*)(Ol + TO::off(row, col * 8)) = oreg[c2];
    }
    if (tid < kBQ) {
      Ll[tid] = lreg;
      Ll[kBQ + tid] = dreg;
    }
  };

  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) dv[i] = f32x16{};
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  if (count > 0) {
    int i0;
    bool part;
    step_at(0, i0, part);
    load_step(i0);
    store_step(0);
    __syncthreads();
  }

  for (int it = 0; it < count; ++it) {
    const int buf = it & 1;
    int i0;
    bool partial;
    step_at(it, i0, partial);
    if (it + 1 < count) {
      int i1;
      bool p1;
      step_at(it + 1, i1, p1);
      load_step(i1);
    }
    const char* Ql = smem + buf * SM::STAGE;
    const char* Ol = Ql + SM::QB;
    const float* Ll = (const float*)(Ol + SM::OB);

    bool need;
    if constexpr (LISTS) {
      need = partial;
    } else {
      const int kl = kw + 31;
      need = false;
      if (mk == kMaskCausal) need = kl > i0 + delta;
      else if (mk == kMaskWindow) need = (kl > i0 + delta) || (kw < i0 + kBQ - 1 + delta - p.mask.window);
      else if (mk == kMaskPrefix) need = (kl >= p.mask.prefix) && (kl > i0 + delta);
      else if (mk == kMaskBlockDiag) need = true;
    }

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      // S = Q K^T: rows = queries (permuted), columns = this lane's key
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Ql + TQ::off(32 * sb + prow, 16 * ks + 8 * g));
        s = mfma_bf16(a, kf[ks], s);
      }
      f32x16 dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Ol + TO::off(32 * sb + prow, 16 * ks + 8 * g));
        dp = mfma_bf16(a, vf[ks], dp);
      }
      // reg r <-> query i0 + 32 sb + 16 (r/8) + 8 g + r % 8
      bf16x8 pb[2], dsb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qi = 32 * sb + 16 * hh + 8 * g;
        const f32x4 la = *(const f32x4*)(Ll + qi), lb = *(const f32x4*)(Ll + qi + 4);
        const f32x4 da = *(const f32x4*)(Ll + kBQ + qi), db4 = *(const f32x4*)(Ll + kBQ + qi + 4);
        u32x4 pk, dk4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv[2], dsv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int r = 8 * hh + 2 * e + z;
            const int ee = 2 * e + z;
            const float lse2 = ee < 4 ? la[ee] : lb[ee - 4];
            const float dd = ee < 4 ? da[ee] : db4[ee - 4];
            const int qidx = i0 + qi + ee;
            float dcap;
            float pr = recompute_p<SOFTCAP, BIAS>(s[r], p, qidx, key, lse2, dcap);
            if (need && qidx < Nq && !mask_visible(p.mask, b, qidx, key, Nq, Nk)) pr = 0.0f;
            pv[z] = pr;
            dsv[z] = pr * (dp[r] - dd) * dcap;
          }
          pk[e] = pack_bf16x2(pv[0], pv[1]);
          dk4[e] = pack_bf16x2(dsv[0], dsv[1]);
        }
        pb[hh] = __builtin_bit_cast(bf16x8, pk);
        dsb[hh] = __builtin_bit_cast(bf16x8, dk4);
      }
      // dV^T += dO^T P, dK^T += Q^T dS (transposed reads of the row-major tiles)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int r0 = 32 * sb + 16 * hh + trow;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db) {
          const u32x2 lo = lds_read_tr(Ol + TO::off(r0, 32 * db + tcol));
          const u32x2 hi = lds_read_tr(Ol + TO::off(r0 + 4, 32 * db + tcol));
          dv[db] = mfma_bf16(join_bf16x8(lo, hi), pb[hh], dv[db]);
        }
#pragma unroll
        for (int db = 0; db < DQK / 32; ++db) {
          const u32x2 lo = lds_read_tr(Ql + TQ::off(r0, 32 * db + tcol));
          const u32x2 hi = lds_read_tr(Ql + TQ::off(r0 + 4, 32 * db + tcol));
          dk[db] = mfma_bf16(join_bf16x8(lo, hi), dsb[hh], dk[db]);
        }
      }
    }

    if (it + 1 < count) store_step(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane = key, reg r <-> d = 32 db + 8 (r/4) + 4 g + r % 4
  if (key < Nk) {
    __bf16* dKg = (__bf16*)bp.dk + b * bp.dks_b + h * bp.dks_h + (int64_t)key * bp.dks_s;
    __bf16* dVg = (__bf16*)bp.dv + b * bp.dvs_b + h * bp.dvs_h + (int64_t)key * bp.dvs_s;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(dk[db][4 * jj] * p.scale, dk[db][4 * jj + 1] * p.scale);
        v[1] = pack_bf16x2(dk[db][4 * jj + 2] * p.scale, dk[db][4 * jj + 3] * p.scale);
        *(u32x2*)(dKg + 32 * db + 8 * jj + 4 * g) = v;
      }
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(dv[db][4 * jj], dv[db][4 * jj + 1]);
        v[1] = pack_bf16x2(dv[db][4 * jj + 2], dv[db][4 * jj + 3]);
        *(u32x2*)(dVg + 32 * db + 8 * jj + 4 * g) = v;
      }
  }
}

// ------------------------------------------------------------------------------- dQ
template <int DQK, int DV>
struct DqSmem {
  static constexpr int KB = kKN * DQK * 2;
  static constexpr int VB = kKN * DV * 2;
  static constexpr int STAGE = KB + VB;
  static constexpr int BYTES = 2 * STAGE;
};

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dq_kernel(const BwdParams bp) {
  using SM = DqSmem<DQK, DV>;
  using TK = SwizzledTile<DQK>;
  using TV = SwizzledTile<DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid >= p.total_work) return;
  const int bh = bid / p.n_tiles;
  const int t = bid - bh * p.n_tiles;
  const int qt = p.longest_first ? (p.n_tiles - 1 - t) : t;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0 = qt * kQM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
  const int Nq = p.Nq, Nk = p.Nk, delta = Nk - Nq;
  const int qw = q0 + 32 * w;
  const int qrow = qw + lq;

  const __bf16* Qg = (const __bf16*)p.q + b * p.qs_b + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + h * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + h * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + b * bp.dos_b + h * bp.dos_h;

  // ---- key-tile sequence (same bands / lists as the forward)
  const int mk = p.mask.kind;
  int count, t_lo = 0, sub = 1, npart = 0, ncols = 0;
  const int* pidx = nullptr;
  const int* fidx = nullptr;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nk;
    if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kQM + delta);
    if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kQM + delta));
    if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
    hi = max(hi, 0);
    t_lo = lo / kKN;
    count = max(0, (hi + kKN - 1) / kKN - t_lo);
  } else {
    const int qs = q0 / p.lists.tile_rows;
    const int hm = (p.lists.heads == 1) ? 0 : h;
    const int row = (b * p.lists.heads + hm) * p.lists.n_rows + qs;
    ncols = p.lists.n_cols;
    npart = clamp_count(p.lists.pcnt[row], ncols);
    const int nfull = clamp_count(p.lists.fcnt[row], ncols);
    pidx = p.lists.pidx + (int64_t)row * ncols;
    fidx = p.lists.fidx + (int64_t)row * ncols;
    sub = p.lists.tile_cols / kKN;
    count = (npart + nfull) * sub;
  }
  auto tile_at = [&](int it, int& n0, bool& partial) {
    if constexpr (!LISTS) {
      n0 = (t_lo + it) * kKN;
      partial = false;
    } else {
      const int e = it / sub, s = it - e * sub;
      int kt2;
      if (e < npart) { kt2 = list_entry(pidx, e, ncols); partial = true; }
      else { kt2 = list_entry(fidx, e - npart, ncols); partial = false; }
      n0 = kt2 * sub * kKN + s * kKN;
    }
  };

  // ---- Q and dO rows of this lane's query as B operands
  bf16x8 qf[DQK / 16], of[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    qf[ks] = (qrow < Nq) ? *(const bf16x8*)(Qg + (int64_t)qrow * p.qs_s + 16 * ks + 8 * g) : bf16x8{};
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    of[ks] = (qrow < Nq) ? *(const bf16x8*)(DOg + (int64_t)qrow * bp.dos_s + 16 * ks + 8 * g) : bf16x8{};
  float lse2 = __builtin_huge_valf(), ddv = 0.0f;
  if (qrow < Nq) {
    const float ls = p.lse[((int64_t)b * p.H + h) * Nq + qrow];
    lse2 = (ls == kNegInf) ? __builtin_huge_valf() : ls * kLog2e;
    ddv = bp.dsum[((int64_t)b * p.H + h) * Nq + qrow];
  }

  constexpr int KCH = kKN * DQK / 8 / kThreads;
  constexpr int VCH = kKN * DV / 8 / kThreads;
  u32x4 kreg[KCH], vreg[VCH];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      const int kk = n0 + row;
      kreg[i] = (kk < Nk) ? *(const u32x4*)(Kg + (int64_t)kk * p.ks_s + col * 8) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      const int kk = n0 + row;
      vreg[i] = (kk < Nk) ? *(const u32x4*)(Vg + (int64_t)kk * p.vs_s + col * 8) : u32x4{};
    }
  };
  auto store_tile = [&](int buf) {
    char* Kl = smem + buf * SM::STAGE;
    char* Vl = Kl + SM::KB;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      *(u32x4*)(Kl + TK::off(row, col * 8)) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      *(u32x4*)(Vl + TV::off(row, col * 8)) = vreg[i];
    }
  };

  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  if (count > 0) {
    int n0;
    bool part;
    tile_at(0, n0, part);
    load_tile(n0);
    store_tile(0);
    __syncthreads();
  }

  for (int it = 0; it < count; ++it) {
    const int buf = it & 1;
    int n0;
    bool partial;
    tile_at(it, n0, partial);
    if (it + 1 < count) {
      int n1;
      bool p1;
      tile_at(it + 1, n1, p1);
      load_tile(n1);
    }
    const char* Kl = smem + buf * SM::STAGE;
    const char* Vl = Kl + SM::KB;

    bool need = (n0 + kKN > Nk);
    if constexpr (LISTS) {
      need = need || partial;
    } else {
      const int last = n0 + kKN - 1;
      if (mk == kMaskCausal) need = need || (last > qw + delta);
      else if (mk == kMaskWindow) need = need || (last > qw + delta) || (n0 < qw + 31 + delta - p.mask.window);
      else if (mk == kMaskPrefix) need = need || (last > qw + delta && last >= p.mask.prefix);
      else if (mk == kMaskBlockDiag) need = true;
    }

    bf16x8 dsb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Kl + TK::off(32 * kb + prow, 16 * ks + 8 * g));
        s = mfma_bf16(a, qf[ks], s);
      }
#pragma unroll
      for (int ks = 0; ks < DV / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(Vl + TV::off(32 * kb + prow, 16 * ks + 8 * g));
        dp = mfma_bf16(a, of[ks], dp);
      }
      // reg r <-> key n0 + 32 kb + 16 (r/8) + 8 g + r % 8, query qrow
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float dsv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int r = 8 * hh + 2 * e + z;
            const int kk = n0 + 32 * kb + 16 * hh + 8 * g + 2 * e + z;
            float dcap;
            float pr = recompute_p<SOFTCAP, BIAS>(s[r], p, qrow, kk, lse2, dcap);
            if (need) {
              bool vis = kk < Nk;
              if (vis && qrow < Nq && (LISTS ? partial : true)) vis = mask_visible(p.mask, b, qrow, kk, Nq, Nk);
              if (!vis) pr = 0.0f;
            }
            dsv[z] = pr * (dp[r] - ddv) * dcap;
          }
          pk[e] = pack_bf16x2(dsv[0], dsv[1]);
        }
        dsb[kb][hh] = __builtin_bit_cast(bf16x8, pk);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int r0 = 32 * kb + 16 * hh + trow;
          const u32x2 lo = lds_read_tr(Kl + TK::off(r0, 32 * db + tcol));
          const u32x2 hi = lds_read_tr(Kl + TK::off(r0 + 4, 32 * db + tcol));
          dq[db] = mfma_bf16(join_bf16x8(lo, hi), dsb[kb][hh], dq[db]);
        }

    if (it + 1 < count) store_tile(buf ^ 1);
    __syncthreads();
  }

  if (qrow < Nq) {
    __bf16* dQg = (__bf16*)bp.dq + b * bp.dqs_b + h * bp.dqs_h + (int64_t)qrow * bp.dqs_s;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(dq[db][4 * jj] * p.scale, dq[db][4 * jj + 1] * p.scale);
        v[1] = pack_bf16x2(dq[db][4 * jj + 2] * p.scale, dq[db][4 * jj + 3] * p.scale);
        *(u32x2*)(dQg + 32 * db + 8 * jj + 4 * g) = v;
      }
  }
}

hipError_t record_stage(const BwdParams& bp, int i, hipStream_t st) {
  if (bp.stage_events == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(bp.stage_events[i]), st);
}

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
hipError_t launch_passes(const BwdParams& bp, const ListParams& tlists, hipStream_t st) {
  {
    hipError_t e0 = record_stage(bp, 1, st);
    if (e0 != hipSuccess) return e0;
    BwdParams kv = bp;
    kv.a.lists = tlists;
    auto kern = bwd_dkdv_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
    constexpr int smem_bytes = DkdvSmem<DQK, DV>::BYTES;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem_bytes);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(bp.grid_padded_kv), dim3(kThreads), smem_bytes, st, kv);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    auto kern = bwd_dq_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
    constexpr int smem_bytes = DqSmem<DQK, DV>::BYTES;
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, smem_bytes);
    if (e != hipSuccess) return e;
    e = record_stage(bp, 2, st);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, dim3(bp.a.grid_padded), dim3(kThreads), smem_bytes, st, bp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return record_stage(bp, 3, st);
  }
}

template <int DQK, int DV>
hipError_t dispatch(const BwdParams& bp, const ListParams& tl, bool lists, bool softcap, bool bias, hipStream_t st) {
  if (lists) {
    if (softcap) return bias ? launch_passes<DQK, DV, true, true, true>(bp, tl, st) : launch_passes<DQK, DV, true, true, false>(bp, tl, st);
    return bias ? launch_passes<DQK, DV, true, false, true>(bp, tl, st) : launch_passes<DQK, DV, true, false, false>(bp, tl, st);
  }
  if (softcap) return bias ? launch_passes<DQK, DV, false, true, true>(bp, tl, st) : launch_passes<DQK, DV, false, true, false>(bp, tl, st);
  return bias ? launch_passes<DQK, DV, false, false, true>(bp, tl, st) : launch_passes<DQK, DV, false, false, false>(bp, tl, st);
}

}  // namespace

int bwd_q_block_rows() { return kQM; }
int bwd_kv_block_rows() { return kBK; }

// bp.a.lists holds the forward lists (per query tile, walked by the dQ pass) and
// bp.tlists the transposed lists (per key tile, walked by the dK/dV pass).
hipError_t launch_bwd_bf16(BwdParams bp, int dqk, int dv, hipStream_t st) {
  AttnParams& p = bp.a;
  p.n_tiles = (p.Nq + kQM - 1) / kQM;
  p.total_work = p.B * p.H * p.n_tiles;
  p.grid_padded = (p.total_work + 7) / 8 * 8;
  bp.n_kv_tiles = (p.Nk + kBK - 1) / kBK;
  bp.total_work_kv = p.B * p.H * bp.n_kv_tiles;
  bp.grid_padded_kv = (bp.total_work_kv + 7) / 8 * 8;

  {
    hipError_t e0 = record_stage(bp, 0, st);
    if (e0 != hipSuccess) return e0;
    const int lpk = dv / 8;
    const int64_t rows = (int64_t)p.B * p.H * p.Nq;
    const int rows_per_blk = kThreads / lpk;
    const unsigned nblk = (unsigned)((rows + rows_per_blk - 1) / rows_per_blk);
    if (dv == 128) hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(nblk), dim3(kThreads), 0, st, bp);
    else if (dv == 64) hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(nblk), dim3(kThreads), 0, st, bp);
    else return hipErrorInvalidValue;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool lists = p.lists.pcnt != nullptr;
  const bool softcap = p.softcap > 0.0f;
  const bool bias = p.bias_log2 != 0.0f;
  const ListParams tl = bp.tlists;
  if (dqk == 128 && dv == 128) return dispatch<128, 128>(bp, tl, lists, softcap, bias, st);
  if (dqk == 64 && dv == 64) return dispatch<64, 64>(bp, tl, lists, softcap, bias, st);
  if (dqk == 192 && dv == 128) return dispatch<192, 128>(bp, tl, lists, softcap, bias, st);
  return hipErrorInvalidValue;
}

}  // namespace fmha
