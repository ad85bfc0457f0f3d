// Fused bf16 attention forward for gfx950: O and LSE in one pass over the key tiles.
//
// Algorithm: the streaming online softmax of the POPCORNBENCH transcript "Kimi-K2.6 l1
// p97" (running row max m, running sum l and un-normalised O, both rescaled by
// exp(m_old - m_new) whenever the max grows; normalise at the end), with the score
// terms and mask kinds of "Enable 2CTA for SM100 block-sparse backward" (fuzz tester:
// softcap, relative-bias score mod, causal / sliding-window / block-diagonal /
// prefix-LM masks, block-sparse tile lists that skip empty tiles and apply the element
// mask only on partial tiles).
//
// Mapping onto CDNA4 (our own design, not the pages' CUDA tiling):
//   * workgroup = 4 wavefronts, 128 query rows (32 per wave); key tiles of 64 rows.
//   * each wave computes S^T = K Q^T for its 32 queries with v_mfma_f32_32x32x16_bf16:
//     K rows come from LDS as the A operand, Q stays in VGPRs as the B operand for the
//     whole pass. In the S^T accumulator every lane owns ONE query row and 16 keys per
//     32-key block, so the row max / row sum need a single cross-lane step (lane ^ 32)
//     and the per-row rescale factor is a per-lane scalar.
//   * K rows are fed to the MFMA in a permuted order (bits 2 and 3 of the row index
//     swapped) so that each lane's accumulator registers hold 8 CONSECUTIVE keys per
//     16-key step; those registers, rounded to bf16, are directly the B operand of
//     O^T += V^T P^T, and the matching V^T operand is read from the row-major V tile
//     with two ds_read_b64_tr_b16 transposed reads (no transpose pass over V).
//   * K and V tiles are double-buffered in LDS; the next tile's global loads are issued
//     before the current tile's MFMAs and written to the other buffer afterwards, so
//     one barrier per tile suffices.
//   * the work item order is XCD-aware (each XCD gets a contiguous run of heads) and,
//     for causal-like masks, longest-first over query tiles.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kBM = 128;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kThreads = 256;

// LDS pitches (bytes). K rows are read 16 bytes per lane from 32 different rows: a
// dword pitch of 4 * odd (mod 64 banks) puts 16 consecutive rows on disjoint banks.
// V is read with the transposed 8-byte read (4 rows x 32 bytes per 16-lane group): a
// dword pitch of 16 or 48 (mod 64) puts those 4 row segments on disjoint banks.
template <int D> struct KPitch { static constexpr int value = D * 2 + 16; };
template <int D> struct VPitch { static constexpr int value = (D == 64) ? 192 : (D == 128 ? 320 : D * 2 + 64); };

template <int DQK, int DV>
struct FwdSmem {
  static constexpr int KP = KPitch<DQK>::value;
  static constexpr int VP = VPitch<DV>::value;
  static constexpr int KB = kBN * KP;
  static constexpr int VB = kBN * VP;
  static constexpr int STAGE = KB + VB;
  static constexpr int BYTES = 2 * STAGE;
};

// Key-tile sequence of one workgroup: analytic band or block-sparse lists.
struct TileSeq {
  int count;
  int t_lo;          // analytic: first tile
  int sub;           // lists: kernel tiles per sparse column tile
  int npart;
  int n_cols;
  const int* pidx;
  const int* fidx;
  __device__ __forceinline__ void at(int it, bool lists, int& n0, bool& partial) const {
    if (!lists) {
      n0 = (t_lo + it) * kBN;
      partial = false;
      return;
    }
    const int e = it / sub, s = it - e * sub;
    int kt;
    if (e < npart) { kt = list_entry(pidx, e, n_cols); partial = true; }
    else { kt = list_entry(fidx, e - npart, n_cols); partial = false; }
    n0 = kt * sub * kBN + s * kBN;
  }
};

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, (DQK <= 128 ? 2 : 1))
void fwd_bf16_kernel(const AttnParams p) {
  using SM = FwdSmem<DQK, DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int bid = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid >= p.total_work) return;
  const int bh = bid / p.n_tiles;
  const int t = bid - bh * p.n_tiles;
  const int qt = p.longest_first ? (p.n_tiles - 1 - t) : t;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0 = qt * kBM;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, g = l >> 5, lq = l & 31;
  const int Nq = p.Nq, Nk = p.Nk, delta = Nk - Nq;

  const __bf16* Qg = (const __bf16*)p.q + b * p.qs_b + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + h * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + h * p.vs_h;

  // ---- tile sequence
  TileSeq seq;
  seq.t_lo = 0; seq.sub = 1; seq.npart = 0; seq.n_cols = 0; seq.pidx = nullptr; seq.fidx = nullptr;
  const int mk = p.mask.kind;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nk;
    if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kBM + delta);
    if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kBM + delta));
    if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
    hi = max(hi, 0);
    const int tlo = lo / kBN, thi = (hi + kBN - 1) / kBN;
    seq.t_lo = tlo;
    seq.count = max(0, thi - tlo);
  } else {
    const int qs = q0 / p.lists.tile_rows;
    const int hm = (p.lists.heads == 1) ? 0 : h;
    const int row = (b * p.lists.heads + hm) * p.lists.n_rows + qs;
    seq.n_cols = p.lists.n_cols;
    seq.npart = clamp_count(p.lists.pcnt[row], p.lists.n_cols);
    const int nfull = clamp_count(p.lists.fcnt[row], p.lists.n_cols);
    seq.pidx = p.lists.pidx + (int64_t)row * p.lists.n_cols;
    seq.fidx = p.lists.fidx + (int64_t)row * p.lists.n_cols;
    seq.sub = p.lists.tile_cols / kBN;
    seq.count = (seq.npart + nfull) * seq.sub;
  }

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the whole pass
  const int qrow = q0 + 32 * w + lq;
  bf16x8 qf[DQK / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks) {
    if (qrow < Nq) qf[ks] = *(const bf16x8*)(Qg + (int64_t)qrow * p.qs_s + 16 * ks + 8 * g);
    else qf[ks] = bf16x8{};
  }

  // ---- global -> register staging of one K/V tile
  constexpr int KCH = kBN * DQK / 8 / kThreads;  // 16-byte chunks per thread
  constexpr int VCH = kBN * DV / 8 / kThreads;
  u32x4 kreg[KCH], vreg[VCH];
  auto load_tile = [&](int n0) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      const int key = n0 + row;
      kreg[i] = (key < Nk) ? *(const u32x4*)(Kg + (int64_t)key * p.ks_s + col * 8) : u32x4{};
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      const int key = n0 + row;
      vreg[i] = (key < Nk) ? *(const u32x4*)(Vg + (int64_t)key * p.vs_s + col * 8) : u32x4{};
    }
  };
  auto store_tile = [&](int buf) {
    char* Kl = smem + buf * SM::STAGE;
    char* Vl = Kl + SM::KB;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DQK / 8), col = c - row * (DQK / 8);
      *(u32x4*)(Kl + row * SM::KP + col * 16) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VCH; ++i) {
      const int c = tid + kThreads * i;
      const int row = c / (DV / 8), col = c - row * (DV / 8);
      *(u32x4*)(Vl + row * SM::VP + col * 16) = vreg[i];
    }
  };

  // ---- running state
  f32x16 o[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) o[i] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float c_eff = (SOFTCAP || BIAS) ? 1.0f : p.scale_log2;
  const int prow = swap_bits23(lq);
  const int qw = q0 + 32 * w;

  if (seq.count > 0) {
    int n0;
    bool part;
    seq.at(0, LISTS, n0, part);
    load_tile(n0);
    store_tile(0);
    __syncthreads();
  }

  for (int it = 0; it < seq.count; ++it) {
    const int buf = it & 1;
    int n0;
    bool partial;
    seq.at(it, LISTS, n0, partial);
    if (it + 1 < seq.count) {
      int n1;
      bool p1;
      seq.at(it + 1, LISTS, n1, p1);
      load_tile(n1);
    }
    const char* Kl = smem + buf * SM::STAGE;
    const char* Vl = Kl + SM::KB;

    // S^T for the wave's 32 queries x 64 keys (two 32-key blocks)
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const char* krow = Kl + (32 * kb + prow) * SM::KP + 16 * g;
#pragma unroll
      for (int ks = 0; ks < DQK / 16; ++ks) {
        const bf16x8 a = *(const bf16x8*)(krow + 32 * ks);
        s[kb] = mfma_bf16(a, qf[ks], s[kb]);
      }
    }

    // does this (wave, tile) need the element mask?
    bool need = (n0 + kBN > Nk);
    if constexpr (LISTS) {
      need = need || partial;
    } else {
      const int last = n0 + kBN - 1;
      if (mk == kMaskCausal) need = need || (last > qw + delta);
      else if (mk == kMaskWindow) need = need || (last > qw + delta) || (n0 < qw + 31 + delta - p.mask.window);
      else if (mk == kMaskPrefix) need = need || (last > qw + delta && last >= p.mask.prefix);
      else if (mk == kMaskBlockDiag) need = true;
    }

    // score transform (softcap / bias) and mask; reg r of block kb holds key
    // n0 + 32 kb + 16 (r / 8) + 8 g + r % 8 of query row qrow.
    if constexpr (SOFTCAP || BIAS) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = score_log2<SOFTCAP, BIAS>(s[kb][r], p, qrow, n0 + 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7));
    }
    if (need) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = n0 + 32 * kb + 16 * (r >> 3) + 8 * g + (r & 7);
          bool vis = key < Nk;
          if (vis && qrow < Nq && (LISTS ? partial : true)) vis = mask_visible(p.mask, b, qrow, key, Nq, Nk);
          if (!vis) s[kb][r] = kNegInf;
        }
    }

    // online softmax (log2 domain)
    float mt = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m_run, mt * c_eff);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.0f;
    bf16x8 pb[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = fast_exp2(__builtin_fmaf(s[kb][8 * hh + 2 * e], c_eff, -m_use));
          const float p1 = fast_exp2(__builtin_fmaf(s[kb][8 * hh + 2 * e + 1], c_eff, -m_use));
          lsum += p0 + p1;
          pk[e] = pack_bf16x2(p0, p1);
        }
        pb[kb][hh] = __builtin_bit_cast(bf16x8, pk);
      }
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    // O^T += V^T P^T; V^T operand through transposed LDS reads
    {
      const int trow = 8 * g + ((l & 15) >> 2);
      const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
#pragma unroll
      for (int db = 0; db < DV / 32; ++db) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const char* base = Vl + (32 * kb + 16 * hh + trow) * SM::VP + (32 * db + tcol) * 2;
            const u32x2 lo = lds_read_tr(base);
            const u32x2 hi = lds_read_tr(base + 4 * SM::VP);
            o[db] = mfma_bf16(join_bf16x8(lo, hi), pb[kb][hh], o[db]);
          }
        }
      }
    }

    if (it + 1 < seq.count) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue
  const float l_tot = l_run + swap_halves(l_run);
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  if (qrow < Nq) {
    __bf16* Og = (__bf16*)p.o + b * p.os_b + h * p.os_h + (int64_t)qrow * p.os_s;
#pragma unroll
    for (int db = 0; db < DV / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv);
        v[1] = pack_bf16x2(o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv);
        *(u32x2*)(Og + 32 * db + 8 * jj + 4 * g) = v;
      }
    if (g == 0) {
      p.lse[((int64_t)b * p.H + h) * Nq + qrow] = empty ? kNegInf : (m_run + fast_log2(l_tot)) * kLn2;
    }
  }
}

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
hipError_t launch_one(const AttnParams& p, hipStream_t st) {
  using SM = FwdSmem<DQK, DV>;
  auto kern = fwd_bf16_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, SM::BYTES);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid_padded), dim3(kThreads), SM::BYTES, st, p);
  return hipGetLastError();
}

template <int DQK, int DV>
hipError_t dispatch_mods(const AttnParams& p, bool lists, bool softcap, bool bias, hipStream_t st) {
  if (lists) {
    if (softcap) return bias ? launch_one<DQK, DV, true, true, true>(p, st) : launch_one<DQK, DV, true, true, false>(p, st);
    return bias ? launch_one<DQK, DV, true, false, true>(p, st) : launch_one<DQK, DV, true, false, false>(p, st);
  }
  if (softcap) return bias ? launch_one<DQK, DV, false, true, true>(p, st) : launch_one<DQK, DV, false, true, false>(p, st);
  return bias ? launch_one<DQK, DV, false, false, true>(p, st) : launch_one<DQK, DV, false, false, false>(p, st);
}

}  // namespace

int fwd_bf16_block_rows() { return kBM; }
int fwd_bf16_tile_keys() { return kBN; }

hipError_t launch_fwd_bf16(AttnParams p, int dqk, int dv, hipStream_t st) {
  p.n_tiles = (p.Nq + kBM - 1) / kBM;
  p.total_work = p.B * p.H * p.n_tiles;
  p.grid_padded = (p.total_work + 7) / 8 * 8;
  const bool lists = p.lists.pcnt != nullptr;
  const bool softcap = p.softcap > 0.0f;
  const bool bias = p.bias_log2 != 0.0f;
  if (dqk == 128 && dv == 128) return dispatch_mods<128, 128>(p, lists, softcap, bias, st);
  if (dqk == 64 && dv == 64) return dispatch_mods<64, 64>(p, lists, softcap, bias, st);
  if (dqk == 192 && dv == 128) return dispatch_mods<192, 128>(p, lists, softcap, bias, st);
  return hipErrorInvalidValue;
}

}  // namespace fmha
