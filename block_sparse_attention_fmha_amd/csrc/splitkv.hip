// Split-KV bf16 forward for long keys and few queries (decode), plus the combine.
//
// "Optimize Flash Dynamic Mask Attention Kernel Configurations" (flash-sparse-attention
// pull request 148) tests a split-KV forward with 1, 2, 4, 8 and 16 splits and notes
// (section "Notes") that a single query against a long key sequence is memory / latency
// bound. The split partials are merged with the two-chunk online-softmax rule of the
// POPCORNBENCH transcript "Kimi-K2.6 l1 p97" (running max, rescaled sums and outputs).
//
// With one query row per K/V head this path is HBM-bound (every K/V byte is used for one
// query row), so it does not use MFMA: there is no matrix to multiply. Each workgroup
// (one query row of one (batch, head), one split) streams its key range once:
//   * D/8 lanes cooperate on one key (16 bytes of the K row each), so a wavefront reads
//     64/(D/8) whole, contiguous K rows per load instruction (fully coalesced);
//   * the dot product is finished with DPP row operations inside the 16-lane row
//     (quad permutes and row mirrors: no LDS traffic);
//   * every lane keeps its own running (m, l, O-slice) in the log2 domain; 8 keys per
//     lane are loaded per iteration so that 16 x 16-byte loads are in flight per lane;
//   * at the end the key slots of the wave and the waves of the same query head are
//     merged with the same (m, l, O) merge and the normalised partial (O_s, LSE_s) is
//     written in fp32.
// Grouped K/V heads (several query heads reading one K/V head): with an even group size
// a workgroup serves GC = 2 or 4 query heads of one group (splitkv_grouped_kernel). Each
// lane loads its K/V row slice once and uses it for all GC heads: the score dot products
// are packed bf16 dot products (v_dot2: the product of two bf16 values is exact in
// fp32) on the bf16 Q and K, and the V slice is converted to fp32 once for the GC heads,
// so the group's K/V bytes cross HBM once and the per-(head, key) VALU work drops. An odd
// group size runs the one-head kernel with the head mapping. Groups of 4 or more query
// heads whose G x Nq rows fit 32 run on the matrix cores instead (splitkv_mfma_kernel):
// there the rows do form a matrix, and the VALU kernels' per-(head, key) work would
// dominate.
// The combine kernel then computes LSE = ln sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s per row (empty splits carry LSE_s = -inf).
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kTileKeys = 64;   // split boundaries are multiples of this
constexpr int kThreads = 256;
constexpr int kUnroll = 8;         // keys per lane slot and loop step, grouped kernel
// one query head per workgroup: 16 keys per lane slot in flight per step (188 VGPRs, two
// waves per SIMD) measured 2-5% faster at 1, 4 and 8 splits than 8 (B8 H32 Nk 32768 D128);
// the grouped kernel keeps 8 (at 16 it holds one wave per SIMD and loses 30% at 64 splits)
constexpr int kUnrollOne = 16;

// Merge running state (m, l, acc) with another one, log2 domain, -inf aware.
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float* acc, float m2, float l2, const float* acc2) {
  const float mn = fmaxf(m, m2);
  const float mu = (mn == kNegInf) ? 0.0f : mn;
  const float a = fast_exp2(m - mu), c = fast_exp2(m2 - mu);
  l = l * a + l2 * c;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * a + acc2[e] * c;
  m = mn;
}

struct SplitParams {
  AttnParams a;
  float* part_o;     // [B*H, S, Nq, Dv]
  float* part_lse;   // [B*H, S, Nq]
  int splits;
  int per_split;     // keys per split (multiple of kTileKeys)
  int group;         // query heads per K/V head (1 = multi-head)
};

template <int D>
__global__ __launch_bounds__(kThreads)
void splitkv_partial_kernel(const SplitParams sp) {
  constexpr int LPK = D / 8;         // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per load instruction
  constexpr int CHUNK = KPW * kUnrollOne;
  const AttnParams& p = sp.a;
  __shared__ float xw[4][LPK][10];

  const int s = blockIdx.x % sp.splits;
  const int rest = blockIdx.x / sp.splits;
  const int qrow = rest % p.Nq;
  const int bh = rest / p.Nq;
  const int b = bh / p.H, h = bh % p.H;
  const int hk = h / sp.group;                  // the K/V head it reads
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int slot = l / LPK, dl = l % LPK;
  const int k_lo = min(p.Nk, s * sp.per_split);
  const int k_hi = min(p.Nk, k_lo + sp.per_split);

  const __bf16* Qg = (const __bf16*)p.q + b * p.qs_b + h * p.qs_h + (int64_t)qrow * p.qs_s;
  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + hk * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + hk * p.vs_h;

  float qv[8];
  bf16x8_to_f32(*(const u32x4*)(Qg + 8 * dl), qv);
#pragma unroll
  for (int e = 0; e < 8; ++e) qv[e] *= p.scale_log2;

  float m = kNegInf, lsum = 0.0f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const bool masked = p.mask.kind != kMaskNone;

  for (int base = k_lo + w * CHUNK; base < k_hi; base += 4 * CHUNK) {
    u32x4 kr[kUnrollOne], vr[kUnrollOne];
#pragma unroll
    for (int u = 0; u < kUnrollOne; ++u) {
      const int key = base + u * KPW + slot;
      const bool in = key < k_hi;
      kr[u] = in ? *(const u32x4*)(Kg + (int64_t)key * p.ks_s + 8 * dl) : u32x4{};
      vr[u] = in ? *(const u32x4*)(Vg + (int64_t)key * p.vs_s + 8 * dl) : u32x4{};
    }
    float sc[kUnrollOne];
#pragma unroll
    for (int u = 0; u < kUnrollOne; ++u) {
      float kf[8];
      bf16x8_to_f32(kr[u], kf);
      float x = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x = __builtin_fmaf(qv[e], kf[e], x);
      sc[u] = group_sum<LPK>(x);
      const int key = base + u * KPW + slot;
      bool vis = key < k_hi;
      if (vis && masked) vis = mask_visible(p.mask, b, qrow, key, p.Nq, p.Nk);
      if (!vis) sc[u] = kNegInf;
    }
    float mt = sc[0];
#pragma unroll
    for (int u = 1; u < kUnrollOne; ++u) mt = fmaxf(mt, sc[u]);
    const float mn = fmaxf(m, mt);
    const float mu = (mn == kNegInf) ? 0.0f : mn;
    const float alpha = fast_exp2(m - mu);
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnrollOne; ++u) {
      const float pu = fast_exp2(sc[u] - mu);
      lsum += pu;
      float vf[8];
      bf16x8_to_f32(vr[u], vf);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(pu, vf[e], acc[e]);
    }
    m = mn;
  }

  // merge the key slots of the wave (lanes dl, dl + LPK, ...)
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    float acc2[8];
    const float m2 = __shfl_xor(m, off), l2 = __shfl_xor(lsum, off);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[e], off);
    merge_state<8>(m, lsum, acc, m2, l2, acc2);
  }
  if (slot == 0) {
    xw[w][dl][0] = m;
    xw[w][dl][1] = lsum;
#pragma unroll
    for (int e = 0; e < 8; ++e) xw[w][dl][2 + e] = acc[e];
  }
  __syncthreads();
  if (w == 0 && slot == 0) {
#pragma unroll
    for (int ww = 1; ww < 4; ++ww) merge_state<8>(m, lsum, acc, xw[ww][dl][0], xw[ww][dl][1], &xw[ww][dl][2]);
    const bool empty = !(lsum > 0.0f);
    const float inv = empty ? 0.0f : 1.0f / lsum;
    const int64_t row = ((int64_t)bh * sp.splits + s) * p.Nq + qrow;
    float* po = sp.part_o + row * D + 8 * dl;
    f32x4 x0 = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    f32x4 x1 = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
    *(f32x4*)po = x0;
    *(f32x4*)(po + 4) = x1;
    if (dl == 0) sp.part_lse[row] = empty ? kNegInf : (m + fast_log2(lsum)) * kLn2;
  }
}

// The two bf16 values packed in a 32-bit word. (A memcpy, not __builtin_bit_cast of a
// vector element: hipcc compiles the latter as a cast of element 0 whatever the index.)
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t x) {
  bf16x2 v;
  __builtin_memcpy(&v, &x, 4);
  return v;
}

// GC query heads (one run of a K/V group) per workgroup, same key walk and merges as the
// one-head kernel; see the file comment.
template <int D, int GC>
__global__ __launch_bounds__(kThreads)
void splitkv_grouped_kernel(const SplitParams sp) {
  constexpr int LPK = D / 8;
  constexpr int KPW = 64 / LPK;
  constexpr int CHUNK = KPW * kUnroll;
  const AttnParams& p = sp.a;
  __shared__ float xw[4][GC][LPK][10];

  const int s = blockIdx.x % sp.splits;
  const int rest = blockIdx.x / sp.splits;
  const int qrow = rest % p.Nq;
  const int bhc = rest / p.Nq;                  // (batch, run of GC query heads)
  const int nhc = p.H / GC;
  const int b = bhc / nhc;
  const int h0 = (bhc - b * nhc) * GC;
  const int hk = h0 / sp.group;                 // GC divides the group: one K/V head
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int slot = l / LPK, dl = l % LPK;
  const int k_lo = min(p.Nk, s * sp.per_split);
  const int k_hi = min(p.Nk, k_lo + sp.per_split);

  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + hk * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + hk * p.vs_h;
  u32x4 qb[GC];   // bf16 Q slice of each head
#pragma unroll
  for (int gi = 0; gi < GC; ++gi)
    qb[gi] = *(const u32x4*)((const __bf16*)p.q + b * p.qs_b + (h0 + gi) * p.qs_h + (int64_t)qrow * p.qs_s + 8 * dl);

  float m[GC], lsum[GC], acc[GC][8];
#pragma unroll
  for (int gi = 0; gi < GC; ++gi) {
    m[gi] = kNegInf;
    lsum[gi] = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[gi][e] = 0.0f;
  }
  const bool masked = p.mask.kind != kMaskNone;

  for (int base = k_lo + w * CHUNK; base < k_hi; base += 4 * CHUNK) {
    u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * KPW + slot;
      const bool in = key < k_hi;
      kr[u] = in ? *(const u32x4*)(Kg + (int64_t)key * p.ks_s + 8 * dl) : u32x4{};
      vr[u] = in ? *(const u32x4*)(Vg + (int64_t)key * p.vs_s + 8 * dl) : u32x4{};
    }
    float sc[GC][kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * KPW + slot;
      bool vis = key < k_hi;
      if (vis && masked) vis = mask_visible(p.mask, b, qrow, key, p.Nq, p.Nk);
#pragma unroll
      for (int gi = 0; gi < GC; ++gi) {
        float x = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) x = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qb[gi][e]), as_bf16x2(kr[u][e]), x, false);
        x = group_sum<LPK>(x);
        sc[gi][u] = vis ? x * p.scale_log2 : kNegInf;
      }
    }
    float mu[GC];
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
      float mt = sc[gi][0];
#pragma unroll
      for (int u = 1; u < kUnroll; ++u) mt = fmaxf(mt, sc[gi][u]);
      const float mn = fmaxf(m[gi], mt);
      mu[gi] = (mn == kNegInf) ? 0.0f : mn;
      const float alpha = fast_exp2(m[gi] - mu[gi]);
      lsum[gi] *= alpha;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[gi][e] *= alpha;
      m[gi] = mn;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float vf[8];
      bf16x8_to_f32(vr[u], vf);
#pragma unroll
      for (int gi = 0; gi < GC; ++gi) {
        const float pu = fast_exp2(sc[gi][u] - mu[gi]);
        lsum[gi] += pu;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[gi][e] = __builtin_fmaf(pu, vf[e], acc[gi][e]);
      }
    }
  }

  // merge the key slots of the wave, then the four waves, per head
#pragma unroll
  for (int gi = 0; gi < GC; ++gi) {
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1) {
      float acc2[8];
      const float m2 = __shfl_xor(m[gi], off), l2 = __shfl_xor(lsum[gi], off);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc2[e] = __shfl_xor(acc[gi][e], off);
      merge_state<8>(m[gi], lsum[gi], acc[gi], m2, l2, acc2);
    }
    if (slot == 0) {
      xw[w][gi][dl][0] = m[gi];
      xw[w][gi][dl][1] = lsum[gi];
#pragma unroll
      for (int e = 0; e < 8; ++e) xw[w][gi][dl][2 + e] = acc[gi][e];
    }
  }
  __syncthreads();
  if (w == 0 && slot == 0) {
#pragma unroll
    for (int gi = 0; gi < GC; ++gi) {
#pragma unroll
      for (int ww = 1; ww < 4; ++ww)
        merge_state<8>(m[gi], lsum[gi], acc[gi], xw[ww][gi][dl][0], xw[ww][gi][dl][1], &xw[ww][gi][dl][2]);
      const bool empty = !(lsum[gi] > 0.0f);
      const float inv = empty ? 0.0f : 1.0f / lsum[gi];
      const int64_t row = ((int64_t)(b * p.H + h0 + gi) * sp.splits + s) * p.Nq + qrow;
      float* po = sp.part_o + row * D + 8 * dl;
      f32x4 x0 = {acc[gi][0] * inv, acc[gi][1] * inv, acc[gi][2] * inv, acc[gi][3] * inv};
      f32x4 x1 = {acc[gi][4] * inv, acc[gi][5] * inv, acc[gi][6] * inv, acc[gi][7] * inv};
      *(f32x4*)po = x0;
      *(f32x4*)(po + 4) = x1;
      if (dl == 0) sp.part_lse[row] = empty ? kNegInf : (m[gi] + fast_log2(lsum[gi])) * kLn2;
    }
  }
}

// Groups on the matrix cores. When one K/V head serves G >= 4 query heads, the
// G x Nq query rows of a (batch, K/V head) are a 32-row matrix, so the scores of a
// 32-key block are one product S^T = K Q^T (K rows in the permuted order of the bf16
// forward: each lane's accumulator then holds 8 consecutive keys of its row per 16-key
// group, which is the B operand of O^T += V^T P^T as is) and V^T comes from transposed
// LDS reads of the block staged in a wave-private region. Each K/V row is read from
// memory once per workgroup for the whole group. One workgroup per (batch, K/V head,
// split); its 4 waves take the split's 32-key blocks round robin, each with its own
// online softmax per row (lanes l and l ^ 32 hold the two halves of a row's 32 keys), and
// are merged at the end through LDS. Rows past G x Nq carry zero queries and are not
// stored. The partials use the layout of the other partial kernels.
constexpr int kMfmaBlock = 32;    // keys per block and wave

// Staged V row pitch in bytes: the transposed reads of 4 rows then hit disjoint banks
// (an odd multiple of 64 bytes modulo 256, as in the bf16 forward).
template <int D> struct DecodeVPitch { static constexpr int value = (D == 64) ? 192 : 320; };

template <int D>
__global__ __launch_bounds__(kThreads, 1)
void splitkv_mfma_kernel(const SplitParams sp) {
  static_assert(D == 64 || D == 128, "head dims 64 and 128");
  constexpr int kVRowBytes = DecodeVPitch<D>::value;
  constexpr int kVStage = kMfmaBlock * kVRowBytes;      // per wave
  constexpr int kMergeO = kMfmaBlock * D * 4;           // one wave's O^T, fp32
  constexpr int CH = D / 8;                             // 16-byte chunks per V row
  constexpr int NV = kMfmaBlock * CH / 64;              // V loads per lane and block
  const AttnParams& p = sp.a;
  // V staging during the key walk; afterwards the O^T of waves 1-3 for the merge
  __shared__ __attribute__((aligned(16))) char lds[3 * kMergeO];
  __shared__ float stats[4][2][kMfmaBlock];
  static_assert(4 * kVStage <= 3 * kMergeO, "V staging fits the merge buffer");

  const int G = sp.group;
  const int Hkv = p.H / G;
  const int s = blockIdx.x % sp.splits;
  const int bk = blockIdx.x / sp.splits;
  const int b = bk / Hkv, hk = bk - (bk / Hkv) * Hkv;
  const int h0 = hk * G;
  const int R = G * p.Nq;                       // rows in use (<= 32, checked on the host)
  const int k_lo = min(p.Nk, s * sp.per_split);
  const int k_hi = min(p.Nk, k_lo + sp.per_split);
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;

  // B operand Q^T: lane row lq = (query head h0 + lq / Nq, query lq % Nq)
  const int gi = lq / p.Nq, qi = lq - (lq / p.Nq) * p.Nq;
  bf16x8 qf[D / 16];
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
    qf[ks] = (lq < R) ? *(const bf16x8*)((const __bf16*)p.q + b * p.qs_b + (h0 + gi) * p.qs_h +
                                         (int64_t)qi * p.qs_s + 16 * ks + 8 * g)
                      : bf16x8{};

  const __bf16* Kg = (const __bf16*)p.k + b * p.ks_b + hk * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + b * p.vs_b + hk * p.vs_h;
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  char* vst = lds + w * kVStage;
  const bool masked = p.mask.kind != kMaskNone;

  float m_run = kNegInf, l_run = 0.0f;
  f32x16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = f32x16{};

  // this wave's blocks start at k_lo + 32 (w + 4 i); rows past k_hi read row k_hi - 1
  // (in bounds, masked out)
  bf16x8 ka[D / 16];
  u32x4 vr[NV];   // lane l: V rows l / CH + (64 / CH) i, 16-byte chunk l % CH
  auto load = [&](int blk) {
    const int kr = min(blk + prow, k_hi - 1);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) ka[ks] = *(const bf16x8*)(Kg + (int64_t)kr * p.ks_s + 16 * ks + 8 * g);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int vrow = min(blk + l / CH + (64 / CH) * i, k_hi - 1);
      vr[i] = *(const u32x4*)(Vg + (int64_t)vrow * p.vs_s + 8 * (l % CH));
    }
  };
  int blk = k_lo + kMfmaBlock * w;
  if (blk < k_hi) load(blk);
  for (; blk < k_hi; blk += 4 * kMfmaBlock) {
    f32x16 sc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[ks], sc, 0, 0, 0);
    // stage the block's V rows; the previous block's transposed reads were issued before
    // these writes by the same wave, and LDS operations of a wave run in order
#pragma unroll
    for (int i = 0; i < NV; ++i) *(u32x4*)(vst + (l / CH + (64 / CH) * i) * kVRowBytes + 16 * (l % CH)) = vr[i];
    const int next = blk + 4 * kMfmaBlock;
    if (next < k_hi) load(next);   // in flight during the softmax and P V of this block
    // reg r holds key blk + 16 (r / 8) + 8 g + r % 8 of row lq
    float x[16];
    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = blk + 16 * (r >> 3) + 8 * g + (r & 7);
      bool vis = key < k_hi;
      if (masked && vis) vis = mask_visible(p.mask, b, qi, key, p.Nq, p.Nk);
      x[r] = vis ? sc[r] * p.scale_log2 : kNegInf;
      mt = fmaxf(mt, x[r]);
    }
    const float mn = fmaxf(m_run, pair_max(mt));
    const float mu = (mn == kNegInf) ? 0.0f : mn;
    const float alpha = fast_exp2(m_run - mu);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) o[i] *= alpha;
    m_run = mn;
    bf16x8 pb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      u32x4 pk;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float p0 = fast_exp2(x[8 * hh + 2 * e] - mu), p1 = fast_exp2(x[8 * hh + 2 * e + 1] - mu);
        l_run += p0 + p1;
        pk[e] = pack_bf16x2(p0, p1);
      }
      pb[hh] = __builtin_bit_cast(bf16x8, pk);
    }
    // O^T += V^T P^T: A = V^T (32 head-dim rows x 16 keys) from transposed reads
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* tp = vst + (trow + 16 * hh) * kVRowBytes + tcol * 2 + 64 * db;
        const bf16x8 va = join_bf16x8(lds_read_tr(tp), lds_read_tr(tp + 4 * kVRowBytes));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb[hh], o[db], 0, 0, 0);
      }
  }
  l_run = pair_sum(l_run);

  // merge the 4 waves: waves 1-3 leave (m, l) and O^T in LDS, wave 0 combines and stores;
  // lane (lq, g) holds O^T[d][lq] for d = 32 db + 8 (r / 4) + 4 g + r % 4
  __syncthreads();   // every wave is done with its V staging region
  if (g == 0) {
    stats[w][0][lq] = m_run;
    stats[w][1][lq] = l_run;
  }
  if (w > 0) {
    float* ob = (float*)(lds + (w - 1) * kMergeO) + lq * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
        *(f32x4*)(ob + 32 * db + 8 * q4 + 4 * g) = f32x4{o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]};
  }
  __syncthreads();
  if (w != 0 || lq >= R) return;
  float mx = m_run;
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) mx = fmaxf(mx, stats[ww][0][lq]);
  const float mu = (mx == kNegInf) ? 0.0f : mx;
  float c[4];
  c[0] = fast_exp2(m_run - mu);
  float tot = l_run * c[0];
#pragma unroll
  for (int ww = 1; ww < 4; ++ww) {
    c[ww] = fast_exp2(stats[ww][0][lq] - mu);
    tot += stats[ww][1][lq] * c[ww];
  }
  const bool empty = !(tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / tot;
  const int64_t row = ((int64_t)(b * p.H + h0 + gi) * sp.splits + s) * p.Nq + qi;
  float* po = sp.part_o + row * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int d = 32 * db + 8 * q4 + 4 * g;
      f32x4 acc = f32x4{o[db][4 * q4], o[db][4 * q4 + 1], o[db][4 * q4 + 2], o[db][4 * q4 + 3]} * c[0];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) acc += *(const f32x4*)((const float*)(lds + (ww - 1) * kMergeO) + lq * D + d) * c[ww];
      *(f32x4*)(po + d) = acc * inv;
    }
  if (g == 0) sp.part_lse[row] = empty ? kNegInf : (mx + fast_log2(tot)) * kLn2;
}

// One workgroup of D threads per (b, h, query row): LSE-weighted merge of the partials.
template <int D>
__global__ __launch_bounds__(D)
void splitkv_combine_kernel(const SplitParams sp) {
  const AttnParams& p = sp.a;
  const int qrow = blockIdx.x % p.Nq;
  const int bh = blockIdx.x / p.Nq;
  const int b = bh / p.H, h = bh % p.H;
  const int d = threadIdx.x;
  const int64_t row0 = (int64_t)bh * sp.splits * p.Nq + qrow;
  float mx = kNegInf;
  for (int s = 0; s < sp.splits; ++s) mx = fmaxf(mx, sp.part_lse[row0 + (int64_t)s * p.Nq]);
  const bool empty = (mx == kNegInf);
  const float mu = empty ? 0.0f : mx;
  float tot = 0.0f, o = 0.0f;
  for (int s = 0; s < sp.splits; ++s) {
    const int64_t row = row0 + (int64_t)s * p.Nq;
    const float wgt = __expf(sp.part_lse[row] - mu);
    tot += wgt;
    o += wgt * sp.part_o[row * D + d];
  }
  const float outv = empty ? 0.0f : o / tot;
  __bf16* Og = (__bf16*)p.o + b * p.os_b + h * p.os_h + (int64_t)qrow * p.os_s;
  Og[d] = (__bf16)outv;
  if (d == 0) p.lse[((int64_t)b * p.H + h) * p.Nq + qrow] = empty ? kNegInf : mu + __logf(tot);
}

}  // namespace

int splitkv_tile_keys() { return kTileKeys; }

size_t splitkv_workspace_bytes(int B, int H, int Nq, int Dv, int splits) {
  const size_t rows = (size_t)B * H * splits * Nq;
  const size_t o_bytes = rows * Dv * sizeof(float);
  return ((o_bytes + 255) / 256) * 256 + rows * sizeof(float);
}

hipError_t launch_fwd_splitkv(AttnParams p, int d, int splits, int group, void* ws, hipStream_t st) {
  SplitParams sp;
  sp.a = p;
  sp.splits = splits;
  sp.group = group;
  const int gc = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;   // query heads per workgroup
  const int tiles = (p.Nk + kTileKeys - 1) / kTileKeys;
  sp.per_split = ((tiles + splits - 1) / splits) * kTileKeys;
  const size_t rows = (size_t)p.B * p.H * splits * p.Nq;
  sp.part_o = (float*)ws;
  sp.part_lse = (float*)((char*)ws + ((rows * d * sizeof(float) + 255) / 256) * 256);
  const unsigned nblk = (unsigned)(p.B * (p.H / gc) * p.Nq * splits);
  const unsigned nrow = (unsigned)(p.B * p.H * p.Nq);
  if (d != 64 && d != 128) return hipErrorInvalidValue;
  // a group whose rows fit one 32-row product runs on the matrix cores when it has 8 or
  // more query heads, or 4-7 with at least 1024 keys per split (measured at B=8 H=32
  // Nk=32768: G = 4 is equal or faster down to 1024 keys per split, slower at 512; G = 1
  // is slower)
  const bool mfma = group * p.Nq <= kMfmaBlock && (group >= 8 || (group >= 4 && sp.per_split >= 1024));
  auto partial = [&](auto d_c) {
    constexpr int DD = decltype(d_c)::value;
    if (mfma)
      hipLaunchKernelGGL(splitkv_mfma_kernel<DD>, dim3((unsigned)(p.B * (p.H / group) * splits)), dim3(kThreads),
                         0, st, sp);
    else if (gc == 4) hipLaunchKernelGGL((splitkv_grouped_kernel<DD, 4>), dim3(nblk), dim3(kThreads), 0, st, sp);
    else if (gc == 2) hipLaunchKernelGGL((splitkv_grouped_kernel<DD, 2>), dim3(nblk), dim3(kThreads), 0, st, sp);
    else hipLaunchKernelGGL(splitkv_partial_kernel<DD>, dim3(nblk), dim3(kThreads), 0, st, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(splitkv_combine_kernel<DD>, dim3(nrow), dim3(DD), 0, st, sp);
    return hipGetLastError();
  };
  return d == 128 ? partial(IntC<128>{}) : partial(IntC<64>{});
}

}  // namespace fmha
