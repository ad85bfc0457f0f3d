// Split-KV bf16 forward for long keys and few queries (decode), plus the combine.
//
// "Optimize Flash Dynamic Mask Attention Kernel Configurations" (flash-sparse-attention
// pull request 148) tests a split-KV forward with 1, 2, 4, 8 and 16 splits and notes
// (section "Notes") that a single query against a long key sequence is memory / latency
// bound. The split partials are merged with the two-chunk online-softmax rule of the
// POPCORNBENCH transcript "Kimi-K2.6 l1 p97" (running max, rescaled sums and outputs).
//
// On CDNA4 this path is HBM-bound (every K/V byte is used for one query row), so it
// does not use MFMA: with one query there is no matrix to multiply. Each workgroup
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
// Grouped K/V heads (several query heads reading one K/V head): the four waves of a
// workgroup take up to four query heads of one group, each streaming the whole key range
// of the split; their loads of the same K/V rows are issued close together and served
// once from memory, so the group's K/V bytes cross HBM once instead of once per query
// head. With fewer heads per workgroup the remaining waves split the keys as above.
// The combine kernel then computes LSE = ln sum_s exp(LSE_s) and
// O = sum_s exp(LSE_s - LSE) O_s per row (empty splits carry LSE_s = -inf).
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kTileKeys = 64;   // split boundaries are multiples of this
constexpr int kThreads = 256;
constexpr int kUnroll = 8;

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
  int hpw;           // query heads per workgroup, one per wave group: 1, 2 or 4 (divides group)
};

template <int D>
__global__ __launch_bounds__(kThreads)
void splitkv_partial_kernel(const SplitParams sp) {
  constexpr int LPK = D / 8;         // lanes per key
  constexpr int KPW = 64 / LPK;      // keys per wave per load instruction
  constexpr int CHUNK = KPW * kUnroll;
  const AttnParams& p = sp.a;
  __shared__ float xw[4][LPK][10];

  const int s = blockIdx.x % sp.splits;
  const int rest = blockIdx.x / sp.splits;
  const int qrow = rest % p.Nq;
  const int bhc = rest / p.Nq;                  // (batch, run of hpw query heads)
  const int nhc = p.H / sp.hpw;
  const int b = bhc / nhc;
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), l = tid & 63;
  // wave w: query head h0 + w % hpw, key slice w / hpw of nsl
  const int hpw = sp.hpw, nsl = 4 / hpw, slice = w / hpw;
  const int h = (bhc - b * nhc) * hpw + w % hpw;
  const int hk = h / sp.group;                  // the K/V head it reads
  const int bh = b * p.H + h;
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

  for (int base = k_lo + slice * CHUNK; base < k_hi; base += nsl * CHUNK) {
    u32x4 kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = base + u * KPW + slot;
      const bool in = key < k_hi;
      kr[u] = in ? *(const u32x4*)(Kg + (int64_t)key * p.ks_s + 8 * dl) : u32x4{};
      vr[u] = in ? *(const u32x4*)(Vg + (int64_t)key * p.vs_s + 8 * dl) : u32x4{};
    }
    float sc[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
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
    for (int u = 1; u < kUnroll; ++u) mt = fmaxf(mt, sc[u]);
    const float mn = fmaxf(m, mt);
    const float mu = (mn == kNegInf) ? 0.0f : mn;
    const float alpha = fast_exp2(m - mu);
    lsum *= alpha;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
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
  if (slice == 0 && slot == 0) {
    // the waves of this query head (w + hpw, w + 2 hpw, ...) in slice order
    for (int sl = 1; sl < nsl; ++sl) {
      const int ww = w + sl * hpw;
      merge_state<8>(m, lsum, acc, xw[ww][dl][0], xw[ww][dl][1], &xw[ww][dl][2]);
    }
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
  sp.hpw = (group % 4 == 0) ? 4 : (group % 2 == 0) ? 2 : 1;
  const int tiles = (p.Nk + kTileKeys - 1) / kTileKeys;
  sp.per_split = ((tiles + splits - 1) / splits) * kTileKeys;
  const size_t rows = (size_t)p.B * p.H * splits * p.Nq;
  sp.part_o = (float*)ws;
  sp.part_lse = (float*)((char*)ws + ((rows * d * sizeof(float) + 255) / 256) * 256);
  const unsigned nblk = (unsigned)(p.B * (p.H / sp.hpw) * p.Nq * splits);
  const unsigned nrow = (unsigned)(p.B * p.H * p.Nq);
  if (d == 128) {
    hipLaunchKernelGGL(splitkv_partial_kernel<128>, dim3(nblk), dim3(kThreads), 0, st, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(splitkv_combine_kernel<128>, dim3(nrow), dim3(128), 0, st, sp);
    return hipGetLastError();
  }
  if (d == 64) {
    hipLaunchKernelGGL(splitkv_partial_kernel<64>, dim3(nblk), dim3(kThreads), 0, st, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(splitkv_combine_kernel<64>, dim3(nrow), dim3(64), 0, st, sp);
    return hipGetLastError();
  }
  return hipErrorInvalidValue;
}

}  // namespace fmha
