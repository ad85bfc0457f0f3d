// fp32 attention forward for gfx950 with the head dimension split across wavefronts.
//
// This is the wide-head path: at D = 1024 a single 32-row fp32 Q tile is 128 KiB and the
// fp32 O accumulator of 32 rows is 512 registers per lane, so neither the LDS tile of
// the bf16 kernel nor a per-wave accumulator over the full D fits. The POPCORNBENCH
// transcript "Kimi-K2.6 l1 p97" (fp32 SDPA at head_dim 1024) accumulates S over D
// chunks and P V into a shared-memory O; on CDNA4 we instead give each of the NW
// wavefronts of a workgroup its own D slice of width DW for everything:
//   * S^T partial = K[:, slice] Q[:, slice]^T with v_mfma_f32_32x32x2_f32 (true fp32,
//     not a reduced-precision tensor format), Q slice resident in VGPRs;
//   * the NW partial S^T tiles are summed through LDS in a fixed wave order (same result
//     in every wave, deterministic), every wave then runs the identical online softmax;
//   * O^T[slice] += V[:, slice]^T P^T with the same MFMA, so the O accumulator of a wave
//     is only its slice (32 queries x DW).
// K and V slices are read straight from global memory (each slice is used by exactly
// one wave, so staging through LDS would buy no reuse). Key tiles are 32 rows.
//
// Score and mask semantics are the same as the bf16 kernel (scale, causal /
// sliding-window / block-diagonal / prefix-LM element masks, fully masked rows give
// O = 0 and LSE = -inf); softcap, bias and block-sparse lists are not offered here.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kBM = 32;
constexpr int kBN = 32;

template <int D, int DW>
__global__ __launch_bounds__((D / DW) * 64, 1)
void fwd_f32_kernel(const AttnParams p) {
  constexpr int NW = D / DW;
  constexpr int VE = DW / 32;  // V / O elements per lane per key row
  __shared__ float red[2][NW][16][64];

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
  const int dsl = w * DW;

  const float* Qg = (const float*)p.q + b * p.qs_b + h * p.qs_h;
  const float* Kg = (const float*)p.k + b * p.ks_b + h * p.ks_h;
  const float* Vg = (const float*)p.v + b * p.vs_b + h * p.vs_h;

  const int mk = p.mask.kind;
  int lo = 0, hi = Nk;
  if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kBM + delta);
  if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kBM + delta));
  if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
  hi = max(hi, 0);
  const int t_lo = lo / kBN;
  const int count = max(0, (hi + kBN - 1) / kBN - t_lo);

  // Q slice: lane (query lq, half g) holds d = dsl + 8 j + 4 g + e for MFMA step 4 j + e
  const int qrow = q0 + lq;
  f32x4 qf[DW / 8];
#pragma unroll
  for (int j = 0; j < DW / 8; ++j)
    qf[j] = (qrow < Nq) ? *(const f32x4*)(Qg + (int64_t)qrow * p.qs_s + dsl + 8 * j + 4 * g) : f32x4{};

  f32x16 o[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;

  for (int it = 0; it < count; ++it) {
    const int n0 = (t_lo + it) * kBN;
    const int buf = it & 1;

    // partial S^T over this wave's D slice
    f32x16 acc = f32x16{};
    {
      const int krow = n0 + lq;
      const float* kp = Kg + (int64_t)krow * p.ks_s + dsl + 4 * g;
#pragma unroll
      for (int j = 0; j < DW / 8; ++j) {
        const f32x4 kv = (krow < Nk) ? *(const f32x4*)(kp + 8 * j) : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(kv[e], qf[j][e], acc);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) red[buf][w][r][l] = acc[r];
    __syncthreads();

    // V slice rows for the 16 PV steps: step s uses key n0 + 8 (s/4) + 4 g + s % 4
    float vv[16][VE];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int vrow = n0 + 8 * (s >> 2) + 4 * g + (s & 3);
      const float* vp = Vg + (int64_t)vrow * p.vs_s + dsl + VE * lq;
      if constexpr (VE == 4) {
        const f32x4 x = (vrow < Nk) ? *(const f32x4*)vp : f32x4{};
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[s][e] = x[e];
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) vv[s][e] = (vrow < Nk) ? vp[e] : 0.0f;
      }
    }

    float sc[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float x = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) x += red[buf][ww][r][l];
      sc[r] = x;
    }

    // mask: reg r is key n0 + 8 (r/4) + 4 g + r % 4 of query qrow
    const int last = n0 + kBN - 1;
    bool need = last >= Nk;
    if (mk == kMaskCausal) need = need || (last > q0 + delta);
    else if (mk == kMaskWindow) need = need || (last > q0 + delta) || (n0 < q0 + kBM - 1 + delta - p.mask.window);
    else if (mk == kMaskPrefix) need = need || (last > q0 + delta && last >= p.mask.prefix);
    else if (mk == kMaskBlockDiag) need = true;
    if (need) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = n0 + 8 * (r >> 2) + 4 * g + (r & 3);
        bool vis = key < Nk && qrow < Nq;
        if (vis) vis = mask_visible(p.mask, b, qrow, key, Nq, Nk);
        if (!vis) sc[r] = kNegInf;
      }
    }

    float mt = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) mt = fmaxf(mt, sc[r]);
    mt = fmaxf(mt, swap_halves(mt));
    const float m_new = fmaxf(m_run, mt * p.scale_log2);
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sc[r] = fast_exp2(__builtin_fmaf(sc[r], p.scale_log2, -m_use));
      lsum += sc[r];
    }
    l_run = l_run * alpha + lsum;
    m_run = m_new;
#pragma unroll
    for (int e = 0; e < VE; ++e)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[e][r] *= alpha;

#pragma unroll
    for (int s = 0; s < 16; ++s)
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = mfma_f32(vv[s][e], sc[s], o[e]);
  }

  const float l_tot = l_run + swap_halves(l_run);
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  if (qrow < Nq) {
    float* Og = (float*)p.o + b * p.os_b + h * p.os_h + (int64_t)qrow * p.os_s + dsl;
    // O^T block e, reg r: d = dsl + VE * (8 (r/4) + 4 g + r % 4) + e
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = 8 * (r >> 2) + 4 * g + (r & 3);
      if constexpr (VE == 4) {
        f32x4 x = {o[0][r] * inv, o[1][r] * inv, o[2][r] * inv, o[3][r] * inv};
        *(f32x4*)(Og + VE * m) = x;
      } else {
#pragma unroll
        for (int e = 0; e < VE; ++e) Og[VE * m + e] = o[e][r] * inv;
      }
    }
    if (w == 0 && g == 0)
      p.lse[((int64_t)b * p.H + h) * Nq + qrow] = empty ? kNegInf : (m_run + fast_log2(l_tot)) * kLn2;
  }
}

template <int D, int DW>
hipError_t launch_d(const AttnParams& p, hipStream_t st) {
  hipLaunchKernelGGL((fwd_f32_kernel<D, DW>), dim3(p.grid_padded), dim3((D / DW) * 64), 0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(AttnParams p, int d, hipStream_t st) {
  p.n_tiles = (p.Nq + kBM - 1) / kBM;
  p.total_work = p.B * p.H * p.n_tiles;
  p.grid_padded = (p.total_work + 7) / 8 * 8;
  if (d == 64) return launch_d<64, 32>(p, st);
  if (d == 128) return launch_d<128, 32>(p, st);
  if (d == 1024) return launch_d<1024, 128>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace fmha
