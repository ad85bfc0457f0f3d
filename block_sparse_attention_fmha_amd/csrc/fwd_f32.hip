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
//   * the NW partial S^T tiles are summed through LDS in a fixed wave order (a
//     reduce-scatter: wave w sums the w-th part of the tile over all partials, every wave
//     then reads the whole sum; deterministic), every wave then runs the identical online
//     softmax;
//   * O^T[slice] += V[:, slice]^T P^T with the same MFMA, so the O accumulator of a wave
//     is only its slice (32 queries x DW).
// Each K and V slice is used by exactly one wave, so nothing is shared through LDS but
// the partial scores. The memory streams are pipelined per wave: the wave's V slice of a
// key tile goes straight into a wave-private LDS region (global_load_lds_dwordx4) while
// the score MFMAs of the same tile run, and the K slice of the next tile is loaded into
// registers while the softmax and the P V MFMAs of the current one run. The two
// workgroup barriers per tile (partials written / partials read) do not wait for
// either stream. Key tiles are 32 rows.
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
struct F32Smem {
  static constexpr int NW = D / DW;
  static constexpr int ROW = DW * 4;                 // bytes of one key row of a V slice
  static constexpr int VSLICE = kBN * ROW;            // one wave's V slice of a key tile
  static constexpr int NV = VSLICE / 1024;            // DMA instructions per slice
  static constexpr int RED = NW * 16 * 64 * 4;        // partial S^T of every wave
  static constexpr int BYTES = NW * VSLICE + RED;
  static_assert(VSLICE % 1024 == 0, "V slice must be whole 1 KiB blocks");
};

// s_waitcnt lgkmcnt(0) + s_barrier, with no wait on vector-memory loads (a __syncthreads
// fence would also drain the K prefetch and the V stream).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int D, int DW>
__global__ __launch_bounds__((D / DW) * 64, 1)
void fwd_f32_kernel(const AttnParams p) {
  using SM = F32Smem<D, DW>;
  constexpr int NW = SM::NW;
  constexpr int VE = DW / 32;  // V / O elements per lane per key row
  constexpr int NK = DW / 8;   // f32x4 K loads per lane per tile
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int bid = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid >= p.total_work) return;
  const int bh = bid / p.n_tiles;
  const int t = bid - bh * p.n_tiles;
  const int qt = p.longest_first ? (p.n_tiles - 1 - t) : t;
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int q0 = qt * kBM;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  const int Nq = p.Nq, Nk = p.Nk, delta = Nk - Nq;
  const int dsl = w * DW;

  const float* Qg = (const float*)p.q + b * p.qs_b + h * p.qs_h;
  const float* Kg = (const float*)p.k + b * p.ks_b + kv_head(p, h) * p.ks_h + dsl + 4 * g;
  const float* Vg = (const float*)p.v + b * p.vs_b + kv_head(p, h) * p.vs_h + dsl;
  char* vslice = smem + w * SM::VSLICE;
  float* red = (float*)(smem + NW * SM::VSLICE);

  const int mk = p.mask.kind;
  int lo = 0, hi = Nk;
  if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kBM + delta);
  if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kBM + delta));
  if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
  hi = max(hi, 0);
  const int t_lo = lo / kBN;
  const int count = max(0, (hi + kBN - 1) / kBN - t_lo);

  // Q slice: lane (query lq, half g) holds d = dsl + 8 j + 4 g + e for MFMA step 4 j + e
  // (rows past Nq read row q0 instead: their results are never stored)
  const int qrow = q0 + lq;
  f32x4 qf[NK];
  {
    const float* qp = Qg + (int64_t)((qrow < Nq) ? qrow : q0) * p.qs_s + dsl + 4 * g;
#pragma unroll
    for (int j = 0; j < NK; ++j) qf[j] = *(const f32x4*)(qp + 8 * j);
  }

  // V slice DMA: instruction j, lane l fills slice bytes 1024 j + 16 l = key row
  // RPI j + l / (ROW / 16), bytes 16 (l % (ROW / 16)) of the row; the row step of the
  // instruction goes into the scalar base. Rows past Nk load row 0 of the tile instead
  // (finite data that only ever meets a zero probability).
  constexpr int RPI = 1024 / SM::ROW;   // key rows per DMA instruction
  const int vrow_l = l / (SM::ROW / 16);
  const uint32_t vcol_l = 16u * (uint32_t)(l % (SM::ROW / 16));
  const uint32_t voff_l = (uint32_t)(vrow_l * (int)(p.vs_s * 4)) + vcol_l;
  const uint32_t vlds = uniform_lds(vslice);
  auto issue_v = [&](int n0) {
    const int left = Nk - n0;
    if (left >= kBN) {
#pragma unroll
      for (int j = 0; j < SM::NV; ++j)
        dma_16b_u(uniform_addr(Vg + (int64_t)(n0 + RPI * j) * p.vs_s), voff_l, vlds + 1024u * j);
    } else {
      // ragged last tile: every instruction addresses from the tile's first row, so each
      // lane offset is non-negative (row * row bytes + column, or just the column of row
      // n0 for rows past Nk); the 32-bit offset is zero-extended by the hardware.
      // (opaque: the per-instruction offsets are not hoisted out of the loop as
      // registers)
      const uint64_t base = uniform_addr(Vg + (int64_t)n0 * p.vs_s);
      const int vr = opaque_int(vrow_l);
      const uint32_t vc = (uint32_t)opaque_int((int)vcol_l);
      const uint32_t rowb = (uint32_t)(p.vs_s * 4);
#pragma unroll
      for (int j = 0; j < SM::NV; ++j) {
        const int row = RPI * j + vr;
        const uint32_t v = (row < left) ? (uint32_t)row * rowb + vc : vc;
        dma_16b_u(base, v, vlds + 1024u * j);
      }
    }
  };
  // K slice of a tile, streamed through a rolling window of KPRE register chunks: chunk j
  // of lane row n0 + lq (rows past Nk read row n0: masked anyway) goes to slot j % KPRE.
  // The first KPRE chunks of a tile are prefetched during the previous tile; chunk
  // j + KPRE is loaded once the MFMAs of chunk j have been issued.
  constexpr int KPRE = NK / 2;
  f32x4 kr[KPRE];
  auto k_ptr = [&](int n0) {
    const int krow = (n0 + lq < Nk) ? n0 + lq : n0;
    return Kg + (int64_t)krow * p.ks_s;
  };
  int band_lo, band_hi;
  band_interval(p.mask, qrow, Nq, Nk, band_lo, band_hi);
  const int* doc_k = (mk == kMaskBlockDiag) ? p.mask.doc_k + (int64_t)b * Nk : nullptr;
  const int row_doc = (mk == kMaskBlockDiag && qrow < Nq) ? p.mask.doc_q[(int64_t)b * Nq + qrow] : 0;

  f32x16 o[VE];
#pragma unroll
  for (int e = 0; e < VE; ++e) o[e] = f32x16{};
  float m_run = kNegInf, l_run = 0.0f;
  // per-lane LDS bases: the lane's partial S^T quads, and its V row (key 4 g, column VE lq)
  float4* red_w = (float4*)red + w * 4 * 64 + l;
  const char* vrd = vslice + 4 * g * SM::ROW + 4 * VE * lq;

  if (count > 0) {
    const float* kp = k_ptr(t_lo * kBN);
#pragma unroll
    for (int j = 0; j < KPRE; ++j) kr[j] = *(const f32x4*)(kp + 8 * j);
  }
  for (int it = 0; it < count; ++it) {
    const int n0 = (t_lo + it) * kBN;

    // the prefetched K(it) chunks have landed (they are the only loads in flight);
    // V(it) streams in behind the score MFMAs
    wait_all_vmem();
    issue_v(n0);

    // partial S^T over this wave's D slice; the compiler waits for the streamed chunks
    // by its own count (no direct-to-LDS load is issued after them)
    f32x16 acc = f32x16{};
    {
      const float* kp = k_ptr(n0);
#pragma unroll
      for (int j = 0; j < NK; ++j) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mfma_f32(kr[j % KPRE][e], qf[j][e], acc);
        if (j + KPRE < NK) kr[j % KPRE] = *(const f32x4*)(kp + 8 * (j + KPRE));
      }
    }
    // prefetch the first chunks of K(it + 1) behind the softmax and the P V MFMAs
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 < count) {
      const float* kp = k_ptr(n0 + kBN);
#pragma unroll
      for (int j = 0; j < KPRE; ++j) kr[j] = *(const f32x4*)(kp + 8 * j);
    }

    // every wave needs the full sum: a reduce-scatter through LDS. Each wave writes its
    // partial; wave w sums the w-th of NW equal parts of the tile over all partials (in
    // wave order) and writes it over that part of wave 0's partial, which only wave w
    // reads; then every wave reads the summed tile. (The previous tile's readers are past
    // the first barrier, so the buffer is free.)
    if (it > 0) lds_barrier();
#pragma unroll
    for (int rq = 0; rq < 4; ++rq)
      red_w[rq * 64] = float4{acc[4 * rq], acc[4 * rq + 1], acc[4 * rq + 2], acc[4 * rq + 3]};
    lds_barrier();
    {
      constexpr int PER = 256 * 4 / NW;                 // floats of the tile per wave (128 at NW = 8)
      static_assert(PER % 64 == 0, "whole floats per lane");
      constexpr int FPL = PER / 64;                     // floats per lane
      float* part = (float*)(smem + NW * SM::VSLICE);   // wave 0's partial; wave ww's at + ww * 1024
      const int f0 = PER * w + FPL * l;
      float x[FPL];
#pragma unroll
      for (int e = 0; e < FPL; ++e) x[e] = part[f0 + e];
#pragma unroll
      for (int ww = 1; ww < NW; ++ww)
#pragma unroll
        for (int e = 0; e < FPL; ++e) x[e] += part[ww * 1024 + f0 + e];
#pragma unroll
      for (int e = 0; e < FPL; ++e) part[f0 + e] = x[e];
    }
    lds_barrier();
    float sc[16];
    {
      const float4* q4 = (const float4*)(smem + NW * SM::VSLICE) + l;
#pragma unroll
      for (int rq = 0; rq < 4; ++rq) {
        const float4 x = q4[rq * 64];
        sc[4 * rq] = x.x; sc[4 * rq + 1] = x.y; sc[4 * rq + 2] = x.z; sc[4 * rq + 3] = x.w;
      }
    }

    // mask: reg r is key n0 + 8 (r/4) + 4 g + r % 4 of query qrow; the row sees keys
    // band_lo <= j < band_hi (band_hi <= Nk), and for the block-diagonal mask only those
    // of its own document
    const int last = n0 + kBN - 1;
    bool need = last >= Nk;
    if (mk == kMaskCausal) need = need || (last > q0 + delta);
    else if (mk == kMaskWindow) need = need || (last > q0 + delta) || (n0 < q0 + kBM - 1 + delta - p.mask.window);
    else if (mk == kMaskPrefix) need = need || (last > q0 + delta && last >= p.mask.prefix);
    else if (mk == kMaskBlockDiag) need = true;
    if (need) {
      const int kb = opaque_int(n0 + 4 * g);
      if (mk == kMaskBlockDiag) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          // an unconditional (clamped) load and a select, no per-key branch: with a
          // short-circuit test here the compiler dropped the -inf store of the first
          // register in the loop body, leaving keys n0 and n0 + 4 of every tile visible
          // to other documents' rows
          const int key = kb + 8 * (r >> 2) + (r & 3);
          const bool vis = (key < Nk) & (doc_k[min(key, Nk - 1)] == row_doc);
          sc[r] = vis ? sc[r] : kNegInf;
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kb + 8 * (r >> 2) + (r & 3);
          if (key < band_lo || key >= band_hi) sc[r] = kNegInf;
        }
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

    // V(it) has landed once only the K(it + 1) prefetch remains in flight
    if (it + 1 < count) wait_vmcnt_at_most(KPRE);
    else wait_lds_dma();
    // P V: step s uses key 8 (s/4) + 4 g + s % 4 of the tile; the LDS reads run two
    // steps ahead of the MFMAs (fenced, so the compiler neither sinks them next to
    // their use nor hoists all sixteen at once)
    auto vread = [&](int s) {
      const char* vp = vrd + (8 * (s >> 2) + (s & 3)) * SM::ROW;
      if constexpr (VE == 4) return *(const f32x4*)vp;
      else return f32x4{((const float*)vp)[0], 0.0f, 0.0f, 0.0f};
    };
    f32x4 vring[2];
    vring[0] = vread(0);
    vring[1] = vread(1);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      __builtin_amdgcn_sched_barrier(0);
      const f32x4 x = vring[s & 1];
#pragma unroll
      for (int e = 0; e < VE; ++e) o[e] = mfma_f32(x[e], sc[s], o[e]);
      if (s + 2 < 16) vring[s & 1] = vread(s + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
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
  auto kern = fwd_f32_kernel<D, DW>;
  constexpr int bytes = F32Smem<D, DW>::BYTES;
  static_assert(bytes <= kMaxLdsBytes, "LDS budget");
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid_padded), dim3((D / DW) * 64), bytes, st, p);
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
