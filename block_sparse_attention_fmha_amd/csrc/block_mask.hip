// Block-sparse tile-mask builder for gfx950.
//
// "Enable 2CTA for SM100 block-sparse backward" (section "Testing Testing Testing")
// builds, before every launch, forward index lists per query tile and separate
// backward lists per key tile from an element mask_mod, at a sparse tile size decoupled
// from the kernel tile, and the kernels then skip empty tiles and apply the element mask
// only on partial tiles ("Summary"). The page also records a latent out-of-bounds bug in
// mask definitions; here the predicate is never evaluated outside [0, Nq) x [0, Nk).
//
// One workgroup per (b, mask head, tile row). Each thread classifies whole tiles: it
// counts the visible in-bounds elements of its tile row by row -- in closed form for the
// band masks (causal, sliding window, prefix-LM: the visible keys of a row are one
// interval) and by comparing document ids for the block-diagonal mask -- then compares
// the count with the tile's in-bounds size (0 = empty, all = full, else partial). The
// classes go to LDS and one thread compacts them into ascending lists (slots past the
// count are -1). The transposed lists are produced by the same kernel with the roles of
// the two axes swapped, so both orientations come from one classification function.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kThreads = 256;

// visible keys of query row i inside [k0, k1)
__device__ __forceinline__ int64_t row_visible(const MaskParams& m, int b, int i, int k0, int k1, int nq,
                                               int nk) {
  const int d = nk - nq;
  int lo = k0, hi = k1;
  switch (m.kind) {
    case kMaskNone: break;
    case kMaskCausal: hi = min(k1, i + d + 1); break;
    case kMaskWindow: lo = max(k0, i + d - m.window); hi = min(k1, i + d + 1); break;
    case kMaskPrefix: hi = min(k1, max(m.prefix, i + d + 1)); break;
    case kMaskBlockDiag: {
      const int di = m.doc_q[(int64_t)b * nq + i];
      const int* dk = m.doc_k + (int64_t)b * nk;
      int64_t c = 0;
      for (int j = k0; j < k1; ++j) c += (dk[j] == di);
      return c;
    }
    default: break;
  }
  return hi > lo ? hi - lo : 0;
}

// TRANSPOSED = false: grid rows are query tiles, entries are key tiles.
// TRANSPOSED = true:  grid rows are key tiles, entries are query tiles.
template <bool TRANSPOSED>
__global__ __launch_bounds__(kThreads)
void classify_kernel(const MaskParams m, int Hm, int nq, int nk, int tile_m, int tile_n, int n_rows,
                     int n_cols, int* pcnt, int* pidx, int* fcnt, int* fidx) {
  extern __shared__ unsigned char cls[];
  const int row = blockIdx.x % n_rows;
  const int bhm = blockIdx.x / n_rows;
  const int b = bhm / Hm;
  for (int col = threadIdx.x; col < n_cols; col += kThreads) {
    const int qt = TRANSPOSED ? col : row;
    const int kt = TRANSPOSED ? row : col;
    const int q0 = qt * tile_m, q1 = min(nq, q0 + tile_m);
    const int k0 = kt * tile_n, k1 = min(nk, k0 + tile_n);
    int64_t vis = 0;
    for (int i = q0; i < q1; ++i) vis += row_visible(m, b, i, k0, k1, nq, nk);
    const int64_t all = (int64_t)(q1 - q0) * (k1 - k0);
    cls[col] = (vis == 0) ? 0 : (vis == all ? 2 : 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const int64_t base = (int64_t)blockIdx.x * n_cols;
    int np = 0, nf = 0;
    for (int col = 0; col < n_cols; ++col) {
      const unsigned char c = cls[col];
      if (c == 1) pidx[base + np++] = col;
      else if (c == 2) fidx[base + nf++] = col;
    }
    for (int e = np; e < n_cols; ++e) pidx[base + e] = -1;
    for (int e = nf; e < n_cols; ++e) fidx[base + e] = -1;
    pcnt[blockIdx.x] = np;
    fcnt[blockIdx.x] = nf;
  }
}

}  // namespace

hipError_t launch_build_block_mask(const MaskParams& m, int B, int Hm, int Nq, int Nk, int tile_m,
                                   int tile_n, const BlockMaskOut& out, hipStream_t st) {
  const int nqt = (Nq + tile_m - 1) / tile_m;
  const int nkt = (Nk + tile_n - 1) / tile_n;
  hipLaunchKernelGGL(classify_kernel<false>, dim3(B * Hm * nqt), dim3(kThreads), nkt, st, m, Hm, Nq, Nk,
                     tile_m, tile_n, nqt, nkt, out.pcnt, out.pidx, out.fcnt, out.fidx);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(classify_kernel<true>, dim3(B * Hm * nkt), dim3(kThreads), nqt, st, m, Hm, Nq, Nk,
                     tile_m, tile_n, nkt, nqt, out.tpcnt, out.tpidx, out.tfcnt, out.tfidx);
  return hipGetLastError();
}

}  // namespace fmha
