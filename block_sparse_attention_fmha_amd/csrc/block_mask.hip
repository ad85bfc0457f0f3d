// Block-sparse tile-mask builder for gfx950.
//
// "Enable 2CTA for SM100 block-sparse backward" (section "Testing Testing Testing")
// builds, before every launch, forward index lists per query tile and separate
// backward lists per key tile from an element mask_mod, at a sparse tile size decoupled
// from the kernel tile, and the kernels then skip empty tiles and apply the element mask
// only on partial tiles ("Summary"). The page also records a latent out-of-bounds bug in
// mask definitions; here the predicate is never evaluated outside [0, Nq) x [0, Nk).
//
// One workgroup per (b, mask head, tile row). Each tile's visible in-bounds elements are
// counted and compared with the tile's in-bounds size (0 = empty, all = full, else
// partial). For the band masks (causal, sliding window, prefix-LM: the visible keys of a
// row are one interval) each thread counts whole tiles in closed form, row by row. For
// the block-diagonal mask the visible pairs of a tile are sum over documents d of
// (row elements in d) x (column elements in d): the workgroup builds its tile row's
// histogram of document ids in an LDS hash table, then every column element adds its
// document's row count to its tile's 64-bit LDS counter (integer sums: exact in any
// order). Tile rows longer than the table holds fall back to comparing every row element
// with every staged column id. The classes go to LDS and the workgroup compacts them into
// ascending lists with a prefix sum (slots past the count are -1). The transposed lists
// are produced by the same kernel with the roles of the two axes swapped, so both
// orientations come from one classification.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kThreads = 256;
constexpr int kIdChunk = 8192;     // document ids staged in LDS at a time
constexpr int kMaxCounted = 4096;  // tiles per row counted in one pass (one 64-bit LDS counter each)
// histogram table of a tile row's document ids: 64-bit slots (0 = free, else 2^32 | id) and
// 32-bit counts, in the id-staging region; at most half full, so probing always ends
constexpr int kTable = 2048;
constexpr int kMaxHistRows = kTable / 2;
static_assert(kTable * 12 <= kIdChunk * 4, "the table lives in the id-staging region");

// dynamic LDS layout: tile classes (n_cols bytes), id chunk, 64-bit counters
__host__ __device__ constexpr int ids_offset(int n_cols) { return (n_cols + 15) / 16 * 16; }
__host__ __device__ constexpr int cnt_offset(int n_cols) { return ids_offset(n_cols) + kIdChunk * 4; }
__host__ __device__ constexpr int lds_bytes(int n_cols) {
  return cnt_offset(n_cols) + 8 * (n_cols < kMaxCounted ? n_cols : kMaxCounted) + 16;
}

// visible keys of query row i inside [k0, k1) under a band mask
__device__ __forceinline__ int64_t row_visible(const MaskParams& m, int i, int k0, int k1, int nq, int nk) {
  const int d = nk - nq;
  int lo = k0, hi = k1;
  switch (m.kind) {
    case kMaskCausal: hi = min(k1, i + d + 1); break;
    case kMaskWindow: lo = max(k0, i + d - m.window); hi = min(k1, i + d + 1); break;
    case kMaskPrefix: hi = min(k1, max(m.prefix, i + d + 1)); break;
    default: break;
  }
  return hi > lo ? hi - lo : 0;
}

// end of the tile starting at t0 with size ts, clipped to n (no int overflow)
__device__ __forceinline__ int tile_end(int t0, int ts, int n) { return (int)min((int64_t)n, (int64_t)t0 + ts); }

// One list row (workgroup `blk` of its orientation).
// TRANSPOSED = false: rows are query tiles, entries are key tiles.
// TRANSPOSED = true:  rows are key tiles, entries are query tiles.
template <bool TRANSPOSED>
__device__ __forceinline__ void classify_row(const MaskParams& m, int Hm, int nq, int nk, int tile_m, int tile_n,
                                             int n_rows, int n_cols, int* pcnt, int* pidx, int* fcnt, int* fidx,
                                             int blk, unsigned char* cls) {
  const int row = blk % n_rows;
  const int bhm = blk / n_rows;
  const int b = bhm / Hm;
  if (m.kind == kMaskBlockDiag && (TRANSPOSED ? min(tile_n, nk - row * tile_n) : min(tile_m, nq - row * tile_m)) <= kMaxHistRows) {
    // ---- histogram path
    unsigned long long* slot = (unsigned long long*)(cls + ids_offset(n_cols));
    int* tcnt = (int*)(slot + kTable);
    unsigned long long* cnt = (unsigned long long*)(cls + cnt_offset(n_cols));
    const int* rdoc = TRANSPOSED ? m.doc_k + (int64_t)b * nk : m.doc_q + (int64_t)b * nq;
    const int* cdoc = TRANSPOSED ? m.doc_q + (int64_t)b * nq : m.doc_k + (int64_t)b * nk;
    const int rt = TRANSPOSED ? tile_n : tile_m, ct = TRANSPOSED ? tile_m : tile_n;
    const int rn = TRANSPOSED ? nk : nq, cn = TRANSPOSED ? nq : nk;
    const int r0 = row * rt, r1 = tile_end(r0, rt, rn), nr = r1 - r0;
    const int t = threadIdx.x;
    auto home = [](int id) { return (int)(((uint32_t)id * 0x9E3779B1u) >> 21); };   // 11 bits = kTable
    for (int e = t; e < kTable; e += kThreads) {
      slot[e] = 0ull;
      tcnt[e] = 0;
    }
    __syncthreads();
    for (int i = r0 + t; i < r1; i += kThreads) {
      const int id = rdoc[i];
      const unsigned long long tag = (1ull << 32) | (uint32_t)id;
      int h = home(id);
      for (;;) {
        const unsigned long long old = atomicCAS(&slot[h], 0ull, tag);
        if (old == 0ull || old == tag) break;
        h = (h + 1) & (kTable - 1);
      }
      atomicAdd(&tcnt[h], 1);
    }
    for (int g0 = 0; g0 < n_cols; g0 += kMaxCounted) {
      const int g1 = min(n_cols, g0 + kMaxCounted);
      __syncthreads();   // table complete / the previous pass's classes written
      for (int c = t; c < g1 - g0; c += kThreads) cnt[c] = 0;
      __syncthreads();
      const int a0 = g0 * ct, a1 = tile_end((g1 - 1) * ct, ct, cn);   // column elements covered
      for (int j = a0 + t; j < a1; j += kThreads) {
        const int id = cdoc[j];
        const unsigned long long tag = (1ull << 32) | (uint32_t)id;
        int h = home(id), c = 0;
        for (;;) {
          const unsigned long long v = slot[h];
          if (v == tag) { c = tcnt[h]; break; }
          if (v == 0ull) break;
          h = (h + 1) & (kTable - 1);
        }
        if (c) atomicAdd(&cnt[j / ct - g0], (unsigned long long)c);
      }
      __syncthreads();
      for (int col = g0 + t; col < g1; col += kThreads) {
        const int c0 = col * ct, c1 = tile_end(c0, ct, cn);
        const unsigned long long vis = cnt[col - g0];
        const unsigned long long all = (unsigned long long)nr * (unsigned long long)(c1 - c0);
        cls[col] = (vis == 0) ? 0 : (vis == all ? 2 : 1);
      }
    }
  } else if (m.kind == kMaskBlockDiag) {
    int* ids = (int*)(cls + ids_offset(n_cols));
    unsigned long long* cnt = (unsigned long long*)(cls + cnt_offset(n_cols));
    // row axis: the grid row's tile; column axis: the tiles being classified
    const int* rdoc = TRANSPOSED ? m.doc_k + (int64_t)b * nk : m.doc_q + (int64_t)b * nq;
    const int* cdoc = TRANSPOSED ? m.doc_q + (int64_t)b * nq : m.doc_k + (int64_t)b * nk;
    const int rt = TRANSPOSED ? tile_n : tile_m, ct = TRANSPOSED ? tile_m : tile_n;
    const int rn = TRANSPOSED ? nk : nq, cn = TRANSPOSED ? nq : nk;
    const int r0 = row * rt, r1 = tile_end(r0, rt, rn), nr = r1 - r0;
    // thread -> (row element, slice of the column tiles): with fewer row elements than
    // threads, the threads of one element split the tiles between them
    const int t = threadIdx.x;
    const int nsl = (nr >= kThreads) ? 1 : kThreads / nr;
    const int slice = (nr >= kThreads) ? 0 : t / nr;
    const int i0 = (slice < nsl) ? r0 + ((nr >= kThreads) ? t : t % nr) : r1;
    const int istep = (nr >= kThreads) ? kThreads : nr;
    // tiles [g0, g1) counted per pass (one 64-bit counter each)
    for (int g0 = 0; g0 < n_cols; g0 += kMaxCounted) {
      const int g1 = min(n_cols, g0 + kMaxCounted);
      for (int c = t; c < g1 - g0; c += kThreads) cnt[c] = 0;
      const int a0 = g0 * ct, a1 = tile_end((g1 - 1) * ct, ct, cn);   // column elements covered
      for (int cc = a0; cc < a1; cc += kIdChunk) {
        const int ce = tile_end(cc, kIdChunk, a1);
        __syncthreads();   // counters cleared / readers of the previous chunk done
        for (int j = cc + t; j < ce; j += kThreads) ids[j - cc] = cdoc[j];
        __syncthreads();
        const int cf = cc / ct, cl = (ce - 1) / ct;   // tiles overlapping this chunk
        for (int i = i0; i < r1; i += istep) {
          const int di = rdoc[i];
          for (int col = cf + slice; col <= cl; col += nsl) {
            const int j0 = max(col * ct, cc) - cc, j1 = tile_end(col * ct, ct, ce) - cc;
            int c = 0;
#pragma unroll 8
            for (int j = j0; j < j1; ++j) c += (ids[j] == di);
            if (c) atomicAdd(&cnt[col - g0], (unsigned long long)c);   // exact in any order
          }
        }
      }
      __syncthreads();
      for (int col = g0 + t; col < g1; col += kThreads) {
        const int c0 = col * ct, c1 = tile_end(c0, ct, cn);
        const unsigned long long vis = cnt[col - g0];
        const unsigned long long all = (unsigned long long)nr * (unsigned long long)(c1 - c0);
        cls[col] = (vis == 0) ? 0 : (vis == all ? 2 : 1);
      }
      __syncthreads();   // before the counters are reused
    }
  } else {
    for (int col = threadIdx.x; col < n_cols; col += kThreads) {
      const int qt = TRANSPOSED ? col : row;
      const int kt = TRANSPOSED ? row : col;
      const int q0 = qt * tile_m, q1 = tile_end(q0, tile_m, nq);
      const int k0 = kt * tile_n, k1 = tile_end(k0, tile_n, nk);
      int64_t vis = 0;
      for (int i = q0; i < q1; ++i) vis += row_visible(m, i, k0, k1, nq, nk);
      const int64_t all = (int64_t)(q1 - q0) * (k1 - k0);
      cls[col] = (vis == 0) ? 0 : (vis == all ? 2 : 1);
    }
  }
  __syncthreads();
  // ---- compaction: thread t takes the contiguous columns [t per, (t + 1) per), counts its
  // partial and full tiles, and an exclusive prefix sum over the threads (in thread order,
  // so the lists stay ascending) gives where its entries go
  {
    const int t = threadIdx.x, l = t & 63, w = t >> 6;
    const int per = (n_cols + kThreads - 1) / kThreads;
    const int c0 = min(n_cols, t * per), c1 = min(n_cols, c0 + per);
    int np = 0, nf = 0;
    for (int col = c0; col < c1; ++col) {
      np += cls[col] == 1;
      nf += cls[col] == 2;
    }
    // inclusive scan within the wave, then across the four waves through LDS
    int sp = np, sf = nf;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int up = __shfl_up(sp, d), uf = __shfl_up(sf, d);
      if (l >= d) sp += up, sf += uf;
    }
    int* wsum = (int*)(cls + ids_offset(n_cols));   // the id / table region is free again
    if (l == 63) {
      wsum[2 * w] = sp;
      wsum[2 * w + 1] = sf;
    }
    __syncthreads();
    int op = sp - np, of = sf - nf, tp = 0, tf = 0;
#pragma unroll
    for (int v = 0; v < kThreads / 64; ++v) {
      if (v < w) op += wsum[2 * v], of += wsum[2 * v + 1];
      tp += wsum[2 * v];
      tf += wsum[2 * v + 1];
    }
    const int64_t base = (int64_t)blk * n_cols;
    for (int col = c0; col < c1; ++col) {
      const unsigned char c = cls[col];
      if (c == 1) pidx[base + op++] = col;
      else if (c == 2) fidx[base + of++] = col;
    }
    for (int e = tp + t; e < n_cols; e += kThreads) pidx[base + e] = -1;
    for (int e = tf + t; e < n_cols; e += kThreads) fidx[base + e] = -1;
    if (t == 0) {
      pcnt[blk] = tp;
      fcnt[blk] = tf;
    }
  }
}

// Both orientations in one launch: the first B Hm n_q_tiles workgroups build the forward
// lists, the rest the transposed ones.
__global__ __launch_bounds__(kThreads)
void classify_kernel(const MaskParams m, int Hm, int nq, int nk, int tile_m, int tile_n, int nqt, int nkt,
                     int fwd_blocks, const BlockMaskOut out) {
  extern __shared__ __attribute__((aligned(16))) unsigned char cls[];
  if ((int)blockIdx.x < fwd_blocks)
    classify_row<false>(m, Hm, nq, nk, tile_m, tile_n, nqt, nkt, out.pcnt, out.pidx, out.fcnt, out.fidx,
                        blockIdx.x, cls);
  else
    classify_row<true>(m, Hm, nq, nk, tile_m, tile_n, nkt, nqt, out.tpcnt, out.tpidx, out.tfcnt, out.tfidx,
                       blockIdx.x - fwd_blocks, cls);
}

}  // namespace

hipError_t launch_build_block_mask(const MaskParams& m, int B, int Hm, int Nq, int Nk, int tile_m,
                                   int tile_n, const BlockMaskOut& out, hipStream_t st) {
  const int nqt = (Nq + tile_m - 1) / tile_m;
  const int nkt = (Nk + tile_n - 1) / tile_n;
  const int bytes = lds_bytes(nkt > nqt ? nkt : nqt);   // either orientation's columns
  hipError_t e = hipFuncSetAttribute((const void*)classify_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  const int fwd_blocks = B * Hm * nqt;
  hipLaunchKernelGGL(classify_kernel, dim3(fwd_blocks + B * Hm * nkt), dim3(kThreads), bytes, st, m, Hm, Nq, Nk,
                     tile_m, tile_n, nqt, nkt, fwd_blocks, out);
  return hipGetLastError();
}

}  // namespace fmha
