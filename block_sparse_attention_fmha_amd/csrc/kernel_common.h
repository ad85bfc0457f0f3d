// Device-side helpers and kernel parameter blocks shared by the HIP kernels.
//
// Everything here is CDNA4 (gfx950) specific: 64-lane wavefronts, the
// v_mfma_f32_32x32x16_bf16 / v_mfma_f32_32x32x2_f32 matrix instructions and the
// ds_read_b64_tr_b16 transposed LDS read.
//
// Operand layouts of v_mfma_f32_32x32x16_bf16 (lane l, g = l / 32):
//   A (32 x 16, M x K): lane l holds row l % 32, k = 8 g + i for its 8 elements i
//   B (16 x 32, K x N): lane l holds column l % 32, k = 8 g + i
//   C (32 x 32):        lane l holds column l % 32, rows 8 (r / 4) + 4 g + r % 4, r = 0..15
// v_mfma_f32_32x32x2_f32 is the same with one element per lane (k = g).
//
// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives, as its element e
// (e = 0..3), element i % 4 of the 8 bytes read by lane 4 e + i / 4 of the group. If lane
// 4 e + c of the group points at row (r0 + e), columns (c0 + 4 c .. c0 + 4 c + 3) of a
// row-major bf16 tile, lane i receives column c0 + i of rows r0 .. r0 + 3: a transposed
// 4 x 16 read that yields MFMA operands with the contraction index along the rows.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fmha {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

enum MaskKind { kMaskNone = 0, kMaskCausal = 1, kMaskWindow = 2, kMaskBlockDiag = 3, kMaskPrefix = 4 };

// Per-tile element-mask test, chosen once per tile so the unrolled element loops carry no
// run-time case: none, a visible interval per row or column, or the document comparison.
// kTestDocVec is the document comparison on a tile whose document ids are all in bounds
// and 16-byte aligned, so they are read with vector loads.
enum MaskTest { kTestNone = 0, kTestBand = 1, kTestDoc = 2, kTestDocVec = 3 };
template <int V> struct IntC { static constexpr int value = V; };

// A value the optimiser may not look through. Used on per-step row or column bases so the
// per-element offsets added to them are not hoisted out of the main loop as dozens of
// loop-invariant registers.
__device__ __forceinline__ int opaque_int(int x) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("" : "+v"(x));
#endif
  return x;
}

// ---------------------------------------------------------------------------------------
// Parameter blocks (passed by value as kernel arguments).

struct MaskParams {
  int kind, window, prefix;
  const int* doc_q;  // [B, Nq]
  const int* doc_k;  // [B, Nk]
};

// Key tiles [*t_lo, *t_lo + *count) of width `tile` that a band mask leaves visible to the
// query rows [q0, q0 + rows): causal and sliding-window rows i see keys up to
// i + Nk - Nq (bottom-right aligned), a sliding window from i + Nk - Nq - window, prefix-LM
// rows also every key below the prefix; no mask and the block-diagonal mask walk every
// tile. Host and device, so that the host plans the forward's key split from the same
// counts the kernels walk.
__host__ __device__ inline void band_tile_range(const MaskParams& m, int q0, int rows, int Nq, int Nk,
                                                int tile, int* t_lo, int* count) {
  const int delta = Nk - Nq;
  int lo = 0, hi = Nk;
  if (m.kind == kMaskCausal || m.kind == kMaskWindow) hi = q0 + rows + delta < Nk ? q0 + rows + delta : Nk;
  if (m.kind == kMaskPrefix) {
    const int reach = m.prefix > q0 + rows + delta ? m.prefix : q0 + rows + delta;
    hi = reach < Nk ? reach : Nk;
  }
  if (m.kind == kMaskWindow) lo = q0 + delta - m.window > 0 ? q0 + delta - m.window : 0;
  if (hi < 0) hi = 0;
  const int tlo = lo / tile, thi = (hi + tile - 1) / tile;
  *t_lo = tlo;
  *count = thi > tlo ? thi - tlo : 0;
}

// Number of contiguous key parts a query tile of `count` key tiles is walked in under a
// key split of at most `splits` parts of about `tiles` tiles each (1: not split).
__host__ __device__ inline int key_pieces(int count, int splits, int tiles) {
  if (splits <= 1) return 1;
  const int n = (count + tiles - 1) / tiles;
  return n < 1 ? 1 : (n > splits ? splits : n);
}

constexpr int kMaxLdsBytes = 160 * 1024;   // LDS per workgroup on gfx950

struct ListParams {  // block-sparse index lists, forward or transposed orientation
  const int* pcnt;
  const int* pidx;
  const int* fcnt;
  const int* fidx;
  int heads, tile_rows, tile_cols, n_rows, n_cols;  // rows = the side the grid walks
};

struct AttnParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t qs_b, qs_s, qs_h, ks_b, ks_s, ks_h, vs_b, vs_s, vs_h, os_b, os_s, os_h;
  int B, H, Nq, Nk;
  int n_tiles;        // tiles of the resident side (query tiles for the forward)
  int total_work;     // B * H * n_tiles
  int grid_padded;    // total_work rounded up to a multiple of 8 (XCD remap)
  int longest_first;  // walk resident tiles from the one with the most keys
  float scale;        // softmax scale
  float scale_log2;   // scale * log2(e)
  float softcap;      // > 0: tanh softcap
  float cap_k1;       // softcap: scale * 2 log2(e) / softcap (raw score -> log2 of exp(2 y))
  float cap_u;        // softcap: softcap * log2(e) (the capped score's log2-unit limit)
  int cap_fixed;      // softcap without bias and 2 cap_u <= 100: the forward may use cap_u as
                      // a fixed softmax maximum (every exp2(u - cap_u) lies in [2^-100, 1])
  // key split of the bf16 forward (kv_splits 1 = off): a query tile whose visible range
  // holds `count` key tiles is walked in key_pieces(count, kv_splits, split_tiles)
  // contiguous parts, workgroup (tile, s) taking part s; a tile walked in more than one
  // part writes normalised fp32 partial O [B*H, n_tiles, kv_splits, tile rows, Dv] and
  // natural-log partial LSE [B*H, n_tiles, kv_splits, tile rows] for the combine
  int kv_splits;
  int split_tiles;
  float* split_o;
  float* split_lse;
  float bias_log2;    // relative-bias slope * log2(e)
  MaskParams mask;
  ListParams lists;
  // packed variable-length sequences (forward only; nullptr = fixed lengths): batch b is
  // the sequence of queries [cu_q[b], cu_q[b+1]) and keys [cu_k[b], cu_k[b+1]) along the
  // sequence axis (the batch strides are unused); LSE is [H, lse_total]
  const int* cu_q;
  const int* cu_k;
  // optional used lengths [B] (nullptr = the whole span): only the first used_q[b] queries
  // and used_k[b] keys of sequence b take part; rows past them are neither read nor written
  const int* used_q;
  const int* used_k;
  int64_t lse_total;
  int group;          // query heads per K/V head (0 or 1: one K/V head per query head)
};

// K/V head read by query head h (grouped-query attention: consecutive groups of
// p.group query heads share one K/V head)
__device__ __forceinline__ int kv_head(const AttnParams& p, int h) { return p.group > 1 ? h / p.group : h; }

struct BwdParams {
  AttnParams a;       // q, k, v, o (forward output), lse (forward LSE)
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* ws;          // workspace: per (b, h) and 64-query block, 64 x lse2 then 64 x D
                      // (lse2 = LSE log2(e), +inf for empty rows and rows past Nq;
                      // D_i = sum_d dO_id O_id, 0 past Nq), plus 512 bytes of tail padding
  int n_qblk;         // 64-query blocks per (b, h): ceil(Nq / 64)
  int64_t dos_b, dos_s, dos_h, dqs_b, dqs_s, dqs_h, dks_b, dks_s, dks_h, dvs_b, dvs_s, dvs_h;
  ListParams tlists;  // transposed block-sparse lists (per key tile) for the dK/dV pass
  void* const* stage_events;  // optional host array of 4 hipEvent_t (host side only)
  int n_kv_tiles;     // key tiles for the dK/dV pass
  int total_work_kv;
  int grid_padded_kv;
};

// Batch entry b: its query / key lengths and first rows. Fixed lengths: every entry has
// p.Nq / p.Nk rows at batch stride b; packed varlen: rows cu[b] .. cu[b+1] of the packed
// sequence axis. row_base() is the element offset of the entry's row 0 in one tensor;
// lse_base() that of (b, h, row 0) in LSE ([B, H, Nq], or [H, total_q] when packed).
struct SeqInfo {
  int nq, nk, qs, ks;
  bool packed;
};
// A used length outside [0, span] is clamped to it (the lengths are read on the device only).
__device__ __forceinline__ SeqInfo seq_info(const AttnParams& p, int b) {
  SeqInfo s{p.Nq, p.Nk, 0, 0, false};
  if (p.cu_q != nullptr) {
    s.qs = p.cu_q[b];
    s.ks = p.cu_k[b];
    s.nq = p.cu_q[b + 1] - s.qs;
    s.nk = p.cu_k[b + 1] - s.ks;
    if (p.used_q != nullptr) s.nq = min(max(p.used_q[b], 0), s.nq);
    if (p.used_k != nullptr) s.nk = min(max(p.used_k[b], 0), s.nk);
    s.packed = true;
  }
  return s;
}
__device__ __forceinline__ int64_t row_base(const SeqInfo& s, bool query_axis, int b, int64_t stride_b,
                                            int64_t stride_s) {
  return s.packed ? (int64_t)(query_axis ? s.qs : s.ks) * stride_s : (int64_t)b * stride_b;
}
__device__ __forceinline__ int64_t lse_base(const AttnParams& p, const SeqInfo& s, int b, int h) {
  return s.packed ? (int64_t)h * p.lse_total + s.qs : ((int64_t)b * p.H + h) * p.Nq;
}

// Work index of (batch, head) pair x < B * nh, decoded as b = bh / nh, h = bh % nh.
// The XCD remap hands every XCD a contiguous run of x. Where batch rows differ in cost,
// x is taken head-major (bh = (x % B) nh + x / B) so that a run spans every batch row of
// one head instead of a few rows of unequal cost: packed variable-length sequences, and
// block-sparse lists (LISTS), whose rows list different numbers of tiles. Other
// fixed-length grids keep x (every (b, h) costs the same).
template <bool LISTS>
__device__ __forceinline__ int work_bh(const AttnParams& p, int x, int nh) {
  return (LISTS || p.cu_q != nullptr) ? (x - (x / p.B) * p.B) * nh + x / p.B : x;
}

// ---------------------------------------------------------------------------------------
// Small device helpers.

// MI355X dispatches consecutive workgroups round-robin over its 8 XCDs, each with its
// own L2. Remapping the linear block id so that every XCD receives a contiguous run of
// work items keeps the key/value stream of one head inside one L2.
__device__ __forceinline__ int xcd_remap(int bid, int grid_padded) {
  const int per = grid_padded >> 3;
  return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// value of lane (l ^ 32)
__device__ __forceinline__ float swap_halves(float x) { return __shfl_xor(x, 32); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

// 8-byte transposed LDS read (see the layout note at the top of this file).
__device__ __forceinline__ u32x2 lds_read_tr(const void* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

__device__ __forceinline__ bf16x8 join_bf16x8(u32x2 lo, u32x2 hi) {
  u32x4 v = {lo[0], lo[1], hi[0], hi[1]};
  return __builtin_bit_cast(bf16x8, v);
}

// One matrix phase as a software pipeline over "items": NA accumulation items
// (acc[i / 4] += T^T bop[(i / 2) % 2][i % 2], one MFMA and two transposed 8-byte reads
// each) followed by NS score items (s[0], s[1] += R bf[ks]^T, two MFMAs and two 16-byte
// row reads each). The LDS reads of item i + AHEAD are issued right after the MFMAs of
// item i and the scheduler is fenced per item, so they stay in flight across the MFMAs
// instead of being sunk next to their use (left to itself the compiler keeps only one or
// two reads in flight and every MFMA waits out the LDS latency).
//   t0: the lane's first transposed-read address (row trow, column tcol of the T tile;
//       item (db, kb, hh) reads rows + 32 kb + 16 hh and + 4, columns + 32 db)
//   r0: the lane's first row-read address (permuted row, half g of the R tile; score
//       item ks reads 16-byte chunk 2 ks and the same 32 rows further)
// Either part may be absent (do_acc / do_s); s is cleared when do_s.
template <int NA, int NS, int TP, int RP, int AHEAD, int NACC, int NBF>
__device__ __forceinline__ void pipelined_matrix(const char* t0, const char* r0, bool do_acc, bool do_s,
                                                 f32x16 (&acc)[NACC], const bf16x8 (&bop)[2][2],
                                                 f32x16 (&s)[2], const bf16x8 (&bf)[NBF]) {
  struct Operand { bf16x8 a, b; };
  constexpr int N = NA + NS;
  auto load = [&](int i) {
    Operand op;
    if (i < NA) {
      const int db = i >> 2, kb = (i >> 1) & 1, hh = i & 1;
      const char* tp = t0 + (32 * kb + 16 * hh) * TP + 64 * db;
      const u32x2 lo = lds_read_tr(tp);
      const u32x2 hi = lds_read_tr(tp + 4 * TP);
      op.a = join_bf16x8(lo, hi);
    } else {
      const int ks = i - NA;
      op.a = *(const bf16x8*)(r0 + 32 * ks);
      op.b = *(const bf16x8*)(r0 + 32 * RP + 32 * ks);
    }
    return op;
  };
  auto run = [&](int i, const Operand& op) {
    if (i < NA) {
      const int db = i >> 2, kb = (i >> 1) & 1, hh = i & 1;
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.a, bop[kb][hh], acc[db], 0, 0, 0);
    } else {
      const int ks = i - NA;
      s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.a, bf[ks], s[0], 0, 0, 0);
      s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(op.b, bf[ks], s[1], 0, 0, 0);
    }
  };
  const int first = do_acc ? 0 : NA, last = do_s ? N : NA;
  if (do_s) {
    s[0] = f32x16{};
    s[1] = f32x16{};
  }
  Operand ring[AHEAD];
#pragma unroll
  for (int i = 0; i < N; ++i)
    if (i >= first && i < first + AHEAD && i < last) ring[i % AHEAD] = load(i);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i < first || i >= last) continue;
    __builtin_amdgcn_sched_barrier(0);
    run(i, ring[i % AHEAD]);
    if (i + AHEAD < last) ring[i % AHEAD] = load(i + AHEAD);
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Is key j visible from query i under the element mask (delta = Nk - Nq)?
__device__ __forceinline__ bool mask_visible(const MaskParams& m, int b, int i, int j, int nq,
                                             int nk) {
  const int d = nk - nq;
  switch (m.kind) {
    case kMaskCausal: return j <= i + d;
    case kMaskWindow: return j <= i + d && j >= i + d - m.window;
    case kMaskBlockDiag: return m.doc_q[(int64_t)b * nq + i] == m.doc_k[(int64_t)b * nk + j];
    case kMaskPrefix: return j < m.prefix || j <= i + d;
    default: return true;
  }
}

// Block-sparse list walking with defensive bounds: counts are clamped to [0, n_cols] and
// an entry outside [0, n_cols) maps to tile n_cols, which lies past the end of the
// sequence, so it is loaded as zeros and fully masked instead of being dereferenced.
__device__ __forceinline__ int clamp_count(int c, int n_cols) { return min(max(c, 0), n_cols); }
__device__ __forceinline__ int list_entry(const int* idx, int e, int n_cols) {
  const int t = idx[e];
  return (t >= 0 && t < n_cols) ? t : n_cols;
}

// Score transform applied to the scaled score x = scale * <q, k> (softcap, then bias).
// Returns the final score in log2 units; `dcap` receives d(softcap(x))/dx = 1 - tanh^2
// (1 without softcap), the factor the backward applies to dS.
// Softcap: with y = x / softcap, tanh(y) = 1 - 2 r, r = 1 / (exp(2 y) + 1), so the capped
// score in log2 units is softcap log2(e) (1 - 2 r) = cap_u - 2 cap_u r: one multiply, the
// exp2, an add, the reciprocal and one fma per score, the constants folded on the host
// (exp(2 y) = inf gives r = 0, tanh = 1; exp(2 y) = 0 gives r = 1, tanh = -1).
template <bool SOFTCAP, bool BIAS>
__device__ __forceinline__ float score_log2_d(float raw, const AttnParams& p, int i, int j, float& dcap) {
  float u;
  dcap = 1.0f;
  if constexpr (SOFTCAP) {
    const float r = fast_rcp(fast_exp2(raw * p.cap_k1) + 1.0f);
    u = __builtin_fmaf(r, -2.0f * p.cap_u, p.cap_u);
    const float th = __builtin_fmaf(r, -2.0f, 1.0f);
    dcap = __builtin_fmaf(-th, th, 1.0f);
  } else {
    u = raw * p.scale_log2;
  }
  if constexpr (BIAS) u += p.bias_log2 * (float)abs(i - j);
  return u;
}

template <bool SOFTCAP, bool BIAS>
__device__ __forceinline__ float score_log2(float raw, const AttnParams& p, int i, int j) {
  float dcap;
  return score_log2_d<SOFTCAP, BIAS>(raw, p, i, j, dcap);
}

// MFMA row permutation: swapping bits 2 and 3 of the A-operand row index makes the C
// registers 8 r' + i (i = 0..7) of lane half g hold rows 16 r' + 8 g + i, i.e. 8
// consecutive rows per lane, which is exactly the K-slot order of the next MFMA's
// B operand.
__device__ __forceinline__ int swap_bits23(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// One direct global->LDS load of 16 bytes per lane: lane i copies gbase + voff (bytes) to
// LDS bytes lds_block + 16 i. Issued through inline asm on purpose: the compiler would
// otherwise treat it as a store to every LDS location and wait for it (vmcnt(0)) before
// the next LDS read, even when that read targets a different tile, which serialises the
// prefetch with the MFMA phase. Callers order it explicitly instead: wait_lds_dma() and
// a barrier before the destination tile is read, and never read a tile while its DMA is
// in flight. M0 has no other user in these kernels. Here the bases are already
// wave-uniform (SGPR values): gu = global byte address, laddr = LDS byte address of the
// 1 KiB block; dma_16b below takes pointers instead.
__device__ __forceinline__ void dma_16b_u(uint64_t gu, uint32_t voff, uint32_t laddr) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"((const char*)(uintptr_t)gu), "s"(laddr) : "memory");
#endif
}

// Wave-uniform copies of a global pointer and of the LDS offset of an LDS pointer. Both
// must be wave-uniform by contract; readfirstlane makes that visible to the compiler where
// it cannot prove it (free when the value already sits in an SGPR).
__device__ __forceinline__ uint64_t uniform_addr(const void* gp) {
  const uint64_t ga = (uint64_t)(uintptr_t)gp;
  // readfirstlane returns int: go through uint32_t so the low word is zero-extended
  const uint32_t glo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ga);
  const uint32_t ghi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(ga >> 32));
  return ((uint64_t)ghi << 32) | (uint64_t)glo;
}
// (the flat address of an LDS location holds its LDS offset in the low 32 bits)
__device__ __forceinline__ uint32_t uniform_lds(const void* lp) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lp);
}

// Pointer form of dma_16b_u; gbase and lds_block must be wave-uniform.
__device__ __forceinline__ void dma_16b(const char* gbase, uint32_t voff, const char* lds_block) {
  dma_16b_u(uniform_addr(gbase), voff, uniform_lds(lds_block));
}

// s_waitcnt vmcnt(n) for a run-time n (wave-uniform); n above 15 waits for 15, which is
// stricter and therefore still correct.
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  switch (n) {
#define FMHA_VMCNT_CASE(k) case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
    FMHA_VMCNT_CASE(1) FMHA_VMCNT_CASE(2) FMHA_VMCNT_CASE(3) FMHA_VMCNT_CASE(4) FMHA_VMCNT_CASE(5)
    FMHA_VMCNT_CASE(6) FMHA_VMCNT_CASE(7) FMHA_VMCNT_CASE(8) FMHA_VMCNT_CASE(9) FMHA_VMCNT_CASE(10)
    FMHA_VMCNT_CASE(11) FMHA_VMCNT_CASE(12) FMHA_VMCNT_CASE(13) FMHA_VMCNT_CASE(14)
#undef FMHA_VMCNT_CASE
    default:
      if (n >= 15) asm volatile("s_waitcnt vmcnt(15)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      break;
  }
}

// Copies rows [row0, row0 + ROWS) of a row-strided bf16 matrix (D columns) into an LDS
// tile with a padded row pitch of PCH 16-byte chunks (PCH >= D/8), using direct
// global->LDS loads (global_load_lds_dwordx4). Each wave instruction fills 1 KiB of
// consecutive LDS, lane i writing bytes 16 i .. 16 i + 15. The per-lane global byte
// offsets (row * row_bytes + chunk * 16) are computed once (init). Every lane of every
// instruction loads, without branches: a lane on a pad slot, or on a row at or past
// `nrows` (a ragged last tile), loads offset 0 instead (row row0, which always exists),
// so its LDS slot receives finite data that callers never use unmasked (pad columns are
// never read; rows past the end are masked or multiplied by zero probabilities). Since
// chunk * 16 < row_bytes, "row < rows left" is "offset < rows left * row_bytes". Each
// tile therefore costs every wave exactly count() instructions, which keeps partial
// vmcnt waits exact. Data is visible to the workgroup after the wave's wait and a
// barrier. Requires ROWS * row_stride * 2 < 2^31 (checked on the host).
template <int ROWS, int D, int PCH, int NTHREADS>
struct LdsDma {
  static constexpr int CH = D / 8;
  static constexpr int NW = NTHREADS / 64;
  static constexpr int NBLK = ROWS * PCH / 64;                 // 1 KiB blocks in the tile
  static constexpr int NI = (NBLK + NW - 1) / NW;              // blocks per wave (max)
  static_assert(ROWS * PCH % 64 == 0, "padded tile must be whole 1 KiB blocks");
  static_assert(PCH >= CH, "pitch shorter than a row");
  uint32_t off[NI];
  int w;

  __device__ __forceinline__ void init(int64_t row_stride, int tid) {
    w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int blk = j * NW + w;
      const int L = blk * 64 + lane;
      const int r = L / PCH, c = L - (L / PCH) * PCH;
      off[j] = (blk < NBLK && c < CH) ? (uint32_t)(r * (int)(row_stride * 2) + c * 16) : 0u;
    }
  }
  // number of DMA instructions this wave issues per tile
  __device__ __forceinline__ int count() const { return (NBLK - w + NW - 1) / NW; }
  // wait until at most `tiles` tiles' worth of this wave's DMA (of this and `other`)
  // remain in flight (loads complete in order)
  template <class Other>
  __device__ __forceinline__ void wait_leaving(const Other& other, int tiles) const {
    wait_vmcnt_at_most(tiles * (count() + other.count()));
  }
  __device__ __forceinline__ void issue(const __bf16* g, int64_t row_stride, int row0, int nrows,
                                        char* lds_tile) const {
    issue_part<0, 1>(g, row_stride, row0, nrows, lds_tile);
  }
  // The instructions j with j % NPART == PART only: lets a caller spread one tile's loads
  // over several points of its code (issue every PART once per tile).
  template <int PART, int NPART>
  __device__ __forceinline__ void issue_part(const __bf16* g, int64_t row_stride, int row0, int nrows,
                                             char* lds_tile) const {
    const int left = nrows - row0;
    // bases made uniform once per call, not once per instruction
    const uint64_t base = uniform_addr(g + (int64_t)row0 * row_stride);
    const uint32_t lbase = uniform_lds(lds_tile) + (uint32_t)w * 1024u;
    const int cnt = __builtin_amdgcn_readfirstlane(count());   // scalar: blocks of this wave
    if (left >= ROWS) {
#pragma unroll
      for (int j = PART; j < NI; j += NPART) {
        if (j >= cnt) break;
        dma_16b_u(base, off[j], lbase + (uint32_t)(j * NW) * 1024u);
      }
    } else {
      const uint32_t lim = (uint32_t)(left * (int)(row_stride * 2));
#pragma unroll
      for (int j = PART; j < NI; j += NPART) {
        if (j >= cnt) break;
        dma_16b_u(base, off[j] < lim ? off[j] : 0u, lbase + (uint32_t)(j * NW) * 1024u);
      }
    }
  }
};

// Zero `bytes` (a multiple of 16) of LDS with the whole workgroup; followed by a barrier.
template <int NTHREADS>
__device__ __forceinline__ void zero_lds(char* lds, int bytes, int tid) {
  for (int o = tid * 16; o < bytes; o += NTHREADS * 16) *(u32x4*)(lds + o) = u32x4{};
  __syncthreads();
}

// Wait until this wave's direct global->LDS loads have landed (vmcnt = 0). The asm form
// is invisible to the compiler's wait-count tracking; wait_all_vmem() is the builtin form,
// which also tells the compiler that every earlier vector-memory load has completed
// (use it once before a loop, so the loop does not re-wait for loads issued before it).
__device__ __forceinline__ void wait_lds_dma() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void wait_all_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Reductions over the two lanes (l, l ^ 32) that share a row, with v_permlane32_swap.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// DPP controls (gfx9 encoding) and a sum over groups of 8 or 16 consecutive lanes that
// stays inside one 16-lane DPP row (no LDS traffic).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

template <int LPK>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(LPK == 8 || LPK == 16, "group of 8 or 16 lanes");
  x += dpp_mov<kDppXor1>(x);
  x += dpp_mov<kDppXor2>(x);
  x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (LPK == 16) x += dpp_mov<kDppRowMirror>(x);
  return x;
}

__device__ __forceinline__ void bf16x2_to_f32(uint32_t x, float* f) {
  f[0] = __uint_as_float(x << 16);
  f[1] = __uint_as_float(x & 0xFFFF0000u);
}

__device__ __forceinline__ void bf16x8_to_f32(const u32x4& x, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __uint_as_float(x[e] << 16);
    f[2 * e + 1] = __uint_as_float(x[e] & 0xFFFF0000u);
  }
}

// Visible keys of query row i under the band masks (none, causal, sliding window,
// prefix-LM) form one interval [lo, hi); block-diagonal is handled separately.
__device__ __forceinline__ void band_interval(const MaskParams& m, int i, int nq, int nk, int& lo, int& hi) {
  const int d = nk - nq;
  lo = 0;
  hi = nk;
  if (m.kind == kMaskCausal || m.kind == kMaskWindow) hi = min(nk, i + d + 1);
  if (m.kind == kMaskWindow) lo = i + d - m.window;
  if (m.kind == kMaskPrefix) hi = min(nk, max(m.prefix, i + d + 1));
}

// Set to -inf the entries of a 32-query x 64-key S^T tile (lane = query row, the layout of
// S^T = K Q^T with permuted K rows) whose key is hidden from the lane's query row.
// Register r of block kb holds key kbase + 32 kb + 16 (r / 8) + r % 8 (kbase = tile start
// + 8 g). Keys lo <= j < hi stay visible (an interval computed once per row).
__device__ __forceinline__ void mask_tile_band(f32x16 (&s)[2], int kbase, int lo, int hi) {
  // key j visible iff lo <= j < hi, i.e. (unsigned)(j - lo) < (unsigned)(hi - lo)
  const unsigned span = hi > lo ? (unsigned)(hi - lo) : 0u;
  const int base = kbase - lo;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const unsigned rel = (unsigned)(base + 32 * kb + 16 * (r >> 3) + (r & 7));
      s[kb][r] = rel < span ? s[kb][r] : kNegInf;
    }
}

// Document (block-diagonal) variant: key j visible iff j < nk and its document is dq.
// The lane's keys are four runs of 8: kbase + 32 kb + 16 h + e. With VEC, when every
// lane's runs are in bounds and 16-byte aligned (one ballot keeps the branch wave-uniform),
// their document ids come in 8 vector loads instead of 32 scalar ones; the 32 ids then in
// flight cost registers, so a kernel at its register limit passes VEC = false.
template <bool VEC>
__device__ __forceinline__ void mask_tile_doc(f32x16 (&s)[2], const int* doc_k, int dq, int kbase, int nk) {
  const bool wide = VEC && kbase + 56 <= nk && ((reinterpret_cast<uintptr_t>(doc_k + kbase) & 15) == 0);
  if (VEC && __builtin_amdgcn_ballot_w64(!wide) == 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int4 a = *(const int4*)(doc_k + kbase + 32 * kb + 16 * h);
        const int4 c = *(const int4*)(doc_k + kbase + 32 * kb + 16 * h + 4);
        const int d[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) s[kb][8 * h + e] = d[e] == dq ? s[kb][8 * h + e] : kNegInf;
      }
    return;
  }
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int j = kbase + 32 * kb + 16 * (r >> 3) + (r & 7);
      const bool vis = (j < nk) & (doc_k[min(j, nk - 1)] == dq);   // unconditional (clamped) load
      s[kb][r] = vis ? s[kb][r] : kNegInf;
    }
}

// Document ids of the 8 consecutive positions j0 .. j0 + 7 of a row of n ids. WIDE
// promises j0 + 8 <= n and doc + j0 16-byte aligned: two vector loads; otherwise eight
// scalar loads clamped to the row (the caller masks j >= n itself).
template <bool WIDE>
__device__ __forceinline__ void doc_ids8(const int* doc, int j0, int n, int (&d)[8]) {
  if constexpr (WIDE) {
    const int4 a = *(const int4*)(doc + j0), c = *(const int4*)(doc + j0 + 4);
    d[0] = a.x, d[1] = a.y, d[2] = a.z, d[3] = a.w;
    d[4] = c.x, d[5] = c.y, d[6] = c.z, d[7] = c.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) d[e] = doc[min(j0 + e, n - 1)];
  }
}

// Tiles of a row band that need the element mask: with tile start n0 (a multiple of
// `tile`), the mask can hide something only if n0 > above or n0 < below. Computed once
// per wave from the band masks' geometry for rows [r0, r0 + 32) (n_other = the column
// side's length, delta = Nk - Nq), so the per-tile test is two scalar compares.
// Columns here are keys (forward and dQ passes).
__device__ __forceinline__ void key_tile_need(const MaskParams& m, int r0, int nk, int delta, int tile,
                                              int& above, int& below) {
  above = nk - tile;            // ragged last tile
  below = INT32_MIN;
  if (m.kind == kMaskCausal || m.kind == kMaskWindow) above = min(above, r0 + delta - tile + 1);
  if (m.kind == kMaskPrefix) above = min(above, max(r0 + delta - tile + 1, m.prefix - tile));
  if (m.kind == kMaskWindow) below = r0 + 31 + delta - m.window;
  if (m.kind == kMaskBlockDiag) above = -1;
}

// ---------------------------------------------------------------------------------------
// Block-sparse tile sequences.
//
// A workgroup walks the tiles of one or two sparse rows (its "halves": the forward and
// dQ passes cover 256 query rows = two 128-row halves, the dK/dV pass one row of keys).
// The listed columns of those rows are merged into one ascending sequence of UNIT-wide
// kernel tiles in LDS. Entry = (kernel tile << 4) | class bits, the class of half hf in
// bits 2 hf, 2 hf + 1: 1 = partial (element mask applies), 2 = full, 0 = not listed for
// that half (all of its elements hidden). Lists are sets: a repeated entry counts once, a
// column listed both partial and full is full, entries outside [0, n_cols) are dropped,
// and so are kernel tiles at or past n_elems (the column side's length).

// LDS bytes of a merged sequence: count word (16 bytes), entries, class words.
__host__ __device__ inline int tile_sequence_bytes(const ListParams& L, int unit) {
  return 16 + 4 * (L.n_cols * (L.tile_cols / unit) + (L.n_cols + 3) / 4);
}

// row0 / row1: flattened index into the [B, heads, n_rows] count arrays of each half, or
// -1 for an absent half. `lds` points at tile_sequence_bytes(L, UNIT) bytes. Contains
// barriers: every thread of the workgroup must call it. Returns the sequence length.
template <int NTHREADS, int UNIT>
__device__ int build_tile_sequence(const ListParams& L, int64_t row0, int64_t row1, int n_elems, char* lds,
                                   int tid) {
  int* total = (int*)lds;
  uint32_t* ent = (uint32_t*)(lds + 16);
  const int sub = L.tile_cols / UNIT;
  uint32_t* cls = ent + L.n_cols * sub;
  const int ncw = (L.n_cols + 3) >> 2;
  for (int i = tid; i < ncw; i += NTHREADS) cls[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    const int64_t row = hf ? row1 : row0;
    if (row < 0) continue;
#pragma unroll
    for (int kind = 0; kind < 2; ++kind) {   // 0: partial list, 1: full list
      const int cnt = clamp_count((kind ? L.fcnt : L.pcnt)[row], L.n_cols);
      const int* idx = (kind ? L.fidx : L.pidx) + row * L.n_cols;
      const uint32_t code = (kind ? 2u : 1u) << (2 * hf);
      for (int e = tid; e < cnt; e += NTHREADS) {
        const int c = idx[e];
        if (c >= 0 && c < L.n_cols) atomicOr(&cls[c >> 2], code << (8 * (c & 3)));
      }
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int nkt = (n_elems + UNIT - 1) / UNIT;   // kernel tiles holding at least one element
    int base = 0;
    for (int c0 = 0; c0 < L.n_cols; c0 += 64) {
      const int c = c0 + tid;
      uint32_t v = c < L.n_cols ? (cls[c >> 2] >> (8 * (c & 3))) & 15u : 0u;
      v = v & ~((v & 10u) >> 1);   // partial and full for the same half: full
      const uint64_t m = __builtin_amdgcn_ballot_w64(v != 0u);
      const int pre = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      if (v != 0u) {
        // the kernel tiles of one column are consecutive slots: the sequence stays ascending
        for (int s = 0; s < sub; ++s) {
          const int kt = c * sub + s;
          if (kt < nkt) ent[(base + pre) * sub + s] = ((uint32_t)kt << 4) | v;
        }
      }
      base += __builtin_popcountll(m);
    }
    if (tid == 0) {
      // only the last column can hold kernel tiles at or past n_elems
      const int cl = L.n_cols - 1;
      const bool last_listed = cl >= 0 && ((cls[cl >> 2] >> (8 * (cl & 3))) & 15u) != 0u;
      *total = base * sub - (last_listed ? L.n_cols * sub - nkt : 0);
    }
  }
  __syncthreads();
  return *total;
}

// Longest walks first under block-sparse lists. The n resident tiles of one (batch, mask
// head) are ranked by how many sparse tiles their list rows name (descending, ties by
// index), and workgroup t of them takes the tile of rank t, so the longest walks start in
// the first dispatch round and the short ones fill in behind them. Tile j covers elements
// [j span, (j + 1) span) of the list side: its row holds element j span and, with
// half > 0, also element j span + half when that lies in bounds and in another list row
// (the forward's two 128-row halves). The rank is a heuristic of the dispatch order
// only; results do not depend on it. `lds` holds n + 1 ints. The ranking costs
// O(n^2 / NTHREADS) LDS compares per workgroup (about 1-2 us at n = 512), so above
// kMaxRankedTiles the natural order j = t is kept: there a workgroup's share of a short
// walk would go to ranking. Contains barriers: every thread of the workgroup calls it.
constexpr int kMaxRankedTiles = 512;
template <int NTHREADS>
__device__ int ranked_tile(const ListParams& L, int64_t rbase, int n, int span, int half, int n_elems, int t,
                           int* lds, int tid) {
  if (n > kMaxRankedTiles) return t;
  for (int j = tid; j < n; j += NTHREADS) {
    const int e0 = j * span;
    const int64_t r0 = rbase + e0 / L.tile_rows;
    int c = clamp_count(L.pcnt[r0], L.n_cols) + clamp_count(L.fcnt[r0], L.n_cols);
    if (half > 0 && e0 + half < n_elems && (e0 + half) / L.tile_rows != e0 / L.tile_rows) {
      const int64_t r1 = rbase + (e0 + half) / L.tile_rows;
      c += clamp_count(L.pcnt[r1], L.n_cols) + clamp_count(L.fcnt[r1], L.n_cols);
    }
    lds[j] = c;
  }
  __syncthreads();
  for (int j = tid; j < n; j += NTHREADS) {
    const int cj = lds[j];
    int rank = 0;
    for (int k = 0; k < n; ++k) {
      const int ck = lds[k];
      rank += (ck > cj) | ((ck == cj) & (k < j));
    }
    if (rank == t) lds[n] = j;   // exactly one j has rank t (ranks are a permutation)
  }
  __syncthreads();
  const int r = lds[n];
  __syncthreads();   // every thread has read the result: the caller may reuse `lds`
  return r;
}

// Key / query tile walk of one workgroup: an analytic run of tiles, or a merged sequence.
template <int UNIT>
struct TileSeq {
  int count;
  int t_lo;               // analytic: first tile
  const uint32_t* ent;    // lists: LDS entries
  __device__ __forceinline__ int start(int it, bool lists) const {
    return lists ? (int)(ent[it] >> 4) * UNIT : (t_lo + it) * UNIT;
  }
  // class bits (2) of half hf; analytic walks report "full" (masking is decided by range)
  __device__ __forceinline__ uint32_t cls(int it, int hf, bool lists) const {
    return lists ? (ent[it] >> (2 * hf)) & 3u : 2u;
  }
};

}  // namespace fmha
