/*
 * fmha.h -- C ABI of libfmha.so: fused, tiled, masked scaled-dot-product attention
 * with online softmax for AMD Instinct MI355X (CDNA4, gfx950).
 *
 * What is computed (per batch b, head h; i = query row, j = key column,
 * delta = Nk - Nq):
 *
 *   S[i,j] = scale * <q_i, k_j>
 *   S[i,j] = softcap * tanh(S[i,j] / softcap)         if softcap > 0
 *   S[i,j] = S[i,j] + bias_slope * |i - j|             (relative bias; 0 = off)
 *   S[i,j] = -inf where the mask hides key j from query i
 *   O_i    = sum_j softmax_j(S[i,:]) v_j,   LSE_i = ln sum_j exp(S[i,j])
 *   A row with no visible key gets O_i = 0 and LSE_i = -inf.
 *
 * Sources (web pages, cited by title and section):
 *   "Enable 2CTA for SM100 block-sparse backward" (flash-attention pull request 2661),
 *     section "Testing Testing Testing": the fuzz tester's forward call (q, k, v, out,
 *     lse, softmax_scale = 1/sqrt(headdim), causal, softcap, window sizes, score_mod,
 *     mask_mod, block_sparse_tensors, return_lse), its backward call (q, k, v, out,
 *     dout, lse -> dq, dk, dv), its mask names (causal, sliding_window,
 *     block_diagonal, prefix_lm), the relative-bias score mod whose backward passes
 *     the gradient through, and the separate forward / backward block-sparse tensors
 *     with sparse tile sizes decoupled from the kernel tile ("Summary").
 *   "Optimize Flash Dynamic Mask Attention Kernel Configurations" (flash-sparse-attention
 *     pull request 148), sections "Changes Made" and "Testing": split-KV forward with
 *     1/2/4/8/16 splits, a deterministic backward, softcap, and a central diagnostic
 *     for unsupported architectures.
 *   POPCORNBENCH transcript "Kimi-K2.6 l1 p97": the math-backend definition
 *     softmax(Q K^T * scale) V and the two-chunk online-softmax merge rule used by the
 *     streaming kernels and the split-KV combine.
 *
 * Mask predicates (readings where the pages name a mask without defining it):
 *   FMHA_MASK_NONE            every key visible
 *   FMHA_MASK_CAUSAL          j <= i + delta            (bottom-right aligned)
 *   FMHA_MASK_SLIDING_WINDOW  i + delta - window <= j <= i + delta (both ends inclusive)
 *   FMHA_MASK_BLOCK_DIAGONAL  doc_q[b][i] == doc_k[b][j]
 *   FMHA_MASK_PREFIX_LM       j < prefix  or  j <= i + delta
 *
 * Conventions for every entry point:
 *   - Every pointer inside an argument struct is a DEVICE pointer unless stated; the
 *     argument structs themselves are host memory, read during the call only.
 *   - The caller owns and allocates every device buffer (outputs, LSE, workspaces,
 *     index lists). The library never allocates or frees device memory and keeps no
 *     state between calls.
 *   - All work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the null
 *     stream). Outputs are valid once the stream has reached that point.
 *   - Arguments are validated on the host before anything is launched; an invalid or
 *     unsupported request returns a negative fmha_status and launches nothing. A
 *     failed launch returns FMHA_ERR_HIP. Nothing is thrown across the ABI.
 *   - Only gfx950 devices are accepted (FMHA_ERR_UNSUPPORTED otherwise).
 */
#ifndef FMHA_H_
#define FMHA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FMHA_OK = 0,
  FMHA_ERR_INVALID_ARG = -1,   /* null pointer, bad shape/stride/size, inconsistent lists */
  FMHA_ERR_UNSUPPORTED = -2,   /* valid request the library does not implement, or not gfx950 */
  FMHA_ERR_HIP = -3,           /* a HIP runtime call or kernel launch failed */
  FMHA_ERR_WORKSPACE = -4,     /* workspace missing or smaller than the *_workspace_size */
  FMHA_ERR_SCRATCH_TOO_SMALL = -5  /* request needs more than the library-owned scratch of a
                                      no-allocation entry point */
} fmha_status;

typedef enum { FMHA_BF16 = 0, FMHA_FP32 = 1 } fmha_dtype;

typedef enum {
  FMHA_MASK_NONE = 0,
  FMHA_MASK_CAUSAL = 1,
  FMHA_MASK_SLIDING_WINDOW = 2,
  FMHA_MASK_BLOCK_DIAGONAL = 3,
  FMHA_MASK_PREFIX_LM = 4
} fmha_mask_kind;

/* Element mask. doc_q / doc_k are device int32 arrays [B, Nq] / [B, Nk] (contiguous),
 * read only for FMHA_MASK_BLOCK_DIAGONAL. */
typedef struct {
  int32_t kind;        /* fmha_mask_kind */
  int32_t window;      /* W >= 0 for SLIDING_WINDOW */
  int32_t prefix;      /* P >= 0 for PREFIX_LM */
  int32_t reserved;    /* must be 0 */
  const int32_t* doc_q;
  const int32_t* doc_k;
} fmha_mask;

/* Block-sparse tile mask (device int32 arrays, contiguous, caller-allocated).
 * The sparse tile is tile_m x tile_n elements; n_q_tiles = ceil(Nq/tile_m),
 * n_kv_tiles = ceil(Nk/tile_n); heads = 1 (one mask broadcast over every head) or H.
 *   Forward lists, per (b, mask head, query tile):
 *     partial_cnt [B, heads, n_q_tiles], partial_idx [B, heads, n_q_tiles, n_kv_tiles]
 *     full_cnt    [B, heads, n_q_tiles], full_idx    [B, heads, n_q_tiles, n_kv_tiles]
 *   Backward (transposed) lists, per (b, mask head, key tile):
 *     t_partial_cnt [B, heads, n_kv_tiles], t_partial_idx [B, heads, n_kv_tiles, n_q_tiles]
 *     t_full_cnt    [B, heads, n_kv_tiles], t_full_idx    [B, heads, n_kv_tiles, n_q_tiles]
 *   Index rows hold `cnt` tile indices followed by -1 padding (build_block_mask writes
 *   them ascending; the forward accepts any order).
 * A FULL tile is attended without the element mask, a PARTIAL tile applies the
 * element mask (fmha_mask), an unlisted tile is skipped. Entries outside the tile range
 * are ignored. The forward treats lists as sets (a repeated entry counts once, a tile in
 * both lists of a row is FULL); the backward requires each tile at most once per row
 * over both lists, as build_block_mask writes them. Rows and columns past Nq / Nk are
 * always excluded.
 * Kernel granularity (FMHA_ERR_UNSUPPORTED otherwise): forward tile_m % 128 == 0 and
 * tile_n % 64 == 0, with n_kv_tiles * tile_n / 64 small enough for the merged tile
 * sequence of a 256-query workgroup to fit in LDS next to the K/V stages (about 3000
 * 64-key tiles at D = 128); backward tile_m % 128 == 0 and tile_n % 128 == 0. */
typedef struct {
  int32_t tile_m, tile_n;
  int32_t n_q_tiles, n_kv_tiles;
  int32_t heads;
  int32_t reserved;    /* must be 0 */
  int32_t *partial_cnt, *partial_idx, *full_cnt, *full_idx;
  int32_t *t_partial_cnt, *t_partial_idx, *t_full_cnt, *t_full_idx;
} fmha_block_sparse;

/* Forward problem. Q [B,Nq,H,Dqk], K [B,Nk,Hkv,Dqk], V [B,Nk,Hkv,Dv], O [B,Nq,H,Dv] are
 * addressed with element strides {batch, seq, head}; the head dim is contiguous
 * (so BSHD and BHSD both work). Rows (seq-stride * elem size) must be 16-byte aligned,
 * and 64 rows must span less than 2^31 bytes (FMHA_ERR_UNSUPPORTED otherwise).
 * LSE is fp32 [B, H, Nq] contiguous. dtype applies to Q, K, V and O.
 * Supported (dtype, Dqk, Dv): bf16 (64,64), (128,128), (192,128); fp32 (64,64),
 * (128,128), (1024,1024) (fp32: no block-sparse lists, no softcap/bias). */
typedef struct {
  int32_t B, H, Nq, Nk, Dqk, Dv;
  int32_t dtype;       /* fmha_dtype */
  int32_t kv_heads;    /* Hkv: K/V heads, 0 (= H) or a divisor of H. Grouped-query
                          attention: query head h reads K/V head h / (H / Hkv) (the grouping
                          of the reference call with enable_gqa in "Enable 2CTA for SM100
                          block-sparse backward", section "Testing Testing Testing").
                          Every entry point accepts Hkv != H; the backward then sums each
                          group's query heads into dK / dV in a fixed order, and takes
                          block-sparse lists only with heads == 1 (FMHA_ERR_UNSUPPORTED
                          otherwise). Not dividing H, or negative: FMHA_ERR_INVALID_ARG. */
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_stride[3];
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
  float scale;         /* > 0; the usual value is 1/sqrt(Dqk) */
  float softcap;       /* 0 = off */
  float bias_slope;    /* 0 = off */
  int32_t reserved2;   /* must be 0 */
  fmha_mask mask;
  const fmha_block_sparse* block_sparse; /* host pointer to the list descriptor, or NULL
                                            for analytic tile ranges from `mask` */
} fmha_fwd_args;

/* Backward buffers. dO, dQ, dK, dV are bf16 with the shapes of O, Q, K, V and element
 * strides {batch, seq, head}. */
typedef struct {
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  int64_t do_stride[3];
  int64_t dq_stride[3];
  int64_t dk_stride[3];
  int64_t dv_stride[3];
  void* workspace;             /* >= fmha_bwd_workspace_size(B, H, Nq) bytes */
  size_t workspace_bytes;
  void* const* stage_events;   /* optional host array of 4 hipEvent_t (or NULL): recorded on
                                  `stream` before the preprocess, dK/dV and dQ kernels and
                                  after the dQ kernel, for per-kernel timing. No work is
                                  skipped or reordered. */
} fmha_bwd_args;

/* Forward: writes O and LSE. Tiles listed as empty (block-sparse) or outside the
 * causal / window band are skipped; masks are evaluated only where a tile straddles
 * the band edge or is listed as partial. */
int fmha_fwd(const fmha_fwd_args* args, void* stream);

/* Forward with an optional workspace, for launches that leave CUs idle: a short query side
 * against a long key range (chunked prefill), or few heads with a causal mask, whose
 * longest 256-row query tile walks many more key tiles than the others. When the bf16
 * forward (no block-sparse lists, Dqk == Dv in {64, 128}) would launch fewer workgroups
 * than the GPU has CUs (B * H * ceil(Nq / 256) < 256), the long query tiles' key ranges
 * are walked in contiguous parts of T key tiles (64 keys each), one workgroup per part;
 * each part writes its normalised partial O and LSE to the workspace, and a combine merges
 * the parts of each tile with the LSE-weighted rule of fmha_fwd_splitkv (the two-chunk
 * online-softmax merge of the POPCORNBENCH transcript "Kimi-K2.6 l1 p97"). The library
 * picks the number of parts (2-16, all running at once on the CUs) from a measured cost
 * model, or none when a split would not pay. The result is the same attention as
 * fmha_fwd within the bf16 tolerance, not bit-identical to it, and deterministic.
 * fmha_fwd_workspace_size returns the bytes this needs for `args` (0 when no split
 * applies, or for invalid args); with a NULL workspace, or one smaller than that, the call
 * is exactly fmha_fwd. The workspace is owned by the caller, device memory, 256-byte
 * aligned (FMHA_ERR_INVALID_ARG otherwise), and must not be used by another call until
 * this one has finished on `stream`. */
size_t fmha_fwd_workspace_size(const fmha_fwd_args* args);
int fmha_fwd_with_workspace(const fmha_fwd_args* args, void* workspace, size_t workspace_bytes,
                            void* stream);

/* Backward from the saved LSE: reads args->q, k, v, o, lse and bwd->dout; writes dQ,
 * dK, dV. bf16 only. Deterministic: no atomics; every gradient element has a single
 * writer and a fixed summation order, so repeated calls give bitwise-identical
 * results. With block-sparse lists the transposed lists drive the dK/dV pass.
 * One empty side is allowed: Nk == 0 writes dQ = 0, Nq == 0 writes dK = dV = 0 (the
 * empty side's pointers may then be NULL). */
size_t fmha_bwd_workspace_size(int32_t B, int32_t H, int32_t Nq);
int fmha_bwd(const fmha_fwd_args* args, const fmha_bwd_args* bwd, void* stream);

/* Split-KV forward for long keys and few queries (decode): the key range is cut into
 * num_splits contiguous, 64-key-aligned chunks of ceil(ceil(Nk/64)/num_splits) tiles;
 * each chunk produces a normalised partial (O_s, LSE_s) in the workspace, then a
 * combine kernel merges them: LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
 * bf16 only, no block-sparse lists, 1 <= num_splits <= 64. Accepts grouped K/V heads
 * (args->kv_heads): the query heads of one group (up to 4 per workgroup, or the whole group
 * as the rows of one matrix product when heads x Nq <= 32 and it has 8 or more heads, or
 * 4-7 with at least 1024 keys per split)
 * stream each K/V row of the group once from memory. The workspace is sized by query heads H. */
size_t fmha_fwd_splitkv_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t Dv,
                                       int32_t num_splits);
int fmha_fwd_splitkv(const fmha_fwd_args* args, int32_t num_splits, void* workspace,
                     size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): fmha_fwd_splitkv with its partials in
 * a library-owned device buffer instead of a caller workspace. The buffer is a fixed
 * fmha_fwd_splitkv_noalloc_max_bytes() (16 MiB) per GPU, held from the first call on that
 * GPU until the process ends; requests whose partials need more
 * (fmha_fwd_splitkv_workspace_size(B, H, Nq, Dv, num_splits) bytes) return
 * FMHA_ERR_SCRATCH_TOO_SMALL before anything is launched. Nothing is allocated by the call.
 * Every call on one GPU uses the same buffer: calls whose executions overlap on one GPU
 * (different streams, or different host threads without ordering) race and must not be
 * issued; calls ordered on one stream are safe. The buffer keeps the last call's partials;
 * each call writes every entry it reads, so nothing needs clearing. Arguments and results
 * otherwise as fmha_fwd_splitkv. */
size_t fmha_fwd_splitkv_noalloc_max_bytes(void);
int fmha_fwd_splitkv_noalloc(const fmha_fwd_args* args, int32_t num_splits, void* stream);

/* Packed variable-length sequences ("Enable 2CTA for SM100 block-sparse backward",
 * section "Testing Testing Testing": the forward call's cu_seqlens_q / cu_seqlens_k and
 * seqused_q / seqused_k arguments). Sequence b (0 <= b < args->B) owns the span of query
 * rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) and key rows [cu_seqlens_k[b], cu_seqlens_k[b+1])
 * of Q [total_q, H, Dqk], K / V [total_k, Hkv, D*] and O [total_q, H, Dv], addressed with the
 * seq and head strides of fmha_fwd_args (its batch strides are ignored). The offset arrays
 * are device int32 [B + 1], ascending, starting at 0.
 * seqused_q / seqused_k (device int32 [B], or NULL = the whole span): only the first
 * seqused_q[b] query rows and seqused_k[b] key rows of each span take part; the sequence is
 * then the problem of those lengths (masks and positions as below), and rows of a span past
 * its used length are neither read nor written (their O / LSE / dQ / dK / dV keep whatever
 * the caller's buffers held). The pages pass these arguments without defining them; this is
 * the plain reading of "used" lengths. A used length outside [0, span] is clamped to it.
 * Every array here is read on the device only, so the caller guarantees that every used
 * query length (the span, or seqused_q[b]) is <= args->Nq, every used key length is
 * <= args->Nk, and every row lies inside the tensors.
 * Masks apply within each sequence (delta = that sequence's key length minus its query
 * length, after seqused). LSE is fp32 [H, total_q]. */
typedef struct {
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_k;
  int32_t total_q;     /* cu_seqlens_q[B] */
  int32_t reserved;    /* must be 0 */
  const int32_t* seqused_q;   /* [B] or NULL */
  const int32_t* seqused_k;   /* [B] or NULL */
} fmha_varlen;

/* Forward over packed variable-length sequences: as fmha_fwd with args->B sequences of at
 * most args->Nq queries and args->Nk keys. bf16 only; causal, sliding-window, prefix-LM or
 * no mask (block-diagonal masks and block-sparse lists: FMHA_ERR_UNSUPPORTED; each
 * sequence already is one document); softcap and relative bias as in fmha_fwd (i, j are
 * positions within the sequence). */
int fmha_fwd_varlen(const fmha_fwd_args* args, const fmha_varlen* varlen, void* stream);

/* Backward over packed variable-length sequences: as fmha_bwd, with the sequences, masks
 * and LSE layout of fmha_fwd_varlen (dO, dQ, dK, dV are packed like O, Q, K, V). The
 * workspace is fmha_bwd_workspace_size(B, H, args->Nq) with args->Nq the longest query
 * sequence. Keys of a sequence without queries get dK = dV = 0, queries of a sequence
 * without keys dQ = 0 (also when total_q is 0). Block-diagonal masks and block-sparse
 * lists: FMHA_ERR_UNSUPPORTED. */
int fmha_bwd_varlen(const fmha_fwd_args* args, const fmha_bwd_args* bwd, const fmha_varlen* varlen,
                    void* stream);

/* Block-sparse tile mask builder: classifies every (tile_m x tile_n) tile of the
 * element mask as empty / partial / full by counting visible in-bounds elements, and
 * writes the forward and transposed index lists into the caller-allocated arrays of
 * `out` (sizes as documented at fmha_block_sparse, for `Hm` mask heads). Fills
 * out->tile_m, tile_n, n_q_tiles, n_kv_tiles, heads on the host. The mask kinds
 * here do not depend on the head, so every mask head gets the same lists. */
int build_block_mask(const fmha_mask* mask, int32_t B, int32_t Hm, int32_t Nq, int32_t Nk,
                     int32_t tile_m, int32_t tile_n, fmha_block_sparse* out, void* stream);

/* Human-readable name of a status code (static storage). */
const char* fmha_status_string(int status);

/* ABI version: bumped whenever a struct layout or the set of entry points changes. */
int fmha_abi_version(void);   /* 4: fmha_fwd_workspace_size / fmha_fwd_with_workspace (3: fmha_varlen.seqused_q /
                                 seqused_k; 2: kv_heads, varlen entry points) */

#ifdef __cplusplus
}
#endif

#endif /* FMHA_H_ */
