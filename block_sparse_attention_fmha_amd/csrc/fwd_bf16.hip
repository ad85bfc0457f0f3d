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
//   * workgroup = 8 wavefronts (2 per SIMD), 256 query rows (32 per wave), 64-key tiles.
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
//   * ping-pong: the two waves sharing a SIMD (wave w and w + 4) alternate between a
//     matrix phase (S(j+1) = K(j+1) Q^T and O += V(j) P(j): 32 MFMAs) and a vector phase
//     (mask, online softmax, P(j+1) in bf16), one phase apart, with a workgroup barrier
//     once per tile (two phases). While one wave feeds the matrix core the other runs its softmax, so the
//     VALU work hides behind the MFMA work instead of serialising with it.
//   * K and V tiles live in 3 LDS stages filled by direct global->LDS loads
//     (global_load_lds_dwordx4, no VGPR staging) issued two phases before first use;
//     padded row pitches keep the 16-byte K row reads and the transposed V reads free
//     of bank conflicts.
//   * the running max is updated lazily: the O / l rescale by exp(m_old - m_new) runs
//     (a wave-uniform branch) only when some row's tile max exceeds the running max by
//     more than 2^8 in probability; otherwise the stale max stays, every p is at most
//     256, and O and l remain consistently scaled. The row sum adds the fp32
//     probabilities whose bf16 roundings feed the MFMA.
//   * the work item order is XCD-aware (each XCD gets a contiguous run of heads) and,
//     for causal-like masks, longest-first over query tiles.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kBM = 256;   // query rows per workgroup
constexpr int kBN = 64;    // keys per tile
constexpr int kThreads = 512;
constexpr int kCUs = 256;           // compute units of the GPU the key split balances over
constexpr int kMaxKeyParts = 16;    // most key parts one query tile is split into
constexpr int kMinPartTiles = 4;    // shortest key part worth a workgroup of its own
constexpr double kSplitFixedUs = 5.0;    // key split: combine launch and fixed cost
constexpr double kSplitUsPerMiB = 0.9;   // key split: per MiB of fp32 partial O
constexpr float kRescaleLog2 = 8.0f;   // stale-max tolerance of the online softmax (log2 units)
// LDS stages of (K, V) tiles: tile t is loaded 2 * stages - 4 phases before first use.
template <int DQK> struct Stages { static constexpr int value = (DQK <= 128) ? 4 : 3; };

// LDS row pitches in 16-byte chunks. K rows are read 16 bytes per lane from 16
// different rows at once: a pitch of 4 * odd dwords (mod 64 banks) puts them on disjoint
// banks. V is read with the transposed 8-byte read (4 rows x 32 bytes per 16-lane group):
// a pitch of 16 or 48 dwords (mod 64) puts those 4 row segments on disjoint banks. Every
// LDS address is then one base register plus immediates.
template <int D> struct KPitchChunks { static constexpr int value = D / 8 + 1; };
template <int D> struct VPitchChunks { static constexpr int value = (D == 64) ? 12 : 20; };

template <int DQK, int DV>
struct FwdSmem {
  static constexpr int KPC = KPitchChunks<DQK>::value;
  static constexpr int VPC = VPitchChunks<DV>::value;
  static constexpr int KP = KPC * 16;          // bytes
  static constexpr int VP = VPC * 16;
  static constexpr int KB = kBN * KP;
  static constexpr int VB = kBN * VP;
  static constexpr int STAGE = KB + VB;
  static constexpr int NST = Stages<DQK>::value;
  static constexpr int BYTES = NST * STAGE;
};

// Max of the 32 S^T entries of a lane as a depth-4 tree of v_max3.
__device__ __forceinline__ float tree_max32(const f32x16 (&s)[2]) {
  float a[11];
#pragma unroll
  for (int i = 0; i < 10; ++i) {
    const int x = 3 * i, y = 3 * i + 1, z = 3 * i + 2;
    a[i] = fmaxf(fmaxf(s[x >> 4][x & 15], s[y >> 4][y & 15]), s[z >> 4][z & 15]);
  }
  a[10] = fmaxf(s[1][14], s[1][15]);
  const float b0 = fmaxf(fmaxf(a[0], a[1]), a[2]), b1 = fmaxf(fmaxf(a[3], a[4]), a[5]);
  const float b2 = fmaxf(fmaxf(a[6], a[7]), a[8]), b3 = fmaxf(a[9], a[10]);
  return fmaxf(fmaxf(b0, b1), fmaxf(b2, b3));
}

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void fwd_bf16_kernel(const AttnParams p) {
  using SM = FwdSmem<DQK, DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int bid0 = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid0 >= p.total_work) return;
  const int ks = p.kv_splits > 1 ? bid0 % p.kv_splits : 0;   // this workgroup's key part
  const int bid = p.kv_splits > 1 ? bid0 / p.kv_splits : bid0;
  const int t = bid - (bid / p.n_tiles) * p.n_tiles;
  const int bh = work_bh<LISTS>(p, bid / p.n_tiles, p.H);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int tid = threadIdx.x;
  // under lists without a band order (causal and prefix-LM walks already shrink from the
  // last tile) the list lengths set the order (fixed lengths: no packed sequences here)
  const int qt = (LISTS && !p.longest_first)
                     ? ranked_tile<kThreads>(p.lists,
                                             ((int64_t)b * p.lists.heads + (p.lists.heads == 1 ? 0 : h)) * p.lists.n_rows,
                                             p.n_tiles, kBM, kBM / 2, p.Nq, t, (int*)smem, tid)
                     : (p.longest_first ? (p.n_tiles - 1 - t) : t);
  const int q0 = qt * kBM;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, so per-wave tests branch on scalars
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  // sequence b: its lengths, the offsets of its first query / key row and of its LSE row
  // (packed variable-length sequences: the grid covers the longest)
  const SeqInfo sq = seq_info(p, b);
  const int Nq = sq.nq, Nk = sq.nk;
  if (q0 >= Nq) return;      // whole workgroup, before any barrier
  const int64_t q_off = row_base(sq, true, b, p.qs_b, p.qs_s), o_off = row_base(sq, true, b, p.os_b, p.os_s);
  const int64_t k_off = row_base(sq, false, b, p.ks_b, p.ks_s), v_off = row_base(sq, false, b, p.vs_b, p.vs_s);
  const int64_t lse_off = lse_base(p, sq, b, h);
  const int delta = Nk - Nq;

  const __bf16* Qg = (const __bf16*)p.q + q_off + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + k_off + kv_head(p, h) * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + v_off + kv_head(p, h) * p.vs_h;

  // ---- tile sequence
  TileSeq<kBN> seq;
  seq.t_lo = 0;
  seq.ent = (const uint32_t*)(smem + SM::BYTES + 16);
  const int mk = p.mask.kind;
  bool part = false;   // one of several key parts of this query tile: writes a partial
  if constexpr (!LISTS) {
    band_tile_range(p.mask, q0, kBM, Nq, Nk, kBN, &seq.t_lo, &seq.count);
    if (p.kv_splits > 1) {
      const int pieces = key_pieces(seq.count, p.kv_splits, p.split_tiles);
      if (ks >= pieces) return;   // whole workgroup, before any barrier
      if (pieces > 1) {           // the ks-th of `pieces` contiguous parts of the tile range
        const int per = (seq.count + pieces - 1) / pieces;
        const int first = min(seq.count, ks * per);
        seq.t_lo += first;
        seq.count = min(per, seq.count - first);
        part = true;
      }
    }
  } else {
    // the two 128-row halves of the workgroup each lie in one sparse row
    const ListParams& L = p.lists;
    const int64_t rbase = ((int64_t)b * L.heads + ((L.heads == 1) ? 0 : h)) * L.n_rows;
    const int64_t r0 = rbase + q0 / L.tile_rows;
    const int64_t r1 = (q0 + kBM / 2 < Nq) ? rbase + (q0 + kBM / 2) / L.tile_rows : -1;
    seq.count = build_tile_sequence<kThreads, kBN>(L, r0, r1, Nk, smem + SM::BYTES, tid);
  }

  // ---- Q fragment (B operand of S^T = K Q^T), resident for the whole pass
  const int qrow = q0 + 32 * w + lq;
  bf16x8 qf[DQK / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks) {
    if (qrow < Nq) qf[ks] = *(const bf16x8*)(Qg + (int64_t)qrow * p.qs_s + 16 * ks + 8 * g);
    else qf[ks] = bf16x8{};
  }

  // ---- running state
  f32x16 o[DV / 32];
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) o[i] = f32x16{};
  float m_run = (SOFTCAP && !BIAS && DQK <= 128 && p.cap_fixed) ? p.cap_u : kNegInf, l_run = 0.0f;
  const float c_eff = (SOFTCAP || BIAS) ? 1.0f : p.scale_log2;
  const int prow = swap_bits23(lq);
  const int qw = q0 + 32 * w;
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const int grp = w >> 2;   // 0: waves 0-3, 1: waves 4-7 (one of each per SIMD)
  // element-mask geometry, computed once: tiles starting past need_above or before
  // need_below need the mask; the lane's row sees keys band_lo <= j < band_hi (band
  // masks) or the keys of its document (block-diagonal mask)
  int need_above, need_below;
  key_tile_need(p.mask, qw, Nk, delta, kBN, need_above, need_below);
  if constexpr (LISTS) need_above = Nk - kBN, need_below = INT32_MIN;   // the list classes decide
  int band_lo, band_hi;
  band_interval(p.mask, qrow, Nq, Nk, band_lo, band_hi);
  const int row_doc = (mk == kMaskBlockDiag && qrow < Nq) ? p.mask.doc_q[(int64_t)b * Nq + qrow] : 0;

  LdsDma<kBN, DQK, SM::KPC, kThreads> kdma;
  LdsDma<kBN, DV, SM::VPC, kThreads> vdma;
  kdma.init(p.ks_s, tid);
  vdma.init(p.vs_s, tid);
  zero_lds<kThreads>(smem, SM::BYTES, tid);   // defensive: every slot is loaded before it is read
  auto issue_tile = [&](int t) {
    const int n0 = seq.start(t, LISTS);
    char* st = smem + (t % SM::NST) * SM::STAGE;
    kdma.issue(Kg, p.ks_s, n0, Nk, st);
    vdma.issue(Vg, p.vs_s, n0, Nk, st + SM::KB);
  };

  f32x16 s[2];
  bf16x8 pb[2][2];
  const int T = seq.count;
  for (int t = 0; t < SM::NST - 2 && t < T; ++t) issue_tile(t);
  wait_all_vmem();   // Q fragments and the first tiles
  __syncthreads();

  // Steps t = 0 .. T, two phases each; waves 4-7 run one phase behind waves 0-3:
  //   waves 0-3, step t: matrix  S(t) = K Q^T (t < T), O += V(t-1) P (t > 0);
  //                      vector  softmax of S(t) into P (t < T)
  //   waves 4-7, step t: vector  softmax of S(t-1) (t > 0);  matrix as above
  // so the two waves of a SIMD alternate between MFMA and VALU work. Tile t's stage is
  // busy during phases 2t .. 2t+3; tile t is issued in step t - NST + 2 (the first NST - 2
  // tiles before the loop), once the stage's previous tile (t - NST) is done. Each wave
  // issues its share at the start of its vector phase: issuing a direct-to-LDS load holds
  // the wave until the vector-memory path takes it (about 1 KiB per 16 clocks per CU), and
  // there the wait is hidden under the partner wave's MFMAs, and each group of four waves
  // has the path to itself (issued by all eight waves after the barrier, the loads held
  // every matrix phase back). Each group runs its own loop with the first and last steps
  // peeled, so nothing
  // conditional sits between the phases and the loop-carried operands keep their
  // registers.
  // Matrix phase: O += V(ts - 1) P (V read transposed) and S = K Q^T (two accumulation
  // chains), one software pipeline with the LDS reads issued two items ahead
  auto matrix = [&](int ts, bool do_acc, bool do_s) {
    const char* v0 = smem + opaque_int(((ts - 1 + SM::NST) % SM::NST) * SM::STAGE + SM::KB + trow * SM::VP + tcol * 2);
    const char* k0 = smem + opaque_int((ts % SM::NST) * SM::STAGE + prow * SM::KP + 16 * g);
    pipelined_matrix<4 * (DV / 32), DQK / 16, SM::VP, SM::KP, 2>(v0, k0, do_acc, do_s, o, pb, s, qf);
  };

  // FIXED: softcap without bias, with the capped score's upper bound cap_u as a fixed
  // softmax maximum (see cap_fixed): no row max and no rescale, P = exp2(u - cap_u)
  auto vector_body = [&](auto fixed_c, int ts) __attribute__((always_inline)) {
    constexpr bool FIXED = decltype(fixed_c)::value;
    const int n0 = seq.start(ts, LISTS);
    bool need = n0 > need_above || n0 < need_below;
    bool elem = true, hide = false;
    if constexpr (LISTS) {
      const uint32_t c = seq.cls(ts, grp, true);   // this wave's query half
      hide = c == 0u;
      elem = c == 1u;
      need = need || c != 2u;
    }
    // score transform (softcap / bias) and mask; reg r of block kb holds key
    // n0 + 32 kb + 16 (r / 8) + 8 g + r % 8 of query row qrow.
    // relative bias alone (BIAS_ONLY): the scores stay raw through the mask and the row
    // max; the bias enters with the exponent (below)
    constexpr bool BIAS_ONLY = BIAS && !SOFTCAP;
    if constexpr (BIAS_ONLY) {
    } else if constexpr (FIXED) {
      // u - cap_u = -2 cap_u / (exp(2 y) + 1): one fma scales the denominator by
      // -1 / (2 cap_u), so its reciprocal is the exponent itself
      const float ik = -0.5f / p.cap_u;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = fast_rcp(__builtin_fmaf(fast_exp2(s[kb][r] * p.cap_k1), ik, ik));
    } else if constexpr (SOFTCAP || BIAS) {
      const int jb = opaque_int(n0 + 8 * g);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          s[kb][r] = score_log2<SOFTCAP, BIAS>(s[kb][r], p, qrow, jb + 32 * kb + 16 * (r >> 3) + (r & 7));
    }
    if (need) {
      // rows past Nq are never stored, so their mask does not matter
      const int kbase = opaque_int(n0 + 8 * g);
      if (hide) mask_tile_band(s, kbase, 0, 0);
      else if (elem && mk == kMaskBlockDiag)   // lists with softcap alone sit at the register limit
        mask_tile_doc<!(LISTS && SOFTCAP && !BIAS)>(s, p.mask.doc_k + (int64_t)b * Nk, row_doc, kbase, Nk);
      else mask_tile_band(s, kbase, elem ? band_lo : 0, elem ? band_hi : Nk);
    }

    // online softmax (log2 domain). The O / l rescale is skipped when no row of the
    // wave raised its running max. O already holds every P V up to tile ts - 1.
    // row max as a shallow tree (short dependency chains: this phase has one wave per
    // SIMD, so latency, not issue rate, bounds it)
    // BIAS_ONLY: i - j = dq - off_r with dq = qrow - n0 - 8 g and off_r in [0, 55] the
    // register's key offset, exact in fp32. The largest bias term of the lane's row is at
    // an end of that range, or 0 where the row's |i - j| reaches 0 (the row inside the
    // tile's keys), so max(raw) scale + that term bounds the row max from above (the
    // lazy rescale below only needs an upper bound)
    const float dq = BIAS_ONLY ? __int_as_float(opaque_int(__float_as_int((float)(qrow - n0 - 8 * g)))) : 0.0f;
    const bool one_side = qw >= n0 + kBN - 1 || qw + 31 < n0;   // the tile's keys on one side of every row
    if constexpr (!FIXED) {
      float mt = tree_max32(s);
      if constexpr (BIAS_ONLY) {
        float bm = fmaxf(p.bias_log2 * __builtin_fabsf(dq), p.bias_log2 * __builtin_fabsf(dq - 55.0f));
        if (!one_side) bm = fmaxf(bm, 0.0f);
        mt = pair_max(__builtin_fmaf(mt, p.scale_log2, bm));
      } else {
        mt = pair_max(mt) * c_eff;
      }
      // lazy rescale: keep a stale running max until some row's max exceeds it by more
      // than kRescaleLog2, so p = exp2(s - m) <= 2^kRescaleLog2 and the rescale runs only
      // on large jumps (usually just the first tile); O and l always share the same m
      if (__builtin_amdgcn_ballot_w64(mt > m_run + kRescaleLog2)) {
        const float m_new = fmaxf(m_run, mt);
        const float alpha = fast_exp2(m_run - ((m_new == kNegInf) ? 0.0f : m_new));
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
        m_run = m_new;
      }
    }
    const float m_use = (m_run == kNegInf) ? 0.0f : m_run;
    if constexpr (BIAS_ONLY) {
      // exponent u - m = raw scale + bias |i - j| - m, in place
      if (one_side) {
        // |i - j| = sign (dq - off_r): with sb = sign bias, one fma with the literal off_r
        // (sb (dq - off_r) - m) and one fma per score
        const float sb = qw >= n0 + kBN - 1 ? p.bias_log2 : -p.bias_log2;
        const float am = __builtin_fmaf(sb, dq, -m_use);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            s[kb][r] = __builtin_fmaf(s[kb][r], p.scale_log2,
                                      __builtin_fmaf(sb, -(float)(32 * kb + 16 * (r >> 3) + (r & 7)), am));
      } else {
        // both sides: a subtraction with a literal, an fma with |.| and an fma per score
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float t = dq - (float)(32 * kb + 16 * (r >> 3) + (r & 7));
            s[kb][r] = __builtin_fmaf(s[kb][r], p.scale_log2, __builtin_fmaf(p.bias_log2, __builtin_fabsf(t), -m_use));
          }
      }
    }
    // four independent partial row sums of the fp32 probabilities (plain adds: the packed
    // bf16 dot product would stall the partner wave's MFMAs, as it shares their pipe)
    float ls[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = (FIXED || BIAS_ONLY) ? fast_exp2(s[kb][8 * hh + 2 * e])
                                                : fast_exp2(__builtin_fmaf(s[kb][8 * hh + 2 * e], c_eff, -m_use));
          const float p1 = (FIXED || BIAS_ONLY) ? fast_exp2(s[kb][8 * hh + 2 * e + 1])
                                                : fast_exp2(__builtin_fmaf(s[kb][8 * hh + 2 * e + 1], c_eff, -m_use));
          pk[e] = pack_bf16x2(p0, p1);
          ls[e] = (kb == 0 && hh == 0) ? p0 + p1 : ls[e] + (p0 + p1);   // no 0 + x: it does not fold
        }
        pb[kb][hh] = __builtin_bit_cast(bf16x8, pk);
      }
    }
    l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
  };
  constexpr bool CAN_FIX = SOFTCAP && !BIAS && DQK <= 128;   // (the wider head has no registers for a second body)
  auto vector = [&](int ts) __attribute__((always_inline)) {
    if constexpr (CAN_FIX) {
      if (p.cap_fixed) {
        vector_body(IntC<1>{}, ts);
        return;
      }
    }
    vector_body(IntC<0>{}, ts);
  };

  // issue tile t + NST - 2 (called at the start of the wave's vector phase of step t)
  auto step_begin = [&](int t) {
    if (t + SM::NST - 2 < T) issue_tile(t + SM::NST - 2);
  };
  auto step_end = [&](int t) {
    // tile t + 1 is read from the next step on; the NST - 3 tiles issued after it may
    // stay in flight (loads complete in order; every tile costs each wave the same
    // number of load instructions)
    const int later = min(SM::NST - 3, max(0, T - 2 - t));
    if (later > 0) kdma.wait_leaving(vdma, later);
    else wait_lds_dma();
    // Once per step: tile t + 1 is visible to all waves and every wave is done with the
    // stage that the next step refills. Within a step the partner waves need no barrier
    // (their state is private and no stage changes), so they alternate freely.
    __syncthreads();
  };

  if (T > 0) {
    if (grp == 0) {
      matrix(0, false, true);
      step_begin(0);
      vector(0);
      step_end(0);
      for (int t = 1; t < T; ++t) {
        matrix(t, true, true);
        step_begin(t);
        vector(t);
        step_end(t);
      }
      matrix(T, true, false);
      step_end(T);
    } else {
      step_begin(0);
      matrix(0, false, true);
      step_end(0);
      for (int t = 1; t < T; ++t) {
        step_begin(t);
        vector(t - 1);
        matrix(t, true, true);
        step_end(t);
      }
      vector(T - 1);
      matrix(T, true, false);
      step_end(T);
    }
  }

  // ---- epilogue
  const float l_tot = pair_sum(l_run);
  const bool empty = !(l_tot > 0.0f);
  const float inv = empty ? 0.0f : 1.0f / l_tot;
  if (!LISTS && part) {   // partial of this key part, for the combine
    if (qrow < Nq) {
      const int64_t prow = (((int64_t)bh * p.n_tiles + qt) * p.kv_splits + ks) * kBM + (qrow - q0);
      float* Po = p.split_o + prow * DV;
#pragma unroll
      for (int db = 0; db < DV / 32; ++db)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          *(f32x4*)(Po + 32 * db + 8 * jj + 4 * g) =
              f32x4{o[db][4 * jj] * inv, o[db][4 * jj + 1] * inv, o[db][4 * jj + 2] * inv, o[db][4 * jj + 3] * inv};
      if (g == 0) p.split_lse[prow] = empty ? kNegInf : (m_run + fast_log2(l_tot)) * kLn2;
    }
    return;
  }
  if (qrow < Nq) {
    __bf16* Og = (__bf16*)p.o + o_off + h * p.os_h + (int64_t)qrow * p.os_s;
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
      p.lse[lse_off + qrow] = empty ? kNegInf : (m_run + fast_log2(l_tot)) * kLn2;
    }
  }
}

// LDS bytes beyond the K/V stages for the block-sparse tile sequence (0 without lists).
int list_bytes(const ListParams& L) { return L.pcnt == nullptr ? 0 : tile_sequence_bytes(L, kBN); }

template <int DQK, int DV>
int smem_bytes(const ListParams& L) { return FwdSmem<DQK, DV>::BYTES + list_bytes(L); }

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
hipError_t launch_one(const AttnParams& p, hipStream_t st) {
  auto kern = fwd_bf16_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
  const int bytes = smem_bytes<DQK, DV>(p.lists);
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(p.grid_padded), dim3(kThreads), bytes, st, p);
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
int fwd_bf16_list_rows() { return kBM / 2; }
int fwd_bf16_tile_keys() { return kBN; }

bool fwd_bf16_lists_fit(int dqk, int dv, int n_cols, int tile_cols) {
  ListParams L{};
  L.pcnt = (const int*)1;   // only the sizes are read
  L.n_cols = n_cols;
  L.tile_cols = tile_cols;
  if ((int64_t)n_cols * (tile_cols / kBN) > (1 << 20)) return false;
  int bytes = 0;
  if (dqk == 128 && dv == 128) bytes = smem_bytes<128, 128>(L);
  else if (dqk == 64 && dv == 64) bytes = smem_bytes<64, 64>(L);
  else if (dqk == 192 && dv == 128) bytes = smem_bytes<192, 128>(L);
  else return false;
  return bytes <= kMaxLdsBytes;
}

// Merge of the key parts of the split query tiles: O = sum_s w_s O_s / sum_s w_s and
// LSE = mu + ln sum_s w_s with w_s = exp(LSE_s - mu), mu = max_s LSE_s, the parts taken in
// a fixed order. One workgroup per 256 * 4 / DV rows of a query tile (DV / 4 threads per
// row, four columns each); the workgroups of a tile walked in one part exit at once.
template <int DV>
__global__ __launch_bounds__(256)
void fwd_split_combine_kernel(const AttnParams p) {
  constexpr int kTpr = DV / 4, kRpp = 256 / kTpr, kChunks = kBM / kRpp;
  const int chunk = blockIdx.x % kChunks;
  const int bt = blockIdx.x / kChunks;
  const int bh = bt / p.n_tiles;
  const int qt = bt - bh * p.n_tiles;
  const int q0 = qt * kBM;
  int tlo, count;
  band_tile_range(p.mask, q0, kBM, p.Nq, p.Nk, kBN, &tlo, &count);
  const int pieces = key_pieces(count, p.kv_splits, p.split_tiles);
  if (pieces <= 1) return;
  const int b = bh / p.H, h = bh - b * p.H;
  const int c = threadIdx.x % kTpr;
  const int r = chunk * kRpp + threadIdx.x / kTpr;
  const int64_t slot0 = ((int64_t)bh * p.n_tiles + qt) * p.kv_splits;
  __bf16* Og = (__bf16*)p.o + b * p.os_b + h * p.os_h;
  float* Lg = p.lse + ((int64_t)b * p.H + h) * p.Nq;
  if (q0 + r < p.Nq) {
    float ls[kMaxKeyParts];
    float mx = kNegInf;
#pragma unroll
    for (int s = 0; s < kMaxKeyParts; ++s) {
      ls[s] = s < pieces ? p.split_lse[(slot0 + s) * kBM + r] : kNegInf;
      mx = fmaxf(mx, ls[s]);
    }
    const bool empty = mx == kNegInf;
    const float mu = empty ? 0.0f : mx;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float tot = 0.0f;
#pragma unroll
    for (int s = 0; s < kMaxKeyParts; ++s) {
      if (s < pieces) {
        const float wgt = exp2f((ls[s] - mu) * kLog2e);
        tot += wgt;
        acc += wgt * *(const f32x4*)(p.split_o + ((slot0 + s) * kBM + r) * DV + 4 * c);
      }
    }
    const float inv = empty ? 0.0f : 1.0f / tot;
    u32x2 v;
    v[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
    v[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
    *(u32x2*)(Og + (int64_t)(q0 + r) * p.os_s + 4 * c) = v;
    if (c == 0) Lg[q0 + r] = empty ? kNegInf : mu + logf(tot);
  }
}

FwdKeySplit fwd_bf16_key_split(int B, int H, int Nq, int Nk, const MaskParams& m, int dqk, int dv, bool lists) {
  // A query tile is one workgroup's walk over its visible key tiles, and a launch that does
  // not fill the CUs lasts as long as its longest walk. When the grid is short of the 256
  // CUs, the longest tiles can be walked in parts of T key tiles, one workgroup each. Every
  // candidate part count s (T = ceil(longest / s), at least kMinPartTiles) whose parts all
  // start at once on the CUs (a second round would cost more than the balance gains) is
  // priced with a cost model measured on MI355X: a 64-key tile of the walk takes about
  // 1.5 us at Dv = 128 and 1.0 us at Dv = 64 with the GPU busy, and a split costs about
  // 5 us plus 0.9 us per MiB of fp32 partial O (written by the parts, read by the
  // combine). The count with the largest predicted saving is used, none if no saving.
  const FwdKeySplit none{1, 0};
  if (lists || dqk != dv || (dv != 64 && dv != 128) || B <= 0 || H <= 0 || Nq <= 0) return none;
  const int n_tiles = (Nq + kBM - 1) / kBM;
  const int64_t heads = (int64_t)B * H;
  if (heads * n_tiles >= kCUs) return none;   // the grid fills the CUs already
  int counts[kCUs];
  int longest = 0;
  for (int qt = 0; qt < n_tiles; ++qt) {
    int tlo;
    band_tile_range(m, qt * kBM, kBM, Nq, Nk, kBN, &tlo, &counts[qt]);
    longest = max(longest, counts[qt]);
  }
  const double tile_us = dv == 128 ? 1.5 : 1.0;
  FwdKeySplit best = none;
  double best_saving = 0.0;
  for (int s = 2; s <= kMaxKeyParts; ++s) {
    const int tiles = (longest + s - 1) / s;
    if (tiles < kMinPartTiles) break;
    int64_t workgroups = 0, part_rows = 0;
    int piece = 0;
    for (int qt = 0; qt < n_tiles; ++qt) {
      const int n = key_pieces(counts[qt], kMaxKeyParts, tiles);
      workgroups += n;
      if (n > 1) part_rows += (int64_t)n * kBM;
      piece = max(piece, (counts[qt] + n - 1) / n);
    }
    if (workgroups * heads > kCUs) continue;
    const double part_mib = (double)(part_rows * heads) * dv * sizeof(float) / (1 << 20);
    const double saving = (longest - piece) * tile_us - (kSplitFixedUs + kSplitUsPerMiB * part_mib);
    if (saving > best_saving) {
      best_saving = saving;
      best = FwdKeySplit{(longest + tiles - 1) / tiles, tiles};
    }
  }
  return best;
}

size_t fwd_bf16_split_workspace_bytes(int B, int H, int Nq, int dv, int splits) {
  const size_t rows = (size_t)B * H * ((Nq + kBM - 1) / kBM) * splits * kBM;
  return ((rows * dv * sizeof(float) + 255) / 256) * 256 + rows * sizeof(float);
}

hipError_t launch_fwd_split_combine(AttnParams p, int dv, hipStream_t st) {
  p.n_tiles = (p.Nq + kBM - 1) / kBM;
  const unsigned grid = (unsigned)(p.B * p.H * p.n_tiles) * (unsigned)(kBM * dv / 1024);
  if (dv == 128) hipLaunchKernelGGL(fwd_split_combine_kernel<128>, dim3(grid), dim3(256), 0, st, p);
  else if (dv == 64) hipLaunchKernelGGL(fwd_split_combine_kernel<64>, dim3(grid), dim3(256), 0, st, p);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_fwd_bf16(AttnParams p, int dqk, int dv, hipStream_t st) {
  p.n_tiles = (p.Nq + kBM - 1) / kBM;
  if (p.kv_splits < 1) p.kv_splits = 1;
  p.total_work = p.B * p.H * p.n_tiles * p.kv_splits;
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
