// bf16 attention backward for gfx950: dQ, dK, dV recomputed from the saved LSE.
//
// The fuzz tester of "Enable 2CTA for SM100 block-sparse backward" drives the backward
// with (q, k, v, out, dout, lse) and separate transposed block-sparse lists; its
// relative-bias backward passes the gradient through unchanged. "Optimize Flash Dynamic
// Mask Attention Kernel Configurations" keeps a seq-k-parallel backward with a
// deterministic grid. Math (per (b, h)):
//   P = exp(S - LSE), dV = P^T dO, dP = dO V^T, D_i = sum_d dO_id O_id,
//   dS = P (dP - D) [x (1 - tanh^2) under softcap], dQ = scale dS K, dK = scale dS^T Q.
//
// Three kernels, no atomics (every gradient element has one writer and a fixed
// summation order, so results are bitwise reproducible):
//   1. preprocess: per 64-query block, lse2 = LSE log2(e) and D = rowsum(dO * O) into the
//      workspace, padded with (+inf, 0) past Nq so that padded queries drop out of every
//      product without masks;
//   2. dK/dV pass: a workgroup owns 128 keys and walks 64-query steps (Q, dO, lse2, D
//      staged in LDS by direct global->LDS loads). The 8 waves form 4 PAIRS, one per SIMD,
//      each pair owning 32 keys. The "P wave" holds K of the keys in VGPRs, computes
//      S = Q K^T, P, and accumulates dV^T += dO^T P; the "dS wave" holds V, computes
//      dP = dO V^T, dS = P (dP - D) with P handed over through LDS, and accumulates
//      dK^T += Q^T dS. Each wave needs half the registers of a wave doing all four
//      products, so two waves fit per SIMD and ping-pong: while one runs its 32 MFMAs of
//      the step the other runs its exp / dS arithmetic, one phase apart, as in the
//      forward. S and dP come out with ONE KEY PER LANE and 8 consecutive queries per
//      register group, which is the B operand of the dV / dK products as is; dO^T / Q^T
//      come from transposed LDS reads;
//   3. dQ pass: a workgroup owns 128 queries and walks 64-key tiles of K / V (direct
//      global->LDS loads, 3-4 stages), again in wave pairs sharing 32 queries, but here
//      the pair splits each tile's keys: both waves hold Q and dO, and each computes
//      S^T = K Q^T, dP^T = V dO^T, P and dS for its 32 keys and accumulates its own
//      partial dQ^T += K^T dS^T (K^T from transposed LDS reads), one phase apart so the
//      MFMAs of one overlap the exp / dS arithmetic of the other. The two partials are
//      added once at the end in a fixed order. Lane = query, as in the forward.
// The dQ pass recomputes S and dP (7 matrix products instead of 5): that is the price
// of determinism without atomics.
//
// Tiles read both row-wise (16-byte MFMA rows) and transposed (8-byte reads of 4 rows)
// use a row pitch of an odd number of 16-byte chunks that is not 0 or +-16 bytes modulo
// 256: conflict-free row reads and at most 2-way conflicted transposed reads.
#include "kernel_common.h"
#include "launch.h"

namespace fmha {
namespace {

constexpr int kThreads = 512;
constexpr int kKB = 128;     // keys per dK/dV workgroup: 4 wave pairs x 32 keys
constexpr int kQS = 64;      // queries per dK/dV step
constexpr int kQM = 128;     // queries per dQ workgroup: 4 wave pairs x 32
constexpr int kKN = 64;      // keys per dQ step
constexpr int kPreThreads = 256;

// Row pitch in 16-byte chunks of a tile read row-wise and transposed.
template <int D> struct DualPitch;
template <> struct DualPitch<64> { static constexpr int value = 9; };
template <> struct DualPitch<128> { static constexpr int value = 19; };
template <> struct DualPitch<192> { static constexpr int value = 25; };
// Row pitch of a tile read row-wise only (odd chunk count: conflict-free 16-byte reads).
template <int D> struct RowPitch { static constexpr int value = D / 8 + 1; };

// ------------------------------------------------------------------------------- preprocess
template <int DV>
__global__ __launch_bounds__(kPreThreads)
void bwd_preprocess_kernel(const BwdParams bp) {
  constexpr int LPK = DV / 8;
  constexpr int ROWS = kPreThreads / LPK;
  const AttnParams& p = bp.a;
  const int npad = bp.n_qblk * 64;
  const int64_t r = (int64_t)blockIdx.x * ROWS + threadIdx.x / LPK;
  const int dl = threadIdx.x % LPK;
  const int64_t total = (int64_t)p.B * p.H * npad;
  const bool in = r < total;
  float x = 0.0f, lse2 = __builtin_huge_valf();
  int64_t bh = 0;
  int i = 0;
  if (in) {
    i = (int)(r % npad);
    bh = r / npad;
    const int h = (int)(bh % p.H), b = (int)(bh / p.H);
    const SeqInfo sq = seq_info(p, b);
    if (i < sq.nq) {
      const __bf16* Og = (const __bf16*)p.o + row_base(sq, true, b, p.os_b, p.os_s) + h * p.os_h +
                         (int64_t)i * p.os_s + 8 * dl;
      const __bf16* Dg = (const __bf16*)bp.dout + row_base(sq, true, b, bp.dos_b, bp.dos_s) + h * bp.dos_h +
                         (int64_t)i * bp.dos_s + 8 * dl;
      float of[8], df[8];
      bf16x8_to_f32(*(const u32x4*)Og, of);
      bf16x8_to_f32(*(const u32x4*)Dg, df);
#pragma unroll
      for (int e = 0; e < 8; ++e) x = __builtin_fmaf(of[e], df[e], x);
      const float ls = p.lse[lse_base(p, sq, b, h) + i];
      lse2 = (ls == kNegInf) ? __builtin_huge_valf() : ls * kLog2e;
    }
  }
  x = group_sum<LPK>(x);
  if (in && dl == 0) {
    float* blk = bp.ws + (bh * bp.n_qblk + i / 64) * 128;
    blk[i % 64] = lse2;
    blk[64 + i % 64] = x;
  }
}

// ------------------------------------------------------------------------------- dK / dV
template <int DQK, int DV>
struct DkdvSmem {
  static constexpr int QPC = DualPitch<DQK>::value, OPC = DualPitch<DV>::value;
  static constexpr int QP = QPC * 16, OP = OPC * 16;   // bytes
  static constexpr int QB = kQS * QP, OB = kQS * OP;
  static constexpr int LB = 1024;                      // lse2[64], D[64], 512 bytes unused
  static constexpr int STAGE = QB + OB + LB;
  static constexpr int XB1 = 4 * 64 * 64;              // P hand-over: 4 pairs x 64 lanes x 64 B
  static constexpr int NST = (4 * STAGE + XB1 <= 148 * 1024) ? 4 : 3;
  // Double-buffered hand-over where it fits: then the workgroup needs a barrier only
  // once per step (two phases) instead of after every phase.
  static constexpr bool DBLX = NST * STAGE + 2 * XB1 <= 152 * 1024;
  static constexpr int XB = DBLX ? 2 * XB1 : XB1;
  static constexpr int BYTES = NST * STAGE + XB;
};

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dkdv_kernel(const BwdParams bp) {
  using SM = DkdvSmem<DQK, DV>;
  constexpr int DM = DQK > DV ? DQK : DV, DN = DQK < DV ? DQK : DV;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, bp.grid_padded_kv);
  if (bid >= bp.total_work_kv) return;
  // work item: (batch b, K/V head hk, key tile kt); with grouped K/V heads the group's
  // query heads h0 .. h0 + G - 1 are walked one after the other (a fixed order: the dK / dV
  // sums stay deterministic)
  const int G = p.group > 1 ? p.group : 1;
  const int Hkv = p.H / G;
  const int kt0 = bid - (bid / bp.n_kv_tiles) * bp.n_kv_tiles;   // ascending: under causal masks
  const int bhk = work_bh<LISTS>(p, bid / bp.n_kv_tiles, Hkv);    // the first key tiles see the most queries
  const int b = bhk / Hkv, hk = bhk - (bhk / Hkv) * Hkv;
  const int h0 = hk * G;
  const int tid = threadIdx.x;
  // under lists without a band order (causal and prefix-LM walks already shrink with the
  // tile index) the transposed list lengths set the order (fixed lengths under lists)
  const int kt = (LISTS && !p.longest_first)
                     ? ranked_tile<kThreads>(p.lists,
                                             ((int64_t)b * p.lists.heads + (p.lists.heads == 1 ? 0 : h0)) * p.lists.n_rows,
                                             bp.n_kv_tiles, kKB, 0, p.Nk, kt0, (int*)smem, tid)
                     : kt0;
  const int k0 = kt * kKB;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  const int role = w >> 2;     // 0: P wave (K; S, P, dV), 1: dS wave (V; dP, dS, dK)
  const int pair = w & 3;      // waves w and w + 4 share a SIMD and the same 32 keys
  const SeqInfo sq = seq_info(p, b);
  const int Nq = sq.nq, Nk = sq.nk, delta = Nk - Nq;
  if (k0 >= Nk) return;        // packed sequences: past this one's keys (whole workgroup, no barrier yet)
  const int kw = k0 + 32 * pair;
  const int key = kw + lq;

  const __bf16* Qg = (const __bf16*)p.q + row_base(sq, true, b, p.qs_b, p.qs_s) + h0 * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + row_base(sq, false, b, p.ks_b, p.ks_s) + hk * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + row_base(sq, false, b, p.vs_b, p.vs_s) + hk * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + row_base(sq, true, b, bp.dos_b, bp.dos_s) + h0 * bp.dos_h;
  const char* WSg = (const char*)(bp.ws + ((int64_t)b * p.H + h0) * bp.n_qblk * 128);

  // ---- query-step sequence
  TileSeq<kQS> seq;
  seq.t_lo = 0;
  seq.ent = (const uint32_t*)(smem + SM::BYTES + 16);
  const int mk = p.mask.kind;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nq;
    if (mk == kMaskCausal || mk == kMaskWindow) lo = max(0, k0 - delta);
    if (mk == kMaskPrefix) lo = (k0 < p.mask.prefix) ? 0 : max(0, k0 - delta);
    if (mk == kMaskWindow) hi = min(Nq, k0 + kKB - 1 - delta + p.mask.window + 1);
    lo = min(lo, Nq);
    seq.t_lo = lo / kQS;
    seq.count = max(0, (hi + kQS - 1) / kQS - seq.t_lo);
  } else {
    const ListParams& L = p.lists;   // transposed lists: rows = key tiles
    // (grouped K/V heads take head-broadcast lists only, so h0 stands for every head)
    const int64_t row = ((int64_t)b * L.heads + ((L.heads == 1) ? 0 : h0)) * L.n_rows + k0 / L.tile_rows;
    seq.count = build_tile_sequence<kThreads, kQS>(L, row, -1, Nq, smem + SM::BYTES, tid);
  }

  // ---- B operand of this wave's S (K) or dP (V): the lane's key, k-slot = head dim
  bf16x8 bf[DM / 16];
  {
    const __bf16* src = role ? Vg : Kg;
    const int64_t st = role ? p.vs_s : p.ks_s;
    const int dr = role ? DV : DQK;
#pragma unroll
    for (int ks = 0; ks < DM / 16; ++ks)
      bf[ks] = (16 * ks < dr && key < Nk) ? *(const bf16x8*)(src + (int64_t)key * st + 16 * ks + 8 * g) : bf16x8{};
  }

  f32x16 acc[DM / 32];
#pragma unroll
  for (int i = 0; i < DM / 32; ++i) acc[i] = f32x16{};
  f32x16 s[2];
  bf16x8 bop[2][2];
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  // hand-over slot of the pair, lane-major (+ 64 i per 16-byte piece); when double-
  // buffered, the buffer of step t (t & 1) sits 1024 pieces further
  u32x4* xch = (u32x4*)(smem + SM::NST * SM::STAGE + pair * 4096) + l;

  // visible queries of the lane's key under the band masks: qlo <= i <= qhi
  int qlo = 0, qhi = 0x3fffffff;
  if (mk == kMaskCausal || mk == kMaskWindow || (mk == kMaskPrefix && key >= p.mask.prefix)) qlo = key - delta;
  if (mk == kMaskWindow) qhi = key - delta + p.mask.window;
  const uint32_t qspan = (uint32_t)qhi - (uint32_t)qlo;   // qlo <= i <= qhi as one unsigned test
  const int kdoc = (mk == kMaskBlockDiag && key < Nk) ? p.mask.doc_k[(int64_t)b * Nk + key] : 0;
  // query steps (start i0) that need the element mask for the wave's 32 keys: i0 < need_below
  // or i0 > need_above (computed once, so the per-step test is two scalar compares)
  int need_below = INT32_MIN, need_above = INT32_MAX;
  if (mk == kMaskCausal || mk == kMaskWindow || (mk == kMaskPrefix && kw + 31 >= p.mask.prefix))
    need_below = kw + 31 - delta;
  if (mk == kMaskWindow) need_above = kw - kQS + 1 - delta + p.mask.window;
  if (mk == kMaskBlockDiag) need_below = INT32_MAX;

  LdsDma<kQS, DQK, SM::QPC, kThreads> qdma;
  LdsDma<kQS, DV, SM::OPC, kThreads> odma;
  qdma.init(p.qs_s, tid);
  odma.init(bp.dos_s, tid);
  constexpr int ld_wave = 7;   // a wave with the fewest tile blocks issues the lse2 / D load
  const int per_step = qdma.count() + odma.count() + (w == ld_wave ? 1 : 0);
  zero_lds<kThreads>(smem, SM::NST * SM::STAGE, tid);   // defensive: every slot is loaded before it is read
  // step t walks query step tq of group head gi (t = gi * Tq + tq)
  const int Tq = seq.count;
  auto head_step = [&](int t, int& gi) {
    if (G == 1) {
      gi = 0;
      return t;
    }
    gi = t / Tq;
    return t - gi * Tq;
  };
  auto issue_step = [&](int t) {
    int gi;
    const int i0 = seq.start(head_step(t, gi), LISTS);
    char* st = smem + (t % SM::NST) * SM::STAGE;
    qdma.issue(Qg + (int64_t)gi * p.qs_h, p.qs_s, i0, Nq, st);
    odma.issue(DOg + (int64_t)gi * bp.dos_h, bp.dos_s, i0, Nq, st + SM::QB);
    if (w == ld_wave)
      dma_16b(WSg + (int64_t)gi * bp.n_qblk * 512, (uint32_t)(i0 / 64) * 512u + 16u * l, st + SM::QB + SM::OB);
  };

  const int T = G * Tq;
  for (int t = 0; t < SM::NST - 2 && t < T; ++t) issue_step(t);
  wait_all_vmem();
  __syncthreads();

  // Steps t = 0 .. T, two phases each; the dS waves run one phase behind the P waves:
  //   P wave,  step t: matrix  s = Q_t K^T (t < T), dV^T += dO_{t-1}^T P_{t-1} (t > 0);
  //                    vector  P_t from s and the saved LSE, into bop and the hand-over
  //   dS wave, step t: vector  dS_{t-1} = P_{t-1} (dP_{t-1} - D) from the hand-over (t > 0);
  //                    matrix  s = dO_t V^T (t < T), dK^T += Q_{t-1}^T dS_{t-1} (t > 0)
  // The hand-over of step t is written in phase 2t+1 and read in phase 2t+2; stage t is
  // read during phases 2t .. 2t+3 and refilled in phase 2t+4 at the earliest.
  // Each role runs its own loop with the first and last steps peeled, so nothing
  // conditional sits between the phases and the loop-carried operands (s, bop, acc) keep
  // their registers from one step to the next.
  // role R's matrix phase: R = 0 (P wave): T = dO (width DV), R-side = Q (width DQK);
  // R = 1 (dS wave): T = Q (width DQK), R-side = dO (width DV)
  auto matrix = [&](auto role_c, int ts, bool do_acc, bool do_s) {
    constexpr int R = decltype(role_c)::value;
    constexpr int TP = R ? SM::QP : SM::OP, RP = R ? SM::OP : SM::QP;
    constexpr int DA = R ? DQK : DV, DR = R ? DV : DQK;
    const int tv = ts - 1;
    const int sv = ((tv < 0 ? 0 : tv) % SM::NST) * SM::STAGE + (R ? 0 : SM::QB);
    const int ss = (ts % SM::NST) * SM::STAGE + (R ? SM::QB : 0);
    // one software pipeline: acc^T += T^T bop for the previous step, then s = R bf^T
    pipelined_matrix<4 * (DA / 32), DR / 16, TP, RP, 2>(smem + opaque_int(sv + trow * TP + tcol * 2),
                                                         smem + opaque_int(ss + prow * RP + 16 * g), do_acc, do_s,
                                                         acc, bop, s, bf);
  };

  // P wave: P_ts = exp2(s * scale_log2 - lse2) (score transform and element mask applied),
  // register r of block kb holding query i0 + 32 kb + 16 (r / 8) + 8 g + r % 8
  auto p_vector = [&](int ts) {
    int gi;
    const int tq = head_step(ts, gi);
    const int i0 = seq.start(tq, LISTS);
    const float* LD = (const float*)(smem + (ts % SM::NST) * SM::STAGE + SM::QB + SM::OB);
    // the batch's query document ids; vector loads need them 16-byte aligned
    const int* dqrow = p.mask.doc_q + (int64_t)b * Nq;
    const bool dq_al = (reinterpret_cast<uintptr_t>(dqrow) & 15) == 0;
    bool need;
    if constexpr (LISTS) need = seq.cls(tq, 0, true) != 2u;
    else need = i0 < need_below || i0 > need_above;
    auto body = [&](auto test_c) {
      constexpr int TEST = decltype(test_c)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int qi = 32 * kb + 16 * hh + 8 * g;
          const f32x4 la = *(const f32x4*)(LD + qi), lb = *(const f32x4*)(LD + qi + 4);
          const int qb = (TEST != kTestNone || BIAS) ? opaque_int(i0 + qi) : 0;
          // relative bias alone: i - j = (i0 + qi - key) + ee, exact in fp32 (as in the forward)
          const float dij = (BIAS && !SOFTCAP) ? __int_as_float(opaque_int(__float_as_int((float)(i0 + qi - key)))) : 0.0f;
          int dqv[8];   // documents of queries qb .. qb + 7
          if constexpr (TEST >= kTestDoc) doc_ids8<TEST == kTestDocVec>(dqrow, qb, Nq, dqv);
          u32x4 pk, pc;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv[2], pd[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int ee = 2 * e + z, r = 8 * hh + ee;
              const float lse2 = ee < 4 ? la[ee] : lb[ee - 4];
              const int qidx = qb + ee;
              // x = u - lse2 (one fma without a score transform); rows past Nq carry
              // lse2 = +inf, so their P is 0 whatever the test says
              float dcap = 1.0f, x;
              if constexpr (BIAS && !SOFTCAP)
                x = __builtin_fmaf(s[kb][r], p.scale_log2, __builtin_fmaf(p.bias_log2, __builtin_fabsf(dij + (float)ee), -lse2));
              else if constexpr (SOFTCAP || BIAS) x = score_log2_d<SOFTCAP, BIAS>(s[kb][r], p, qidx, key, dcap) - lse2;
              else x = __builtin_fmaf(s[kb][r], p.scale_log2, -lse2);
              if constexpr (TEST == kTestBand) {
                if ((uint32_t)qidx - (uint32_t)qlo > qspan) x = kNegInf;
              } else if constexpr (TEST >= kTestDoc) {
                if ((qidx < Nq) & (key < Nk) & (dqv[ee] != kdoc)) x = kNegInf;
              }
              pv[z] = fast_exp2(x);
              pd[z] = pv[z] * dcap;
            }
            pk[e] = pack_bf16x2(pv[0], pv[1]);
            pc[e] = SOFTCAP ? pack_bf16x2(pd[0], pd[1]) : pk[e];
          }
          bop[kb][hh] = __builtin_bit_cast(bf16x8, pk);
          xch[(SM::DBLX ? 1024 * (ts & 1) : 0) + 64 * (2 * kb + hh)] = pc;
        }
    };
    if (!need) body(IntC<kTestNone>{});
    else if (mk != kMaskBlockDiag) body(IntC<kTestBand>{});
    else if (dq_al && i0 + 64 <= Nq) body(IntC<kTestDocVec>{});   // the step's 64 queries in bounds
    else body(IntC<kTestDoc>{});
  };

  // dS wave: dS_ts = P (dP - D) from the handed-over P, into bop
  auto ds_vector = [&](int ts) {
    const float* Dl = (const float*)(smem + (ts % SM::NST) * SM::STAGE + SM::QB + SM::OB) + 64;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qi = 32 * kb + 16 * hh + 8 * g;
        const f32x4 da = *(const f32x4*)(Dl + qi), db4 = *(const f32x4*)(Dl + qi + 4);
        const u32x4 pc = xch[(SM::DBLX ? 1024 * (ts & 1) : 0) + 64 * (2 * kb + hh)];
        u32x4 dk4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pf[2];
          bf16x2_to_f32(pc[e], pf);
          float dsv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int ee = 2 * e + z, r = 8 * hh + ee;
            const float dd = ee < 4 ? da[ee] : db4[ee - 4];
            dsv[z] = pf[z] * (s[kb][r] - dd);
          }
          dk4[e] = pack_bf16x2(dsv[0], dsv[1]);
        }
        bop[kb][hh] = __builtin_bit_cast(bf16x8, dk4);
      }
  };

  // Step t refills the stage of step t - 2 (read up to step t - 1) with step t + NST - 2;
  // each wave issues its share at the start of its vector phase, where the time the
  // vector-memory path takes to accept the loads is hidden under the partner's MFMAs (as
  // in the forward). The hand-over of step t is written in its second phase and read in
  // the first phase of step t + 1, so with a double-buffered hand-over the end-of-step
  // barrier alone orders every LDS reuse; otherwise a barrier also separates the two
  // phases.
  auto step_begin = [&](int t) {
    if (t + SM::NST - 2 < T) issue_step(t + SM::NST - 2);
  };
  auto mid = [&]() {
    if (!SM::DBLX) __syncthreads();
  };
  auto step_end = [&](int t) {
    // stage t + 1 is read from the next step on; the NST - 3 steps issued after it may
    // stay in flight (loads complete in order)
    const int later = min(SM::NST - 3, max(0, T - 2 - t));
    if (later > 0) wait_vmcnt_at_most(later * per_step);
    else wait_lds_dma();
    __syncthreads();
  };

  // ---- epilogue: lane = key, reg r <-> d = 32 db + 8 (r/4) + 4 g + r % 4. Called on
  // each role's own path, so registers only one role uses are not kept live by the other.
  auto store = [&](bool isk) {
    if (key >= Nk) return;
    __bf16* dst = isk ? (__bf16*)bp.dk + row_base(sq, false, b, bp.dks_b, bp.dks_s) + hk * bp.dks_h + (int64_t)key * bp.dks_s
                      : (__bf16*)bp.dv + row_base(sq, false, b, bp.dvs_b, bp.dvs_s) + hk * bp.dvs_h + (int64_t)key * bp.dvs_s;
    const float sc = isk ? p.scale : 1.0f;
    const int dw = isk ? DQK : DV;
#pragma unroll
    for (int db = 0; db < DM / 32; ++db) {
      if (32 * db >= DN && 32 * db >= dw) continue;
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(acc[db][4 * jj] * sc, acc[db][4 * jj + 1] * sc);
        v[1] = pack_bf16x2(acc[db][4 * jj + 2] * sc, acc[db][4 * jj + 3] * sc);
        *(u32x2*)(dst + 32 * db + 8 * jj + 4 * g) = v;
      }
    }
  };

  if (role == 0) {
    if (T > 0) {
      matrix(IntC<0>{}, 0, false, true);
      mid();
      step_begin(0);
      p_vector(0);
      step_end(0);
      for (int t = 1; t < T; ++t) {
        matrix(IntC<0>{}, t, true, true);
        mid();
        step_begin(t);
        p_vector(t);
        step_end(t);
      }
      matrix(IntC<0>{}, T, true, false);
      mid();
      step_end(T);
    }
    store(false);
  } else {
    if (T > 0) {
      step_begin(0);
      mid();
      matrix(IntC<1>{}, 0, false, true);
      step_end(0);
      for (int t = 1; t < T; ++t) {
        step_begin(t);
        ds_vector(t - 1);
        mid();
        matrix(IntC<1>{}, t, true, true);
        step_end(t);
      }
      ds_vector(T - 1);
      mid();
      matrix(IntC<1>{}, T, true, false);
      step_end(T);
    }
    store(true);
  }
}

// ------------------------------------------------------------------------------- dK / dV, query split
// At D = 64 each MFMA carries half the work of D = 128 while the exp / dS work per score
// is the same, and the role split above leaves every exp of a step on the P wave. There
// the pair splits each 64-query step instead: both waves hold K and V, and each computes
// S, dP, P and dS for its own 32 queries and accumulates its own partial dK^T and dV^T
// (16 MFMAs and 16 exps per lane and step on each side, no P hand-over). At the end the
// half-0 wave stores dK and the half-1 wave dV, each adding the partner's partial handed
// over through the idle stage memory (own + other: the same sum bitwise either way).
// Holding K, V and both accumulators fits two waves per SIMD only at D <= 64.
template <int DQK, int DV>
struct DkdvSplitSmem {
  static constexpr int QPC = DualPitch<DQK>::value, OPC = DualPitch<DV>::value;
  static constexpr int QP = QPC * 16, OP = OPC * 16;   // bytes
  static constexpr int QB = kQS * QP, OB = kQS * OP;
  static constexpr int LB = 1024;                      // lse2[64], D[64], 512 bytes unused
  static constexpr int STAGE = QB + OB + LB;
  static constexpr int NST = (4 * STAGE <= 148 * 1024) ? 4 : 3;
  static constexpr int BYTES = NST * STAGE;
  // closing exchange: 8 waves x the other wave's accumulator blocks x 4 KiB
  static constexpr int XBYTES = 8 * ((DQK > DV ? DQK : DV) / 32) * 4096;
  static_assert(XBYTES <= BYTES, "the closing exchange reuses the stages");
};

// One matrix phase of the query-split dK / dV pass (items as in dq_matrix):
//   NDV items dv[i / 2] += dO^T P (A: transposed dO reads at t_o, queries + 16 (i % 2), head
//     dims + 32 (i / 2); B = pb[i % 2]), NDK items dk[..] += Q^T dS (transposed Q reads at
//     t_q; B = dsb), NS items s += Q K^T (16-byte Q row reads at r_q + 32 ks; B = kf[ks]),
//     NP items dp += dO V^T (dO row reads at r_o + 32 ks; B = vf[ks]).
template <int NDV, int NDK, int NS, int NP, int QP, int OP, int AHEAD>
__device__ __forceinline__ void dkdv_matrix(const char* t_o, const char* t_q, const char* r_q, const char* r_o,
                                            bool do_acc, bool do_s, f32x16 (&dv)[NDV / 2], f32x16 (&dk)[NDK / 2],
                                            const bf16x8 (&pb)[2], const bf16x8 (&dsb)[2], f32x16& s, f32x16& dp,
                                            const bf16x8 (&kf)[NS], const bf16x8 (&vf)[NP]) {
  constexpr int NA = NDV + NDK, N = NA + NS + NP;
  auto load = [&](int i) -> bf16x8 {
    if (i < NDV) {
      const char* tp = t_o + 16 * (i & 1) * OP + 64 * (i >> 1);
      return join_bf16x8(lds_read_tr(tp), lds_read_tr(tp + 4 * OP));
    }
    if (i < NA) {
      const int j = i - NDV;
      const char* tp = t_q + 16 * (j & 1) * QP + 64 * (j >> 1);
      return join_bf16x8(lds_read_tr(tp), lds_read_tr(tp + 4 * QP));
    }
    if (i < NA + NS) return *(const bf16x8*)(r_q + 32 * (i - NA));
    return *(const bf16x8*)(r_o + 32 * (i - NA - NS));
  };
  auto run = [&](int i, const bf16x8& a) {
    if (i < NDV) dv[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[i & 1], dv[i >> 1], 0, 0, 0);
    else if (i < NA) dk[(i - NDV) >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, dsb[(i - NDV) & 1], dk[(i - NDV) >> 1], 0, 0, 0);
    else if (i < NA + NS) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[i - NA], s, 0, 0, 0);
    else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[i - NA - NS], dp, 0, 0, 0);
  };
  const int first = do_acc ? 0 : NA, last = do_s ? N : NA;
  if (do_s) {
    s = f32x16{};
    dp = f32x16{};
  }
  bf16x8 ring[AHEAD];
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

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dkdv_split_kernel(const BwdParams bp) {
  using SM = DkdvSplitSmem<DQK, DV>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, bp.grid_padded_kv);
  if (bid >= bp.total_work_kv) return;
  // work item: (batch b, K/V head hk, key tile kt); grouped query heads walked in order
  const int G = p.group > 1 ? p.group : 1;
  const int Hkv = p.H / G;
  const int kt0 = bid - (bid / bp.n_kv_tiles) * bp.n_kv_tiles;
  const int bhk = work_bh<LISTS>(p, bid / bp.n_kv_tiles, Hkv);
  const int b = bhk / Hkv, hk = bhk - (bhk / Hkv) * Hkv;
  const int h0 = hk * G;
  const int tid = threadIdx.x;
  // under lists without a band order (causal and prefix-LM walks already shrink with the
  // tile index) the transposed list lengths set the order (fixed lengths under lists)
  const int kt = (LISTS && !p.longest_first)
                     ? ranked_tile<kThreads>(p.lists,
                                             ((int64_t)b * p.lists.heads + (p.lists.heads == 1 ? 0 : h0)) * p.lists.n_rows,
                                             bp.n_kv_tiles, kKB, 0, p.Nk, kt0, (int*)smem, tid)
                     : kt0;
  const int k0 = kt * kKB;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  const int half = w >> 2;     // queries 32 half .. 32 half + 31 of every step
  const int pair = w & 3;      // waves w and w + 4 share a SIMD and the same 32 keys
  const SeqInfo sq = seq_info(p, b);
  const int Nq = sq.nq, Nk = sq.nk, delta = Nk - Nq;
  if (k0 >= Nk) return;        // packed sequences: past this one's keys (whole workgroup, no barrier yet)
  const int kw = k0 + 32 * pair;
  const int key = kw + lq;

  const __bf16* Qg = (const __bf16*)p.q + row_base(sq, true, b, p.qs_b, p.qs_s) + h0 * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + row_base(sq, false, b, p.ks_b, p.ks_s) + hk * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + row_base(sq, false, b, p.vs_b, p.vs_s) + hk * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + row_base(sq, true, b, bp.dos_b, bp.dos_s) + h0 * bp.dos_h;
  const char* WSg = (const char*)(bp.ws + ((int64_t)b * p.H + h0) * bp.n_qblk * 128);

  // ---- query-step sequence (as in the role-split pass)
  TileSeq<kQS> seq;
  seq.t_lo = 0;
  seq.ent = (const uint32_t*)(smem + SM::BYTES + 16);
  const int mk = p.mask.kind;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nq;
    if (mk == kMaskCausal || mk == kMaskWindow) lo = max(0, k0 - delta);
    if (mk == kMaskPrefix) lo = (k0 < p.mask.prefix) ? 0 : max(0, k0 - delta);
    if (mk == kMaskWindow) hi = min(Nq, k0 + kKB - 1 - delta + p.mask.window + 1);
    lo = min(lo, Nq);
    seq.t_lo = lo / kQS;
    seq.count = max(0, (hi + kQS - 1) / kQS - seq.t_lo);
  } else {
    const ListParams& L = p.lists;   // transposed lists: rows = key tiles
    const int64_t row = ((int64_t)b * L.heads + ((L.heads == 1) ? 0 : h0)) * L.n_rows + k0 / L.tile_rows;
    seq.count = build_tile_sequence<kThreads, kQS>(L, row, -1, Nq, smem + SM::BYTES, tid);
  }

  // ---- B operands of S (K) and dP (V): the lane's key, k-slot = head dim
  bf16x8 kf[DQK / 16], vf[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    kf[ks] = key < Nk ? *(const bf16x8*)(Kg + (int64_t)key * p.ks_s + 16 * ks + 8 * g) : bf16x8{};
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    vf[ks] = key < Nk ? *(const bf16x8*)(Vg + (int64_t)key * p.vs_s + 16 * ks + 8 * g) : bf16x8{};

  f32x16 dk[DQK / 32], dv[DV / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dk[i] = f32x16{};
#pragma unroll
  for (int i = 0; i < DV / 32; ++i) dv[i] = f32x16{};
  f32x16 s, dp;
  bf16x8 pb[2], dsb[2];
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);

  // visible queries of the lane's key under the band masks: qlo <= i <= qhi
  int qlo = 0, qhi = 0x3fffffff;
  if (mk == kMaskCausal || mk == kMaskWindow || (mk == kMaskPrefix && key >= p.mask.prefix)) qlo = key - delta;
  if (mk == kMaskWindow) qhi = key - delta + p.mask.window;
  const uint32_t qspan = (uint32_t)qhi - (uint32_t)qlo;
  const int kdoc = (mk == kMaskBlockDiag && key < Nk) ? p.mask.doc_k[(int64_t)b * Nk + key] : 0;
  int need_below = INT32_MIN, need_above = INT32_MAX;
  if (mk == kMaskCausal || mk == kMaskWindow || (mk == kMaskPrefix && kw + 31 >= p.mask.prefix))
    need_below = kw + 31 - delta;
  if (mk == kMaskWindow) need_above = kw - kQS + 1 - delta + p.mask.window;
  if (mk == kMaskBlockDiag) need_below = INT32_MAX;

  LdsDma<kQS, DQK, SM::QPC, kThreads> qdma;
  LdsDma<kQS, DV, SM::OPC, kThreads> odma;
  qdma.init(p.qs_s, tid);
  odma.init(bp.dos_s, tid);
  constexpr int ld_wave = 7;   // a wave with the fewest tile blocks issues the lse2 / D load
  const int per_step = qdma.count() + odma.count() + (w == ld_wave ? 1 : 0);
  zero_lds<kThreads>(smem, SM::NST * SM::STAGE, tid);   // defensive: every slot is loaded before it is read
  const int Tq = seq.count;
  auto head_step = [&](int t, int& gi) {
    if (G == 1) {
      gi = 0;
      return t;
    }
    gi = t / Tq;
    return t - gi * Tq;
  };
  auto issue_step = [&](int t) {
    int gi;
    const int i0 = seq.start(head_step(t, gi), LISTS);
    char* st = smem + (t % SM::NST) * SM::STAGE;
    qdma.issue(Qg + (int64_t)gi * p.qs_h, p.qs_s, i0, Nq, st);
    odma.issue(DOg + (int64_t)gi * bp.dos_h, bp.dos_s, i0, Nq, st + SM::QB);
    if (w == ld_wave)
      dma_16b(WSg + (int64_t)gi * bp.n_qblk * 512, (uint32_t)(i0 / 64) * 512u + 16u * l, st + SM::QB + SM::OB);
  };

  const int T = G * Tq;
  for (int t = 0; t < SM::NST - 2 && t < T; ++t) issue_step(t);
  wait_all_vmem();
  __syncthreads();

  // Steps t = 0 .. T, two phases each; the half-1 waves run one phase behind:
  //   half 0, step t: matrix [dV, dK of step t-1; S, dP of step t], vector P, dS of step t
  //   half 1, step t: vector P, dS of step t-1, matrix [the same as half 0's]
  // Stage t is read during steps t and t+1.
  auto matrix = [&](int ts, bool do_acc, bool do_s) {
    const int sv = ((ts - 1 + SM::NST) % SM::NST) * SM::STAGE, sc = (ts % SM::NST) * SM::STAGE;
    const int trq = (32 * half + trow), rrq = 32 * half + prow;
    const char* t_o = smem + opaque_int(sv + SM::QB + trq * SM::OP + tcol * 2);
    const char* t_q = smem + opaque_int(sv + trq * SM::QP + tcol * 2);
    const char* r_q = smem + opaque_int(sc + rrq * SM::QP + 16 * g);
    const char* r_o = smem + opaque_int(sc + SM::QB + rrq * SM::OP + 16 * g);
    dkdv_matrix<2 * (DV / 32), 2 * (DQK / 32), DQK / 16, DV / 16, SM::QP, SM::OP, 2>(
        t_o, t_q, r_q, r_o, do_acc, do_s, dv, dk, pb, dsb, s, dp, kf, vf);
  };

  // P = exp2(u - lse2) and dS = P (dP - D) [x (1 - tanh^2)] of step ts into pb / dsb;
  // reg r holds query i0 + 32 half + 16 (r / 8) + 8 g + r % 8 of the lane's key
  auto vector = [&](int ts) {
    int gi;
    const int tq = head_step(ts, gi);
    const int i0 = seq.start(tq, LISTS);
    const float* LD = (const float*)(smem + (ts % SM::NST) * SM::STAGE + SM::QB + SM::OB);
    bool need;
    if constexpr (LISTS) need = seq.cls(tq, 0, true) != 2u;
    else need = i0 < need_below || i0 > need_above;
    auto body = [&](auto test_c) {
      constexpr int TEST = decltype(test_c)::value;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int qi = 32 * half + 16 * hh + 8 * g;
        const f32x4 la = *(const f32x4*)(LD + qi), lb = *(const f32x4*)(LD + qi + 4);
        const f32x4 da = *(const f32x4*)(LD + 64 + qi), db4 = *(const f32x4*)(LD + 64 + qi + 4);
        const int qb = (TEST != kTestNone || BIAS) ? opaque_int(i0 + qi) : 0;
        const float dij = (BIAS && !SOFTCAP) ? __int_as_float(opaque_int(__float_as_int((float)(i0 + qi - key)))) : 0.0f;
        u32x4 pk, dk4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv[2], dsv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int ee = 2 * e + z, r = 8 * hh + ee;
            const float lse2 = ee < 4 ? la[ee] : lb[ee - 4];
            const float dd = ee < 4 ? da[ee] : db4[ee - 4];
            const int qidx = qb + ee;
            // x = u - lse2 (one fma without a score transform); rows past Nq carry
            // lse2 = +inf, so their P is 0 whatever the test says
            float dcap = 1.0f, x;
            if constexpr (BIAS && !SOFTCAP)
              x = __builtin_fmaf(s[r], p.scale_log2, __builtin_fmaf(p.bias_log2, __builtin_fabsf(dij + (float)ee), -lse2));
            else if constexpr (SOFTCAP || BIAS) x = score_log2_d<SOFTCAP, BIAS>(s[r], p, qidx, key, dcap) - lse2;
            else x = __builtin_fmaf(s[r], p.scale_log2, -lse2);
            if constexpr (TEST == kTestBand) {
              if ((uint32_t)qidx - (uint32_t)qlo > qspan) x = kNegInf;
            } else if constexpr (TEST == kTestDoc) {
              const int dq = p.mask.doc_q[(int64_t)b * Nq + min(qidx, Nq - 1)];
              if ((qidx < Nq) & (key < Nk) & (dq != kdoc)) x = kNegInf;
            }
            pv[z] = fast_exp2(x);
            dsv[z] = pv[z] * dcap * (dp[r] - dd);
          }
          pk[e] = pack_bf16x2(pv[0], pv[1]);
          dk4[e] = pack_bf16x2(dsv[0], dsv[1]);
        }
        pb[hh] = __builtin_bit_cast(bf16x8, pk);
        dsb[hh] = __builtin_bit_cast(bf16x8, dk4);
      }
    };
    if (!need) body(IntC<kTestNone>{});
    else if (mk != kMaskBlockDiag) body(IntC<kTestBand>{});
    else body(IntC<kTestDoc>{});   // (a vector-load body measured no gain here)
  };

  // Step t refills the stage of step t - 2 (read up to step t - 1) with step t + NST - 2,
  // each wave's share issued at the start of its vector phase (as in the other passes)
  auto step_begin = [&](int t) {
    if (t + SM::NST - 2 < T) issue_step(t + SM::NST - 2);
  };
  auto step_end = [&](int t) {
    const int later = min(SM::NST - 3, max(0, T - 2 - t));
    if (later > 0) wait_vmcnt_at_most(later * per_step);
    else wait_lds_dma();
    __syncthreads();
  };

  if (T > 0) {
    if (half == 0) {
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

  // ---- closing exchange and epilogue: half 0 stores dK, half 1 dV; each hands the other
  // accumulator to its partner through the (idle) stage memory and adds the partner's.
  // Lane = key, reg r of block db <-> d = 32 db + 8 (r / 4) + 4 g + r % 4.
  constexpr int NBM = (DQK > DV ? DQK : DV) / 32;
  auto finish = [&](auto half_c) {
    constexpr int HF = decltype(half_c)::value;
    constexpr int NO = HF == 0 ? DV / 32 : DQK / 32;     // blocks handed over
    constexpr int NK = HF == 0 ? DQK / 32 : DV / 32;     // blocks kept
    f32x4* xo = (f32x4*)(smem + w * NBM * 4096) + l;
    const f32x4* xi = (const f32x4*)(smem + (w ^ 4) * NBM * 4096) + l;
#pragma unroll
    for (int j = 0; j < NO; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& a = HF == 0 ? dv[j] : dk[j];
        xo[64 * (4 * j + c)] = f32x4{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
      }
    __syncthreads();
    if (key >= Nk) return;
    const bool isk = HF == 0;
    __bf16* dst = isk ? (__bf16*)bp.dk + row_base(sq, false, b, bp.dks_b, bp.dks_s) + hk * bp.dks_h + (int64_t)key * bp.dks_s
                      : (__bf16*)bp.dv + row_base(sq, false, b, bp.dvs_b, bp.dvs_s) + hk * bp.dvs_h + (int64_t)key * bp.dvs_s;
    const float sc = isk ? p.scale : 1.0f;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const f32x16& a = HF == 0 ? dk[j] : dv[j];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 o = xi[64 * (4 * j + c)];
        u32x2 v;
        v[0] = pack_bf16x2((a[4 * c] + o[0]) * sc, (a[4 * c + 1] + o[1]) * sc);
        v[1] = pack_bf16x2((a[4 * c + 2] + o[2]) * sc, (a[4 * c + 3] + o[3]) * sc);
        *(u32x2*)(dst + 32 * j + 8 * c + 4 * g) = v;
      }
    }
  };
  if (half == 0) finish(IntC<0>{});
  else finish(IntC<1>{});
}

// ------------------------------------------------------------------------------- dQ, DQK != DV
// Used where the head dims differ (192 / 128): with Q, dO and the wider dQ^T accumulator
// all held by each wave, the key-split pass below would exceed the register budget of two
// waves per SIMD. Here the pair splits the work by role instead: the "S wave" holds Q,
// computes S^T = K Q^T and P and hands P over through LDS; the "dQ wave" holds dO,
// computes dP^T = V dO^T and dS, and accumulates dQ^T += K^T dS^T.
template <int DQK, int DV, bool LISTS>
struct DqRolesSmem {
  static constexpr int KPC = DualPitch<DQK>::value, VPC = RowPitch<DV>::value;
  static constexpr int KP = KPC * 16, VP = VPC * 16;
  static constexpr int KB = kKN * KP, VB = kKN * VP;
  static constexpr int STAGE = KB + VB;
  static constexpr int XB1 = 4 * 64 * 64;              // P hand-over: 4 pairs x 64 lanes x 64 B
  // Double-buffered hand-over (barrier once per tile), and as many stages as then fit:
  // the S and dQ waves have unequal phases (16 vs 32 MFMAs), so a barrier after every
  // phase costs more than the fourth stage gains (measured: 1.95 vs 2.25 ms at the
  // causal 16K D = 128 shape).
  static constexpr bool DBLX = true;
  static constexpr int XB = 2 * XB1;
  static constexpr int NST = (4 * STAGE + XB <= (LISTS ? 148 : 160) * 1024) ? 4 : 3;
  static constexpr int BYTES = NST * STAGE + XB;
};

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dq_roles_kernel(const BwdParams bp) {
  using SM = DqRolesSmem<DQK, DV, LISTS>;
  constexpr int DM = DQK > DV ? DQK : DV;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid >= p.total_work) return;
  const int t = bid - (bid / p.n_tiles) * p.n_tiles;
  const int bh = work_bh<LISTS>(p, bid / p.n_tiles, p.H);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int tid = threadIdx.x;
  // under lists without a band order (causal and prefix-LM walks already shrink from the
  // last tile) the list lengths set the order (fixed lengths under lists)
  const int qt = (LISTS && !p.longest_first)
                     ? ranked_tile<kThreads>(p.lists,
                                             ((int64_t)b * p.lists.heads + (p.lists.heads == 1 ? 0 : h)) * p.lists.n_rows,
                                             p.n_tiles, kQM, 0, p.Nq, t, (int*)smem, tid)
                     : (p.longest_first ? (p.n_tiles - 1 - t) : t);
  const int q0 = qt * kQM;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  const int role = w >> 2;     // 0: S wave (Q; S^T, P), 1: dQ wave (dO; dP^T, dS, dQ^T)
  const int pair = w & 3;      // waves w and w + 4 share a SIMD and the same 32 queries
  const SeqInfo sq = seq_info(p, b);
  const int Nq = sq.nq, Nk = sq.nk, delta = Nk - Nq;
  if (q0 >= Nq) return;        // packed sequences: past this one's queries (whole workgroup, no barrier yet)
  const int qw = q0 + 32 * pair;
  const int qrow = qw + lq;

  const __bf16* Qg = (const __bf16*)p.q + row_base(sq, true, b, p.qs_b, p.qs_s) + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + row_base(sq, false, b, p.ks_b, p.ks_s) + kv_head(p, h) * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + row_base(sq, false, b, p.vs_b, p.vs_s) + kv_head(p, h) * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + row_base(sq, true, b, bp.dos_b, bp.dos_s) + h * bp.dos_h;

  // ---- key-tile sequence (same bands / lists as the forward)
  TileSeq<kKN> seq;
  seq.t_lo = 0;
  seq.ent = (const uint32_t*)(smem + SM::BYTES + 16);
  const int mk = p.mask.kind;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nk;
    if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kQM + delta);
    if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kQM + delta));
    if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
    hi = max(hi, 0);
    seq.t_lo = lo / kKN;
    seq.count = max(0, (hi + kKN - 1) / kKN - seq.t_lo);
  } else {
    const ListParams& L = p.lists;   // the workgroup's 128 queries lie in one sparse row
    const int64_t row = ((int64_t)b * L.heads + ((L.heads == 1) ? 0 : h)) * L.n_rows + q0 / L.tile_rows;
    seq.count = build_tile_sequence<kThreads, kKN>(L, row, -1, Nk, smem + SM::BYTES, tid);
  }

  // ---- B operand of this wave's S^T (Q) or dP^T (dO): the lane's query, k-slot = head dim
  bf16x8 bf[DM / 16];
  {
    const __bf16* src = role ? DOg : Qg;
    const int64_t st = role ? bp.dos_s : p.qs_s;
    const int dr = role ? DV : DQK;
#pragma unroll
    for (int ks = 0; ks < DM / 16; ++ks)
      bf[ks] = (16 * ks < dr && qrow < Nq) ? *(const bf16x8*)(src + (int64_t)qrow * st + 16 * ks + 8 * g) : bf16x8{};
  }
  // lse2 (S wave) or D (dQ wave) of the lane's query
  float rowv = role ? 0.0f : __builtin_huge_valf();
  if (qrow < Nq) rowv = bp.ws[((int64_t)bh * bp.n_qblk + qrow / 64) * 128 + (role ? 64 : 0) + qrow % 64];
  const int dqd = (mk == kMaskBlockDiag && qrow < Nq) ? p.mask.doc_q[(int64_t)b * Nq + qrow] : 0;
  // element-mask geometry, computed once (as in the forward)
  int need_above, need_below;
  key_tile_need(p.mask, qw, Nk, delta, kKN, need_above, need_below);
  if constexpr (LISTS) need_above = Nk - kKN, need_below = INT32_MIN;   // the list classes decide
  int band_lo, band_hi;
  band_interval(p.mask, qrow, Nq, Nk, band_lo, band_hi);

  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const float c_eff = (SOFTCAP || BIAS) ? 1.0f : p.scale_log2;
  u32x4* xch = (u32x4*)(smem + SM::NST * SM::STAGE + pair * 4096) + l;   // + 64 i

  LdsDma<kKN, DQK, SM::KPC, kThreads> kdma;
  LdsDma<kKN, DV, SM::VPC, kThreads> vdma;
  kdma.init(p.ks_s, tid);
  vdma.init(p.vs_s, tid);
  zero_lds<kThreads>(smem, SM::NST * SM::STAGE, tid);   // defensive: every slot is loaded before it is read
  auto issue_tile = [&](int t) {
    const int n0 = seq.start(t, LISTS);
    char* st = smem + (t % SM::NST) * SM::STAGE;
    kdma.issue(Kg, p.ks_s, n0, Nk, st);
    vdma.issue(Vg, p.vs_s, n0, Nk, st + SM::KB);
  };

  f32x16 s[2];
  bf16x8 dsb[2][2];
  const int T = seq.count;
  for (int t = 0; t < SM::NST - 2 && t < T; ++t) issue_tile(t);
  wait_all_vmem();
  __syncthreads();

  // Steps t = 0 .. T, two phases each; the dQ waves run one phase behind the S waves:
  //   S wave,  step t (t < T): matrix  s = S^T of tile t;  vector  P of tile t -> hand-over
  //   dQ wave, step t: vector  dS of tile t-1 from the handed-over P (t > 0);
  //                    matrix  dQ^T += K^T dS^T of tile t-1 (t > 0), s = dP^T of tile t (t < T)
  // The hand-over of tile t is written in phase 2t+1 and read in phase 2t+2; tile t's
  // stage is read during phases 2t .. 2t+3. Each role runs its own loop (first and last
  // steps peeled) so nothing conditional sits between the phases.
  // S^T of tile ts: A = K rows in the permuted order, width DQK
  auto matrix_s = [&](int ts) {
    const char* k0 = smem + opaque_int((ts % SM::NST) * SM::STAGE + prow * SM::KP + 16 * g);
    pipelined_matrix<0, DQK / 16, SM::KP, SM::KP, 2>(k0, k0, false, true, dq, dsb, s, bf);
  };
  // dQ^T += K^T dS^T of tile ts - 1 (K read transposed), then dP^T of tile ts (A = V rows
  // in the permuted order, width DV)
  auto matrix_dq = [&](int ts, bool do_acc, bool do_s) {
    const char* k0 = smem + opaque_int(((ts - 1 + SM::NST) % SM::NST) * SM::STAGE + trow * SM::KP + tcol * 2);
    const char* v0 = smem + opaque_int((ts % SM::NST) * SM::STAGE + SM::KB + prow * SM::VP + 16 * g);
    pipelined_matrix<4 * (DQK / 32), DV / 16, SM::KP, SM::VP, 2>(k0, v0, do_acc, do_s, dq, dsb, s, bf);
  };

  // S wave: P of tile ts (score transform, element mask, exp against the row's lse2) into
  // the hand-over; reg r of block kb holds key n0 + 32 kb + 16 (r / 8) + 8 g + r % 8
  auto p_vector = [&](int ts) {
    const int n0 = seq.start(ts, LISTS);
    bool need = n0 > need_above || n0 < need_below;
    bool elem = true, hide = false;
    if constexpr (LISTS) {
      const uint32_t c = seq.cls(ts, 0, true);
      hide = c == 0u;
      elem = c == 1u;
      need = need || c != 2u;
    }
    // visible keys of the lane's row in this tile: lo <= j < hi (and equal documents);
    // rows past Nq carry rowv = +inf, so their P is 0 whatever the test says
    const int* dkd = p.mask.doc_k + (int64_t)b * Nk;
    // a 64-key tile in bounds with an aligned row: the documents come in vector loads
    const bool dk_wide = n0 + 64 <= Nk && (reinterpret_cast<uintptr_t>(dkd) & 15) == 0;
    const bool bdw = need && !hide && elem && mk == kMaskBlockDiag;   // wave-uniform
    const bool band = elem && mk != kMaskBlockDiag;
    const int lo = band ? band_lo : 0, hi = hide ? 0 : band ? band_hi : Nk;
    const unsigned span = hi > lo ? (unsigned)(hi - lo) : 0u;
    auto body = [&](auto test_c) {
      constexpr int TEST = decltype(test_c)::value;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const int jb = (TEST != kTestNone || BIAS) ? opaque_int(n0 + 32 * kb + 16 * hh + 8 * g) : 0;
          // relative bias alone: i - j = (qrow - jb) - (2 e + z), exact in fp32 (as in the forward)
          const float dij = (BIAS && !SOFTCAP) ? __int_as_float(opaque_int(__float_as_int((float)(qrow - jb)))) : 0.0f;
          int dkv[8];   // documents of keys jb .. jb + 7
          if constexpr (TEST >= kTestDoc) doc_ids8<TEST == kTestDocVec>(dkd, jb, Nk, dkv);
          u32x4 pk;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float pv[2];
#pragma unroll
            for (int z = 0; z < 2; ++z) {
              const int r = 8 * hh + 2 * e + z;
              const int j = jb + 2 * e + z;
              // x = u - lse2, the relative bias folded with -lse2 into one fma
              float dcap = 1.0f, x;
              if constexpr (BIAS && !SOFTCAP)
                x = __builtin_fmaf(s[kb][r], p.scale_log2,
                                   __builtin_fmaf(p.bias_log2, __builtin_fabsf(dij - (float)(2 * e + z)), -rowv));
              else if constexpr (SOFTCAP || BIAS) x = score_log2_d<SOFTCAP, BIAS>(s[kb][r], p, qrow, j, dcap) - rowv;
              else x = __builtin_fmaf(s[kb][r], c_eff, -rowv);
              if constexpr (TEST != kTestNone) {
                bool vis = (unsigned)(j - lo) < span;
                if constexpr (TEST >= kTestDoc) vis = vis & (dkv[2 * e + z] == dqd);
                if (!vis) x = kNegInf;
              }
              pv[z] = fast_exp2(x);
              if constexpr (SOFTCAP) pv[z] *= dcap;
            }
            pk[e] = pack_bf16x2(pv[0], pv[1]);
          }
          xch[(SM::DBLX ? 1024 * (ts & 1) : 0) + 64 * (2 * kb + hh)] = pk;
        }
    };
    if (!need) body(IntC<kTestNone>{});
    else if (!bdw) body(IntC<kTestBand>{});
    else if (dk_wide) body(IntC<kTestDocVec>{});
    else body(IntC<kTestDoc>{});
  };

  // dQ wave: dS = P (dP - D) of tile ts from the handed-over P, into dsb
  auto ds_vector = [&](int ts) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const u32x4 pc = xch[(SM::DBLX ? 1024 * (ts & 1) : 0) + 64 * (2 * kb + hh)];
        u32x4 dk4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pf[2];
          bf16x2_to_f32(pc[e], pf);
          const int r = 8 * hh + 2 * e;
          dk4[e] = pack_bf16x2(pf[0] * (s[kb][r] - rowv), pf[1] * (s[kb][r + 1] - rowv));
        }
        dsb[kb][hh] = __builtin_bit_cast(bf16x8, dk4);
      }
  };

  auto step_begin = [&](int t) {
    if (t + SM::NST - 2 < T) issue_tile(t + SM::NST - 2);
  };
  auto mid = [&]() {   // as in the dK/dV pass
    if (!SM::DBLX) __syncthreads();
  };
  auto step_end = [&](int t) {
    const int later = min(SM::NST - 3, max(0, T - 2 - t));
    if (later > 0) kdma.wait_leaving(vdma, later);
    else wait_lds_dma();
    __syncthreads();
  };

  // ---- epilogue (dQ wave): lane = query, reg r <-> d = 32 db + 8 (r/4) + 4 g + r % 4;
  // on the dQ waves' own path, so the S waves do not keep dq[] live through their loop
  auto store = [&]() {
    if (qrow >= Nq) return;
    __bf16* dQg = (__bf16*)bp.dq + row_base(sq, true, b, bp.dqs_b, bp.dqs_s) + h * bp.dqs_h + (int64_t)qrow * bp.dqs_s;
#pragma unroll
    for (int db = 0; db < DQK / 32; ++db)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        u32x2 v;
        v[0] = pack_bf16x2(dq[db][4 * jj] * p.scale, dq[db][4 * jj + 1] * p.scale);
        v[1] = pack_bf16x2(dq[db][4 * jj + 2] * p.scale, dq[db][4 * jj + 3] * p.scale);
        *(u32x2*)(dQg + 32 * db + 8 * jj + 4 * g) = v;
      }
  };

  if (role == 0) {
    if (T > 0) {
      for (int t = 0; t < T; ++t) {
        step_begin(t);
        matrix_s(t);
        mid();
        p_vector(t);
        step_end(t);
      }
      step_begin(T);
      mid();
      step_end(T);
    }
  } else {
    if (T > 0) {
      step_begin(0);
      mid();
      matrix_dq(0, false, true);
      step_end(0);
      for (int t = 1; t < T; ++t) {
        step_begin(t);
        ds_vector(t - 1);
        mid();
        matrix_dq(t, true, true);
        step_end(t);
      }
      step_begin(T);
      ds_vector(T - 1);
      mid();
      matrix_dq(T, true, false);
      step_end(T);
    }
    store();
  }
}

// ------------------------------------------------------------------------------- dQ
template <int DQK, int DV, bool LISTS>
struct DqSmem {
  static constexpr int KPC = DualPitch<DQK>::value, VPC = RowPitch<DV>::value;
  static constexpr int KP = KPC * 16, VP = VPC * 16;
  static constexpr int KB = kKN * KP, VB = kKN * VP;
  static constexpr int STAGE = KB + VB;
  static constexpr int NST = (4 * STAGE <= (LISTS ? 148 : 160) * 1024) ? 4 : 3;
  static constexpr int BYTES = NST * STAGE;
  // closing exchange of partial dQ^T: 8 waves x DQK / 64 accumulator blocks x 4 KiB
  static constexpr int XBYTES = 8 * (DQK / 64) * 4096;
  static_assert(XBYTES <= BYTES, "the closing exchange reuses the K / V stages");
};

// One matrix phase of the dQ pass as a software pipeline over single-MFMA items:
//   NT items acc[i / 2] += K^T dS^T (A from two transposed 8-byte reads of the K tile at
//      t0, keys + 16 (i % 2), head dims + 32 (i / 2); B = ds[i % 2]),
//   NK items s += K Q^T (A = 16-byte K row read at k0 + 32 ks; B = qf[ks]),
//   NV items dp += V dO^T (A = 16-byte V row read at v0 + 32 ks; B = of[ks]).
// The read of item i + AHEAD is issued right after item i's MFMA and the scheduler is
// fenced per item, so reads stay in flight across the MFMAs (as in pipelined_matrix).
template <int NT, int NK, int NV, int KP, int AHEAD, int NACC>
__device__ __forceinline__ void dq_matrix(const char* t0, const char* k0, const char* v0, bool do_t, bool do_s,
                                          f32x16 (&acc)[NACC], const bf16x8 (&ds)[2], f32x16& s, f32x16& dp,
                                          const bf16x8 (&qf)[NK], const bf16x8 (&of)[NV]) {
  constexpr int N = NT + NK + NV;
  auto load = [&](int i) -> bf16x8 {
    if (i < NT) {
      const char* tp = t0 + 16 * (i & 1) * KP + 64 * (i >> 1);
      return join_bf16x8(lds_read_tr(tp), lds_read_tr(tp + 4 * KP));
    }
    if (i < NT + NK) return *(const bf16x8*)(k0 + 32 * (i - NT));
    return *(const bf16x8*)(v0 + 32 * (i - NT - NK));
  };
  auto run = [&](int i, const bf16x8& a) {
    if (i < NT) acc[i >> 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ds[i & 1], acc[i >> 1], 0, 0, 0);
    else if (i < NT + NK) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[i - NT], s, 0, 0, 0);
    else dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, of[i - NT - NK], dp, 0, 0, 0);
  };
  const int first = do_t ? 0 : NT, last = do_s ? N : NT;
  if (do_s) {
    s = f32x16{};
    dp = f32x16{};
  }
  bf16x8 ring[AHEAD];
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

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
__global__ __launch_bounds__(kThreads, 1)
void bwd_dq_kernel(const BwdParams bp) {
  using SM = DqSmem<DQK, DV, LISTS>;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const AttnParams& p = bp.a;

  const int bid = xcd_remap(blockIdx.x, p.grid_padded);
  if (bid >= p.total_work) return;
  const int t = bid - (bid / p.n_tiles) * p.n_tiles;
  const int bh = work_bh<LISTS>(p, bid / p.n_tiles, p.H);
  const int b = bh / p.H, h = bh - (bh / p.H) * p.H;
  const int tid = threadIdx.x;
  // under lists without a band order (causal and prefix-LM walks already shrink from the
  // last tile) the list lengths set the order (fixed lengths under lists)
  const int qt = (LISTS && !p.longest_first)
                     ? ranked_tile<kThreads>(p.lists,
                                             ((int64_t)b * p.lists.heads + (p.lists.heads == 1 ? 0 : h)) * p.lists.n_rows,
                                             p.n_tiles, kQM, 0, p.Nq, t, (int*)smem, tid)
                     : (p.longest_first ? (p.n_tiles - 1 - t) : t);
  const int q0 = qt * kQM;

  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63, g = l >> 5, lq = l & 31;
  const int half = w >> 2;     // keys 32 half .. 32 half + 31 of every tile
  const int pair = w & 3;      // waves w and w + 4 share a SIMD and the same 32 queries
  const SeqInfo sq = seq_info(p, b);
  const int Nq = sq.nq, Nk = sq.nk, delta = Nk - Nq;
  if (q0 >= Nq) return;        // packed sequences: past this one's queries (whole workgroup, no barrier yet)
  const int qw = q0 + 32 * pair;
  const int qrow = qw + lq;

  const __bf16* Qg = (const __bf16*)p.q + row_base(sq, true, b, p.qs_b, p.qs_s) + h * p.qs_h;
  const __bf16* Kg = (const __bf16*)p.k + row_base(sq, false, b, p.ks_b, p.ks_s) + kv_head(p, h) * p.ks_h;
  const __bf16* Vg = (const __bf16*)p.v + row_base(sq, false, b, p.vs_b, p.vs_s) + kv_head(p, h) * p.vs_h;
  const __bf16* DOg = (const __bf16*)bp.dout + row_base(sq, true, b, bp.dos_b, bp.dos_s) + h * bp.dos_h;

  // ---- key-tile sequence (same bands / lists as the forward)
  TileSeq<kKN> seq;
  seq.t_lo = 0;
  seq.ent = (const uint32_t*)(smem + SM::BYTES + 16);
  const int mk = p.mask.kind;
  if constexpr (!LISTS) {
    int lo = 0, hi = Nk;
    if (mk == kMaskCausal || mk == kMaskWindow) hi = min(Nk, q0 + kQM + delta);
    if (mk == kMaskPrefix) hi = min(Nk, max(p.mask.prefix, q0 + kQM + delta));
    if (mk == kMaskWindow) lo = max(0, q0 + delta - p.mask.window);
    hi = max(hi, 0);
    seq.t_lo = lo / kKN;
    seq.count = max(0, (hi + kKN - 1) / kKN - seq.t_lo);
  } else {
    const ListParams& L = p.lists;   // the workgroup's 128 queries lie in one sparse row
    const int64_t row = ((int64_t)b * L.heads + ((L.heads == 1) ? 0 : h)) * L.n_rows + q0 / L.tile_rows;
    seq.count = build_tile_sequence<kThreads, kKN>(L, row, -1, Nk, smem + SM::BYTES, tid);
  }

  // ---- B operands of S^T (Q) and dP^T (dO): the lane's query, k-slot = head dim
  bf16x8 qf[DQK / 16], of[DV / 16];
#pragma unroll
  for (int ks = 0; ks < DQK / 16; ++ks)
    qf[ks] = qrow < Nq ? *(const bf16x8*)(Qg + (int64_t)qrow * p.qs_s + 16 * ks + 8 * g) : bf16x8{};
#pragma unroll
  for (int ks = 0; ks < DV / 16; ++ks)
    of[ks] = qrow < Nq ? *(const bf16x8*)(DOg + (int64_t)qrow * bp.dos_s + 16 * ks + 8 * g) : bf16x8{};
  // lse2 and D of the lane's query; rows past Nq carry lse2 = +inf, so their P is 0
  float lse2 = __builtin_huge_valf(), dsum = 0.0f;
  if (qrow < Nq) {
    const float* wq = bp.ws + ((int64_t)bh * bp.n_qblk + qrow / 64) * 128 + qrow % 64;
    lse2 = wq[0];
    dsum = wq[64];
  }
  const int dqd = (mk == kMaskBlockDiag && qrow < Nq) ? p.mask.doc_q[(int64_t)b * Nq + qrow] : 0;
  // element-mask geometry, computed once (as in the forward)
  int need_above, need_below;
  key_tile_need(p.mask, qw, Nk, delta, kKN, need_above, need_below);
  if constexpr (LISTS) need_above = Nk - kKN, need_below = INT32_MIN;   // the list classes decide
  int band_lo, band_hi;
  band_interval(p.mask, qrow, Nq, Nk, band_lo, band_hi);

  f32x16 dq[DQK / 32];
#pragma unroll
  for (int i = 0; i < DQK / 32; ++i) dq[i] = f32x16{};
  const int prow = swap_bits23(lq);
  const int trow = 8 * g + ((l & 15) >> 2);
  const int tcol = 16 * ((l >> 4) & 1) + 4 * (l & 3);
  const float c_eff = (SOFTCAP || BIAS) ? 1.0f : p.scale_log2;

  LdsDma<kKN, DQK, SM::KPC, kThreads> kdma;
  LdsDma<kKN, DV, SM::VPC, kThreads> vdma;
  kdma.init(p.ks_s, tid);
  vdma.init(p.vs_s, tid);
  zero_lds<kThreads>(smem, SM::NST * SM::STAGE, tid);   // defensive: every slot is loaded before it is read
  auto issue_tile = [&](int t) {
    const int n0 = seq.start(t, LISTS);
    char* st = smem + (t % SM::NST) * SM::STAGE;
    kdma.issue(Kg, p.ks_s, n0, Nk, st);
    vdma.issue(Vg, p.vs_s, n0, Nk, st + SM::KB);
  };

  f32x16 s, dp;
  bf16x8 ds[2];
  const int T = seq.count;
  for (int t = 0; t < SM::NST - 2 && t < T; ++t) issue_tile(t);
  wait_all_vmem();
  __syncthreads();

  // Steps t = 0 .. T, two phases each. Both waves of a pair do the same work on their own
  // 32 keys of each tile; the half-1 wave runs one phase behind, so one wave's MFMAs
  // overlap the other's vector work on their shared SIMD:
  //   half 0, step t: matrix [dQ^T += K^T dS^T of tile t-1; S^T, dP^T of tile t], vector dS of tile t
  //   half 1, step t: vector dS of tile t-1, matrix [the same as half 0's]
  // Tile t's stage is read during steps t and t+1. No data passes between the waves until
  // the closing exchange.
  auto matrix = [&](int ts, bool do_dq, bool do_s) {
    const int sp = (ts - 1 + SM::NST) % SM::NST, sc = ts % SM::NST;
    const char* t0 = smem + opaque_int(sp * SM::STAGE + (32 * half + trow) * SM::KP + tcol * 2);
    const char* k0 = smem + opaque_int(sc * SM::STAGE + (32 * half + prow) * SM::KP + 16 * g);
    const char* v0 = smem + opaque_int(sc * SM::STAGE + SM::KB + (32 * half + prow) * SM::VP + 16 * g);
    dq_matrix<DQK / 16, DQK / 16, DV / 16, SM::KP, 2>(t0, k0, v0, do_dq, do_s, dq, ds, s, dp, qf, of);
  };

  // dS = P (dP - D) of tile ts (score transform, element mask, exp against the row's lse2)
  // into ds; reg r of s / dp holds key n0 + 32 half + 16 (r / 8) + 8 g + r % 8, so
  // ds[hh] (regs 8 hh .. 8 hh + 7) is the B operand of the dQ^T product as is
  auto vector = [&](int ts) {
    const int n0 = seq.start(ts, LISTS);
    bool need = n0 > need_above || n0 < need_below;
    bool elem = true, hide = false;
    if constexpr (LISTS) {
      const uint32_t c = seq.cls(ts, 0, true);
      hide = c == 0u;
      elem = c == 1u;
      need = need || c != 2u;
    }
    // visible keys of the lane's row in this tile: lo <= j < hi (and equal documents)
    const int* dkd = p.mask.doc_k + (int64_t)b * Nk;
    // a 64-key tile in bounds with an aligned row: the documents come in vector loads
    const bool dk_wide = n0 + 64 <= Nk && (reinterpret_cast<uintptr_t>(dkd) & 15) == 0;
    const bool bdw = need && !hide && elem && mk == kMaskBlockDiag;   // wave-uniform
    const bool band = elem && mk != kMaskBlockDiag;
    const int lo = band ? band_lo : 0, hi = hide ? 0 : band ? band_hi : Nk;
    const unsigned span = hi > lo ? (unsigned)(hi - lo) : 0u;
    auto body = [&](auto test_c) {
      constexpr int TEST = decltype(test_c)::value;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int jb = (TEST != kTestNone || BIAS) ? opaque_int(n0 + 32 * half + 16 * hh + 8 * g) : 0;
        // relative bias alone: i - j = (qrow - jb) - (2 e + z), exact in fp32 (as in the forward)
        const float dij = (BIAS && !SOFTCAP) ? __int_as_float(opaque_int(__float_as_int((float)(qrow - jb)))) : 0.0f;
        int dkv[8];   // documents of keys jb .. jb + 7
        if constexpr (TEST >= kTestDoc) doc_ids8<TEST == kTestDocVec>(dkd, jb, Nk, dkv);
        u32x4 pk;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float dv[2];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const int r = 8 * hh + 2 * e + z;
            const int j = jb + 2 * e + z;
            // x = u - lse2, the relative bias folded with -lse2 into one fma
            float dcap = 1.0f, x;
            if constexpr (BIAS && !SOFTCAP)
              x = __builtin_fmaf(s[r], p.scale_log2,
                                 __builtin_fmaf(p.bias_log2, __builtin_fabsf(dij - (float)(2 * e + z)), -lse2));
            else if constexpr (SOFTCAP || BIAS) x = score_log2_d<SOFTCAP, BIAS>(s[r], p, qrow, j, dcap) - lse2;
            else x = __builtin_fmaf(s[r], c_eff, -lse2);
            if constexpr (TEST != kTestNone) {
              bool vis = (unsigned)(j - lo) < span;
              if constexpr (TEST >= kTestDoc) vis = vis & (dkv[2 * e + z] == dqd);
              if (!vis) x = kNegInf;
            }
            float pv = fast_exp2(x);
            if constexpr (SOFTCAP) pv *= dcap;
            dv[z] = pv * (dp[r] - dsum);
          }
          pk[e] = pack_bf16x2(dv[0], dv[1]);
        }
        ds[hh] = __builtin_bit_cast(bf16x8, pk);
      }
    };
    if (!need) body(IntC<kTestNone>{});
    else if (!bdw) body(IntC<kTestBand>{});
    else if (dk_wide) body(IntC<kTestDocVec>{});
    else body(IntC<kTestDoc>{});
  };

  // End of step t: tile t + 1 (read from the next step on) must have landed; the loads of
  // the NST - 3 tiles issued after it may stay in flight.
  auto step_end = [&](int t) {
    const int later = min(SM::NST - 3, max(0, T - 2 - t));
    if (later > 0) kdma.wait_leaving(vdma, later);
    else wait_lds_dma();
    __syncthreads();
  };

  // Step t refills the stage of tile t - 2 (read up to step t - 1) with tile t + NST - 2;
  // each wave issues its share at the start of its vector phase, where the time the
  // vector-memory path takes to accept the loads is hidden under the partner's MFMAs (as
  // in the forward). The half-1 waves have no vector phase in step 0 and issue first.
  auto step_begin = [&](int t) {
    if (t + SM::NST - 2 < T) issue_tile(t + SM::NST - 2);
  };

  if (T > 0) {
    if (half == 0) {
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

  // ---- closing exchange and epilogue: each wave holds dQ^T over its own keys; it keeps
  // head-dim blocks [half NB, half NB + NB) and hands the other NB to its partner through
  // the (now idle) stage memory. Both add own + other, which is the same sum bitwise in
  // either wave, so the result has one fixed summation order. Lane = query,
  // reg r of block db <-> d = 32 db + 8 (r / 4) + 4 g + r % 4.
  constexpr int NB = DQK / 64;
  auto finish = [&](auto half_c) {
    constexpr int HF = decltype(half_c)::value;
    f32x4* xo = (f32x4*)(smem + w * NB * 4096) + l;
    const f32x4* xi = (const f32x4*)(smem + (w ^ 4) * NB * 4096) + l;
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x16& a = dq[(1 - HF) * NB + j];
        xo[64 * (4 * j + c)] = f32x4{a[4 * c], a[4 * c + 1], a[4 * c + 2], a[4 * c + 3]};
      }
    __syncthreads();
    if (qrow >= Nq) return;
    __bf16* dQg = (__bf16*)bp.dq + row_base(sq, true, b, bp.dqs_b, bp.dqs_s) + h * bp.dqs_h + (int64_t)qrow * bp.dqs_s;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int db = HF * NB + j;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const f32x4 o = xi[64 * (4 * j + c)];
        u32x2 v;
        v[0] = pack_bf16x2((dq[db][4 * c] + o[0]) * p.scale, (dq[db][4 * c + 1] + o[1]) * p.scale);
        v[1] = pack_bf16x2((dq[db][4 * c + 2] + o[2]) * p.scale, (dq[db][4 * c + 3] + o[3]) * p.scale);
        *(u32x2*)(dQg + 32 * db + 8 * c + 4 * g) = v;
      }
    }
  };
  if (half == 0) finish(IntC<0>{});
  else finish(IntC<1>{});
}

hipError_t record_stage(const BwdParams& bp, int i, hipStream_t st) {
  if (bp.stage_events == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(bp.stage_events[i]), st);
}

int list_bytes(const ListParams& L, int unit) { return L.pcnt == nullptr ? 0 : tile_sequence_bytes(L, unit); }

template <int DQK, int DV, bool LISTS, bool SOFTCAP, bool BIAS>
hipError_t launch_passes(const BwdParams& bp, hipStream_t st) {
  {
    hipError_t e0 = record_stage(bp, 1, st);
    if (e0 != hipSuccess) return e0;
    BwdParams kv = bp;
    kv.a.lists = bp.tlists;
    // query-split pass at D <= 64 with equal head dims, role-split pass otherwise
    void (*kern)(const BwdParams);
    int bytes = list_bytes(kv.a.lists, kQS);
    if constexpr (DQK == DV && DQK <= 64) {
      kern = bwd_dkdv_split_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
      bytes += DkdvSplitSmem<DQK, DV>::BYTES;
    } else {
      kern = bwd_dkdv_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
      bytes += DkdvSmem<DQK, DV>::BYTES;
    }
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    if (bp.grid_padded_kv > 0) {   // no keys: no dK / dV to write
      hipLaunchKernelGGL(kern, dim3(bp.grid_padded_kv), dim3(kThreads), bytes, st, kv);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    // key-split pass; role-split pass for unequal head dims
    void (*kern)(const BwdParams);
    int bytes = list_bytes(bp.a.lists, kKN);
    if constexpr (DQK == DV) {
      kern = bwd_dq_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
      bytes += DqSmem<DQK, DV, LISTS>::BYTES;
    } else {
      kern = bwd_dq_roles_kernel<DQK, DV, LISTS, SOFTCAP, BIAS>;
      bytes += DqRolesSmem<DQK, DV, LISTS>::BYTES;
    }
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    e = record_stage(bp, 2, st);
    if (e != hipSuccess) return e;
    if (bp.a.grid_padded > 0) {   // no queries: no dQ to write
      hipLaunchKernelGGL(kern, dim3(bp.a.grid_padded), dim3(kThreads), bytes, st, bp);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return record_stage(bp, 3, st);
  }
}

template <int DQK, int DV>
hipError_t dispatch(const BwdParams& bp, bool lists, bool softcap, bool bias, hipStream_t st) {
  if (lists) {
    if (softcap) return bias ? launch_passes<DQK, DV, true, true, true>(bp, st) : launch_passes<DQK, DV, true, true, false>(bp, st);
    return bias ? launch_passes<DQK, DV, true, false, true>(bp, st) : launch_passes<DQK, DV, true, false, false>(bp, st);
  }
  if (softcap) return bias ? launch_passes<DQK, DV, false, true, true>(bp, st) : launch_passes<DQK, DV, false, true, false>(bp, st);
  return bias ? launch_passes<DQK, DV, false, false, true>(bp, st) : launch_passes<DQK, DV, false, false, false>(bp, st);
}

template <int DQK, int DV>
constexpr int dkdv_smem_bytes() {
  if constexpr (DQK == DV && DQK <= 64) return DkdvSplitSmem<DQK, DV>::BYTES;
  else return DkdvSmem<DQK, DV>::BYTES;
}

template <int DQK, int DV, bool LISTS>
constexpr int dq_smem_bytes() {
  if constexpr (DQK == DV) return DqSmem<DQK, DV, LISTS>::BYTES;
  else return DqRolesSmem<DQK, DV, LISTS>::BYTES;
}

template <int DQK, int DV>
bool lists_fit_dims(const ListParams& fwd, const ListParams& tr) {
  return dkdv_smem_bytes<DQK, DV>() + list_bytes(tr, kQS) <= kMaxLdsBytes &&
         dq_smem_bytes<DQK, DV, true>() + list_bytes(fwd, kKN) <= kMaxLdsBytes;
}

}  // namespace

int bwd_q_block_rows() { return kQM; }
int bwd_kv_block_rows() { return kKB; }

size_t bwd_workspace_bytes(int B, int H, int Nq) {
  const size_t nqb = (size_t)((Nq + 63) / 64);
  return (size_t)B * H * nqb * 128 * sizeof(float) + 512;
}

bool bwd_lists_fit(int dqk, int dv, const ListParams& fwd, const ListParams& tr) {
  if ((int64_t)fwd.n_cols * (fwd.tile_cols / kKN) > (1 << 20) || (int64_t)tr.n_cols * (tr.tile_cols / kQS) > (1 << 20))
    return false;
  if (dqk == 128 && dv == 128) return lists_fit_dims<128, 128>(fwd, tr);
  if (dqk == 64 && dv == 64) return lists_fit_dims<64, 64>(fwd, tr);
  if (dqk == 192 && dv == 128) return lists_fit_dims<192, 128>(fwd, tr);
  return false;
}

// bp.a.lists holds the forward lists (per query tile, walked by the dQ pass) and
// bp.tlists the transposed lists (per key tile, walked by the dK/dV pass).
hipError_t launch_bwd_bf16(BwdParams bp, int dqk, int dv, hipStream_t st) {
  AttnParams& p = bp.a;
  p.n_tiles = (p.Nq + kQM - 1) / kQM;
  p.total_work = p.B * p.H * p.n_tiles;
  p.grid_padded = (p.total_work + 7) / 8 * 8;
  bp.n_kv_tiles = (p.Nk + kKB - 1) / kKB;
  bp.total_work_kv = p.B * (p.H / (p.group > 1 ? p.group : 1)) * bp.n_kv_tiles;   // per K/V head
  bp.grid_padded_kv = (bp.total_work_kv + 7) / 8 * 8;
  bp.n_qblk = (p.Nq + 63) / 64;

  {
    hipError_t e0 = record_stage(bp, 0, st);
    if (e0 != hipSuccess) return e0;
    const int lpk = dv / 8;
    const int64_t rows = (int64_t)p.B * p.H * bp.n_qblk * 64;
    const int rows_per_blk = kPreThreads / lpk;
    const unsigned nblk = (unsigned)((rows + rows_per_blk - 1) / rows_per_blk);
    if (dv != 128 && dv != 64) return hipErrorInvalidValue;
    if (nblk == 0) {}   // no queries: nothing to preprocess
    else if (dv == 128) hipLaunchKernelGGL(bwd_preprocess_kernel<128>, dim3(nblk), dim3(kPreThreads), 0, st, bp);
    else hipLaunchKernelGGL(bwd_preprocess_kernel<64>, dim3(nblk), dim3(kPreThreads), 0, st, bp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const bool lists = p.lists.pcnt != nullptr;
  const bool softcap = p.softcap > 0.0f;
  const bool bias = p.bias_log2 != 0.0f;
  if (dqk == 128 && dv == 128) return dispatch<128, 128>(bp, lists, softcap, bias, st);
  if (dqk == 64 && dv == 64) return dispatch<64, 64>(bp, lists, softcap, bias, st);
  if (dqk == 192 && dv == 128) return dispatch<192, 128>(bp, lists, softcap, bias, st);
  return hipErrorInvalidValue;
}

}  // namespace fmha
