// C ABI of libfmha.so: argument validation, parameter packing and kernel dispatch.
// Every check runs on the host before anything is enqueued; nothing throws across the
// ABI. The only state kept between calls is a per-device record of the architecture
// check (gfx950 or not).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/fmha.h"
#include "kernel_common.h"
#include "launch.h"

namespace {

using fmha::AttnParams;
using fmha::BwdParams;
using fmha::ListParams;
using fmha::MaskParams;

bool debug_enabled() {
  const char* e = std::getenv("FMHA_DEBUG");
  return e != nullptr && e[0] != '\0' && e[0] != '0';
}

#define FMHA_LOG(...)                         \
  do {                                        \
    if (debug_enabled()) {                    \
      std::fprintf(stderr, "[fmha] " __VA_ARGS__); \
      std::fputc('\n', stderr);               \
    }                                         \
  } while (0)

// Architecture check, cached per device ordinal: 1 = gfx950, -1 = other, 0 = unknown.
constexpr int kMaxDevices = 64;
int g_arch_ok[kMaxDevices];
std::mutex g_arch_mu;

int check_device() {
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) {
    FMHA_LOG("hipGetDevice failed: %s", hipGetErrorString(ge));
    return FMHA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FMHA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_arch_mu);
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FMHA_ERR_HIP;
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    FMHA_LOG("device %d arch %s", dev, prop.gcnArchName);
  }
  return g_arch_ok[dev] == 1 ? FMHA_OK : FMHA_ERR_UNSUPPORTED;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool strides_ok(const int64_t s[3], int esize) {
  for (int i = 0; i < 3; ++i) {
    if (s[i] < 0) return false;
    if ((s[i] * esize) % 16 != 0) return false;
  }
  return true;
}

// The tile loaders address 64 rows of a tile with 32-bit byte offsets from the tile's
// first row: the sequence stride must keep 64 rows under 2^31 bytes.
bool seq_stride_fits(const int64_t s[3], int esize) { return s[1] * esize * 64 < ((int64_t)1 << 31); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int validate_mask(const fmha_mask& m) {
  if (m.kind < FMHA_MASK_NONE || m.kind > FMHA_MASK_PREFIX_LM) return FMHA_ERR_INVALID_ARG;
  if (m.reserved != 0 || m.window < 0 || m.prefix < 0) return FMHA_ERR_INVALID_ARG;
  if (m.kind == FMHA_MASK_BLOCK_DIAGONAL && (m.doc_q == nullptr || m.doc_k == nullptr))
    return FMHA_ERR_INVALID_ARG;
  return FMHA_OK;
}

MaskParams mask_params(const fmha_mask& m) {
  MaskParams mp;
  mp.kind = m.kind;
  mp.window = m.window;
  mp.prefix = m.prefix;
  mp.doc_q = m.doc_q;
  mp.doc_k = m.doc_k;
  return mp;
}

bool supported_dims(int dtype, int dqk, int dv) {
  if (dtype == FMHA_BF16)
    return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 192 && dv == 128);
  if (dtype == FMHA_FP32) return dqk == dv && (dqk == 64 || dqk == 128 || dqk == 1024);
  return false;
}

// Shape / pointer / stride / option checks shared by every entry point. Q / O / LSE are
// checked whenever there are queries; K / V whenever there are keys and something reads
// them: the forward only with queries, the backward (kv_read_alone) also without, since its
// dK / dV pass then still runs over the keys and writes zeros.
int validate_fwd(const fmha_fwd_args* a, bool kv_read_alone = false) {
  if (a == nullptr) return FMHA_ERR_INVALID_ARG;
  if (a->B < 0 || a->H < 0 || a->Nq < 0 || a->Nk < 0) return FMHA_ERR_INVALID_ARG;
  if (a->reserved2 != 0) return FMHA_ERR_INVALID_ARG;
  if (a->kv_heads < 0 || (a->kv_heads > 0 && a->H % a->kv_heads != 0)) return FMHA_ERR_INVALID_ARG;
  if (a->dtype != FMHA_BF16 && a->dtype != FMHA_FP32) return FMHA_ERR_INVALID_ARG;
  if (!supported_dims(a->dtype, a->Dqk, a->Dv)) return FMHA_ERR_UNSUPPORTED;
  if (!(a->scale > 0.0f) || !std::isfinite(a->scale)) return FMHA_ERR_INVALID_ARG;
  if (!(a->softcap >= 0.0f) || !std::isfinite(a->softcap)) return FMHA_ERR_INVALID_ARG;
  if (!std::isfinite(a->bias_slope)) return FMHA_ERR_INVALID_ARG;
  int rc = validate_mask(a->mask);
  if (rc != FMHA_OK) return rc;
  if (a->dtype == FMHA_FP32 && (a->softcap != 0.0f || a->bias_slope != 0.0f || a->block_sparse != nullptr))
    return FMHA_ERR_UNSUPPORTED;
  const int64_t work = (int64_t)a->B * a->H * ceil_div(a->Nq > a->Nk ? a->Nq : a->Nk, 32);
  if (work > (int64_t)1 << 30) return FMHA_ERR_UNSUPPORTED;
  const bool has_q = (int64_t)a->B * a->H * a->Nq > 0;
  const bool has_k = (int64_t)a->B * a->H * a->Nk > 0 && (has_q || kv_read_alone);
  const int es = a->dtype == FMHA_BF16 ? 2 : 4;
  if (has_q) {
    if (!a->q || !a->o || !a->lse) return FMHA_ERR_INVALID_ARG;
    if (!aligned16(a->q) || !aligned16(a->o)) return FMHA_ERR_INVALID_ARG;
    if (!strides_ok(a->q_stride, es) || !strides_ok(a->o_stride, es)) return FMHA_ERR_INVALID_ARG;
    if (!seq_stride_fits(a->q_stride, es) || !seq_stride_fits(a->o_stride, es)) return FMHA_ERR_UNSUPPORTED;
  }
  if (has_k) {
    if (!a->k || !a->v) return FMHA_ERR_INVALID_ARG;
    if (!aligned16(a->k) || !aligned16(a->v)) return FMHA_ERR_INVALID_ARG;
    if (!strides_ok(a->k_stride, es) || !strides_ok(a->v_stride, es)) return FMHA_ERR_INVALID_ARG;
    if (!seq_stride_fits(a->k_stride, es) || !seq_stride_fits(a->v_stride, es)) return FMHA_ERR_UNSUPPORTED;
  }
  return FMHA_OK;
}

int validate_lists(const fmha_block_sparse* bs, int B, int H, int Nq, int Nk, int dqk, int dv, bool need_transposed) {
  if (bs->reserved != 0) return FMHA_ERR_INVALID_ARG;
  if (bs->tile_m <= 0 || bs->tile_n <= 0) return FMHA_ERR_INVALID_ARG;
  if (bs->n_q_tiles != ceil_div(Nq, bs->tile_m) || bs->n_kv_tiles != ceil_div(Nk, bs->tile_n))
    return FMHA_ERR_INVALID_ARG;
  if (bs->heads != 1 && bs->heads != H) return FMHA_ERR_INVALID_ARG;
  if (!bs->partial_cnt || !bs->partial_idx || !bs->full_cnt || !bs->full_idx) return FMHA_ERR_INVALID_ARG;
  // sparse tiles must be whole multiples of the kernel tiles
  if (bs->tile_m % fmha::fwd_bf16_list_rows() != 0 || bs->tile_n % fmha::fwd_bf16_tile_keys() != 0)
    return FMHA_ERR_UNSUPPORTED;
  if (!need_transposed && !fmha::fwd_bf16_lists_fit(dqk, dv, bs->n_kv_tiles, bs->tile_n))
    return FMHA_ERR_UNSUPPORTED;
  if (need_transposed) {
    if (!bs->t_partial_cnt || !bs->t_partial_idx || !bs->t_full_cnt || !bs->t_full_idx)
      return FMHA_ERR_INVALID_ARG;
    if (bs->tile_n % fmha::bwd_kv_block_rows() != 0 || bs->tile_m % fmha::bwd_q_block_rows() != 0)
      return FMHA_ERR_UNSUPPORTED;
  }
  (void)B;
  return FMHA_OK;
}

// K/V carry one head per query head (kv_heads 0 or H)
bool multi_head(const fmha_fwd_args* a) { return a->kv_heads == 0 || a->kv_heads == a->H; }

AttnParams attn_params(const fmha_fwd_args* a) {
  AttnParams p;
  std::memset(&p, 0, sizeof(p));
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.qs_b = a->q_stride[0]; p.qs_s = a->q_stride[1]; p.qs_h = a->q_stride[2];
  p.ks_b = a->k_stride[0]; p.ks_s = a->k_stride[1]; p.ks_h = a->k_stride[2];
  p.vs_b = a->v_stride[0]; p.vs_s = a->v_stride[1]; p.vs_h = a->v_stride[2];
  p.os_b = a->o_stride[0]; p.os_s = a->o_stride[1]; p.os_h = a->o_stride[2];
  p.B = a->B;
  p.H = a->H;
  p.Nq = a->Nq;
  p.Nk = a->Nk;
  p.scale = a->scale;
  p.scale_log2 = a->scale * fmha::kLog2e;
  p.softcap = a->softcap;
  p.cap_k1 = a->softcap > 0.0f ? a->scale * 2.0f * fmha::kLog2e / a->softcap : 0.0f;
  p.cap_u = a->softcap * fmha::kLog2e;
  p.cap_fixed = (a->softcap > 0.0f && a->bias_slope == 0.0f && 2.0f * p.cap_u <= 100.0f) ? 1 : 0;
  p.kv_splits = 1;
  p.split_tiles = 0;
  p.split_o = nullptr;
  p.split_lse = nullptr;
  p.bias_log2 = a->bias_slope * fmha::kLog2e;
  p.mask = mask_params(a->mask);
  // longest-first query-tile order pays off when tiles carry different key counts
  p.longest_first = (a->mask.kind == FMHA_MASK_CAUSAL || a->mask.kind == FMHA_MASK_PREFIX_LM) ? 1 : 0;
  p.group = a->kv_heads > 0 ? a->H / a->kv_heads : 1;
  return p;
}

ListParams fwd_lists(const fmha_block_sparse* bs) {
  ListParams l;
  std::memset(&l, 0, sizeof(l));
  if (!bs) return l;
  l.pcnt = bs->partial_cnt;
  l.pidx = bs->partial_idx;
  l.fcnt = bs->full_cnt;
  l.fidx = bs->full_idx;
  l.heads = bs->heads;
  l.tile_rows = bs->tile_m;
  l.tile_cols = bs->tile_n;
  l.n_rows = bs->n_q_tiles;
  l.n_cols = bs->n_kv_tiles;
  return l;
}

ListParams bwd_lists(const fmha_block_sparse* bs) {
  ListParams l;
  std::memset(&l, 0, sizeof(l));
  if (!bs) return l;
  l.pcnt = bs->t_partial_cnt;
  l.pidx = bs->t_partial_idx;
  l.fcnt = bs->t_full_cnt;
  l.fidx = bs->t_full_idx;
  l.heads = bs->heads;
  l.tile_rows = bs->tile_n;
  l.tile_cols = bs->tile_m;
  l.n_rows = bs->n_kv_tiles;
  l.n_cols = bs->n_q_tiles;
  return l;
}

// Library-owned scratch of fmha_fwd_splitkv_noalloc: one array per GPU the library runs on,
// held until the process ends. Host code must never pass the array's own name to a kernel or
// copy (on the host it is only a stand-in); it uses the device address that
// hipGetSymbolAddress returns, looked up once per device with that device current.
constexpr size_t kScratchBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = 0;
  const hipError_t ge = hipGetDevice(&dev);
  if (ge != hipSuccess) {
    FMHA_LOG("hipGetDevice failed: %s", hipGetErrorString(ge));
    return FMHA_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return FMHA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      FMHA_LOG("hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return FMHA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return FMHA_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return FMHA_OK;
  FMHA_LOG("HIP error: %s", hipGetErrorString(e));
  return FMHA_ERR_HIP;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

extern "C" {

int fmha_abi_version(void) { return 4; }

const char* fmha_status_string(int status) {
  switch (status) {
    case FMHA_OK: return "FMHA_OK";
    case FMHA_ERR_INVALID_ARG: return "FMHA_ERR_INVALID_ARG";
    case FMHA_ERR_UNSUPPORTED: return "FMHA_ERR_UNSUPPORTED";
    case FMHA_ERR_HIP: return "FMHA_ERR_HIP";
    case FMHA_ERR_WORKSPACE: return "FMHA_ERR_WORKSPACE";
    case FMHA_ERR_SCRATCH_TOO_SMALL: return "FMHA_ERR_SCRATCH_TOO_SMALL";
    default: return "FMHA_ERR_UNKNOWN";
  }
}

// key split the bf16 forward would use for these arguments (splits 1 = none)
static fmha::FwdKeySplit fwd_key_split(const fmha_fwd_args* a) {
  if (a->dtype != FMHA_BF16) return fmha::FwdKeySplit{1, 0};
  const AttnParams p = attn_params(a);
  return fmha::fwd_bf16_key_split(a->B, a->H, a->Nq, a->Nk, p.mask, a->Dqk, a->Dv, a->block_sparse != nullptr);
}

static size_t fwd_split_bytes(const fmha_fwd_args* a, const fmha::FwdKeySplit& ks) {
  return ks.splits > 1 ? align256(fmha::fwd_bf16_split_workspace_bytes(a->B, a->H, a->Nq, a->Dv, ks.splits)) : 0;
}

size_t fmha_fwd_workspace_size(const fmha_fwd_args* a) {
  if (validate_fwd(a) != FMHA_OK || (int64_t)a->B * a->H * a->Nq == 0) return 0;
  return fwd_split_bytes(a, fwd_key_split(a));
}

int fmha_fwd_with_workspace(const fmha_fwd_args* a, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_fwd(a);
  if (rc != FMHA_OK) return rc;
  if ((int64_t)a->B * a->H * a->Nq == 0) return FMHA_OK;
  const fmha::FwdKeySplit ks = fwd_key_split(a);
  const size_t need = fwd_split_bytes(a, ks);
  if (need == 0 || workspace == nullptr || workspace_bytes < need) return fmha_fwd(a, stream);
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0) return FMHA_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  AttnParams p = attn_params(a);
  p.lists = fwd_lists(nullptr);
  p.kv_splits = ks.splits;
  p.split_tiles = ks.tiles;
  const size_t rows = (size_t)a->B * a->H * ((a->Nq + fmha::fwd_bf16_block_rows() - 1) / fmha::fwd_bf16_block_rows()) *
                      ks.splits * fmha::fwd_bf16_block_rows();
  p.split_o = static_cast<float*>(workspace);
  p.split_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * a->Dv * sizeof(float)));
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  FMHA_LOG("fwd bf16 key-split x%d (%d tiles) B=%d H=%d Nq=%d Nk=%d D=%d mask=%d", ks.splits, ks.tiles, a->B, a->H,
           a->Nq, a->Nk, a->Dv, a->mask.kind);
  hipError_t e = fmha::launch_fwd_bf16(p, a->Dqk, a->Dv, st);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(fmha::launch_fwd_split_combine(p, a->Dv, st));
}

int fmha_fwd(const fmha_fwd_args* a, void* stream) {
  int rc = validate_fwd(a);
  if (rc != FMHA_OK) return rc;
  if ((int64_t)a->B * a->H * a->Nq == 0) return FMHA_OK;
  if (a->block_sparse) {
    if (a->dtype != FMHA_BF16) return FMHA_ERR_UNSUPPORTED;
    rc = validate_lists(a->block_sparse, a->B, a->H, a->Nq, a->Nk, a->Dqk, a->Dv, false);
    if (rc != FMHA_OK) return rc;
  }
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  AttnParams p = attn_params(a);
  p.lists = fwd_lists(a->block_sparse);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (a->dtype == FMHA_BF16) {
    FMHA_LOG("fwd bf16 B=%d H=%d Nq=%d Nk=%d Dqk=%d Dv=%d mask=%d lists=%d softcap=%g bias=%g", a->B, a->H,
             a->Nq, a->Nk, a->Dqk, a->Dv, a->mask.kind, a->block_sparse != nullptr, a->softcap, a->bias_slope);
    return hip_status(fmha::launch_fwd_bf16(p, a->Dqk, a->Dv, st));
  }
  FMHA_LOG("fwd fp32 B=%d H=%d Nq=%d Nk=%d D=%d mask=%d", a->B, a->H, a->Nq, a->Nk, a->Dqk, a->mask.kind);
  return hip_status(fmha::launch_fwd_f32(p, a->Dqk, st));
}

int fmha_fwd_varlen(const fmha_fwd_args* a, const fmha_varlen* vl, void* stream) {
  if (a == nullptr || vl == nullptr) return FMHA_ERR_INVALID_ARG;
  int rc = validate_fwd(a);
  if (rc != FMHA_OK) return rc;
  if (vl->reserved != 0 || vl->total_q < 0 || !vl->cu_seqlens_q || !vl->cu_seqlens_k) return FMHA_ERR_INVALID_ARG;
  if (a->dtype != FMHA_BF16 || a->block_sparse != nullptr || a->mask.kind == FMHA_MASK_BLOCK_DIAGONAL)
    return FMHA_ERR_UNSUPPORTED;
  if ((int64_t)a->B * a->H * a->Nq == 0 || vl->total_q == 0) return FMHA_OK;
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  AttnParams p = attn_params(a);
  p.cu_q = vl->cu_seqlens_q;
  p.cu_k = vl->cu_seqlens_k;
  p.used_q = vl->seqused_q;
  p.used_k = vl->seqused_k;
  p.lse_total = vl->total_q;
  FMHA_LOG("fwd varlen bf16 B=%d H=%d maxNq=%d maxNk=%d total_q=%d Dqk=%d Dv=%d mask=%d", a->B, a->H, a->Nq, a->Nk,
           vl->total_q, a->Dqk, a->Dv, a->mask.kind);
  return hip_status(fmha::launch_fwd_bf16(p, a->Dqk, a->Dv, reinterpret_cast<hipStream_t>(stream)));
}

size_t fmha_bwd_workspace_size(int32_t B, int32_t H, int32_t Nq) {
  if (B < 0 || H < 0 || Nq < 0) return 0;
  return align256(fmha::bwd_workspace_bytes(B, H, Nq));
}

// fmha_bwd and fmha_bwd_varlen (vl != nullptr: packed variable-length sequences)
static int bwd_impl(const fmha_fwd_args* a, const fmha_bwd_args* g, const fmha_varlen* vl, void* stream) {
  int rc = validate_fwd(a, true);
  if (rc != FMHA_OK) return rc;
  // grouped K/V heads walk every query head of a group in one dK/dV workgroup, which can
  // only follow one list row: head-broadcast lists only
  if (!multi_head(a) && a->block_sparse != nullptr && a->block_sparse->heads != 1) return FMHA_ERR_UNSUPPORTED;
  if (g == nullptr) return FMHA_ERR_INVALID_ARG;
  if (vl != nullptr) {
    if (vl->reserved != 0 || vl->total_q < 0 || !vl->cu_seqlens_q || !vl->cu_seqlens_k) return FMHA_ERR_INVALID_ARG;
    if (a->block_sparse != nullptr || a->mask.kind == FMHA_MASK_BLOCK_DIAGONAL) return FMHA_ERR_UNSUPPORTED;
  }
  if (a->dtype != FMHA_BF16) return FMHA_ERR_UNSUPPORTED;
  if ((int64_t)a->B * a->H * a->Nq == 0 && (int64_t)a->B * a->H * a->Nk == 0) return FMHA_OK;
  // one side may be empty: no keys gives dQ = 0, no queries dK = dV = 0 (the kernels of
  // the other side see no steps and store zeros); only the non-empty side's buffers are used
  const bool has_q = a->Nq > 0, has_k = a->Nk > 0;
  if ((has_q && (!g->dout || !g->dq)) || (has_k && (!g->dk || !g->dv || !a->k || !a->v)))
    return FMHA_ERR_INVALID_ARG;
  if (!aligned16(g->dout) || !aligned16(g->dq) || !aligned16(g->dk) || !aligned16(g->dv))
    return FMHA_ERR_INVALID_ARG;
  if (!strides_ok(g->do_stride, 2) || !strides_ok(g->dq_stride, 2) || !strides_ok(g->dk_stride, 2) ||
      !strides_ok(g->dv_stride, 2))
    return FMHA_ERR_INVALID_ARG;
  if (!seq_stride_fits(g->do_stride, 2)) return FMHA_ERR_UNSUPPORTED;
  const size_t need = fmha_bwd_workspace_size(a->B, a->H, a->Nq);
  if (g->workspace == nullptr || g->workspace_bytes < need || !aligned16(g->workspace)) return FMHA_ERR_WORKSPACE;
  if (a->block_sparse) {
    rc = validate_lists(a->block_sparse, a->B, a->H, a->Nq, a->Nk, a->Dqk, a->Dv, true);
    if (rc != FMHA_OK) return rc;
  }
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  BwdParams bp;
  std::memset(&bp, 0, sizeof(bp));
  bp.a = attn_params(a);
  bp.a.lists = fwd_lists(a->block_sparse);
  bp.tlists = bwd_lists(a->block_sparse);
  bp.dout = g->dout;
  bp.dq = g->dq;
  bp.dk = g->dk;
  bp.dv = g->dv;
  bp.ws = static_cast<float*>(g->workspace);
  if (!fmha::bwd_lists_fit(a->Dqk, a->Dv, bp.a.lists, bp.tlists)) return FMHA_ERR_UNSUPPORTED;
  bp.dos_b = g->do_stride[0]; bp.dos_s = g->do_stride[1]; bp.dos_h = g->do_stride[2];
  bp.dqs_b = g->dq_stride[0]; bp.dqs_s = g->dq_stride[1]; bp.dqs_h = g->dq_stride[2];
  bp.dks_b = g->dk_stride[0]; bp.dks_s = g->dk_stride[1]; bp.dks_h = g->dk_stride[2];
  bp.dvs_b = g->dv_stride[0]; bp.dvs_s = g->dv_stride[1]; bp.dvs_h = g->dv_stride[2];
  bp.stage_events = g->stage_events;
  if (vl != nullptr) {
    bp.a.cu_q = vl->cu_seqlens_q;
    bp.a.cu_k = vl->cu_seqlens_k;
    bp.a.used_q = vl->seqused_q;
    bp.a.used_k = vl->seqused_k;
    bp.a.lse_total = vl->total_q;
  }
  FMHA_LOG("bwd bf16 B=%d H=%d Nq=%d Nk=%d Dqk=%d Dv=%d mask=%d lists=%d varlen=%d", a->B, a->H, a->Nq, a->Nk,
           a->Dqk, a->Dv, a->mask.kind, a->block_sparse != nullptr, vl != nullptr);
  return hip_status(fmha::launch_bwd_bf16(bp, a->Dqk, a->Dv, reinterpret_cast<hipStream_t>(stream)));
}

int fmha_bwd(const fmha_fwd_args* a, const fmha_bwd_args* g, void* stream) { return bwd_impl(a, g, nullptr, stream); }

int fmha_bwd_varlen(const fmha_fwd_args* a, const fmha_bwd_args* g, const fmha_varlen* vl, void* stream) {
  if (vl == nullptr) return FMHA_ERR_INVALID_ARG;
  return bwd_impl(a, g, vl, stream);
}

size_t fmha_fwd_splitkv_workspace_size(int32_t B, int32_t H, int32_t Nq, int32_t Dv, int32_t num_splits) {
  if (B < 0 || H < 0 || Nq < 0 || Dv <= 0 || num_splits < 1) return 0;
  return fmha::splitkv_workspace_bytes(B, H, Nq, Dv, num_splits);
}

size_t fmha_fwd_splitkv_noalloc_max_bytes(void) { return kScratchBytes; }

int fmha_fwd_splitkv_noalloc(const fmha_fwd_args* a, int32_t num_splits, void* stream) {
  // the size check comes first: it needs no device
  if (a != nullptr && a->B >= 0 && a->H >= 0 && a->Nq >= 0 && a->Dv > 0 && num_splits >= 1 &&
      fmha::splitkv_workspace_bytes(a->B, a->H, a->Nq, a->Dv, num_splits) > kScratchBytes) {
    FMHA_LOG("fmha_fwd_splitkv_noalloc: %zu partial bytes exceed the %zu-byte scratch",
             fmha::splitkv_workspace_bytes(a->B, a->H, a->Nq, a->Dv, num_splits), kScratchBytes);
    return FMHA_ERR_SCRATCH_TOO_SMALL;
  }
  int rc = validate_fwd(a);
  if (rc != FMHA_OK) return rc;
  if (num_splits < 1 || num_splits > 64) return FMHA_ERR_INVALID_ARG;
  if ((int64_t)a->B * a->H * a->Nq == 0) return FMHA_OK;
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  void* ptr = nullptr;
  rc = scratch_address(&ptr);
  if (rc != FMHA_OK) return rc;
  return fmha_fwd_splitkv(a, num_splits, ptr, kScratchBytes, stream);
}

int fmha_fwd_splitkv(const fmha_fwd_args* a, int32_t num_splits, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int rc = validate_fwd(a);
  if (rc != FMHA_OK) return rc;
  if (num_splits < 1 || num_splits > 64) return FMHA_ERR_INVALID_ARG;
  if (a->dtype != FMHA_BF16 || a->block_sparse != nullptr || a->softcap != 0.0f || a->bias_slope != 0.0f)
    return FMHA_ERR_UNSUPPORTED;
  if (a->Dqk != a->Dv || (a->Dqk != 64 && a->Dqk != 128)) return FMHA_ERR_UNSUPPORTED;
  if ((int64_t)a->B * a->H * a->Nq == 0) return FMHA_OK;
  if ((int64_t)a->B * a->H * a->Nq * num_splits > ((int64_t)1 << 31) - 1) return FMHA_ERR_UNSUPPORTED;
  const size_t need = fmha::splitkv_workspace_bytes(a->B, a->H, a->Nq, a->Dv, num_splits);
  if (workspace == nullptr || workspace_bytes < need || !aligned16(workspace)) return FMHA_ERR_WORKSPACE;
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  AttnParams p = attn_params(a);
  const int group = a->kv_heads > 0 ? a->H / a->kv_heads : 1;
  FMHA_LOG("fwd splitkv B=%d H=%d Hkv=%d Nq=%d Nk=%d D=%d splits=%d", a->B, a->H, a->H / group, a->Nq, a->Nk, a->Dv,
           num_splits);
  return hip_status(
      fmha::launch_fwd_splitkv(p, a->Dv, num_splits, group, workspace, reinterpret_cast<hipStream_t>(stream)));
}

int build_block_mask(const fmha_mask* mask, int32_t B, int32_t Hm, int32_t Nq, int32_t Nk, int32_t tile_m,
                     int32_t tile_n, fmha_block_sparse* out, void* stream) {
  if (mask == nullptr || out == nullptr) return FMHA_ERR_INVALID_ARG;
  int rc = validate_mask(*mask);
  if (rc != FMHA_OK) return rc;
  if (B < 1 || Hm < 1 || Nq < 1 || Nk < 1 || tile_m < 1 || tile_n < 1) return FMHA_ERR_INVALID_ARG;
  const int64_t nqt = ceil_div(Nq, tile_m), nkt = ceil_div(Nk, tile_n);
  if (nqt > 65536 || nkt > 65536 || (int64_t)B * Hm * (nqt > nkt ? nqt : nkt) > ((int64_t)1 << 31) - 1)
    return FMHA_ERR_UNSUPPORTED;
  if (!out->partial_cnt || !out->partial_idx || !out->full_cnt || !out->full_idx || !out->t_partial_cnt ||
      !out->t_partial_idx || !out->t_full_cnt || !out->t_full_idx)
    return FMHA_ERR_INVALID_ARG;
  rc = check_device();
  if (rc != FMHA_OK) return rc;
  out->tile_m = tile_m;
  out->tile_n = tile_n;
  out->n_q_tiles = (int32_t)nqt;
  out->n_kv_tiles = (int32_t)nkt;
  out->heads = Hm;
  out->reserved = 0;
  fmha::BlockMaskOut o{out->partial_cnt, out->partial_idx, out->full_cnt, out->full_idx,
                       out->t_partial_cnt, out->t_partial_idx, out->t_full_cnt, out->t_full_idx};
  FMHA_LOG("build_block_mask kind=%d B=%d Hm=%d Nq=%d Nk=%d tile=%dx%d", mask->kind, B, Hm, Nq, Nk, tile_m,
           tile_n);
  return hip_status(fmha::launch_build_block_mask(mask_params(*mask), B, Hm, Nq, Nk, tile_m, tile_n, o,
                                                  reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
