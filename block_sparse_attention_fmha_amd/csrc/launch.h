// Host-side launchers of the HIP kernels (internal to libfmha.so).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_common.h"

namespace fmha {

// bf16 forward: (Dqk, Dv) in {(64,64), (128,128), (192,128)}. Fills the tiling fields
// of `p` (n_tiles, total_work, grid_padded) itself.
hipError_t launch_fwd_bf16(AttnParams p, int dqk, int dv, hipStream_t st);
int fwd_bf16_block_rows();   // query rows per workgroup
int fwd_bf16_list_rows();    // block-sparse tile_m must be a multiple (each half-workgroup reads one sparse row)
int fwd_bf16_tile_keys();    // keys per tile (block-sparse tile_n must be a multiple)
// Whether the merged tile sequence of a list row fits the forward kernel's LDS.
bool fwd_bf16_lists_fit(int dqk, int dv, int n_cols, int tile_cols);
// Key split of the bf16 forward for one launch: at most `splits` parts per query tile, of
// about `tiles` key tiles each (splits 1: none). Only without block-sparse lists and with
// Dqk == Dv in {64, 128}.
struct FwdKeySplit { int splits, tiles; };
FwdKeySplit fwd_bf16_key_split(int B, int H, int Nq, int Nk, const MaskParams& m, int dqk, int dv, bool lists);
size_t fwd_bf16_split_workspace_bytes(int B, int H, int Nq, int dv, int splits);
// Merges the partials of the split query tiles (p as given to launch_fwd_bf16, with
// kv_splits, split_tiles, split_o, split_lse set).
hipError_t launch_fwd_split_combine(AttnParams p, int dv, hipStream_t st);

// fp32 forward, D-split across wavefronts: D in {64, 128, 1024}, Dqk == Dv, analytic masks.
hipError_t launch_fwd_f32(AttnParams p, int d, hipStream_t st);

// bf16 split-KV forward (partials + combine). `ws` holds the partials.
size_t splitkv_workspace_bytes(int B, int H, int Nq, int Dv, int splits);
int splitkv_tile_keys();
// `group` query heads share each K/V head (1 = multi-head).
hipError_t launch_fwd_splitkv(AttnParams p, int d, int splits, int group, void* ws, hipStream_t st);

// bf16 backward: preprocess, dK/dV pass, dQ pass.
hipError_t launch_bwd_bf16(BwdParams p, int dqk, int dv, hipStream_t st);
int bwd_q_block_rows();      // block-sparse tile_m must be a multiple (one sparse row per dQ half-workgroup)
int bwd_kv_block_rows();     // block-sparse tile_n must be a multiple (one sparse row per dK/dV workgroup)
size_t bwd_workspace_bytes(int B, int H, int Nq);
// Whether the merged tile sequences of both list orientations fit the kernels' LDS.
bool bwd_lists_fit(int dqk, int dv, const ListParams& fwd, const ListParams& tr);

// Block-mask builder: forward lists (per query tile) and transposed lists (per key tile).
struct BlockMaskOut {
  int *pcnt, *pidx, *fcnt, *fidx, *tpcnt, *tpidx, *tfcnt, *tfidx;
};
hipError_t launch_build_block_mask(const MaskParams& m, int B, int Hm, int Nq, int Nk,
                                   int tile_m, int tile_n, const BlockMaskOut& out,
                                   hipStream_t st);

}  // namespace fmha
