// Host-side launchers of the gfx950 kernels (one per kernel family).  Each
// enqueues its kernels on `st` and returns the launch status.
#pragma once

#include "common.hpp"

namespace moe {

void router_logits_plan(int T, int H, int ncols, bool bf16, int *mt, int *n_split,
                        int *blocks_per_split);
hipError_t launch_router_logits(const LogitsArgs &a, bool bf16, hipStream_t st);
hipError_t launch_router_select(const SelectArgs &a, hipStream_t st);
hipError_t launch_permute(const PermuteArgs &a, hipStream_t st);

enum WFormat { W_F32 = 0, W_BF16 = 1, W_MXFP4 = 2 };

// Routed or shared expert GEMMs.  `max_groups` bounds the number of active
// groups (host-known), `max_rows` the rows of any group; the launchers size
// their grids from these bounds and read the actual schedule on the device.
hipError_t launch_gate_up(const ExpertGemmArgs &a, WFormat wf, int max_groups, int max_rows,
                          hipStream_t st);
hipError_t launch_down(const ExpertGemmArgs &a, WFormat wf, int max_groups, int max_rows,
                       hipStream_t st);

// Tiled grouped GEMM (large token counts).  max_rows_total bounds the rows of
// all groups together, max_groups the number of groups.
hipError_t launch_tiled(const TiledGemmArgs &t, bool gate_up, WFormat wf, long max_rows_total,
                        int max_groups, hipStream_t st);
int tiled_tile_rows();

hipError_t launch_combine(const CombineArgs &a, bool bf16_out, hipStream_t st);
hipError_t launch_fill_i32(int32_t *p, int32_t v, size_t n, hipStream_t st);

}  // namespace moe
