// Host-side launchers of the gfx950 kernels (each enqueues on `stream`).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace inkling {

// ---- router (router.hip) -------------------------------------------------
// zpart[ks][T][NE] = partial fp64 logits over the ks-th slice of the hidden dim.
hipError_t launch_router_logits(int dtype, const void* x, const float* bank, double* zpart, int T, int H,
                                int NE, int ksplit, hipStream_t stream);
// Sums the partial logits, selects top_k on sigmoid + bias, writes gammas.
hipError_t launch_router_select(const double* zpart, int ksplit, const float* bias, int T, int E, int S, int k,
                                float route_scale, float global_scale, int32_t* topk_idx, float* topk_w,
                                float* shared_g, hipStream_t stream);
int router_ksplit(int T, int H, int NE);

// ---- permutation (permute.hip) -------------------------------------------
hipError_t launch_build_masks(const int32_t* topk_idx, const uint8_t* pad, int T, int E, int k, uint64_t* masks,
                              int W, hipStream_t stream);
// counts / offsets / per-word prefix; optionally the routed tile list for
// row tiles of `bm` rows (tiles may be NULL) and zeroed GEMM round counters
// (kRoundCounters ints, or NULL).
hipError_t launch_scan(const uint64_t* masks, int W, int E, int32_t* prefix, int32_t* counts, int32_t* offsets,
                       int bm, RoutedTile* tiles, int32_t* num_tiles, int32_t* round_counters, hipStream_t stream);
hipError_t launch_scatter(const int32_t* topk_idx, const float* topk_w, const uint8_t* pad, const uint64_t* masks,
                          const int32_t* prefix, const int32_t* offsets, int T, int E, int k, int W,
                          int32_t* sorted_slots, int32_t* row_token, float* row_gamma, int32_t* pos,
                          hipStream_t stream);

// ---- grouped GEMMs and combine (gemm.hip) ---------------------------------
struct MoeGemmParams {
    int dtype;       // 0 f32, 1 bf16: x, weights, act
    int out_dtype;   // 0 f32, 1 bf16: out
    int cfg;         // tile configuration id (see gemm.hip)
    int T, H, E, S, I, k;
    const void* x;
    const void* w_gu;     // [E][2I][H]
    const void* w_d;      // [E][H][I]
    const void* wsh_gu;   // [S][2I][H]
    const void* wsh_d;    // [S][H][I]
    const RoutedTile* tiles;
    const int32_t* num_tiles;
    const int32_t* offsets;
    const int32_t* row_token;   // sorted row -> token
    const int32_t* row_slot;    // sorted row -> slot t*k + i
    const float* row_gamma;     // sorted row -> gamma
    const float* shared_g;
    const int32_t* pos;         // slot -> sorted row, -1 if not dispatched
    void* act_r;   // [T*k][I] sorted rows
    void* act_sh;  // [T][S*I]
    void* y;       // [T*k][H] fp32, slot rows
    void* ysh;     // [T][H] fp32
    void* out;     // [T][H]
    int32_t* round_counters;   // kRoundCounters ints, zero before gate_up
    int has_routed;            // 0: shared tiles only (dense MLP); tiles / num_tiles unused
    int max_routed_tiles;
};
int gemm_cfg_for(int dtype, int T, int H, int E, int k, int I);
int gemm_cfg_bm(int cfg);
hipError_t launch_gate_up(const MoeGemmParams& p, hipStream_t stream);
// routed (act_r -> y) and shared (act_sh -> ysh) down projections, one launch
hipError_t launch_down(const MoeGemmParams& p, hipStream_t stream);
hipError_t launch_combine(const MoeGemmParams& p, hipStream_t stream);
// gamma[t] = value for t < T; the GEMM round counters zeroed (the dense MLP's
// stand-in for the router and the permutation)
hipError_t launch_dense_prep(float* gamma, int T, float value, int32_t* round_counters, hipStream_t stream);

}  // namespace inkling
