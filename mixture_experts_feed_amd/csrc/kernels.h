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
// z[T][NE] = the partial logits summed over the ksplit slices, in slice order
// (read back with ksplit = 1, they give the same sums bit for bit)
hipError_t launch_logits_sum(const double* zpart, int ksplit, int T, int NE, double* z, hipStream_t stream);

// ---- permutation (permute.hip) -------------------------------------------
hipError_t launch_build_masks(const int32_t* topk_idx, const uint8_t* pad, int T, int E, int k, uint64_t* masks,
                              int W, hipStream_t stream);
// counts / offsets / per-word prefix; optionally the routed tile list for
// row tiles of `bm` rows (tiles may be NULL) and zeroed GEMM round counters
// (kRoundCounters ints, or NULL).
hipError_t launch_scan(const uint64_t* masks, int W, int E, int32_t* prefix, int32_t* counts, int32_t* offsets,
                       int bm, RoutedTile* tiles, int32_t* num_tiles, int32_t* round_counters, hipStream_t stream);
hipError_t launch_scatter(const int32_t* topk_idx, const float* topk_w, const uint8_t* pad, const uint64_t* masks,
                          const int32_t* prefix, const int32_t* offsets, int T, int k, int W,
                          int32_t* sorted_slots, int32_t* row_token, float* row_gamma, int32_t* pos,
                          hipStream_t stream);
// T <= 64: the three steps above in one launch (same outputs)
hipError_t launch_permute_small(const int32_t* topk_idx, const float* topk_w, const uint8_t* pad, int T, int E, int k,
                                int bm, int32_t* counts, int32_t* offsets, RoutedTile* tiles, int32_t* num_tiles,
                                int32_t* round_counters, int32_t* sorted_slots, int32_t* row_token, float* row_gamma,
                                int32_t* pos, hipStream_t stream);

// compute units of the current device, queried once per process (256 if the
// query fails)
int device_cu_count();

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
    void* y;       // [T*k][H] slot rows: fp16 for bf16 layers, fp32 for fp32 ones
    void* ysh;     // [T][H] fp32 shared sums (when the combine is not fused; see launch_down)
    int fused_combine;   // gemm_fused_combine(cfg, T, H, S)
    void* out;     // [T][H]
    float* h_save_r;   // optional: gate_up projection of the routed rows [T*k][2I] fp32 (sorted rows)
    float* h_save_sh;  // optional: ... of the shared experts [T][S*2I] fp32
    int32_t* round_counters;   // kRoundCounters ints, zero before gate_up
    int has_routed;            // 0: shared tiles only (dense MLP); tiles / num_tiles unused
    int max_routed_tiles;
};
// tile configuration: 0 (256 x 256 tiles) unless experts receive <= 48 rows on
// average, then 1 (128 weight rows x 16 tokens)
int gemm_cfg_for(int T, int E, int k);
int gemm_cfg_bm(int cfg);
// whether the combine runs in the epilogue of a shared down launch of its own
// (256 x 256 tiles and at least one round of shared tiles, 256 or more), or the
// shared down tiles join the routed down launch (fp32 sums ysh) and the combine
// kernel follows
bool gemm_fused_combine(int cfg, int T, int H, int S);
hipError_t launch_gate_up(const MoeGemmParams& p, hipStream_t stream);
// routed down projection: act_r rows -> y (one row per slot t*k + i; fp16 for
// bf16 layers, fp32 for fp32 ones); with shared experts and no fused combine,
// the shared down projection in the same launch -> ysh (fp32)
hipError_t launch_down(const MoeGemmParams& p, hipStream_t stream);
// shared down projection (act_sh against the S down weights concatenated along
// K) with the combine in its epilogue: out[t] = shared sum + sum_i y[t*k + i],
// rounded once (S > 0; without routed rows, has_routed = 0, just the shared sum)
hipError_t launch_down_out(const MoeGemmParams& p, hipStream_t stream);
// out[t] = ysh[t] (shared experts) + sum_i y[t*k + i], rounded once: the
// combine when it is not fused, and of a layer without shared experts
hipError_t launch_combine(const MoeGemmParams& p, hipStream_t stream);
// ---- backward GEMMs (gemm.hip) ---------------------------------------------
// h = gate_up(x) (no SwiGLU, fp32) for routed rows [T*k][2I] and shared [T][S*2I]
hipError_t launch_gate_up_raw(const MoeGemmParams& p, void* h_r, void* h_sh, hipStream_t stream);
struct BwdActBufs {
    const void* dout;    // [T][H]
    const void* h_r;     // [T*k][2I] fp32
    const void* h_sh;    // [T][S*2I] fp32
    void* dh_r;          // [T*k][2I]
    void* dh_sh;         // [T][S*2I]
    void* a_r;           // [T*k][I]
    void* a_sh;          // [T][S*I]
    float* dgp_r;        // [T*k][I/64]
    float* dgp_sh;       // [T][S*I/64]
};
// dact = down^T dout per routed row / shared token (the down weights read in
// their stored layout), then the SwiGLU backward: dh, a and partial
// routing-weight gradients (round counters 16..23)
hipError_t launch_dact(const MoeGemmParams& p, const BwdActBufs& b, hipStream_t stream);
// dx rows = gate_up^T dh: routed dh_r -> dx_r [T*k][H] (slot rows; fp16 for bf16 layers, else fp32),
// shared dh_sh [T][S*2I] -> dx_sh [T][H] fp32; the gate_up weights read in
// their stored layout (round counters 8..15)
hipError_t launch_dx(const MoeGemmParams& p, const void* dh_r, const void* dh_sh, void* dx_r, void* dx_sh,
                     hipStream_t stream);
// out_p[m][n] = sum_k B_p[k][m] A_p[k][n] over K rows of the operands for
// problems p < E (routed: rows offsets[p] .. offsets[p+1] of A_r and B_r, K
// padded to poff[p+1] - poff[p] with zero rows of B) and S shared ones (K_s
// rows, the first T of them real; shared problem s at element offsets
// s*a_sh_stride of A_s and s*b_sh_stride of B_s)
struct WgradParams {
    int dtype, E, S, M, N, T;
    const void* A_r;
    const void* B_r;
    const void* A_s;
    const void* B_s;
    const int32_t* poff;
    const int32_t* offsets;
    const void* zero;   // max(M) zeros of the operand type
    int lda_r, ldb_r, lda_s, ldb_s, K_s;
    long long a_sh_stride, b_sh_stride;
    void* out_r;        // fp32, or bf16 when out_bf16
    void* out_s;
    int out_bf16;
    int32_t* counters;   // 8 ints, zero at launch (the tile queue of each XCD)
};
hipError_t launch_wgrad(const WgradParams& w, hipStream_t stream);

// ---- backward, other kernels (backward.hip) --------------------------------
// out[r] = src[row_token[r]] (rows of D elements) for the sorted rows r <
// offsets[E] (at most max_rows)
hipError_t launch_gather_rows(int dtype, const void* src, const int32_t* row_token, const int32_t* offsets, int E,
                              int max_rows, int D, void* out, hipStream_t stream);
// poff [E+1]: experts' row counts rounded up to 64, prefix-summed
hipError_t launch_padded_offsets(const int32_t* counts, int E, int32_t* poff, hipStream_t stream);
// n 32-bit words of zeros (a kernel, so that the call can be graph-captured)
hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream);
hipError_t launch_router_backward(const double* zpart, int ksplit, const int32_t* topk_idx, const int32_t* pos,
                                  const float* dgp_r, const float* dgp_sh, int T, int E, int S, int k, int I,
                                  float route_scale, float global_scale, float* dz, float* dzc, hipStream_t stream);
// dx = dxs (if given) + the token's dispatched routed rows (fp16 when
// row_dtype is 1, else fp32) + sum_j dzc_j bank_j, in fp32 in that order,
// rounded once to out_dtype
hipError_t launch_dx_combine(int row_dtype, int out_dtype, const void* dxr, const float* dxs, const int32_t* pos,
                             const int32_t* topk_idx, const float* dzc, const float* bank, void* dx, int T, int H,
                             int E, int S, int k, hipStream_t stream);
// d bank = dz^T x (fp32), as kBankSplit token-range partials summed in order
hipError_t launch_dbank(int dtype, const float* dz, const void* x, int T, int H, int NE, float* part, float* dbank,
                        hipStream_t stream);
int dbank_partial_floats(int H, int NE);

// gamma[t] = value for t < T; the GEMM round counters zeroed (the dense MLP's
// stand-in for the router and the permutation)
hipError_t launch_dense_prep(float* gamma, int T, float value, int32_t* round_counters, hipStream_t stream);

}  // namespace inkling
