// C ABI of the gfx950 Inkling MoE feed-forward: argument checks, workspace
// layout and the launch sequence (router -> permutation -> grouped GEMMs).
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/inkling_moe.h"
#include "common.h"
#include "kernels.h"

using namespace inkling;

namespace {

thread_local int g_last_hip_error = 0;
thread_local void* const* g_stage_events = nullptr;

inline hipError_t mark(int i, hipStream_t s) {
    if (g_stage_events == nullptr || g_stage_events[i] == nullptr) return hipSuccess;
    return hipEventRecord((hipEvent_t)g_stage_events[i], s);
}

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Layout {
    int ksplit, W, cfg, bm, max_tiles;
    bool fused;
    size_t zpart, topk_idx, topk_w, shared_g, masks, prefix, counts, offsets, tiles, num_tiles, round_counters;
    size_t sorted_slots, row_token, row_gamma, pos, act_r, act_sh, y, ysh, total;
};

int check_dims(const inkling_moe_dims_t* d) {
    if (d == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    if (d->T < 0 || d->hidden <= 0 || d->n_routed <= 0 || d->top_k <= 0 || d->n_shared < 0 ||
        d->intermediate <= 0)
        return INKLING_ERR_INVALID_ARGUMENT;
    if (d->top_k > d->n_routed) return INKLING_ERR_INVALID_ARGUMENT;
    if (d->dtype != INKLING_F32 && d->dtype != INKLING_BF16) return INKLING_ERR_UNSUPPORTED;
    if (d->out_dtype != INKLING_F32 && d->out_dtype != INKLING_BF16) return INKLING_ERR_UNSUPPORTED;
    if (d->hidden % 64 != 0 || d->intermediate % 64 != 0) return INKLING_ERR_UNSUPPORTED;
    if (d->n_routed > 512 || d->n_routed + d->n_shared > 512 || d->top_k > 32 || d->n_shared > 16)
        return INKLING_ERR_UNSUPPORTED;
    // int32 row / slot indices (and token counts padded to 256)
    if (d->T * (int64_t)d->top_k > INT32_MAX - 256) return INKLING_ERR_UNSUPPORTED;
    return INKLING_OK;
}

Layout make_layout(const inkling_moe_dims_t* d) {
    Layout L = {};
    const int64_t T = d->T;
    const int E = d->n_routed, S = d->n_shared, k = d->top_k, H = d->hidden, I = d->intermediate;
    const size_t es = d->dtype == INKLING_BF16 ? 2 : 4;
    const int NE = E + S;
    L.ksplit = router_ksplit((int)T, H, NE);
    L.W = (int)((T + 63) / 64);
    L.cfg = gemm_cfg_for((int)T, E, k);
    L.bm = gemm_cfg_bm(L.cfg);
    L.max_tiles = (int)((T * k + L.bm - 1) / L.bm) + E;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.zpart = take((size_t)L.ksplit * T * NE * sizeof(double));
    L.topk_idx = take((size_t)T * k * 4);
    L.topk_w = take((size_t)T * k * 4);
    L.shared_g = take((size_t)T * S * 4);
    L.masks = take((size_t)E * L.W * 8);
    L.prefix = take((size_t)E * L.W * 4);
    L.counts = take((size_t)E * 4);
    L.offsets = take((size_t)(E + 1) * 4);
    L.tiles = take((size_t)L.max_tiles * sizeof(RoutedTile));
    L.num_tiles = take(4);
    L.round_counters = take(kRoundCounters * 4);
    L.sorted_slots = take((size_t)T * k * 4);
    L.row_token = take((size_t)T * k * 4);
    L.row_gamma = take((size_t)T * k * 4);
    L.pos = take((size_t)T * k * 4);
    L.act_r = take((size_t)T * k * I * es);
    L.act_sh = take((size_t)T * S * I * es);
    L.y = take((size_t)T * k * H * es);   // fp16 rows for bf16 layers, fp32 for fp32 ones
    // fp32 shared sums, unless the routed rows are added in the shared down
    // projection's epilogue
    L.fused = gemm_fused_combine(L.cfg, (int)T, H, S);
    L.ysh = take(S > 0 && !L.fused ? (size_t)T * H * sizeof(float) : 0);
    L.total = o;
    return L;
}

template <typename P>
P* at(void* ws, size_t off) {
    return reinterpret_cast<P*>(reinterpret_cast<uint8_t*>(ws) + off);
}

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return INKLING_ERR_HIP;
}

#define HIP_TRY(expr)                          \
    do {                                       \
        hipError_t _e = (expr);                \
        if (_e != hipSuccess) return hip_fail(_e); \
    } while (0)

int check_gate(const inkling_gate_t* g) {
    if (g == nullptr || g->gate_bank == nullptr || g->correction_bias == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    return INKLING_OK;
}

// Router and permutation shared by both entry points.  Writes the routing
// outputs into `r` (pointers already resolved to caller or workspace buffers).
struct RouteBufs {
    int32_t* topk_idx;
    float* topk_w;
    float* shared_g;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_slots;
    int32_t* row_token;
    float* row_gamma;
    int32_t* pos;
    RoutedTile* tiles;
    int32_t* num_tiles;
};

// z_out: also write the summed logits [T][E+S] there (the training forward);
// z_in: take the logits from there instead of computing them (the backward
// from a training forward's saved buffer: the same sums, so the same routing)
int run_route(const inkling_moe_dims_t* d, const Layout& L, const void* x, const inkling_gate_t* g,
              const uint8_t* pad, const RouteBufs& rb, bool permute, void* ws, hipStream_t s,
              double* z_out = nullptr, const double* z_in = nullptr) {
    const int T = (int)d->T, E = d->n_routed, S = d->n_shared, k = d->top_k, H = d->hidden;
    const double* zp = z_in;
    int ks = 1;
    if (z_in == nullptr) {
        double* zpart = at<double>(ws, L.zpart);
        HIP_TRY(launch_router_logits(d->dtype, x, g->gate_bank, zpart, T, H, E + S, L.ksplit, s));
        if (z_out != nullptr) HIP_TRY(launch_logits_sum(zpart, L.ksplit, T, E + S, z_out, s));
        zp = zpart;
        ks = L.ksplit;
    }
    HIP_TRY(mark(1, s));
    HIP_TRY(launch_router_select(zp, ks, g->correction_bias, T, E, S, k, g->route_scale, g->global_scale,
                                 rb.topk_idx, rb.topk_w, rb.shared_g, s));
    HIP_TRY(mark(2, s));
    if (!permute) return INKLING_OK;
    int32_t* rc = rb.tiles ? at<int32_t>(ws, L.round_counters) : nullptr;
    if (L.W == 1) {
        HIP_TRY(launch_permute_small(rb.topk_idx, rb.topk_w, pad, T, E, k, rb.tiles ? L.bm : 0, rb.counts, rb.offsets,
                                     rb.tiles, rb.num_tiles, rc, rb.sorted_slots, rb.row_token, rb.row_gamma, rb.pos,
                                     s));
    } else {
        uint64_t* masks = at<uint64_t>(ws, L.masks);
        int32_t* prefix = at<int32_t>(ws, L.prefix);
        HIP_TRY(launch_build_masks(rb.topk_idx, pad, T, E, k, masks, L.W, s));
        HIP_TRY(launch_scan(masks, L.W, E, prefix, rb.counts, rb.offsets, rb.tiles ? L.bm : 0, rb.tiles, rb.num_tiles,
                            rc, s));
        HIP_TRY(launch_scatter(rb.topk_idx, rb.topk_w, pad, masks, prefix, rb.offsets, T, k, L.W, rb.sorted_slots,
                               rb.row_token, rb.row_gamma, rb.pos, s));
    }
    HIP_TRY(mark(3, s));
    return INKLING_OK;
}

}  // namespace

// ---- backward -----------------------------------------------------------------
struct BwdLayout {
    Layout F;   // the forward's routing and row buffers
    int Tpad;
    size_t dx_r, dx_sh, h_r, h_sh, dh_r, dh_sh, dgp_r, dgp_sh, dz, dzc, poff, x_sorted, dout_sorted, zero, dbank_part, total;
};

BwdLayout make_bwd_layout(const inkling_moe_dims_t* d) {
    BwdLayout B = {};
    B.F = make_layout(d);
    // every backward GEMM uses the 256x256 tiles (the activation-gradient
    // epilogue sums 64-column slices per wave), so the routed tile list is
    // built for 256-row tiles
    B.F.cfg = 0;
    B.F.bm = gemm_cfg_bm(0);
    B.F.max_tiles = (int)((d->T * d->top_k + B.F.bm - 1) / B.F.bm) + d->n_routed;
    const size_t T = (size_t)d->T, E = d->n_routed, S = d->n_shared, k = d->top_k, H = d->hidden, I = d->intermediate;
    const size_t es = d->dtype == INKLING_BF16 ? 2 : 4;
    B.Tpad = (int)((T + 63) / 64 * 64);
    size_t o = B.F.total;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    B.dx_r = take(T * k * H * es);   // routed dx rows: fp16 for bf16 layers, else fp32
    B.dx_sh = take(T * (S > 0 ? H : 0) * 4);
    B.h_r = take(T * k * 2 * I * 4);
    B.h_sh = take(T * S * 2 * I * 4);
    B.dh_r = take(T * k * 2 * I * es);
    B.dh_sh = take(T * S * 2 * I * es);
    B.dgp_r = take(T * k * (I / 64) * 4);
    B.dgp_sh = take(T * S * (I / 64) * 4);
    B.dz = take(T * (E + S) * 4);
    B.dzc = take(T * (k + S) * 4);
    B.poff = take((E + 1) * 4);
    B.x_sorted = take(T * k * H * es);
    B.dout_sorted = take(T * k * H * es);
    B.zero = take(std::max(H, 2 * I) * 4);
    B.dbank_part = take((size_t)dbank_partial_floats((int)H, (int)(E + S)) * 4);
    B.total = o;
    return B;
}

// ---- InklingDenseMLP ------------------------------------------------------
int check_dense_dims(const inkling_dense_dims_t* d) {
    if (d == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    if (d->T < 0 || d->hidden <= 0 || d->intermediate <= 0) return INKLING_ERR_INVALID_ARGUMENT;
    if (d->dtype != INKLING_F32 && d->dtype != INKLING_BF16) return INKLING_ERR_UNSUPPORTED;
    if (d->out_dtype != INKLING_F32 && d->out_dtype != INKLING_BF16) return INKLING_ERR_UNSUPPORTED;
    if (d->hidden % 64 != 0 || d->intermediate % 64 != 0) return INKLING_ERR_UNSUPPORTED;
    if (d->T > INT32_MAX) return INKLING_ERR_UNSUPPORTED;
    return INKLING_OK;
}

struct DenseLayout {
    size_t gamma, round_counters, act, total;
};

DenseLayout make_dense_layout(const inkling_dense_dims_t* d) {
    DenseLayout L = {};
    const size_t T = (size_t)d->T, es = d->dtype == INKLING_BF16 ? 2 : 4;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        size_t at = o;
        o = align_up(o + bytes);
        return at;
    };
    L.gamma = take(T * 4);
    L.round_counters = take(kRoundCounters * 4);
    L.act = take(T * (size_t)d->intermediate * es);
    L.total = o;
    return L;
}

extern "C" {

int inkling_moe_workspace_size(const inkling_moe_dims_t* dims, size_t* bytes) {
    int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (bytes == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    *bytes = make_layout(dims).total;
    return INKLING_OK;
}

int inkling_moe_route(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                      const uint8_t* padding_mask, inkling_route_out_t* r, void* workspace, size_t workspace_bytes,
                      void* stream) {
    int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T == 0) return INKLING_OK;
    if (x == nullptr || (rc = check_gate(gate)) != INKLING_OK) return INKLING_ERR_INVALID_ARGUMENT;
    if (r == nullptr || r->topk_indices == nullptr || r->topk_weights == nullptr ||
        (dims->n_shared > 0 && r->shared_gammas == nullptr))
        return INKLING_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace == nullptr || workspace_bytes < L.total) return INKLING_ERR_WORKSPACE;
    RouteBufs rb = {};
    rb.topk_idx = r->topk_indices;
    rb.topk_w = r->topk_weights;
    rb.shared_g = r->shared_gammas ? r->shared_gammas : at<float>(workspace, L.shared_g);
    const bool permute = r->expert_counts || r->expert_offsets || r->sorted_slots;
    rb.counts = r->expert_counts;
    rb.offsets = r->expert_offsets ? r->expert_offsets : at<int32_t>(workspace, L.offsets);
    rb.sorted_slots = r->sorted_slots;
    return run_route(dims, L, x, gate, padding_mask, rb, permute, workspace, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// the forward; with `saved`, the gate_up projections are also written there
// (fp32: routed rows [T*k][2I] in expert-sorted order, then shared [T][S*2I])
// saved buffer of the training forward: the gate_up projections h (fp32,
// [T*k][2I] by expert-sorted row, then [T][S*2I]), then the gate logits z
// (fp64, [T][E+S])
size_t saved_h_bytes(const inkling_moe_dims_t* d) {
    return (size_t)d->T * (size_t)(d->top_k + d->n_shared) * 2 * (size_t)d->intermediate * sizeof(float);
}
size_t saved_bytes(const inkling_moe_dims_t* d) {
    return saved_h_bytes(d) + (size_t)d->T * (size_t)(d->n_routed + d->n_shared) * sizeof(double);
}
double* saved_logits(const inkling_moe_dims_t* d, const void* saved) {
    return reinterpret_cast<double*>(static_cast<char*>(const_cast<void*>(saved)) + saved_h_bytes(d));
}

int forward_impl(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                 const inkling_experts_t* w, const uint8_t* padding_mask, void* out, inkling_route_out_t* r,
                 void* saved, void* workspace, size_t workspace_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T == 0) return INKLING_OK;
    if (x == nullptr || out == nullptr || check_gate(gate) != INKLING_OK || w == nullptr)
        return INKLING_ERR_INVALID_ARGUMENT;
    if (w->routed_gate_up == nullptr || w->routed_down == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    if (dims->n_shared > 0 && (w->shared_gate_up == nullptr || w->shared_down == nullptr))
        return INKLING_ERR_INVALID_ARGUMENT;
    if (out == x) return INKLING_ERR_INVALID_ARGUMENT;
    const Layout L = make_layout(dims);
    if (workspace == nullptr || workspace_bytes < L.total) return INKLING_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    RouteBufs rb = {};
    rb.topk_idx = (r && r->topk_indices) ? r->topk_indices : at<int32_t>(workspace, L.topk_idx);
    rb.topk_w = (r && r->topk_weights) ? r->topk_weights : at<float>(workspace, L.topk_w);
    rb.shared_g = (r && r->shared_gammas) ? r->shared_gammas : at<float>(workspace, L.shared_g);
    rb.counts = (r && r->expert_counts) ? r->expert_counts : at<int32_t>(workspace, L.counts);
    rb.offsets = (r && r->expert_offsets) ? r->expert_offsets : at<int32_t>(workspace, L.offsets);
    rb.sorted_slots = (r && r->sorted_slots) ? r->sorted_slots : at<int32_t>(workspace, L.sorted_slots);
    rb.row_token = at<int32_t>(workspace, L.row_token);
    rb.row_gamma = at<float>(workspace, L.row_gamma);
    rb.pos = at<int32_t>(workspace, L.pos);
    rb.tiles = at<RoutedTile>(workspace, L.tiles);
    rb.num_tiles = at<int32_t>(workspace, L.num_tiles);
    HIP_TRY(mark(0, s));
    rc = run_route(dims, L, x, gate, padding_mask, rb, true, workspace, s,
                   saved != nullptr ? saved_logits(dims, saved) : nullptr);
    if (rc != INKLING_OK) return rc;

    MoeGemmParams p = {};
    p.dtype = dims->dtype;
    p.out_dtype = dims->out_dtype;
    p.cfg = L.cfg;
    p.T = (int)dims->T;
    p.H = dims->hidden;
    p.E = dims->n_routed;
    p.S = dims->n_shared;
    p.I = dims->intermediate;
    p.k = dims->top_k;
    p.x = x;
    p.w_gu = w->routed_gate_up;
    p.w_d = w->routed_down;
    p.wsh_gu = w->shared_gate_up;
    p.wsh_d = w->shared_down;
    p.tiles = rb.tiles;
    p.num_tiles = rb.num_tiles;
    p.offsets = rb.offsets;
    p.row_token = rb.row_token;
    p.row_slot = rb.sorted_slots;
    p.row_gamma = rb.row_gamma;
    p.shared_g = rb.shared_g;
    p.pos = rb.pos;
    p.act_r = at<void>(workspace, L.act_r);
    p.act_sh = at<void>(workspace, L.act_sh);
    p.y = at<void>(workspace, L.y);
    p.ysh = at<void>(workspace, L.ysh);
    p.fused_combine = L.fused ? 1 : 0;
    p.out = out;
    p.max_routed_tiles = L.max_tiles;
    p.round_counters = at<int32_t>(workspace, L.round_counters);
    p.has_routed = 1;
    if (saved != nullptr) {
        p.h_save_r = static_cast<float*>(saved);
        p.h_save_sh = p.h_save_r + (size_t)dims->T * dims->top_k * 2 * dims->intermediate;
    }
    HIP_TRY(launch_gate_up(p, s));
    HIP_TRY(mark(4, s));
    HIP_TRY(launch_down(p, s));
    HIP_TRY(mark(5, s));
    if (L.fused) HIP_TRY(launch_down_out(p, s));
    else HIP_TRY(launch_combine(p, s));
    HIP_TRY(mark(6, s));
    return INKLING_OK;
}


}  // namespace

extern "C" {

int inkling_moe_forward(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                        const inkling_experts_t* w, const uint8_t* padding_mask, void* out,
                        inkling_route_out_t* r, void* workspace, size_t workspace_bytes, void* stream) {
    return forward_impl(dims, x, gate, w, padding_mask, out, r, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the forward with a static scratch (no workspace argument) ----------------
namespace {

// One array per GPU, in the library's device code: each device it runs on
// holds its own copy from the module's load until the process ends.  In host
// code the name `scratch` is a host-side stand-in, not a device address; the
// device address comes from hipGetSymbolAddress, taken once per device with
// that device current, and only that address is ever passed on.
__device__ __align__(256) uint8_t scratch[INKLING_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_of_current_device(void** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return INKLING_ERR_UNSUPPORTED;
    void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (p == nullptr) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
        if (p == nullptr) {
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess || p == nullptr) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol);
            g_scratch_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *ptr = p;
    return INKLING_OK;
}

}  // namespace

extern "C" {

int inkling_moe_forward_noalloc(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                                const inkling_experts_t* w, const uint8_t* padding_mask, void* out,
                                inkling_route_out_t* r, void* stream) {
    const int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T == 0) return INKLING_OK;
    // every buffer the forward reads is written by it first (its counters are
    // zeroed by the permutation), so what an earlier call left does not matter
    if (make_layout(dims).total > INKLING_NOALLOC_SCRATCH_BYTES) return INKLING_ERR_TOO_LARGE;
    void* ws = nullptr;
    const int rs = scratch_of_current_device(&ws);
    if (rs != INKLING_OK) return rs;
    return forward_impl(dims, x, gate, w, padding_mask, out, r, nullptr, ws, INKLING_NOALLOC_SCRATCH_BYTES, stream);
}

int inkling_moe_saved_size(const inkling_moe_dims_t* dims, size_t* bytes) {
    const int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (bytes == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    *bytes = saved_bytes(dims);
    return INKLING_OK;
}

int inkling_moe_forward_train(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                              const inkling_experts_t* w, const uint8_t* padding_mask, void* out, void* saved,
                              void* workspace, size_t workspace_bytes, void* stream) {
    const int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T > 0 && saved == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    return forward_impl(dims, x, gate, w, padding_mask, out, nullptr, saved, workspace, workspace_bytes, stream);
}

int inkling_dense_mlp_workspace_size(const inkling_dense_dims_t* dims, size_t* bytes) {
    const int rc = check_dense_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (bytes == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    *bytes = make_dense_layout(dims).total;
    return INKLING_OK;
}

int inkling_dense_mlp_forward(const inkling_dense_dims_t* dims, const void* x, const void* gate_up, const void* down,
                              float global_scale, void* out, void* workspace, size_t workspace_bytes, void* stream) {
    const int rc = check_dense_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T == 0) return INKLING_OK;
    if (x == nullptr || gate_up == nullptr || down == nullptr || out == nullptr || out == x)
        return INKLING_ERR_INVALID_ARGUMENT;
    const DenseLayout L = make_dense_layout(dims);
    if (workspace == nullptr || workspace_bytes < L.total) return INKLING_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int T = (int)dims->T, H = dims->hidden, I = dims->intermediate;
    // one always-on expert over every token, its gamma = global_scale
    MoeGemmParams p = {};
    p.dtype = dims->dtype == INKLING_BF16 ? 1 : 0;
    p.out_dtype = dims->out_dtype == INKLING_BF16 ? 1 : 0;
    p.cfg = gemm_cfg_for(T, 1, 1);
    p.T = T;
    p.H = H;
    p.E = 0;
    p.S = 1;
    p.I = I;
    p.k = 0;
    p.x = x;
    p.wsh_gu = gate_up;
    p.wsh_d = down;
    p.shared_g = at<float>(workspace, L.gamma);
    p.act_sh = at<void>(workspace, L.act);
    p.out = out;
    p.round_counters = at<int32_t>(workspace, L.round_counters);
    p.has_routed = 0;
    HIP_TRY(launch_dense_prep(at<float>(workspace, L.gamma), T, global_scale, p.round_counters, s));
    HIP_TRY(launch_gate_up(p, s));
    HIP_TRY(launch_down_out(p, s));
    return INKLING_OK;
}

int inkling_moe_backward_workspace_size(const inkling_moe_dims_t* dims, size_t* bytes) {
    const int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (bytes == nullptr) return INKLING_ERR_INVALID_ARGUMENT;
    *bytes = make_bwd_layout(dims).total;
    return INKLING_OK;
}

int inkling_moe_backward(const inkling_moe_dims_t* dims, const void* x, const inkling_gate_t* gate,
                         const inkling_experts_t* w, const uint8_t* padding_mask, const void* dout,
                         const void* saved, void* dx, inkling_moe_grads_t* g, void* workspace,
                         size_t workspace_bytes, void* stream) {
    int rc = check_dims(dims);
    if (rc != INKLING_OK) return rc;
    if (dims->T == 0) return INKLING_OK;
    if (x == nullptr || dout == nullptr || dx == nullptr || check_gate(gate) != INKLING_OK || w == nullptr ||
        g == nullptr)
        return INKLING_ERR_INVALID_ARGUMENT;
    const int S = dims->n_shared;
    if (w->routed_gate_up == nullptr || w->routed_down == nullptr ||
        (S > 0 && (w->shared_gate_up == nullptr || w->shared_down == nullptr)))
        return INKLING_ERR_INVALID_ARGUMENT;
    if (g->d_gate_bank == nullptr || g->d_routed_gate_up == nullptr || g->d_routed_down == nullptr ||
        (S > 0 && (g->d_shared_gate_up == nullptr || g->d_shared_down == nullptr)))
        return INKLING_ERR_INVALID_ARGUMENT;
    if (g->weight_grad_dtype != INKLING_F32 && g->weight_grad_dtype != INKLING_BF16) return INKLING_ERR_UNSUPPORTED;
    if (dx == x || dx == dout) return INKLING_ERR_INVALID_ARGUMENT;
    const BwdLayout B = make_bwd_layout(dims);
    const Layout& L = B.F;
    if (workspace == nullptr || workspace_bytes < B.total) return INKLING_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    const int T = (int)dims->T, E = dims->n_routed, k = dims->top_k, H = dims->hidden, I = dims->intermediate;
    const int dt = dims->dtype == INKLING_BF16 ? 1 : 0;

    // 1. routing and permutation, as in the forward
    RouteBufs rb = {};
    rb.topk_idx = at<int32_t>(workspace, L.topk_idx);
    rb.topk_w = at<float>(workspace, L.topk_w);
    rb.shared_g = at<float>(workspace, L.shared_g);
    rb.counts = at<int32_t>(workspace, L.counts);
    rb.offsets = at<int32_t>(workspace, L.offsets);
    rb.sorted_slots = at<int32_t>(workspace, L.sorted_slots);
    rb.row_token = at<int32_t>(workspace, L.row_token);
    rb.row_gamma = at<float>(workspace, L.row_gamma);
    rb.pos = at<int32_t>(workspace, L.pos);
    rb.tiles = at<RoutedTile>(workspace, L.tiles);
    rb.num_tiles = at<int32_t>(workspace, L.num_tiles);
    // routing: from the training forward's logits when they were kept
    const double* z_kept = saved != nullptr ? saved_logits(dims, saved) : nullptr;
    rc = run_route(dims, L, x, gate, padding_mask, rb, true, workspace, s, nullptr, z_kept);
    if (rc != INKLING_OK) return rc;
    int32_t* poff = at<int32_t>(workspace, B.poff);
    HIP_TRY(launch_padded_offsets(rb.counts, E, poff, s));

    MoeGemmParams p = {};
    p.dtype = dt;
    p.out_dtype = dims->out_dtype == INKLING_BF16 ? 1 : 0;
    p.cfg = L.cfg;
    p.T = T;
    p.H = H;
    p.E = E;
    p.S = S;
    p.I = I;
    p.k = k;
    p.x = x;
    p.w_gu = w->routed_gate_up;
    p.w_d = w->routed_down;
    p.wsh_gu = w->shared_gate_up;
    p.wsh_d = w->shared_down;
    p.tiles = rb.tiles;
    p.num_tiles = rb.num_tiles;
    p.offsets = rb.offsets;
    p.row_token = rb.row_token;
    p.row_slot = rb.sorted_slots;
    p.row_gamma = rb.row_gamma;
    p.shared_g = rb.shared_g;
    p.pos = rb.pos;
    p.max_routed_tiles = L.max_tiles;
    p.round_counters = at<int32_t>(workspace, L.round_counters);
    p.has_routed = 1;

    // 2. h = gate_up(x) per routed row and per token for the shared experts:
    //    kept by inkling_moe_forward_train, else recomputed
    const void* h_r;
    const void* h_sh;
    if (saved != nullptr) {
        h_r = saved;
        h_sh = static_cast<const float*>(saved) + (size_t)T * k * 2 * I;
    } else {
        void* hr = at<void>(workspace, B.h_r);
        void* hs = at<void>(workspace, B.h_sh);
        HIP_TRY(launch_gate_up_raw(p, hr, hs, s));
        h_r = hr;
        h_sh = hs;
    }

    // 3. dact and the SwiGLU backward
    BwdActBufs ab = {};
    ab.dout = dout;
    ab.h_r = h_r;
    ab.h_sh = h_sh;
    ab.dh_r = at<void>(workspace, B.dh_r);
    ab.dh_sh = at<void>(workspace, B.dh_sh);
    ab.a_r = at<void>(workspace, L.act_r);
    ab.a_sh = at<void>(workspace, L.act_sh);
    ab.dgp_r = at<float>(workspace, B.dgp_r);
    ab.dgp_sh = at<float>(workspace, B.dgp_sh);
    HIP_TRY(launch_dact(p, ab, s));

    // 4. gate: dz of the selected and shared logits
    float* dz = at<float>(workspace, B.dz);
    float* dzc = at<float>(workspace, B.dzc);
    HIP_TRY(launch_router_backward(z_kept != nullptr ? z_kept : at<double>(workspace, L.zpart),
                                   z_kept != nullptr ? 1 : L.ksplit, rb.topk_idx, rb.pos, ab.dgp_r, ab.dgp_sh,
                                   T, E, S, k, I, gate->route_scale, gate->global_scale, dz, dzc, s));

    // 5. dx rows: the gate_up projections against dh (the down-GEMM shape,
    //    K = 2I); then dx = shared + routed rows + gate term, rounded once
    HIP_TRY(launch_dx(p, ab.dh_r, ab.dh_sh, at<void>(workspace, B.dx_r), at<void>(workspace, B.dx_sh), s));
    HIP_TRY(launch_dx_combine(dt, p.out_dtype, at<void>(workspace, B.dx_r),
                              S > 0 ? at<float>(workspace, B.dx_sh) : nullptr, rb.pos, rb.topk_idx, dzc,
                              gate->gate_bank, dx, T, H, E, S, k, s));

    // 6. gate bank gradient
    HIP_TRY(launch_dbank(dt, dz, x, T, H, E + S, at<float>(workspace, B.dbank_part), g->d_gate_bank, s));

    // 7. weight gradients, contracting over the rows of an expert (or the
    //    tokens): the expert-sorted rows of a and dh as they are, x and dout
    //    gathered into expert order
    void* x_sorted = at<void>(workspace, B.x_sorted);
    void* dout_sorted = at<void>(workspace, B.dout_sorted);
    void* zero = at<void>(workspace, B.zero);
    HIP_TRY(launch_zero_words(static_cast<uint32_t*>(zero), (size_t)std::max(H, 2 * I), s));
    HIP_TRY(launch_gather_rows(dt, x, rb.row_token, rb.offsets, E, T * k, H, x_sorted, s));
    HIP_TRY(launch_gather_rows(dt, dout, rb.row_token, rb.offsets, E, T * k, H, dout_sorted, s));
    WgradParams wd = {};   // d down[e][h][i] = sum_r dout[t(r)][h] a[r][i]
    wd.dtype = dt;
    wd.E = E;
    wd.S = S;
    wd.M = H;
    wd.N = I;
    wd.T = T;
    wd.poff = poff;
    wd.offsets = rb.offsets;
    wd.zero = zero;
    wd.A_r = ab.a_r;
    wd.lda_r = I;
    wd.B_r = dout_sorted;
    wd.ldb_r = H;
    wd.A_s = ab.a_sh;      // [T][S*I], expert s at column s*I
    wd.lda_s = S * I;
    wd.a_sh_stride = I;
    wd.B_s = dout;
    wd.ldb_s = H;
    wd.b_sh_stride = 0;
    wd.K_s = B.Tpad;
    wd.out_r = g->d_routed_down;
    wd.out_s = g->d_shared_down;
    wd.out_bf16 = g->weight_grad_dtype == INKLING_BF16 ? 1 : 0;
    wd.counters = p.round_counters + 24;
    HIP_TRY(launch_wgrad(wd, s));
    WgradParams wg = wd;   // d gate_up[e][n][h] = sum_r dh[r][n] x[t(r)][h]
    wg.M = 2 * I;
    wg.N = H;
    wg.A_r = x_sorted;
    wg.lda_r = H;
    wg.B_r = ab.dh_r;
    wg.ldb_r = 2 * I;
    wg.A_s = x;
    wg.lda_s = H;
    wg.a_sh_stride = 0;
    wg.B_s = ab.dh_sh;     // [T][S*2I], expert s at column s*2I
    wg.ldb_s = S * 2 * I;
    wg.b_sh_stride = (long long)2 * I;
    wg.out_r = g->d_routed_gate_up;
    wg.out_s = g->d_shared_gate_up;
    wg.counters = p.round_counters + 32;
    HIP_TRY(launch_wgrad(wg, s));
    return INKLING_OK;
}

const char* inkling_moe_strerror(int code) {
    switch (code) {
        case INKLING_OK: return "success";
        case INKLING_ERR_INVALID_ARGUMENT: return "invalid argument (null pointer, negative size or top_k > n_routed)";
        case INKLING_ERR_UNSUPPORTED: return "unsupported dtype or size";
        case INKLING_ERR_WORKSPACE: return "workspace missing or too small";
        case INKLING_ERR_HIP: return "HIP launch failed (see inkling_moe_last_hip_error)";
        case INKLING_ERR_TOO_LARGE:
            return "sizes need more scratch than the static array of inkling_moe_forward_noalloc "
                   "(INKLING_NOALLOC_SCRATCH_BYTES); use inkling_moe_forward with a workspace";
        default: return "unknown error code";
    }
}

int inkling_moe_last_hip_error(void) { return g_last_hip_error; }

int inkling_moe_set_stage_events(void* const* events, int n_events) {
    if (events != nullptr && n_events < INKLING_STAGE_EVENTS) return INKLING_ERR_INVALID_ARGUMENT;
    g_stage_events = events;
    return INKLING_OK;
}

}  // extern "C"
