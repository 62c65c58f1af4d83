// Token permutation on gfx950: per-expert token bitmasks, a per-expert prefix
// scan of their popcounts, and a scatter of the routed slots into expert-sorted
// order (the dispatch that precedes the grouped expert GEMMs of InklingMoE on the
// Inkling layers page).
//
// A token never selects the same expert twice, so within an expert the stable
// (ascending slot) order is ascending token order.  Bit t%64 of masks[e][t/64]
// marks token t as routed to expert e; a slot's rank inside its expert is the
// prefix popcount of that expert's mask words before it.  Everything is integer
// arithmetic, so the order is deterministic without sorting.
#include "common.h"
#include "kernels.h"

namespace inkling {

namespace {

constexpr int kMaxExperts = 512;

// grid W = ceil(T/64), block 64: lane = token within the word.
__global__ __launch_bounds__(64) void build_masks_kernel(const int32_t* __restrict__ topk_idx,
                                                         const uint8_t* __restrict__ pad, int T, int E, int k,
                                                         uint64_t* __restrict__ masks, int W) {
    __shared__ unsigned long long m[kMaxExperts];
    const int lane = threadIdx.x, w = blockIdx.x;
    for (int e = lane; e < E; e += 64) m[e] = 0ull;
    __syncthreads();
    const int t = w * 64 + lane;
    if (t < T && (pad == nullptr || pad[t] == 0)) {
        for (int i = 0; i < k; ++i) atomicOr(&m[topk_idx[(size_t)t * k + i]], 1ull << lane);
    }
    __syncthreads();
    for (int e = lane; e < E; e += 64) masks[(size_t)e * W + w] = m[e];
}

// One workgroup of 1024 threads.
__global__ __launch_bounds__(1024) void scan_kernel(const uint64_t* __restrict__ masks, int W, int E,
                                                    int32_t* __restrict__ prefix, int32_t* __restrict__ counts,
                                                    int32_t* __restrict__ offsets, int bm,
                                                    RoutedTile* __restrict__ tiles,
                                                    int32_t* __restrict__ num_tiles,
                                                    int32_t* __restrict__ round_counters) {
    __shared__ int32_t cnt[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t tstart[kMaxExperts + 1];
    const int lane = lane_id(), wv = threadIdx.x >> 6, nw = blockDim.x >> 6;
    if (round_counters != nullptr && threadIdx.x < kRoundCounters) round_counters[threadIdx.x] = 0;
    for (int e = wv; e < E; e += nw) {
        int carry = 0;
        for (int base = 0; base < W; base += 64) {
            const int w = base + lane;
            const int c = w < W ? __popcll(masks[(size_t)e * W + w]) : 0;
            int incl = c;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d);
                if (lane >= d) incl += o;
            }
            if (w < W) prefix[(size_t)e * W + w] = carry + incl - c;
            carry += __shfl(incl, 63);
        }
        if (lane == 0) cnt[e] = carry;
    }
    __syncthreads();
    if (wv == 0) {
        // exclusive scans over experts of the counts and of the row-tile counts
        int carry = 0, tcarry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = e < E ? cnt[e] : 0;
            const int tc = (e < E && bm > 0) ? (c + bm - 1) / bm : 0;
            int incl = c, tincl = tc;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d);
                const int to = __shfl_up(tincl, d);
                if (lane >= d) {
                    incl += o;
                    tincl += to;
                }
            }
            if (e < E) {
                off[e] = carry + incl - c;
                tstart[e] = tcarry + tincl - tc;
            }
            carry += __shfl(incl, 63);
            tcarry += __shfl(tincl, 63);
        }
        if (lane == 0) {
            off[E] = carry;
            tstart[E] = tcarry;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        offsets[e] = off[e];
        if (e < E && counts != nullptr) counts[e] = cnt[e];
    }
    if (tiles != nullptr) {
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            const int n = tstart[e + 1] - tstart[e];
            for (int j = 0; j < n; ++j) tiles[tstart[e] + j] = RoutedTile{e, j * bm};
        }
        if (threadIdx.x == 0) *num_tiles = tstart[E];
    }
}

// grid W, block 64: lane = token within the word.
__global__ __launch_bounds__(64) void scatter_kernel(const int32_t* __restrict__ topk_idx,
                                                     const float* __restrict__ topk_w,
                                                     const uint8_t* __restrict__ pad,
                                                     const uint64_t* __restrict__ masks,
                                                     const int32_t* __restrict__ prefix,
                                                     const int32_t* __restrict__ offsets, int T, int k, int W,
                                                     int32_t* __restrict__ sorted_slots,
                                                     int32_t* __restrict__ row_token, float* __restrict__ row_gamma,
                                                     int32_t* __restrict__ pos) {
    const int lane = threadIdx.x, w = blockIdx.x;
    const int t = w * 64 + lane;
    if (t >= T) return;
    const bool padded = pad != nullptr && pad[t] != 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int i = 0; i < k; ++i) {
        const int slot = t * k + i;
        if (padded) {
            if (pos) pos[slot] = -1;
            continue;
        }
        const int e = topk_idx[slot];
        const int rank = prefix[(size_t)e * W + w] + __popcll(masks[(size_t)e * W + w] & below);
        const int row = offsets[e] + rank;
        if (sorted_slots) sorted_slots[row] = slot;
        if (row_token) row_token[row] = t;
        if (row_gamma) row_gamma[row] = topk_w[slot];
        if (pos) pos[slot] = row;
    }
}

// T <= 64 (a single mask word): the mask, scan and scatter steps above in one
// workgroup, with the masks in LDS and every prefix zero.
__global__ __launch_bounds__(1024) void permute_small_kernel(
    const int32_t* __restrict__ topk_idx, const float* __restrict__ topk_w, const uint8_t* __restrict__ pad, int T,
    int E, int k, int bm, int32_t* __restrict__ counts, int32_t* __restrict__ offsets, RoutedTile* __restrict__ tiles,
    int32_t* __restrict__ num_tiles, int32_t* __restrict__ round_counters, int32_t* __restrict__ sorted_slots,
    int32_t* __restrict__ row_token, float* __restrict__ row_gamma, int32_t* __restrict__ pos) {
    __shared__ unsigned long long m[kMaxExperts];
    __shared__ int32_t off[kMaxExperts + 1];
    __shared__ int32_t tstart[kMaxExperts + 1];
    const int tid = threadIdx.x, lane = lane_id(), wv = tid >> 6;
    const int n_slots = T * k;
    if (round_counters != nullptr && tid < kRoundCounters) round_counters[tid] = 0;
    for (int e = tid; e < E; e += blockDim.x) m[e] = 0ull;
    __syncthreads();
    for (int sl = tid; sl < n_slots; sl += blockDim.x) {
        const int t = sl / k;
        if (pad == nullptr || pad[t] == 0) atomicOr(&m[topk_idx[sl]], 1ull << t);
    }
    __syncthreads();
    if (wv == 0) {
        // exclusive scans over experts of the counts and of the row-tile counts
        int carry = 0, tcarry = 0;
        for (int base = 0; base < E; base += 64) {
            const int e = base + lane;
            const int c = e < E ? __popcll(m[e]) : 0;
            const int tc = (e < E && bm > 0) ? (c + bm - 1) / bm : 0;
            int incl = c, tincl = tc;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int o = __shfl_up(incl, d);
                const int to = __shfl_up(tincl, d);
                if (lane >= d) {
                    incl += o;
                    tincl += to;
                }
            }
            if (e < E) {
                off[e] = carry + incl - c;
                tstart[e] = tcarry + tincl - tc;
            }
            carry += __shfl(incl, 63);
            tcarry += __shfl(tincl, 63);
        }
        if (lane == 0) {
            off[E] = carry;
            tstart[E] = tcarry;
        }
    }
    __syncthreads();
    for (int e = tid; e <= E; e += blockDim.x) {
        offsets[e] = off[e];
        if (e < E && counts != nullptr) counts[e] = __popcll(m[e]);
    }
    if (tiles != nullptr) {
        for (int e = tid; e < E; e += blockDim.x) {
            const int n = tstart[e + 1] - tstart[e];
            for (int j = 0; j < n; ++j) tiles[tstart[e] + j] = RoutedTile{e, j * bm};
        }
        if (tid == 0) *num_tiles = tstart[E];
    }
    for (int sl = tid; sl < n_slots; sl += blockDim.x) {
        const int t = sl / k;
        if (pad != nullptr && pad[t] != 0) {
            if (pos) pos[sl] = -1;
            continue;
        }
        const int e = topk_idx[sl];
        const uint64_t below = (t == 0) ? 0ull : (~0ull >> (64 - t));
        const int row = off[e] + __popcll(m[e] & below);
        if (sorted_slots) sorted_slots[row] = sl;
        if (row_token) row_token[row] = t;
        if (row_gamma) row_gamma[row] = topk_w[sl];
        if (pos) pos[sl] = row;
    }
}

}  // namespace

hipError_t launch_permute_small(const int32_t* topk_idx, const float* topk_w, const uint8_t* pad, int T, int E, int k,
                                int bm, int32_t* counts, int32_t* offsets, RoutedTile* tiles, int32_t* num_tiles,
                                int32_t* round_counters, int32_t* sorted_slots, int32_t* row_token, float* row_gamma,
                                int32_t* pos, hipStream_t stream) {
    hipLaunchKernelGGL(permute_small_kernel, dim3(1), dim3(1024), 0, stream, topk_idx, topk_w, pad, T, E, k, bm, counts,
                       offsets, tiles, num_tiles, round_counters, sorted_slots, row_token, row_gamma, pos);
    return hipGetLastError();
}

hipError_t launch_build_masks(const int32_t* topk_idx, const uint8_t* pad, int T, int E, int k, uint64_t* masks,
                              int W, hipStream_t stream) {
    hipLaunchKernelGGL(build_masks_kernel, dim3(W), dim3(64), 0, stream, topk_idx, pad, T, E, k, masks, W);
    return hipGetLastError();
}

hipError_t launch_scan(const uint64_t* masks, int W, int E, int32_t* prefix, int32_t* counts, int32_t* offsets,
                       int bm, RoutedTile* tiles, int32_t* num_tiles, int32_t* round_counters, hipStream_t stream) {
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(1024), 0, stream, masks, W, E, prefix, counts, offsets, bm, tiles,
                       num_tiles, round_counters);
    return hipGetLastError();
}

hipError_t launch_scatter(const int32_t* topk_idx, const float* topk_w, const uint8_t* pad, const uint64_t* masks,
                          const int32_t* prefix, const int32_t* offsets, int T, int k, int W,
                          int32_t* sorted_slots, int32_t* row_token, float* row_gamma, int32_t* pos,
                          hipStream_t stream) {
    hipLaunchKernelGGL(scatter_kernel, dim3(W), dim3(64), 0, stream, topk_idx, topk_w, pad, masks, prefix, offsets, T,
                       k, W, sorted_slots, row_token, row_gamma, pos);
    return hipGetLastError();
}

}  // namespace inkling
