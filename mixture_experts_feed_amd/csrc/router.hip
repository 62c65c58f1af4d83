// InklingGate on gfx950: gate logits in fp64 on the matrix cores, then top-k
// selection on sigmoid + correction bias and the log-sigmoid softmax gammas.
//
// Follows the Inkling layers page (nemo_automodel.components.models.inkling.layers),
// InklingGate and InklingCorrectionBias: the gate bank holds the routed rows
// followed by the shared rows; selection uses sigmoid(logit) + bias; the
// returned weights are softmax(log sigmoid([selected routed || shared] logits))
// scaled by route_scale * global_scale.
//
// Precision: the page fixes fp32 gate operands.  Logits are accumulated here in
// fp64 from the exactly widened fp32 bank and bf16/fp32 hidden states, and
// sigmoid, selection and softmax run in fp64, so the selected experts are those
// of exact arithmetic unless two scores differ by less than ~1e-13.
#include "common.h"
#include "kernels.h"

namespace inkling {

namespace {

constexpr int kTokTile = 64;   // tokens per workgroup (4 waves x 16)
constexpr int kExpTile = 16;   // logits columns per workgroup
constexpr int kKChunk = 32;    // hidden-dim chunk staged in LDS

template <typename TX>
__device__ __forceinline__ void load8(const TX* p, double* v);

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, double* v) {
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = (double)__uint_as_float(w[j] << 16);
        v[2 * j + 1] = (double)__uint_as_float(w[j] & 0xFFFF0000u);
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* p, double* v) {
    float4 a = *reinterpret_cast<const float4*>(p);
    float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// zpart[ks][t][e] = sum over h in slice ks of x[t][h] * bank[e][h], in fp64.
// grid (ceil(T/64), ceil(NE/16), ksplit), block 256: wave w owns tokens
// [16w, 16w+16) of the tile against the tile's 16 bank rows.
template <typename TX>
__global__ __launch_bounds__(256) void router_logits_kernel(const TX* __restrict__ x, const float* __restrict__ bank,
                                                            double* __restrict__ zpart, int T, int H, int NE,
                                                            int klen) {
    __shared__ double xs[kTokTile][kKChunk + 1];
    __shared__ double gs[kExpTile][kKChunk + 1];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int t0 = blockIdx.x * kTokTile, e0 = blockIdx.y * kExpTile, ks = blockIdx.z;
    const int kbeg = ks * klen;
    const int kend = min(H, kbeg + klen);
    f64x4_t acc = {0.0, 0.0, 0.0, 0.0};
    const int xr = tid >> 2, xc = (tid & 3) * 8;
    const int gr = tid >> 4, gc = (tid & 15) * 2;
    for (int k0 = kbeg; k0 < kend; k0 += kKChunk) {
        double v[8];
        const int t = t0 + xr;
        if (t < T) {
            load8<TX>(x + (size_t)t * H + k0 + xc, v);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.0;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) xs[xr][xc + j] = v[j];
        const int e = e0 + gr;
        if (e < NE) {
            float2 g = *reinterpret_cast<const float2*>(bank + (size_t)e * H + k0 + gc);
            gs[gr][gc] = (double)g.x;
            gs[gr][gc + 1] = (double)g.y;
        } else {
            gs[gr][gc] = 0.0;
            gs[gr][gc + 1] = 0.0;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < kKChunk; kk += 4) {
            // A (16 tokens x 4): lane holds A[lane%16][lane/16]; B (4 x 16 bank rows): B[lane/16][lane%16]
            const double a = xs[wv * 16 + (lane & 15)][kk + (lane >> 4)];
            const double b = gs[lane & 15][kk + (lane >> 4)];
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, acc, 0, 0, 0);
        }
        __syncthreads();
    }
    // fp64 16x16x4 result layout: lane holds D[i][j] for rows i = lane/16 + 4*r
    // (r = 0..3) and column j = lane % 16 (unlike the fp32 16x16 layouts, whose
    // rows are 4*(lane/16) + r).
    const int e = e0 + (lane & 15);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = t0 + wv * 16 + (lane >> 4) + 4 * r;
        if (t < T && e < NE) zpart[((size_t)ks * T + t) * NE + e] = acc[r];
    }
}

constexpr int kMaxPerLane = 8;  // experts per lane: n_routed + n_shared <= 512

__device__ __forceinline__ double log_sigmoid(double z) {
    // log sigma(z) = -log(1 + e^-z), evaluated on the side that cannot overflow
    return z >= 0.0 ? -log1p(exp(-z)) : z - log1p(exp(z));
}

// One wave per token.  Lane j holds logits of experts j, j+64, ... .
__global__ __launch_bounds__(256) void router_select_kernel(const double* __restrict__ zpart, int ksplit,
                                                            const float* __restrict__ bias, int T, int E, int S,
                                                            int k, double scale, int32_t* __restrict__ topk_idx,
                                                            float* __restrict__ topk_w,
                                                            float* __restrict__ shared_g) {
    __shared__ double zs[4][512];
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;  // wave-uniform; no block-level barrier below
    const int NE = E + S;
    double sc[kMaxPerLane];
    bool live[kMaxPerLane];
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) {
        const int e = lane + 64 * j;
        live[j] = false;
        sc[j] = 0.0;
        if (e < NE) {
            double z = 0.0;
            for (int s = 0; s < ksplit; ++s) z += zpart[((size_t)s * T + t) * NE + e];
            zs[wv][e] = z;
            if (e < E) {
                sc[j] = 1.0 / (1.0 + exp(-z)) + (double)bias[e];
                live[j] = true;
            }
        }
    }
    // k rounds of a wave-wide argmax; larger score wins, equal scores -> lower index
    int my_sel = -1;   // lane i < k keeps the i-th pick
    for (int i = 0; i < k; ++i) {
        double bs = 0.0;
        int be = 0x7FFFFFFF;
#pragma unroll
        for (int j = 0; j < kMaxPerLane; ++j) {
            const int e = lane + 64 * j;
            if (live[j] && (be == 0x7FFFFFFF || sc[j] > bs || (sc[j] == bs && e < be))) {
                bs = sc[j];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const double os = __shfl_xor(bs, off);
            const int oe = __shfl_xor(be, off);
            if (oe != 0x7FFFFFFF && (be == 0x7FFFFFFF || os > bs || (os == bs && oe < be))) {
                bs = os;
                be = oe;
            }
        }
        // be is now wave-uniform
        if ((be & 63) == lane) {
#pragma unroll
            for (int j = 0; j < kMaxPerLane; ++j)
                if (lane + 64 * j == be) live[j] = false;
        }
        if (lane == i) my_sel = be;
    }
    // gammas: lane i < k -> selected routed expert i; lane k + s -> shared expert s
    double ell = -INFINITY;
    const int n_g = k + S;
    if (lane < k) ell = log_sigmoid(zs[wv][my_sel]);
    else if (lane < n_g) ell = log_sigmoid(zs[wv][E + (lane - k)]);
    double m = ell;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off));
    const double p = lane < n_g ? exp(ell - m) : 0.0;
    double sum = p;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off);
    const double g = p / sum * scale;
    if (lane < k) {
        topk_idx[(size_t)t * k + lane] = my_sel;
        topk_w[(size_t)t * k + lane] = (float)g;
    } else if (lane < n_g) {
        shared_g[(size_t)t * S + (lane - k)] = (float)g;
    }
}

}  // namespace

int router_ksplit(int T, int H, int NE) {
    const int tiles = ((T + kTokTile - 1) / kTokTile) * ((NE + kExpTile - 1) / kExpTile);
    int ks = 1;
    // split the hidden dim until ~512 workgroups exist, keeping >= 256 per slice
    while (tiles * ks * 2 <= 512 && (H / (ks * 2)) >= 256 && (H % (ks * 2 * kKChunk)) == 0) ks *= 2;
    return ks;
}

hipError_t launch_router_logits(int dtype, const void* x, const float* bank, double* zpart, int T, int H, int NE,
                                int ksplit, hipStream_t stream) {
    dim3 grid((T + kTokTile - 1) / kTokTile, (NE + kExpTile - 1) / kExpTile, ksplit);
    const int klen = H / ksplit;
    if (dtype == 1)
        hipLaunchKernelGGL(router_logits_kernel<bf16_t>, grid, dim3(256), 0, stream, (const bf16_t*)x, bank, zpart,
                           T, H, NE, klen);
    else
        hipLaunchKernelGGL(router_logits_kernel<float>, grid, dim3(256), 0, stream, (const float*)x, bank, zpart, T,
                           H, NE, klen);
    return hipGetLastError();
}

hipError_t launch_router_select(const double* zpart, int ksplit, const float* bias, int T, int E, int S, int k,
                                float route_scale, float global_scale, int32_t* topk_idx, float* topk_w,
                                float* shared_g, hipStream_t stream) {
    const double scale = (double)route_scale * (double)global_scale;
    hipLaunchKernelGGL(router_select_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, zpart, ksplit, bias, T, E, S, k,
                       scale, topk_idx, topk_w, shared_g);
    return hipGetLastError();
}

}  // namespace inkling
