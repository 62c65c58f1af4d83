// Backward of the Inkling MoE feed-forward on gfx950: the kernels around the
// grouped GEMMs (which live in gemm.hip).
//
// Gradients of L = <dout, out> follow the chain rule through the layer of the
// Inkling layers page (InklingMoE.forward, InklingGate, inkling_swiglu,
// InklingSharedExperts):
//   per routed slot / shared expert: dact = down^T dout, dgamma = dact . p,
//     dh = [dgate, dup] of the SwiGLU times gamma, dx += gate_up^T dh,
//     d down += dout (x) a, d gate_up += dh (x) x;
//   gate: gamma = c softmax(l), l_j = log sigmoid(z_j) over the selected
//     routed and the shared logits, c = route_scale * global_scale:
//     dz_j = q_j (c dgamma_j - sum_m q_m c dgamma_m) (1 - sigmoid(z_j)),
//     dx += sum_j dz_j bank_j, d bank_j = sum_t dz_tj x_t.
// The correction bias only moves the selection and has no gradient.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace inkling {

namespace {

// out[r] = src[row_token[r]] for r < offsets[E]: rows of D elements (D a
// multiple of 64), 16-byte vectors, one row per block iteration.
template <typename TE>
__global__ __launch_bounds__(256) void gather_rows_kernel(const TE* __restrict__ src,
                                                          const int32_t* __restrict__ row_token,
                                                          const int32_t* __restrict__ offsets, int E, int D,
                                                          TE* __restrict__ out) {
    constexpr int V = 16 / sizeof(TE);
    const int rows = offsets[E];
    const int nv = D / V;
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const uint4* s = reinterpret_cast<const uint4*>(src + (size_t)row_token[r] * D);
        uint4* o = reinterpret_cast<uint4*>(out + (size_t)r * D);
        for (int v = threadIdx.x; v < nv; v += 256) o[v] = s[v];
    }
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

// poff[e] = sum over e' < e of counts rounded up to 64 (poff[E] the total);
// one block.
__global__ __launch_bounds__(1024) void padded_offsets_kernel(const int32_t* __restrict__ counts, int E,
                                                              int32_t* __restrict__ poff) {
    __shared__ int32_t sc[1024];
    const int tid = threadIdx.x;
    int carry = 0;
    for (int base = 0; base < E; base += 1024) {
        const int e = base + tid;
        const int v = e < E ? (counts[e] + 63) / 64 * 64 : 0;
        sc[tid] = v;
        __syncthreads();
        for (int d = 1; d < 1024; d <<= 1) {
            const int o = tid >= d ? sc[tid - d] : 0;
            __syncthreads();
            sc[tid] += o;
            __syncthreads();
        }
        if (e < E) poff[e] = carry + sc[tid] - v;
        carry += sc[1023];
        __syncthreads();
    }
    if (tid == 0) poff[E] = carry;
}

// One wave per token: routing-weight gradients (sums of the 64-column
// partials in column order), then the gate-logit gradients of the k selected
// routed and the S shared logits (fp64).  dz [T][E+S] (zeros elsewhere) and
// the compact dzc [T][k+S] (selection order, then shared).
__global__ __launch_bounds__(256) void router_backward_kernel(
    const double* __restrict__ zpart, int ksplit, const int32_t* __restrict__ topk_idx,
    const int32_t* __restrict__ pos, const float* __restrict__ dgp_r, const float* __restrict__ dgp_sh, int T, int E,
    int S, int k, int I, double scale, float* __restrict__ dz, float* __restrict__ dzc) {
    const int lane = lane_id(), wv = threadIdx.x >> 6;
    const int t = blockIdx.x * 4 + wv;
    if (t >= T) return;   // wave-uniform
    const int NE = E + S, nj = k + S, chunks = I / 64;
    // lane j < k + S: expert e_j, its logit, its routing-weight gradient
    double zj = 0.0, dg = 0.0;
    int ej = -1;
    if (lane < nj) {
        if (lane < k) {
            ej = topk_idx[(size_t)t * k + lane];
            const int row = pos[(size_t)t * k + lane];
            if (row >= 0)
                for (int c = 0; c < chunks; ++c) dg += (double)dgp_r[(size_t)row * chunks + c];
        } else {
            const int s = lane - k;
            ej = E + s;
            for (int c = 0; c < chunks; ++c) dg += (double)dgp_sh[((size_t)t * S + s) * chunks + c];
        }
        for (int s = 0; s < ksplit; ++s) zj += zpart[((size_t)s * T + t) * NE + ej];
    }
    // q_j = sigmoid(z_j) / sum sigmoid (the log-sigmoid softmax in closed form)
    const double sg = lane < nj ? 1.0 / (1.0 + exp(-zj)) : 0.0;
    double ssum = sg;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ssum += __shfl_xor(ssum, off);
    const double q = sg / ssum;
    const double dq = scale * dg;
    double qdq = q * dq;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) qdq += __shfl_xor(qdq, off);
    const double dzj = lane < nj ? q * (dq - qdq) * (1.0 - sg) : 0.0;
    if (lane < nj) dzc[(size_t)t * nj + lane] = (float)dzj;
    // dense row: lane owns columns base + lane (the trip counts are uniform
    // over the wave, so every shuffle has all lanes active); the selected
    // routed experts are distinct
    for (int base = 0; base < NE; base += 64) {
        const int e = base + lane;
        float v = 0.f;
        for (int j = 0; j < nj; ++j) {
            const int ejj = __shfl(ej, j);
            const double dv = __shfl(dzj, j);
            if (ejj == e) v = (float)dv;
        }
        if (e < NE) dz[(size_t)t * NE + e] = v;
    }
}

typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));

// four consecutive elements of a routed dx row (fp16 or fp32) as fp32
template <typename TR>
__device__ __forceinline__ float4 load_row4(const TR* p) {
    if constexpr (sizeof(TR) == 2) {
        const f16x4_t v = *reinterpret_cast<const f16x4_t*>(p);
        return make_float4((float)v[0], (float)v[1], (float)v[2], (float)v[3]);
    } else {
        return *reinterpret_cast<const float4*>(p);
    }
}

// dx[t][h] = dx_sh[t][h] + sum over dispatched slots of dxr[t*k+i][h]
//            + sum over j < k+S of dzc[t][j] * bank[e_j][h]; in fp32 in that
//            order, rounded once.  TR: fp16 routed rows (bf16 layers) or fp32.
template <typename TR, typename TO>
__global__ __launch_bounds__(256) void dx_combine_kernel(const TR* __restrict__ dxr, const float* __restrict__ dxs,
                                                         const int32_t* __restrict__ pos,
                                                         const int32_t* __restrict__ topk_idx,
                                                         const float* __restrict__ dzc,
                                                         const float* __restrict__ bank, TO* __restrict__ dx, int H,
                                                         int E, int S, int k) {
    // one workgroup per token: its slots, experts and gate terms are uniform
    // (scalar loads)
    const int t = blockIdx.x, hq = H >> 2, nj = k + S;
    const int k8 = min(k, 8);
    for (int c4 = threadIdx.x; c4 < hq; c4 += blockDim.x) {
        const int c = c4 * 4;
        float4 s = dxs ? *reinterpret_cast<const float4*>(dxs + (size_t)t * H + c) : make_float4(0.f, 0.f, 0.f, 0.f);
        if (k8 > 0) {
            // the first 8 slot rows are loaded unconditionally (a smaller k
            // re-reads its last row, not added; a slot that was not
            // dispatched holds stale values, not added), so that all are in
            // flight before the first add; then the rest one by one
            const TR* rows = dxr + (size_t)t * k * H + c;
            float4 u[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) u[q] = load_row4(rows + (size_t)min(q, k8 - 1) * H);
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (q < k8 && pos[(size_t)t * k + q] >= 0) {
                    s.x += u[q].x;
                    s.y += u[q].y;
                    s.z += u[q].z;
                    s.w += u[q].w;
                }
            for (int i = 8; i < k; ++i)
                if (pos[(size_t)t * k + i] >= 0) {
                    const float4 v = load_row4(rows + (size_t)i * H);
                    s.x += v.x;
                    s.y += v.y;
                    s.z += v.z;
                    s.w += v.w;
                }
        }
        for (int j = 0; j < nj; ++j) {
            const int e = j < k ? topk_idx[(size_t)t * k + j] : E + (j - k);
            const float g = dzc[(size_t)t * nj + j];
            const float4 b = *reinterpret_cast<const float4*>(bank + (size_t)e * H + c);
            s.x += g * b.x;
            s.y += g * b.y;
            s.z += g * b.z;
            s.w += g * b.w;
        }
        float w[4] = {s.x, s.y, s.z, s.w};
        if constexpr (sizeof(TO) == 2) {
            uint2 q;
            q.x = (uint32_t)f32_to_bf16(w[0]) | ((uint32_t)f32_to_bf16(w[1]) << 16);
            q.y = (uint32_t)f32_to_bf16(w[2]) | ((uint32_t)f32_to_bf16(w[3]) << 16);
            *reinterpret_cast<uint2*>(dx + (size_t)t * H + c) = q;
        } else {
            *reinterpret_cast<float4*>(dx + (size_t)t * H + c) = make_float4(w[0], w[1], w[2], w[3]);
        }
    }
}

constexpr int kBankSplit = 32;   // token ranges summed separately, then in order
constexpr int kBankJW = 3;       // 16-row blocks of the bank per wave

// part[ts][j][h] = sum over t in token range ts of dz[t][j] * x[t][h], on the
// fp32 matrix cores (x widened exactly, products and sums in fp32); grid
// (H/64, ceil(NE/(16*kBankJW)), kBankSplit), one wave of 48 bank rows x 64
// hidden columns.  MFMA operands come straight from global memory: lane l
// holds dz[t + l/16][j0 + l%16] (A, rows = bank rows) and, for the MFMA of
// column block v, x[t + l/16][h0 + 4(l%16) + v] (B, columns = hidden): a lane's
// four B values are one 8- or 16-byte load.  Four tokens per step, in
// ascending order.
template <typename TX>
__global__ __launch_bounds__(64) void dbank_partial_kernel(const float* __restrict__ dz, const TX* __restrict__ x,
                                                           int T, int H, int NE, float* __restrict__ part) {
    const int lane = threadIdx.x, kr = lane >> 4, cl = lane & 15;
    const int h0 = blockIdx.x * 64, jb0 = blockIdx.y * kBankJW;
    const int tlen = (T + kBankSplit - 1) / kBankSplit;
    const int tb = blockIdx.z * tlen, te = min(T, tb + tlen);
    f32x4_t acc[kBankJW][4];
#pragma unroll
    for (int u = 0; u < kBankJW; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int t = tb; t < te; t += 4) {
        const int tt = t + kr;
        const bool tv = tt < te;
        float a[kBankJW], b[4];
#pragma unroll
        for (int u = 0; u < kBankJW; ++u) {
            const int j = (jb0 + u) * 16 + cl;
            a[u] = (tv && j < NE) ? dz[(size_t)tt * NE + j] : 0.f;
        }
        if (tv) {
            const TX* xp = x + (size_t)tt * H + h0 + 4 * cl;
            if constexpr (sizeof(TX) == 2) {
                const uint2 q = *reinterpret_cast<const uint2*>(xp);
                b[0] = __uint_as_float(q.x << 16);
                b[1] = __uint_as_float(q.x & 0xFFFF0000u);
                b[2] = __uint_as_float(q.y << 16);
                b[3] = __uint_as_float(q.y & 0xFFFF0000u);
            } else {
                const float4 q = *reinterpret_cast<const float4*>(xp);
                b[0] = q.x;
                b[1] = q.y;
                b[2] = q.z;
                b[3] = q.w;
            }
        } else {
#pragma unroll
            for (int v = 0; v < 4; ++v) b[v] = 0.f;
        }
#pragma unroll
        for (int u = 0; u < kBankJW; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[u], b[v], acc[u][v], 0, 0, 0);
    }
    // lane l holds rows j0 + 4(l/16) + r, columns h0 + 4(l%16) + v (v = block)
#pragma unroll
    for (int u = 0; u < kBankJW; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int j = (jb0 + u) * 16 + 4 * kr + r;
            if (j < NE)
                *reinterpret_cast<float4*>(part + ((size_t)blockIdx.z * NE + j) * H + h0 + 4 * cl) =
                    make_float4(acc[u][0][r], acc[u][1][r], acc[u][2][r], acc[u][3][r]);
        }
}

__global__ __launch_bounds__(256) void dbank_reduce_kernel(const float* __restrict__ part, int n, float* __restrict__ out) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    float s = 0.f;
#pragma unroll
    for (int ts = 0; ts < kBankSplit; ++ts) s += part[(size_t)ts * n + i];
    out[i] = s;
}

}  // namespace

hipError_t launch_gather_rows(int dtype, const void* src, const int32_t* row_token, const int32_t* offsets, int E,
                              int max_rows, int D, void* out, hipStream_t stream) {
    if (max_rows <= 0 || D <= 0) return hipSuccess;
    const int blocks = std::min(max_rows, 4096);
    if (dtype == 1)
        hipLaunchKernelGGL(gather_rows_kernel<bf16_t>, dim3(blocks), dim3(256), 0, stream, (const bf16_t*)src,
                           row_token, offsets, E, D, (bf16_t*)out);
    else
        hipLaunchKernelGGL(gather_rows_kernel<float>, dim3(blocks), dim3(256), 0, stream, (const float*)src,
                           row_token, offsets, E, D, (float*)out);
    return hipGetLastError();
}

hipError_t launch_padded_offsets(const int32_t* counts, int E, int32_t* poff, hipStream_t stream) {
    hipLaunchKernelGGL(padded_offsets_kernel, dim3(1), dim3(1024), 0, stream, counts, E, poff);
    return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, size_t n, hipStream_t stream) {
    if (n == 0) return hipSuccess;
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 1024);
    hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, stream, p, n);
    return hipGetLastError();
}

hipError_t launch_router_backward(const double* zpart, int ksplit, const int32_t* topk_idx, const int32_t* pos,
                                  const float* dgp_r, const float* dgp_sh, int T, int E, int S, int k, int I,
                                  float route_scale, float global_scale, float* dz, float* dzc, hipStream_t stream) {
    const double scale = (double)route_scale * (double)global_scale;
    hipLaunchKernelGGL(router_backward_kernel, dim3((T + 3) / 4), dim3(256), 0, stream, zpart, ksplit, topk_idx, pos,
                       dgp_r, dgp_sh, T, E, S, k, I, scale, dz, dzc);
    return hipGetLastError();
}

hipError_t launch_dx_combine(int row_dtype, int out_dtype, const void* dxr, const float* dxs, const int32_t* pos,
                             const int32_t* topk_idx, const float* dzc, const float* bank, void* dx, int T, int H,
                             int E, int S, int k, hipStream_t stream) {
    if (T <= 0) return hipSuccess;
    const int blocks = T;
    auto go = [&](auto tr, auto to) {
        using TR = decltype(tr);
        using TO = decltype(to);
        hipLaunchKernelGGL((dx_combine_kernel<TR, TO>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const TR*>(dxr), dxs, pos, topk_idx, dzc, bank, static_cast<TO*>(dx), H, E, S,
                           k);
    };
    if (row_dtype == 1) {
        if (out_dtype == 1) go(f16_t{}, bf16_t{});
        else go(f16_t{}, float{});
    } else {
        if (out_dtype == 1) go(float{}, bf16_t{});
        else go(float{}, float{});
    }
    return hipGetLastError();
}

hipError_t launch_dbank(int dtype, const float* dz, const void* x, int T, int H, int NE, float* part, float* dbank,
                        hipStream_t stream) {
    dim3 grid(H / 64, (NE + 16 * kBankJW - 1) / (16 * kBankJW), kBankSplit);
    if (dtype == 1)
        hipLaunchKernelGGL(dbank_partial_kernel<bf16_t>, grid, dim3(64), 0, stream, dz, (const bf16_t*)x, T, H, NE,
                           part);
    else
        hipLaunchKernelGGL(dbank_partial_kernel<float>, grid, dim3(64), 0, stream, dz, (const float*)x, T, H, NE, part);
    const int n = NE * H;
    hipLaunchKernelGGL(dbank_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, part, n, dbank);
    return hipGetLastError();
}

int dbank_partial_floats(int H, int NE) { return kBankSplit * NE * H; }

}  // namespace inkling
