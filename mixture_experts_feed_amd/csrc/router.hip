// InklingGate on gfx950: gate logits in fp64 on the matrix cores, then top-k
// selection on sigmoid + correction bias and the log-sigmoid softmax gammas.
//
// Follows the Inkling layers page (nemo_automodel.components.models.inkling.layers),
// InklingGate and InklingCorrectionBias: the gate bank holds the routed rows
// followed by the shared rows; selection uses sigmoid(logit) + bias; the
// returned weights are route_scale * global_scale times
// softmax(log sigmoid([selected routed || shared] logits)).
//
// Precision: the page fixes fp32 gate operands.  Logits are accumulated here in
// fp64 from the exactly widened fp32 bank and bf16/fp32 hidden states, and
// sigmoid, selection and softmax run in fp64, so the selected experts are those
// of exact arithmetic unless two scores differ by less than ~1e-13.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace inkling {

namespace {

constexpr int kExpTile = 48;   // logits columns per workgroup (3 blocks of 16)
constexpr int kKChunk = 64;    // hidden-dim chunk staged in LDS (two buffers)
// Token tiles: 128 tokens, 12 waves (three per SIMD, so that every SIMD carries
// the same MFMA work), each wave two 16-token blocks sharing one widened bank
// fragment; below kBigTileTokens tokens, 32 tokens and 6 waves of one block,
// which waste fewer MFMAs on empty rows.
constexpr int kBigTileTokens = 2048;
int router_tok_tile(int T) { return T >= kBigTileTokens ? 128 : 32; }
template <int TOK, int WTOK>
constexpr int router_threads() { return 64 * (TOK / 16 / WTOK) * (kExpTile / 16); }

// kRowVals consecutive values of a row, kept as raw 16-byte words
constexpr int kRowVals = 16;
template <typename TX>
struct RowVals {
    static constexpr int kWords = kRowVals * sizeof(TX) / 16;
    uint4 q[kWords];
    __device__ __forceinline__ void load(const TX* p) {
#pragma unroll
        for (int i = 0; i < kWords; ++i) q[i] = reinterpret_cast<const uint4*>(p)[i];
    }
    __device__ __forceinline__ void zero() {
#pragma unroll
        for (int i = 0; i < kWords; ++i) q[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    __device__ __forceinline__ TX get(int j) const {
        constexpr int per = 16 / sizeof(TX);   // values per 16-byte word
        const uint4& w = q[j / per];
        const int e = j % per;
        if constexpr (sizeof(TX) == 2) {
            const uint32_t d = (e >> 1) == 0 ? w.x : (e >> 1) == 1 ? w.y : (e >> 1) == 2 ? w.z : w.w;
            return (TX)((e & 1) ? (d >> 16) : (d & 0xFFFFu));
        } else {
            const uint32_t d = e == 0 ? w.x : e == 1 ? w.y : e == 2 ? w.z : w.w;
            return __uint_as_float(d);
        }
    }
};

// exact widening to fp64
__device__ __forceinline__ double widen(bf16_t v) { return (double)__uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ double widen(float v) { return (double)v; }

// zpart[ks][t][e] = sum over h in slice ks of x[t][h] * bank[e][h], in fp64.
// grid (ceil(T/TOK), ceil(NE/48), ksplit); wave w owns the WTOK 16x16 blocks of
// tokens 16*WTOK*(w % nw).. against bank rows 16*(w / nw).. of the tile (nw =
// TOK/16/WTOK).  Operands are staged in LDS in their own precision and widened
// to fp64 (exactly) as the MFMA fragments are read; the next chunk's global
// loads are in flight while the current one is multiplied.
template <typename TX, int TOK, int WTOK>
__global__ __launch_bounds__((router_threads<TOK, WTOK>())) void router_logits_kernel(const TX* __restrict__ x,
                                                                       const float* __restrict__ bank,
                                                                       double* __restrict__ zpart, int T, int H,
                                                                       int NE, int klen) {
    // [buffer][16-row block][k][row in block]: an MFMA operand fragment (lane l
    // holds row l%16 at k = l/16) is one contiguous run of 64 elements
    constexpr int kTokTile = TOK, kWaveTok = WTOK, kTokWaves = TOK / 16 / WTOK;
    constexpr int kRouterThreads = router_threads<TOK, WTOK>();
    __shared__ TX xs[2][kTokTile / 16][kKChunk][16];
    __shared__ float gs[2][kExpTile / 16][kKChunk][16];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int t0 = blockIdx.x * kTokTile, e0 = blockIdx.y * kExpTile, ks = blockIdx.z;
    const int kbeg = ks * klen;
    const int nchunks = min(klen, H - kbeg) / kKChunk;
    const int tb = (wv % kTokWaves) * kWaveTok, eb = wv / kTokWaves;   // first token block, bank-row block
    // kChains accumulators per token block (k-steps taken round-robin) so
    // consecutive MFMAs of a wave are independent
    constexpr int kChains = 4;
    f64x4_t acc[kWaveTok][kChains];
#pragma unroll
    for (int u = 0; u < kWaveTok; ++u)
#pragma unroll
        for (int i = 0; i < kChains; ++i) acc[u][i] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    // staging: threads [0, 128) load kRowVals hidden values of one token row,
    // threads [128, 320) kRowVals bank values of one bank row
    constexpr int kPerRow = kKChunk / kRowVals;   // threads per row
    constexpr int kXThreads = kTokTile * kPerRow, kGThreads = kExpTile * kPerRow;
    static_assert(kXThreads + kGThreads <= kRouterThreads, "staging threads");
    const bool ld_x = tid < kXThreads, ld_g = tid >= kXThreads && tid < kXThreads + kGThreads;
    const int li = ld_x ? tid : tid - kXThreads;
    const int lr = li / kPerRow, lc = (li % kPerRow) * kRowVals;
    const int t = t0 + lr, e = e0 + lr;
    // two register sets: chunk c+2 is loaded while chunk c is multiplied
    RowVals<TX> vx0, vx1;
    RowVals<float> vg0, vg1;
    auto gload = [&](RowVals<TX>& vx, RowVals<float>& vg, int c) __attribute__((always_inline)) {
        if (c >= nchunks) return;
        const int k0 = kbeg + c * kKChunk;
        if (ld_x) {
            if (t < T) vx.load(x + (size_t)t * H + k0 + lc);
            else vx.zero();
        } else if (ld_g) {
            if (e < NE) vg.load(bank + (size_t)e * H + k0 + lc);
            else vg.zero();
        }
    };
    auto step = [&](RowVals<TX>& vx, RowVals<float>& vg, int c, auto B_) __attribute__((always_inline)) {
        constexpr int buf = decltype(B_)::value;
        if (ld_x) {
#pragma unroll
            for (int j = 0; j < kRowVals; ++j) xs[buf][lr >> 4][lc + j][lr & 15] = vx.get(j);
        } else if (ld_g) {
#pragma unroll
            for (int j = 0; j < kRowVals; ++j) gs[buf][lr >> 4][lc + j][lr & 15] = vg.get(j);
        }
        // one barrier per chunk: buffer buf was last read two chunks ago, and
        // every wave has passed the previous chunk's barrier since
        __syncthreads();
        gload(vx, vg, c + 2);
#pragma unroll
        for (int kk = 0; kk < kKChunk; kk += 4 * kChains) {
            // A (16 tokens x 4): lane holds A[lane%16][lane/16]; B (4 x 16 bank rows): B[lane/16][lane%16]
            double a[kWaveTok][kChains], b[kChains];
#pragma unroll
            for (int i = 0; i < kChains; ++i) {
                b[i] = widen(gs[buf][eb][kk + 4 * i + (lane >> 4)][lane & 15]);
#pragma unroll
                for (int u = 0; u < kWaveTok; ++u) a[u][i] = widen(xs[buf][tb + u][kk + 4 * i + (lane >> 4)][lane & 15]);
            }
#pragma unroll
            for (int i = 0; i < kChains; ++i)
#pragma unroll
                for (int u = 0; u < kWaveTok; ++u)
                    acc[u][i] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[u][i], b[i], acc[u][i], 0, 0, 0);
        }
    };
    gload(vx0, vg0, 0);
    gload(vx1, vg1, 1);
    for (int c = 0; c < nchunks; c += 2) {
        step(vx0, vg0, c, std::integral_constant<int, 0>{});
        if (c + 1 < nchunks) step(vx1, vg1, c + 1, std::integral_constant<int, 1>{});
    }
    // fp64 16x16x4 result layout: lane holds D[i][j] for rows i = lane/16 + 4*r
    // (r = 0..3) and column j = lane % 16 (unlike the fp32 16x16 layouts, whose
    // rows are 4*(lane/16) + r).
    const int eo = e0 + eb * 16 + (lane & 15);
#pragma unroll
    for (int u = 0; u < kWaveTok; ++u)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int to = t0 + (tb + u) * 16 + (lane >> 4) + 4 * r;
            if (to < T && eo < NE)
                zpart[((size_t)ks * T + to) * NE + eo] = (acc[u][0][r] + acc[u][1][r]) + (acc[u][2][r] + acc[u][3][r]);
        }
}

constexpr int kMaxPerLane = 8;  // experts per lane: n_routed + n_shared <= 512
constexpr int kFewPerLane = 3;  // n_routed + n_shared <= 192

__device__ __forceinline__ double log_sigmoid(double z) {
    // log sigma(z) = -log(1 + e^-z), evaluated on the side that cannot overflow
    return z >= 0.0 ? -log1p(exp(-z)) : z - log1p(exp(z));
}

// One wave per token.  Lane j holds logits of experts j, j+64, ... (PL of them);
// the partial logits of BATCH hidden-dim slices are loaded together.
template <int PL, int BATCH>
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
    double sc[PL];
    bool live[PL];
    // logits: sum of the hidden-dim slices in slice order
    constexpr int kBatch = BATCH;
    double z[PL];
#pragma unroll
    for (int j = 0; j < PL; ++j) z[j] = 0.0;
    for (int s0 = 0; s0 < ksplit; s0 += kBatch) {
        double p[kBatch][PL];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int j = 0; j < PL; ++j) {
                const int e = lane + 64 * j;
                p[u][j] = (s0 + u < ksplit && e < NE) ? zpart[((size_t)(s0 + u) * T + t) * NE + e] : 0.0;
            }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int j = 0; j < PL; ++j)
                if (s0 + u < ksplit) z[j] += p[u][j];
    }
#pragma unroll
    for (int j = 0; j < PL; ++j) {
        const int e = lane + 64 * j;
        live[j] = false;
        sc[j] = 0.0;
        if (e < NE) {
            zs[wv][e] = z[j];
            if (e < E) {
                sc[j] = 1.0 / (1.0 + exp(-z[j])) + (double)bias[e];
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
        for (int j = 0; j < PL; ++j) {
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
            for (int j = 0; j < PL; ++j)
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

// z[i] = the partial logits of element i summed over the slices in slice
// order, from 0.0 (the order router_select_kernel and the router backward
// sum them in, so either reads the same values from z with one slice)
__global__ __launch_bounds__(256) void zsum_kernel(const double* __restrict__ zpart, int ksplit, size_t n,
                                                   double* __restrict__ z) {
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    double s = 0.0;
    for (int p = 0; p < ksplit; ++p) s += zpart[(size_t)p * n + i];
    z[i] = s;
}

}  // namespace

hipError_t launch_logits_sum(const double* zpart, int ksplit, int T, int NE, double* z, hipStream_t stream) {
    const size_t n = (size_t)T * NE;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(zsum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, zpart, ksplit, n, z);
    return hipGetLastError();
}

int router_ksplit(int T, int H, int NE) {
    const int tok = router_tok_tile(T);
    const int tiles = ((T + tok - 1) / tok) * ((NE + kExpTile - 1) / kExpTile);
    int ks = 1;
    // split the hidden dim until ~3 workgroups per CU exist (768), keeping >= 256 per slice
    while (tiles * ks * 2 <= 768 && (H / (ks * 2)) >= 256 && (H % (ks * 2 * kKChunk)) == 0) ks *= 2;
    return ks;
}

hipError_t launch_router_logits(int dtype, const void* x, const float* bank, double* zpart, int T, int H, int NE,
                                int ksplit, hipStream_t stream) {
    const int tok = router_tok_tile(T);
    dim3 grid((T + tok - 1) / tok, (NE + kExpTile - 1) / kExpTile, ksplit);
    const int klen = H / ksplit;
    if (tok == 128) {
        constexpr int threads = router_threads<128, 2>();
        if (dtype == 1)
            hipLaunchKernelGGL((router_logits_kernel<bf16_t, 128, 2>), grid, dim3(threads), 0, stream,
                               (const bf16_t*)x, bank, zpart, T, H, NE, klen);
        else
            hipLaunchKernelGGL((router_logits_kernel<float, 128, 2>), grid, dim3(threads), 0, stream,
                               (const float*)x, bank, zpart, T, H, NE, klen);
    } else {
        constexpr int threads = router_threads<32, 1>();
        if (dtype == 1)
            hipLaunchKernelGGL((router_logits_kernel<bf16_t, 32, 1>), grid, dim3(threads), 0, stream,
                               (const bf16_t*)x, bank, zpart, T, H, NE, klen);
        else
            hipLaunchKernelGGL((router_logits_kernel<float, 32, 1>), grid, dim3(threads), 0, stream,
                               (const float*)x, bank, zpart, T, H, NE, klen);
    }
    return hipGetLastError();
}

hipError_t launch_router_select(const double* zpart, int ksplit, const float* bias, int T, int E, int S, int k,
                                float route_scale, float global_scale, int32_t* topk_idx, float* topk_w,
                                float* shared_g, hipStream_t stream) {
    const double scale = (double)route_scale * (double)global_scale;
    // few experts per lane and many slices (the few-token splits): every
    // slice's loads at once; otherwise four slices at a time
    const dim3 grid((T + 3) / 4);
    if (E + S <= 64 * kFewPerLane && ksplit > 8)
        hipLaunchKernelGGL((router_select_kernel<kFewPerLane, 16>), grid, dim3(256), 0, stream, zpart, ksplit, bias, T,
                           E, S, k, scale, topk_idx, topk_w, shared_g);
    else if (E + S <= 64 * kFewPerLane && ksplit > 4)
        hipLaunchKernelGGL((router_select_kernel<kFewPerLane, 8>), grid, dim3(256), 0, stream, zpart, ksplit, bias, T,
                           E, S, k, scale, topk_idx, topk_w, shared_g);
    else if (E + S <= 64 * kFewPerLane)
        hipLaunchKernelGGL((router_select_kernel<kFewPerLane, 4>), grid, dim3(256), 0, stream, zpart, ksplit, bias, T,
                           E, S, k, scale, topk_idx, topk_w, shared_g);
    else
        hipLaunchKernelGGL((router_select_kernel<kMaxPerLane, 4>), grid, dim3(256), 0, stream, zpart, ksplit, bias, T,
                           E, S, k, scale, topk_idx, topk_w, shared_g);
    return hipGetLastError();
}

}  // namespace inkling
