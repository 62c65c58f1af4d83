// Grouped expert GEMMs of the Inkling MoE on gfx950 matrix cores.
//
// Every expert product here is out[row][n] = sum_k W[n][k] * X[row][k] with
// both operands K-contiguous (nn.Linear weights [out, in] and row-major token
// rows).  The weights are the MFMA A operand (MFMA rows = output columns n) and
// the token rows the B operand (MFMA columns = tokens), so each lane's 16x16
// accumulator holds four consecutive output columns of one token.  For the
// gate_up projection those four columns are [g_j, u_j, g_j+1, u_j+1] of the
// interleaved layout (inkling_swiglu on the Inkling layers page: ::2 gate,
// 1::2 up), so SwiGLU and the routing-weight scale are applied in registers.
//
// Three launches per forward:
//   gate_up       routed tiles (rows gathered through the expert-sorted token
//                 list, scaled by that slot's gamma) and shared tiles (all
//                 tokens against the S shared experts concatenated along N,
//                 scaled by the token's shared gamma) -> act_r, act_sh;
//   down routed   act_r rows of each expert -> y (one fp32 row per routed slot);
//   down shared   act_sh [T][S*I] against the shared down weights
//                 concatenated along K (the sum over shared experts happens in
//                 the reduction), with the routed rows y[pos(t, i)] added in the
//                 epilogue -> out.  With S = 0 the reduction is empty and the
//                 kernel is the combine alone.
#include "common.h"
#include "kernels.h"

namespace inkling {

namespace {

enum { kModeGateUp = 0, kModeDown = 1, kModeDownCombine = 2 };

constexpr int kRowBytes = 128;   // bytes of K per row staged per pipeline step
constexpr int kChunks = kRowBytes / 16;

struct GemmKArgs {
    const void* A_routed;   // [E][N_r][K_r]
    const void* A_shared;   // see seg_s
    const void* B_routed;   // x [T][H] (gate_up, gathered) or act_r [T*k][I]
    const void* B_shared;   // x [T][H] or act_sh [T][S*I]
    const RoutedTile* tiles;
    const int32_t* num_tiles;
    const int32_t* offsets;
    const int32_t* row_token;
    const float* row_gamma;
    const float* shared_g;
    const int32_t* pos;
    const void* y;
    void* out_routed;
    void* out_shared;
    int T, H, I, S, k;
    int K_r, N_r;
    int K_s, N_s;
    int seg_s;              // shared A(n, kk) = A_shared + (kk/seg)*N_s*seg + n*seg + kk%seg
    int shared_blocks, shared_mtiles;
    int max_routed_tiles;
};

template <typename TE>
__device__ __forceinline__ void mma16(f32x4_t& acc, const uint4& a, const uint4& b);

template <>
__device__ __forceinline__ void mma16<bf16_t>(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                  acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mma16<float>(f32x4_t& acc, const uint4& a, const uint4& b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}

__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

template <typename TE>
__device__ __forceinline__ void store2(TE* p, float a, float b);
template <>
__device__ __forceinline__ void store2<bf16_t>(bf16_t* p, float a, float b) {
    *reinterpret_cast<uint32_t*>(p) = (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}
template <>
__device__ __forceinline__ void store2<float>(float* p, float a, float b) {
    *reinterpret_cast<float2*>(p) = make_float2(a, b);
}

template <typename TE>
__device__ __forceinline__ void store4(TE* p, const float* v);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
    uint2 q;
    q.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
    q.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = q;
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

template <typename TE>
__device__ __forceinline__ void load4f(const TE* p, float* v);
template <>
__device__ __forceinline__ void load4f<bf16_t>(const bf16_t* p, float* v) {
    uint2 q = *reinterpret_cast<const uint2*>(p);
    v[0] = __uint_as_float(q.x << 16);
    v[1] = __uint_as_float(q.x & 0xFFFF0000u);
    v[2] = __uint_as_float(q.y << 16);
    v[3] = __uint_as_float(q.y & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ void load4f<float>(const float* p, float* v) {
    float4 q = *reinterpret_cast<const float4*>(p);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
}

// BN weight rows x BM token rows per workgroup; WN x WM waves (= 4).
// TE: operand / intermediate type; TO: type of the layer output (combine mode).
template <typename TE, typename TO, int BN, int BM, int WN, int WM, int MODE>
__global__ __launch_bounds__(256) void moe_gemm_kernel(const GemmKArgs a) {
    static_assert(WN * WM == 4, "four waves");
    constexpr int EPC = 16 / sizeof(TE);          // elements per 16-byte chunk
    constexpr int BK = kRowBytes / sizeof(TE);    // K elements per step
    constexpr int WTN = BN / WN, WTM = BM / WM;   // wave tile
    constexpr int FN = WTN / 16, FM = WTM / 16;
    static_assert(FN >= 1 && FM >= 1, "wave tile at least 16x16");
    constexpr int NA = (BN * kChunks + 255) / 256;
    constexpr int NB = (BM * kChunks + 255) / 256;

    __shared__ __attribute__((aligned(16))) uint8_t lds[2][(BN + BM) * kRowBytes];

    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int wn0 = (wv % WN) * WTN, wm0 = (wv / WN) * WTM;

    // ---- which tile -------------------------------------------------------
    int b = blockIdx.x;
    const bool is_shared = b < a.shared_blocks;
    int K, N, seg, n0, rows_valid, grow0 = 0, t0 = 0, expert = 0;
    const TE* A;
    const TE* Bsrc;
    if (is_shared) {
        const int mt = b % a.shared_mtiles, nt = b / a.shared_mtiles;
        t0 = mt * BM;
        rows_valid = min(BM, a.T - t0);
        n0 = nt * BN;
        K = a.K_s;
        N = a.N_s;
        seg = a.seg_s;
        A = reinterpret_cast<const TE*>(a.A_shared);
        Bsrc = reinterpret_cast<const TE*>(a.B_shared);
    } else {
        b -= a.shared_blocks;
        const int ti = b % a.max_routed_tiles, nt = b / a.max_routed_tiles;
        if (ti >= *a.num_tiles) return;
        const RoutedTile tl = a.tiles[ti];
        expert = tl.expert;
        const int base = a.offsets[expert];
        rows_valid = min(BM, a.offsets[expert + 1] - base - tl.row_start);
        grow0 = base + tl.row_start;
        n0 = nt * BN;
        K = a.K_r;
        N = a.N_r;
        seg = a.K_r;
        A = reinterpret_cast<const TE*>(a.A_routed) + (size_t)expert * a.N_r * a.K_r;
        Bsrc = reinterpret_cast<const TE*>(a.B_routed);
    }

    // ---- per-thread load assignments (16-byte chunks) ----------------------
    // chunk L = i*256 + tid -> row L / kChunks, chunk L % kChunks
    const TE* brow[NB];
    bool bval[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) {
        const int L = i * 256 + tid;
        const int r = L / kChunks;
        bval[i] = (L < BM * kChunks) && (r < rows_valid);
        brow[i] = Bsrc;
        if (bval[i]) {
            size_t row;
            if (is_shared) row = (size_t)(t0 + r);
            else if (MODE == kModeGateUp) row = (size_t)a.row_token[grow0 + r];
            else row = (size_t)(grow0 + r);
            brow[i] = Bsrc + row * K + (L % kChunks) * EPC;
        }
    }

    f32x4_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    uint4 ra[NA], rb[NB];
    auto gload = [&](int k0) {
        const int s = k0 / seg;
        const TE* Ab = A + (size_t)s * N * seg + (k0 - s * seg);
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int L = i * 256 + tid;
            if (L < BN * kChunks) {
                const int r = L / kChunks, c = L % kChunks;
                ra[i] = *reinterpret_cast<const uint4*>(Ab + (size_t)(n0 + r) * seg + c * EPC);
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            if (bval[i]) rb[i] = *reinterpret_cast<const uint4*>(brow[i] + k0);
            else rb[i] = make_uint4(0, 0, 0, 0);
        }
    };
    auto sstore = [&](int st) {
        uint8_t* la = lds[st];
        uint8_t* lb = lds[st] + BN * kRowBytes;
#pragma unroll
        for (int i = 0; i < NA; ++i) {
            const int L = i * 256 + tid;
            if (L < BN * kChunks) {
                const int r = L / kChunks, c = L % kChunks;
                *reinterpret_cast<uint4*>(la + r * kRowBytes + ((c ^ (r & 7)) << 4)) = ra[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NB; ++i) {
            const int L = i * 256 + tid;
            if (L < BM * kChunks) {
                const int r = L / kChunks, c = L % kChunks;
                *reinterpret_cast<uint4*>(lb + r * kRowBytes + ((c ^ (r & 7)) << 4)) = rb[i];
            }
        }
    };

    const int nk = K / BK;
    if (nk > 0) {
        gload(0);
        sstore(0);
        __syncthreads();
    }
    for (int kt = 0; kt < nk; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const uint8_t* la = lds[st];
        const uint8_t* lb = lds[st] + BN * kRowBytes;
#pragma unroll
        for (int s = 0; s < kChunks / 4; ++s) {
            const int c = 4 * s + (lane >> 4);
            uint4 af[FN], bfr[FM];
#pragma unroll
            for (int i = 0; i < FN; ++i) {
                const int r = wn0 + 16 * i + (lane & 15);
                af[i] = *reinterpret_cast<const uint4*>(la + r * kRowBytes + ((c ^ (r & 7)) << 4));
            }
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int r = wm0 + 16 * j + (lane & 15);
                bfr[j] = *reinterpret_cast<const uint4*>(lb + r * kRowBytes + ((c ^ (r & 7)) << 4));
            }
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) mma16<TE>(acc[i][j], af[i], bfr[j]);
        }
        if (kt + 1 < nk) sstore(st ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    // acc[i][j][r]: output column n = n0 + wn0 + 16i + 4*(lane/16) + r, row m = wm0 + 16j + lane%16
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int m = wm0 + 16 * j + (lane & 15);
        if (m >= rows_valid) continue;
#pragma unroll
        for (int i = 0; i < FN; ++i) {
            const int n = n0 + wn0 + 16 * i + 4 * (lane >> 4);
            const f32x4_t v = acc[i][j];
            if (MODE == kModeGateUp) {
                if (is_shared) {
                    const int t = t0 + m;
                    const int s = n / (2 * a.I);
                    const float g = a.shared_g[(size_t)t * a.S + s];
                    TE* o = reinterpret_cast<TE*>(a.out_shared) + (size_t)t * a.S * a.I + (n >> 1);
                    store2<TE>(o, silu(v[0]) * v[1] * g, silu(v[2]) * v[3] * g);
                } else {
                    const int row = grow0 + m;
                    const float g = a.row_gamma[row];
                    TE* o = reinterpret_cast<TE*>(a.out_routed) + (size_t)row * a.I + (n >> 1);
                    store2<TE>(o, silu(v[0]) * v[1] * g, silu(v[2]) * v[3] * g);
                }
            } else if (MODE == kModeDown) {
                // per-slot rows stay fp32 so the output is rounded once, in the combine
                const int row = grow0 + m;
                float w[4] = {v[0], v[1], v[2], v[3]};
                store4<float>(reinterpret_cast<float*>(a.out_routed) + (size_t)row * a.H + n, w);
            } else {
                const int t = t0 + m;
                float w[4] = {v[0], v[1], v[2], v[3]};
                for (int q = 0; q < a.k; ++q) {
                    const int p = a.pos[(size_t)t * a.k + q];
                    if (p < 0) continue;
                    float yv[4];
                    load4f<float>(reinterpret_cast<const float*>(a.y) + (size_t)p * a.H + n, yv);
                    w[0] += yv[0]; w[1] += yv[1]; w[2] += yv[2]; w[3] += yv[3];
                }
                store4<TO>(reinterpret_cast<TO*>(a.out_shared) + (size_t)t * a.H + n, w);
            }
        }
    }
}

// ---- tile configurations ---------------------------------------------------
// cfg 0: 128 weight rows x 128 tokens, waves 2x2 (many rows per expert)
// cfg 1: 128 weight rows x 16 tokens,  waves 4x1 (few rows per expert: decode)
constexpr int kBN = 128;

template <typename TE, typename TO, int MODE>
hipError_t launch_mode(int cfg, const GemmKArgs& a, int blocks, hipStream_t stream) {
    if (blocks <= 0) return hipSuccess;
    if (cfg == 0)
        hipLaunchKernelGGL((moe_gemm_kernel<TE, TO, 128, 128, 2, 2, MODE>), dim3(blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL((moe_gemm_kernel<TE, TO, 128, 16, 4, 1, MODE>), dim3(blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}

template <int MODE>
hipError_t launch_dispatch(const MoeGemmParams& p, const GemmKArgs& a, int blocks, hipStream_t stream) {
    if (MODE == kModeDownCombine && p.out_dtype != p.dtype) {
        if (p.dtype == 1) return launch_mode<bf16_t, float, MODE>(p.cfg, a, blocks, stream);
        return launch_mode<float, bf16_t, MODE>(p.cfg, a, blocks, stream);
    }
    if (p.dtype == 1) return launch_mode<bf16_t, bf16_t, MODE>(p.cfg, a, blocks, stream);
    return launch_mode<float, float, MODE>(p.cfg, a, blocks, stream);
}

GemmKArgs base_args(const MoeGemmParams& p) {
    GemmKArgs a = {};
    a.tiles = p.tiles;
    a.num_tiles = p.num_tiles;
    a.offsets = p.offsets;
    a.row_token = p.row_token;
    a.row_gamma = p.row_gamma;
    a.shared_g = p.shared_g;
    a.pos = p.pos;
    a.y = p.y;
    a.T = p.T;
    a.H = p.H;
    a.I = p.I;
    a.S = p.S;
    a.k = p.k;
    a.max_routed_tiles = p.max_routed_tiles;
    return a;
}

}  // namespace

int gemm_cfg_for(int dtype, int T, int H, int E, int k, int I) {
    (void)dtype; (void)H; (void)I;
    const double rows_per_expert = (double)T * k / E;
    return rows_per_expert <= 48.0 ? 1 : 0;
}

int gemm_cfg_bm(int cfg) { return cfg == 0 ? 128 : 16; }

hipError_t launch_gate_up(const MoeGemmParams& p, hipStream_t stream) {
    GemmKArgs a = base_args(p);
    const int bm = gemm_cfg_bm(p.cfg);
    a.A_routed = p.w_gu;
    a.B_routed = p.x;
    a.out_routed = p.act_r;
    a.K_r = p.H;
    a.N_r = 2 * p.I;
    a.A_shared = p.wsh_gu;
    a.B_shared = p.x;
    a.out_shared = p.act_sh;
    a.K_s = p.H;
    a.N_s = 2 * p.I * p.S;
    a.seg_s = p.H;
    a.shared_mtiles = (p.T + bm - 1) / bm;
    a.shared_blocks = p.S > 0 ? a.shared_mtiles * (a.N_s / kBN) : 0;
    const int blocks = a.shared_blocks + p.max_routed_tiles * (a.N_r / kBN);
    return launch_dispatch<kModeGateUp>(p, a, blocks, stream);
}

hipError_t launch_down_routed(const MoeGemmParams& p, hipStream_t stream) {
    GemmKArgs a = base_args(p);
    a.A_routed = p.w_d;
    a.B_routed = p.act_r;
    a.out_routed = p.y;
    a.K_r = p.I;
    a.N_r = p.H;
    a.shared_blocks = 0;
    a.shared_mtiles = 1;
    const int blocks = p.max_routed_tiles * (p.H / kBN);
    return launch_dispatch<kModeDown>(p, a, blocks, stream);
}

hipError_t launch_down_shared_combine(const MoeGemmParams& p, hipStream_t stream) {
    GemmKArgs a = base_args(p);
    const int bm = gemm_cfg_bm(p.cfg);
    a.A_shared = p.wsh_d;
    a.B_shared = p.act_sh;
    a.out_shared = p.out;
    a.K_s = p.S * p.I;
    a.N_s = p.H;
    a.seg_s = p.I;
    a.shared_mtiles = (p.T + bm - 1) / bm;
    a.shared_blocks = a.shared_mtiles * (p.H / kBN);
    a.max_routed_tiles = 1;
    return launch_dispatch<kModeDownCombine>(p, a, a.shared_blocks, stream);
}

}  // namespace inkling
