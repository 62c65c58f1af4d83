// Shared device/host helpers of the gfx950 Inkling MoE library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace inkling {

typedef uint16_t bf16_t;  // storage type of bfloat16 values

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16_t;  // IEEE half: the activation between the two expert projections of a bf16 layer
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef double f64x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// Round-to-nearest-even float -> bfloat16 (inputs are finite).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (bf16_t)(u >> 16);
}

template <typename TE>
__device__ __forceinline__ float to_f32(TE v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename TE>
__device__ __forceinline__ TE from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

constexpr int kWave = 64;

// Tile descriptor of the routed grouped GEMMs: expert id and first row of the
// tile within that expert's block of expert-sorted rows.
// Per-XCD counters of the grouped GEMM launches (8 each: gate_up or the
// backward's recompute of it, down or dx, dact, and the two weight-gradient
// launches): tiles finished (tile-round rendezvous) or tiles taken (tile
// queue).  Written to zero by the permutation (the dense MLP: its prep
// kernel) before each use.
constexpr int kRoundCounters = 40;

struct RoutedTile {
    int32_t expert;
    int32_t row_start;
};

}  // namespace inkling
