// Device-side building blocks shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pml.h"

namespace pml {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v2f __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
#ifndef PML_GMAX
#define PML_GMAX 8
#endif
constexpr int kGMax = PML_GMAX;  // rows of one piece scored against a shared key block
constexpr int kCostBase = 3;    // schedule weight of a block: kCostBase + rows (3 measured best of 1, 2, 3, 4, 8)

// Tokens per unit of work (one step of a wave): a block_kv 32 cache is scored
// two pages at a time, so every step covers 64 tokens.
constexpr int kMinStep = 64;
__host__ __device__ inline int step_tokens(int block_kv) { return block_kv < kMinStep ? kMinStep : block_kv; }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-uniform copy of x (lane 0's value, in a scalar register).
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Workgroup barrier that only orders LDS: waits for this wave's LDS traffic,
// then s_barrier. Unlike __syncthreads it does not drain outstanding global
// loads, so key blocks requested ahead stay in flight across it.
__device__ __forceinline__ void barrier_lds() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Plain (compiler-tracked) loads from LDS through a generic pointer that
// points into a __shared__ array.
template <typename T>
__device__ __forceinline__ T lds_ld(const void *p) {
    return *(const __attribute__((address_space(3))) T *)(const __attribute__((address_space(3))) void *)p;
}

template <typename T>
__device__ __forceinline__ void lds_st(void *p, T v) {
    *(__attribute__((address_space(3))) T *)(__attribute__((address_space(3))) void *)p = v;
}

// D = A(16x128 fp8) * B(128x16 fp8), fresh accumulator (unscaled opcode).
__device__ __forceinline__ v4f mfma_fp8(const v8i &a, const v8i &b) {
    v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// D = A(16x128 fp8, e8m0 scale per row and 32-block of k) * B(128x16 fp8 when
// FMT_B == 0, e2m1 when FMT_B == 4, e8m0 scale per column and 32-block).
template <int FMT_B>
__device__ __forceinline__ v4f mfma_scaled(const v8i &a, const v8i &b, int a_scale, int b_scale) {
    v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, FMT_B, 0, a_scale, 0, b_scale);
}

// D = A(16x128) * B(128x16) with both operand formats given (0 fp8, 4 e2m1)
// and an e8m0 scale per row / column and 32-block of k for each.
template <int FMT_A, int FMT_B>
__device__ __forceinline__ v4f mfma_scaled_ab(const v8i &a, const v8i &b, int a_scale, int b_scale) {
    v4f z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, FMT_A, FMT_B, 0, a_scale, 0, b_scale);
}

// Exchange halves between two registers (gfx950 v_permlane32_swap / 16_swap).
// swap32(x, y): x <- (x.lanes[0,32), y.lanes[0,32)), y <- (x.lanes[32,64), y.lanes[32,64)).
__device__ __forceinline__ void swap32(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(y), false, false);
    x = __int_as_float(r[0]);
    y = __int_as_float(r[1]);
}
// swap16(x, y): rows of 16 lanes; x <- (x.R0, y.R0, x.R2, y.R2), y <- (x.R1, y.R1, x.R3, y.R3).
__device__ __forceinline__ void swap16(float &x, float &y) {
    auto r = __builtin_amdgcn_permlane16_swap(__float_as_int(x), __float_as_int(y), false, false);
    x = __int_as_float(r[0]);
    y = __int_as_float(r[1]);
}

}  // namespace pml
