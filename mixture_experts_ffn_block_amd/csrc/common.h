// common.h -- device types and helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint16_t bf16_t;  // bf16 bit pattern in memory

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

__device__ __forceinline__ float bf16_to_f32(bf16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// fp32 -> bf16, round to nearest even (gfx950 has a native converter; the
// compiler emits it for this cast).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
    __bf16 h = static_cast<__bf16>(f);
    return __builtin_bit_cast(bf16_t, h);
}

// two fp32 -> packed pair of bf16 (low half = a)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

// SiLU(g) = g / (1 + exp(-g)) in fp32, the quotient as g times the hardware
// reciprocal (v_rcp_f32, within 1 ulp): the correctly rounded division expands to
// about ten instructions, and the GEMM1 epilogues evaluate this for every output
__device__ __forceinline__ float silu_f32(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

// fp32 -> OCP e4m3 byte, round to nearest even; the caller clamps to +-448.
// gfx950's v_cvt_pk_fp8_f32 converts to the OCP float8_e4m3fn format.
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    int both = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
    return static_cast<uint32_t>(both);
}

// E8M0 code of the MX block scale: the smallest s = 2^e with a <= fmax * s, code
// e + 127 within [0, 254]; 0 for an all-zero block ("DeepGEMM FusedMoE on
// Blackwell", MXFP8 1x32 and the UE8M0 scale format). fmax * 2^e is exact in
// fp32 (or overflows to inf), so the comparisons decide exactly.
__device__ __forceinline__ uint32_t mx_scale_code(float a, float fmax) {
    if (!(a > 0.0f)) return 0;
    int e = 0;
    frexpf(a / fmax, &e);  // a / fmax lies in about [2^(e-1), 2^e): the answer is near e
    while (e > -127 && a <= ldexpf(fmax, e - 1)) --e;
    while (e < 127 && a > ldexpf(fmax, e)) ++e;
    return static_cast<uint32_t>(e + 127);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

__host__ __device__ __forceinline__ int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
