// Helpers of the fp32-MFMA kernels that walk a sequence 8 tokens at a time
// (short runs, and the chunked prefill for every head size): range-checked
// buffer access to token rows, the 16x16x4 fp32 MFMA, and 8 x 8 products on
// one wave.
#pragma once

#include "dev_common.h"

namespace kda {
namespace f32m {

typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u2 __attribute__((ext_vector_type(2)));

// Buffer resource over `bytes` bytes from a uniform base: accesses at or past
// the end read zeros or are dropped, which masks the tokens past a sequence.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
// element i (the pointer argument only selects the element type)
__device__ __forceinline__ float bld(__amdgpu_buffer_rsrc_t r, uint32_t i, const float*) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(4 * i), 0, 0));
}
__device__ __forceinline__ float bld(__amdgpu_buffer_rsrc_t r, uint32_t i, const bf16_t*) {
    return __uint_as_float(static_cast<uint32_t>(__builtin_amdgcn_raw_buffer_load_b16(r, static_cast<int>(2 * i), 0, 0)) << 16);
}
// two consecutive elements from element i (i even)
__device__ __forceinline__ f2 bld2(__amdgpu_buffer_rsrc_t r, uint32_t i, const float*) {
    const u2 x = __builtin_amdgcn_raw_buffer_load_b64(r, static_cast<int>(4 * i), 0, 0);
    return f2{__uint_as_float(x[0]), __uint_as_float(x[1])};
}
__device__ __forceinline__ f2 bld2(__amdgpu_buffer_rsrc_t r, uint32_t i, const bf16_t*) {
    const uint32_t x = __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(2 * i), 0, 0);
    return f2{__uint_as_float(x << 16), __uint_as_float(x & 0xffff0000u)};
}
__device__ __forceinline__ void bst(__amdgpu_buffer_rsrc_t r, uint32_t i, float y, float*) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(y), r, static_cast<int>(4 * i), 0, 0);
}
__device__ __forceinline__ void bst(__amdgpu_buffer_rsrc_t r, uint32_t i, float y, bf16_t*) {
    __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(y), r, static_cast<int>(2 * i), 0, 0);
}
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, uint32_t i, f2 y, float*) {
    __builtin_amdgcn_raw_buffer_store_b64(u2{__float_as_uint(y[0]), __float_as_uint(y[1])}, r, static_cast<int>(4 * i), 0, 0);
}
__device__ __forceinline__ void bst2(__amdgpu_buffer_rsrc_t r, uint32_t i, f2 y, bf16_t*) {
    const uint32_t x = static_cast<uint32_t>(f32_to_bf16(y[0])) | (static_cast<uint32_t>(f32_to_bf16(y[1])) << 16);
    __builtin_amdgcn_raw_buffer_store_b32(x, r, static_cast<int>(2 * i), 0, 0);
}

__device__ __forceinline__ f4 mfma4(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Z = X Y for 8 x 8 matrices in LDS (row-major); lane (a, b) = (l / 8, l % 8).
__device__ __forceinline__ float mat8(const float* X, const float* Y, int a, int b) {
    const f4 x0 = *reinterpret_cast<const f4*>(X + 8 * a);
    const f4 x1 = *reinterpret_cast<const f4*>(X + 8 * a + 4);
    float z = x0[0] * Y[b];
    z += x0[1] * Y[8 + b];
    z += x0[2] * Y[16 + b];
    z += x0[3] * Y[24 + b];
    z += x1[0] * Y[32 + b];
    z += x1[1] * Y[40 + b];
    z += x1[2] * Y[48 + b];
    z += x1[3] * Y[56 + b];
    return z;
}

// On lane (a, b) = (l / 8, l % 8) of one wave, with N = -A strictly lower
// (N^8 = 0) at (a, b) and P at (a, b): writes T = (I + N)(I + N^2)(I + N^4)
// = (I + A)^-1 to M[64..127] and P T to M[128..191] (row-major); M[0..63]
// and M[192..255] are scratch.  Ends with the products visible to the wave.
__device__ __forceinline__ void solve8(float* M, float nab, float pab, int a, int b, int l) {
    float* const M0 = M;
    float* const M1 = M + 64;
    float* const M2 = M + 128;
    float* const M3 = M + 192;
    M0[l] = nab;
    M3[l] = pab;
    __builtin_amdgcn_wave_barrier();
    const float n2 = mat8(M0, M0, a, b);
    M1[l] = n2;
    __builtin_amdgcn_wave_barrier();
    const float n3 = mat8(M0, M1, a, b);
    const float n4 = mat8(M1, M1, a, b);
    const float t1 = (a == b ? 1.f : 0.f) + nab + n2 + n3;
    __builtin_amdgcn_wave_barrier();
    M2[l] = t1;
    M0[l] = n4;
    __builtin_amdgcn_wave_barrier();
    const float tt = t1 + mat8(M2, M0, a, b);
    __builtin_amdgcn_wave_barrier();
    M1[l] = tt;
    __builtin_amdgcn_wave_barrier();
    const float pt = mat8(M3, M1, a, b);
    M2[l] = pt;
    __builtin_amdgcn_wave_barrier();
}

}  // namespace f32m
}  // namespace kda
