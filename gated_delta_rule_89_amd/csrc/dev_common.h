// Device helpers shared by the KDA kernels (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest, ties to even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float x) { p[i] = x; }
};
template <> struct Elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) {
        return bf16_to_f32(p[i].bits);
    }
    __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float x) {
        p[i].bits = f32_to_bf16(x);
    }
};

template <typename T>
__device__ __forceinline__ float ld(const T* p, int64_t i) { return Elem<T>::load(p, i); }
template <typename T>
__device__ __forceinline__ void st(T* p, int64_t i, float x) { Elem<T>::store(p, i, x); }

// exp(x) for the forget gate.  v_exp_f32 computes 2^x; the scaling by
// log2(e) is the usual change of base.
__device__ __forceinline__ float gate_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }

}  // namespace kda
