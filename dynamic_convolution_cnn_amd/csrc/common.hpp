// Device-side helpers shared by the gfx950 kernels of the dynamic
// convolution library: storage types, bf16 conversion, the MFMA operand
// vector types and wave reductions. Host code includes only kernels.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dynconv {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// bf16 storage is handled as raw 16-bit patterns (uint16_t) in memory.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// Two floats to a packed pair of bf16 (round to nearest even; gfx950
// lowers this to v_cvt_pk_bf16_f32). `lo` lands in bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2_t v = {lo, hi};
    bf16x2_t b = __builtin_convertvector(v, bf16x2_t);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return (uint16_t)(pack_bf16x2(f, 0.0f) & 0xffffu);
}

// Storage element <-> float for the two supported element types.
template <typename T> struct Elem;
template <> struct Elem<float> {
    static __device__ __forceinline__ float load(const float *p) { return *p; }
    static __device__ __forceinline__ float to_f32(float v) { return v; }
    static __device__ __forceinline__ float from_f32(float v) { return v; }
};
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t *p) { return bf16_to_f32(*p); }
    static __device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }
    static __device__ __forceinline__ uint16_t from_f32(float v) { return f32_to_bf16(v); }
};

// Sum over the 64 lanes of a wave; every lane receives the total. The
// reduction tree is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}
// Sum within aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__host__ __device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Workgroup barrier for LDS traffic only. __syncthreads() also waits for
// every outstanding global load of the wave (vmcnt(0)), which would drain
// the prefetches a software pipeline keeps in flight across its per-step
// barriers. Here each wave waits only for its own LDS operations
// (lgkmcnt(0); s_waitcnt encoding with vmcnt and expcnt at their maxima),
// then meets the others at s_barrier. The empty asm statements keep the
// compiler from moving memory accesses across the barrier. Global memory
// written before the barrier is NOT made visible by it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

}  // namespace dynconv
