// Device-side helpers shared by the gfx950 kernels of the routed attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));   // 16-byte register vector

// Validated sizes of one call (host fills it, kernels take it by value).
struct Shape {
    int B, T, W, Hq, Hkv, d, beta, P, K, cap, npr, R, L, dtype;
    int NB, A, G, ds;
};

static constexpr int WAVE = 64;

// Host helpers (defined in capi.cpp), cached per (kernel, device) so that
// repeated launches make no runtime queries:
//  - raise a kernel's dynamic LDS limit to at least `bytes` (bytes > 64 KiB);
//  - workgroups of `threads` threads and `lds` bytes resident at once on the
//    current device (compute units x occupancy, at least 1).
hipError_t mono_lds_limit(const void *fn, size_t bytes);
long mono_resident_workgroups(const void *fn, int threads, size_t lds);

__device__ __forceinline__ float bf16_bits_to_f32(u16 b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// Round to nearest bfloat16, ties to even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ u16 f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(u16, (__bf16)f);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bfloat16 pair (low half = a), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    const f32x2_t x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2_t));
}

// Load 8 consecutive activations starting at element i (16-byte aligned for
// bf16, 32-byte aligned for fp32) as floats.
template <bool BF16>
__device__ __forceinline__ void load8(const void *base, size_t i, float *out) {
    if constexpr (BF16) {
        const uint4 v = *reinterpret_cast<const uint4 *>(reinterpret_cast<const u16 *>(base) + i);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            out[2 * e] = __uint_as_float(w[e] << 16);
            out[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
    } else {
        const float4 *p = reinterpret_cast<const float4 *>(reinterpret_cast<const float *>(base) + i);
        const float4 a = p[0], b = p[1];
        out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
        out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    }
}

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, size_t i) {
    if constexpr (BF16) return bf16_bits_to_f32(reinterpret_cast<const u16 *>(base)[i]);
    else return reinterpret_cast<const float *>(base)[i];
}

template <bool BF16>
__device__ __forceinline__ void store1(void *base, size_t i, float v) {
    if constexpr (BF16) reinterpret_cast<u16 *>(base)[i] = f32_to_bf16_bits(v);
    else reinterpret_cast<float *>(base)[i] = v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (WAVE - 1); }

// Broadcast a value known to be wave-uniform into a scalar register.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
