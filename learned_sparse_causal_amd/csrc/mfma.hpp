// MFMA fragments for gfx950: one 16x16 output tile, k consumed 32 at a time.
//
// Lane l of a 16x16x32 bf16 MFMA holds A[m = l%16][k = 8(l/16) .. 8(l/16)+7]
// and B[k = 8(l/16) .. +7][n = l%16]; the fp32 accumulator holds
// D[m = 4(l/16) + r][n = l%16], r = 0..3.  The fp32 path issues eight
// 16x16x4 MFMAs whose k index (l/16) stands for element e of the same
// 8-element fragments, so both paths load fragments identically.
#pragma once

#include "common.hpp"

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

template <bool BF16>
struct Frag8;

template <>
struct Frag8<true> {
    bf16x8 v;
};

template <>
struct Frag8<false> {
    float v[8];
};

__device__ __forceinline__ void mma32(f32x4 &acc, const Frag8<true> &a, const Frag8<true> &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma32(f32x4 &acc, const Frag8<false> &a, const Frag8<false> &b) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[e], b.v[e], acc, 0, 0, 0);
}

// 8 contiguous LDS elements (16-byte aligned for bf16, 32-byte for fp32).
__device__ __forceinline__ Frag8<true> lds_frag8(const u16 *p) {
    Frag8<true> f;
    f.v = *reinterpret_cast<const bf16x8 *>(p);
    return f;
}

__device__ __forceinline__ Frag8<false> lds_frag8(const float *p) {
    Frag8<false> f;
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}

// Two runs of 4 contiguous LDS elements (8-byte aligned for bf16).
__device__ __forceinline__ Frag8<true> lds_frag4x2(const u16 *p0, const u16 *p1) {
    const uint2 a = *reinterpret_cast<const uint2 *>(p0);
    const uint2 b = *reinterpret_cast<const uint2 *>(p1);
    uint4 w = {a.x, a.y, b.x, b.y};
    Frag8<true> f;
    f.v = __builtin_bit_cast(bf16x8, w);
    return f;
}

__device__ __forceinline__ Frag8<false> lds_frag4x2(const float *p0, const float *p1) {
    Frag8<false> f;
    const float4 a = *reinterpret_cast<const float4 *>(p0);
    const float4 b = *reinterpret_cast<const float4 *>(p1);
    f.v[0] = a.x; f.v[1] = a.y; f.v[2] = a.z; f.v[3] = a.w;
    f.v[4] = b.x; f.v[5] = b.y; f.v[6] = b.z; f.v[7] = b.w;
    return f;
}

// Fragment from 8 floats in registers (rounded to bf16 for the bf16 path).
__device__ __forceinline__ Frag8<true> reg_frag8_bf16(const float *x) {
    uint4 w;
    w.x = pack_bf16x2(x[0], x[1]);
    w.y = pack_bf16x2(x[2], x[3]);
    w.z = pack_bf16x2(x[4], x[5]);
    w.w = pack_bf16x2(x[6], x[7]);
    Frag8<true> f;
    f.v = __builtin_bit_cast(bf16x8, w);
    return f;
}

template <bool BF16>
__device__ __forceinline__ Frag8<BF16> reg_frag8(const float *x) {
    if constexpr (BF16) {
        return reg_frag8_bf16(x);
    } else {
        Frag8<false> f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f.v[e] = x[e];
        return f;
    }
}
