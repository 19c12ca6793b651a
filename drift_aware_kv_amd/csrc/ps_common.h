// ps_common.h -- device helpers and host-side argument checks shared by the
// libpolestar_drift kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include <algorithm>
#include <stdint.h>

#include "polestar_drift.h"
#include "ps_profile.h"

namespace ps {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;
constexpr int kMaxK = 1024;
constexpr int kMaxTopK = 64;

// ---------------------------------------------------------------------------
// number formats
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> struct Elem;
template <> struct Elem<uint16_t> {
    static __device__ __forceinline__ float get(const uint16_t* p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ void put(uint16_t* p, size_t i, float v) { p[i] = (uint16_t)f32_to_bf16(v); }
};
template <> struct Elem<float> {
    static __device__ __forceinline__ float get(const float* p, size_t i) { return p[i]; }
    static __device__ __forceinline__ void put(float* p, size_t i, float v) { p[i] = v; }
};

// 8 consecutive elements as fp32 (one 16-byte load for bf16, two for fp32)
__device__ __forceinline__ void load8(const uint16_t* p, float v[8])
{
    uint4 q = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ void load8(const float* p, float v[8])
{
    float4 a = reinterpret_cast<const float4*>(p)[0];
    float4 b = reinterpret_cast<const float4*>(p)[1];
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(uint16_t* p, const float v[8])
{
    uint4 q;
    q.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
    q.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
    q.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
    q.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
    *reinterpret_cast<uint4*>(p) = q;
}
__device__ __forceinline__ void store8(float* p, const float v[8])
{
    reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
    reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}

// E4M3 (bias 7, no infinities, 0x7e = 448): nearest, ties to even, saturating.
// Only non-negative scales are encoded; 0, negatives and NaN give 0.
__device__ __forceinline__ uint32_t e4m3_encode(float x)
{
    if (!(x > 0.0f)) return 0u;
    if (x >= 448.0f) return 0x7eu;
    const uint32_t u = __float_as_uint(x);
    const int ex = (int)(u >> 23) - 127;
    if (ex < -6) {
        // subnormal range: value = m * 2^-9, m = round_even(x * 512); the
        // scaling is exact, and m = 8 is the smallest normal (code 0x08)
        return (uint32_t)__builtin_rintf(x * 512.0f);
    }
    const uint32_t mant = u & 0x7fffffu;
    const uint32_t keep = mant >> 20, rem = mant & 0xfffffu;
    uint32_t code = ((uint32_t)(ex + 7) << 3) | keep;
    if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) code += 1u;  // carries into the exponent
    return code > 0x7eu ? 0x7eu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c)
{
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 magnitude index by threshold: nearest of {0,.5,1,1.5,2,3,4,6}, ties to
// the even index, saturating; NaN -> 0; a zero magnitude is +0.
__device__ __forceinline__ uint32_t e2m1_encode(float v)
{
    const float a = fabsf(v);
    const uint32_t i = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                       (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                       (uint32_t)(a > 5.0f);
    if (i == 0) return 0u;
    return (v < 0.0f ? 8u : 0u) | i;
}

__device__ __forceinline__ float e2m1_decode(uint32_t n)
{
    // magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 by index
    const uint32_t i = n & 7u;
    float m = i < 4 ? 0.5f * (float)i : (float)(2u << ((i - 4u) >> 1)) * (1.0f + 0.5f * (float)(i & 1u));
    return (n & 8u) ? -m : m;
}

// ---------------------------------------------------------------------------
// wave helpers
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

__device__ __forceinline__ double shfl_xor_d(double v, int m) { return __shfl_xor(v, m, 64); }

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}
__device__ __forceinline__ double wave_sum_d(double v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup b runs on
// XCD b % 8).  Return a logical index such that the workgroups of one XCD get
// consecutive logical indices, so tiles that share data (one window's tiles)
// share one XCD's L2.
__device__ __forceinline__ int xcd_remap(int b, int nblocks)
{
    const int x = b & 7, i = b >> 3, q = nblocks >> 3, r = nblocks & 7;
    return x * q + (x < r ? x : r) + i;
}

}  // namespace ps

// ---------------------------------------------------------------------------
// host-side checks (no HIP calls)
// ---------------------------------------------------------------------------
namespace ps_host {

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

inline bool dtype_ok(int dt) { return dt == PS_F32 || dt == PS_BF16; }

inline size_t elem_size(int dt) { return dt == PS_BF16 ? 2 : 4; }

inline ps_status check_window(const ps_shape* s)
{
    if (!s) return PS_ERR_NULL;
    if (s->W < 0 || s->N < 1 || s->N >= (1 << 24) || s->d < 16 || s->d % 16 != 0) return PS_ERR_SHAPE;
    if ((int64_t)s->N * s->d >= ((int64_t)1 << 31)) return PS_ERR_SHAPE;
    return PS_OK;
}

// scratch of the grouped NVFP4 coder: the grouped row order, the list of rows
// for the exact path and its count (int32 each)
inline size_t residual_ws_bytes(const ps_shape* s)
{
    return 8 * (size_t)s->W * (size_t)s->N + 16;
}

inline ps_status check_clusters(const ps_shape* s)
{
    ps_status st = check_window(s);
    if (st != PS_OK) return st;
    if (s->K < 1 || s->K > s->N || s->K > ps::kMaxK) return PS_ERR_SHAPE;
    return PS_OK;
}

inline ps_status check_heads(const ps_shape* s)
{
    if (s->Hq < 1 || s->Hkv < 1 || s->Hq % s->Hkv != 0 || s->dh < 8 || s->dh % 8 != 0) return PS_ERR_SHAPE;
    if ((int64_t)s->N * s->Hkv * s->dh >= ((int64_t)1 << 31)) return PS_ERR_SHAPE;
    return PS_OK;
}

inline size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

// The exact NVFP4 coder over the bf16 rows listed in list[0 .. *listed)
// (rows of up to 4096 elements), against their clusters' centres in C.
// Enqueued on st.
void residual_listed(const ps_shape* s, const uint16_t* H, const float* row_norm, const float* C,
                     const int32_t* assign, const int32_t* list, const int32_t* listed, uint8_t* codes,
                     uint8_t* bscale, float* rscale, hipStream_t st);

}  // namespace ps_host
