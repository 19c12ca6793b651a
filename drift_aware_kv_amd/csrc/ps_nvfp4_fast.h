// ps_nvfp4_fast.h -- the hardware conversions and the reciprocal of the NVFP4
// coder's fast path (gfx950).  Each stands in for one correctly rounded step
// of the coder's convention only where it provably gives the same result:
//
//  - fp32 -> E2M1 (`e2m1x2_fast`, the fp32 -> fp4 conversion with scale 1.0,
//    followed by `plus_zero`): nearest, ties to even, saturating at 6, over
//    every finite fp32 input;
//  - fp32 -> E4M3 (`e4m3_fast`): nearest, ties to even, saturating at 448,
//    over [0, 464), which holds every block-scale quotient of the coder;
//  - E4M3 -> fp32 (`e4m3_fast_decode`): exact, over the codes 0 .. 0x7e;
//  - `recip_nr`: 1/b within 2^-52 (relative) for every normal fp32 b in
//    [2^-126, 2^126).
//
// The sweeps that establish these over every input of their ranges run on
// the GPU in the test suite, against the E2M1 rounding table of the OCP
// microscaling specification and the E4M3 rounding the CPU oracle implements.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ps {

// The fp32 -> fp4 conversion returns a negative input that rounds to zero as
// -0 (nibble 0x8); the convention stores every zero as +0.  Clears the sign
// of every zero-magnitude nibble of a packed word.
__device__ __forceinline__ uint32_t plus_zero(uint32_t w)
{
    const uint32_t m = w & 0x77777777u;                              // magnitudes
    const uint32_t nz = (m | (m >> 1) | (m >> 2)) & 0x11111111u;     // magnitude != 0
    return m | (w & (nz << 3));
}

// Byte SEL (0..3) of w replaced by the E2M1 codes of a (low nibble) and b
// (high nibble); a negative input that rounds to zero gives -0, which
// `plus_zero` then clears.
template <int SEL>
__device__ __forceinline__ uint32_t e2m1x2_fast(uint32_t w, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a, b, 1.0f, SEL);
}

// E4M3 code of a non-negative fp32 q in [0, 464)
__device__ __forceinline__ uint32_t e4m3_fast(float q)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q, q, 0, false) & 0xffu;
}

// value of an E4M3 code 0 .. 0x7e
__device__ __forceinline__ float e4m3_fast_decode(uint32_t code)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// 1/b: the fp32 reciprocal estimate refined by two Newton steps in fp64 (the
// relative error e of the estimate becomes about e^4 plus fp64 rounding)
__device__ __forceinline__ double recip_nr(float b)
{
    const double b64 = (double)b;
    double y = (double)__builtin_amdgcn_rcpf(b);
#pragma unroll
    for (int it = 0; it < 2; ++it) y = fma(y, fma(-b64, y, 1.0), y);
    return y;
}

}  // namespace ps
