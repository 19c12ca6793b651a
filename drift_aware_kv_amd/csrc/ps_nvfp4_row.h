// ps_nvfp4_row.h -- the fast path of the NVFP4 residual coder for one row
// held in registers (Polestar technical summary 2.A, local window and
// clustering: residuals to the cluster centres are stored in NVFP4), shared by
// the coder kernels and the K-Means update that codes a cluster's members
// right after rebuilding its centre (gfx950, wave64).
#pragma once

#include "ps_common.h"
#include "ps_nvfp4_fast.h"

namespace ps {

// Quotients on the fast path: for fp32 a and b, the fp32 rounding of
// a * y, with y within 2^-51 (relative) of 1/b, equals the correctly rounded
// fp32 quotient a / b whenever that quotient is zero or at least 2^-125 in
// magnitude.  A quotient that is not an fp32 number lies at least 2^-49
// (relative) from every fp32 rounding midpoint (with m a midpoint of 25
// significant bits, a - m*b is a non-zero multiple of 2^(e_m + e_b - 47),
// since a has at most 24 significant bits), while the fp64 product is within
// 2^-50 of a / b.  y is RN64(1/b) for the norm n and the constants 6 and
// 2688; for the row scale g and each block's eff, both normal fp32 numbers in
// [2^-126, 2^126) on this path, it is the fp32 reciprocal estimate refined by
// two Newton steps in fp64 (`recip_nr`, within 2^-52 over that range).  Below the normal
// range the midpoints are coarser than that argument covers: a row with a
// non-zero |h| or |r| whose exponent is 125 or more below its divisor's, or
// subnormal, is redone with divisions (`residual_row_exact`); so is a row with
// a non-finite residual or with a largest |r| below 2^-100, under which the
// block-scale quotients lose their margin.  With max |r| >= 2^-100 a block whose Ab/6 is below 2^-125
// has (Ab/6)/g below 2^-13, which encodes to the E4M3 zero either way.
//
// E2M1 and E4M3 rounding on the fast path use gfx950's conversions
// (ps_nvfp4_fast.h states the range over which each equals the convention's
// rounding; the test suite sweeps every input of those ranges on the GPU).

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, m, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_min_u(uint32_t v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, m, 64));
    return v;
}

// a non-zero magnitude (fp32 bits) too small against a divisor (fp32 bits)
// for the reciprocal-product argument: subnormal, or 125+ binades below
__device__ __forceinline__ bool tiny_against(uint32_t mag, uint32_t div)
{
    const int e = (int)(mag >> 23);
    return mag != 0u && (e == 0 || e + 125 <= (int)(div >> 23));
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u16x2 wave_min_u16x2(u16x2 v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v = __builtin_elementwise_min(v, __builtin_bit_cast(u16x2, __shfl_xor(__builtin_bit_cast(int, v), m, 64)));
    return v;
}

// Block layout of the fast path: thread i of the row owns the 16-element
// blocks i, i + TPR, ..., so every block scale is computed once, by the thread
// that codes the block.  Blocks past the row read the last block again (always
// in bounds) and are masked.
template <typename T, int TPR, int BPL>
__device__ __forceinline__ void load_hblocks(const T* __restrict__ h, int tid, int nb,
                                             uint4 (&hq)[BPL][sizeof(T) == 2 ? 2 : 4])
{
    constexpr int HW = sizeof(T) == 2 ? 2 : 4;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const uint4* hp = reinterpret_cast<const uint4*>(h + 16 * min(tid + TPR * b, nb - 1));
#pragma unroll
        for (int q = 0; q < HW; ++q) hq[b][q] = hp[q];
    }
}

template <int TPR, int BPL>
__device__ __forceinline__ void load_cblocks(const float* __restrict__ c, int tid, int nb, float (&cv)[BPL][16])
{
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const float4* cp = reinterpret_cast<const float4*>(c + 16 * min(tid + TPR * b, nb - 1));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 v = cp[q];
            cv[b][4 * q] = v.x; cv[b][4 * q + 1] = v.y; cv[b][4 * q + 2] = v.z; cv[b][4 * q + 3] = v.w;
        }
    }
}

// Fast NVFP4 coding of one row: reciprocal products instead of divisions, the
// hardware E4M3 and E2M1 conversions (checked exhaustively against the
// software rounding: E4M3 over every fp32 in [0, 464), which holds every block
// scale quotient, E2M1 over every finite fp32), and the checks folded into
// integer max/min over magnitude bit patterns (which also catch NaN and
// infinity).  The row's largest |r| and smallest non-zero |h| are combined in
// one reduction; from them every thread takes the same decision whether the
// row needs the exact path, before any block is coded.  Quotients r/eff below
// 2^-125 need no check: they encode to the E2M1 zero however they round.
// Returns false without writing anything when the exact path is needed.
// The row's h and centre blocks arrive loaded (load_hblocks, load_cblocks).
template <typename T, int NW, int BPL, bool FULL>
__device__ __forceinline__ bool residual_row_fast(const uint4 (&hq)[BPL][sizeof(T) == 2 ? 2 : 4],
                                                  const float (&cv)[BPL][16], float n,
                                                  uint8_t* __restrict__ cr, uint8_t* __restrict__ br,
                                                  float* __restrict__ rs, int d, uint32_t (*red)[3])
{
    constexpr int TPR = 64 * NW;
    constexpr bool packed = sizeof(T) == 2;
    if (!(n > 0.0f) || n == INFINITY) return false;   // row-uniform: zero, negative or non-finite norm
    const int tid = (int)(threadIdx.x % TPR), wave = tid >> 6;
    const int nb = d >> 4;
    const double inv_n = 1.0 / (double)n;
    float r[BPL][16];
    uint32_t bmax[BPL];
    // bf16: per half, 2|h| - 2 (mod 2^16): the sign drops out, zero maps to
    // 0xfffe above every non-zero magnitude; fp32: |h| - 1 over the bit patterns
    u16x2 hkey = {0xffff, 0xffff};
    uint32_t hmin = ~0u;
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        const bool valid = FULL || tid + TPR * b < nb;
        float hv[16];
        if (packed) {
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const uint32_t w4[4] = {hq[b][q].x, hq[b][q].y, hq[b][q].z, hq[b][q].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const u16x2 x = __builtin_bit_cast(u16x2, w4[t]);
                    hkey = __builtin_elementwise_min(hkey, x * (u16x2){2, 2} + (u16x2){0xfffe, 0xfffe});
                    hv[8 * q + 2 * t] = __uint_as_float(w4[t] << 16);
                    hv[8 * q + 2 * t + 1] = __uint_as_float(w4[t] & 0xffff0000u);
                }
            }
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint32_t w4[4] = {hq[b][q].x, hq[b][q].y, hq[b][q].z, hq[b][q].w};
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    hmin = min(hmin, (w4[t] & 0x7fffffffu) - 1u);
                    hv[4 * q + t] = __uint_as_float(w4[t]);
                }
            }
        }
        float m = 0.0f;                          // NaN-propagating max of |r|
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            float rv = (float)((double)hv[t] * inv_n) - cv[b][t];
            if (!FULL) rv = valid ? rv : 0.0f;
            r[b][t] = rv;
            m = __builtin_elementwise_maximum(m, fabsf(rv));
        }
        bmax[b] = __float_as_uint(m);            // non-negative: bit order is value order, NaN on top
    }
    uint32_t Am = 0;
#pragma unroll
    for (int b = 0; b < BPL; ++b) Am = max(Am, bmax[b]);
    Am = wave_max_u(Am);
    uint32_t hm;                                 // smallest non-zero |h| minus one, fp32-bit order
    if (packed) {
        hkey = wave_min_u16x2(hkey);
        const uint32_t k16 = min((uint32_t)hkey.x, (uint32_t)hkey.y);
        hm = k16 >= 0xfffeu ? ~0u : ((((k16 + 2u) >> 1)) << 16) - 1u;
    } else {
        hm = wave_min_u(hmin);
    }
    if (NW > 1) {
        if ((tid & 63) == 0) {
            red[wave][0] = Am;
            red[wave][1] = hm;
        }
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NW; ++q) {
            Am = max(Am, red[q][0]);
            hm = min(hm, red[q][1]);
        }
    }
    // row-uniform decision
    if (Am >= 0x7f800000u) return false;                 // a NaN or infinite residual
    const bool zero_row = Am == 0u;
    if (!zero_row && Am < 0x0d800000u) return false;     // max |r| below 2^-100
    if (tiny_against(hm + 1u, __float_as_uint(n))) return false;
    const float g = (float)((double)__uint_as_float(Am) * (1.0 / 2688.0));   // >= 2^-112 unless zero
    const double inv_g = zero_row ? 0.0 : recip_nr(g);
#pragma unroll
    for (int b = 0; b < BPL; ++b) {
        uint32_t w0 = 0, w1 = 0, sb = 0;
        if (!zero_row) {
            const float q1 = (float)((double)__uint_as_float(bmax[b]) * (1.0 / 6.0));
            const float q2 = (float)((double)q1 * inv_g);
            sb = e4m3_fast(q2);
            const float eff = e4m3_fast_decode(sb) * g;
            if (eff != 0.0f) {
                const double y = recip_nr(eff);
                float v[16];
#pragma unroll
                for (int t = 0; t < 16; ++t) v[t] = (float)((double)r[b][t] * y);
                w0 = e2m1x2_fast<0>(w0, v[0], v[1]);
                w0 = e2m1x2_fast<1>(w0, v[2], v[3]);
                w0 = e2m1x2_fast<2>(w0, v[4], v[5]);
                w0 = e2m1x2_fast<3>(w0, v[6], v[7]);
                w1 = e2m1x2_fast<0>(w1, v[8], v[9]);
                w1 = e2m1x2_fast<1>(w1, v[10], v[11]);
                w1 = e2m1x2_fast<2>(w1, v[12], v[13]);
                w1 = e2m1x2_fast<3>(w1, v[14], v[15]);
                w0 = plus_zero(w0);
                w1 = plus_zero(w1);
            }
        }
        // 32-bit offsets from the row's base, made opaque so that the compiler
        // forms them per row instead of keeping them live across a row loop
        unsigned blk = (unsigned)(tid + TPR * b);
        __asm__ volatile("" : "+v"(blk));
        if (FULL || blk < (unsigned)nb) {
            *reinterpret_cast<uint2*>(cr + 8u * blk) = make_uint2(w0, w1);
            br[blk] = (uint8_t)sb;
        }
    }
    if (tid == 0) *rs = zero_row ? 0.0f : g;
    return true;
}

}  // namespace ps
