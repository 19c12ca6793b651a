// ps_hwcheck.hip -- test-only GPU sweeps over every input of the ranges on
// which the NVFP4 coder's fast path relies on gfx950's conversions and on its
// Newton reciprocal (ps_nvfp4_fast.h).  The expected results come from the
// caller as rounding thresholds: the bit pattern at which each code begins
// (E2M1: from the OCP microscaling rounding table; E4M3: from the nearest-even
// rule over the format's values).  Not part of the library: the test suite
// builds it beside itself and calls it through ctypes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ps_nvfp4_fast.h"

using namespace ps;

namespace {

struct Thr7 { uint32_t t[7]; };

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const unsigned long long o = __shfl_xor(v, m, 64);
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v)
{
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        const unsigned long long o = __shfl_xor(v, m, 64);
        v = o > v ? o : v;
    }
    return v;
}

// out[0] += mismatches, out[1] = min(out[1], first mismatching pattern)
__device__ __forceinline__ void report(unsigned long long bad, unsigned long long first,
                                       unsigned long long* out)
{
    bad = wave_sum_u64(bad);
    first = wave_min_u64(first);
    if ((threadIdx.x & 63) == 0 && bad) {
        atomicAdd(out, bad);
        atomicMin(out + 1, first);
    }
}

// Every fp32 pattern u in [base, base + count) that is finite: the fast E2M1
// code of u, written into all eight nibbles of a word (both halves of each of
// the four byte positions the coder uses), against sign | #{thresholds <= |u|}
// (zero magnitude always +0).
__global__ __launch_bounds__(256) void k_e2m1(uint64_t base, uint64_t count, Thr7 thr, unsigned long long* out)
{
    unsigned long long bad = 0, first = ~0ull;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
        const uint32_t u = (uint32_t)(base + i);
        if ((u & 0x7f800000u) == 0x7f800000u) continue;      // inf / NaN: never on the fast path
        const float f = __uint_as_float(u);
        uint32_t w = e2m1x2_fast<0>(0u, f, f);
        w = e2m1x2_fast<1>(w, f, f);
        w = e2m1x2_fast<2>(w, f, f);
        w = plus_zero(e2m1x2_fast<3>(w, f, f));
        const uint32_t a = u & 0x7fffffffu;
        uint32_t idx = 0;
#pragma unroll
        for (int t = 0; t < 7; ++t) idx += a >= thr.t[t];
        const uint32_t want = idx ? (((u >> 31) << 3) | idx) : 0u;
        if (w != want * 0x11111111u) {
            ++bad;
            first = first < u ? first : u;
        }
    }
    report(bad, first, out);
}

// u in [base, base + count) (non-negative fp32 patterns below 464): the fast
// E4M3 code against #{thresholds <= u} (thr[0 .. n) ascending)
__global__ __launch_bounds__(256) void k_e4m3(uint64_t base, uint64_t count, const uint32_t* __restrict__ thr,
                                               int n, unsigned long long* out)
{
    unsigned long long bad = 0, first = ~0ull;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
        const uint32_t u = (uint32_t)(base + i);
        int lo = 0, hi = n;                 // first threshold above u
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (thr[mid] <= u) lo = mid + 1; else hi = mid;
        }
        if (e4m3_fast(__uint_as_float(u)) != (uint32_t)lo) {
            ++bad;
            first = first < u ? first : u;
        }
    }
    report(bad, first, out);
}

// decoded values of codes 0 .. n-1
__global__ void k_e4m3_decode(float* __restrict__ out, int n)
{
    const int c = blockIdx.x * blockDim.x + threadIdx.x;
    if (c < n) out[c] = e4m3_fast_decode((uint32_t)c);
}

// b over fp32 patterns [base, base + count): r = fma(-b, y, 1) for
// y = recip_nr(b); out[0] += #{|r| >= limit}, out[1] = first such pattern,
// out[2] = max |r| as fp64 bits (non-negative doubles order as integers)
__global__ __launch_bounds__(256) void k_recip(uint64_t base, uint64_t count, double limit,
                                                unsigned long long* out)
{
    unsigned long long bad = 0, first = ~0ull, worst = 0;
    const uint64_t stride = (uint64_t)gridDim.x * 256;
    for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
        const uint32_t u = (uint32_t)(base + i);
        const float b = __uint_as_float(u);
        const double y = recip_nr(b);
        const double r = fabs(fma(-(double)b, y, 1.0));
        const unsigned long long rb = (unsigned long long)__double_as_longlong(r);
        worst = rb > worst ? rb : worst;
        if (!(r < limit)) {
            ++bad;
            first = first < u ? first : u;
        }
    }
    report(bad, first, out);
    worst = wave_max_u64(worst);
    if ((threadIdx.x & 63) == 0) atomicMax(out + 2, worst);
}

constexpr int kGrid = 8192;

}  // namespace

extern "C" int psx_e2m1_sweep(uint64_t base, uint64_t count, const uint32_t* thr7, unsigned long long* out)
{
    Thr7 t;
    for (int i = 0; i < 7; ++i) t.t[i] = thr7[i];
    hipLaunchKernelGGL(k_e2m1, dim3(kGrid), dim3(256), 0, 0, base, count, t, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int psx_e4m3_sweep(uint64_t base, uint64_t count, const uint32_t* thr_dev, int n,
                              unsigned long long* out)
{
    hipLaunchKernelGGL(k_e4m3, dim3(kGrid), dim3(256), 0, 0, base, count, thr_dev, n, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int psx_e4m3_decode(float* out, int n)
{
    hipLaunchKernelGGL(k_e4m3_decode, dim3((n + 255) / 256), dim3(256), 0, 0, out, n);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}

extern "C" int psx_recip_sweep(uint64_t base, uint64_t count, double limit, unsigned long long* out)
{
    hipLaunchKernelGGL(k_recip, dim3(kGrid), dim3(256), 0, 0, base, count, limit, out);
    return hipGetLastError() == hipSuccess ? 0 : 1;
}
