// ps_nvfp4.hip -- NVFP4 residual coding of the window rows (Polestar
// technical summary 2.A, local window and clustering: residuals to the
// cluster centres are stored in NVFP4) and the refresh gather of the rows of
// the selected clusters (2.A, sparse updates; 2.C, only the selected clusters
// are fetched), for gfx950.
//
// Both kernels are bandwidth bound: one wave per row, 16-byte coalesced
// loads, E4M3/E2M1 rounding in integer/fp32 arithmetic (every fp32 step is one
// correctly rounded operation, matching the stated convention bit for bit).
#include "ps_common.h"

using namespace ps;

namespace {

// Correctly rounded fp32 quotient a / b from an fp64 product with the fp64
// reciprocal of b.  For fp32 a and b, a quotient that is not an fp32 number
// lies at least 2^-49 (relative) from every fp32 rounding midpoint: with m a
// midpoint (25 significant bits) a - m*b is a non-zero multiple of
// 2^(e_m + e_b - 47), since a has at most 24 significant bits.  The product
// a * RN64(1/b) is within 2^-52 of a / b, so its fp32 rounding is the
// correctly rounded quotient.  Below the fp32 normal range the midpoints are
// coarser than that argument covers, so such quotients take the division.
__device__ __forceinline__ float div_by_recip(float a, double inv_b, float b)
{
    const double q = (double)a * inv_b;
    if (q != 0.0 && fabs(q) < 0x1p-125) return a / b;
    return (float)q;
}

// One wave per row.  Lane l holds 8-element chunks l, l+64, ...; a 16-element
// NVFP4 block is the chunk pair (2m, 2m+1), i.e. lanes l and l^1.
template <typename T, int CPL>
__global__ __launch_bounds__(256) void k_residual(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                   const float* __restrict__ C, const int32_t* __restrict__ assign,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                   float* __restrict__ rscale, int64_t rows, int N, int d, int K)
{
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;  // uniform per wave
    const int lane = lane_id();
    const int w = (int)(row / N);
    const float n = row_norm[row];
    const double inv_n = n > 0.0f ? 1.0 / (double)n : 0.0;
    int a = assign[row];
    if (a < 0 || a >= K) a = 0;
    const float* c = C + ((size_t)w * K + a) * d;
    const T* h = H + (size_t)row * d;
    const int nch = d >> 3;

    float r[CPL][8];
    float A = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        if (ch < nch) {
            float hv[8], cv[8];
            load8(h + 8 * ch, hv);
            load8(c + 8 * ch, cv);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const float x = n > 0.0f ? div_by_recip(hv[t], inv_n, n) : 0.0f;
                r[i][t] = x - cv[t];
                const float m = fabsf(r[i][t]);
                if (m > A) A = m;
            }
        } else {
#pragma unroll
            for (int t = 0; t < 8; ++t) r[i][t] = 0.0f;
        }
    }
    A = wave_max(A);
    uint8_t* cr = codes + (size_t)row * (d >> 1);
    uint8_t* br = bscale + (size_t)row * (d >> 4);
    if (!(A > 0.0f)) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            const int ch = lane + 64 * i;
            if (ch < nch) {
                *reinterpret_cast<uint32_t*>(cr + 4 * ch) = 0u;
                if (!(ch & 1)) br[ch >> 1] = 0;
            }
        }
        if (lane == 0) rscale[row] = 0.0f;
        return;
    }
    const float g = A / 2688.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = lane + 64 * i;
        float Ab = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float m = fabsf(r[i][t]);
            if (m > Ab) Ab = m;
        }
        Ab = fmaxf(Ab, __shfl_xor(Ab, 1, 64));
        if (ch < nch) {
            const float t6 = Ab / 6.0f;
            const uint32_t sb = e4m3_encode(t6 / g);
            const float eff = e4m3_decode(sb) * g;
            uint32_t word = 0;
            if (eff != 0.0f) {
                const double inv_eff = 1.0 / (double)eff;
#pragma unroll
                for (int t = 0; t < 8; ++t) word |= e2m1_encode(div_by_recip(r[i][t], inv_eff, eff)) << (4 * t);
            }
            *reinterpret_cast<uint32_t*>(cr + 4 * ch) = word;
            if (!(ch & 1)) br[ch >> 1] = (uint8_t)sb;
        }
    }
    if (lane == 0) rscale[row] = g;
}

// stable compaction of the members of the selected clusters, one wave per window
__global__ __launch_bounds__(64) void k_gather_select(const int32_t* __restrict__ assign,
                                                       const int32_t* __restrict__ idx, int k, int cap,
                                                       int32_t* __restrict__ pos, int32_t* __restrict__ count,
                                                       int N, int K)
{
    __shared__ uint8_t sel[kMaxK];
    const int w = blockIdx.x, lane = lane_id();
    for (int c = lane; c < K; c += 64) sel[c] = 0;
    __syncthreads();
    for (int r = lane; r < k; r += 64) {
        const int c = idx[(size_t)w * k + r];
        if (c >= 0 && c < K) sel[c] = 1;
    }
    __syncthreads();
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int32_t* a = assign + (size_t)w * N;
    int running = 0;
    for (int base = 0; base < N; base += 64) {
        const int j = base + lane;
        bool p = false;
        if (j < N) {
            const int c = a[j];
            p = c >= 0 && c < K && sel[c];
        }
        const uint64_t m = __ballot(p);
        const int slot = running + __popcll(m & lt);
        if (p && slot < cap) pos[(size_t)w * cap + slot] = j;
        running += __popcll(m);
    }
    if (lane == 0) count[w] = running;
}

// rebuild / copy the gathered rows; grid (G, W), each workgroup strides over slots
template <typename T>
__global__ __launch_bounds__(256) void k_gather_rows(const int32_t* __restrict__ pos,
                                                      const int32_t* __restrict__ count, int cap,
                                                      const int32_t* __restrict__ assign,
                                                      const uint8_t* __restrict__ codes,
                                                      const uint8_t* __restrict__ bscale,
                                                      const float* __restrict__ rscale,
                                                      const float* __restrict__ C,
                                                      const float* __restrict__ row_norm,
                                                      T* __restrict__ H_hat, const T* __restrict__ Kc,
                                                      const T* __restrict__ Vc, T* __restrict__ K_out,
                                                      T* __restrict__ V_out, int N, int d, int K, int KV)
{
    const int w = blockIdx.y;
    const int cnt = count[w];
    const int M = cnt < cap ? cnt : cap;
    const int kv16 = (int)((size_t)KV * sizeof(T) / 16);
    for (int slot = blockIdx.x; slot < M; slot += gridDim.x) {
        const int j = pos[(size_t)w * cap + slot];
        const size_t row = (size_t)w * N + j;
        const size_t orow = (size_t)w * cap + slot;
        if (H_hat) {
            int a = assign[row];
            if (a < 0 || a >= K) a = 0;
            const float g = rscale[row], n = row_norm[row];
            const float* c = C + ((size_t)w * K + a) * d;
            for (int ch = threadIdx.x; ch < (d >> 3); ch += 256) {
                const uint32_t word = *reinterpret_cast<const uint32_t*>(codes + row * (size_t)(d >> 1) + 4 * ch);
                const float sh = e4m3_decode(bscale[row * (size_t)(d >> 4) + (ch >> 1)]);
                float cv[8], o[8];
                load8(c + 8 * ch, cv);
#pragma unroll
                for (int t = 0; t < 8; ++t) {
                    const float rh = (e2m1_decode((word >> (4 * t)) & 15u) * sh) * g;
                    o[t] = (cv[t] + rh) * n;
                }
                store8(H_hat + orow * d + 8 * ch, o);
            }
        }
        if (Kc) {
            const uint4* src = reinterpret_cast<const uint4*>(Kc + row * KV);
            uint4* dst = reinterpret_cast<uint4*>(K_out + orow * KV);
            for (int i = threadIdx.x; i < kv16; i += 256) dst[i] = src[i];
        }
        if (Vc) {
            const uint4* src = reinterpret_cast<const uint4*>(Vc + row * KV);
            uint4* dst = reinterpret_cast<uint4*>(V_out + orow * KV);
            for (int i = threadIdx.x; i < kv16; i += 256) dst[i] = src[i];
        }
    }
}

template <typename T, int CPL>
void launch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                     uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int64_t rows = (int64_t)s->W * s->N;
    PS_LAUNCH("k_residual<T, CPL>", (k_residual<T, CPL>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st,
                       (const T*)H, rn, C, a, codes, bscale, rscale, rows, s->N, s->d, s->K);
}

template <typename T>
void dispatch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                       uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int cpl = (s->d / 8 + 63) / 64;
    if (cpl <= 1)      launch_residual<T, 1>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (cpl <= 2) launch_residual<T, 2>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (cpl <= 4) launch_residual<T, 4>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (cpl <= 8) launch_residual<T, 8>(s, H, rn, C, a, codes, bscale, rscale, st);
    else               launch_residual<T, 16>(s, H, rn, C, a, codes, bscale, rscale, st);
}

}  // namespace

extern "C" ps_status ps_residual_nvfp4(const ps_shape* s, ps_dtype dtype, const void* H,
                                       const float* row_norm, const float* C, const int32_t* assign,
                                       uint8_t* codes, uint8_t* bscale, float* rscale, void* stream)
{
    using namespace ps_host;
    if (!s || !H || !row_norm || !C || !assign || !codes || !bscale || !rscale) return PS_ERR_NULL;
    if (!dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = check_clusters(s);
    if (st != PS_OK) return st;
    if (s->d > 8192) return PS_ERR_SHAPE;
    if (!aligned16(H) || !aligned16(row_norm) || !aligned16(C) || !aligned16(assign) || !aligned16(codes) ||
        !aligned16(bscale) || !aligned16(rscale))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    if (dtype == PS_BF16) dispatch_residual<uint16_t>(s, H, row_norm, C, assign, codes, bscale, rscale, stm);
    else                  dispatch_residual<float>(s, H, row_norm, C, assign, codes, bscale, rscale, stm);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" ps_status ps_refresh_gather(const ps_shape* s, ps_dtype dtype, const int32_t* assign,
                                       const int32_t* idx, int32_t k, int32_t cap, int32_t* pos,
                                       int32_t* count, const uint8_t* codes, const uint8_t* bscale,
                                       const float* rscale, const float* C, const float* row_norm,
                                       void* H_hat, const void* Kc, const void* Vc, void* K_out,
                                       void* V_out, void* stream)
{
    using namespace ps_host;
    if (!s || !assign || !idx || !count || (!pos && cap > 0)) return PS_ERR_NULL;
    if (H_hat && (!codes || !bscale || !rscale || !C || !row_norm)) return PS_ERR_NULL;
    if ((Kc == nullptr) != (K_out == nullptr) || (Vc == nullptr) != (V_out == nullptr)) return PS_ERR_NULL;
    if (!dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = check_clusters(s);
    if (st != PS_OK) return st;
    if ((Kc || Vc) && (st = check_heads(s)) != PS_OK) return st;
    if (k < 1 || k > s->K || cap < 0) return PS_ERR_RANGE;
    if (!aligned16(assign) || !aligned16(idx) || !aligned16(count) || (pos && !aligned16(pos))) return PS_ERR_ALIGN;
    if (H_hat && (!aligned16(codes) || !aligned16(bscale) || !aligned16(rscale) || !aligned16(C) ||
                  !aligned16(row_norm) || !aligned16(H_hat)))
        return PS_ERR_ALIGN;
    if ((Kc && (!aligned16(Kc) || !aligned16(K_out))) || (Vc && (!aligned16(Vc) || !aligned16(V_out))))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    PS_LAUNCH("k_gather_select", k_gather_select, dim3(s->W), dim3(64), 0, stm, assign, idx, k, cap, pos, count, s->N, s->K);
    if (cap > 0 && (H_hat || Kc || Vc)) {
        const int64_t expect = ((int64_t)s->N * k + s->K - 1) / s->K;
        int G = (int)((expect + 3) / 4);
        if (G < 1) G = 1;
        if (G > cap) G = cap;
        const int KV = (Kc || Vc) ? s->Hkv * s->dh : 0;
        if (dtype == PS_BF16)
            PS_LAUNCH("k_gather_rows<uint16_t>", k_gather_rows<uint16_t>, dim3(G, s->W), dim3(256), 0, stm, pos, count, cap, assign,
                               codes, bscale, rscale, C, row_norm, (uint16_t*)H_hat, (const uint16_t*)Kc,
                               (const uint16_t*)Vc, (uint16_t*)K_out, (uint16_t*)V_out, s->N, s->d, s->K, KV);
        else
            PS_LAUNCH("k_gather_rows<float>", k_gather_rows<float>, dim3(G, s->W), dim3(256), 0, stm, pos, count, cap, assign,
                               codes, bscale, rscale, C, row_norm, (float*)H_hat, (const float*)Kc,
                               (const float*)Vc, (float*)K_out, (float*)V_out, s->N, s->d, s->K, KV);
    }
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}
