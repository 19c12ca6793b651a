// ps_nvfp4.hip -- NVFP4 residual coding of the window rows (Polestar
// technical summary 2.A, local window and clustering: residuals to the
// cluster centres are stored in NVFP4) and the refresh gather of the rows of
// the selected clusters (2.A, sparse updates; 2.C, only the selected clusters
// are fetched), for gfx950.
//
// Both kernels are bandwidth bound: one workgroup per row, 16-byte coalesced
// loads all issued before use, E4M3/E2M1 rounding in integer/fp32 arithmetic
// (every fp32 step is one correctly rounded operation, matching the stated
// convention bit for bit).
#include "ps_common.h"

using namespace ps;

namespace {

// Quotients on the fast path: for fp32 a and b, the fp32 rounding of
// a * RN64(1/b) equals the correctly rounded fp32 quotient a / b whenever that
// quotient is zero or at least 2^-125 in magnitude.  A quotient that is not an
// fp32 number lies at least 2^-49 (relative) from every fp32 rounding
// midpoint (with m a midpoint of 25 significant bits, a - m*b is a non-zero
// multiple of 2^(e_m + e_b - 47), since a has at most 24 significant bits),
// while the fp64 product is within 2^-52 of a / b.  Below the normal range the
// midpoints are coarser than that argument covers; such a row is redone with
// divisions (`exact`).  A quotient a / b is below 2^-125 exactly when
// 0 < |a| < 2^-125 * b, which is what the fast path tests.
//
// E2M1 rounding on the fast path uses gfx950's fp32 -> fp4 conversion with
// scale 1.0: checked exhaustively over every finite fp32 input, it returns the
// nearest-even, saturating E2M1 code of the convention except that a negative
// input rounding to zero comes back as -0 (nibble 0x8); `plus_zero` clears
// those signs.  Non-finite inputs are sent to the exact path.
__device__ __forceinline__ uint32_t plus_zero(uint32_t w)
{
    const uint32_t m = w & 0x77777777u;                              // magnitudes
    const uint32_t nz = (m | (m >> 1) | (m >> 2)) & 0x11111111u;     // magnitude != 0
    return m | (w & (nz << 3));
}

// NVFP4 coding of one row by one workgroup of TPR threads (one or four
// waves).  Thread i holds 8-element chunks i, i+TPR, ...; a 16-element block
// is the chunk pair (2m, 2m+1), i.e. threads i and i^1 of one wave.  All of a
// thread's loads are issued before any use.  With exact = false the quotients
// are fp64 products and E2M1 uses the hardware conversion; the function
// returns false without writing anything if any quotient of the row is tiny
// or any value is non-finite (decided by a workgroup vote).
template <typename T, int TPR, int CPL, bool exact>
__device__ __forceinline__ bool residual_row(const T* __restrict__ h, const float* __restrict__ c, float n,
                                             uint8_t* __restrict__ cr, uint8_t* __restrict__ br,
                                             float* __restrict__ rs, int d, float* red)
{
    constexpr int NW = TPR / 64;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int nch = d >> 3;
    const bool full = nch == TPR * CPL;          // every chunk of every thread is in the row
    const bool pos_n = n > 0.0f;                 // row-uniform
    const double inv_n = pos_n ? 1.0 / (double)n : 0.0;
    const float t1 = n * 0x1p-125f;              // |h| below this: tiny quotient
    bool bad = false;
    // chunks past the row read the last chunk again (always in bounds) and
    // are masked to zero; bf16 chunks stay packed until used
    constexpr bool packed = sizeof(T) == 2;
    uint4 hq[CPL][packed ? 1 : 2];
    float r[CPL][8];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = min(tid + TPR * i, nch - 1);
        const uint4* hp = reinterpret_cast<const uint4*>(h + 8 * ch);
        hq[i][0] = hp[0];
        if (!packed) hq[i][packed ? 0 : 1] = hp[1];
        load8(c + 8 * ch, r[i]);
    }
    float A = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const bool valid = full || tid + TPR * i < nch;
        float hv[8];
        if (packed) {
            const uint32_t w4[4] = {hq[i][0].x, hq[i][0].y, hq[i][0].z, hq[i][0].w};
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                hv[2 * t] = __uint_as_float(w4[t] << 16);
                hv[2 * t + 1] = __uint_as_float(w4[t] & 0xffff0000u);
            }
        } else {
            const uint4 a = hq[i][0], b = hq[i][packed ? 0 : 1];
            const uint32_t w8[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int t = 0; t < 8; ++t) hv[t] = __uint_as_float(w8[t]);
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            float x = 0.0f;
            if (pos_n) {
                if (exact) {
                    x = hv[t] / n;
                } else {
                    x = (float)((double)hv[t] * inv_n);
                    bad |= (fabsf(hv[t]) < t1) & (hv[t] != 0.0f);
                }
            }
            r[i][t] = valid ? x - r[i][t] : 0.0f;
            A = fmaxf(A, fabsf(r[i][t]));
        }
    }
    A = wave_max(A);
    if (NW > 1) {
        if ((tid & 63) == 0) red[wave] = A;
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NW; ++q) A = fmaxf(A, red[q]);
    }
    const bool zero_row = !(A > 0.0f);
    const float g = A / 2688.0f;
    uint32_t words[CPL], scales[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        float Ab = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) Ab = fmaxf(Ab, fabsf(r[i][t]));
        Ab = fmaxf(Ab, __shfl_xor(Ab, 1, 64));
        uint32_t word = 0, sb = 0;
        if (!zero_row) {
            sb = e4m3_encode((Ab / 6.0f) / g);
            const float eff = e4m3_decode(sb) * g;
            if (eff != 0.0f) {
                if (exact) {
#pragma unroll
                    for (int t = 0; t < 8; ++t) word |= e2m1_encode(r[i][t] / eff) << (4 * t);
                } else {
                    const double inv_eff = 1.0 / (double)eff;
                    const float t2 = eff * 0x1p-125f, big = eff * 8.0f;
                    float v[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float a = fabsf(r[i][t]);
                        bad |= ((a < t2) & (r[i][t] != 0.0f)) | !(a <= big);
                        v[t] = (float)((double)r[i][t] * inv_eff);
                    }
                    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[0], v[1], 1.0f, 0);
                    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[2], v[3], 1.0f, 1);
                    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[4], v[5], 1.0f, 2);
                    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, v[6], v[7], 1.0f, 3);
                    word = plus_zero(word);
                }
            }
        }
        words[i] = word;
        scales[i] = sb;
    }
    if (!exact) {
        const bool any_bad = NW > 1 ? __syncthreads_or(bad) != 0 : __any(bad) != 0;
        if (any_bad) return false;
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = tid + TPR * i;
        if (ch < nch) {
            *reinterpret_cast<uint32_t*>(cr + 4 * ch) = words[i];
            if (!(ch & 1)) br[ch >> 1] = (uint8_t)scales[i];
        }
    }
    if (tid == 0) *rs = zero_row ? 0.0f : g;
    return true;
}

// One workgroup per row; consecutive rows (one window's, sharing its centres)
// stay on one XCD.
template <typename T, int TPR, int CPL>
__global__ __launch_bounds__(TPR) void k_residual(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                   const float* __restrict__ C, const int32_t* __restrict__ assign,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                   float* __restrict__ rscale, int N, int d, int K)
{
    __shared__ float red[TPR / 64];
    const int64_t row = xcd_remap(blockIdx.x, gridDim.x);
    const int w = (int)(row / N);
    int a = assign[row];
    if (a < 0 || a >= K) a = 0;
    const float* c = C + ((size_t)w * K + a) * d;
    const T* h = H + (size_t)row * d;
    uint8_t* cr = codes + (size_t)row * (d >> 1);
    uint8_t* br = bscale + (size_t)row * (d >> 4);
    const float n = row_norm[row];
    if (!residual_row<T, TPR, CPL, false>(h, c, n, cr, br, rscale + row, d, red)) {
        __syncthreads();  // red[] is reused
        residual_row<T, TPR, CPL, true>(h, c, n, cr, br, rscale + row, d, red);
    }
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

template <typename T, int TPR, int CPL>
void launch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                     uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int64_t rows = (int64_t)s->W * s->N;
    PS_LAUNCH("k_residual<T, TPR, CPL>", (k_residual<T, TPR, CPL>), dim3((unsigned)rows), dim3(TPR), 0, st,
              (const T*)H, rn, C, a, codes, bscale, rscale, s->N, s->d, s->K);
}

// rows of at most 512 elements: one wave per row; longer rows: four waves
template <typename T>
void dispatch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                       uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int nch = s->d / 8;
    if (nch <= 64)        launch_residual<T, 64, 1>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (nch <= 256)  launch_residual<T, 256, 1>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (nch <= 512)  launch_residual<T, 256, 2>(s, H, rn, C, a, codes, bscale, rscale, st);
    else                  launch_residual<T, 256, 4>(s, H, rn, C, a, codes, bscale, rscale, st);
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

namespace {

// The address a kernel uses for a buffer it reads: device memory as it is,
// pinned host memory through the device mapping of its allocation; anything
// else (pageable host memory, unknown addresses) is refused before a launch.
ps_status device_view(const void* p, const void** out)
{
    hipPointerAttribute_t a{};
    if (hipPointerGetAttributes(&a, p) != hipSuccess) {
        (void)hipGetLastError();
        return PS_ERR_MEMORY;
    }
    if (a.type == hipMemoryTypeDevice || a.type == hipMemoryTypeManaged) {
        *out = p;
        return PS_OK;
    }
    if (a.type == hipMemoryTypeHost && a.devicePointer) {
        *out = a.devicePointer;
        return PS_OK;
    }
    return PS_ERR_MEMORY;
}

}  // namespace

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
    if (H_hat && cap > 0) {
        const void *c = nullptr, *b = nullptr, *r = nullptr;
        if ((st = device_view(codes, &c)) != PS_OK || (st = device_view(bscale, &b)) != PS_OK ||
            (st = device_view(rscale, &r)) != PS_OK)
            return st;
        codes = (const uint8_t*)c;
        bscale = (const uint8_t*)b;
        rscale = (const float*)r;
    }
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
