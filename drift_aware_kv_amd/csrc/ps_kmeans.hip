// ps_kmeans.hip -- spherical K-Means of the local window's hidden states and
// the centroid keys (Polestar technical summary 2.A, local window and
// clustering; sparse updates), for gfx950.
//
// One Lloyd iteration over all W windows is three launches:
//   assign  bf16 MFMA (16x16x32) scores of token tiles against every centre,
//           argmax in registers.  The first iteration of a call also writes
//           the fp64 row norms; later ones mark the clusters whose member set
//           changed.  The operand is the bf16 copy of the centres, made once
//           per call and then kept by the update.
//   bucket  stable counting sort of each window's rows by cluster (wave
//           ballots), giving every cluster its ascending member list.
//   update  one workgroup per (window, cluster): fp64 fused multiply-add of
//           the member rows scaled by 1/n_j in ascending order, fp64 norm,
//           fp32 centre plus its bf16 copy for the next assignment; after the
//           first iteration only clusters whose member set changed run.
// After the last iteration the keys kernel averages the member key rows.
// The fit-and-code call (ps_kmeans_fit_nvfp4) replaces the first update by
// one that also codes every cluster's member rows in NVFP4 right after
// rebuilding its centre; later updates mark the clusters they rebuild, and
// those clusters' rows are coded again after the last iteration.
#include "ps_common.h"
#include "ps_nvfp4_row.h"

#include <math.h>

#include <mutex>

using namespace ps;

// Tile shape of the assignment kernel: 16-token blocks per wave for K <= 64
// and for larger K, and the d-width of one LDS stage (multiple of 32).
#ifndef PS_ASSIGN_NB_SMALLK
#define PS_ASSIGN_NB_SMALLK 4
#endif
#ifndef PS_ASSIGN_NB_LARGEK
#define PS_ASSIGN_NB_LARGEK 2
#endif
#ifndef PS_ASSIGN_DK
#define PS_ASSIGN_DK 64
#endif


namespace {

// ---------------------------------------------------------------------------
// seeding
// ---------------------------------------------------------------------------

// c_k = x_{floor(kN/K)} = h / n (fp32 division), n from an fp64 sum of squares
template <typename T>
__global__ __launch_bounds__(256) void k_init_strided(const T* __restrict__ H, float* __restrict__ C,
                                                       int N, int d, int K)
{
    const int w = blockIdx.y, k = blockIdx.x;
    const int j = (int)(((int64_t)k * N) / K);
    const T* h = H + ((size_t)w * N + j) * d;
    __shared__ double red[4];
    double ss = 0.0;
    for (int e = threadIdx.x; e < d; e += 256) {
        double v = (double)Elem<T>::get(h, e);
        ss = fma(v, v, ss);
    }
    ss = wave_sum_d(ss);
    if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const float n = (float)sqrt(red[0] + red[1] + red[2] + red[3]);
    float* c = C + ((size_t)w * K + k) * d;
    for (int e = threadIdx.x; e < d; e += 256) {
        float v = Elem<T>::get(h, e);
        c[e] = n > 0.0f ? v / n : 0.0f;
    }
}

// Farthest-first traversal under cosine similarity, one workgroup per window:
// c_0 = x_0; then the non-zero row least similar to all chosen centres.
// m (the running best similarity) and the norms live in the workspace.
template <typename T>
__global__ __launch_bounds__(256) void k_init_farthest(const T* __restrict__ H, float* __restrict__ C,
                                                        double* __restrict__ mbuf,
                                                        float* __restrict__ nbuf, int N, int d, int K)
{
    extern __shared__ float cdyn[];  // the current centre, d floats
    __shared__ double redv[4];
    __shared__ int redi[4];
    const int w = blockIdx.x, wave = threadIdx.x >> 6, lane = lane_id();
    const T* Hw = H + (size_t)w * N * d;
    double* m = mbuf + (size_t)w * N;
    float* nrm = nbuf + (size_t)w * N;
    for (int j = wave; j < N; j += 4) {
        double ss = 0.0;
        for (int e = lane; e < d; e += 64) {
            double v = (double)Elem<T>::get(Hw, (size_t)j * d + e);
            ss = fma(v, v, ss);
        }
        ss = wave_sum_d(ss);
        if (lane == 0) nrm[j] = (float)sqrt(ss);
    }
    __threadfence_block();
    __syncthreads();
    int seed = 0;
    for (int k = 0; k < K; ++k) {
        if (k > 0) {
            double bv = 0.0;
            int bi = -1;
            for (int j = threadIdx.x; j < N; j += 256) {
                if (!(nrm[j] > 0.0f)) continue;
                if (bi < 0 || m[j] < bv) { bv = m[j]; bi = j; }
            }
#pragma unroll
            for (int s = 32; s >= 1; s >>= 1) {
                double ov = __shfl_xor(bv, s, 64);
                int oi = __shfl_xor(bi, s, 64);
                if (oi >= 0 && (bi < 0 || ov < bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
            }
            if (lane == 0) { redv[wave] = bv; redi[wave] = bi; }
            __syncthreads();
            bv = redv[0];
            bi = redi[0];
            for (int q = 1; q < 4; ++q) {
                int oi = redi[q];
                double ov = redv[q];
                if (oi >= 0 && (bi < 0 || ov < bv || (ov == bv && oi < bi))) { bv = ov; bi = oi; }
            }
            seed = bi < 0 ? 0 : bi;
            __syncthreads();
        }
        const float ns = nrm[seed];
        for (int e = threadIdx.x; e < d; e += 256) {
            float v = Elem<T>::get(Hw, (size_t)seed * d + e);
            float x = ns > 0.0f ? v / ns : 0.0f;
            cdyn[e] = x;
            C[((size_t)w * K + k) * d + e] = x;
        }
        __syncthreads();
        for (int j = wave; j < N; j += 4) {
            const float nj = nrm[j];
            double dot = 0.0;
            for (int e = lane; e < d; e += 64) {
                float v = Elem<T>::get(Hw, (size_t)j * d + e);
                float x = nj > 0.0f ? v / nj : 0.0f;
                dot = fma((double)x, (double)cdyn[e], dot);
            }
            dot = wave_sum_d(dot);
            if (lane == 0 && (k == 0 || dot > m[j])) m[j] = dot;
        }
        __threadfence_block();
        __syncthreads();
    }
}

// bf16 copy of the incoming centres (the first assignment's operand): eight
// elements per thread, two 16-byte loads and one 16-byte store
__global__ __launch_bounds__(256) void k_centres_to_bf16(const float* __restrict__ C,
                                                          uint16_t* __restrict__ Cb, size_t n8)
{
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n8; i += (size_t)gridDim.x * 256) {
        float v[8];
        load8(C + 8 * i, v);
        store8(Cb + 8 * i, v);
    }
}

// ---------------------------------------------------------------------------
// assignment, bf16: scores D[cluster][token] = Cb . H^T on MFMA 16x16x32
// ---------------------------------------------------------------------------
// Workgroup = 4 waves; a wave owns NB 16-token blocks (16*NB tokens); the M
// dimension runs over up to 16*KB clusters per pass (more passes when
// K > 16*KB).  MFMA operand layout (16x16x32 bf16): lane l supplies
// row/column (l % 16) and reduction elements 8*(l/16)..+8; the result element
// r of lane l is D[4*(l/16) + r][l % 16].  Centres are staged through LDS in
// 64-wide d-chunks (double-buffered, padded rows: conflict-free 16-byte
// reads); each wave streams its token rows straight into registers one chunk
// ahead (NB*2 16-byte loads per lane per chunk, each load covering 16 rows x
// 64 contiguous bytes).  FIRST: the first iteration of a call, which also
// writes the fp64 row norms and marks nothing; later iterations mark the old
// and new cluster of every row that moves and skip windows at a fixed point.
// F32C: `Cop` is the caller's fp32 centres, each staged piece rounded to bf16
// on its way to LDS (the same rounding as the stored copy, which the first
// update then writes for every cluster); otherwise `Cop` is that bf16 copy.
template <int KB, int NB, bool FIRST, bool F32C>
__global__ __launch_bounds__(256) void k_assign_bf16(const uint16_t* __restrict__ H,
                                                      const void* __restrict__ Cop,
                                                      int32_t* __restrict__ assign,
                                                      float* __restrict__ row_norm, int N, int d,
                                                      int K, int tiles, int nblocks,
                                                      int32_t* __restrict__ dirty,
                                                      const int32_t* __restrict__ conv, int* __restrict__ work)
{
    constexpr int DK = PS_ASSIGN_DK;       // d elements per LDS stage
    constexpr int NS = DK / 32;            // MFMA k-steps per stage
    constexpr int ROWB = DK * 2 + 16;      // padded LDS row stride (bytes)
    constexpr int MROWS = 16 * KB;
    constexpr int NPIECE = MROWS * (DK / 8);        // 16-byte pieces per stage
    constexpr int PIECES = (NPIECE + 255) / 256;    // per thread
    constexpr int TPW = 16 * NB;                    // tokens per wave
    __shared__ __attribute__((aligned(16))) uint8_t lds[2][MROWS * ROWB];

    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / tiles, tile = L - w * tiles;
    if (!FIRST && conv[w]) return;  // window at a fixed point: nothing can change
    if (work && threadIdx.x == 0) atomicAdd(work, 1);   // kernel timer: one tile processed
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const uint16_t* Hw = H + (size_t)w * N * d;
    const uint16_t* Cw = reinterpret_cast<const uint16_t*>(Cop) + (size_t)w * K * d;    // later passes
    const float* Cf = reinterpret_cast<const float*>(Cop) + (size_t)w * K * d;          // first pass

    int tok[NB];
    bool tv[NB];
    const uint16_t* hrow[NB];   // the token's row, clamped into the window
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
        tok[nb] = tile * 4 * TPW + wave * TPW + nb * 16 + r16;
        tv[nb] = tok[nb] < N;
        hrow[nb] = Hw + (size_t)min(tok[nb], N - 1) * d;
    }
    float bestv[NB];
    int besti[NB];
    double ss[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) { bestv[nb] = -INFINITY; besti[nb] = 0; ss[nb] = 0.0; }
    const int nchunks = (d + DK - 1) / DK;

    for (int cg = 0; cg < K; cg += MROWS) {
        const bool norm_pass = FIRST && cg == 0;
        floatx4 acc[KB][NB];
#pragma unroll
        for (int mb = 0; mb < KB; ++mb)
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};

        // Every load is issued unconditionally, its address clamped into the
        // window (row N - 1 or K - 1, column d - 8); pieces outside are zeroed
        // where they are used.  So no load sits behind a branch, and the wait
        // before a chunk's MFMAs covers that chunk's loads only, not the next
        // chunk's, which stay in flight.
        uint4 cpre[PIECES];
        float4 cpre32[F32C ? PIECES : 1][2];
        uint4 hcur[NB][NS], hnext[NB][NS];
        auto load_c = [&](int c0) {
#pragma unroll
            for (int p = 0; p < PIECES; ++p) {
                const int piece = min(p * 256 + (int)threadIdx.x, NPIECE - 1);
                const int row = piece / (DK / 8), col = (piece % (DK / 8)) * 8;
                const size_t off = (size_t)min(cg + row, K - 1) * d + min(c0 + col, d - 8);
                if (F32C) {
                    cpre32[F32C ? p : 0][0] = *reinterpret_cast<const float4*>(Cf + off);
                    cpre32[F32C ? p : 0][1] = *reinterpret_cast<const float4*>(Cf + off + 4);
                } else {
                    cpre[p] = *reinterpret_cast<const uint4*>(Cw + off);
                }
            }
        };
        auto store_c = [&](int buf, int c0) {
#pragma unroll
            for (int p = 0; p < PIECES; ++p) {
                const int piece = p * 256 + threadIdx.x;
                const int row = piece / (DK / 8), col = (piece % (DK / 8)) * 8;
                const bool ok = cg + row < K && c0 + col < d;
                if (F32C) {
                    const float4 a = cpre32[F32C ? p : 0][0], b = cpre32[F32C ? p : 0][1];
                    cpre[p] = make_uint4(f32_to_bf16(a.x) | (f32_to_bf16(a.y) << 16),
                                         f32_to_bf16(a.z) | (f32_to_bf16(a.w) << 16),
                                         f32_to_bf16(b.x) | (f32_to_bf16(b.y) << 16),
                                         f32_to_bf16(b.z) | (f32_to_bf16(b.w) << 16));
                }
                if (piece < NPIECE)
                    *reinterpret_cast<uint4*>(&lds[buf][row * ROWB + col * 2]) = ok ? cpre[p] : make_uint4(0, 0, 0, 0);
            }
        };
        auto load_h = [&](int c0, uint4 (&hr)[NB][NS]) {
#pragma unroll
            for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                for (int s = 0; s < NS; ++s)
                    hr[nb][s] = *reinterpret_cast<const uint4*>(hrow[nb] + min(c0 + 32 * s + 8 * q, d - 8));
        };

        load_c(0);
        load_h(0, hcur);
        store_c(0, 0);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const bool more = c + 1 < nchunks;
            if (more) {
                load_c((c + 1) * DK);
                load_h((c + 1) * DK, hnext);
            }
            const uint8_t* buf = lds[c & 1];
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                const bool in_d = c * DK + 32 * s + 8 * q < d;
                uint4 hv[NB];
#pragma unroll
                for (int nb = 0; nb < NB; ++nb) hv[nb] = (tv[nb] && in_d) ? hcur[nb][s] : make_uint4(0, 0, 0, 0);
                if (norm_pass) {
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb) {
                        const uint32_t wv[4] = {hv[nb].x, hv[nb].y, hv[nb].z, hv[nb].w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const double lo = (double)__uint_as_float(wv[i] << 16);
                            const double hi = (double)__uint_as_float(wv[i] & 0xffff0000u);
                            ss[nb] = fma(lo, lo, ss[nb]);
                            ss[nb] = fma(hi, hi, ss[nb]);
                        }
                    }
                }
                // one LDS read of a centre fragment feeds NB MFMAs
#pragma unroll
                for (int mb = 0; mb < KB; ++mb) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8*>(buf + (16 * mb + r16) * ROWB + 64 * s + 16 * q);
#pragma unroll
                    for (int nb = 0; nb < NB; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            a, __builtin_bit_cast(bf16x8, hv[nb]), acc[mb][nb], 0, 0, 0);
                }
            }
            if (more) store_c((c + 1) & 1, (c + 1) * DK);
            __syncthreads();
            if (more) {
#pragma unroll
                for (int nb = 0; nb < NB; ++nb)
#pragma unroll
                    for (int s = 0; s < NS; ++s) hcur[nb][s] = hnext[nb][s];
            }
        }
        // merge this cluster group's scores into the running argmax (ascending
        // cluster order within a lane; strict > keeps the lowest index)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cl = cg + 16 * mb + 4 * q + r;
                    const float v = acc[mb][nb][r];
                    if (cl < K && v > bestv[nb]) { bestv[nb] = v; besti[nb] = cl; }
                }
    }
    // combine the four lanes (q = 0..3) that hold the same token
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            const float ov = __shfl_xor(bestv[nb], m, 64);
            const int oi = __shfl_xor(besti[nb], m, 64);
            if (ov > bestv[nb] || (ov == bestv[nb] && oi < besti[nb])) { bestv[nb] = ov; besti[nb] = oi; }
            if (FIRST) ss[nb] += shfl_xor_d(ss[nb], m);
        }
        if (q == 0 && tv[nb]) {
            int32_t* ap = assign + (size_t)w * N + tok[nb];
            if (FIRST) {
                row_norm[(size_t)w * N + tok[nb]] = (float)sqrt(ss[nb]);
            } else {
                // membership changed: both clusters must be recomputed
                const int old = *ap;
                if (old != besti[nb]) {
                    if (old >= 0 && old < K) dirty[(size_t)w * K + old] = 1;
                    dirty[(size_t)w * K + besti[nb]] = 1;
                }
            }
            *ap = besti[nb];
        }
    }
}

// ---------------------------------------------------------------------------
// assignment, bf16, K > 128: a 512-thread workgroup owns 256 tokens and runs
// over the clusters 256 at a time.  Wave v (0..7) computes clusters
// [64 * (v & 3), +64) of the group against tokens [128 * (v >> 2), +128) of
// the tile: 4 x 8 MFMA blocks of 16x16.  Both operands are staged through
// LDS in 64-wide d-chunks, each chunk loaded once for the eight waves
// (double-buffered, padded 144-byte rows); per chunk a wave reads 8 KB of
// centre and 16 KB of token fragments for 64 MFMAs.  Each score accumulates
// over d in the same ascending order as in the smaller kernel, so the
// scores, and the argmax, are identical.  The buffer-load kernel below runs
// the same tiles faster (no staging registers, deeper prefetch); this one
// serves d not a multiple of 64, or a device that refuses that kernel's
// 160 KB of LDS.
// ---------------------------------------------------------------------------
constexpr int kWideTok = 256;                  // tokens per workgroup
constexpr int kWideCl = 256;                   // clusters per pass
constexpr int kWideDK = 64;                    // d elements per chunk
constexpr int kWideRowB = kWideDK * 2 + 16;    // padded LDS row (bytes)
constexpr int kWideTile = 256 * kWideRowB;     // one operand tile
constexpr size_t kWideLds = 4 * (size_t)kWideTile;  // centre and token tiles, two buffers

template <bool FIRST>
__global__ __launch_bounds__(512) void k_assign_wide(const uint16_t* __restrict__ H,
                                                      const uint16_t* __restrict__ Cb,
                                                      int32_t* __restrict__ assign,
                                                      float* __restrict__ row_norm, int N, int d, int K,
                                                      int tiles, int nblocks, int32_t* __restrict__ dirty,
                                                      const int32_t* __restrict__ conv, int* __restrict__ work)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t wlds[];
    constexpr int NS = kWideDK / 32;
    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / tiles, tile = L - w * tiles;
    if (!FIRST && conv[w]) return;  // window at a fixed point: nothing can change
    if (work && threadIdx.x == 0) atomicAdd(work, 1);   // kernel timer: one tile processed
    const int tid = threadIdx.x, lane = lane_id(), v = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int cq = v & 3, th = v >> 2;
    const int tok0 = tile * kWideTok;
    const uint16_t* Hw = H + (size_t)w * N * d;
    const uint16_t* Cw = Cb + (size_t)w * K * d;
    const int nchunks = (d + kWideDK - 1) / kWideDK;

    // staging: thread t moves the 16-byte pieces t + 512 u (u < 4) of each
    // 256-row tile: row (t >> 3) + 64 u, columns 8 (t & 7) .. + 8
    const int srow = tid >> 3, scol = (tid & 7) * 8;
    double ss[4] = {0.0, 0.0, 0.0, 0.0};  // first pass: sums of squares of the 4 token rows

    float bestv[8];
    int besti[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) { bestv[nt] = -INFINITY; besti[nt] = 0; }

    for (int cg = 0; cg < K; cg += kWideCl) {
        const bool norm_pass = FIRST && cg == 0;
        floatx4 acc[4][8];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[mb][nt] = floatx4{0.f, 0.f, 0.f, 0.f};
        uint4 cpre[4], hpre[4];
        auto load = [&](int c0) {
            const int e = c0 + scol;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int row = srow + 64 * u;
                const int cl = cg + row, tk = tok0 + row;
                cpre[u] = (cl < K && e < d) ? *reinterpret_cast<const uint4*>(Cw + (size_t)cl * d + e)
                                            : make_uint4(0, 0, 0, 0);
                hpre[u] = (tk < N && e < d) ? *reinterpret_cast<const uint4*>(Hw + (size_t)tk * d + e)
                                            : make_uint4(0, 0, 0, 0);
            }
        };
        auto store = [&](int buf) {
            uint8_t* cbuf = wlds + (size_t)buf * 2 * kWideTile;
            uint8_t* hbuf = cbuf + kWideTile;
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int off = (srow + 64 * u) * kWideRowB + scol * 2;
                *reinterpret_cast<uint4*>(cbuf + off) = cpre[u];
                *reinterpret_cast<uint4*>(hbuf + off) = hpre[u];
                if (norm_pass) {
                    const uint32_t wv[4] = {hpre[u].x, hpre[u].y, hpre[u].z, hpre[u].w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const double lo = (double)__uint_as_float(wv[i] << 16);
                        const double hi = (double)__uint_as_float(wv[i] & 0xffff0000u);
                        ss[u] = fma(lo, lo, ss[u]);
                        ss[u] = fma(hi, hi, ss[u]);
                    }
                }
            }
        };
        load(0);
        store(0);
        __syncthreads();
        for (int c = 0; c < nchunks; ++c) {
            const bool more = c + 1 < nchunks;
            if (more) load((c + 1) * kWideDK);
            const uint8_t* cbuf = wlds + (size_t)(c & 1) * 2 * kWideTile;
            const uint8_t* hbuf = cbuf + kWideTile;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                bf16x8 a[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    a[mb] = *reinterpret_cast<const bf16x8*>(cbuf + (64 * cq + 16 * mb + r16) * kWideRowB +
                                                              64 * s + 16 * q);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(
                        hbuf + (128 * th + 16 * nt + r16) * kWideRowB + 64 * s + 16 * q);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        acc[mb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[mb][nt], 0, 0, 0);
                }
            }
            if (more) store((c + 1) & 1);
            __syncthreads();
        }
        // merge this group's scores (ascending cluster order within a lane;
        // strict > keeps the lowest index)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cl = cg + 64 * cq + 16 * mb + 4 * q + r;
                    const float sv = acc[mb][nt][r];
                    if (cl < K && sv > bestv[nt]) { bestv[nt] = sv; besti[nt] = cl; }
                }
    }
    // the four lanes (q) of a token, then the four cluster quarters (waves)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            const float ov = __shfl_xor(bestv[nt], m, 64);
            const int oi = __shfl_xor(besti[nt], m, 64);
            if (ov > bestv[nt] || (ov == bestv[nt] && oi < besti[nt])) { bestv[nt] = ov; besti[nt] = oi; }
        }
    float* bv = reinterpret_cast<float*>(wlds);             // [2][4][128]; the tiles are free now
    int* bi = reinterpret_cast<int*>(wlds + 4096);
    if (q == 0) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int t = (th * 4 + cq) * 128 + 16 * nt + r16;
            bv[t] = bestv[nt];
            bi[t] = besti[nt];
        }
    }
    if (FIRST) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int m = 1; m <= 4; m <<= 1) ss[u] += shfl_xor_d(ss[u], m);
    }
    __syncthreads();
    if (FIRST && (tid & 7) == 0) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int tk = tok0 + srow + 64 * u;
            if (tk < N) row_norm[(size_t)w * N + tk] = (float)sqrt(ss[u]);
        }
    }
    if (tid < kWideTok) {
        const int tk = tok0 + tid;
        if (tk < N) {
            const int h2 = tid >> 7, tt = tid & 127;
            float best = bv[(h2 * 4) * 128 + tt];
            int bidx = bi[(h2 * 4) * 128 + tt];
#pragma unroll
            for (int cqq = 1; cqq < 4; ++cqq) {
                const float ov = bv[(h2 * 4 + cqq) * 128 + tt];
                const int oi = bi[(h2 * 4 + cqq) * 128 + tt];
                if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
            }
            int32_t* ap = assign + (size_t)w * N + tk;
            if (!FIRST) {
                // membership changed: both clusters must be recomputed
                const int old = *ap;
                if (old != bidx) {
                    if (old >= 0 && old < K) dirty[(size_t)w * K + old] = 1;
                    dirty[(size_t)w * K + bidx] = 1;
                }
            }
            *ap = bidx;
        }
    }
}

// ---------------------------------------------------------------------------
// assignment, bf16, K > 128, d a multiple of 64: the tile kernel above with
// its operands brought in by buffer loads that write LDS directly (no staging
// registers).  Same tiles, wave layout and per-score accumulation order as
// k_assign_wide, so identical scores.  In the first pass of a call each
// thread also sums the squares of half a token row of every chunk (fp64, four
// partial sums), for the row norms.  Those reads of the token tile are written
// as inline assembly with their own wait: the compiler would otherwise make
// them wait for every buffer load still writing LDS (the later chunks), which
// is the prefetch this kernel is built on.
//
// A chunk is 64 d-elements: every row piece a load requests is a whole
// 128-byte line (a 32-element chunk reads half lines, and the per-CU load
// rate drops by about a third with it).  Tokens come from HBM and are kept two chunks ahead
// (three 32 KB token buffers), centres come from L2 and are kept one chunk
// ahead (two 32 KB centre buffers): 160 KB of LDS.  In chunk c's step, after
// the barrier, each wave issues the centres of chunk c + 1 and then the
// tokens of chunk c + 2, so before chunk c is read it waits until at most the
// (4 loads of the) tokens of chunk c + 1 are outstanding.
//
// Row r of a 256-row tile keeps its eight 16-byte pieces at slots
// p ^ ((r >> 1) & 7): the sixteen rows of one fragment read then fall on
// sixteen distinct 16-byte bank groups.  One buffer load of a wave writes
// 1 KB of LDS, lane l -> row 8 i + (l >> 3), slot l & 7, so the lane fetches
// the piece that belongs in that slot; each wave moves 32 rows of each tile
// per chunk.  Rows past K or N lie past the buffer descriptors' ranges and
// load as zeros.
// ---------------------------------------------------------------------------
// raw buffer descriptor over `bytes` bytes at p (gfx9 descriptor word 3):
// offsets at or past `bytes` read as zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t window_rsrc(const void* p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)bytes, 0x00020000);
}

constexpr int kDmaDK = 64;                            // d elements per chunk
constexpr int kDmaTile = 256 * 128;                   // one operand tile of one chunk (bytes)
constexpr int kDmaTokBufs = 3;
constexpr int kDmaCenBufs = 2;
constexpr size_t kDmaLds = (size_t)(kDmaTokBufs + kDmaCenBufs) * kDmaTile;   // 160 KB

// s_waitcnt with vmcnt <= n (n < 16), lgkmcnt 0, expcnt untouched (gfx9 encoding)
#define PS_WAIT_VM_LGKM0(n) __builtin_amdgcn_s_waitcnt((n) | (0x7 << 4))

template <bool FIRST>
__global__ __launch_bounds__(512) void k_assign_wide_dma(const uint16_t* __restrict__ H,
                                                          const uint16_t* __restrict__ Cb,
                                                          int32_t* __restrict__ assign,
                                                          float* __restrict__ row_norm, int N, int d, int K,
                                                          int tiles, int nblocks, int32_t* __restrict__ dirty,
                                                          const int32_t* __restrict__ conv, int* __restrict__ work)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t wlds[];
    uint8_t* const tbufs = wlds;                                  // [3][256 rows][128 B]
    uint8_t* const cbufs = wlds + kDmaTokBufs * kDmaTile;         // [2][256 rows][128 B]
    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / tiles, tile = L - w * tiles;
    if (!FIRST && conv[w]) return;  // window at a fixed point: nothing can change
    if (work && threadIdx.x == 0) atomicAdd(work, 1);   // kernel timer: one tile processed
    const int tid = threadIdx.x, lane = lane_id(), v = tid >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int cq = v & 3, th = v >> 2;
    const int tok0 = tile * 256;
    const uint32_t rowb = (uint32_t)d * 2u;
    const __amdgpu_buffer_rsrc_t hrs = window_rsrc(H + (size_t)w * N * d, (uint32_t)N * rowb);
    const __amdgpu_buffer_rsrc_t crs = window_rsrc(Cb + (size_t)w * K * d, (uint32_t)K * rowb);
    const int nchunks = d / kDmaDK;
    // first pass: this thread's half (pieces 4 nh .. 4 nh + 3) of token row nr
    const int nr = tid >> 1, nh = tid & 1, nsw = (nr >> 1) & 7;
    double ss[4] = {0.0, 0.0, 0.0, 0.0};
    // slots of this lane's fragment pieces: k-step ks reads piece 4 ks + q of
    // rows r16 (mod 16), and (r >> 1) & 7 = (r16 >> 1) & 7 for those rows
    const int sw = (r16 >> 1) & 7;
    const int slot0 = 16 * (q ^ sw), slot1 = 16 * ((4 + q) ^ sw);

    // the rows and pieces this lane loads: row 32 v + 8 i + (lane >> 3)
    uint32_t mrow[4], mpiece[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        mrow[i] = (uint32_t)(32 * v + 8 * i + (lane >> 3));
        mpiece[i] = 16u * (uint32_t)((lane & 7) ^ ((mrow[i] >> 1) & 7));
    }
    float bestv[8];
    int besti[8];
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) { bestv[nt] = -INFINITY; besti[nt] = 0; }

    for (int cg = 0; cg < K; cg += kWideCl) {
        uint32_t coff[4], hoff[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            coff[i] = ((uint32_t)cg + mrow[i]) * rowb + mpiece[i];
            hoff[i] = ((uint32_t)tok0 + mrow[i]) * rowb + mpiece[i];
        }
        auto issue_tok = [&](int c) {
            uint8_t* buf = tbufs + (size_t)(c % kDmaTokBufs) * kDmaTile + (size_t)v * 4096;
            const int so = c * kDmaDK * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    hrs, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, hoff[i], so, 0, 0);
        };
        auto issue_cen = [&](int c) {
            uint8_t* buf = cbufs + (size_t)(c & 1) * kDmaTile + (size_t)v * 4096;
            const int so = c * kDmaDK * 2;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    crs, (__attribute__((address_space(3))) void*)(buf + i * 1024), 16, coff[i], so, 0, 0);
        };
        floatx4 acc[4][8];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[mb][nt] = floatx4{0.f, 0.f, 0.f, 0.f};

        issue_tok(0);
        issue_cen(0);
        if (nchunks > 1) issue_tok(1);
        for (int c = 0; c < nchunks; ++c) {
            // chunk c's loads are done once at most the tokens of chunk c + 1
            // (issued after them) are outstanding
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            if (c + 1 < nchunks) PS_WAIT_VM_LGKM0(4);
            else                 PS_WAIT_VM_LGKM0(0);
            __builtin_amdgcn_s_barrier();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            // every wave is past chunk c - 1: its buffers take chunk c + 1's
            // centres and chunk c + 2's tokens
            if (c + 1 < nchunks) issue_cen(c + 1);
            if (c + 2 < nchunks) issue_tok(c + 2);
            const uint8_t* cb = cbufs + (size_t)(c & 1) * kDmaTile;
            const uint8_t* hb = tbufs + (size_t)(c % kDmaTokBufs) * kDmaTile;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                const int slot = ks ? slot1 : slot0;
                bf16x8 a[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    a[mb] = *reinterpret_cast<const bf16x8*>(cb + (64 * cq + 16 * mb + r16) * 128 + slot);
#pragma unroll
                for (int nt = 0; nt < 8; ++nt) {
                    const bf16x8 b = *reinterpret_cast<const bf16x8*>(hb + (128 * th + 16 * nt + r16) * 128 + slot);
#pragma unroll
                    for (int mb = 0; mb < 4; ++mb)
                        acc[mb][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[mb], b, acc[mb][nt], 0, 0, 0);
                }
            }
            if (FIRST && cg == 0) {
                // the four pieces of this thread's half row (chunk c is
                // complete in LDS: its loads were waited for before the
                // barrier, and later loads write other buffers)
                const uint32_t base = (uint32_t)(size_t)(const __attribute__((address_space(3))) uint8_t*)(hb + nr * 128);
                uint4 pv[4];
                asm volatile("ds_read_b128 %0, %4\n\t"
                             "ds_read_b128 %1, %5\n\t"
                             "ds_read_b128 %2, %6\n\t"
                             "ds_read_b128 %3, %7\n\t"
                             "s_waitcnt lgkmcnt(0)"
                             : "=&v"(pv[0]), "=&v"(pv[1]), "=&v"(pv[2]), "=&v"(pv[3])
                             : "v"(base + 16u * (uint32_t)((4 * nh + 0) ^ nsw)),
                               "v"(base + 16u * (uint32_t)((4 * nh + 1) ^ nsw)),
                               "v"(base + 16u * (uint32_t)((4 * nh + 2) ^ nsw)),
                               "v"(base + 16u * (uint32_t)((4 * nh + 3) ^ nsw))
                             : "memory");
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t wd[4] = {pv[j].x, pv[j].y, pv[j].z, pv[j].w};
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const double lo = (double)__uint_as_float(wd[t] << 16);
                        const double hi = (double)__uint_as_float(wd[t] & 0xffff0000u);
                        ss[t] = fma(lo, lo, ss[t]);
                        ss[t] = fma(hi, hi, ss[t]);
                    }
                }
            }
        }
        // every wave is done reading the buffers before they are refilled
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        PS_WAIT_VM_LGKM0(0);
        __builtin_amdgcn_s_barrier();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        // merge this group's scores (ascending cluster order within a lane;
        // strict > keeps the lowest index)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int cl = cg + 64 * cq + 16 * mb + 4 * q + r;
                    const float sv = acc[mb][nt][r];
                    if (cl < K && sv > bestv[nt]) { bestv[nt] = sv; besti[nt] = cl; }
                }
    }
    if (FIRST) {
        // the two halves of a row sit in adjacent lanes
        double t = (ss[0] + ss[1]) + (ss[2] + ss[3]);
        t += shfl_xor_d(t, 1);
        const int tk = tok0 + nr;
        if (nh == 0 && tk < N) row_norm[(size_t)w * N + tk] = (float)sqrt(t);
    }
    // the four lanes (q) of a token, then the four cluster quarters (waves)
#pragma unroll
    for (int nt = 0; nt < 8; ++nt)
#pragma unroll
        for (int m = 16; m <= 32; m <<= 1) {
            const float ov = __shfl_xor(bestv[nt], m, 64);
            const int oi = __shfl_xor(besti[nt], m, 64);
            if (ov > bestv[nt] || (ov == bestv[nt] && oi < besti[nt])) { bestv[nt] = ov; besti[nt] = oi; }
        }
    float* bv = reinterpret_cast<float*>(wlds);             // [2][4][128]; the buffers are free now
    int* bi = reinterpret_cast<int*>(wlds + 4096);
    if (q == 0) {
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) {
            const int t = (th * 4 + cq) * 128 + 16 * nt + r16;
            bv[t] = bestv[nt];
            bi[t] = besti[nt];
        }
    }
    __syncthreads();
    if (tid < 256) {
        const int tk = tok0 + tid;
        if (tk < N) {
            const int h2 = tid >> 7, tt = tid & 127;
            float best = bv[(h2 * 4) * 128 + tt];
            int bidx = bi[(h2 * 4) * 128 + tt];
#pragma unroll
            for (int cqq = 1; cqq < 4; ++cqq) {
                const float ov = bv[(h2 * 4 + cqq) * 128 + tt];
                const int oi = bi[(h2 * 4 + cqq) * 128 + tt];
                if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
            }
            int32_t* ap = assign + (size_t)w * N + tk;
            if (!FIRST) {
                // membership changed: both clusters must be recomputed
                const int old = *ap;
                if (old != bidx) {
                    if (old >= 0 && old < K) dirty[(size_t)w * K + old] = 1;
                    dirty[(size_t)w * K + bidx] = 1;
                }
            }
            *ap = bidx;
        }
    }
}

// assignment, fp32 path (exact centres): one thread per row
__global__ __launch_bounds__(256) void k_assign_f32(const float* __restrict__ H, const float* __restrict__ C,
                                                     int32_t* __restrict__ assign,
                                                     float* __restrict__ row_norm, int W, int N, int d,
                                                     int K, int first, int32_t* __restrict__ dirty,
                                                     const int32_t* __restrict__ conv, int* __restrict__ work)
{
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int w = (int)(min(row, (int64_t)W * N - 1) / N);
    const bool active = row < (int64_t)W * N && (first || !conv[w]);
    if (work) {   // kernel timer: rows processed
        const uint64_t b = __ballot(active);
        if (lane_id() == 0 && b) atomicAdd(work, __popcll(b));
    }
    if (!active) return;
    const float* h = H + (size_t)row * d;
    const float* Cw = C + (size_t)w * K * d;
    float bestv = -INFINITY;
    int besti = 0;
    for (int k = 0; k < K; ++k) {
        float s = 0.0f;
        for (int e = 0; e < d; ++e) s = fmaf(h[e], Cw[(size_t)k * d + e], s);
        if (s > bestv) { bestv = s; besti = k; }
    }
    if (!first) {
        const int old = assign[row];
        if (old != besti) {
            if (old >= 0 && old < K) dirty[(size_t)w * K + old] = 1;
            dirty[(size_t)w * K + besti] = 1;
        }
    }
    assign[row] = besti;
    if (first) {
        double ss = 0.0;
        for (int e = 0; e < d; ++e) ss = fma((double)h[e], (double)h[e], ss);
        row_norm[row] = (float)sqrt(ss);
    }
}

// ---------------------------------------------------------------------------
// bucket: stable counting sort of rows by cluster, one 8-wave workgroup per
// window.  Wave v owns the v-th of eight consecutive row ranges: it counts its
// rows per cluster into its own LDS histogram; the cluster offsets are the
// prefix over clusters of the totals, and wave v's first slot in cluster c is
// offs[c] plus the counts of waves 0..v-1 in c; then each wave writes its rows
// in ascending order (lanes of one cluster ranked by a match-any ballot).  So
// every cluster lists its members in ascending row order, as a sequential
// sort would.  After the first iteration, a window none of whose clusters
// changed keeps its member lists (they are a function of the unchanged
// assignment) and, unless every pass is to run in full, is marked converged,
// which makes every later assignment pass of that window a no-op (the
// iteration would reproduce exactly the same centres and assignments).
// ---------------------------------------------------------------------------
constexpr int kBucketWaves = 8;

__global__ __launch_bounds__(64 * kBucketWaves) void k_bucket(const int32_t* __restrict__ assign,
                                                               int32_t* __restrict__ perm,
                                                               int32_t* __restrict__ offs,
                                                               const int32_t* __restrict__ dirty,
                                                               int32_t* __restrict__ conv, int N, int K, int first,
                                                               int fixed_point_exit, int32_t* __restrict__ listed)
{
    constexpr int NW = kBucketWaves;
    __shared__ int cnt[NW][kMaxK];
    const int w = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    if (first) {
        if (tid == 0) conv[w] = 0;
        if (listed && w == 0 && tid == 0) *listed = 0;   // rows listed by the coding update
    } else {
        if (conv[w]) return;
        bool any = false;
        for (int k = tid; k < K; k += 64 * NW) any |= dirty[(size_t)w * K + k] != 0;
        if (!__syncthreads_or(any)) {
            if (fixed_point_exit && tid == 0) conv[w] = 1;
            return;
        }
    }
    const int32_t* a = assign + (size_t)w * N;
    const int seg = (N + 64 * NW - 1) / (64 * NW) * 64;
    const int j0 = min(wave * seg, N), j1 = min(j0 + seg, N);
    for (int k = lane; k < K; k += 64) cnt[wave][k] = 0;
    __syncthreads();
    for (int j = j0 + lane; j < j1; j += 64) {
        int c = a[j];
        c = (c < 0 || c >= K) ? 0 : c;
        atomicAdd(&cnt[wave][c], 1);
    }
    __syncthreads();
    if (wave == 0) {
        int running = 0;
        for (int base = 0; base < K; base += 64) {
            const int k = base + lane;
            int v = 0;
            if (k < K)
                for (int u = 0; u < NW; ++u) v += cnt[u][k];
            int incl = v;
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const int o = __shfl_up(incl, s, 64);
                if (lane >= s) incl += o;
            }
            const int excl = running + incl - v;
            if (k < K) {
                offs[(size_t)w * (K + 1) + k] = excl;
                int start = excl;
                for (int u = 0; u < NW; ++u) {
                    const int t = cnt[u][k];
                    cnt[u][k] = start;
                    start += t;
                }
            }
            running += __shfl(incl, 63, 64);
        }
        if (lane == 0) offs[(size_t)w * (K + 1) + K] = running;
    }
    __syncthreads();
    const int nbits = K > 1 ? 32 - __clz(K - 1) : 0;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int* cur = cnt[wave];
    for (int base = j0; base < j1; base += 64) {
        const int j = base + lane;
        const bool valid = j < j1;
        int c = valid ? a[j] : 0;
        c = (c < 0 || c >= K) ? 0 : c;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            const uint64_t bb = __ballot(valid && ((c >> b) & 1));
            peers &= ((c >> b) & 1) ? bb : ~bb;
        }
        int rank = 0, total = 0, start = 0;
        if (valid) {
            rank = __popcll(peers & lt);
            total = __popcll(peers);
            start = cur[c];
        }
        // every lane has read its cluster's start before the last of its
        // peers moves it (the wave's LDS accesses complete in order)
        __builtin_amdgcn_wave_barrier();
        if (valid) {
            perm[(size_t)w * N + start + rank] = j;
            if (rank == total - 1) cur[c] = start + total;
        }
        __builtin_amdgcn_wave_barrier();
    }
}

// ---------------------------------------------------------------------------
// ordered member sums (update and keys): a batch of up to 256 members of one
// cluster is staged in LDS (row ids and weights, in ascending member order),
// then every thread sums its 8 * CH elements [e0 + 8 (t + 256 c), + 8) over
// the batch in that order, in fp64.  Two members' rows are requested while
// the previous two are added; every load is issued unconditionally (past the
// batch: the last member again, past the row: its last 8 elements, neither
// added), so each wait covers exactly the rows it needs.
// ---------------------------------------------------------------------------
template <typename T, int CH, bool WEIGHTED, int CACHE = 0>
__device__ __forceinline__ void member_sums(const T* __restrict__ rows, int rowlen, int e0,
                                            const int* mid, const double* mw, int nv, double (&acc)[CH][8],
                                            uint16_t* cache = nullptr)
{
    if (nv <= 0) return;
    int off[CH];
    bool in_row[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = e0 + (int)(threadIdx.x + 256 * c) * 8;
        in_row[c] = e < rowlen;
        off[c] = min(e, rowlen - 8);
    }
    float A[2][CH][8], B[2][CH][8];
    auto load = [&](int m, float (&X)[2][CH][8]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const T* r = rows + (size_t)mid[min(m + u, nv - 1)] * rowlen;
#pragma unroll
            for (int c = 0; c < CH; ++c) load8(r + off[c], X[u][c]);
        }
    };
    auto add = [&](int m, const float (&X)[2][CH][8]) {
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            if (m + u >= nv) break;
            const double wt = WEIGHTED ? mw[m + u] : 1.0;
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (!in_row[c]) continue;   // past the row: the sums stay exact zeros
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    acc[c][i] = WEIGHTED ? fma((double)X[u][c][i], wt, acc[c][i]) : acc[c][i] + (double)X[u][c][i];
                if constexpr (CACHE > 0) {
                    // the first CACHE members' rows kept in LDS for a later pass: the
                    // upper halves of the fp32 values are the rows' bf16 bits
                    if (m + u < CACHE) {
                        uint4 q;
                        q.x = (__float_as_uint(X[u][c][0]) >> 16) | (__float_as_uint(X[u][c][1]) & 0xffff0000u);
                        q.y = (__float_as_uint(X[u][c][2]) >> 16) | (__float_as_uint(X[u][c][3]) & 0xffff0000u);
                        q.z = (__float_as_uint(X[u][c][4]) >> 16) | (__float_as_uint(X[u][c][5]) & 0xffff0000u);
                        q.w = (__float_as_uint(X[u][c][6]) >> 16) | (__float_as_uint(X[u][c][7]) & 0xffff0000u);
                        *reinterpret_cast<uint4*>(cache + (size_t)(m + u) * rowlen + off[c]) = q;
                    }
                }
            }
        }
    };
    load(0, A);
    for (int m = 0; m < nv; m += 4) {
        load(m + 2, B);
        add(m, A);
        load(m + 4, A);
        add(m + 2, B);
    }
}

// Stage members [b0, b0 + 256) of the ascending list pm[beg .. end) into LDS,
// keeping those `keep` accepts, in order; returns how many were kept.  The
// caller's previous batch must no longer be read (a barrier comes first).
template <typename Keep>
__device__ __forceinline__ int stage_members(const int32_t* __restrict__ pm, int b0, int end, int* mid,
                                             double* mw, int* wcnt, Keep keep)
{
    const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
    int j = 0;
    double wt = 0.0;
    bool ok = false;
    if (b0 + t < end) {
        j = pm[b0 + t];
        ok = keep(j, wt);
    }
    const uint64_t bal = __ballot(ok);
    __syncthreads();
    if (lane == 0) wcnt[wv] = __popcll(bal);
    __syncthreads();
    int pos = __popcll(bal & ((1ull << lane) - 1ull));
    for (int q = 0; q < wv; ++q) pos += wcnt[q];
    if (ok) {
        mid[pos] = j;
        mw[pos] = wt;
    }
    const int nv = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    __syncthreads();
    return nv;
}

// ---------------------------------------------------------------------------
// update: one workgroup per (window, cluster), or per `cpb` consecutive
// clusters of the batch when most clusters are expected unchanged (the
// updates after the first): fewer workgroups that exit at once
// ---------------------------------------------------------------------------
template <typename T, int CH>
__device__ __forceinline__ void update_cluster(const T* __restrict__ H, const float* __restrict__ row_norm,
                                               const int32_t* __restrict__ perm,
                                               const int32_t* __restrict__ offs, float* __restrict__ C,
                                               uint16_t* __restrict__ Cb, int32_t* __restrict__ counts,
                                               double* __restrict__ nrm_out, int32_t* __restrict__ dirty,
                                               int32_t* __restrict__ stale, int N, int d, int K, int w, int k,
                                               int all, int* __restrict__ work)
{
    __shared__ double red[4];
    // an unchanged member set gives a bit-identical sum: keep the centre
    if (!all && !dirty[(size_t)w * K + k]) return;
    if (work && threadIdx.x == 0) atomicAdd(work, 1);   // kernel timer: one cluster re-summed
    // a centre rebuilt after the update that coded the rows: its members are coded again
    if (stale && threadIdx.x == 0) stale[(size_t)w * K + k] = 1;
    const int beg = offs[(size_t)w * (K + 1) + k], end = offs[(size_t)w * (K + 1) + k + 1];
    const int32_t* pm = perm + (size_t)w * N;
    const T* Hw = H + (size_t)w * N * d;
    const float* rn = row_norm + (size_t)w * N;

    __shared__ int mid[256];
    __shared__ double mw[256];
    __shared__ int wcnt[4];
    double acc[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = 0.0;
    // members whose norm is not positive (zero, or a non-finite row) add nothing
    for (int b0 = beg; b0 < end; b0 += 256) {
        const int nv = stage_members(pm, b0, end, mid, mw, wcnt, [&](int j, double& wt) {
            const float n = rn[j];
            if (!(n > 0.0f)) return false;
            wt = 1.0 / (double)n;
            return true;
        });
        member_sums<T, CH, true>(Hw, d, 0, mid, mw, nv, acc);
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fma(acc[c][i], acc[c][i], ss);
    ss = wave_sum_d(ss);
    if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double nrm = sqrt(red[0] + red[1] + red[2] + red[3]);
    const int nk = end - beg;
    if (threadIdx.x == 0) {
        counts[(size_t)w * K + k] = nk;
        nrm_out[(size_t)w * K + k] = nrm;
        dirty[(size_t)w * K + k] = 0;
    }
    if (nk > 0 && nrm > 0.0) {
        float* c_out = C + ((size_t)w * K + k) * d;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int e = (threadIdx.x + 256 * c) * 8;
            if (e < d) {
                float v[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (float)(acc[c][i] / nrm);
                store8(c_out + e, v);
                if (Cb) store8(Cb + ((size_t)w * K + k) * d + e, v);
            }
        }
    } else if (all && Cb) {
        // a kept centre: its bf16 copy for the later passes (the first pass
        // read the fp32 centres directly)
        const float* c_in = C + ((size_t)w * K + k) * d;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int e = (threadIdx.x + 256 * c) * 8;
            if (e < d) {
                float v[8];
                load8(c_in + e, v);
                store8(Cb + ((size_t)w * K + k) * d + e, v);
            }
        }
    }
}

template <typename T, int CH>
__global__ __launch_bounds__(256) void k_update(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                 const int32_t* __restrict__ perm,
                                                 const int32_t* __restrict__ offs, float* __restrict__ C,
                                                 uint16_t* __restrict__ Cb, int32_t* __restrict__ counts,
                                                 double* __restrict__ nrm_out, int32_t* __restrict__ dirty,
                                                 int32_t* __restrict__ stale, int N, int d, int K, int nblocks,
                                                 int cpb, int nclusters, int all, int* __restrict__ work)
{
    const int Lg = xcd_remap(blockIdx.x, nblocks);
    const int g0 = Lg * cpb, lane = lane_id();
    // the workgroup's clusters to rebuild, one flag load per cluster, all at once (every wave
    // takes the same mask); cluster g of the batch is (g / K, g % K), its flag dirty[g]
    const bool todo = lane < cpb && g0 + lane < nclusters && (all || dirty[g0 + lane] != 0);
    const uint64_t mask = __ballot(todo);
    for (int i = 0; i < cpb; ++i) {
        if (!((mask >> i) & 1)) continue;        // workgroup-uniform
        __syncthreads();                         // the previous cluster's LDS reads are done
        const int g = g0 + i, w = g / K, k = g - w * K;
        update_cluster<T, CH>(H, row_norm, perm, offs, C, Cb, counts, nrm_out, dirty, stale, N, d, K, w, k, all,
                              work);
    }
}

// The member rows pm[beg .. end) of one cluster (rows of one window: Hw,
// rn, window row offset wrow) coded against the centre cs (LDS, fp32) by the
// workgroup's four waves, one row per wave at a time, with the coder's fast
// path; rows it declines are listed for the exact coder.
template <int BPL, bool FULL, int CACHE = 0>
__device__ __forceinline__ void code_members(const uint16_t* __restrict__ Hw, const float* __restrict__ rn,
                                             const int32_t* __restrict__ pm, int beg, int end, const float* cs,
                                             uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                             float* __restrict__ rscale, int32_t* __restrict__ list,
                                             int32_t* __restrict__ listed, size_t wrow, int d,
                                             const uint16_t* rc = nullptr, const int* rc_id = nullptr)
{
    const int lane = lane_id(), nb = d >> 4;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    for (int m = beg + wave; m < end; m += 4) {
        const int j = pm[m];
        const size_t row = wrow + j;
        uint4 hq[BPL][2];
        const int sl = m - beg;
        bool cached = false;
        if constexpr (CACHE > 0) cached = sl < CACHE && rc_id[sl] == j;   // wave-uniform
        if (cached) {                            // the row the update kept in LDS
#pragma unroll
            for (int b = 0; b < BPL; ++b) {
                const uint4* hp = reinterpret_cast<const uint4*>(rc + (size_t)sl * d + 16 * min(lane + 64 * b, nb - 1));
                hq[b][0] = hp[0];
                hq[b][1] = hp[1];
            }
        } else {
            load_hblocks<uint16_t, 64, BPL>(Hw + (size_t)j * d, lane, nb, hq);
        }
        // the centre's blocks from LDS for each row (registers stay free between rows)
        float cv[BPL][16];
#pragma unroll
        for (int b = 0; b < BPL; ++b) {
            const float4* cp = reinterpret_cast<const float4*>(cs + 16 * min(lane + 64 * b, nb - 1));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = cp[q];
                cv[b][4 * q] = v.x; cv[b][4 * q + 1] = v.y; cv[b][4 * q + 2] = v.z; cv[b][4 * q + 3] = v.w;
            }
        }
        if (!residual_row_fast<uint16_t, 1, BPL, FULL>(hq, cv, rn[j], codes + row * (size_t)(d >> 1),
                                                       bscale + row * (size_t)(d >> 4), rscale + row, d, nullptr)) {
            if (lane == 0) list[atomicAdd(listed, 1)] = (int32_t)row;
        }
    }
}

// member rows the coding update keeps in LDS between rebuilding the centre and
// coding them (8 KB each at 4096 elements; three workgroups still fit a CU)
constexpr int kCodeCache = 4;

// The first update of a call that also codes the residuals (bf16 rows of up
// to 4096 elements): each workgroup rebuilds its cluster's centre exactly as
// k_update does (every cluster, as in any first update), then its four waves
// code the cluster's member rows against that centre with the coder's fast
// path, one row per wave at a time, while the rows just summed are still in
// the caches.  Rows the fast path declines are listed for the exact coder.
// A later update that rebuilds a centre marks it `stale`; after the last
// iteration only those clusters' rows are coded again, so every row ends up
// coded against the final centre of its final cluster, as a separate coder
// call would code it.  Three workgroups per compute unit (168 registers).
template <int CH, int BPL, bool FULL>
__global__ __launch_bounds__(256, 3) void k_update_code(const uint16_t* __restrict__ H,
                                                        const float* __restrict__ row_norm,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offs, float* __restrict__ C,
                                                        uint16_t* __restrict__ Cb, int32_t* __restrict__ counts,
                                                        double* __restrict__ nrm_out, int32_t* __restrict__ dirty,
                                                        int32_t* __restrict__ stale, uint8_t* __restrict__ codes,
                                                        uint8_t* __restrict__ bscale, float* __restrict__ rscale,
                                                        int32_t* __restrict__ list, int32_t* __restrict__ listed,
                                                        int N, int d, int K, int nblocks)
{
    __shared__ double red[4];
    __shared__ int mid[256];
    __shared__ double mw[256];
    __shared__ int wcnt[4];
    __shared__ float cs[4096];                   // the centre, for the coding waves
    __shared__ __attribute__((aligned(16))) uint16_t rc[kCodeCache * 4096];   // the first members' rows
    __shared__ int rc_id[kCodeCache];
    const int Lg = xcd_remap(blockIdx.x, nblocks);
    const int w = Lg / K, k = Lg - w * K;
    const int beg = offs[(size_t)w * (K + 1) + k], end = offs[(size_t)w * (K + 1) + k + 1];
    const int32_t* pm = perm + (size_t)w * N;
    const uint16_t* Hw = H + (size_t)w * N * d;
    const float* rn = row_norm + (size_t)w * N;

    double acc[CH][8];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[c][i] = 0.0;
    for (int b0 = beg; b0 < end; b0 += 256) {
        const int nv = stage_members(pm, b0, end, mid, mw, wcnt, [&](int j, double& wt) {
            const float n = rn[j];
            if (!(n > 0.0f)) return false;
            wt = 1.0 / (double)n;
            return true;
        });
        if (b0 == beg) {
            // the first batch's first rows stay in LDS (their row ids beside them)
            if (threadIdx.x < kCodeCache) rc_id[threadIdx.x] = (int)threadIdx.x < nv ? mid[threadIdx.x] : -1;
            member_sums<uint16_t, CH, true, kCodeCache>(Hw, d, 0, mid, mw, nv, acc, rc);
        } else {
            member_sums<uint16_t, CH, true>(Hw, d, 0, mid, mw, nv, acc);
        }
    }
    double ss = 0.0;
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fma(acc[c][i], acc[c][i], ss);
    ss = wave_sum_d(ss);
    if (lane_id() == 0) red[threadIdx.x >> 6] = ss;
    __syncthreads();
    const double nrm = sqrt(red[0] + red[1] + red[2] + red[3]);
    const int nk = end - beg;
    if (threadIdx.x == 0) {
        counts[(size_t)w * K + k] = nk;
        nrm_out[(size_t)w * K + k] = nrm;
        dirty[(size_t)w * K + k] = 0;
        stale[(size_t)w * K + k] = 0;
    }
    const bool fresh = nk > 0 && nrm > 0.0;
    float* c_at = C + ((size_t)w * K + k) * d;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
        const int e = (threadIdx.x + 256 * c) * 8;
        if (e < d) {
            float v[8];
            if (fresh) {
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = (float)(acc[c][i] / nrm);
                store8(c_at + e, v);
            } else {
                load8(c_at + e, v);              // a kept centre
            }
            if (Cb) store8(Cb + ((size_t)w * K + k) * d + e, v);
            if (nk > 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i) cs[e + i] = v[i];
            }
        }
    }
    if (nk == 0) return;                         // workgroup-uniform
    __syncthreads();
    code_members<BPL, FULL, kCodeCache>(Hw, rn, pm, beg, end, cs, codes, bscale, rscale, list, listed,
                                        (size_t)w * N, d, rc, rc_id);
}

// Coding again after the last iteration: the rows of each cluster rebuilt
// after the coding update (stale), against its final centre in C; a
// workgroup takes `cpb` consecutive clusters and skips the unmarked ones.
template <int BPL, bool FULL>
__global__ __launch_bounds__(256, 3) void k_code_stale(const uint16_t* __restrict__ H,
                                                       const float* __restrict__ row_norm,
                                                       const int32_t* __restrict__ perm,
                                                       const int32_t* __restrict__ offs,
                                                       const float* __restrict__ C,
                                                       const int32_t* __restrict__ stale,
                                                       uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                       float* __restrict__ rscale, int32_t* __restrict__ list,
                                                       int32_t* __restrict__ listed, int N, int d, int K,
                                                       int nblocks, int cpb, int nclusters, int* __restrict__ work)
{
    __shared__ float cs[4096];
    const int Lg = xcd_remap(blockIdx.x, nblocks);
    const int g0 = Lg * cpb, lane = lane_id();
    // the workgroup's clusters to code, one flag load per cluster, all at once
    const bool todo = lane < cpb && g0 + lane < nclusters && stale[g0 + lane] != 0;
    const uint64_t mask = __ballot(todo);
    for (int i = 0; i < cpb; ++i) {
        if (!((mask >> i) & 1)) continue;        // workgroup-uniform
        const int g = g0 + i, w = g / K, k = g - w * K;
        const int beg = offs[(size_t)w * (K + 1) + k], end = offs[(size_t)w * (K + 1) + k + 1];
        if (end == beg) continue;
        if (work && threadIdx.x == 0) atomicAdd(work, 1);   // kernel timer: one cluster coded
        __syncthreads();                         // the previous cluster's coding no longer reads cs
        const float* c = C + ((size_t)w * K + k) * d;
        for (int e = 8 * (int)threadIdx.x; e < d; e += 8 * 256) {
            float v[8];
            load8(c + e, v);
#pragma unroll
            for (int q = 0; q < 8; ++q) cs[e + q] = v[q];
        }
        __syncthreads();
        code_members<BPL, FULL>(H + (size_t)w * N * d, row_norm + (size_t)w * N, perm + (size_t)w * N, beg, end,
                                cs, codes, bscale, rscale, list, listed, (size_t)w * N, d);
    }
}

// centroid keys: mean of the member key rows, fp64 in ascending member order,
// rounded to fp32 then dtype; each thread owns 16 elements of a 4096-element
// block of the key row, blocks in turn
template <typename T>
__global__ __launch_bounds__(256) void k_keys(const T* __restrict__ Kr, const int32_t* __restrict__ perm,
                                               const int32_t* __restrict__ offs, T* __restrict__ Ck,
                                               int N, int KV, int K, int nblocks)
{
    constexpr int CH = 2;
    const int Lg = xcd_remap(blockIdx.x, nblocks);
    const int w = Lg / K, k = Lg - w * K;
    const int beg = offs[(size_t)w * (K + 1) + k], end = offs[(size_t)w * (K + 1) + k + 1];
    if (end == beg) return;
    const int32_t* pm = perm + (size_t)w * N;
    const T* Kw = Kr + (size_t)w * N * KV;
    __shared__ int mid[256];
    __shared__ double mw[256];
    __shared__ int wcnt[4];
    for (int e0 = 0; e0 < KV; e0 += 256 * 8 * CH) {
        double acc[CH][8];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[c][i] = 0.0;
        for (int b0 = beg; b0 < end; b0 += 256) {
            const int nv = stage_members(pm, b0, end, mid, mw, wcnt, [](int, double&) { return true; });
            member_sums<T, CH, false>(Kw, KV, e0, mid, mw, nv, acc);
        }
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int e = e0 + (int)(threadIdx.x + 256 * c) * 8;
            if (e < KV) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (float)(acc[c][i] / (double)(end - beg));
                store8(Ck + ((size_t)w * K + k) * KV + e, o);
            }
        }
    }
}

// objective of each window: sum over clusters of the fp64 norms of the
// centre sums, added in ascending cluster order by one lane after the wave
// has staged the window's K norms in LDS with coalesced loads
__global__ __launch_bounds__(64) void k_objective(const double* __restrict__ nrm, double* __restrict__ obj, int K)
{
    __shared__ double v[kMaxK];
    const int w = blockIdx.x, lane = lane_id();
    for (int k = lane; k < K; k += 64) v[k] = nrm[(size_t)w * K + k];
    __syncthreads();
    if (lane == 0) {
        double s = 0.0;
        for (int k = 0; k < K; ++k) s += v[k];
        obj[w] = s;
    }
}

// workspace layout
struct KmWs {
    uint16_t* Cb;
    int32_t* perm;
    int32_t* offs;
    int32_t* dirty;
    int32_t* conv;
    double* nrm;
    double* fm;
    float* fn;
    int32_t* stale;    // with coding: clusters rebuilt after the coding update
    int32_t* list;     // with coding: rows for the exact coder (a row at most twice:
                       // by the coding update and again if its cluster is rebuilt), and their count
    int32_t* listed;
    size_t bytes;
};

KmWs km_layout(const ps_shape* s, int dtype, void* base, bool coding = false)
{
    using ps_host::round256;
    const size_t W = (size_t)s->W, N = (size_t)s->N, K = (size_t)s->K, d = (size_t)s->d;
    size_t off = 0;
    KmWs L{};
    char* b = (char*)base;
    auto take = [&](size_t bytes) {
        char* p = b ? b + off : nullptr;
        off += round256(bytes);
        return p;
    };
    L.Cb = dtype == PS_BF16 ? (uint16_t*)take(W * K * d * 2) : nullptr;
    L.perm = (int32_t*)take(W * N * 4);
    L.offs = (int32_t*)take(W * (K + 1) * 4);
    L.dirty = (int32_t*)take(W * K * 4);
    L.conv = (int32_t*)take(W * 4);
    L.nrm = (double*)take(W * K * 8);
    L.fm = (double*)take(W * N * 8);
    L.fn = (float*)take(W * N * 4);
    if (coding) {
        L.stale = (int32_t*)take(W * K * 4);
        L.list = (int32_t*)take(2 * W * N * 4);
        L.listed = (int32_t*)take(16);
    }
    L.bytes = off;
    return L;
}

// clusters per workgroup in the updates after the first: most clusters are
// unchanged there, so on large batches four share a workgroup (a quarter of
// the workgroups to dispatch); one each on small batches and in the first
// update, where every cluster is rebuilt
int update_cpb(const ps_shape* s, int all)
{
    return (!all && s->W * s->K >= 16384) ? 4 : 1;
}

template <typename T, int CH>
void launch_update(const ps_shape* s, const void* H, const float* rn, const KmWs& ws, float* C,
                   int32_t* counts, int all, hipStream_t st)
{
    const int nclusters = s->W * s->K, cpb = update_cpb(s, all);
    const int nblocks = (nclusters + cpb - 1) / cpb;
    PS_LAUNCH_COUNTED("k_update<T, CH>", nclusters, (k_update<T, CH>), dim3(nblocks), dim3(256), 0, st,
                      (const T*)H, rn, ws.perm, ws.offs, C, ws.Cb, counts, ws.nrm, ws.dirty, ws.stale, s->N, s->d,
                      s->K, nblocks, cpb, nclusters, all);
}

// outputs of the residual coding folded into a K-Means call
struct Coding {
    uint8_t* codes;
    uint8_t* bscale;
    float* rscale;
};

// The coding update applies to bf16 rows of up to 4096 elements (the
// coder's one-wave-per-row form) on batches of fewer than 2^31 rows.
bool coding_update_fits(const ps_shape* s, ps_dtype dtype)
{
    return dtype == PS_BF16 && s->d <= 4096 && (int64_t)s->W * s->N < ((int64_t)1 << 31);
}

template <int CH, int BPL>
void launch_update_code(const ps_shape* s, const void* H, const float* rn, const KmWs& ws, float* C,
                        int32_t* counts, const Coding& cd, hipStream_t st)
{
    const int nblocks = s->W * s->K;
    if (s->d / 16 == 64 * BPL)
        PS_LAUNCH("k_update_code<CH, BPL, FULL>", (k_update_code<CH, BPL, true>), dim3(nblocks), dim3(256), 0, st,
                  (const uint16_t*)H, rn, ws.perm, ws.offs, C, ws.Cb, counts, ws.nrm, ws.dirty, ws.stale, cd.codes,
                  cd.bscale, cd.rscale, ws.list, ws.listed, s->N, s->d, s->K, nblocks);
    else
        PS_LAUNCH("k_update_code<CH, BPL, FULL>", (k_update_code<CH, BPL, false>), dim3(nblocks), dim3(256), 0, st,
                  (const uint16_t*)H, rn, ws.perm, ws.offs, C, ws.Cb, counts, ws.nrm, ws.dirty, ws.stale, cd.codes,
                  cd.bscale, cd.rscale, ws.list, ws.listed, s->N, s->d, s->K, nblocks);
}

template <int BPL>
void launch_code_stale(const ps_shape* s, const void* H, const float* rn, const KmWs& ws, const float* C,
                       const Coding& cd, hipStream_t st)
{
    const int nclusters = s->W * s->K, cpb = update_cpb(s, 0);
    const int nblocks = (nclusters + cpb - 1) / cpb;
    if (s->d / 16 == 64 * BPL)
        PS_LAUNCH_COUNTED("k_code_stale<BPL, FULL>", nclusters, (k_code_stale<BPL, true>), dim3(nblocks), dim3(256), 0,
                          st, (const uint16_t*)H, rn, ws.perm, ws.offs, C, ws.stale, cd.codes, cd.bscale, cd.rscale,
                          ws.list, ws.listed, s->N, s->d, s->K, nblocks, cpb, nclusters);
    else
        PS_LAUNCH_COUNTED("k_code_stale<BPL, FULL>", nclusters, (k_code_stale<BPL, false>), dim3(nblocks), dim3(256),
                          0, st, (const uint16_t*)H, rn, ws.perm, ws.offs, C, ws.stale, cd.codes, cd.bscale,
                          cd.rscale, ws.list, ws.listed, s->N, s->d, s->K, nblocks, cpb, nclusters);
}

template <bool FIRST>
void launch_assign_wide(const ps_shape* s, const void* H, const KmWs& ws, int32_t* assign, float* rn,
                        hipStream_t st)
{
    const int tiles = (s->N + kWideTok - 1) / kWideTok;
    const int nblocks = s->W * tiles;
    // the LDS limits are raised once per device (outside any stream capture
    // that a caller may run later).  Without the 160 KB the LDS-fed kernel
    // needs, the passes run the register-staged kernel; a failure to raise the
    // latter's limit shows up as a launch error.
    static int8_t dma_ok[64] = {};               // 0 unknown, 1 raised, -1 refused
    static bool raised[64] = {};
    int dev = 0;
    const bool known = hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64;
    if (known && !raised[dev]) {
        raised[dev] = hipFuncSetAttribute((const void*)k_assign_wide<true>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLds) == hipSuccess &&
                      hipFuncSetAttribute((const void*)k_assign_wide<false>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)kWideLds) == hipSuccess;
        const int lds = (int)kDmaLds;
        dma_ok[dev] = hipFuncSetAttribute((const void*)k_assign_wide_dma<true>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess &&
                      hipFuncSetAttribute((const void*)k_assign_wide_dma<false>,
                                          hipFuncAttributeMaxDynamicSharedMemorySize, lds) == hipSuccess
                          ? 1 : -1;
        (void)hipGetLastError();
    }
    if (s->d % kDmaDK == 0 && known && dma_ok[dev] == 1) {
        PS_LAUNCH_COUNTED(FIRST ? "k_assign_wide_dma<true>" : "k_assign_wide_dma<false>", nblocks,
                          k_assign_wide_dma<FIRST>, dim3(nblocks), dim3(512), kDmaLds, st, (const uint16_t*)H, ws.Cb,
                          assign, rn, s->N, s->d, s->K, tiles, nblocks, ws.dirty, ws.conv);
        return;
    }
    PS_LAUNCH_COUNTED(FIRST ? "k_assign_wide<true>" : "k_assign_wide<false>", nblocks, k_assign_wide<FIRST>,
                      dim3(nblocks), dim3(512), kWideLds, st, (const uint16_t*)H, ws.Cb, assign, rn, s->N, s->d,
                      s->K, tiles, nblocks, ws.dirty, ws.conv);
}

template <int KB, int NB>
void launch_assign_bf16(const ps_shape* s, const void* H, const float* C, const KmWs& ws, int32_t* assign,
                        float* rn, int first, hipStream_t st)
{
    const int tiles = (s->N + 64 * NB - 1) / (64 * NB);
    const int nblocks = s->W * tiles;
    if (first == 1)
        PS_LAUNCH_COUNTED("k_assign_bf16<KB, NB, true>", nblocks, (k_assign_bf16<KB, NB, true, true>),
                          dim3(nblocks), dim3(256), 0, st, (const uint16_t*)H, (const void*)C, assign, rn, s->N,
                          s->d, s->K, tiles, nblocks, ws.dirty, ws.conv);
    else if (first)
        PS_LAUNCH_COUNTED("k_assign_bf16<KB, NB, true>/bf16", nblocks, (k_assign_bf16<KB, NB, true, false>),
                          dim3(nblocks), dim3(256), 0, st, (const uint16_t*)H, (const void*)ws.Cb, assign, rn, s->N,
                          s->d, s->K, tiles, nblocks, ws.dirty, ws.conv);
    else
        PS_LAUNCH_COUNTED("k_assign_bf16<KB, NB, false>", nblocks, (k_assign_bf16<KB, NB, false, false>),
                          dim3(nblocks), dim3(256), 0, st, (const uint16_t*)H, ws.Cb, assign, rn, s->N, s->d,
                          s->K, tiles, nblocks, ws.dirty, ws.conv);
}

// compute units of the current device (cached per device; 256 if unknown)
int device_cus()
{
    static int cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        cus[dev] = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0
                       ? n : 256;
        (void)hipGetLastError();
    }
    return cus[dev];
}

// The tile kernel with NB 16-token blocks per wave, or with one when the
// launch would leave compute units idle (few windows): a quarter of the
// tokens per workgroup and four times the workgroups.  The number of tokens
// a wave owns does not change any score's accumulation order, so both give
// bit-identical results.  Such a small launch is bound by its few compute
// units' load rate, so its first pass reads the bf16 copy of the centres
// (written by k_centres_to_bf16 before it: half the bytes of the fp32
// centres, the same rounding); `first` is 1 for the fp32 operand, 2 for that.
bool assign_bf16_small(const ps_shape* s, int NB)
{
    const int64_t tiles = (int64_t)s->W * ((s->N + 64 * NB - 1) / (64 * NB));
    return NB > 1 && tiles < device_cus();
}

template <int KB, int NB>
void launch_assign_bf16_fit(const ps_shape* s, const void* H, const float* C, const KmWs& ws, int32_t* assign,
                            float* rn, int first, hipStream_t st)
{
    if (assign_bf16_small(s, NB))
        launch_assign_bf16<KB, 1>(s, H, C, ws, assign, rn, first ? 2 : 0, st);
    else
        launch_assign_bf16<KB, NB>(s, H, C, ws, assign, rn, first ? 1 : 0, st);
}

}  // namespace

extern "C" ps_status ps_workspace_size(const ps_shape* s, ps_dtype dtype, size_t* bytes)
{
    if (!s || !bytes) return PS_ERR_NULL;
    if (!ps_host::dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = ps_host::check_clusters(s);
    if (st != PS_OK) return st;
    *bytes = std::max(km_layout(s, dtype, nullptr, coding_update_fits(s, dtype)).bytes,
                      ps_host::residual_ws_bytes(s));
    return PS_OK;
}

namespace {

// every host-known check of a K-Means call except the workspace's
ps_status kmeans_fit_check(const ps_shape* s, ps_dtype dtype, const void* H, const void* Kr, ps_init init,
                           int32_t iters, uint32_t flags, const float* C, const int32_t* assign,
                           const int32_t* counts, const float* row_norm, const void* Ck, const double* objective)
{
    using namespace ps_host;
    if (!s || !H || !C || !assign || !counts || !row_norm) return PS_ERR_NULL;
    if ((Kr == nullptr) != (Ck == nullptr)) return PS_ERR_NULL;
    if (!dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = check_clusters(s);
    if (st != PS_OK) return st;
    if (Kr && (st = check_heads(s)) != PS_OK) return st;
    if (iters < 1) return PS_ERR_RANGE;
    if (init != PS_INIT_GIVEN && init != PS_INIT_STRIDED && init != PS_INIT_FARTHEST) return PS_ERR_RANGE;
    if (flags & ~(uint32_t)(PS_KMEANS_FIXED_POINT_EXIT | PS_KMEANS_ALL_PASSES)) return PS_ERR_RANGE;
    if ((flags & PS_KMEANS_FIXED_POINT_EXIT) && (flags & PS_KMEANS_ALL_PASSES)) return PS_ERR_RANGE;
    if (s->d > 8192) return PS_ERR_SHAPE;  // update kernel: at most 4 chunks of 2048 per thread
    if (!aligned16(H) || !aligned16(C) || !aligned16(assign) || !aligned16(counts) ||
        !aligned16(row_norm) || (Kr && (!aligned16(Kr) || !aligned16(Ck))) ||
        (objective && !aligned16(objective)))
        return PS_ERR_ALIGN;
    return PS_OK;
}

// The K-Means call; with `cd`, the rows' residual coding too (the caller has
// checked the coder's arguments and that ws holds km_layout(.., fuse) bytes).
ps_status kmeans_fit_impl(const ps_shape* s, ps_dtype dtype, const void* H, const void* Kr, ps_init init,
                          int32_t iters, uint32_t flags, float* C, int32_t* assign, int32_t* counts,
                          float* row_norm, void* Ck, double* objective, void* ws, size_t ws_bytes,
                          void* stream, const Coding* cd = nullptr)
{
    using namespace ps_host;
    ps_status st = kmeans_fit_check(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck,
                                    objective);
    if (st != PS_OK) return st;
    const bool fuse = cd && coding_update_fits(s, dtype);
    const KmWs need = km_layout(s, dtype, nullptr, fuse);
    if (!ws || ws_bytes < need.bytes) return PS_ERR_WORKSPACE;
    if (!aligned16(ws)) return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;

    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    const KmWs L = km_layout(s, dtype, ws, fuse);
    const int W = s->W, N = s->N, d = s->d, K = s->K;
    const bool bf = dtype == PS_BF16;

    if (init == PS_INIT_STRIDED) {
        if (bf) PS_LAUNCH("k_init_strided<uint16_t>", k_init_strided<uint16_t>, dim3(K, W), dim3(256), 0, stm, (const uint16_t*)H, C, N, d, K);
        else    PS_LAUNCH("k_init_strided<float>", k_init_strided<float>, dim3(K, W), dim3(256), 0, stm, (const float*)H, C, N, d, K);
    } else if (init == PS_INIT_FARTHEST) {
        const size_t shm = (size_t)d * sizeof(float);
        if (bf) PS_LAUNCH("k_init_farthest<uint16_t>", k_init_farthest<uint16_t>, dim3(W), dim3(256), shm, stm, (const uint16_t*)H, C, L.fm, L.fn, N, d, K);
        else    PS_LAUNCH("k_init_farthest<float>", k_init_farthest<float>, dim3(W), dim3(256), shm, stm, (const float*)H, C, L.fm, L.fn, N, d, K);
    }
    const int KBn = (K + 15) / 16;
    const bool small = KBn <= 8 && assign_bf16_small(s, KBn <= 4 ? PS_ASSIGN_NB_SMALLK : PS_ASSIGN_NB_LARGEK);
    if (bf && (K > 128 || small)) {
        // the tile kernels above 128 clusters, and a launch too small to fill
        // the device, read the bf16 copy from the first pass on; otherwise the
        // first pass rounds the fp32 centres itself
        const size_t n8 = (size_t)W * K * d / 8;
        const int blocks = (int)std::min<size_t>((n8 + 255) / 256, 8192);
        PS_LAUNCH("k_centres_to_bf16", k_centres_to_bf16, dim3(blocks), dim3(256), 0, stm, C, L.Cb, n8);
    }
    const int CH = (d + 2047) / 2048;
    // Iteration 0 assigns against the incoming centres and rebuilds every
    // cluster (the rows themselves are new).  Later iterations mark the two
    // clusters of every row that moves; only those are rebuilt, and a window
    // whose last iteration moved no row is at a fixed point: its later
    // iterations are skipped (unless PS_KMEANS_ALL_PASSES), bit-identically.
    const int fpx = (flags & PS_KMEANS_ALL_PASSES) ? 0 : 1;
    for (int it = 0; it < iters; ++it) {
        const int first = it == 0;
        if (bf) {
            if (KBn <= 1)      launch_assign_bf16_fit<1, PS_ASSIGN_NB_SMALLK>(s, H, C, L, assign, row_norm, first, stm);
            else if (KBn <= 2) launch_assign_bf16_fit<2, PS_ASSIGN_NB_SMALLK>(s, H, C, L, assign, row_norm, first, stm);
            else if (KBn <= 4) launch_assign_bf16_fit<4, PS_ASSIGN_NB_SMALLK>(s, H, C, L, assign, row_norm, first, stm);
            else if (KBn <= 8) launch_assign_bf16_fit<8, PS_ASSIGN_NB_LARGEK>(s, H, C, L, assign, row_norm, first, stm);
            else if (first)    launch_assign_wide<true>(s, H, L, assign, row_norm, stm);
            else               launch_assign_wide<false>(s, H, L, assign, row_norm, stm);
        } else {
            const int64_t rows = (int64_t)W * N;
            PS_LAUNCH_COUNTED("k_assign_f32", rows, k_assign_f32, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0,
                              stm, (const float*)H, C, assign, row_norm, W, N, d, K, first, L.dirty, L.conv);
        }
        PS_LAUNCH("k_bucket", k_bucket, dim3(W), dim3(64 * kBucketWaves), 0, stm, assign, L.perm, L.offs, L.dirty, L.conv, N, K,
                  first, fpx, L.listed);
        if (fuse && first) {
            const int nb = d / 16;
            if (nb <= 64)       launch_update_code<1, 1>(s, H, row_norm, L, C, counts, *cd, stm);
            else if (nb <= 128) launch_update_code<1, 2>(s, H, row_norm, L, C, counts, *cd, stm);
            else                launch_update_code<2, 4>(s, H, row_norm, L, C, counts, *cd, stm);
        } else if (bf) {
            switch (CH) {
            case 1: launch_update<uint16_t, 1>(s, H, row_norm, L, C, counts, first, stm); break;
            case 2: launch_update<uint16_t, 2>(s, H, row_norm, L, C, counts, first, stm); break;
            case 3: launch_update<uint16_t, 3>(s, H, row_norm, L, C, counts, first, stm); break;
            default: launch_update<uint16_t, 4>(s, H, row_norm, L, C, counts, first, stm); break;
            }
        } else {
            switch (CH) {
            case 1: launch_update<float, 1>(s, H, row_norm, L, C, counts, first, stm); break;
            case 2: launch_update<float, 2>(s, H, row_norm, L, C, counts, first, stm); break;
            case 3: launch_update<float, 3>(s, H, row_norm, L, C, counts, first, stm); break;
            default: launch_update<float, 4>(s, H, row_norm, L, C, counts, first, stm); break;
            }
        }
    }
    if (Kr) {
        const int KV = s->Hkv * s->dh;
        const int nblocks = W * K;
        if (bf) PS_LAUNCH("k_keys<uint16_t>", k_keys<uint16_t>, dim3(nblocks), dim3(256), 0, stm, (const uint16_t*)Kr, L.perm, L.offs, (uint16_t*)Ck, N, KV, K, nblocks);
        else    PS_LAUNCH("k_keys<float>", k_keys<float>, dim3(nblocks), dim3(256), 0, stm, (const float*)Kr, L.perm, L.offs, (float*)Ck, N, KV, K, nblocks);
    }
    if (objective)
        PS_LAUNCH("k_objective", k_objective, dim3(W), dim3(64), 0, stm, L.nrm, objective, K);
    if (fuse) {
        // the rows of clusters rebuilt after the coding update, then every
        // row the fast path declined
        const int nb = d / 16;
        if (nb <= 64)       launch_code_stale<1>(s, H, row_norm, L, C, *cd, stm);
        else if (nb <= 128) launch_code_stale<2>(s, H, row_norm, L, C, *cd, stm);
        else                launch_code_stale<4>(s, H, row_norm, L, C, *cd, stm);
        residual_listed(s, (const uint16_t*)H, row_norm, C, assign, L.list, L.listed, cd->codes, cd->bscale,
                        cd->rscale, stm);
    }
    if (hipGetLastError() != hipSuccess) return PS_ERR_DEVICE;
    if (cd && !fuse)   // the coder as its own call, on the workspace the fit no longer needs
        return ps_residual_nvfp4(s, dtype, H, row_norm, C, assign, cd->codes, cd->bscale, cd->rscale, ws,
                                 ws_bytes, stream);
    return PS_OK;
}

}  // namespace

extern "C" ps_status ps_kmeans_fit(const ps_shape* s, ps_dtype dtype, const void* H, const void* Kr,
                                   ps_init init, int32_t iters, uint32_t flags, float* C, int32_t* assign,
                                   int32_t* counts, float* row_norm, void* Ck, double* objective,
                                   void* ws, size_t ws_bytes, void* stream)
{
    return kmeans_fit_impl(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck, objective, ws,
                           ws_bytes, stream);
}

extern "C" ps_status ps_kmeans_fit_nvfp4(const ps_shape* s, ps_dtype dtype, const void* H, const void* Kr,
                                         ps_init init, int32_t iters, uint32_t flags, float* C, int32_t* assign,
                                         int32_t* counts, float* row_norm, void* Ck, double* objective,
                                         uint8_t* codes, uint8_t* bscale, float* rscale, void* ws,
                                         size_t ws_bytes, void* stream)
{
    using namespace ps_host;
    ps_status st = kmeans_fit_check(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck,
                                    objective);
    if (st != PS_OK) return st;
    if (!codes || !bscale || !rscale) return PS_ERR_NULL;
    if (!aligned16(codes) || !aligned16(bscale) || !aligned16(rscale)) return PS_ERR_ALIGN;
    const size_t need = std::max(km_layout(s, dtype, nullptr, coding_update_fits(s, dtype)).bytes,
                                 residual_ws_bytes(s));
    if (!ws || ws_bytes < need) return PS_ERR_WORKSPACE;
    const Coding cd{codes, bscale, rscale};
    return kmeans_fit_impl(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck, objective, ws,
                           ws_bytes, stream, &cd);
}

// ---------------------------------------------------------------------------
// Allocation-free variant: the K-Means scratch lives in a file-scope device
// array, one copy per device, whose device address is looked up once per
// device (in host code the array's name is not a device address).  Every
// kernel writes the scratch it later reads within the same call, so the
// previous call's contents are never read; calls that overlap on one device
// share the array and race.
// ---------------------------------------------------------------------------
static __device__ __align__(256) uint8_t scratch[PS_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

// device address of `scratch` on the current device
ps_status static_scratch(void** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return PS_ERR_DEVICE;
    }
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return PS_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PS_OK;
}

}  // namespace

extern "C" ps_status ps_kmeans_fit_static(const ps_shape* s, ps_dtype dtype, const void* H, const void* Kr,
                                          ps_init init, int32_t iters, uint32_t flags, float* C,
                                          int32_t* assign, int32_t* counts, float* row_norm, void* Ck,
                                          double* objective, void* stream)
{
    ps_status st = kmeans_fit_check(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck,
                                    objective);
    if (st != PS_OK) return st;
    if (km_layout(s, dtype, nullptr).bytes > (size_t)PS_STATIC_SCRATCH_BYTES) return PS_ERR_SCRATCH_LIMIT;
    if (s->W == 0) return PS_OK;
    void* ws = nullptr;
    if ((st = static_scratch(&ws)) != PS_OK) return st;
    return kmeans_fit_impl(s, dtype, H, Kr, init, iters, flags, C, assign, counts, row_norm, Ck, objective, ws,
                           (size_t)PS_STATIC_SCRATCH_BYTES, stream);
}
