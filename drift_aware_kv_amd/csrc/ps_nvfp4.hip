// ps_nvfp4.hip -- NVFP4 residual coding of the window rows (Polestar
// technical summary 2.A, local window and clustering: residuals to the
// cluster centres are stored in NVFP4) and the refresh gather of the rows of
// the selected clusters (2.A, sparse updates; 2.C, only the selected clusters
// are fetched), for gfx950.
//
// The coder gives each row one wave (four for rows longer than 4096), each
// thread owning whole 16-element blocks, with 16-byte loads all issued before
// use and at most one cross-wave exchange per row.  Its fast path replaces
// divisions by reciprocal products and uses the hardware E4M3/E2M1
// conversions, each proven or exhaustively checked to give the results of the
// stated convention (every fp32 step one correctly rounded operation) bit for
// bit; rows outside the proof's conditions take the exact path.  The gather is bandwidth bound: one workgroup per selected row.
#include "ps_common.h"
#include "ps_nvfp4_fast.h"
#include "ps_nvfp4_row.h"

using namespace ps;

namespace {

// One row is coded by NW waves (TPR = 64 * NW threads).  Thread i of the row
// owns the 8-element chunks i, i + TPR, ..., so each load instruction of a wave
// covers 64 consecutive chunks; a 16-element block is the chunk pair held by
// threads 2m and 2m + 1 (adjacent lanes).  Chunks past the row read the last
// chunk again (always in bounds) and are masked.
template <typename T, int TPR, int CPL>
__device__ __forceinline__ void load_chunks(const T* __restrict__ h, const float* __restrict__ c, int tid,
                                            int nch, uint4 (&hq)[CPL][sizeof(T) == 2 ? 1 : 2],
                                            float (&r)[CPL][8])
{
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = min(tid + TPR * i, nch - 1);
        const uint4* hp = reinterpret_cast<const uint4*>(h + 8 * ch);
        hq[i][0] = hp[0];
        if (sizeof(T) != 2) hq[i][sizeof(T) == 2 ? 0 : 1] = hp[1];
        const float4* cp = reinterpret_cast<const float4*>(c + 8 * ch);
        const float4 a = cp[0], b = cp[1];
        r[i][0] = a.x; r[i][1] = a.y; r[i][2] = a.z; r[i][3] = a.w;
        r[i][4] = b.x; r[i][5] = b.y; r[i][6] = b.z; r[i][7] = b.w;
    }
}

template <typename T>
__device__ __forceinline__ void unpack8(const uint4 (&q)[sizeof(T) == 2 ? 1 : 2], float (&hv)[8])
{
    if (sizeof(T) == 2) {
        const uint32_t w[4] = {q[0].x, q[0].y, q[0].z, q[0].w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            hv[2 * t] = __uint_as_float(w[t] << 16);
            hv[2 * t + 1] = __uint_as_float(w[t] & 0xffff0000u);
        }
    } else {
        const uint4 a = q[0], b = q[sizeof(T) == 2 ? 0 : 1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int t = 0; t < 8; ++t) hv[t] = __uint_as_float(w[t]);
    }
}

template <int TPR, int CPL>
__device__ __forceinline__ void store_chunks(const uint32_t (&words)[CPL], const uint32_t (&scales)[CPL],
                                             int tid, int nch, uint8_t* __restrict__ cr, uint8_t* __restrict__ br)
{
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int ch = tid + TPR * i;
        if (ch < nch) {
            *reinterpret_cast<uint32_t*>(cr + 4 * ch) = words[i];
            if (!(ch & 1)) br[ch >> 1] = (uint8_t)scales[i];
        }
    }
}

// Exact NVFP4 coding of one row: every quotient a correctly rounded fp32
// division, E2M1 by threshold comparison (the rows the fast path declines).
template <typename T, int NW, int CPL>
__device__ __forceinline__ void residual_row_exact(const T* __restrict__ h, const float* __restrict__ c, float n,
                                                   uint8_t* __restrict__ cr, uint8_t* __restrict__ br,
                                                   float* __restrict__ rs, int d, uint32_t (*red)[3])
{
    constexpr int TPR = 64 * NW;
    const int tid = (int)(threadIdx.x % TPR), wave = tid >> 6;
    const int nch = d >> 3;
    const bool full = nch == TPR * CPL;
    const bool pos_n = n > 0.0f;
    uint4 hq[CPL][sizeof(T) == 2 ? 1 : 2];
    float r[CPL][8];
    load_chunks<T, TPR, CPL>(h, c, tid, nch, hq, r);
    float cmax[CPL];
    float A = 0.0f;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const bool valid = full || tid + TPR * i < nch;
        float hv[8];
        unpack8<T>(hq[i], hv);
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const float x = pos_n ? hv[t] / n : 0.0f;
            r[i][t] = valid ? x - r[i][t] : 0.0f;
            m = fmaxf(m, fabsf(r[i][t]));
        }
        cmax[i] = m;
        A = fmaxf(A, m);
    }
    A = wave_max(A);
    if (NW > 1) {
        if ((tid & 63) == 0) red[wave][0] = __float_as_uint(A);
        __syncthreads();
#pragma unroll
        for (int q = 0; q < NW; ++q) A = fmaxf(A, __uint_as_float(red[q][0]));
    }
    const bool zero_row = !(A > 0.0f);
    const float g = A / 2688.0f;
    uint32_t words[CPL], scales[CPL];
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const float Ab = fmaxf(cmax[i], __shfl_xor(cmax[i], 1, 64));
        uint32_t word = 0, sb = 0;
        if (!zero_row) {
            sb = e4m3_encode((Ab / 6.0f) / g);
            const float eff = e4m3_decode(sb) * g;
            if (eff != 0.0f) {
#pragma unroll
                for (int t = 0; t < 8; ++t) word |= e2m1_encode(r[i][t] / eff) << (4 * t);
            }
        }
        words[i] = word;
        scales[i] = sb;
    }
    store_chunks<TPR, CPL>(words, scales, tid, nch, cr, br);
    if (tid == 0) *rs = zero_row ? 0.0f : g;
}

// NW waves per row: four one-wave rows per workgroup, or one row of NW waves
// per workgroup (64 * NW threads); one exchange (and with one wave per row,
// none) per row.  Consecutive rows (one window's,
// sharing its centres) stay on one XCD.  BPL blocks of 16 per thread on the
// fast path; the exact path holds the same elements as 2 * BPL chunks of 8.
template <typename T, int NW, int BPL, bool FULL>
__global__ __launch_bounds__(256) void k_residual(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                   const float* __restrict__ C, const int32_t* __restrict__ assign,
                                                   uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                   float* __restrict__ rscale, int64_t rows, int N, int d, int K)
{
    constexpr int RPB = NW == 1 ? 4 : 1;         // rows per workgroup
    __shared__ uint32_t red[4][3];
    const int64_t row = (int64_t)xcd_remap(blockIdx.x, gridDim.x) * RPB + (RPB > 1 ? (int)(threadIdx.x / (64 * NW)) : 0);
    // with one row per workgroup every thread has the same row; with several,
    // a whole wave leaves together and no barrier follows on this path
    if (row >= rows) return;
    const int w = rows < ((int64_t)1 << 32) ? (int)((uint32_t)row / (uint32_t)N) : (int)(row / N);
    int a = assign[row];
    if (a < 0 || a >= K) a = 0;
    const float* c = C + ((size_t)w * K + a) * d;
    const T* h = H + (size_t)row * d;
    uint8_t* cr = codes + (size_t)row * (d >> 1);
    uint8_t* br = bscale + (size_t)row * (d >> 4);
    const float n = row_norm[row];
    constexpr int TPR = 64 * NW;
    uint4 hq[BPL][sizeof(T) == 2 ? 2 : 4];
    float cv[BPL][16];
    load_hblocks<T, TPR, BPL>(h, (int)(threadIdx.x % TPR), d >> 4, hq);
    load_cblocks<TPR, BPL>(c, (int)(threadIdx.x % TPR), d >> 4, cv);
    if (!residual_row_fast<T, NW, BPL, FULL>(hq, cv, n, cr, br, rscale + row, d, red)) {
        if (NW > 1) __syncthreads();  // red[] is reused
        residual_row_exact<T, NW, 2 * BPL>(h, c, n, cr, br, rscale + row, d, red);
    }
}

// Rows of each window grouped by cluster: perm[w][.] lists the window's rows
// with each cluster's members contiguous, clusters in ascending order (the
// order within a cluster is unspecified: no result depends on it).
// Assignments outside [0, K) count as cluster 0, as the coder reads them.
// One workgroup per window; the first also clears the count of listed rows.
__global__ __launch_bounds__(1024) void k_group_rows(const int32_t* __restrict__ assign,
                                                      int32_t* __restrict__ perm, int32_t* __restrict__ listed,
                                                      int N, int K)
{
    __shared__ int base[kMaxK];
    __shared__ int wsum[16];
    const int w = blockIdx.x, t = threadIdx.x;
    if (w == 0 && t == 0) *listed = 0;
    for (int c = t; c < K; c += 1024) base[c] = 0;
    __syncthreads();
    const int32_t* a = assign + (size_t)w * N;
    for (int j = t; j < N; j += 1024) {
        const int c = a[j];
        atomicAdd(&base[(unsigned)c < (unsigned)K ? c : 0], 1);
    }
    __syncthreads();
    // exclusive prefix sum of the counts; thread t owns cluster t
    const int v = t < K ? base[t] : 0;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if ((t & 63) >= o) x += y;
    }
    if ((t & 63) == 63) wsum[t >> 6] = x;
    __syncthreads();
    int off = x - v;
    for (int q = 0; q < (t >> 6); ++q) off += wsum[q];
    if (t < K) base[t] = off;
    __syncthreads();
    for (int j = t; j < N; j += 1024) {
        const int c = a[j];
        const int p = atomicAdd(&base[(unsigned)c < (unsigned)K ? c : 0], 1);
        perm[(size_t)w * N + p] = j;
    }
}

// The coder over grouped rows: each wave codes kGroupRows consecutive entries
// of its window's perm, one row at a time, and keeps the current cluster's
// centre blocks in registers, reloading them only when the cluster changes, so
// each centre is read about once per wave instead of once per row.  Rows the
// fast path declines are appended to a list for k_residual_listed.  One wave
// per row (rows of up to 4096 elements), three waves per SIMD (168
// registers); the workgroups of a window stay on one XCD.
constexpr int kGroupRows = 16;

template <typename T, int BPL, bool FULL>
__global__ __launch_bounds__(256, 3) void k_residual_grouped(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                           const float* __restrict__ C,
                                                           const int32_t* __restrict__ assign,
                                                           const int32_t* __restrict__ perm,
                                                           int32_t* __restrict__ list, int32_t* __restrict__ listed,
                                                           uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                           float* __restrict__ rscale, int N, int d, int K, int tiles,
                                                           int nblocks)
{
    constexpr int HW = sizeof(T) == 2 ? 2 : 4;
    const int tile = xcd_remap(blockIdx.x, nblocks);
    const int w = tile / tiles;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int p0 = (tile - w * tiles) * (4 * kGroupRows) + wave * kGroupRows;
    const int p1 = min(p0 + kGroupRows, N);
    if (p0 >= p1) return;
    const int lane = (int)(threadIdx.x & 63), nb = d >> 4;
    const size_t wrow = (size_t)w * N;
    const int32_t* pw = perm + wrow;
    float cv[BPL][16];
    int cur = -1;
    for (int p = p0; p < p1; ++p) {
        const int j = min(max(pw[p], 0), N - 1);
        const size_t row = wrow + j;
        int a = assign[row];
        if (a < 0 || a >= K) a = 0;
        const float n = row_norm[row];
        uint4 hq[BPL][HW];
        load_hblocks<T, 64, BPL>(H + row * d, lane, nb, hq);
        if (a != cur) {
            load_cblocks<64, BPL>(C + ((size_t)w * K + a) * d, lane, nb, cv);
            cur = a;
        }
        if (!residual_row_fast<T, 1, BPL, FULL>(hq, cv, n, codes + row * (size_t)(d >> 1),
                                                bscale + row * (size_t)(d >> 4), rscale + row, d, nullptr)) {
            if (lane == 0) list[atomicAdd(listed, 1)] = (int32_t)row;
        }
    }
}

// The exact coder over the listed rows, one wave per row; every wave reads the
// count and strides over the list.
template <typename T, int CPL>
__global__ __launch_bounds__(256) void k_residual_listed(const T* __restrict__ H, const float* __restrict__ row_norm,
                                                          const float* __restrict__ C,
                                                          const int32_t* __restrict__ assign,
                                                          const int32_t* __restrict__ list,
                                                          const int32_t* __restrict__ listed,
                                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ bscale,
                                                          float* __restrict__ rscale, int N, int d, int K)
{
    const int total = *listed;
    const int stride = (int)gridDim.x * 4;
    for (int i = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); i < total; i += stride) {
        const size_t row = (size_t)list[i];
        const int w = (int)(row / (size_t)N);
        int a = assign[row];
        if (a < 0 || a >= K) a = 0;
        residual_row_exact<T, 1, CPL>(H + row * d, C + ((size_t)w * K + a) * d, row_norm[row],
                                      codes + row * (size_t)(d >> 1), bscale + row * (size_t)(d >> 4),
                                      rscale + row, d, nullptr);
    }
}

// stable compaction of the members of the selected clusters, one 8-wave
// workgroup per window: wave v owns the v-th of eight consecutive row ranges,
// counts its members, and writes them from the count of waves 0..v-1 on, in
// ascending order (a ballot prefix within each 64 rows)
constexpr int kSelectWaves = 8;

__global__ __launch_bounds__(64 * kSelectWaves) void k_gather_select(const int32_t* __restrict__ assign,
                                                                      const int32_t* __restrict__ idx, int k,
                                                                      int cap, int32_t* __restrict__ pos,
                                                                      int32_t* __restrict__ count, int N, int K)
{
    constexpr int NW = kSelectWaves;
    __shared__ uint8_t sel[kMaxK];
    __shared__ int wcnt[NW];
    const int w = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
    for (int c = tid; c < K; c += 64 * NW) sel[c] = 0;
    __syncthreads();
    for (int r = tid; r < k; r += 64 * NW) {
        const int c = idx[(size_t)w * k + r];
        if (c >= 0 && c < K) sel[c] = 1;
    }
    __syncthreads();
    const int32_t* a = assign + (size_t)w * N;
    const int seg = (N + 64 * NW - 1) / (64 * NW) * 64;
    const int j0 = min(wave * seg, N), j1 = min(j0 + seg, N);
    int mine = 0;
    for (int base = j0; base < j1; base += 64) {
        const int j = base + lane;
        bool p = false;
        if (j < j1) {
            const int c = a[j];
            p = c >= 0 && c < K && sel[c];
        }
        mine += __popcll(__ballot(p));
    }
    if (lane == 0) wcnt[wave] = mine;
    __syncthreads();
    int running = 0, total = 0;
    for (int v = 0; v < NW; ++v) {
        if (v < wave) running += wcnt[v];
        total += wcnt[v];
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = j0; base < j1; base += 64) {
        const int j = base + lane;
        bool p = false;
        if (j < j1) {
            const int c = a[j];
            p = c >= 0 && c < K && sel[c];
        }
        const uint64_t m = __ballot(p);
        const int slot = running + __popcll(m & lt);
        if (p && slot < cap) pos[(size_t)w * cap + slot] = j;
        running += __popcll(m);
    }
    if (tid == 0) count[w] = total;
}

// rebuild / copy the gathered rows: G workgroups per window, each striding
// over the window's slots.  A slot's reads (codes, block scales, centre row,
// K and V rows; up to 512 pieces of each per round) are all issued before its
// first store, so a workgroup waits on memory once per round rather than once
// per piece.  After the XCD remap a window's workgroups are consecutive, so
// they run on one XCD and the centre rows of its selected clusters, read once
// per gathered row, come from that XCD's L2 after the first.
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
                                                      T* __restrict__ V_out, int N, int d, int K, int KV,
                                                      int G, int nblocks)
{
    const int L = xcd_remap(blockIdx.x, nblocks);
    const int w = L / G, gb = L - w * G, tid = threadIdx.x;
    const int cnt = count[w];
    const int M = cnt < cap ? cnt : cap;
    const int nh = H_hat ? (d >> 3) : 0;                              // 8-element chunks
    const int npc = (int)((size_t)KV * sizeof(T) / 16);               // 16-byte pieces of a K/V row
    const int nk = Kc ? npc : 0, nv = Vc ? npc : 0;
    const int rounds = (max(nh, max(nk, nv)) + 511) / 512;
    for (int slot = gb; slot < M; slot += G) {
        const int j = pos[(size_t)w * cap + slot];
        const size_t row = (size_t)w * N + j;
        const size_t orow = (size_t)w * cap + slot;
        float g = 0.0f, n = 0.0f;
        const float* c = C;
        if (H_hat) {
            int a = assign[row];
            if (a < 0 || a >= K) a = 0;
            g = rscale[row];
            n = row_norm[row];
            c = C + ((size_t)w * K + a) * d;
        }
        const uint32_t* cw = reinterpret_cast<const uint32_t*>(codes + row * (size_t)(d >> 1));
        const uint8_t* bs = bscale + row * (size_t)(d >> 4);
        const uint4* ks = Kc ? reinterpret_cast<const uint4*>(Kc + row * KV) : nullptr;
        const uint4* vs = Vc ? reinterpret_cast<const uint4*>(Vc + row * KV) : nullptr;
        for (int r = 0; r < rounds; ++r) {
            uint32_t word[2] = {0u, 0u}, sb[2] = {0u, 0u};
            float cv[2][8];
            uint4 kq[2], vq[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = 512 * r + 256 * u + tid;
                if (i < nh) {
                    word[u] = cw[i];
                    sb[u] = bs[i >> 1];
                    load8(c + 8 * i, cv[u]);
                }
                if (i < nk) kq[u] = ks[i];
                if (i < nv) vq[u] = vs[i];
            }
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = 512 * r + 256 * u + tid;
                if (i < nh) {
                    const float sh = e4m3_decode(sb[u]);
                    float o[8];
#pragma unroll
                    for (int t = 0; t < 8; ++t) {
                        const float rh = (e2m1_decode((word[u] >> (4 * t)) & 15u) * sh) * g;
                        o[t] = (cv[u][t] + rh) * n;
                    }
                    store8(H_hat + orow * d + 8 * i, o);
                }
                if (i < nk) reinterpret_cast<uint4*>(K_out + orow * KV)[i] = kq[u];
                if (i < nv) reinterpret_cast<uint4*>(V_out + orow * KV)[i] = vq[u];
            }
        }
    }
}

template <typename T, int NW, int BPL>
void launch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                     uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int64_t rows = (int64_t)s->W * s->N;
    const int rpb = NW == 1 ? 4 : 1;
    const dim3 grid((unsigned)((rows + rpb - 1) / rpb)), block(64 * NW * rpb);
    if (s->d / 16 == 64 * NW * BPL)
        PS_LAUNCH("k_residual<T, NW, BPL, FULL>", (k_residual<T, NW, BPL, true>), grid, block, 0, st,
                  (const T*)H, rn, C, a, codes, bscale, rscale, rows, s->N, s->d, s->K);
    else
        PS_LAUNCH("k_residual<T, NW, BPL, FULL>", (k_residual<T, NW, BPL, false>), grid, block, 0, st,
                  (const T*)H, rn, C, a, codes, bscale, rscale, rows, s->N, s->d, s->K);
}

template <typename T, int BPL>
void launch_listed(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                   const int32_t* list, const int32_t* listed, uint8_t* codes, uint8_t* bscale, float* rscale,
                   hipStream_t st)
{
    const size_t rows = (size_t)s->W * s->N;
    const unsigned lb = (unsigned)std::min<size_t>((rows + 3) / 4, 1024);
    PS_LAUNCH("k_residual_listed<T, CPL>", (k_residual_listed<T, 2 * BPL>), dim3(lb), dim3(256), 0, st,
              (const T*)H, rn, C, a, list, listed, codes, bscale, rscale, s->N, s->d, s->K);
}

template <typename T, int BPL>
void launch_residual_grouped(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                             int32_t* ws, uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const size_t rows = (size_t)s->W * s->N;
    int32_t* perm = ws;
    int32_t* list = ws + rows;
    int32_t* listed = ws + 2 * rows;
    PS_LAUNCH("k_group_rows", k_group_rows, dim3(s->W), dim3(1024), 0, st, a, perm, listed, s->N, s->K);
    const int tiles = (s->N + 4 * kGroupRows - 1) / (4 * kGroupRows);
    const int nblocks = s->W * tiles;
    if (s->d / 16 == 64 * BPL)
        PS_LAUNCH("k_residual_grouped<T, BPL, FULL>", (k_residual_grouped<T, BPL, true>), dim3(nblocks), dim3(256),
                  0, st, (const T*)H, rn, C, a, perm, list, listed, codes, bscale, rscale, s->N, s->d, s->K, tiles,
                  nblocks);
    else
        PS_LAUNCH("k_residual_grouped<T, BPL, FULL>", (k_residual_grouped<T, BPL, false>), dim3(nblocks), dim3(256),
                  0, st, (const T*)H, rn, C, a, perm, list, listed, codes, bscale, rscale, s->N, s->d, s->K, tiles,
                  nblocks);
    launch_listed<T, BPL>(s, H, rn, C, a, list, listed, codes, bscale, rscale, st);
}

// rows of up to 4096 elements: one wave per row, 1, 2 or 4 blocks of 16 per
// thread, over rows grouped by cluster when scratch is given; longer rows (up
// to 8192): four waves, 2 blocks per thread, in row order
template <typename T>
void dispatch_residual(const ps_shape* s, const void* H, const float* rn, const float* C, const int32_t* a,
                       int32_t* perm, uint8_t* codes, uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int nb = s->d / 16;
    if (perm && nb <= 256 && (int64_t)s->W * s->N < ((int64_t)1 << 31)) {
        if (nb <= 64)       launch_residual_grouped<T, 1>(s, H, rn, C, a, perm, codes, bscale, rscale, st);
        else if (nb <= 128) launch_residual_grouped<T, 2>(s, H, rn, C, a, perm, codes, bscale, rscale, st);
        else                launch_residual_grouped<T, 4>(s, H, rn, C, a, perm, codes, bscale, rscale, st);
        return;
    }
    if (nb <= 64)        launch_residual<T, 1, 1>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (nb <= 128)  launch_residual<T, 1, 2>(s, H, rn, C, a, codes, bscale, rscale, st);
    else if (nb <= 256)  launch_residual<T, 1, 4>(s, H, rn, C, a, codes, bscale, rscale, st);
    else                 launch_residual<T, 4, 2>(s, H, rn, C, a, codes, bscale, rscale, st);
}

}  // namespace

void ps_host::residual_listed(const ps_shape* s, const uint16_t* H, const float* row_norm, const float* C,
                              const int32_t* assign, const int32_t* list, const int32_t* listed, uint8_t* codes,
                              uint8_t* bscale, float* rscale, hipStream_t st)
{
    const int nb = s->d / 16;
    if (nb <= 64)       launch_listed<uint16_t, 1>(s, H, row_norm, C, assign, list, listed, codes, bscale, rscale, st);
    else if (nb <= 128) launch_listed<uint16_t, 2>(s, H, row_norm, C, assign, list, listed, codes, bscale, rscale, st);
    else                launch_listed<uint16_t, 4>(s, H, row_norm, C, assign, list, listed, codes, bscale, rscale, st);
}

extern "C" ps_status ps_residual_nvfp4(const ps_shape* s, ps_dtype dtype, const void* H,
                                       const float* row_norm, const float* C, const int32_t* assign,
                                       uint8_t* codes, uint8_t* bscale, float* rscale, void* ws,
                                       size_t ws_bytes, void* stream)
{
    using namespace ps_host;
    if (!s || !H || !row_norm || !C || !assign || !codes || !bscale || !rscale) return PS_ERR_NULL;
    if (!dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = check_clusters(s);
    if (st != PS_OK) return st;
    if (s->d > 8192) return PS_ERR_SHAPE;
    if (!aligned16(H) || !aligned16(row_norm) || !aligned16(C) || !aligned16(assign) || !aligned16(codes) ||
        !aligned16(bscale) || !aligned16(rscale) || (ws && !aligned16(ws)))
        return PS_ERR_ALIGN;
    if (ws && ws_bytes < residual_ws_bytes(s)) return PS_ERR_WORKSPACE;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    int32_t* perm = (int32_t*)ws;
    (void)hipGetLastError();
    if (dtype == PS_BF16) dispatch_residual<uint16_t>(s, H, row_norm, C, assign, perm, codes, bscale, rscale, stm);
    else                  dispatch_residual<float>(s, H, row_norm, C, assign, perm, codes, bscale, rscale, stm);
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
    PS_LAUNCH("k_gather_select", k_gather_select, dim3(s->W), dim3(64 * kSelectWaves), 0, stm, assign, idx, k, cap, pos, count, s->N, s->K);
    if (cap > 0 && (H_hat || Kc || Vc)) {
        // two workgroups per slot at the mean selection size (N k / K rows)
        const int64_t expect = ((int64_t)s->N * k + s->K - 1) / s->K;
        int G = (int)std::min<int64_t>(2 * expect, 65535);
        if (G < 1) G = 1;
        if (G > cap) G = cap;
        G = (int)std::max<int64_t>(1, std::min<int64_t>(G, INT32_MAX / std::max(s->W, 1)));
        const int nblocks = G * s->W;
        const int KV = (Kc || Vc) ? s->Hkv * s->dh : 0;
        if (dtype == PS_BF16)
            PS_LAUNCH("k_gather_rows<uint16_t>", k_gather_rows<uint16_t>, dim3(nblocks), dim3(256), 0, stm, pos, count,
                      cap, assign, codes, bscale, rscale, C, row_norm, (uint16_t*)H_hat, (const uint16_t*)Kc,
                      (const uint16_t*)Vc, (uint16_t*)K_out, (uint16_t*)V_out, s->N, s->d, s->K, KV, G, nblocks);
        else
            PS_LAUNCH("k_gather_rows<float>", k_gather_rows<float>, dim3(nblocks), dim3(256), 0, stm, pos, count, cap,
                      assign, codes, bscale, rscale, C, row_norm, (float*)H_hat, (const float*)Kc, (const float*)Vc,
                      (float*)K_out, (float*)V_out, s->N, s->d, s->K, KV, G, nblocks);
    }
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}
