// ps_attn.hip -- proxy attention of the decode block against the centroid
// keys, the KL drift between consecutive steps, and the top-k selection of
// the most drifted clusters (Polestar technical summary 2.A: drift
// measurement; sparse updates), for gfx950.
#include "ps_common.h"

using namespace ps;

namespace {

// e^x and ln x on the hardware's base-2 exponential and logarithm
// (v_exp_f32, v_log_f32, about one ulp each) after one fp32 scaling: the
// math library's expf and logf add range reduction and special-case selects,
// about a dozen VALU instructions a call, which made the softmax and KL
// epilogue the larger half of proxy attention's instruction stream.
// exp_hw(-inf) = 0; results below 2^-126 may flush to zero.
__device__ __forceinline__ float exp_hw(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }
__device__ __forceinline__ float log_hw(float x) { return __builtin_amdgcn_logf(x) * 0.693147180559945309f; }

// Per-cluster score term for one (head, query, cluster): the additive KL
// share p (l - l'), its magnitude, or the attention-weighted drift p * D.
__device__ __forceinline__ float score_term(int kind, float p, float t, float D)
{
    return kind == PS_SCORE_ATTN_WEIGHTED ? p * D : (kind == PS_SCORE_KL_SHARE_ABS ? fabsf(t) : t);
}

// ---------------------------------------------------------------------------
// proxy attention, bf16: z[k][i] = sigma * <Ck[k][g(h)], Q[i][h]> on MFMA
// 16x16x32, one workgroup per window, one head per wave at a time.
// Lane l holds clusters 16*mb + 4*(l/16) + r of query 16*nb + (l % 16).
// Clusters run in groups of 16*KB; with one group the log-softmax is done in
// registers and, given the previous step's distribution, the drift is fused
// into the epilogue: D_{h,i} by two lane shuffles, per-cluster scores
// accumulated per lane over the wave's heads and queries, then combined over
// queries (shuffles) and waves (LDS) in a fixed order.  With several groups a
// running max and sum are kept across groups, the raw logits are parked in
// the output row and rebased in a second pass by the lane that wrote them, and
// the drift runs as a separate pass (fused = 0).  With hsplit the grid has a
// second dimension over groups of four heads and every wave computes one head
// of its window; the per-cluster scores sum over all heads, so there the
// kernel stops at each row's drift D_{h,i} (fused = 2, written to D_hi) and
// k_drift_scores adds the scores up.
// ---------------------------------------------------------------------------
template <int KB, int NBQ>
__global__ __launch_bounds__(256) void k_proxy_bf16(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ Ck, float sigma,
                                                     float* __restrict__ logp, const float* __restrict__ prev,
                                                     int kind, int fused, float* __restrict__ D_hi,
                                                     float* __restrict__ D_i, float* __restrict__ score,
                                                     int Hq, int Hkv, int dh, int Nb, int K, int hsplit)
{
    constexpr int GK = 16 * KB;
    __shared__ float sred[4][GK];
    __shared__ float dred[4][16 * NBQ];
    const int w = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int G = Hq / Hkv;
    const int ngroups = (K + GK - 1) / GK;
    const bool vec = (K & 3) == 0;
    float sacc[KB][4];
    float dacc[NBQ];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) dacc[nb] = 0.0f;

    // the previous step's log-probabilities of this lane's (query, cluster)
    // pairs are requested with the head's operands (one memory wait per head
    // instead of two), where registers allow (up to 8 16x16 blocks of pairs
    // per lane); addresses clamped into the tensor, values outside masked
    // where used
    constexpr bool kEarlyPrev = KB * NBQ <= 8;
    const bool early = kEarlyPrev && fused && prev != nullptr && ngroups == 1;
    const int h0 = hsplit ? 4 * (int)blockIdx.y + wave : wave;
    const int hstep = hsplit ? Hq : 4;
    for (int h = h0; h < Hq; h += hstep) {
        const int g = h / G;
        float M[NBQ], S[NBQ];
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) { M[nb] = -INFINITY; S[nb] = 0.0f; }
        float ppre[kEarlyPrev ? NBQ : 1][kEarlyPrev ? KB : 1][4];
        if (kEarlyPrev && early) {
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
                const int i = min(16 * nb + r16, Nb - 1);
                const float* pr = prev + (((size_t)w * Hq + h) * Nb + i) * K;
#pragma unroll
                for (int mb = 0; mb < KB; ++mb) {
                    const int k0 = 16 * mb + 4 * q;
                    if (vec) {
                        const float4 v4 = *reinterpret_cast<const float4*>(pr + min(k0, K - 4));
                        ppre[nb][mb][0] = v4.x; ppre[nb][mb][1] = v4.y;
                        ppre[nb][mb][2] = v4.z; ppre[nb][mb][3] = v4.w;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r) ppre[nb][mb][r] = pr[min(k0 + r, K - 1)];
                    }
                }
            }
        }
        floatx4 acc[KB][NBQ];
        for (int cg = 0; cg < K; cg += GK) {
#pragma unroll
            for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                for (int nb = 0; nb < NBQ; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
            // up to U 32-wide k-steps per batch (fewer for wide cluster
            // groups, to stay in registers): all their loads are issued first,
            // unconditionally (addresses clamped into the tensors), and pieces
            // outside are zeroed where the MFMAs take them
            constexpr int U = KB <= 4 ? 4 : (KB <= 8 ? 2 : 1);
            for (int e0 = 0; e0 < dh; e0 += 32 * U) {
                uint4 bq[U][NBQ], av[U][KB];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int e = min(e0 + 32 * u + 8 * q, dh - 8);
#pragma unroll
                    for (int nb = 0; nb < NBQ; ++nb) {
                        const int i = min(16 * nb + r16, Nb - 1);
                        bq[u][nb] = *reinterpret_cast<const uint4*>(Q + (((size_t)w * Nb + i) * Hq + h) * dh + e);
                    }
#pragma unroll
                    for (int mb = 0; mb < KB; ++mb) {
                        const int kk = min(cg + 16 * mb + r16, K - 1);
                        av[u][mb] = *reinterpret_cast<const uint4*>(Ck + (((size_t)w * K + kk) * Hkv + g) * dh + e);
                    }
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (e0 + 32 * u >= dh) break;
                    const bool in_e = e0 + 32 * u + 8 * q < dh;
                    bf16x8 b[NBQ];
#pragma unroll
                    for (int nb = 0; nb < NBQ; ++nb)
                        b[nb] = __builtin_bit_cast(bf16x8, (in_e && 16 * nb + r16 < Nb) ? bq[u][nb]
                                                                                         : make_uint4(0, 0, 0, 0));
#pragma unroll
                    for (int mb = 0; mb < KB; ++mb) {
                        const bf16x8 a = __builtin_bit_cast(
                            bf16x8, (in_e && cg + 16 * mb + r16 < K) ? av[u][mb] : make_uint4(0, 0, 0, 0));
#pragma unroll
                        for (int nb = 0; nb < NBQ; ++nb)
                            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nb], acc[mb][nb], 0, 0, 0);
                    }
                }
            }
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) {
                const int i = 16 * nb + r16;
                float zmax = -INFINITY;
#pragma unroll
                for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = cg + 16 * mb + 4 * q + r;
                        const float z = acc[mb][nb][r] * sigma;
                        acc[mb][nb][r] = z;
                        if (kk < K) zmax = fmaxf(zmax, z);
                    }
                zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
                zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
                float se = 0.0f;
#pragma unroll
                for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int kk = cg + 16 * mb + 4 * q + r;
                        if (kk < K) se += exp_hw(acc[mb][nb][r] - zmax);
                    }
                se += __shfl_xor(se, 16, 64);
                se += __shfl_xor(se, 32, 64);
                const float Mn = fmaxf(M[nb], zmax);
                S[nb] = S[nb] * exp_hw(M[nb] - Mn) + se * exp_hw(zmax - Mn);
                M[nb] = Mn;
                if (ngroups > 1 && i < Nb) {
                    float* out = logp + (((size_t)w * Hq + h) * Nb + i) * K;
#pragma unroll
                    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int kk = cg + 16 * mb + 4 * q + r;
                            if (kk < K) out[kk] = acc[mb][nb][r];
                        }
                }
            }
        }
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const int i = 16 * nb + r16;
            const bool iv = i < Nb;
            const float lse = M[nb] + log_hw(S[nb]);
            const size_t row = (((size_t)w * Hq + h) * Nb + (iv ? i : 0)) * K;
            float* out = logp + row;
            if (ngroups == 1) {
                float lv[KB][4], pv[KB][4], tv[KB][4];
                float tsum = 0.0f;
#pragma unroll
                for (int mb = 0; mb < KB; ++mb) {
                    const int k0 = 16 * mb + 4 * q;
#pragma unroll
                    for (int r = 0; r < 4; ++r) lv[mb][r] = acc[mb][nb][r] - lse;
                    if (iv) {
                        if (vec && k0 + 3 < K) {
                            *reinterpret_cast<float4*>(out + k0) = make_float4(lv[mb][0], lv[mb][1], lv[mb][2], lv[mb][3]);
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r)
                                if (k0 + r < K) out[k0 + r] = lv[mb][r];
                        }
                    }
                    if (fused && prev) {
                        float pp[4] = {0.f, 0.f, 0.f, 0.f};
                        if (kEarlyPrev) {
#pragma unroll
                            for (int r = 0; r < 4; ++r) pp[r] = ppre[kEarlyPrev ? nb : 0][kEarlyPrev ? mb : 0][r];
                        } else if (iv) {
                            const float* pr = prev + row;
                            if (vec && k0 + 3 < K) {
                                const float4 v = *reinterpret_cast<const float4*>(pr + k0);
                                pp[0] = v.x; pp[1] = v.y; pp[2] = v.z; pp[3] = v.w;
                            } else {
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    if (k0 + r < K) pp[r] = pr[k0 + r];
                            }
                        }
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const bool ok = iv && k0 + r < K;
                            pv[mb][r] = ok ? exp_hw(lv[mb][r]) : 0.0f;
                            tv[mb][r] = ok ? pv[mb][r] * (lv[mb][r] - pp[r]) : 0.0f;
                            tsum += tv[mb][r];
                        }
                    }
                }
                if (fused) {
                    float D = 0.0f;
                    if (prev) {
                        D = tsum + __shfl_xor(tsum, 16, 64);
                        D = D + __shfl_xor(D, 32, 64);
                        if (fused == 1) {
#pragma unroll
                            for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                                for (int r = 0; r < 4; ++r)
                                    sacc[mb][r] += score_term(kind, pv[mb][r], tv[mb][r], D);
                        }
                    }
                    if (iv) {
                        dacc[nb] += D;
                        if (D_hi && q == 0) D_hi[((size_t)w * Hq + h) * Nb + i] = D;
                    }
                }
            } else if (iv) {
                for (int cg = 0; cg < K; cg += GK)
#pragma unroll
                    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int kk = cg + 16 * mb + 4 * q + r;
                            if (kk < K) out[kk] = out[kk] - lse;
                        }
            }
        }
    }
    if (fused != 1) return;
    // scores: sum over the 16 query lanes, then over the four waves in order
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = sacc[mb][r];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            if (r16 == 0) sred[wave][16 * mb + 4 * q + r] = v;
        }
    if (q == 0) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) dred[wave][16 * nb + r16] = dacc[nb];
    }
    __syncthreads();
    const float invH = 1.0f / (float)Hq;
    for (int k = threadIdx.x; k < K; k += 256)
        score[(size_t)w * K + k] = (((sred[0][k] + sred[1][k]) + sred[2][k]) + sred[3][k]) * invH;
    for (int i = threadIdx.x; i < Nb; i += 256)
        D_i[(size_t)w * Nb + i] = (((dred[0][i] + dred[1][i]) + dred[2][i]) + dred[3][i]) * invH;
}

// ---------------------------------------------------------------------------
// proxy attention above 64 clusters, head-parallel, for K = 16 KB and
// dh = 128: one wave per (window, head, block of 16 queries), four per
// workgroup, the query blocks of a head in neighbouring waves (the second
// wave's key rows come from L2).  The wave loads its 16 query rows whole
// (four 16-byte pieces per lane, all in flight at once), then streams the
// head's key rows 16 at a time, also whole, through a ring of P blocks in
// registers, so that P blocks are in flight while one block's 4 MFMAs run;
// at two waves per SIMD one wave's epilogue overlaps the other's stream.  The
// previous step's log-probabilities of the 16 queries are all requested
// before the softmax.  Every logit accumulates the same k-steps in the same
// order as in k_proxy_bf16, and the softmax, drift and D_{h,i} follow the
// same per-lane order, so the results are the same bit for bit.
// ---------------------------------------------------------------------------
template <int KB>
__global__ __launch_bounds__(256) void k_proxy_head(const uint16_t* __restrict__ Q,
                                                     const uint16_t* __restrict__ Ck, float sigma,
                                                     float* __restrict__ logp, const float* __restrict__ prev,
                                                     float* __restrict__ D_hi, int units, int Hq, int Hkv, int Nb,
                                                     int nqb)
{
    constexpr int DS = 4;                      // 32-wide k-steps of dh = 128
    constexpr int K = 16 * KB;
    constexpr int P = KB < 6 ? KB : 6;         // key blocks in flight
    const int lane = lane_id(), q = lane >> 4, r16 = lane & 15;
    const int unit = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6);
    if (unit >= units) return;
    const int pair = unit / nqb, qb = unit - pair * nqb;
    const int w = pair / Hq, h = pair - w * Hq, g = h / (Hq / Hkv);
    const int i = 16 * qb + r16;
    const bool iv = i < Nb;
    uint4 qv[DS];
    {
        const uint16_t* qr = Q + (((size_t)w * Nb + min(i, Nb - 1)) * Hq + h) * 128 + 8 * q;
#pragma unroll
        for (int u = 0; u < DS; ++u) qv[u] = *reinterpret_cast<const uint4*>(qr + 32 * u);
    }
    const uint16_t* kr = Ck + (((size_t)w * K + r16) * Hkv + g) * 128 + 8 * q;
    const size_t kblock = (size_t)16 * Hkv * 128;  // 16 key rows
    uint4 cv[P][DS];
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
        for (int u = 0; u < DS; ++u) cv[p][u] = *reinterpret_cast<const uint4*>(kr + p * kblock + 32 * u);
    if (!iv)
#pragma unroll
        for (int u = 0; u < DS; ++u) qv[u] = make_uint4(0, 0, 0, 0);
    floatx4 acc[KB];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb) {
        acc[mb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < DS; ++u)
            acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, cv[mb % P][u]),
                                                              __builtin_bit_cast(bf16x8, qv[u]), acc[mb], 0, 0, 0);
        if (mb + P < KB) {
#pragma unroll
            for (int u = 0; u < DS; ++u)
                cv[mb % P][u] = *reinterpret_cast<const uint4*>(kr + (mb + P) * kblock + 32 * u);
        }
    }
    const size_t row = (((size_t)w * Hq + h) * Nb + (iv ? i : Nb - 1)) * K;
    float4 pp[KB];
    if (prev) {
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) pp[mb] = *reinterpret_cast<const float4*>(prev + row + 16 * mb + 4 * q);
    }
    float zmax = -INFINITY;
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float z = acc[mb][r] * sigma;
            acc[mb][r] = z;
            zmax = fmaxf(zmax, z);
        }
    zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
    zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
    float se = 0.0f;
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) se += exp_hw(acc[mb][r] - zmax);
    se += __shfl_xor(se, 16, 64);
    se += __shfl_xor(se, 32, 64);
    // with a single group of clusters the running sum of k_proxy_bf16 is
    // se * 2^0 = se exactly, and its running max is zmax
    const float lse = zmax + log_hw(se);
    float* out = logp + row;
    float tsum = 0.0f;
#pragma unroll
    for (int mb = 0; mb < KB; ++mb) {
        float lv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) lv[r] = acc[mb][r] - lse;
        if (iv) *reinterpret_cast<float4*>(out + 16 * mb + 4 * q) = make_float4(lv[0], lv[1], lv[2], lv[3]);
        if (prev) {
            const float pq[4] = {pp[mb].x, pp[mb].y, pp[mb].z, pp[mb].w};
#pragma unroll
            for (int r = 0; r < 4; ++r) tsum += iv ? exp_hw(lv[r]) * (lv[r] - pq[r]) : 0.0f;
        }
    }
    if (prev) {
        float D = tsum + __shfl_xor(tsum, 16, 64);
        D = D + __shfl_xor(D, 32, 64);
        if (iv && D_hi && q == 0) D_hi[((size_t)w * Hq + h) * Nb + i] = D;
    }
}

// ---------------------------------------------------------------------------
// proxy attention, bf16, with the drift fused, software-pipelined over heads.
// For one cluster group (K <= 16*KB), dh <= 128 and a previous step, the
// same per-lane arithmetic as k_proxy_bf16 in the same order (identical
// results), but a wave requests its next head's operands and previous
// log-probabilities before it computes the current head, so every wave keeps
// one head's loads (about 32 KB) in flight while its MFMAs and softmax/KL
// epilogue run; in k_proxy_bf16 all waves load, wait, then compute together
// and the memory system idles during the epilogue.  Two heads' operands need
// about 256 registers, so the kernel runs one wave per SIMD.
// ---------------------------------------------------------------------------
template <int KB, int NBQ>
struct ProxyHeadOps {
    uint4 q[4][NBQ];       // Q rows 16*nb + (lane % 16), dh pieces 32*u + 8*(lane / 16)
    uint4 c[4][KB];        // centroid-key rows 16*mb + (lane % 16), same pieces
    float p[NBQ][KB][4];   // previous log-probabilities of the lane's (query, cluster) pairs
};

// Requests head h's operands (K a multiple of 4: whole float4s of the previous
// log-probabilities); every address clamped into its tensor, pieces and
// pairs outside the shape masked where they are used.
template <int KB, int NBQ>
__device__ __forceinline__ void proxy_head_load(ProxyHeadOps<KB, NBQ>& o, const uint16_t* __restrict__ Q,
                                                const uint16_t* __restrict__ Ck, const float* __restrict__ prev,
                                                int w, int h, int g, int q, int r16, int Hq, int Hkv, int dh,
                                                int Nb, int K)
{
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = min(32 * u + 8 * q, dh - 8);
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const int i = min(16 * nb + r16, Nb - 1);
            o.q[u][nb] = *reinterpret_cast<const uint4*>(Q + (((size_t)w * Nb + i) * Hq + h) * dh + e);
        }
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            const int kk = min(16 * mb + r16, K - 1);
            o.c[u][mb] = *reinterpret_cast<const uint4*>(Ck + (((size_t)w * K + kk) * Hkv + g) * dh + e);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const int i = min(16 * nb + r16, Nb - 1);
        const float* pr = prev + (((size_t)w * Hq + h) * Nb + i) * K;
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            const float4 v4 = *reinterpret_cast<const float4*>(pr + min(16 * mb + 4 * q, K - 4));
            o.p[nb][mb][0] = v4.x; o.p[nb][mb][1] = v4.y;
            o.p[nb][mb][2] = v4.z; o.p[nb][mb][3] = v4.w;
        }
    }
}

// One head from loaded operands: scores on MFMA, log-softmax over the K
// clusters, log-probabilities stored, D_{h,i} and the per-lane score terms.
template <int KB, int NBQ>
__device__ __forceinline__ void proxy_head_compute(const ProxyHeadOps<KB, NBQ>& o, float sigma,
                                                   float* __restrict__ logp, int kind, float* __restrict__ D_hi,
                                                   float (&sacc)[KB][4], float (&dacc)[NBQ], int w, int h,
                                                   int q, int r16, int Hq, int dh, int Nb, int K)
{
    floatx4 acc[KB][NBQ];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        if (32 * u >= dh) break;
        const bool in_e = 32 * u + 8 * q < dh;
        bf16x8 b[NBQ];
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb)
            b[nb] = __builtin_bit_cast(bf16x8, (in_e && 16 * nb + r16 < Nb) ? o.q[u][nb] : make_uint4(0, 0, 0, 0));
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, (in_e && 16 * mb + r16 < K) ? o.c[u][mb] : make_uint4(0, 0, 0, 0));
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nb], acc[mb][nb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const int i = 16 * nb + r16;
        const bool iv = i < Nb;
        // the log-sum-exp exactly as k_proxy_bf16 forms it for one group
        float zmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < KB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = acc[mb][nb][r] * sigma;
                acc[mb][nb][r] = z;
                if (16 * mb + 4 * q + r < K) zmax = fmaxf(zmax, z);
            }
        zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
        zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
        float se = 0.0f;
#pragma unroll
        for (int mb = 0; mb < KB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (16 * mb + 4 * q + r < K) se += exp_hw(acc[mb][nb][r] - zmax);
        se += __shfl_xor(se, 16, 64);
        se += __shfl_xor(se, 32, 64);
        const float lse = zmax + log_hw(se);
        float* out = logp + (((size_t)w * Hq + h) * Nb + (iv ? i : 0)) * K;
        float pv[KB][4], tv[KB][4];
        float tsum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < KB; ++mb) {
            const int k0 = 16 * mb + 4 * q;
            float lv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) lv[r] = acc[mb][nb][r] - lse;
            if (iv) {
                if (k0 < K) *reinterpret_cast<float4*>(out + k0) = make_float4(lv[0], lv[1], lv[2], lv[3]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool ok = iv && k0 + r < K;
                pv[mb][r] = ok ? exp_hw(lv[r]) : 0.0f;
                tv[mb][r] = ok ? pv[mb][r] * (lv[r] - o.p[nb][mb][r]) : 0.0f;
                tsum += tv[mb][r];
            }
        }
        float D = tsum + __shfl_xor(tsum, 16, 64);
        D = D + __shfl_xor(D, 32, 64);
#pragma unroll
        for (int mb = 0; mb < KB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[mb][r] += score_term(kind, pv[mb][r], tv[mb][r], D);
        if (iv) {
            dacc[nb] += D;
            if (D_hi && q == 0) D_hi[((size_t)w * Hq + h) * Nb + i] = D;
        }
    }
}

template <int KB, int NBQ>
__global__ __launch_bounds__(256, 1) void k_proxy_pipe(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ Ck, float sigma,
                                                        float* __restrict__ logp, const float* __restrict__ prev,
                                                        int kind, float* __restrict__ D_hi, float* __restrict__ D_i,
                                                        float* __restrict__ score, int Hq, int Hkv, int dh, int Nb,
                                                        int K)
{
    __shared__ float sred[4][16 * KB];
    __shared__ float dred[4][16 * NBQ];
    const int w = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int G = Hq / Hkv;
    float sacc[KB][4];
    float dacc[NBQ];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) dacc[nb] = 0.0f;
    // the wave's heads are wave, wave + 4, ...; loads past the last head are
    // clamped to it (issued so that every trip requests the same loads) and
    // never used
    ProxyHeadOps<KB, NBQ> A, B;
    int hl = min(wave, Hq - 1);
    proxy_head_load(A, Q, Ck, prev, w, hl, hl / G, q, r16, Hq, Hkv, dh, Nb, K);
    for (int h = wave; h < Hq; h += 8) {
        hl = min(h + 4, Hq - 1);
        proxy_head_load(B, Q, Ck, prev, w, hl, hl / G, q, r16, Hq, Hkv, dh, Nb, K);
        proxy_head_compute(A, sigma, logp, kind, D_hi, sacc, dacc, w, h, q, r16, Hq, dh, Nb, K);
        if (h + 4 >= Hq) break;
        hl = min(h + 8, Hq - 1);
        proxy_head_load(A, Q, Ck, prev, w, hl, hl / G, q, r16, Hq, Hkv, dh, Nb, K);
        proxy_head_compute(B, sigma, logp, kind, D_hi, sacc, dacc, w, h + 4, q, r16, Hq, dh, Nb, K);
    }
    // scores: sum over the 16 query lanes, then over the four waves in order
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = sacc[mb][r];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            if (r16 == 0) sred[wave][16 * mb + 4 * q + r] = v;
        }
    if (q == 0) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) dred[wave][16 * nb + r16] = dacc[nb];
    }
    __syncthreads();
    const float invH = 1.0f / (float)Hq;
    for (int k = threadIdx.x; k < K; k += 256)
        score[(size_t)w * K + k] = (((sred[0][k] + sred[1][k]) + sred[2][k]) + sred[3][k]) * invH;
    for (int i = threadIdx.x; i < Nb; i += 256)
        D_i[(size_t)w * Nb + i] = (((dred[0][i] + dred[1][i]) + dred[2][i]) + dred[3][i]) * invH;
}

// ---------------------------------------------------------------------------
// proxy attention, bf16, drift fused, for K = 64 clusters and dh = 128 (every
// operand row 256 bytes), whole rows per load.  The MFMA fragment layout
// makes each load instruction of k_proxy_pipe read 16 rows x 64 bytes, half
// of every 128-byte line it touches, which measured at about two thirds of
// the per-CU load rate of whole lines.  Here a load instruction reads 4 rows
// x 256 bytes (lane l: row 4 j + l / 16, 16-byte piece l % 16) into
// registers, one head ahead as in k_proxy_pipe; the wave stores the pieces
// into its own LDS tiles (Q, centroid keys, previous log-probabilities),
// piece p of row r at slot p ^ (r % 16), and reads the MFMA fragments and the
// epilogue's previous values back from there: the sixteen rows one fragment
// read touches fall on sixteen distinct 16-byte slots, so no bank conflicts.
// Two waves per workgroup (32 KB of LDS each); a wave's heads are wave,
// wave + 2, ...; results bit-identical to k_proxy_bf16's.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int NBQ>
struct ProxyRowOps {
    u32x4 q[4 * NBQ];   // Q rows 4 j + lane / 16, piece lane % 16
    u32x4 c[16];        // centroid-key rows 4 j + lane / 16
    u32x4 p[4 * NBQ];   // previous log-probability rows 4 j + lane / 16 (four floats a piece)
};

constexpr int kRowTileQ = 0;            // byte offsets in a wave's 32 KB of LDS
constexpr int kRowTileC = 32 * 256;
constexpr int kRowTileP = 96 * 256;
constexpr int kRowTileBytes = 128 * 256;

template <int NBQ>
__device__ __forceinline__ void proxy_rows_load(ProxyRowOps<NBQ>& o, const uint16_t* __restrict__ Q,
                                                const uint16_t* __restrict__ Ck, const float* __restrict__ prev,
                                                int w, int h, int g, int lane, int Hq, int Hkv, int Nb)
{
    const int rr = lane >> 4, pc = lane & 15;
#pragma unroll
    for (int j = 0; j < 4 * NBQ; ++j) {
        const int i = min(4 * j + rr, Nb - 1);
        o.q[j] = *reinterpret_cast<const u32x4*>(Q + (((size_t)w * Nb + i) * Hq + h) * 128 + 8 * pc);
    }
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const int k = 4 * j + rr;
        o.c[j] = *reinterpret_cast<const u32x4*>(Ck + (((size_t)w * 64 + k) * Hkv + g) * 128 + 8 * pc);
    }
#pragma unroll
    for (int j = 0; j < 4 * NBQ; ++j) {
        const int i = min(4 * j + rr, Nb - 1);
        o.p[j] = *reinterpret_cast<const u32x4*>(prev + (((size_t)w * Hq + h) * Nb + i) * 64 + 4 * pc);
    }
}

template <int NBQ>
__device__ __forceinline__ void proxy_rows_compute(const ProxyRowOps<NBQ>& o, uint8_t* __restrict__ tile,
                                                   float sigma, float* __restrict__ logp, int kind,
                                                   float* __restrict__ D_hi, float (&sacc)[4][4],
                                                   float (&dacc)[NBQ], int w, int h, int lane, int Hq, int Nb)
{
    const int rr = lane >> 4, pc = lane & 15;
    const int q = lane >> 4, r16 = lane & 15;
    // whole rows into the wave's tiles: row r = 4 j + rr has r % 16 = 4 (j % 4) + rr
#pragma unroll
    for (int j = 0; j < 4 * NBQ; ++j) {
        const int off = (4 * j + rr) * 256 + 16 * (pc ^ (4 * (j & 3) + rr));
        *reinterpret_cast<u32x4*>(tile + kRowTileQ + off) = o.q[j];
        *reinterpret_cast<u32x4*>(tile + kRowTileP + off) = o.p[j];
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
        *reinterpret_cast<u32x4*>(tile + kRowTileC + (4 * j + rr) * 256 + 16 * (pc ^ (4 * (j & 3) + rr))) = o.c[j];
    floatx4 acc[4][NBQ];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) acc[mb][nb] = floatx4{0.f, 0.f, 0.f, 0.f};
    // fragment reads: row 16 x + r16, piece 4 u + q at slot (4 u + q) ^ r16
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int so = 16 * ((4 * u + q) ^ r16);
        bf16x8 b[NBQ];
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const uint4 v = *reinterpret_cast<const uint4*>(tile + kRowTileQ + (16 * nb + r16) * 256 + so);
            b[nb] = __builtin_bit_cast(bf16x8, 16 * nb + r16 < Nb ? v : make_uint4(0, 0, 0, 0));
        }
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const bf16x8 a =
                __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(tile + kRowTileC + (16 * mb + r16) * 256 + so));
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb)
                acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[nb], acc[mb][nb], 0, 0, 0);
        }
    }
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) {
        const int i = 16 * nb + r16;
        const bool iv = i < Nb;
        float zmax = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float z = acc[mb][nb][r] * sigma;
                acc[mb][nb][r] = z;
                zmax = fmaxf(zmax, z);
            }
        zmax = fmaxf(zmax, __shfl_xor(zmax, 16, 64));
        zmax = fmaxf(zmax, __shfl_xor(zmax, 32, 64));
        float se = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) se += exp_hw(acc[mb][nb][r] - zmax);
        se += __shfl_xor(se, 16, 64);
        se += __shfl_xor(se, 32, 64);
        const float lse = zmax + log_hw(se);
        float* out = logp + (((size_t)w * Hq + h) * Nb + (iv ? i : 0)) * 64;
        float pv[4][4], tv[4][4];
        float tsum = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int k0 = 16 * mb + 4 * q;
            const float4 pp = *reinterpret_cast<const float4*>(tile + kRowTileP + i * 256 + 16 * ((4 * mb + q) ^ r16));
            const float ppv[4] = {pp.x, pp.y, pp.z, pp.w};
            float lv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) lv[r] = acc[mb][nb][r] - lse;
            if (iv) *reinterpret_cast<float4*>(out + k0) = make_float4(lv[0], lv[1], lv[2], lv[3]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                pv[mb][r] = iv ? exp_hw(lv[r]) : 0.0f;
                tv[mb][r] = iv ? pv[mb][r] * (lv[r] - ppv[r]) : 0.0f;
                tsum += tv[mb][r];
            }
        }
        float D = tsum + __shfl_xor(tsum, 16, 64);
        D = D + __shfl_xor(D, 32, 64);
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[mb][r] += score_term(kind, pv[mb][r], tv[mb][r], D);
        if (iv) {
            dacc[nb] += D;
            if (D_hi && q == 0) D_hi[((size_t)w * Hq + h) * Nb + i] = D;
        }
    }
}

template <int NBQ>
__global__ __launch_bounds__(128, 1) void k_proxy_rows(const uint16_t* __restrict__ Q,
                                                        const uint16_t* __restrict__ Ck, float sigma,
                                                        float* __restrict__ logp, const float* __restrict__ prev,
                                                        int kind, float* __restrict__ D_hi, float* __restrict__ D_i,
                                                        float* __restrict__ score, int Hq, int Hkv, int Nb)
{
    __shared__ __attribute__((aligned(16))) uint8_t tiles[2][kRowTileBytes];
    const int w = blockIdx.x;
    const int lane = lane_id(), wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    const int G = Hq / Hkv;
    uint8_t* const tile = tiles[wave];
    // per-lane partial sums in four streams, heads h % 4 = 0..3 (this wave
    // keeps streams wave and wave + 2), combined in stream order at the end:
    // the same additions in the same order as the four-wave kernels, so a
    // window's results do not depend on which kernel the launch size picks
    float sacc[2][4][4];
    float dacc[2][NBQ];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sacc[t][mb][r] = 0.0f;
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) dacc[t][nb] = 0.0f;
    }
    // loads past the wave's last head are clamped to it and never used
    ProxyRowOps<NBQ> A, B;
    int hl = min(wave, Hq - 1);
    proxy_rows_load(A, Q, Ck, prev, w, hl, hl / G, lane, Hq, Hkv, Nb);
    for (int h = wave; h < Hq; h += 4) {
        hl = min(h + 2, Hq - 1);
        proxy_rows_load(B, Q, Ck, prev, w, hl, hl / G, lane, Hq, Hkv, Nb);
        proxy_rows_compute(A, tile, sigma, logp, kind, D_hi, sacc[0], dacc[0], w, h, lane, Hq, Nb);
        if (h + 2 >= Hq) break;
        hl = min(h + 4, Hq - 1);
        proxy_rows_load(A, Q, Ck, prev, w, hl, hl / G, lane, Hq, Hkv, Nb);
        proxy_rows_compute(B, tile, sigma, logp, kind, D_hi, sacc[1], dacc[1], w, h + 2, lane, Hq, Nb);
    }
    // scores: sum over the 16 query lanes, then over the four streams in
    // order; a wave's partials go to the start of its own tile, which it no
    // longer reads: [stream wave: 64 scores, 32 drifts][stream wave + 2: ...]
    float* const red = reinterpret_cast<float*>(tile);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int mb = 0; mb < 4; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float v = sacc[t][mb][r];
                v += __shfl_xor(v, 1, 64);
                v += __shfl_xor(v, 2, 64);
                v += __shfl_xor(v, 4, 64);
                v += __shfl_xor(v, 8, 64);
                if (r16 == 0) red[96 * t + 16 * mb + 4 * q + r] = v;
            }
        if (q == 0) {
#pragma unroll
            for (int nb = 0; nb < NBQ; ++nb) red[96 * t + 64 + 16 * nb + r16] = dacc[t][nb];
        }
    }
    __syncthreads();
    // stream v is wave v % 2's partial set v / 2
    const float* s0 = reinterpret_cast<const float*>(tiles[0]);
    const float* s1 = reinterpret_cast<const float*>(tiles[1]);
    const float* s2 = s0 + 96;
    const float* s3 = s1 + 96;
    const float invH = 1.0f / (float)Hq;
    for (int k = threadIdx.x; k < 64; k += 128)
        score[(size_t)w * 64 + k] = (((s0[k] + s1[k]) + s2[k]) + s3[k]) * invH;
    for (int i = threadIdx.x; i < Nb; i += 128)
        D_i[(size_t)w * Nb + i] = (((s0[64 + i] + s1[64 + i]) + s2[64 + i]) + s3[64 + i]) * invH;
}

// proxy attention, fp32 path: one thread per (h, i), three passes over K
__global__ __launch_bounds__(256) void k_proxy_f32(const float* __restrict__ Q, const float* __restrict__ Ck,
                                                    float sigma, float* __restrict__ logp, int Hq, int Hkv,
                                                    int dh, int Nb, int K)
{
    const int w = blockIdx.y;
    const int pair = blockIdx.x * 256 + threadIdx.x;
    if (pair >= Hq * Nb) return;
    const int h = pair / Nb, i = pair - h * Nb;
    const int g = h / (Hq / Hkv);
    const float* qv = Q + (((size_t)w * Nb + i) * Hq + h) * dh;
    auto zk = [&](int k) {
        const float* kv = Ck + (((size_t)w * K + k) * Hkv + g) * dh;
        float s = 0.0f;
        for (int e = 0; e < dh; ++e) s = fmaf(qv[e], kv[e], s);
        return s * sigma;
    };
    float zmax = -INFINITY;
    for (int k = 0; k < K; ++k) zmax = fmaxf(zmax, zk(k));
    float se = 0.0f;
    for (int k = 0; k < K; ++k) se += exp_hw(zk(k) - zmax);
    const float lse = zmax + log_hw(se);
    float* out = logp + (((size_t)w * Hq + h) * Nb + i) * K;
    for (int k = 0; k < K; ++k) out[k] = zk(k) - lse;
}

// ---------------------------------------------------------------------------
// drift from stored distributions, one workgroup per window, one pass: a wave
// takes a (head, query) row at a time, lane l the clusters l, l+64, ...; each
// term is computed once, D by a wave reduction, the per-cluster scores
// accumulated per lane and combined over the waves in order.
// ---------------------------------------------------------------------------
template <int KM>
__global__ __launch_bounds__(256) void k_drift_kl(const float* __restrict__ cur, const float* __restrict__ prev,
                                                   int kind, float* __restrict__ D_hi, float* __restrict__ D_i,
                                                   float* __restrict__ score, int Hq, int Nb, int K)
{
    extern __shared__ float dsh[];  // Hq * Nb drift values, then 4 * K score partials
    float* sp = dsh + Hq * Nb;
    const int w = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6;
    const size_t base = (size_t)w * Hq * Nb * K;
    float sacc[KM];
#pragma unroll
    for (int m = 0; m < KM; ++m) sacc[m] = 0.0f;
    for (int pr = wave; pr < Hq * Nb; pr += 4) {
        const float* lc = cur + base + (size_t)pr * K;
        const float* lp = prev + base + (size_t)pr * K;
        float pv[KM], tv[KM];
        float part = 0.0f;
#pragma unroll
        for (int m = 0; m < KM; ++m) {
            const int k = lane + 64 * m;
            pv[m] = tv[m] = 0.0f;
            if (k < K) {
                const float l = lc[k];
                pv[m] = exp_hw(l);
                tv[m] = pv[m] * (l - lp[k]);
            }
            part += tv[m];
        }
        const float D = wave_sum(part);
#pragma unroll
        for (int m = 0; m < KM; ++m) sacc[m] += score_term(kind, pv[m], tv[m], D);
        if (lane == 0) {
            dsh[pr] = D;
            if (D_hi) D_hi[(size_t)w * Hq * Nb + pr] = D;
        }
    }
#pragma unroll
    for (int m = 0; m < KM; ++m) {
        const int k = lane + 64 * m;
        if (k < K) sp[wave * K + k] = sacc[m];
    }
    __syncthreads();
    const float invH = 1.0f / (float)Hq;
    for (int i = threadIdx.x; i < Nb; i += 256) {
        float s = 0.0f;
        for (int h = 0; h < Hq; ++h) s += dsh[h * Nb + i];
        D_i[(size_t)w * Nb + i] = s * invH;
    }
    for (int k = threadIdx.x; k < K; k += 256)
        score[(size_t)w * K + k] = (((sp[k] + sp[K + k]) + sp[2 * K + k]) + sp[3 * K + k]) * invH;
}

// ---------------------------------------------------------------------------
// per-cluster scores and per-token drift in the fused kernels' order, from the
// stored distributions and the per-row drifts D_hi: one four-wave workgroup
// per window at K = 16 KB clusters.  Wave v takes heads v, v + 4, ... in
// order (the fused kernels' head streams), lane l the clusters
// 16 mb + 4 (l / 16) + r of queries 16 nb + (l % 16), and adds, head by head
// and query block by query block, exactly the terms k_proxy_bf16 adds in
// registers (the same exponential of the same stored log-probability, the
// same product, the same drift D_{h,i}, zero terms for rows past Nb); then
// the same butterfly over the 16 query lanes and the same sum over the four
// waves.  So a window's scores and D_i do not depend on whether its
// log-probabilities came from the fused kernels or from k_proxy_head.  The
// next head's values are requested before the current head's terms.
// ---------------------------------------------------------------------------
template <int KB, int NBQ>
__global__ __launch_bounds__(256) void k_drift_scores_streams(const float* __restrict__ cur,
                                                               const float* __restrict__ prev,
                                                               const float* __restrict__ D_hi, int kind,
                                                               float* __restrict__ D_i, float* __restrict__ score,
                                                               int Hq, int Nb)
{
    constexpr int K = 16 * KB;
    __shared__ float sred[4][K];
    __shared__ float dred[4][16 * NBQ];
    const int w = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6;
    const int q = lane >> 4, r16 = lane & 15;
    float sacc[KB][4];
    float dacc[NBQ];
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) sacc[mb][r] = 0.0f;
#pragma unroll
    for (int nb = 0; nb < NBQ; ++nb) dacc[nb] = 0.0f;
    float4 lc[2][NBQ][KB], lp[2][NBQ][KB];
    float dv[2][NBQ];
    auto load = [&](int h, int b) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const int i = min(16 * nb + r16, Nb - 1);
            const size_t rowi = ((size_t)w * Hq + h) * Nb + i;
#pragma unroll
            for (int mb = 0; mb < KB; ++mb) {
                lc[b][nb][mb] = *reinterpret_cast<const float4*>(cur + rowi * K + 16 * mb + 4 * q);
                lp[b][nb][mb] = *reinterpret_cast<const float4*>(prev + rowi * K + 16 * mb + 4 * q);
            }
            dv[b][nb] = D_hi[rowi];
        }
    };
    auto add = [&](int b) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) {
            const bool iv = 16 * nb + r16 < Nb;
            const float D = iv ? dv[b][nb] : 0.0f;
#pragma unroll
            for (int mb = 0; mb < KB; ++mb) {
                const float lv[4] = {lc[b][nb][mb].x, lc[b][nb][mb].y, lc[b][nb][mb].z, lc[b][nb][mb].w};
                const float pq[4] = {lp[b][nb][mb].x, lp[b][nb][mb].y, lp[b][nb][mb].z, lp[b][nb][mb].w};
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float pv = iv ? exp_hw(lv[r]) : 0.0f;
                    const float tv = iv ? pv * (lv[r] - pq[r]) : 0.0f;
                    sacc[mb][r] += score_term(kind, pv, tv, D);
                }
            }
            if (iv) dacc[nb] += D;
        }
    };
    if (wave < Hq) load(wave, 0);
    for (int h = wave; h < Hq; h += 8) {
        if (h + 4 < Hq) load(h + 4, 1);
        add(0);
        if (h + 4 >= Hq) break;
        if (h + 8 < Hq) load(h + 8, 0);
        add(1);
    }
    // scores: sum over the 16 query lanes, then over the four waves in order
#pragma unroll
    for (int mb = 0; mb < KB; ++mb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float v = sacc[mb][r];
            v += __shfl_xor(v, 1, 64);
            v += __shfl_xor(v, 2, 64);
            v += __shfl_xor(v, 4, 64);
            v += __shfl_xor(v, 8, 64);
            if (r16 == 0) sred[wave][16 * mb + 4 * q + r] = v;
        }
    if (q == 0) {
#pragma unroll
        for (int nb = 0; nb < NBQ; ++nb) dred[wave][16 * nb + r16] = dacc[nb];
    }
    __syncthreads();
    const float invH = 1.0f / (float)Hq;
    for (int k = threadIdx.x; k < K; k += 256)
        score[(size_t)w * K + k] = (((sred[0][k] + sred[1][k]) + sred[2][k]) + sred[3][k]) * invH;
    for (int i = threadIdx.x; i < Nb; i += 256)
        D_i[(size_t)w * Nb + i] = (((dred[0][i] + dred[1][i]) + dred[2][i]) + dred[3][i]) * invH;
}

// ---------------------------------------------------------------------------
// per-cluster scores and per-token drift from stored distributions and the
// per-row drifts D_hi (which the head-parallel proxy kernel writes): grid
// (W, K / 64) of 16-wave workgroups, lane l of every wave owns cluster
// 64 blockIdx.y + l, wave v the rows (h, i) = v, v + 16, ... in order (8
// rows' loads in flight: 16 waves keep enough bytes in flight when a single
// window gives only K / 64 workgroups), the 16 waves' sums combined in order;
// blockIdx.y == 0 also averages D_hi over the heads for D_i.  The order of
// every sum depends on the shape only.
// ---------------------------------------------------------------------------
constexpr int kScoreWaves = 16;

__global__ __launch_bounds__(64 * kScoreWaves) void k_drift_scores(const float* __restrict__ cur,
                                                                    const float* __restrict__ prev,
                                                                    const float* __restrict__ D_hi, int kind,
                                                                    float* __restrict__ D_i,
                                                                    float* __restrict__ score, int Hq, int Nb,
                                                                    int K)
{
    constexpr int NW = kScoreWaves;
    __shared__ float part[NW][64];
    const int w = blockIdx.x, lane = lane_id(), wave = threadIdx.x >> 6;
    const int k = 64 * (int)blockIdx.y + lane;
    const bool kv = k < K;
    const int kc = kv ? k : K - 1;
    const int rows = Hq * Nb;
    const size_t base = (size_t)w * rows * K;
    const float* Dw = D_hi + (size_t)w * rows;
    float acc = 0.0f;
    constexpr int U = 8;
    for (int r0 = wave; r0 < rows; r0 += NW * U) {
        float lc[U], lp[U], dv[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int r = min(r0 + NW * u, rows - 1);
            lc[u] = cur[base + (size_t)r * K + kc];
            lp[u] = prev[base + (size_t)r * K + kc];
            dv[u] = Dw[r];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (r0 + NW * u >= rows) break;
            const float p = exp_hw(lc[u]);
            acc += score_term(kind, p, p * (lc[u] - lp[u]), dv[u]);
        }
    }
    part[wave][lane] = acc;
    __syncthreads();
    const float invH = 1.0f / (float)Hq;
    if (threadIdx.x < 64 && kv) {
        float sum = part[0][lane];
#pragma unroll
        for (int v = 1; v < NW; ++v) sum += part[v][lane];
        score[(size_t)w * K + k] = sum * invH;
    }
    if (blockIdx.y == 0) {
        for (int i = threadIdx.x; i < Nb; i += 64 * NW) {
            float sum = 0.0f;
            for (int h = 0; h < Hq; ++h) sum += Dw[h * Nb + i];
            D_i[(size_t)w * Nb + i] = sum * invH;
        }
    }
}

// Cosine-dissimilarity drift of each cluster: one wave per (window, cluster),
// 16-byte loads of both unit centres, products and sums in fp64 (each fp32
// product is exact in fp64), one wave reduction, then 1 - dot rounded once.
__global__ __launch_bounds__(256) void k_drift_cosine(const float* __restrict__ cur,
                                                      const float* __restrict__ prev, int d,
                                                      int64_t pairs, float* __restrict__ score)
{
    const int64_t p = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (p >= pairs) return;
    const int lane = lane_id();
    const float* a = cur + p * d;
    const float* b = prev + p * d;
    double dot = 0.0;
    for (int e = 4 * lane; e < d; e += 256) {          // d % 16 == 0: whole float4s
        const float4 x = *reinterpret_cast<const float4*>(a + e);
        const float4 y = *reinterpret_cast<const float4*>(b + e);
        dot = fma((double)x.x, (double)y.x, dot);
        dot = fma((double)x.y, (double)y.y, dot);
        dot = fma((double)x.z, (double)y.z, dot);
        dot = fma((double)x.w, (double)y.w, dot);
    }
    dot = wave_sum_d(dot);
    if (lane == 0) score[p] = (float)(1.0 - dot);
}

__global__ void k_zero(float* __restrict__ p, size_t n)
{
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0.0f;
}

// ---------------------------------------------------------------------------
// top-k: wave-level radix select on order-preserving 32-bit keys, one wave
// per window.  key(s): larger is better; NaN -> 0 (after every number);
// -0 -> +0.  Four 8-bit digit passes find the k-th largest key T; the result
// is every key > T plus the lowest-index keys == T, sorted by (key desc,
// index asc).
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t order_key(float f)
{
    if (f != f) return 0u;
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(64) void k_topk(const float* __restrict__ score, int K, int k,
                                              int32_t* __restrict__ idx, float* __restrict__ val)
{
    __shared__ uint32_t keys[kMaxK];
    __shared__ int hist[256];
    __shared__ uint64_t sel[kMaxTopK];
    const int w = blockIdx.x, lane = lane_id();
    const float* sw = score + (size_t)w * K;
    for (int c = lane; c < K; c += 64) keys[c] = order_key(sw[c]);
    uint32_t prefix = 0, pmask = 0;
    int kr = k;
    for (int pass = 0; pass < 4; ++pass) {
        const int shift = 24 - 8 * pass;
        for (int b = lane; b < 256; b += 64) hist[b] = 0;
        __syncthreads();
        for (int c = lane; c < K; c += 64) {
            const uint32_t key = keys[c];
            if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
        }
        __syncthreads();
        // lane l owns bins 4l..4l+3; suffix sums over lanes from the top
        int hb[4], own = 0;
#pragma unroll
        for (int t = 0; t < 4; ++t) { hb[t] = hist[4 * lane + t]; own += hb[t]; }
        int suf = own;  // inclusive suffix sum over lanes >= lane
#pragma unroll
        for (int s = 1; s < 64; s <<= 1) {
            const int o = __shfl_down(suf, s, 64);
            if (lane + s < 64) suf += o;
        }
        int cum = suf - own;  // count in bins above this lane's
        int found = -1, newkr = 0;
#pragma unroll
        for (int t = 3; t >= 0; --t) {
            if (found < 0 && cum < kr && cum + hb[t] >= kr) { found = 4 * lane + t; newkr = kr - cum; }
            cum += hb[t];
        }
        const uint64_t fb = __ballot(found >= 0);
        const int src = __ffsll((unsigned long long)fb) - 1;
        const int digit = __shfl(found, src, 64);
        kr = __shfl(newkr, src, 64);
        prefix |= (uint32_t)digit << shift;
        pmask |= 255u << shift;
        __syncthreads();
    }
    // collect: keys > T, then the first kr keys == T in ascending index
    const uint32_t T = prefix;
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    int ngt = 0, neq = 0;
    const int want_gt = k - kr;
    for (int base = 0; base < K; base += 64) {
        const int c = base + lane;
        const uint32_t key = c < K ? keys[c] : 0u;
        const bool gt = c < K && key > T;
        const bool eq = c < K && key == T;
        const uint64_t mg = __ballot(gt), me = __ballot(eq);
        const uint64_t comp = ((uint64_t)key << 32) | (uint32_t)(0xffffffffu - (uint32_t)c);
        if (gt) {
            const int r = ngt + __popcll(mg & lt);
            if (r < want_gt) sel[r] = comp;
        }
        if (eq) {
            const int r = neq + __popcll(me & lt);
            if (r < kr) sel[want_gt + r] = comp;
        }
        ngt += __popcll(mg);
        neq += __popcll(me);
    }
    __syncthreads();
    if (lane < k) {
        const uint64_t mine = sel[lane];
        int rank = 0;
        for (int t = 0; t < k; ++t) rank += sel[t] > mine;
        const int c = (int)(0xffffffffu - (uint32_t)(mine & 0xffffffffu));
        idx[(size_t)w * k + rank] = c;
        if (val) val[(size_t)w * k + rank] = sw[c];
    }
}

// compute units of the current device (cached per device; 256 if unknown)
int attn_device_cus()
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

// Drift-step proxy attention (a previous step given) takes the whole-row
// kernel at K = 64, dh = 128 when its two waves per window give every SIMD
// a wave (four per compute unit); with fewer windows, or other shapes whose
// operands fit, the four-wave pipelined kernel; otherwise k_proxy_bf16.
// Above 64 clusters every (window, head) gets its own wave and the drift
// follows in its own pass, whatever the number of windows: k_proxy_head (one
// wave per block of 16 queries) at K = 128 or 256 and dh = 128, otherwise
// k_proxy_bf16 with hsplit.
void enqueue_zero(float* p, size_t n, hipStream_t st);

template <int KB, int NBQ>
void launch_proxy(const ps_shape* s, const void* Q, const void* Ck, float sigma, float* logp, const float* prev,
                  int kind, int fused, float* D_hi, float* D_i, float* score, hipStream_t st)
{
    if constexpr (KB <= 4) {
        // a few windows (most compute units idle under one workgroup per
        // window): one wave per (window, head, 16 queries), then the scores
        // and D_i in the fused kernels' order from the rows' drifts, so the
        // results are those of the fused kernels bit for bit
        const int nqb = (s->Nb + 15) / 16;
        const int64_t units = (int64_t)s->W * s->Hq * nqb;
        if (fused == 1 && D_hi && s->K == 16 * KB && s->dh == 128 && 4 * (int64_t)s->W < attn_device_cus()) {
            PS_LAUNCH("k_proxy_head<KB>", (k_proxy_head<KB>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st,
                      (const uint16_t*)Q, (const uint16_t*)Ck, sigma, logp, prev, prev ? D_hi : nullptr, (int)units,
                      s->Hq, s->Hkv, s->Nb, nqb);
            if (prev) {
                PS_LAUNCH("k_drift_scores_streams<KB, NBQ>", (k_drift_scores_streams<KB, NBQ>), dim3(s->W), dim3(256),
                          0, st, logp, prev, D_hi, kind, D_i, score, s->Hq, s->Nb);
            } else {
                enqueue_zero(D_i, (size_t)s->W * s->Nb, st);
                enqueue_zero(score, (size_t)s->W * s->K, st);
                enqueue_zero(D_hi, (size_t)s->W * s->Hq * s->Nb, st);
            }
            return;
        }
    }
    if constexpr (KB > 4) {
        const int nqb = (s->Nb + 15) / 16;
        const int64_t units = (int64_t)s->W * s->Hq * nqb;
        if (fused != 1 && s->K == 16 * KB && s->dh == 128 && units <= INT32_MAX - 3) {
            PS_LAUNCH("k_proxy_head<KB>", (k_proxy_head<KB>), dim3((unsigned)((units + 3) / 4)), dim3(256), 0, st,
                      (const uint16_t*)Q, (const uint16_t*)Ck, sigma, logp, fused == 2 ? prev : nullptr,
                      fused == 2 ? D_hi : nullptr, (int)units, s->Hq, s->Hkv, s->Nb, nqb);
            return;
        }
    }
    if (fused != 1) {
        PS_LAUNCH("k_proxy_bf16<KB, NBQ>/heads", (k_proxy_bf16<KB, NBQ>), dim3(s->W, (s->Hq + 3) / 4), dim3(256), 0,
                  st, (const uint16_t*)Q, (const uint16_t*)Ck, sigma, logp, prev, kind, fused, D_hi, D_i, score,
                  s->Hq, s->Hkv, s->dh, s->Nb, s->K, 1);
        return;
    }
    if constexpr (KB == 4 && NBQ <= 2) {
        if (fused && prev && s->dh == 128 && s->K == 64 && 2 * (int64_t)s->W >= 4 * (int64_t)attn_device_cus()) {
            PS_LAUNCH("k_proxy_rows<NBQ>", k_proxy_rows<NBQ>, dim3(s->W), dim3(128), 0, st, (const uint16_t*)Q,
                      (const uint16_t*)Ck, sigma, logp, prev, kind, D_hi, D_i, score, s->Hq, s->Hkv, s->Nb);
            return;
        }
    }
    if constexpr (KB * NBQ <= 8) {
        if (fused && prev && s->dh <= 128 && s->K % 4 == 0) {
            PS_LAUNCH("k_proxy_pipe<KB, NBQ>", (k_proxy_pipe<KB, NBQ>), dim3(s->W), dim3(256), 0, st,
                      (const uint16_t*)Q, (const uint16_t*)Ck, sigma, logp, prev, kind, D_hi, D_i, score, s->Hq,
                      s->Hkv, s->dh, s->Nb, s->K);
            return;
        }
    }
    PS_LAUNCH("k_proxy_bf16<KB, NBQ>", (k_proxy_bf16<KB, NBQ>), dim3(s->W), dim3(256), 0, st, (const uint16_t*)Q,
              (const uint16_t*)Ck, sigma, logp, prev, kind, fused, D_hi, D_i, score, s->Hq, s->Hkv, s->dh, s->Nb,
              s->K, 0);
}

template <int KB>
void launch_proxy_nb(const ps_shape* s, const void* Q, const void* Ck, float sigma, float* logp, const float* prev,
                     int kind, int fused, float* D_hi, float* D_i, float* score, hipStream_t st)
{
    const int nbq = (s->Nb + 15) / 16;
    if (nbq <= 1)      launch_proxy<KB, 1>(s, Q, Ck, sigma, logp, prev, kind, fused, D_hi, D_i, score, st);
    else if (nbq <= 2) launch_proxy<KB, 2>(s, Q, Ck, sigma, logp, prev, kind, fused, D_hi, D_i, score, st);
    else               launch_proxy<KB, 4>(s, Q, Ck, sigma, logp, prev, kind, fused, D_hi, D_i, score, st);
}

ps_status check_drift_shape(const ps_shape* s)
{
    if (!s) return PS_ERR_NULL;
    if (s->W < 0 || s->Hq < 1 || s->Nb < 1 || s->K < 1 || s->K > kMaxK) return PS_ERR_SHAPE;
    if ((int64_t)s->Hq * s->Nb + 4 * (int64_t)s->K > 16384) return PS_ERR_SHAPE;
    return PS_OK;
}

template <int KM>
void launch_drift(const ps_shape* s, const float* cur, const float* prev, ps_score kind, float* D_hi, float* D_i,
                  float* score, hipStream_t st)
{
    const size_t shm = ((size_t)s->Hq * s->Nb + 4 * (size_t)s->K) * sizeof(float);
    PS_LAUNCH("k_drift_kl<KM>", (k_drift_kl<KM>), dim3(s->W), dim3(256), shm, st, cur, prev, (int)kind, D_hi, D_i,
              score, s->Hq, s->Nb, s->K);
}

void enqueue_drift(const ps_shape* s, const float* cur, const float* prev, ps_score kind, float* D_hi, float* D_i,
                   float* score, hipStream_t st)
{
    const int km = (s->K + 63) / 64;
    if (km <= 1)      launch_drift<1>(s, cur, prev, kind, D_hi, D_i, score, st);
    else if (km <= 2) launch_drift<2>(s, cur, prev, kind, D_hi, D_i, score, st);
    else if (km <= 4) launch_drift<4>(s, cur, prev, kind, D_hi, D_i, score, st);
    else if (km <= 8) launch_drift<8>(s, cur, prev, kind, D_hi, D_i, score, st);
    else              launch_drift<16>(s, cur, prev, kind, D_hi, D_i, score, st);
}

void enqueue_zero(float* p, size_t n, hipStream_t st)
{
    if (!p || n == 0) return;
    const int blocks = (int)std::min<size_t>((n + 255) / 256, 4096);
    PS_LAUNCH("k_zero", k_zero, dim3(blocks), dim3(256), 0, st, p, n);
}

}  // namespace

extern "C" ps_status ps_drift_kl(const ps_shape* s, const float* logp_cur, const float* logp_prev,
                                 ps_score kind, float* D_hi, float* D_i, float* score, void* stream)
{
    using namespace ps_host;
    if (!s || !logp_cur || !logp_prev || !D_i || !score) return PS_ERR_NULL;
    ps_status st = check_drift_shape(s);
    if (st != PS_OK) return st;
    if (kind < PS_SCORE_KL_SHARE || kind > PS_SCORE_ATTN_WEIGHTED) return PS_ERR_RANGE;
    if (!aligned16(logp_cur) || !aligned16(logp_prev) || !aligned16(D_i) || !aligned16(score) ||
        (D_hi && !aligned16(D_hi)))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    enqueue_drift(s, logp_cur, logp_prev, kind, D_hi, D_i, score, stm);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" ps_status ps_proxy_attn(const ps_shape* s, ps_dtype dtype, const void* Q, const void* Ck,
                                   float softmax_scale, float* logp_cur, const float* logp_prev,
                                   ps_score kind, float* D_hi, float* D_i, float* score, void* stream)
{
    using namespace ps_host;
    if (!s || !Q || !Ck || !logp_cur || !D_i || !score) return PS_ERR_NULL;
    if (!dtype_ok(dtype)) return PS_ERR_DTYPE;
    ps_status st = check_drift_shape(s);
    if (st != PS_OK) return st;
    if (s->Hkv < 1 || s->Hq % s->Hkv != 0 || s->dh < 8 || s->dh % 8 != 0) return PS_ERR_SHAPE;
    if (s->Nb > 64) return PS_ERR_SHAPE;
    if (kind < PS_SCORE_KL_SHARE || kind > PS_SCORE_ATTN_WEIGHTED) return PS_ERR_RANGE;
    if (logp_prev == logp_cur) return PS_ERR_RANGE;
    if (!aligned16(Q) || !aligned16(Ck) || !aligned16(logp_cur) || !aligned16(D_i) || !aligned16(score) ||
        (logp_prev && !aligned16(logp_prev)) || (D_hi && !aligned16(D_hi)))
        return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    bool fused = false, heads = false, rowdrift = false;
    if (dtype == PS_BF16) {
        const int kb = (s->K + 15) / 16;
        // Up to 64 clusters the drift is fused into one workgroup per window.
        // Above, the (window, head) pairs spread over the device, each wave
        // writing its rows' drifts to D_hi, and k_drift_scores adds up the
        // scores (the one-workgroup form leaves most compute units idle
        // there); without D_hi to hold the rows' drifts, the fused form up to
        // 256 clusters, and above 256 clusters (several cluster groups, whose
        // rows are finished only after all groups) a drift pass of its own.
        // These choices depend on the shape and on D_hi only, never on the
        // number of windows; below 65 clusters a few windows run head-parallel
        // with the fused form's score order (launch_proxy), bit-identical.
        heads = kb > 4 && (!logp_prev || D_hi || kb > 16);
        rowdrift = heads && logp_prev && kb <= 16;
        fused = !heads && kb <= 16;
        const int f = rowdrift ? 2 : (fused ? 1 : 0);
        const int k = (int)kind;
        if (kb <= 1)       launch_proxy_nb<1>(s, Q, Ck, softmax_scale, logp_cur, logp_prev, k, f, D_hi, D_i, score, stm);
        else if (kb <= 2)  launch_proxy_nb<2>(s, Q, Ck, softmax_scale, logp_cur, logp_prev, k, f, D_hi, D_i, score, stm);
        else if (kb <= 4)  launch_proxy_nb<4>(s, Q, Ck, softmax_scale, logp_cur, logp_prev, k, f, D_hi, D_i, score, stm);
        else if (kb <= 8)  launch_proxy_nb<8>(s, Q, Ck, softmax_scale, logp_cur, logp_prev, k, f, D_hi, D_i, score, stm);
        else               launch_proxy_nb<16>(s, Q, Ck, softmax_scale, logp_cur, logp_prev, k, f, D_hi, D_i, score, stm);
    } else {
        const int pairs = s->Hq * s->Nb;
        PS_LAUNCH("k_proxy_f32", k_proxy_f32, dim3((pairs + 255) / 256, s->W), dim3(256), 0, stm, (const float*)Q,
                  (const float*)Ck, softmax_scale, logp_cur, s->Hq, s->Hkv, s->dh, s->Nb, s->K);
    }
    if (!fused) {
        if (rowdrift) {
            PS_LAUNCH("k_drift_scores", k_drift_scores, dim3(s->W, (s->K + 63) / 64), dim3(64 * kScoreWaves), 0, stm, logp_cur,
                      logp_prev, D_hi, (int)kind, D_i, score, s->Hq, s->Nb, s->K);
        } else if (logp_prev) {
            enqueue_drift(s, logp_cur, logp_prev, kind, D_hi, D_i, score, stm);
        } else {
            enqueue_zero(D_i, (size_t)s->W * s->Nb, stm);
            enqueue_zero(score, (size_t)s->W * s->K, stm);
            enqueue_zero(D_hi, (size_t)s->W * s->Hq * s->Nb, stm);
        }
    }
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" ps_status ps_topk_clusters(const ps_shape* s, const float* score, int32_t k, int32_t* idx, float* val,
                                      void* stream)
{
    using namespace ps_host;
    if (!s || !score || !idx) return PS_ERR_NULL;
    if (s->W < 0 || s->K < 1 || s->K > kMaxK) return PS_ERR_SHAPE;
    if (k < 1 || k > s->K || k > kMaxTopK) return PS_ERR_RANGE;
    if (!aligned16(score) || !aligned16(idx) || (val && !aligned16(val))) return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    PS_LAUNCH("k_topk", k_topk, dim3(s->W), dim3(64), 0, stm, score, s->K, k, idx, val);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" ps_status ps_drift_cosine(const ps_shape* s, const float* C_cur, const float* C_prev,
                                     float* score, void* stream)
{
    using namespace ps_host;
    if (!s || !C_cur || !C_prev || !score) return PS_ERR_NULL;
    if (s->W < 0 || s->K < 1 || s->K > kMaxK || s->d < 16 || s->d % 16 != 0) return PS_ERR_SHAPE;
    if ((int64_t)s->K * s->d >= ((int64_t)1 << 31)) return PS_ERR_SHAPE;
    if (!aligned16(C_cur) || !aligned16(C_prev) || !aligned16(score)) return PS_ERR_ALIGN;
    if (s->W == 0) return PS_OK;
    const int64_t pairs = (int64_t)s->W * s->K;
    hipStream_t stm = (hipStream_t)stream;
    (void)hipGetLastError();
    PS_LAUNCH("k_drift_cosine", k_drift_cosine, dim3((unsigned)((pairs + 3) / 4)), dim3(256), 0, stm,
              C_cur, C_prev, s->d, pairs, score);
    return hipGetLastError() == hipSuccess ? PS_OK : PS_ERR_DEVICE;
}

extern "C" const char* ps_status_string(ps_status st)
{
    switch (st) {
    case PS_OK: return "PS_OK";
    case PS_ERR_NULL: return "PS_ERR_NULL: a required pointer is NULL";
    case PS_ERR_SHAPE: return "PS_ERR_SHAPE: a dimension is outside the supported limits";
    case PS_ERR_DTYPE: return "PS_ERR_DTYPE: unsupported element type";
    case PS_ERR_ALIGN: return "PS_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
    case PS_ERR_RANGE: return "PS_ERR_RANGE: a scalar argument is out of range";
    case PS_ERR_WORKSPACE: return "PS_ERR_WORKSPACE: workspace missing or too small";
    case PS_ERR_DEVICE: return "PS_ERR_DEVICE: a HIP launch or runtime call failed";
    case PS_ERR_MEMORY: return "PS_ERR_MEMORY: a buffer is neither device memory nor device-mapped pinned host memory";
    case PS_ERR_SCRATCH_LIMIT:
        return "PS_ERR_SCRATCH_LIMIT: the shape needs more K-Means scratch than the static scratch holds "
               "(PS_STATIC_SCRATCH_BYTES); use ps_kmeans_fit with a workspace";
    }
    return "unknown ps_status";
}
