/*
 * polestar_oracle.c -- CPU oracle for the Polestar-Cache drift-detection path.
 *
 * TEST INFRASTRUCTURE ONLY (see polestar_oracle.h).  Plain loops, one thread,
 * fp64 accumulation, no blocking or reordering beyond the definitions.
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC.
 *
 * Citations name the explainer pages of "Polestar: Drift-Aware Cache
 * Calibration and Token Commitment for Efficient Inference of Diffusion LLMs",
 * technical summary section 2.A (items: drift measurement, local window and
 * clustering, sparse updates).  Where the pages leave a step open, the reading
 * taken is stated next to the code.
 */
#include "polestar_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#define ERR_NULL  (-1)
#define ERR_SHAPE (-2)
#define ERR_DTYPE (-3)
#define ERR_RANGE (-5)

/* ------------------------------------------------------------------------- */
/* number formats                                                            */
/* ------------------------------------------------------------------------- */

float pso_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* bf16 keeps the top 16 bits of the fp32 pattern; round to nearest, ties to
 * the even result.  Adding 0x7fff plus the kept LSB carries into the kept part
 * exactly when the dropped half is above one half ulp, or equal to it with an
 * odd kept LSB. */
uint16_t pso_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

/* OCP 8-bit E4M3 ("FN": no infinities, 0x7f/0xff are NaN).  Exponent bias 7,
 * 3 mantissa bits, subnormals m * 2^-9, largest finite 448 = 0x7e. */
float pso_e4m3_decode(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0) v = ldexp((double)m, -9);
    else        v = ldexp((double)(8 + m), e - 10);
    return (float)(s ? -v : v);
}

/* Scale encoder: nearest finite E4M3 value by exhaustive search over the 127
 * non-negative finite codes, ties to the even code; values at or above 448
 * saturate to 448.  Negative, zero and NaN inputs give code 0. */
uint8_t pso_e4m3_encode(float x)
{
    if (!(x > 0.0f)) return 0;
    if (x >= 448.0f) return 0x7e;
    int best = 0;
    double bestd = (double)x;
    for (int c = 1; c <= 0x7e; ++c) {
        double dist = fabs((double)x - (double)pso_e4m3_decode((uint8_t)c));
        if (dist < bestd || (dist == bestd && (c & 1) == 0)) { best = c; bestd = dist; }
    }
    return (uint8_t)best;
}

/* FP4 E2M1 magnitudes indexed by the 3-bit code (exponent<<1 | mantissa). */
static const double e2m1_mag[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

float pso_e2m1_decode(uint8_t nib)
{
    double m = e2m1_mag[nib & 7];
    return (float)((nib & 8) ? -m : m);
}

/* Nearest E2M1 magnitude, ties to the even code, saturating at 6.  A result of
 * magnitude zero is always +0 (nibble 0x0). */
uint8_t pso_e2m1_encode(float v)
{
    double a = fabs((double)v);
    int best = 0;
    if (a >= 6.0) {
        best = 7;
    } else {
        double bestd = a;
        for (int i = 1; i < 8; ++i) {
            double dist = fabs(a - e2m1_mag[i]);
            if (dist < bestd || (dist == bestd && (i & 1) == 0)) { best = i; bestd = dist; }
        }
    }
    if (best == 0) return 0;
    return (uint8_t)((v < 0.0f ? 8 : 0) | best);
}

/* ------------------------------------------------------------------------- */
/* helpers                                                                   */
/* ------------------------------------------------------------------------- */

static float ld(const void* p, int dtype, size_t i)
{
    return dtype == PSO_BF16 ? pso_bf16_to_f32(((const uint16_t*)p)[i]) : ((const float*)p)[i];
}

static void st(void* p, int dtype, size_t i, float v)
{
    if (dtype == PSO_BF16) ((uint16_t*)p)[i] = pso_f32_to_bf16(v);
    else                   ((float*)p)[i] = v;
}

/* the value the assignment step multiplies with: bf16 rounding on the bf16 path */
static double centroid_operand(float c, int dtype)
{
    return dtype == PSO_BF16 ? (double)pso_bf16_to_f32(pso_f32_to_bf16(c)) : (double)c;
}

static int check_dtype(int dtype) { return dtype == PSO_F32 || dtype == PSO_BF16; }

static int check_window_shape(const pso_shape* s)
{
    if (s->W < 0 || s->N < 1 || s->d < 16 || s->d % 16 != 0) return 0;
    return 1;
}

static int check_cluster_shape(const pso_shape* s)
{
    return check_window_shape(s) && s->K >= 1 && s->K <= s->N;
}

static int check_head_shape(const pso_shape* s)
{
    return s->Hq >= 1 && s->Hkv >= 1 && s->Hq % s->Hkv == 0 && s->dh >= 1;
}

/* n_j = ||h_j||_2, fp64 sum of squares, rounded once to fp32 */
static float row_norm_one(const void* H, int dtype, size_t row_off, int d)
{
    double ss = 0.0;
    for (int e = 0; e < d; ++e) {
        double h = (double)ld(H, dtype, row_off + (size_t)e);
        ss += h * h;
    }
    return (float)sqrt(ss);
}

/* unit row x_j = h_j / n_j as an fp32 division; a zero row stays zero */
static float unit_elem(float h, float n) { return n > 0.0f ? h / n : 0.0f; }

/* ------------------------------------------------------------------------- */
/* O1 row norms -- spherical clustering works on unit-normalised hidden
 * states (Polestar 2.A/window: spherical K-Means).                           */
/* ------------------------------------------------------------------------- */
int pso_row_norms(const pso_shape* s, int dtype, const void* H, float* row_norm)
{
    if (!s || !H || !row_norm) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_window_shape(s)) return ERR_SHAPE;
    for (int w = 0; w < s->W; ++w)
        for (int j = 0; j < s->N; ++j) {
            size_t r = (size_t)w * s->N + j;
            row_norm[r] = row_norm_one(H, dtype, r * (size_t)s->d, s->d);
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O2 initialisation.  The pages name spherical K-Means but no seeding
 * (Polestar 2.A/window).  Readings: STRIDED c_k = x_{floor(kN/K)};
 * FARTHEST = farthest-first traversal under cosine similarity (Gonzalez 1985):
 * c_0 = x_0, then repeatedly the row least similar to every chosen centre.   */
/* ------------------------------------------------------------------------- */
static void init_window(const pso_shape* s, int dtype, const void* H, int init, int w, float* Cw)
{
    const int N = s->N, d = s->d, K = s->K;
    const size_t base = (size_t)w * N * d;
    if (init == PSO_INIT_STRIDED) {
        for (int k = 0; k < K; ++k) {
            int j = (int)(((int64_t)k * N) / K);
            size_t off = base + (size_t)j * d;
            float n = row_norm_one(H, dtype, off, d);
            for (int e = 0; e < d; ++e) Cw[(size_t)k * d + e] = unit_elem(ld(H, dtype, off + e), n);
        }
        return;
    }
    /* FARTHEST */
    float* X = (float*)malloc(sizeof(float) * (size_t)N * d);
    double* m = (double*)malloc(sizeof(double) * (size_t)N);
    char* zero = (char*)malloc((size_t)N);
    for (int j = 0; j < N; ++j) {
        size_t off = base + (size_t)j * d;
        float n = row_norm_one(H, dtype, off, d);
        zero[j] = !(n > 0.0f);
        for (int e = 0; e < d; ++e) X[(size_t)j * d + e] = unit_elem(ld(H, dtype, off + e), n);
    }
    int seed = 0;
    for (int k = 0; k < K; ++k) {
        if (k > 0) {
            /* least-similar non-zero row; ties -> lowest j */
            seed = -1;
            for (int j = 0; j < N; ++j) {
                if (zero[j]) continue;
                if (seed < 0 || m[j] < m[seed]) seed = j;
            }
            if (seed < 0) seed = 0;
        }
        for (int e = 0; e < d; ++e) Cw[(size_t)k * d + e] = X[(size_t)seed * d + e];
        for (int j = 0; j < N; ++j) {
            double dot = 0.0;
            for (int e = 0; e < d; ++e)
                dot += (double)X[(size_t)j * d + e] * (double)Cw[(size_t)k * d + e];
            if (k == 0 || dot > m[j]) m[j] = dot;
        }
    }
    free(X);
    free(m);
    free(zero);
}

int pso_kmeans_init(const pso_shape* s, int dtype, const void* H, int init, float* C)
{
    if (!s || !H || !C) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_cluster_shape(s)) return ERR_SHAPE;
    if (init != PSO_INIT_STRIDED && init != PSO_INIT_FARTHEST) return ERR_RANGE;
    for (int w = 0; w < s->W; ++w) init_window(s, dtype, H, init, w, C + (size_t)w * s->K * s->d);
    return 0;
}

/* The update step of one window: for every cluster, S_k = sum of the unit
 * rows of its members (fp64, each added as fma(h, 1/n_j, S) in ascending j),
 * c_k = S_k / ||S_k|| rounded to fp32; an empty cluster (or ||S_k|| = 0) keeps
 * its centre.  Returns sum_k ||S_k||.  S is scratch of d doubles. */
static double update_window(const pso_shape* s, int dtype, const void* H, int w, const float* rn,
                            const int32_t* aw, float* Cw, int32_t* nw, double* S)
{
    const int N = s->N, d = s->d, K = s->K;
    const size_t hb = (size_t)w * N * d;
    double obj = 0.0;
    for (int k = 0; k < K; ++k) {
        int cnt = 0;
        for (int e = 0; e < d; ++e) S[e] = 0.0;
        for (int j = 0; j < N; ++j) {
            if (aw[j] != k) continue;
            ++cnt;
            if (!(rn[j] > 0.0f)) continue;
            const double inv = 1.0 / (double)rn[j];
            for (int e = 0; e < d; ++e)
                S[e] = fma((double)ld(H, dtype, hb + (size_t)j * d + e), inv, S[e]);
        }
        nw[k] = cnt;
        double ss = 0.0;
        for (int e = 0; e < d; ++e) ss += S[e] * S[e];
        double nrm = sqrt(ss);
        obj += nrm;
        if (cnt > 0 && nrm > 0.0)
            for (int e = 0; e < d; ++e) Cw[(size_t)k * d + e] = (float)(S[e] / nrm);
    }
    return obj;
}

int pso_kmeans_update(const pso_shape* s, int dtype, const void* H, const float* row_norm,
                      const int32_t* assign, float* C, int32_t* counts, double* objective)
{
    if (!s || !H || !row_norm || !assign || !C || !counts) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_cluster_shape(s)) return ERR_SHAPE;
    for (size_t i = 0; i < (size_t)s->W * s->N; ++i)
        if (assign[i] < 0 || assign[i] >= s->K) return ERR_RANGE;
    double* S = (double*)malloc(sizeof(double) * (size_t)s->d);
    for (int w = 0; w < s->W; ++w) {
        double obj = update_window(s, dtype, H, w, row_norm + (size_t)w * s->N, assign + (size_t)w * s->N,
                                   C + (size_t)w * s->K * s->d, counts + (size_t)w * s->K, S);
        if (objective) objective[w] = obj;
    }
    free(S);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O3/O4 spherical K-Means (Dhillon & Modha 2001) on the window's hidden
 * states, then the centroid keys (Polestar 2.A/window: clustering;
 * 2.A/sparse: proxy attention runs against the cluster centres).
 *
 * One Lloyd iteration:
 *   assign  a_j = argmax_k <h_j, b(c_k)>   (b = bf16 rounding on the bf16
 *           path, identity on fp32; argmax is invariant to n_j > 0, so raw h)
 *   update  S_k = sum_{a_j = k} h_j / n_j in fp64, each term added as one
 *           fused multiply-add of h by the fp64 reciprocal of n_j, members in
 *           ascending j; c_k = S_k / ||S_k|| rounded to fp32;
 *           a cluster with no members (or ||S_k|| = 0) keeps its centre.
 * Returned assign is the last assignment, C the last update, so every c_k is
 * the normalised mean of its members.  objective = sum_k ||S_k||.
 * Centroid keys (reading: mean of member key rows per KV head, which equals
 * W_K applied to the mean hidden state for a linear, bias-free key map):
 *   Ck[k][g] = sum_{a_j=k} Kr[j][g] / n_k, fp64, rounded to fp32 then dtype;
 *   empty clusters keep the previous Ck.                                     */
/* ------------------------------------------------------------------------- */
int pso_kmeans_fit(const pso_shape* s, int dtype, const void* H, const void* Kr, int init,
                   int iters, float* C, int32_t* assign, int32_t* counts, float* row_norm,
                   void* Ck, double* objective)
{
    if (!s || !H || !C || !assign || !counts || !row_norm) return ERR_NULL;
    if ((Kr == NULL) != (Ck == NULL)) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_cluster_shape(s)) return ERR_SHAPE;
    if (Kr && !check_head_shape(s)) return ERR_SHAPE;
    if (iters < 1) return ERR_RANGE;
    if (init != PSO_INIT_GIVEN && init != PSO_INIT_STRIDED && init != PSO_INIT_FARTHEST)
        return ERR_RANGE;

    const int N = s->N, d = s->d, K = s->K;
    const int KV = Kr ? s->Hkv * s->dh : 0;
    double* S = (double*)malloc(sizeof(double) * (size_t)d);
    double* B = (double*)malloc(sizeof(double) * (size_t)K * d);
    double* acc = (double*)malloc(sizeof(double) * (size_t)(KV > 0 ? KV : 1));

    for (int w = 0; w < s->W; ++w) {
        const size_t hb = (size_t)w * N * d;
        float* Cw = C + (size_t)w * K * d;
        int32_t* aw = assign + (size_t)w * N;
        int32_t* nw = counts + (size_t)w * K;
        float* rn = row_norm + (size_t)w * N;

        if (init != PSO_INIT_GIVEN) init_window(s, dtype, H, init, w, Cw);
        for (int j = 0; j < N; ++j) rn[j] = row_norm_one(H, dtype, hb + (size_t)j * d, d);

        double obj = 0.0;
        for (int it = 0; it < iters; ++it) {
            /* assignment */
            for (size_t i = 0; i < (size_t)K * d; ++i) B[i] = centroid_operand(Cw[i], dtype);
            for (int j = 0; j < N; ++j) {
                int best = 0;
                double bests = 0.0;
                for (int e = 0; e < d; ++e) S[e] = (double)ld(H, dtype, hb + (size_t)j * d + e);
                for (int k = 0; k < K; ++k) {
                    double dot = 0.0;
                    for (int e = 0; e < d; ++e) dot += S[e] * B[(size_t)k * d + e];
                    if (k == 0 || dot > bests) { best = k; bests = dot; }
                }
                aw[j] = best;
            }
            /* update */
            obj = update_window(s, dtype, H, w, rn, aw, Cw, nw, S);
        }
        if (objective) objective[w] = obj;

        if (Kr) {
            const size_t kb = (size_t)w * N * KV;
            const size_t cb = (size_t)w * K * KV;
            for (int k = 0; k < K; ++k) {
                if (nw[k] == 0) continue;
                for (int i = 0; i < KV; ++i) acc[i] = 0.0;
                for (int j = 0; j < N; ++j) {
                    if (aw[j] != k) continue;
                    for (int i = 0; i < KV; ++i) acc[i] += (double)ld(Kr, dtype, kb + (size_t)j * KV + i);
                }
                for (int i = 0; i < KV; ++i)
                    st(Ck, dtype, cb + (size_t)k * KV + i, (float)(acc[i] / (double)nw[k]));
            }
        }
    }
    free(S);
    free(B);
    free(acc);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O5 NVFP4 residuals (Polestar 2.A/window: the residual of each hidden state
 * to its centre is stored in NVFP4).  The pages give no format details.
 * Reading: residual in unit space r = x_j - c_{a_j}; E2M1 elements, one E4M3
 * scale per 16 elements, one fp32 scale per row:
 *   A = max|r|, g = A / 2688 (2688 = 6 * 448, so the largest block scale
 *   lands on 448); per 16-block s_b = E4M3((A_b / 6) / g), eff = dec(s_b) * g;
 *   code = E2M1(r / eff), or 0 where eff = 0.  Every step is one fp32
 *   operation, correctly rounded.  Nibble 2i is the low half of byte i.       */
/* ------------------------------------------------------------------------- */
int pso_residual_nvfp4(const pso_shape* s, int dtype, const void* H, const float* row_norm,
                       const float* C, const int32_t* assign, uint8_t* codes, uint8_t* bscale,
                       float* rscale)
{
    if (!s || !H || !row_norm || !C || !assign || !codes || !bscale || !rscale) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_cluster_shape(s)) return ERR_SHAPE;
    const int N = s->N, d = s->d, K = s->K, nb = d / 16;
    float* r = (float*)malloc(sizeof(float) * (size_t)d);
    for (int w = 0; w < s->W; ++w) {
        for (int j = 0; j < N; ++j) {
            const size_t row = (size_t)w * N + j;
            int a = assign[row];
            if (a < 0 || a >= K) a = 0;
            const float* c = C + ((size_t)w * K + a) * d;
            const float n = row_norm[row];
            float A = 0.0f;
            for (int e = 0; e < d; ++e) {
                float x = unit_elem(ld(H, dtype, row * d + e), n);
                r[e] = x - c[e];
                float m = fabsf(r[e]);
                if (m > A) A = m;
            }
            uint8_t* cr = codes + row * (size_t)(d / 2);
            uint8_t* br = bscale + row * (size_t)nb;
            if (!(A > 0.0f)) {
                rscale[row] = 0.0f;
                memset(cr, 0, (size_t)d / 2);
                memset(br, 0, (size_t)nb);
                continue;
            }
            const float g = A / 2688.0f;
            rscale[row] = g;
            for (int b = 0; b < nb; ++b) {
                float Ab = 0.0f;
                for (int e = 16 * b; e < 16 * b + 16; ++e)
                    if (fabsf(r[e]) > Ab) Ab = fabsf(r[e]);
                float t = Ab / 6.0f;
                uint8_t sb = pso_e4m3_encode(t / g);
                br[b] = sb;
                float eff = pso_e4m3_decode(sb) * g;
                for (int e = 16 * b; e < 16 * b + 16; e += 2) {
                    uint8_t lo = 0, hi = 0;
                    if (eff != 0.0f) {
                        lo = pso_e2m1_encode(r[e] / eff);
                        hi = pso_e2m1_encode(r[e + 1] / eff);
                    }
                    cr[e / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        }
    }
    free(r);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O7 drift (Polestar 2.A/drift: D_i = KL(A_i^t || A_i^{t-1}) between a
 * token's attention distributions at consecutive steps).  Reading: A_i is the
 * proxy-attention distribution of block query i over the K centroid keys, per
 * head; D_i is the mean over heads.  The cluster score that the top-k ranks
 * (the pages say only "most drifted clusters") is, by default, each cluster's
 * additive share of the KL sum:  s_k = (1/Hq) sum_{h,i} p (l - l').
 *   ABS: |term|;  ATTN_WEIGHTED: p_{h,i,k} * D_{h,i}.                         */
/* ------------------------------------------------------------------------- */
int pso_drift_kl(const pso_shape* s, const float* logp_cur, const float* logp_prev,
                 int score_kind, float* D_hi, float* D_i, float* score)
{
    if (!s || !logp_cur || !logp_prev || !D_i || !score) return ERR_NULL;
    if (s->W < 0 || s->Hq < 1 || s->Nb < 0 || s->K < 1) return ERR_SHAPE;
    if (score_kind < PSO_SCORE_KL_SHARE || score_kind > PSO_SCORE_ATTN_WEIGHTED) return ERR_RANGE;
    const int Hq = s->Hq, Nb = s->Nb, K = s->K;
    double* sacc = (double*)malloc(sizeof(double) * (size_t)K);
    double* dacc = (double*)malloc(sizeof(double) * (size_t)(Nb > 0 ? Nb : 1));
    for (int w = 0; w < s->W; ++w) {
        for (int k = 0; k < K; ++k) sacc[k] = 0.0;
        for (int i = 0; i < Nb; ++i) dacc[i] = 0.0;
        for (int h = 0; h < Hq; ++h) {
            for (int i = 0; i < Nb; ++i) {
                const size_t o = (((size_t)w * Hq + h) * Nb + i) * K;
                double D = 0.0;
                for (int k = 0; k < K; ++k) {
                    double l = (double)logp_cur[o + k], lp = (double)logp_prev[o + k];
                    D += exp(l) * (l - lp);
                }
                for (int k = 0; k < K; ++k) {
                    double l = (double)logp_cur[o + k], lp = (double)logp_prev[o + k];
                    double p = exp(l), term = p * (l - lp);
                    if (score_kind == PSO_SCORE_KL_SHARE)          sacc[k] += term;
                    else if (score_kind == PSO_SCORE_KL_SHARE_ABS) sacc[k] += fabs(term);
                    else                                           sacc[k] += p * D;
                }
                if (D_hi) D_hi[((size_t)w * Hq + h) * Nb + i] = (float)D;
                dacc[i] += D;
            }
        }
        for (int i = 0; i < Nb; ++i) D_i[(size_t)w * Nb + i] = (float)(dacc[i] / (double)Hq);
        for (int k = 0; k < K; ++k) score[(size_t)w * K + k] = (float)(sacc[k] / (double)Hq);
    }
    free(sacc);
    free(dacc);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O6 proxy attention (Polestar 2.A/sparse: each step computes attention
 * against the cluster centres).  z_{h,i,k} = sigma <q_{i,h}, Ck_{k,g(h)}>,
 * l = z - logsumexp_k z.  Readings: sigma is the caller's softmax scale
 * (1/sqrt(dh) by default), no log-count bias, consecutive query heads share a
 * KV head: g(h) = floor(h / (Hq/Hkv)).  The drift of the stored (fp32) l
 * against logp_prev follows when logp_prev is given; at window formation
 * (no previous step) D and s are zero.                                        */
/* ------------------------------------------------------------------------- */
int pso_proxy_attn(const pso_shape* s, int dtype, const void* Q, const void* Ck,
                   float softmax_scale, float* logp_cur, const float* logp_prev, int score_kind,
                   float* D_hi, float* D_i, float* score)
{
    if (!s || !Q || !Ck || !logp_cur || !D_i || !score) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (s->W < 0 || s->Nb < 0 || s->K < 1 || !check_head_shape(s)) return ERR_SHAPE;
    if (score_kind < PSO_SCORE_KL_SHARE || score_kind > PSO_SCORE_ATTN_WEIGHTED) return ERR_RANGE;
    const int Hq = s->Hq, Hkv = s->Hkv, dh = s->dh, Nb = s->Nb, K = s->K;
    const int G = Hq / Hkv;
    const double sigma = (double)softmax_scale;
    double* z = (double*)malloc(sizeof(double) * (size_t)K);
    for (int w = 0; w < s->W; ++w) {
        for (int h = 0; h < Hq; ++h) {
            const int g = h / G;
            for (int i = 0; i < Nb; ++i) {
                const size_t qo = (((size_t)w * Nb + i) * Hq + h) * dh;
                double zmax = 0.0;
                for (int k = 0; k < K; ++k) {
                    const size_t ko = (((size_t)w * K + k) * Hkv + g) * dh;
                    double dot = 0.0;
                    for (int e = 0; e < dh; ++e)
                        dot += (double)ld(Q, dtype, qo + e) * (double)ld(Ck, dtype, ko + e);
                    z[k] = sigma * dot;
                    if (k == 0 || z[k] > zmax) zmax = z[k];
                }
                double se = 0.0;
                for (int k = 0; k < K; ++k) se += exp(z[k] - zmax);
                const double lse = zmax + log(se);
                const size_t lo = (((size_t)w * Hq + h) * Nb + i) * K;
                for (int k = 0; k < K; ++k) logp_cur[lo + k] = (float)(z[k] - lse);
            }
        }
    }
    free(z);
    if (logp_prev) return pso_drift_kl(s, logp_cur, logp_prev, score_kind, D_hi, D_i, score);
    for (size_t i = 0; i < (size_t)s->W * Nb; ++i) D_i[i] = 0.0f;
    for (size_t i = 0; i < (size_t)s->W * K; ++i) score[i] = 0.0f;
    if (D_hi)
        for (size_t i = 0; i < (size_t)s->W * Hq * Nb; ++i) D_hi[i] = 0.0f;
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O8 top-k clusters (Polestar 2.A/sparse: the k most drifted clusters).
 * Order: score descending, then index ascending; NaN ranks after every
 * number; -0 and +0 are equal.                                               */
/* ------------------------------------------------------------------------- */
static int ranks_before(float a, int ia, float b, int ib)
{
    int na = isnan(a), nb = isnan(b);
    if (na != nb) return nb;          /* the number ranks before the NaN */
    if (!na && a != b) return a > b;
    return ia < ib;
}

int pso_topk_clusters(const pso_shape* s, const float* score, int32_t k, int32_t* idx, float* val)
{
    if (!s || !score || !idx) return ERR_NULL;
    if (s->W < 0 || s->K < 1) return ERR_SHAPE;
    if (k < 1 || k > s->K) return ERR_RANGE;
    const int K = s->K;
    int* ord = (int*)malloc(sizeof(int) * (size_t)K);
    for (int w = 0; w < s->W; ++w) {
        const float* sw = score + (size_t)w * K;
        for (int i = 0; i < K; ++i) ord[i] = i;
        /* insertion sort: obviously stable and obviously a total order */
        for (int i = 1; i < K; ++i) {
            int x = ord[i], p = i;
            while (p > 0 && ranks_before(sw[x], x, sw[ord[p - 1]], ord[p - 1])) {
                ord[p] = ord[p - 1];
                --p;
            }
            ord[p] = x;
        }
        for (int r = 0; r < k; ++r) {
            idx[(size_t)w * k + r] = ord[r];
            if (val) val[(size_t)w * k + r] = sw[ord[r]];
        }
    }
    free(ord);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O9 refresh gather (Polestar 2.A/sparse: the positions of the selected
 * clusters are recomputed; 2.C: only the selected clusters are fetched).
 * pos = { j : assign_j in idx } in ascending order, count = |pos| (the true
 * size even when it exceeds cap; only min(count, cap) rows are written).
 * H_hat row = dtype((c_{a_j} + rhat) * n_j) with rhat_e = (E2M1 * s_b) * g_j;
 * K_out/V_out rows are copies.  Slots past count are left untouched.         */
/* ------------------------------------------------------------------------- */
int pso_refresh_gather(const pso_shape* s, int dtype, const int32_t* assign, const int32_t* idx,
                       int32_t k, int32_t cap, int32_t* pos, int32_t* count,
                       const uint8_t* codes, const uint8_t* bscale, const float* rscale,
                       const float* C, const float* row_norm, void* H_hat, const void* Kc,
                       const void* Vc, void* K_out, void* V_out)
{
    if (!s || !assign || !idx || !pos || !count) return ERR_NULL;
    if (H_hat && (!codes || !bscale || !rscale || !C || !row_norm)) return ERR_NULL;
    if ((Kc == NULL) != (K_out == NULL) || (Vc == NULL) != (V_out == NULL)) return ERR_NULL;
    if (!check_dtype(dtype)) return ERR_DTYPE;
    if (!check_cluster_shape(s)) return ERR_SHAPE;
    if ((Kc || Vc) && !check_head_shape(s)) return ERR_SHAPE;
    if (k < 1 || k > s->K || cap < 0) return ERR_RANGE;
    const int N = s->N, d = s->d, K = s->K, nb = d / 16;
    const int KV = s->Hkv * s->dh;
    char* sel = (char*)malloc((size_t)K);
    for (int w = 0; w < s->W; ++w) {
        for (int c = 0; c < K; ++c) sel[c] = 0;
        for (int r = 0; r < k; ++r) {
            int c = idx[(size_t)w * k + r];
            if (c >= 0 && c < K) sel[c] = 1;
        }
        int cnt = 0;
        for (int j = 0; j < N; ++j) {
            const size_t row = (size_t)w * N + j;
            int a = assign[row];
            if (a < 0 || a >= K || !sel[a]) continue;
            if (cnt < cap) {
                const size_t slot = (size_t)w * cap + cnt;
                pos[slot] = j;
                if (H_hat) {
                    const float g = rscale[row], n = row_norm[row];
                    const float* c = C + ((size_t)w * K + a) * d;
                    for (int e = 0; e < d; ++e) {
                        uint8_t byte = codes[row * (size_t)(d / 2) + e / 2];
                        uint8_t nib = (e & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 15);
                        float sh = pso_e4m3_decode(bscale[row * (size_t)nb + e / 16]);
                        float rhat = (pso_e2m1_decode(nib) * sh) * g;
                        st(H_hat, dtype, slot * d + e, (c[e] + rhat) * n);
                    }
                }
                const size_t es = dtype == PSO_BF16 ? 2 : 4;   /* rows are copied byte for byte */
                if (Kc) memcpy((char*)K_out + slot * KV * es, (const char*)Kc + row * KV * es, KV * es);
                if (Vc) memcpy((char*)V_out + slot * KV * es, (const char*)Vc + row * KV * es, KV * es);
            }
            ++cnt;
        }
        count[w] = cnt;
    }
    free(sel);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O12 cosine-dissimilarity drift (Polestar 2.A/drift names cosine
 * dissimilarity as the measure KL is compared against).  Reading: with
 * warm-started spherical K-Means the cosine dissimilarity of cluster k between
 * steps is 1 - <c_k(t), c_k(t-1)> of its unit centres, i.e. how far the
 * centre moved; it scores clusters for the same top-k selection.            */
/* ------------------------------------------------------------------------- */
int pso_drift_cosine(const pso_shape* s, const float* C_cur, const float* C_prev, float* score)
{
    if (!s || !C_cur || !C_prev || !score) return ERR_NULL;
    if (s->W < 0 || s->K < 1 || s->d < 1) return ERR_SHAPE;
    const size_t K = (size_t)s->K, d = (size_t)s->d;
    for (size_t wk = 0; wk < (size_t)s->W * K; ++wk) {
        const float* a = C_cur + wk * d;
        const float* b = C_prev + wk * d;
        double dot = 0.0;
        for (size_t e = 0; e < d; ++e) dot += (double)a[e] * (double)b[e];
        score[wk] = (float)(1.0 - dot);
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O10 current-block commitment (Polestar 2.B/current).  The drift delta of a
 * block row is its drift now minus the mean of its earlier drifts; the row is
 * committed when that delta exceeds the confidence-conditioned threshold
 * alpha * (tau_s - c)^2, or, as under the plain static rule, when c >= tau_s.
 * Readings: the history mean covers the earlier steps only (not the current
 * one), a row with no history yet cannot fire the drift rule, and a window
 * whose count is 0 starts a fresh history (its stored sums are ignored).  Every
 * operation on the drift is one IEEE fp64 operation in the order written.   */
/* ------------------------------------------------------------------------- */
int pso_commit_block(const pso_shape* s, const float* D_i, const float* conf, int32_t block_start,
                     float alpha, float tau_s, double* hist_sum, int32_t* hist_n,
                     uint8_t* commit, float* delta)
{
    if (!s || !D_i || !conf || !hist_sum || !hist_n || !commit) return ERR_NULL;
    if (s->W < 0 || s->N < 1 || s->Nb < 0 || s->Nb > s->N) return ERR_SHAPE;
    if (block_start < 0 || block_start > s->N - s->Nb) return ERR_RANGE;
    if (!isfinite(alpha) || alpha < 0.0f || !isfinite(tau_s)) return ERR_RANGE;
    const int N = s->N, Nb = s->Nb;
    for (int w = 0; w < s->W; ++w) {
        const int32_t n = hist_n[w] > 0 ? hist_n[w] : 0;
        for (int i = 0; i < Nb; ++i) {
            const size_t r = (size_t)w * Nb + i;
            const double D = (double)D_i[r];
            const float c = conf[(size_t)w * N + block_start + i];
            int drift_rule = 0;
            double dl = 0.0;
            if (n > 0) {
                const double mean = hist_sum[r] / (double)n;
                const double gap = (double)tau_s - (double)c;
                dl = D - mean;
                drift_rule = dl > (double)alpha * (gap * gap);
            }
            const int conf_rule = c >= tau_s;
            commit[r] = (uint8_t)(drift_rule | (conf_rule << 1));
            if (delta) delta[r] = (float)dl;
            hist_sum[r] = (n > 0 ? hist_sum[r] : 0.0) + D;
        }
        hist_n[w] = n + 1;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O11 suffix-block commitment (Polestar 2.B/suffix).  When the last layer's
 * top-k drifted clusters include a suffix-window cluster, suffix rows whose
 * confidence reaches tau_s are committed.  Reading: a cluster belongs to the
 * suffix window when strictly more than half of its members are suffix rows
 * (rows after the decode block); top-k entries outside [0, K) are ignored.  */
/* ------------------------------------------------------------------------- */
int pso_commit_suffix(const pso_shape* s, const int32_t* assign, const int32_t* idx, int32_t k,
                      int32_t block_start, const float* conf, float tau_s, uint8_t* flag,
                      uint8_t* commit)
{
    if (!s || !assign || !idx || !conf || !flag || !commit) return ERR_NULL;
    if (s->W < 0 || s->N < 1 || s->Nb < 0 || s->Nb > s->N || s->K < 1) return ERR_SHAPE;
    if (k < 1 || k > s->K) return ERR_RANGE;
    if (block_start < 0 || block_start > s->N - s->Nb) return ERR_RANGE;
    if (!isfinite(tau_s)) return ERR_RANGE;
    const int N = s->N, K = s->K, first = block_start + s->Nb;
    int32_t* members = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    int32_t* in_suffix = (int32_t*)malloc(sizeof(int32_t) * (size_t)K);
    for (int w = 0; w < s->W; ++w) {
        for (int c = 0; c < K; ++c) members[c] = in_suffix[c] = 0;
        for (int j = 0; j < N; ++j) {
            const int a = assign[(size_t)w * N + j];
            if (a < 0 || a >= K) continue;
            members[a] += 1;
            if (j >= first) in_suffix[a] += 1;
        }
        int f = 0;
        for (int r = 0; r < k; ++r) {
            const int c = idx[(size_t)w * k + r];
            if (c >= 0 && c < K && 2 * in_suffix[c] > members[c]) f = 1;
        }
        flag[w] = (uint8_t)f;
        for (int j = 0; j < N; ++j) {
            const size_t r = (size_t)w * N + j;
            commit[r] = (uint8_t)(f && j >= first && conf[r] >= tau_s);
        }
    }
    free(members);
    free(in_suffix);
    return 0;
}
