/*
 * polestar_oracle.h -- CPU oracle for the Polestar-Cache drift-detection path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, single-threaded C
 * implementation used to check the HIP library.  Only the test suite, the smoke
 * check and the benchmark's CPU-baseline leg may load it.  The product path
 * never links, loads or calls anything in this directory, and this directory
 * includes nothing from the product path.
 *
 * Source of the method: "Polestar: Drift-Aware Cache Calibration and Token
 * Commitment for Efficient Inference of Diffusion LLMs" (Lee, Ramachandran,
 * Kundu, Krishna), as summarised on its gist.science explainer pages
 * (arXiv 2607.14107), technical summary section 2.A "Polestar-Cache" and
 * section 2.B "Polestar-Commit".  Below, "Polestar 2.A/drift" means the
 * drift-measurement item of section 2.A, "Polestar 2.A/window" the
 * local-window-and-clustering item, "Polestar 2.A/sparse" the sparse-updates
 * item; "Polestar 2.B/current" and "Polestar 2.B/suffix" are the current-block
 * and suffix-block commitment items of section 2.B.
 *
 * Arithmetic: fp32 storage, fp64 accumulation of every sum and dot product,
 * rounded once to fp32 (or bf16) when stored.  bf16 inputs are widened exactly.
 * Ties always go to the lowest index.  Natural logarithms.
 *
 * All arrays are host memory, row-major, contiguous.  Every function returns 0
 * on success and a negative number on a bad argument (nothing is written then).
 */
#ifndef POLESTAR_ORACLE_H
#define POLESTAR_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t W;   /* windows (sequences x layers), all independent        */
    int32_t N;   /* tokens per window                                    */
    int32_t d;   /* hidden size; multiple of 16                          */
    int32_t Hq;  /* query heads                                          */
    int32_t Hkv; /* key/value heads; Hq % Hkv == 0                       */
    int32_t dh;  /* head dim                                             */
    int32_t Nb;  /* decode-block rows (the queries)                      */
    int32_t K;   /* clusters; 1 <= K <= N                                */
} pso_shape;

enum { PSO_F32 = 0, PSO_BF16 = 1 };
enum { PSO_INIT_GIVEN = 0, PSO_INIT_STRIDED = 1, PSO_INIT_FARTHEST = 2 };
enum { PSO_SCORE_KL_SHARE = 0, PSO_SCORE_KL_SHARE_ABS = 1, PSO_SCORE_ATTN_WEIGHTED = 2 };

/* ---- number formats ------------------------------------------------------ */
float    pso_bf16_to_f32(uint16_t b);
uint16_t pso_f32_to_bf16(float f);             /* round to nearest even    */
float    pso_e4m3_decode(uint8_t code);        /* OCP E4M3 (FN), bias 7    */
uint8_t  pso_e4m3_encode(float x);             /* x >= 0; nearest, ties to even, saturating at 448 */
float    pso_e2m1_decode(uint8_t nibble);      /* sign<<3 | magnitude idx  */
uint8_t  pso_e2m1_encode(float v);             /* nearest, ties to even, saturating at 6; 0 -> 0x0 */

/* ---- the path --------------------------------------------------------------
 * H  : [W][N][d]       dtype       hidden states of the window
 * Kr : [W][N][Hkv][dh] dtype       key rows of the window (nullable)
 * C  : [W][K][d]       f32         unit centroids (in/out)
 * Ck : [W][K][Hkv][dh] dtype       centroid keys (in/out)
 */
int pso_row_norms(const pso_shape* s, int dtype, const void* H, float* row_norm);

int pso_kmeans_init(const pso_shape* s, int dtype, const void* H, int init, float* C);

/* init (unless GIVEN), then `iters` Lloyd iterations, then the centroid keys.
 * objective: [W] fp64 (nullable).  Ck/Kr nullable together. */
int pso_kmeans_fit(const pso_shape* s, int dtype, const void* H, const void* Kr, int init,
                   int iters, float* C, int32_t* assign, int32_t* counts, float* row_norm,
                   void* Ck, double* objective);

/* The update step alone, from a given assignment (all values in [0, K)). */
int pso_kmeans_update(const pso_shape* s, int dtype, const void* H, const float* row_norm,
                      const int32_t* assign, float* C, int32_t* counts, double* objective);

int pso_residual_nvfp4(const pso_shape* s, int dtype, const void* H, const float* row_norm,
                       const float* C, const int32_t* assign, uint8_t* codes, uint8_t* bscale,
                       float* rscale);

/* Q: [W][Nb][Hq][dh] dtype, Ck: [W][K][Hkv][dh] dtype; logp: [W][Hq][Nb][K] f32.
 * If logp_prev is non-NULL the drift (pso_drift_kl) of the stored logp_cur
 * against it is also written; if NULL, D_hi/D_i/score are set to zero. */
int pso_proxy_attn(const pso_shape* s, int dtype, const void* Q, const void* Ck,
                   float softmax_scale, float* logp_cur, const float* logp_prev, int score_kind,
                   float* D_hi, float* D_i, float* score);

int pso_drift_kl(const pso_shape* s, const float* logp_cur, const float* logp_prev,
                 int score_kind, float* D_hi, float* D_i, float* score);

int pso_topk_clusters(const pso_shape* s, const float* score, int32_t k, int32_t* idx,
                      float* val);

int pso_refresh_gather(const pso_shape* s, int dtype, const int32_t* assign, const int32_t* idx,
                       int32_t k, int32_t cap, int32_t* pos, int32_t* count,
                       const uint8_t* codes, const uint8_t* bscale, const float* rscale,
                       const float* C, const float* row_norm, void* H_hat, const void* Kc,
                       const void* Vc, void* K_out, void* V_out);

/* Cosine-dissimilarity drift of each cluster between consecutive steps (the
 * alternative the drift-measurement item compares KL against):
 * score [W][K] f32 = fp32(1 - sum_e C_cur[k][e] * C_prev[k][e]), the sum in
 * fp64 in ascending e.  C_cur, C_prev: [W][K][d] f32 unit centres. */
int pso_drift_cosine(const pso_shape* s, const float* C_cur, const float* C_prev, float* score);

/* ---- Polestar-Commit (technical summary section 2.B) --------------------- */

/* Current-block commitment.  D_i: [W][Nb] f32 drift of the block rows (the
 * D_i that pso_drift_kl writes); conf: [W][N] f32 per-position confidence
 * of the window, block row i at position block_start + i.  hist_sum [W][Nb]
 * f64 and hist_n [W] i32 are the caller's running history (sum of the earlier
 * drifts of each block row and how many there were; a negative count counts
 * as 0); both are advanced by this call.  commit [W][Nb] u8: bit 0 = the
 * drift rule fired, bit 1 = the confidence rule fired.  delta [W][Nb] f32
 * (nullable) = D - history mean, 0 where there is no history. */
int pso_commit_block(const pso_shape* s, const float* D_i, const float* conf, int32_t block_start,
                     float alpha, float tau_s, double* hist_sum, int32_t* hist_n,
                     uint8_t* commit, float* delta);

/* Suffix-block commitment.  assign: [W][N] i32, idx: [W][k] i32 top-k
 * clusters, conf: [W][N] f32.  Suffix rows are [block_start + Nb, N).
 * flag [W] u8 = 1 when a top-k cluster is a suffix cluster (strictly more
 * than half of its members are suffix rows).  commit [W][N] u8 = 1 on suffix
 * rows with flag set and conf >= tau_s, 0 on every other row. */
int pso_commit_suffix(const pso_shape* s, const int32_t* assign, const int32_t* idx, int32_t k,
                      int32_t block_start, const float* conf, float tau_s, uint8_t* flag,
                      uint8_t* commit);

#ifdef __cplusplus
}
#endif
#endif
