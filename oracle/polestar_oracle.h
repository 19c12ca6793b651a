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
 * (arXiv 2607.14107), technical summary section 2.A "Polestar-Cache".  Below,
 * "Polestar 2.A/drift" means the drift-measurement item of that section,
 * "Polestar 2.A/window" the local-window-and-clustering item, and
 * "Polestar 2.A/sparse" the sparse-updates item.
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

#ifdef __cplusplus
}
#endif
#endif
