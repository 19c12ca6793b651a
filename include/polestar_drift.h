/*
 * polestar_drift.h -- C ABI of libpolestar_drift, the drift-detection hot path
 * of Polestar-Cache for diffusion LLMs, on AMD Instinct MI355X (gfx950).
 *
 * Method source: "Polestar: Drift-Aware Cache Calibration and Token Commitment
 * for Efficient Inference of Diffusion LLMs" (Lee, Ramachandran, Kundu,
 * Krishna), as summarised on its gist.science explainer pages (arXiv
 * 2607.14107).  Citations below name that summary's section 2.A
 * ("Polestar-Cache") and its items: "drift measurement", "local window and
 * clustering", "sparse updates"; section 2.B ("Polestar-Commit") and its
 * items "current-block commitment" and "suffix-block commitment"; and
 * section 2.C ("system optimisation").
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Windows.  W independent windows (sequences x layers) are processed per
 *    call; every tensor has the window index outermost.  A window's results
 *    never depend on another window's data.
 *  - Memory.  Every tensor argument is caller-owned DEVICE memory, row-major
 *    and contiguous, 16-byte aligned (PS_ERR_ALIGN otherwise).  The library
 *    never allocates, frees or synchronises inside these calls; scratch space
 *    is passed in through `ws`.
 *  - Element types.  `dtype` selects the type of H, Kr, Kc, Vc, Q, Ck, H_hat,
 *    K_out and V_out: PS_BF16 (bfloat16 bit patterns) or PS_F32.  Centroids C,
 *    row norms, log-probabilities, drift and scores are always fp32.
 *  - Streams.  `stream` is a hipStream_t passed as void* (NULL = the null
 *    stream).  Each call checks its host-known arguments synchronously, then
 *    enqueues its kernels on `stream` and returns; on any error nothing is
 *    enqueued.  A launch failure returns PS_ERR_DEVICE.
 *  - State.  The library keeps no state between calls.  Cross-step state
 *    (C, Ck, the previous step's log-probabilities) is caller-owned, so
 *    saving those buffers resumes the path exactly.
 *  - Limits.  d % 16 == 0; 1 <= K <= min(N, 1024); Hq % Hkv == 0;
 *    dh % 8 == 0; N < 2^24; every tensor below 2^31 elements per window.
 *  - Determinism.  Every result is a deterministic function of the inputs:
 *    all reductions run in a fixed order, no floating-point atomics.
 */
#ifndef POLESTAR_DRIFT_H
#define POLESTAR_DRIFT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PS_OK = 0,
    PS_ERR_NULL = 1,      /* a required pointer is NULL                        */
    PS_ERR_SHAPE = 2,     /* a dimension violates the limits above             */
    PS_ERR_DTYPE = 3,     /* unsupported ps_dtype                              */
    PS_ERR_ALIGN = 4,     /* a tensor pointer is not 16-byte aligned           */
    PS_ERR_RANGE = 5,     /* a scalar argument is out of range (iters, k, ...) */
    PS_ERR_WORKSPACE = 6, /* ws is NULL or smaller than ps_workspace_size      */
    PS_ERR_DEVICE = 7,    /* a HIP launch or runtime call failed               */
    PS_ERR_MEMORY = 8,    /* a pointer the GPU must read is neither device
                             memory nor pinned host memory mapped for it   */
    PS_ERR_SCRATCH_LIMIT = 9  /* the shape needs more scratch than the
                             static scratch of ps_kmeans_fit_static holds  */
} ps_status;

typedef enum { PS_F32 = 0, PS_BF16 = 1 } ps_dtype;

/* Seeding of spherical K-Means.  GIVEN: start from the caller's C (the warm
 * start from the previous denoising step).  STRIDED: c_k = x_{floor(kN/K)}.
 * FARTHEST: farthest-first traversal under cosine similarity from x_0. */
typedef enum { PS_INIT_GIVEN = 0, PS_INIT_STRIDED = 1, PS_INIT_FARTHEST = 2 } ps_init;

/* How per-token drift becomes a per-cluster score for the top-k:
 * KL_SHARE: s_k = (1/Hq) sum_{h,i} p (l - l'), cluster k's additive share of
 * the summed KL; KL_SHARE_ABS: the same with |p (l - l')|; ATTN_WEIGHTED:
 * s_k = (1/Hq) sum_{h,i} p_{h,i,k} D_{h,i}. */
typedef enum {
    PS_SCORE_KL_SHARE = 0,
    PS_SCORE_KL_SHARE_ABS = 1,
    PS_SCORE_ATTN_WEIGHTED = 2
} ps_score;

/* ps_kmeans_fit flags.  By default (PS_KMEANS_DEFAULT, or the same behaviour
 * named explicitly: PS_KMEANS_FIXED_POINT_EXIT), once an iteration moves no
 * row of a window, every later iteration would reproduce the same centres and
 * assignments exactly, so the remaining passes of that window are skipped;
 * results are bit-identical to running all iterations.  PS_KMEANS_ALL_PASSES
 * runs every pass of every window in full (same results; for timing and
 * testing).  Both bits together: PS_ERR_RANGE. */
typedef enum {
    PS_KMEANS_DEFAULT = 0,
    PS_KMEANS_FIXED_POINT_EXIT = 1,
    PS_KMEANS_ALL_PASSES = 2
} ps_kmeans_flags;

typedef struct {
    int32_t W;   /* windows                                    */
    int32_t N;   /* tokens per window (prefix + block + suffix) */
    int32_t d;   /* hidden size                                */
    int32_t Hq;  /* query heads                                */
    int32_t Hkv; /* key/value heads                            */
    int32_t dh;  /* head dim                                   */
    int32_t Nb;  /* decode-block rows (proxy-attention queries) */
    int32_t K;   /* clusters per window                        */
} ps_shape;

/* Human-readable name of a status code (static storage). */
const char* ps_status_string(ps_status status);

/* Bytes of scratch that ps_kmeans_fit, ps_kmeans_fit_nvfp4 and
 * ps_residual_nvfp4 need for this shape and dtype. */
ps_status ps_workspace_size(const ps_shape* shape, ps_dtype dtype, size_t* bytes);

/*
 * ps_kmeans_fit -- spherical K-Means of each window's hidden states
 * (section 2.A, local window and clustering: the hidden states in a local
 * window around the decode block are clustered with spherical K-Means), plus
 * the centroid keys that proxy attention runs against (2.A, sparse updates).
 *
 *   H        [W][N][d]        dtype  in   hidden states of the window
 *   Kr       [W][N][Hkv][dh]  dtype  in   key rows (nullable, with Ck)
 *   init, iters                      in   seeding; Lloyd iterations (>= 1)
 *   flags                            in   ps_kmeans_flags (others: PS_ERR_RANGE)
 *   C        [W][K][d]        f32    in/out  unit centres (input read only
 *                                     for PS_INIT_GIVEN)
 *   assign   [W][N]           int32  out  cluster of each row, last iteration
 *   counts   [W][K]           int32  out  members per cluster
 *   row_norm [W][N]           f32    out  ||h_j||_2 (fp64 sum, rounded once)
 *   Ck       [W][K][Hkv][dh]  dtype  in/out  mean key row of each cluster
 *                                     (empty clusters keep their entry)
 *   objective [W]             f64    out  sum_k ||S_k|| (nullable)
 *   ws, ws_bytes                     scratch of ps_workspace_size bytes
 *
 * One Lloyd iteration: a_j = argmax_k <h_j, bf16(c_k)> (the exact c_k on the
 * fp32 path; ties to the lowest k), then S_k = sum_{a_j=k} h_j / n_j in fp64
 * and c_k = S_k / ||S_k||; empty clusters keep their centre.  The returned C
 * is the last update, so each c_k is the normalised mean of its members.
 * Clusters whose member set did not change since the previous iteration keep
 * their centre without being re-summed (the sum would be bit-identical).
 * Also requires d <= 8192 (PS_ERR_SHAPE above).
 */
ps_status ps_kmeans_fit(const ps_shape* shape, ps_dtype dtype, const void* H, const void* Kr,
                        ps_init init, int32_t iters, uint32_t flags, float* C, int32_t* assign,
                        int32_t* counts,
                        float* row_norm, void* Ck, double* objective, void* ws, size_t ws_bytes,
                        void* stream);

/* Bytes of the library's static K-Means scratch, one copy per device. */
#define PS_STATIC_SCRATCH_BYTES (64u << 20)

/*
 * ps_kmeans_fit_static -- ps_kmeans_fit for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and results, with the
 * scratch taken from a static device array of PS_STATIC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends.  The
 * call allocates and frees nothing; the caller still passes every input and
 * output.  A shape whose ps_kmeans_fit workspace would exceed that size
 * (ps_workspace_size gives the larger of two needs; this call needs only
 * the K-Means part, e.g. about 2.1 MiB per window of 8192 rows x 4096 with
 * 256 clusters, 0.55 MiB per window of 1024 rows x 4096 with 64) returns
 * PS_ERR_SCRATCH_LIMIT before anything is enqueued.  Every call on a device
 * uses that device's one array: calls that overlap on one device (several
 * streams or threads at once) race, so a caller serialises them.  Other
 * arguments, limits and errors as ps_kmeans_fit.
 */
ps_status ps_kmeans_fit_static(const ps_shape* shape, ps_dtype dtype, const void* H, const void* Kr,
                               ps_init init, int32_t iters, uint32_t flags, float* C, int32_t* assign,
                               int32_t* counts, float* row_norm, void* Ck, double* objective,
                               void* stream);

/*
 * ps_kmeans_fit_nvfp4 -- ps_kmeans_fit followed by ps_residual_nvfp4 of its
 * outputs (H, row_norm, C, assign), in one call: the clusters of section 2.A
 * (local window and clustering) and the NVFP4 residuals stored for them.
 * Every output is bit-identical to the two calls made in turn.  With bf16
 * rows of up to 4096 elements the first Lloyd update codes each cluster's
 * member rows right after rebuilding its centre, while those rows are still
 * cached, and after the last iteration only the rows of clusters rebuilt
 * since are coded again; otherwise the coder runs after the fit.
 *
 *   codes [W][N][d/2] u8, bscale [W][N][d/16] u8, rscale [W][N] f32   out
 *                                    (as ps_residual_nvfp4)
 *   ws, ws_bytes                     scratch of ps_workspace_size bytes
 *                                    (smaller or NULL: PS_ERR_WORKSPACE)
 *   every other argument, limit and error as ps_kmeans_fit; NULL codes,
 *   bscale or rscale: PS_ERR_NULL.
 */
ps_status ps_kmeans_fit_nvfp4(const ps_shape* shape, ps_dtype dtype, const void* H, const void* Kr,
                              ps_init init, int32_t iters, uint32_t flags, float* C, int32_t* assign,
                              int32_t* counts, float* row_norm, void* Ck, double* objective,
                              uint8_t* codes, uint8_t* bscale, float* rscale, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * ps_residual_nvfp4 -- NVFP4 coding of each row's residual to its centre
 * (section 2.A, local window and clustering: residuals are quantised with
 * NVFP4).  The pages give no format details; this library's convention:
 *   r = h_j / n_j - c_{a_j} (fp32), A = max|r|, g_j = A / 2688;
 *   per 16 elements: s_b = E4M3((A_b / 6) / g_j) (nearest, ties to even,
 *   saturating at 448), eff = s_b * g_j; code = E2M1(r / eff) (nearest,
 *   ties to even, saturating at 6; zero is +0); all zero where A or eff is 0.
 *
 *   H [W][N][d] dtype, row_norm [W][N] f32, C [W][K][d] f32,
 *   assign [W][N] int32 (values outside [0,K) read cluster 0)      in
 *   codes  [W][N][d/2]  u8   out  element 2i in the low nibble of byte i;
 *                                 nibble = sign<<3 | E2M1 magnitude index
 *   bscale [W][N][d/16] u8   out  E4M3 (bias 7, 0x7e = 448)
 *   rscale [W][N]       f32  out  g_j
 *   ws, ws_bytes                     scratch, or NULL: with at least
 *                                    8*W*N + 16 bytes (ps_workspace_size is
 *                                    always enough; the contents are
 *                                    overwritten), rows of up to 4096
 *                                    elements are coded grouped by cluster,
 *                                    each centre read about once per 16
 *                                    member rows; results are identical
 *                                    either way.  A smaller non-NULL ws:
 *                                    PS_ERR_WORKSPACE.
 *
 * Also requires d <= 8192 (PS_ERR_SHAPE above).
 */
ps_status ps_residual_nvfp4(const ps_shape* shape, ps_dtype dtype, const void* H,
                            const float* row_norm, const float* C, const int32_t* assign,
                            uint8_t* codes, uint8_t* bscale, float* rscale, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * ps_proxy_attn -- attention of the decode block's queries against the
 * cluster centres' keys (section 2.A, sparse updates: "proxy attention" is
 * computed at every step from the cluster centres), as log-probabilities:
 *   z_{h,i,k} = softmax_scale * <Q[i][h], Ck[k][g(h)]>, g(h) = h / (Hq/Hkv),
 *   logp = z - logsumexp_k z.
 * If logp_prev is given, the drift of logp_cur against it follows
 * (ps_drift_kl); if NULL (window formation) D_hi, D_i and score are zeroed.
 *
 *   Q [W][Nb][Hq][dh] dtype, Ck [W][K][Hkv][dh] dtype               in
 *   logp_cur  [W][Hq][Nb][K] f32  out
 *   logp_prev [W][Hq][Nb][K] f32  in   (nullable; must not alias logp_cur)
 *   D_hi [W][Hq][Nb] f32 out (nullable), D_i [W][Nb] f32 out, score [W][K] f32 out
 *
 * Also requires Nb <= 64 and Hq * Nb + 4 * K <= 16384 (PS_ERR_SHAPE above).
 */
ps_status ps_proxy_attn(const ps_shape* shape, ps_dtype dtype, const void* Q, const void* Ck,
                        float softmax_scale, float* logp_cur, const float* logp_prev,
                        ps_score score_kind, float* D_hi, float* D_i, float* score, void* stream);

/*
 * ps_drift_kl -- per-token drift between consecutive steps (section 2.A,
 * drift measurement: D_i = KL(A_i^(t) || A_i^(t-1)) of a token's attention
 * distributions).  Per head: D_{h,i} = sum_k p (l - l'), p = exp(l);
 * D_i = (1/Hq) sum_h D_{h,i}; the per-cluster score per ps_score.
 *
 *   logp_cur, logp_prev [W][Hq][Nb][K] f32 in
 *   D_hi [W][Hq][Nb] f32 out (nullable), D_i [W][Nb] f32 out, score [W][K] f32 out
 *
 * Also requires Hq * Nb + 4 * K <= 16384 (PS_ERR_SHAPE above).
 */
ps_status ps_drift_kl(const ps_shape* shape, const float* logp_cur, const float* logp_prev,
                      ps_score score_kind, float* D_hi, float* D_i, float* score, void* stream);

/*
 * ps_drift_cosine -- cosine-dissimilarity drift of every cluster between two
 * consecutive steps, the measure the pages' drift-measurement item (section
 * 2.A) sets KL against, here as an alternative cluster score for the same
 * top-k selection.  With warm-started spherical K-Means a cluster's cosine
 * dissimilarity is 1 - <c_k(t), c_k(t-1)> of its unit centres, i.e. how far
 * the centre moved:
 *   score[w][k] = fp32(1 - sum_e C_cur[w][k][e] * C_prev[w][k][e]),
 * the products and their sum in fp64 (the order of the sum may differ from
 * a sequential one by fp64 rounding, below one fp32 ulp of the result).
 *
 *   C_cur, C_prev [W][K][d] f32 in (C_prev = the centres before this step's
 *   K-Means; the call does not check that they are unit vectors)
 *   score [W][K] f32 out
 */
ps_status ps_drift_cosine(const ps_shape* shape, const float* C_cur, const float* C_prev,
                          float* score, void* stream);

/*
 * ps_topk_clusters -- the k most drifted clusters of each window (section
 * 2.A, sparse updates: the top-k drifted clusters are selected).  Order:
 * score descending, then index ascending; NaN ranks after every number;
 * -0 equals +0.
 *
 *   score [W][K] f32 in;  idx [W][k] int32 out;  val [W][k] f32 out (nullable)
 *   1 <= k <= min(K, 64)
 */
ps_status ps_topk_clusters(const ps_shape* shape, const float* score, int32_t k, int32_t* idx,
                           float* val, void* stream);

/*
 * ps_refresh_gather -- the rows to refresh: the positions of the selected
 * clusters, their hidden states rebuilt from centre + NVFP4 residual, and
 * their cached key/value rows (section 2.A, sparse updates: a sparse pass
 * recomputes only those positions; 2.C: only the selected clusters are
 * fetched).
 *
 *   assign [W][N] int32, idx [W][k] int32 (entries outside [0,K) select
 *   nothing), k, cap                                                  in
 *   pos   [W][cap] int32  out  ascending member positions (first min(count,cap));
 *                              may be NULL when cap == 0
 *   count [W]      int32  out  true number of positions, even beyond cap
 *   codes, bscale, rscale, C, row_norm  (as ps_residual_nvfp4)        in
 *         codes, bscale and rscale may instead sit in pinned host memory
 *         (hipHostMalloc, mapped for the device): the pages keep the
 *         quantised residual store in pinned CPU memory and fetch only the
 *         selected clusters (section 2.C, CPU offloading); the kernel then
 *         reads just the selected rows across PCIe through the allocation's
 *         device mapping.  Other host memory gives PS_ERR_MEMORY.
 *   H_hat [W][cap][d] dtype out (nullable; needs the five inputs above):
 *         dtype((c + (e2m1 * s_b) * g_j) * n_j)
 *   Kc, Vc [W][N][Hkv][dh] dtype in (nullable) -> K_out, V_out
 *         [W][cap][Hkv][dh] dtype out: byte copies of the selected rows
 * Slots at or past count are left untouched.
 */
ps_status ps_refresh_gather(const ps_shape* shape, ps_dtype dtype, const int32_t* assign,
                            const int32_t* idx, int32_t k, int32_t cap, int32_t* pos,
                            int32_t* count, const uint8_t* codes, const uint8_t* bscale,
                            const float* rscale, const float* C, const float* row_norm,
                            void* H_hat, const void* Kc, const void* Vc, void* K_out,
                            void* V_out, void* stream);

/*
 * ps_commit_block -- current-block commitment (section 2.B, current-block
 * commitment).  The drift delta of block row i is its drift now minus the
 * mean of its drifts at the earlier steps of the window's history; the row
 * commits when that delta exceeds the confidence-conditioned threshold
 * alpha * (tau_s - c)^2, or when its confidence c reaches tau_s (the static
 * rule).  With no history yet (count <= 0) only the confidence rule can fire.
 * Every operation on the drift is one IEEE fp64 operation:
 *   mean = hist_sum / n; gap = tau_s - c; delta = D - mean;
 *   drift rule: delta > alpha * (gap * gap).
 *
 *   D_i  [W][Nb] f32 in      drift of the block rows (as ps_drift_kl writes)
 *   conf [W][N]  f32 in      per-position confidence of the window; block row
 *                            i sits at position block_start + i
 *   block_start              0 <= block_start <= N - Nb
 *   alpha >= 0, tau_s        finite (PS_ERR_RANGE otherwise)
 *   hist_sum [W][Nb] f64 in/out  sum of each row's earlier drifts; D is added
 *   hist_n   [W]     i32 in/out  number of earlier steps; a count <= 0 starts
 *                            a fresh history (hist_sum is then ignored); set
 *                            to n + 1.  Zero it when a window is re-formed.
 *   commit [W][Nb] u8 out    bit 0: the drift rule fired; bit 1: c >= tau_s
 *   delta  [W][Nb] f32 out   (nullable) fp32 of the delta; 0 with no history
 * A NaN drift or confidence fires neither rule; a NaN drift makes the row's
 * history sum NaN.
 */
ps_status ps_commit_block(const ps_shape* shape, const float* D_i, const float* conf,
                          int32_t block_start, float alpha, float tau_s, double* hist_sum,
                          int32_t* hist_n, uint8_t* commit, float* delta, void* stream);

/*
 * ps_commit_suffix -- suffix-block commitment (section 2.B, suffix-block
 * commitment).  Pass the windows whose update packet decides (the pages use
 * the last layer's).  A cluster belongs to the suffix window when strictly
 * more than half of its members are suffix rows, i.e. rows at or after
 * block_start + Nb.  When any of the window's top-k clusters is such a
 * cluster, its suffix rows with confidence >= tau_s commit.
 *
 *   assign [W][N] i32 in     cluster of each row; values outside [0,K) count
 *                            for no cluster
 *   idx    [W][k] i32 in     top-k clusters (ps_topk_clusters); entries
 *                            outside [0,K) are ignored; 1 <= k <= K
 *   block_start              0 <= block_start <= N - Nb
 *   conf   [W][N] f32 in     per-position confidence; tau_s finite
 *   flag   [W]    u8  out    1 when a top-k cluster is a suffix cluster
 *   commit [W][N] u8  out    1 on suffix rows of flagged windows with
 *                            conf >= tau_s; 0 on every other row
 */
ps_status ps_commit_suffix(const ps_shape* shape, const int32_t* assign, const int32_t* idx,
                           int32_t k, int32_t block_start, const float* conf, float tau_s,
                           uint8_t* flag, uint8_t* commit, void* stream);

/*
 * Kernel timer (instrumentation, not part of the method; off by default).
 * ps_profile_begin creates 2*max_launches HIP events and a device counter per
 * launch on the current device and switches recording on: from then on every
 * kernel the calls above enqueue is bracketed by two events on the stream it
 * runs on (launches past the capacity are counted as dropped), and the
 * kernels whose work depends on the data (the Lloyd passes, which skip the
 * windows at a fixed point; the centre update, which re-sums only changed
 * clusters) count the units of work they process.  ps_profile_end switches
 * recording off.  ps_profile_summary waits for the recorded events and
 * writes one text line per kernel,
 * "name\tlaunches\ttotal_ms\tmin_ms\tmax_ms\tunits_done\tunits", then
 * "#dropped\t<n>"; units is the total work of the kernel's launches (tiles,
 * rows or clusters), units_done the part processed, both 0 for kernels that
 * always do their full work; PS_ERR_RANGE if `len` is too small.  Not
 * thread-safe; not for use under graph capture.
 */
ps_status ps_profile_begin(int32_t max_launches);
ps_status ps_profile_end(void);
ps_status ps_profile_summary(char* buf, size_t len);

#ifdef __cplusplus
}
#endif

#endif /* POLESTAR_DRIFT_H */
