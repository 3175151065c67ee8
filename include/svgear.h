/*
 * svgear.h -- C ABI of the SVG-EAR sparse-attention hot path on AMD MI355X (gfx950).
 *
 * The method: SVG-EAR, "Parameter-Free Linear Compensation for Sparse Video
 * Generation via Error-aware Routing" (arXiv 2603.08982), built on Sparse
 * VideoGen2's semantic-aware permutation (arXiv 2505.18875).  The pages this
 * library follows describe its interface as routines that cluster the tokens
 * and return the sorted order, average each cluster, pick which cluster pairs
 * to compute, and compute them while estimating the rest (SVG-EAR task page,
 * "What the agent has to build" and the walkthrough's steps 1-3).
 *
 * Conventions shared by every call
 *   - Tensors are dense, row-major [B, H, N, D] (or [B, H, C, D] for
 *     centroids/means, [B, H, N] for per-token integers, [B, H, C+1] for
 *     offsets, [B, H, Cq, Ck] for routing tables).  B*H independent
 *     (batch, head) slices are processed in one launch.
 *   - Self-attention only: queries and keys share N.
 *   - D is 64 or 128.  Element types: SVGEAR_BF16 (bfloat16) or SVGEAR_F32.
 *     Centroids, means, scores and LSE are always float32.
 *   - All pointers are DEVICE pointers (hipMalloc'd or equivalent), owned by
 *     the caller, and must stay valid until the work queued on `stream`
 *     finishes.  The library never allocates, frees or retains memory; the
 *     scratch it needs is the caller's `ws` buffer of at least the size the
 *     matching *_workspace() query returns (256-byte aligned).  The one
 *     exception is svgear_sparse_attn_noalloc, whose scratch is a static
 *     device array of the library (below).
 *   - Every call is asynchronous on `stream` and never synchronises.  Calls
 *     that share a workspace or outputs must be ordered on one stream.
 *   - Arguments are validated before anything is queued.  On any non-OK
 *     status nothing was queued and outputs are untouched, except
 *     SVGEAR_ERR_HIP (a launch failed; outputs are undefined).
 *     svgear_last_error() returns a message for the calling thread's last
 *     non-OK status.  No call aborts or throws.
 *   - Results are bitwise deterministic run to run (no float atomics).
 *   - Setting the environment variable SVGEAR_FAULT to one of kmeans,
 *     kmeanspp, centroids, centroid_variances, route, route_topp, attn,
 *     quantize_fp8 makes that call return SVGEAR_ERR_INJECTED without queuing
 *     work (for testing a caller's dense fallback; attn covers every attention
 *     entry point).
 */
#ifndef SVGEAR_H
#define SVGEAR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SVGEAR_OK = 0,
    SVGEAR_ERR_INVALID_ARG = 1,   /* a pointer is null, a size is out of range, ... */
    SVGEAR_ERR_UNSUPPORTED = 2,   /* a valid request this build does not implement */
    SVGEAR_ERR_WORKSPACE = 3,     /* ws is null, misaligned or smaller than required */
    SVGEAR_ERR_HIP = 4,           /* a HIP launch failed */
    SVGEAR_ERR_INJECTED = 5       /* SVGEAR_FAULT named this call */
} svgear_status;

typedef enum { SVGEAR_BF16 = 0, SVGEAR_F32 = 1 } svgear_dtype;

/* Library version string, e.g. "svgear 0.1.0 gfx950". */
const char* svgear_version(void);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* svgear_last_error(void);

/* Largest cluster count any call accepts (C, Cq, Ck). */
#define SVGEAR_MAX_CLUSTERS 4096

/* ------------------------------------------------------------------------
 * svgear_kmeans -- Lloyd k-means of one tensor (Q or K), per (batch, head),
 * emitting the cluster-contiguous permutation.
 *
 * SVG2 summary, "Semantic-Aware Permutation via k-Means Clustering": Q and K
 * are clustered independently per head on their activation vectors (C_q and
 * C_k clusters, Euclidean distance); "Efficient System-Algorithm
 * Co-Design": centroids cached from the previous denoising step warm-start
 * the next one (1-3 rounds instead of 100+).  SVG-EAR task page, walkthrough
 * step 1: the clustering also returns the sorted order.
 *
 *   x          [B,H,N,D] dtype dt, the tokens.
 *   centroids  [B,H,C,D] float32, IN: start (cold init or the cached
 *              centroids); OUT: centroids after the last update.
 *   iters      rounds of (assign, update), >= 1.  Assign: each token to
 *              its nearest centroid by squared L2 distance; ties go to the
 *              lowest index (distances within 1e-5 relative of the minimum
 *              may resolve either way).  Update: each non-empty cluster's
 *              centroid becomes the mean of its members; an empty cluster
 *              keeps its centroid.  The first three updates sum every
 *              cluster from the sorted tokens; with more rounds, the third
 *              keeps exact fixed-point sums (values rounded to a step of at
 *              most 2^-30 of the largest row norm, per head) and every later
 *              update adds or removes only the tokens whose label changed,
 *              so results do not depend on the order of any addition.
 *   labels     [B,H,N] int32 OUT, the last assignment.
 *   perm       [B,H,N] int32 OUT, perm[p] = source token of permuted slot p:
 *              tokens grouped by label, original order inside a cluster.
 *   offsets    [B,H,C+1] int32 OUT, cluster c occupies [offsets[c], offsets[c+1]).
 *   Limits: 1 <= C <= min(N, SVGEAR_MAX_CLUSTERS), 1 <= N < 2^24.
 * ---------------------------------------------------------------------- */
size_t svgear_kmeans_workspace(int B, int H, int N, int D, int C);
svgear_status svgear_kmeans(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                            int iters, float* centroids, int32_t* labels, int32_t* perm,
                            int32_t* offsets, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_centroids -- gather into cluster-contiguous order and average each
 * cluster in one pass.
 *
 * SVG-EAR task page, "What the agent has to build": one routine averages each
 * cluster; walkthrough step 1: a small kernel averages each cluster's values
 * in one pass.  SVG2 summary: Q' = pi_q Q, K' = pi_k K, V' = pi_k V, with K
 * and V sharing pi_k.
 *
 *   x          [B,H,N,D] dtype dt.
 *   perm, offsets as produced by svgear_kmeans (any valid permutation whose
 *              clusters are the offsets' ranges is accepted).
 *   x_perm     [B,H,N,D] dtype dt OUT (nullable): x_perm[p] = x[perm[p]].
 *   means      [B,H,C,D] float32 OUT (nullable): mean of each cluster's
 *              rows; an empty cluster gets 0.
 * ---------------------------------------------------------------------- */
size_t svgear_centroids_workspace(int B, int H, int N, int D, int C);
svgear_status svgear_centroids(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                               const int32_t* perm, const int32_t* offsets, void* x_perm,
                               float* means, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_kmeanspp -- k-means++ cold seeding (D^2 sampling) of C centroids
 * per (batch, head), for a cold svgear_kmeans start.
 *
 * SVG2 summary, "Efficient System-Algorithm Co-Design": without a cached
 * start, k-means begins from k-means++ initial centroids.  Seed 0 is uniform;
 * each later seed is drawn with probability proportional to the squared
 * distance to the nearest seed so far.  The randomness is the caller's: one
 * uniform 64-bit word per seed.
 *
 * Exact rules (so that any implementation following them picks the same
 * tokens): D^2 is summed over the coordinates in index order in fp64 with one
 * rounding per product and per sum; the weights are floor(D^2 * 2^k) as
 * uint64, k the largest integer with N * max D^2 * 2^k < 2^62 for the
 * distances to seed 0; seed c (c >= 1) is the first token whose inclusive
 * prefix of weights exceeds floor(words[c] * total / 2^64); seed 0, and any
 * seed drawn when every weight is 0 (fewer distinct rows than seeds), is
 * token floor(words[c] * N / 2^64).  Inputs must be finite.
 *
 *   x          [B,H,N,D] dtype dt.
 *   words      [B,H,C] uint64, device: uniform random words, one per seed.
 *   centroids  [B,H,C,D] float32 OUT: the seeds' rows (exact copies).
 *   chosen     nullable [B,H,C] int32 OUT: the seeds' token indices.
 *   ws         at least svgear_kmeanspp_workspace(B, H, N, D) bytes
 *              (8 bytes per token plus per-tile sums).
 * Limits as svgear_kmeans (1 <= C <= min(N, SVGEAR_MAX_CLUSTERS)).  Launches
 * about 2 C kernels on stream; deterministic.
 * ---------------------------------------------------------------------- */
size_t svgear_kmeanspp_workspace(int B, int H, int N, int D);
svgear_status svgear_kmeanspp(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                              const uint64_t* words, float* centroids, int32_t* chosen, void* ws,
                              size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_route -- error-aware routing: probe error / block cost, greedy
 * fill to the density budget.
 *
 * FrontierCS blog on SVG-EAR, probe paragraph: the query cluster's mean
 * q_bar_i is scored against every key k of a block, s_k = q_bar_i.k / sqrt(d)
 * (here: times `scale`), and the block's error is the sum over its keys of
 * || e^{s_bar} v_bar - e^{s_k} v_k ||^2 with s_bar, v_bar belonging to the
 * key's cluster; the error is divided by the block's token pairs.  Pith
 * review, "What carries the argument": blocks are taken greedily by highest
 * error-to-cost ratio under a density budget.
 *
 * Readings fixed here: both exponentials are taken relative to the row
 * maximum M_i = max_k s_ik (leaves each row's ranking unchanged); the ratio
 * is r_ij = e_ij / (|Q_i| |K_j|) rounded to float32 (0 for an empty cluster);
 * per query cluster the non-empty key clusters are ordered by (r desc, j asc)
 * and taken while the keys already taken are < density * N (as a double), so
 * the block that crosses the budget is included; empty key clusters are
 * never taken; rows of empty query clusters are all zero.
 *
 *   q_means    [B,H,Cq,D] float32, the probes (query-cluster means).
 *   q_offsets  [B,H,Cq+1] int32 (only the sizes |Q_i| are used).
 *   k_perm, v_perm  [B,H,N,D] dtype dt, keys/values in cluster order.
 *   k_means, v_means [B,H,Ck,D] float32, the key-cluster means.
 *   k_offsets  [B,H,Ck+1] int32.
 *   scale      > 0 (normally 1/sqrt(D)).   density in (0, 1].
 *   scores_in  nullable [B,H,Cq,Ck] float32: when given, the probe is skipped
 *              and the selection runs on these ratios (the key, value and
 *              query-mean pointers may then be null).
 *   scores_out nullable [B,H,Cq,Ck] float32 OUT: the ratios used.
 *   mask       [B,H,Cq,Ck] uint8 OUT: 1 = compute the block exactly.
 * ---------------------------------------------------------------------- */
size_t svgear_route_workspace(int B, int H, int N, int D, int Cq, int Ck);
svgear_status svgear_route(const float* q_means, const int32_t* q_offsets, int Cq,
                           const void* k_perm, const void* v_perm, svgear_dtype dt,
                           const float* k_means, const float* v_means, const int32_t* k_offsets,
                           int Ck, int B, int H, int N, int D, float scale, float density,
                           const float* scores_in, float* scores_out, uint8_t* mask, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_route_topp -- routing under the SVG2 top-p budget.
 *
 * SVG2 summary, "Centroid-Based Top-p Selection": the centroid score
 * S_ij = q_bar_i.k_bar_j * scale gives each key cluster an estimated share of
 * query cluster i's attention mass, P'_ij = |K_j| e^{S_ij} / sum_l |K_l| e^{S_il};
 * clusters are taken in descending P' until the shares taken reach top_p.
 * FrontierCS blog on SVG-EAR, budget paragraph: SVG-EAR keeps that selection's
 * token pairs as the budget and spends them on the blocks with the most error
 * per pair.
 *
 * Readings fixed here: P' is evaluated in fp64 relative to the row's largest
 * S over non-empty clusters and rounded to float32; non-empty key clusters
 * are ordered by (P' desc, j asc) and their shares are added in that order in
 * double, a cluster being taken while the sum before it is < top_p, so the
 * cluster that reaches top_p is included; top_p = 1 takes every non-empty
 * cluster.  Row i's budget is the number of keys in its top-p clusters
 * (pairs = |Q_i| times that).  With error_ranked = 1 the mask is the greedy
 * fill of svgear_route (ratio desc, j asc, taken while the keys before are
 * < the row's budget, crossing block included) with the row's own budget in
 * place of density * N; with error_ranked = 0 the mask is the top-p selection
 * itself (the SVG2 router).  Rows of empty query clusters are all zero.
 *
 *   q_means .. scale   as for svgear_route.   top_p in (0, 1].
 *   error_ranked 0 or 1, as above.
 *   probs_in   nullable [B,H,Cq,Ck] float32: when given, P' is taken from it
 *              instead of the centroids.
 *   scores_in  nullable [B,H,Cq,Ck] float32, error_ranked = 1 only: ratios
 *              given, the probe is skipped.
 *   probs_out  nullable [B,H,Cq,Ck] float32 OUT: the P' used (0 for empty
 *              key clusters and rows of empty query clusters).
 *   scores_out nullable [B,H,Cq,Ck] float32 OUT, error_ranked = 1 only.
 *   budget_out nullable [B,H,Cq] int32 OUT: keys per row of the top-p set.
 *   mask       [B,H,Cq,Ck] uint8 OUT.
 * Pointers that the chosen inputs make unnecessary may be null: q_means and
 * k_means when probs_in is given and no probe runs; k_perm, v_perm, v_means
 * unless error_ranked = 1 without scores_in.  ws: at least
 * svgear_route_workspace(...) bytes.  Asynchronous on stream.
 * ---------------------------------------------------------------------- */
svgear_status svgear_route_topp(const float* q_means, const int32_t* q_offsets, int Cq,
                                const void* k_perm, const void* v_perm, svgear_dtype dt,
                                const float* k_means, const float* v_means,
                                const int32_t* k_offsets, int Ck, int B, int H, int N, int D,
                                float scale, float top_p, int error_ranked,
                                const float* probs_in, const float* scores_in, float* probs_out,
                                float* scores_out, int32_t* budget_out, uint8_t* mask, void* ws,
                                size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_sparse_attn -- dynamic-block-size sparse attention with centroid
 * compensation, output in original token order.
 *
 * SVG2 summary, "Custom dynamic block-size sparse attention kernel": blocks
 * are the (query cluster, key cluster) rectangles of the permuted layout,
 * of any size.  SVG-EAR: each skipped non-empty key cluster j enters the same
 * softmax as one key k_bar_j with value v_bar_j and score q.k_bar_j * scale +
 * ln n_j, i.e. weight n_j e^{q.k_bar_j scale} (FrontierCS blog toy example;
 * task page walkthrough step 3).  For query token t of cluster i:
 *   o_t = [sum_{j sel} sum_{u in K_j} e^{s_tu} v_u + sum_{j skipped, n_j>0} n_j e^{q_t.k_bar_j scale} v_bar_j]
 *         / [the same sums without the values],   s_tu = q_t.k_u * scale.
 * The output row goes back to the token's original position (SVG2 summary,
 * inverse permutation of O).
 *
 *   q_perm, k_perm, v_perm  [B,H,N,D] dtype dt, cluster-contiguous copies.
 *   q_perm_idx [B,H,N] int32: original index of each permuted query slot
 *              (the perm output of svgear_kmeans for Q).
 *   q_offsets  [B,H,Cq+1], k_offsets [B,H,Ck+1] int32.
 *   k_means, v_means [B,H,Ck,D] float32.
 *   mask       [B,H,Cq,Ck] uint8 from svgear_route (any 0/1 table works).
 *   out        [B,H,N,D] dtype dt OUT, original token order.
 *   lse        nullable [B,H,N] float32 OUT: natural-log sum of the weights.
 * A query cluster with nothing selected and every key cluster empty cannot
 * occur (the key clusters partition N >= 1 keys).
 * bf16: the pseudo-keys enter with k_bar and v_bar rounded to bf16, like the
 * keys and values (in the variance variant below the variances too).
 * Workspace (svgear_sparse_attn_workspace; 0 for invalid sizes): the tile
 * list and the bf16 copies of k_means, v_means (and k_vars), about 6 D Ck + 4 (Cq + 1)
 * bytes per (batch, head).
 * ---------------------------------------------------------------------- */
size_t svgear_sparse_attn_workspace(int B, int H, int N, int D, int Cq, int Ck);
svgear_status svgear_sparse_attn(const void* q_perm, const void* k_perm, const void* v_perm,
                                 svgear_dtype dt, const int32_t* q_perm_idx,
                                 const int32_t* q_offsets, int Cq, const int32_t* k_offsets,
                                 int Ck, const float* k_means, const float* v_means,
                                 const uint8_t* mask, int B, int H, int N, int D, float scale,
                                 void* out, float* lse, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------------------------
 * svgear_sparse_attn_noalloc -- svgear_sparse_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): same arguments, results and errors,
 * minus the workspace.  Its scratch (the tile list and the bf16 pseudo-key
 * rows, svgear_sparse_attn_workspace(...) bytes) is a static device array of
 * SVGEAR_NOALLOC_SCRATCH_BYTES that each GPU holds until the process ends;
 * the call allocates and frees nothing.  Sizes whose workspace exceeds that
 * limit return SVGEAR_ERR_INVALID_ARG before anything is queued.  Every call
 * on one GPU shares that GPU's array (the GPU is the stream's device, or the
 * current device for the null stream), so calls that overlap on one GPU race:
 * order them on one stream.  The first call on a device looks up the array's
 * device address (hipGetSymbolAddress) with that device current.
 * ---------------------------------------------------------------------- */
#define SVGEAR_NOALLOC_SCRATCH_BYTES (32u << 20)
svgear_status svgear_sparse_attn_noalloc(const void* q_perm, const void* k_perm, const void* v_perm,
                                         svgear_dtype dt, const int32_t* q_perm_idx,
                                         const int32_t* q_offsets, int Cq, const int32_t* k_offsets,
                                         int Ck, const float* k_means, const float* v_means,
                                         const uint8_t* mask, int B, int H, int N, int D, float scale,
                                         void* out, float* lse, hipStream_t stream);

/* ------------------------------------------------------------------------
 * Variance-corrected compensation (a variant; FrontierCS blog on SVG-EAR,
 * the paragraph on the centroid's low guess): the centroid score q.k_bar
 * under-estimates the average of e^{s} over the cluster, and a second-order
 * expansion raises it by sigma^2 / 2, sigma^2 = (1/d) sum_i q_i^2 Var(k_i)
 * with one variance per key coordinate.  A strength factor scales the term.
 * ---------------------------------------------------------------------- */

/* svgear_centroid_variances -- per-cluster, per-coordinate population
 * variance of x's rows: Var_c(x_i) = mean over c's rows of (x_i - mean_c,i)^2
 * (the blog's two-key example, scores 0 and 2, has variance 1: the mean of
 * the squared deviations).
 *
 *   x, perm, offsets  as for svgear_centroids.
 *   means      [B,H,C,D] float32: the cluster means (svgear_centroids).
 *   vars       [B,H,C,D] float32 OUT; an empty cluster gets 0.
 *   ws         at least svgear_centroids_workspace(B, H, N, D, C) bytes.
 * Deterministic (fixed summation order); asynchronous on stream. */
svgear_status svgear_centroid_variances(const void* x, svgear_dtype dt, int B, int H, int N, int D, int C,
                                        const int32_t* perm, const int32_t* offsets, const float* means,
                                        float* vars, void* ws, size_t ws_bytes, hipStream_t stream);

/* svgear_sparse_attn_var -- svgear_sparse_attn with every skipped cluster's
 * score raised by strength * sigma^2 / 2, sigma^2 = scale^2 sum_i
 * q_t,i^2 k_vars[j][i] for query token t: the pseudo-key weight becomes
 * n_j e^{q_t.k_bar_j scale + strength sigma^2 / 2}.  strength = 0 gives
 * svgear_sparse_attn's result.  Arguments as svgear_sparse_attn, plus
 *   k_vars     [B,H,Ck,D] float32: per-coordinate key variances
 *              (svgear_centroid_variances of K).
 *   strength   >= 0, finite.
 * bf16 inputs only (SVGEAR_ERR_UNSUPPORTED for float32); the workspace size
 * is svgear_sparse_attn_workspace's. */
svgear_status svgear_sparse_attn_var(const void* q_perm, const void* k_perm, const void* v_perm,
                                     svgear_dtype dt, const int32_t* q_perm_idx,
                                     const int32_t* q_offsets, int Cq, const int32_t* k_offsets,
                                     int Ck, const float* k_means, const float* v_means,
                                     const float* k_vars, float strength,
                                     const uint8_t* mask, int B, int H, int N, int D, float scale,
                                     void* out, float* lse, void* ws, size_t ws_bytes,
                                     hipStream_t stream);

/* ------------------------------------------------------------------------
 * FP8 variant (SVG2 summary, results on HunyuanVideo: SVG2 combined with
 * FP8 quantisation, 2.30x -> 2.55x end to end).  The pages give no scheme;
 * here Q' and K' are stored as OCP e4m3fn codes with one power-of-two scale
 * per (batch, head), the exact blocks' scores are e4m3 matrix products with
 * fp32 accumulation, and V, the weights and the pseudo-keys stay as in the
 * bf16 path.
 * ---------------------------------------------------------------------- */

/* svgear_quantize_fp8 -- x8 = e4m3fn(x * 2^-e) rounded to nearest even, with
 * e = exps[b,h] the smallest integer such that max|x| over the slice <= 448 * 2^e
 * (0 for an all-zero slice), so x ~ decode(x8) * 2^e.  The scaling by 2^-e is
 * exact; the e4m3 rounding is the only one.
 *   x          [B,H,N,D] dtype dt (finite values).
 *   x8         [B,H,N,D] uint8 OUT: the e4m3fn codes.
 *   exps       [B,H] int32 OUT.
 *   ws         at least svgear_quantize_fp8_workspace(B, H) bytes. */
size_t svgear_quantize_fp8_workspace(int B, int H);
svgear_status svgear_quantize_fp8(const void* x, svgear_dtype dt, int B, int H, int N, int D,
                                  uint8_t* x8, int32_t* exps, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* svgear_sparse_attn_fp8 -- svgear_sparse_attn with q = decode(q8) * 2^q_exp
 * and k = decode(k8) * 2^k_exp (outputs of svgear_quantize_fp8 on the
 * permuted Q' and K'); v_perm is bf16; k_means and v_means are the fp32 means
 * of the unquantised keys and values.  The exact blocks' scores are
 * scale * 2^(q_exp + k_exp) * (e4m3 codes product, fp32 accumulation); a
 * skipped cluster's score is scale * q.k_bar_j + ln n_j with the dequantised
 * q.  Same workspace, layouts, tile list and output as svgear_sparse_attn
 * (out bf16 in original token order, lse nullable). */
svgear_status svgear_sparse_attn_fp8(const uint8_t* q8, const int32_t* q_exp, const uint8_t* k8,
                                     const int32_t* k_exp, const void* v_perm,
                                     const int32_t* q_perm_idx, const int32_t* q_offsets, int Cq,
                                     const int32_t* k_offsets, int Ck, const float* k_means,
                                     const float* v_means, const uint8_t* mask, int B, int H, int N,
                                     int D, float scale, void* out, float* lse, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SVGEAR_H */
