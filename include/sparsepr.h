/*
 * sparsepr.h -- C ABI of the SparsePR attention call on AMD Instinct MI355X (gfx950).
 *
 * The call replaces one dense softmax attention O = softmax(s Q K^T) V with four stages
 * (paper "Partition the Support, Reconstruct the Residual", abstract; project website,
 * Method section, stages 01-04):
 *   sparsepr_plan          stages 01-02 and the routing half of 03: Response-Coupled
 *                          Partitioning (key groups by sampled-query responses, query
 *                          groups by responses to key-group centroids), group routing
 *                          under an executed-pair density budget, stratified probe rows;
 *   sparsepr_attend        stage 03 and the exact half of 04: block-sparse attention over
 *                          the selected (query group, key group) cells, and exact dense
 *                          attention on the probe rows;
 *   sparsepr_fit_residual  stage 04: weighted ridge fit of an affine map from a probe's
 *                          sparse output to its residual (dense minus sparse);
 *   sparsepr_apply         stage 04: adds the predicted residual to every unprobed row,
 *                          probe rows take their exact output.
 *
 * Layouts. Q, K, V and every output of shape [B, H, N, d] are dense row-major ("BHND"):
 * element (b, h, n, i) sits at ((b*H + h)*N + n)*d + i. Heads are independent; the
 * library treats the B*H heads as one flat index. Element types: SPARSEPR_F32 inputs
 * give float outputs, SPARSEPR_BF16 inputs (bfloat16, round-to-nearest-even) give
 * bfloat16 outputs; the probe buffers and the coefficients are always float.
 *
 * Ownership. Every pointer argument except the config, the plan handle and the
 * host-side info array is a device pointer owned by the caller. The plan handle owns
 * host metadata only; all device-side plan state lives in the caller's workspace, which
 * must stay alive and untouched from sparsepr_plan until the last call that uses it.
 * The library allocates no device memory.
 *
 * Streams. Every device-side call only validates its arguments and enqueues kernels on
 * the given stream (a hipStream_t passed as void*; NULL = the default stream); it
 * returns before the work is done. Calls on one plan must be issued on one stream in
 * order plan -> attend -> fit_residual -> apply. A plan handle is not thread-safe.
 *
 * Errors. Argument errors are detected on the host and returned before anything is
 * enqueued (nothing is modified). A failure to enqueue returns SPARSEPR_ERR_HIP.
 * Conditions found on the device (a non-positive Cholesky pivot in the ridge solve)
 * are recorded in a per-head status word in the workspace and reported by
 * sparsepr_plan_info, which synchronises the stream.
 */
#ifndef SPARSEPR_H
#define SPARSEPR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARSEPR_OK = 0,
  SPARSEPR_ERR_INVALID_ARG = 1,   /* null pointer, size or range error                    */
  SPARSEPR_ERR_UNSUPPORTED = 2,   /* head_dim not 64/128, dtype unknown, groups > 1024      */
  SPARSEPR_ERR_WORKSPACE = 3,     /* workspace missing or smaller than required             */
  SPARSEPR_ERR_HIP = 4,           /* a HIP runtime call failed                              */
  SPARSEPR_ERR_NUMERICAL = 5,     /* ridge system not positive definite (device status)    */
  SPARSEPR_ERR_STATE = 6,         /* calls out of order (e.g. attend before plan)           */
  SPARSEPR_ERR_TOO_LARGE = 7      /* sparsepr_plan_static: the plan needs more device state */
                                  /* than SPARSEPR_STATIC_WORKSPACE_BYTES                   */
} sparsepr_status;

typedef enum { SPARSEPR_F32 = 0, SPARSEPR_BF16 = 1 } sparsepr_dtype;

/* Plain-old-data configuration; zero-initialise, then set every field. */
typedef struct {
  int32_t batch, heads, seq_len, head_dim; /* B, H, N, d; d in {64, 128}                  */
  int32_t dtype;                           /* sparsepr_dtype                              */
  float softmax_scale;                     /* s; 0 selects 1/sqrt(d)                      */
  int32_t n_sampled;                       /* S sampled queries per head, 1 <= S <= N     */
  int32_t n_key_groups;                    /* C_k requested key groups, 1..min(N, 1024)  */
  int32_t n_query_groups;                  /* C_q requested query groups, 1..min(N,1024) */
  int32_t n_probes;                        /* M exact probe rows per head, 0 <= M <= N    */
  double density;                          /* rho: executed pairs incl. probes / N^2, >0  */
  int32_t kmeans_max_iter;                 /* Lloyd iteration limit (paper Table C.1: 25) */
  float kmeans_tol;                        /* relative inertia decrease to stop (1e-4)    */
  float ridge_lambda;                      /* lambda >= 0 on the linear part of the map   */
  int32_t penalize_bias;                   /* nonzero: lambda on the bias row too         */
  uint64_t seed;                           /* seeds the counter-based selection hash      */
  int32_t assign_precision;                /* bf16 inputs, Lloyd assignment products:     */
                                           /*   0 centroid operand rounded to bf16,       */
                                           /*   1 bf16 + bf16 remainder (~16-bit operand) */
  int32_t warm_iters;                      /* Lloyd limit of sparsepr_plan_warm; 0 -> 2   */
                                           /* (paper Table C.1: 2 for subsequent calls)   */
  /* Comparison settings of paper Tables 2 and 4 (0 = the method everywhere):             */
  int32_t partition;                       /* 0 response-coupled; 1 semantic (k-means on  */
                                           /*   raw K and raw Q); 2 key-response K/V      */
                                           /*   groups with semantic query groups         */
  int32_t correction;                      /* 0 weighted ridge; 1 mean-only (Theta bias = */
                                           /*   weighted mean probe residual); 2 none     */
                                           /*   (unprobed rows keep the sparse output)    */
  int32_t probe_selector;                  /* 0 query-group stratified; 1 random (smallest*/
                                           /*   probe hash over all tokens); 2 uniform    */
                                           /*   (tokens floor((2p+1)N/2M)); 1, 2 weigh 1  */
  int32_t key_rank;                        /* key response rank r_K (paper Table C.1: 48); */
                                           /*   0 = full; k-means of the keys on their     */
                                           /*   responses projected on the r_K leading     */
                                           /*   directions of the sampled queries (metric  */
                                           /*   G truncated to its r_K largest eigenvalues)*/
                                           /*   applied when 0 < r_K < min(d, S)           */
  int32_t attn_tile_rows;                  /* query rows per block-sparse attention tile: */
                                           /*   128 or 256; 0 = 256 when B*H*N >= 1024*256 */
                                           /*   (enough tiles to fill the GPU), else 128;   */
                                           /*   outputs do not depend on it                */
  int32_t output_rank;                     /* output truncation of the residual fit (paper */
                                           /*   Table D.2 holds "no output truncation"): 0 */
                                           /*   none; 0 < r < d projects the predicted     */
                                           /*   residual on the r leading eigenvectors of  */
                                           /*   R^T W R of the probe residuals; r >= d is  */
                                           /*   the whole observed span (no change)        */
} sparsepr_config;

typedef struct sparsepr_plan_s* sparsepr_plan_t;

/* Per-head facts of a plan, read back by sparsepr_plan_info. */
typedef struct {
  int32_t key_groups;      /* realised C_k' (empty clusters dropped)                       */
  int32_t query_groups;    /* realised C_q'                                                */
  int32_t key_iters;       /* Lloyd assignments run for the key groups                     */
  int32_t query_iters;     /* Lloyd assignments run for the query groups                   */
  int64_t executed_pairs;  /* sum over selected cells n_q*n_k, plus M*N probe pairs         */
  int64_t budget;          /* floor(rho N^2) - M N                                         */
  int64_t tau;             /* routing threshold on the integer group masses                */
  int32_t budget_exceeded; /* 1 if one key group per query group already exceeds budget   */
  int32_t status;          /* sparsepr_status of the device-side steps of this head        */
} sparsepr_head_info;

/* Plan-state arrays that sparsepr_plan_export can copy out (per head, int32 unless noted). */
typedef enum {
  SPARSEPR_EXPORT_SAMPLED = 0,       /* [S] sampled query ids, ascending                  */
  SPARSEPR_EXPORT_KEY_LABELS = 1,    /* [N] compacted key-group id of each token          */
  SPARSEPR_EXPORT_QUERY_LABELS = 2,  /* [N] compacted query-group id of each token        */
  SPARSEPR_EXPORT_KEY_PERM = 3,      /* [N] tokens sorted stably by key group             */
  SPARSEPR_EXPORT_QUERY_PERM = 4,    /* [N] tokens sorted stably by query group           */
  SPARSEPR_EXPORT_KEY_OFFSETS = 5,   /* [C_k+1] group starts in KEY_PERM (first C_k'+1)   */
  SPARSEPR_EXPORT_QUERY_OFFSETS = 6, /* [C_q+1] group starts in QUERY_PERM                */
  SPARSEPR_EXPORT_ROUTE_ROWPTR = 7,  /* [C_q+1] CSR row starts of the selected cells      */
  SPARSEPR_EXPORT_ROUTE_COLS = 8,    /* [C_q*C_k] selected key groups, ascending per row  */
  SPARSEPR_EXPORT_PROBES = 9,        /* [M] probe rows, group-major, ascending token id   */
  SPARSEPR_EXPORT_PROBE_WEIGHTS = 10,/* [M] float ridge weights, summing to M             */
  SPARSEPR_EXPORT_GROUP_MASS = 11,   /* [C_q*C_k] int64 masses u (row stride C_k)         */
  SPARSEPR_EXPORT_KEY_CENTROIDS = 12,/* [C_k*d] float key-space centroids (row stride d)  */
  SPARSEPR_EXPORT_KEY_SEEDS = 13,    /* [C_k] Forgy seed rows of the key k-means, ascending */
  SPARSEPR_EXPORT_QUERY_SEEDS = 14   /* [C_q] Forgy seed rows of the query k-means;        */
                                     /*   both written by sparsepr_plan only (a warm or    */
                                     /*   labels-given plan leaves them as they were)      */
} sparsepr_export_kind;

/* Validates cfg and creates a plan handle. Host only: touches no device. */
sparsepr_status sparsepr_plan_create(const sparsepr_config* cfg, sparsepr_plan_t* out);
void sparsepr_plan_destroy(sparsepr_plan_t plan);

/* Bytes of device workspace a plan needs (256-byte aligned base required). */
size_t sparsepr_workspace_bytes(sparsepr_plan_t plan);

/* Stages 01-02 and routing (paper abstract; website Method stages 01-03):
 * q, k: [B,H,N,d] of cfg.dtype. Binds `workspace` to the plan. */
sparsepr_status sparsepr_plan(sparsepr_plan_t plan, const void* q, const void* k,
                              void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): sparsepr_plan with the plan's device
 * state placed in a library-owned static device array of SPARSEPR_STATIC_WORKSPACE_BYTES
 * per GPU instead of a caller workspace. The caller still passes q, k and, later, every
 * output buffer. Calls no hipMalloc, hipFree or other allocating routine. Returns
 * SPARSEPR_ERR_TOO_LARGE, before anything is enqueued, when sparsepr_workspace_bytes(plan)
 * exceeds the limit (128 MiB holds, e.g., 8 heads x 16,384 tokens, d = 128, 64 groups).
 * Later sparsepr_attend / _fit_residual / _apply / _plan_info / _plan_export /
 * _plan_set_probes on the handle use the array (on the GPU current at this call);
 * sparsepr_plan_warm and sparsepr_dense_attention need a caller workspace.
 * Sharing: every handle planned this way on one GPU uses the one array, which keeps the
 * last call's contents, so a later sparsepr_plan_static on that GPU replaces the state of
 * earlier handles; calls that overlap on one GPU (other streams or threads) race. */
#define SPARSEPR_STATIC_WORKSPACE_BYTES (128u << 20)
sparsepr_status sparsepr_plan_static(sparsepr_plan_t plan, const void* q, const void* k, void* stream);

/* Warm-started planning for a subsequent call (paper Table C.1: the first k-means runs up
 * to 25 iterations, subsequent ones up to 2). Both k-means start from the groups the
 * previous successful sparsepr_plan / sparsepr_plan_warm / sparsepr_plan_from_labels on this
 * handle left in `workspace`: key groups from their mean keys (mapped to responses under
 * the current sampled queries), query groups from their means of (s / RMS_i) q_i (mapped
 * through the current key centroids); the groups realised then are the ones requested now,
 * and any left empty are dropped. At most cfg.warm_iters iterations per k-means, same
 * tolerance rule. q, k: [B,H,N,d] of cfg.dtype (the new call's inputs). Returns
 * SPARSEPR_ERR_STATE when there is no previous plan in this workspace (none yet, another
 * workspace, or sparsepr_dense_attention used it since). */
sparsepr_status sparsepr_plan_warm(sparsepr_plan_t plan, const void* q, const void* k,
                                   void* workspace, size_t workspace_bytes, void* stream);

/* The same plan from caller-given partitions (used to check the downstream steps against
 * a reference partition): key_labels / query_labels [B*H, N] int32 in [0, C_k) /
 * [0, C_q) (empty groups are dropped and ids compacted as in sparsepr_plan);
 * group_mass (nullable) [B*H, C_q, C_k] int64 masses indexed by compacted ids, with row
 * stride C_k; when NULL the masses are computed from the labels. Probes are selected
 * from the query groups as in sparsepr_plan. */
sparsepr_status sparsepr_plan_from_labels(sparsepr_plan_t plan, const void* q, const void* k,
                                          const int32_t* key_labels, const int32_t* query_labels,
                                          const int64_t* group_mass, void* workspace,
                                          size_t workspace_bytes, void* stream);

/* Stage 03 + exact probes (paper abstract; website Method stage 03 and PFRR panel):
 * o_sparse [B,H,N,d] of cfg.dtype receives block-sparse attention in token order;
 * o_probe_sparse [B,H,M,d] float receives the same block-sparse rows for the probes
 * before rounding to cfg.dtype; o_probe_dense [B,H,M,d] float receives the exact
 * attention of the probe rows. Probe order is SPARSEPR_EXPORT_PROBES order. q, k, v
 * must be the tensors given to sparsepr_plan. */
sparsepr_status sparsepr_attend(sparsepr_plan_t plan, const void* q, const void* k, const void* v,
                                void* o_sparse, float* o_probe_sparse, float* o_probe_dense, void* stream);

/* Probe rows chosen by the caller, replacing those of the current plan (paper Table 2: the
 * repair comparisons hold the probe indices fixed across partitions). probes [B*H, M] int32
 * device, any order, each head's rows in [0, N) and distinct; weights [B*H, M] float device
 * or NULL for unit weights. The rows are copied to the host and checked (the call
 * synchronises the stream): ERR_INVALID_ARG if out of range or repeated, ERR_STATE if no
 * plan is current in this workspace. A later plan call selects probes again. */
sparsepr_status sparsepr_plan_set_probes(sparsepr_plan_t plan, const int32_t* probes, const float* weights,
                                         void* workspace, size_t workspace_bytes, void* stream);

/* Stage 04 fit (paper abstract; website PFRR panel): coeffs [B,H,d+1,d] float receives
 * Theta = (Z^T W Z + Lambda)^-1 Z^T W R with Z = [o_probe_sparse, 1],
 * R = o_probe_dense - o_probe_sparse, W = diag(weights), Lambda = diag(lambda 1_d, 0)
 * (lambda on the bias too if cfg.penalize_bias). probe_weights [B,H,M] float overrides
 * the plan's weights when non-NULL. Solved in float64; a pivot at or below 1e-12 x the
 * largest diagonal entry sets the head's status to SPARSEPR_ERR_NUMERICAL and writes
 * zero coefficients. With M = 0 the coefficients are zero. With cfg.output_rank = r
 * (0 < r < d), Theta is then replaced by Theta P, P the orthogonal projector on the r
 * leading eigenvectors of R^T W R (website PFRR panel: a low-rank probe-residual subspace). */
sparsepr_status sparsepr_fit_residual(sparsepr_plan_t plan, const float* o_probe_sparse,
                                      const float* o_probe_dense, const float* probe_weights,
                                      float* coeffs, void* stream);

/* Stage 04 apply (paper abstract): out_i = o_i + [o_i, 1] Theta for unprobed rows,
 * out_p = o_probe_dense for probe rows. out [B,H,N,d] of cfg.dtype may alias o_sparse. */
sparsepr_status sparsepr_apply(sparsepr_plan_t plan, const void* o_sparse, const float* o_probe_dense,
                               const float* coeffs, void* out, void* stream);

/* Exact dense attention softmax(s Q K^T) V with the same kernels (reference baseline):
 * needs a plan for the shapes and its workspace (plan state is overwritten). */
sparsepr_status sparsepr_dense_attention(sparsepr_plan_t plan, const void* q, const void* k,
                                         const void* v, void* out, void* workspace,
                                         size_t workspace_bytes, void* stream);

/* Synchronises `stream` and copies per-head facts into info[0 .. n_heads-1] (host). */
sparsepr_status sparsepr_plan_info(sparsepr_plan_t plan, sparsepr_head_info* info, int32_t n_heads,
                                   void* stream);

/* Bytes of one export for all heads; sparsepr_plan_export copies it device-to-device. */
size_t sparsepr_export_bytes(sparsepr_plan_t plan, int32_t which);
sparsepr_status sparsepr_plan_export(sparsepr_plan_t plan, int32_t which, void* dst, size_t dst_bytes,
                                     void* stream);

/* Per-stage timing (for benchmarks). When enabled, every later call records a pair of HIP
 * events around each stage on its stream. sparsepr_stage_times waits for the recorded
 * events and returns, per stage, the mean elapsed milliseconds over the calls since the
 * previous sparsepr_stage_times (the most recent 64 of them), then starts a new count.
 * Enabling creates HIP events (needs a device); disabling destroys them. */
typedef enum {
  SPARSEPR_STAGE_PLAN = 0,     /* sparsepr_plan / sparsepr_plan_from_labels                   */
  SPARSEPR_STAGE_PERMUTE = 1,  /* group-contiguous K and transposed V                         */
  SPARSEPR_STAGE_SPARSE = 2,   /* block-sparse attention kernel                               */
  SPARSEPR_STAGE_PROBES = 3,   /* exact attention of the probe rows                           */
  SPARSEPR_STAGE_FIT = 4,      /* ridge normal equations and Cholesky solve                   */
  SPARSEPR_STAGE_APPLY = 5,    /* residual apply                                              */
  SPARSEPR_NUM_STAGES = 6
} sparsepr_stage;
sparsepr_status sparsepr_set_stage_timing(sparsepr_plan_t plan, int32_t enable);
sparsepr_status sparsepr_stage_times(sparsepr_plan_t plan, float* ms, int32_t n);

const char* sparsepr_status_string(sparsepr_status s);

#ifdef __cplusplus
}
#endif

#endif /* SPARSEPR_H */
