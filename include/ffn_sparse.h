/*
 * ffn_sparse.h -- C ABI of the MI355X (gfx950) activation-sparse FFN library, libffn_sparse.so
 * (the sparse FFN, its mixture-of-experts form, and, at the end of this file, the attention block
 * with a head-level active set).
 *
 * The operator is the neuron-aware sparse FFN of PowerInfer / PowerInfer-2:
 *  - "PowerInfer: Fast LLM Serving with a Consumer-grade GPU" (unite.ai): section "Adaptive sparse
 *    predictor" (a small per-layer model predicts which FFN neurons fire for the current token),
 *    section "Online stage" (neurons predicted inactive are skipped), section "Neuron-aware
 *    operator" (the active neurons' row / column vectors are computed directly, with no
 *    conversion to a dense format), section "Neuron placement and management" (computed neurons
 *    keep their original positions);
 *  - nearauto.com PowerInfer article, section "PowerInfer architecture", Fig. 8 (only activated
 *    neurons are computed, and partial results from disjoint neuron sets are summed);
 *  - citnews.com.cn PowerInfer-2 article, section "Dynamic neuron cache" (inactive neurons do not
 *    change the output), section on neuron-cluster computation (prefill with most neurons active
 *    runs as large dense clusters, decode as small sparse ones) and section on low-cost
 *    sparsification (dReLU: both gate and up are rectified);
 *  - nearauto.com section "Experiments", Fig. 13 (INT4-quantised models), Fig. 14 (batch sizes).
 *
 * For one token x (d values) and a layer with ffn neurons:
 *   predictor   z = P1 x + c1              (rank values)
 *               s = P2 z + c2              (ffn scores)
 *               A = { i : sigmoid(s_i) > threshold }, ascending
 *   neurons     u_i = W_up[i] . x + b_up_i,   g_i = W_gate[i] . x + b_gate_i      (i in A)
 *               h_i = max(u_i,0) (ReLU) | max(g_i,0) u_i (ReGLU) | max(g_i,0) max(u_i,0) (dReLU)
 *   output      y = b_down + sum_{i in A} h_i W_down_t[i]      (W_down stored transposed)
 *
 * Conventions shared by every entry point:
 *  - Every function returns an ffn_status; none throws, exits or prints.  Arguments are checked
 *    before anything is enqueued: on FFN_ERR_INVALID_ARGUMENT / FFN_ERR_UNSUPPORTED /
 *    FFN_ERR_WORKSPACE_TOO_SMALL nothing was enqueued and no output was touched.  FFN_ERR_HIP
 *    from a forward (a launch the runtime refused) can leave the kernels enqueued before it in
 *    place; the outputs are then unspecified.  ffn_last_error() gives a message.
 *  - Pointers named "device" are HIP device pointers (hipMalloc / torch CUDA tensors); they stay
 *    owned by the caller and must outlive the plan that references them.  Every device pointer
 *    must be 16-byte aligned.
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Forward calls only
 *    enqueue work on it: they never allocate, never synchronise and never use memset nodes, so a
 *    caller may capture them in a HIP graph.
 *  - Shapes: d % 8 == 0 (d % 32 == 0 for int4), d <= 8192 (fp32 rows: d <= 4096),
 *    ffn % 32 == 0, ffn <= 32768, rank % 8 == 0, rank <= 2048 (fp16 predictor) / 1024 (fp32
 *    predictor), 1 <= B <= max_batch <= 4096.  Anything else gives FFN_ERR_UNSUPPORTED or
 *    FFN_ERR_INVALID_ARGUMENT.
 *  - A plan is not re-entrant: forward calls on one plan must be ordered (one stream).  Plans used
 *    one after another on one stream may share one workspace.
 */
#ifndef FFN_SPARSE_H
#define FFN_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FFN_OK = 0,
    FFN_ERR_INVALID_ARGUMENT = 1,   /* NULL where a pointer is required, bad enum, B out of range */
    FFN_ERR_UNSUPPORTED = 2,        /* shape / dtype combination the kernels do not cover        */
    FFN_ERR_WORKSPACE_TOO_SMALL = 3,
    FFN_ERR_HIP = 4,                /* a HIP runtime call failed (message in ffn_last_error)     */
    FFN_ERR_INTERNAL = 5
} ffn_status;

typedef enum { FFN_ACT_RELU = 0, FFN_ACT_REGLU = 1, FFN_ACT_DRELU = 2 } ffn_act;

/* Storage types.  FFN_I4G32: signed two's-complement nibbles, element 2k in the low nibble of
 * byte k of a row, plus one fp16 scale per 32 consecutive elements of the row; w = scale * q. */
typedef enum { FFN_F32 = 0, FFN_F16 = 1, FFN_I4G32 = 2 } ffn_dtype;

typedef enum { FFN_PATH_AUTO = 0, FFN_PATH_SPARSE = 1, FFN_PATH_DENSE = 2 } ffn_path;

typedef struct {
    int32_t d;          /* model width                                                       */
    int32_t ffn;        /* FFN neurons                                                       */
    int32_t rank;       /* predictor rank; 0 = no predictor (sparse forward then needs a mask) */
    int32_t act;        /* ffn_act                                                           */
    int32_t w_dtype;    /* up / gate / down_t storage: FFN_F32 | FFN_F16 | FFN_I4G32         */
    int32_t x_dtype;    /* token storage: FFN_F32 | FFN_F16                                  */
    int32_t p_dtype;    /* predictor storage: FFN_F32 | FFN_F16                              */
    float threshold;    /* tau in (0, 1]: neuron active iff sigmoid(s) > tau, strictly       */
    int32_t max_batch;  /* largest B any forward call on this plan will pass                  */
} ffn_layer_desc;

typedef struct {                       /* all device pointers, caller-owned                   */
    const void *w_up, *w_gate, *w_down_t; /* [ffn][d] row-major; int4: [ffn][d/2] bytes      */
    const void *s_up, *s_gate, *s_down_t; /* int4 only: [ffn][d/32] fp16 scales, else NULL   */
    const float *b_up, *b_gate, *b_down;  /* [ffn], [ffn], [d] fp32; each may be NULL (= 0)  */
    const void *p1, *p2;                  /* [rank][d], [ffn][rank] in p_dtype               */
    const float *c1, *c2;                 /* [rank], [ffn] fp32; may be NULL (= 0)           */
} ffn_layer_weights;                      /* w_gate / s_gate / b_gate are ignored for ReLU     */

typedef struct ffn_plan ffn_plan;          /* opaque host object                              */

/* Bytes of device workspace a plan for `desc` needs (upper bound for any B <= max_batch). */
ffn_status ffn_workspace_size(const ffn_layer_desc *desc, size_t *bytes);

/*
 * Validate desc and weights, lay out the caller's device workspace and return a plan.
 * `workspace` (device, >= ffn_workspace_size bytes) is owned by the caller and must outlive the
 * plan.  calibrate = 1 (fp16 layers with max_batch >= 2) times the plan's dense path against
 * its sparse path over a density sweep for B = 2, 4, ..., max_batch on `stream` and stores the
 * crossover density per batch bucket used by FFN_PATH_AUTO; it is the only call that
 * synchronises, and it allocates (and frees) its own scratch inputs.  calibrate = 0 keeps the
 * built-in crossover table: 1 (never dense) below 64 tokens, where the batched kernels read the
 * union of a pass's sets once; from 64 tokens on 1 / ceil(B / 32) for the bucket's smallest B,
 * the union density at which the sparse passes (one per 32 tokens, each re-reading the union's
 * rows) read as many row bytes as the dense GEMMs' single read of every row.
 */
ffn_status ffn_sparse_plan(const ffn_layer_desc *desc, const ffn_layer_weights *weights,
                           void *workspace, size_t workspace_bytes, void *stream,
                           int32_t calibrate, ffn_plan **out);

/*
 * y[B][d] (fp32, fully overwritten) = FFN of the B tokens x[B][d] (x_dtype), each over its own
 * active set (device pointers).
 *   mask    [B][ffn] uint8 0/1 or NULL.  NULL: the predictor picks each token's set (needs
 *           rank > 0).  Non-NULL: the caller's set replaces the predictor's (test hook; also
 *           how a caller runs a precomputed set).
 *   idx     [B][ffn] int32 or NULL: token b's active neurons in ascending order in
 *           idx[b*ffn .. b*ffn + cnt[b]); the rest of the row is left unspecified.
 *   cnt     [B] int32 or NULL: |A_b|.
 *   scores  [B][ffn] fp32 or NULL: the predictor scores s (only written when mask == NULL).
 *   path    ffn_path.  SPARSE: only the rows of active neurons are read (one token: the batch-1
 *           kernels; several fp16 tokens: passes of up to 32 tokens over the union of their
 *           sets, on the matrix cores).  DENSE: every neuron's rows are read (fp16: the
 *           batched kernels for fewer than 64 tokens, two MFMA GEMMs from 64 on), each token's
 *           h still zeroed outside its own set.  AUTO: the device compares the union density
 *           of the call's sets with the plan's crossover density for B and takes DENSE above
 *           it, SPARSE below.  All paths give the same y within rounding.  fp32 and int4
 *           layers have no matrix-core path: every path runs their per-token kernels.
 * Errors: FFN_ERR_INVALID_ARGUMENT for NULL x / y, B out of [1, max_batch], mask == NULL with
 * rank == 0, bad path.
 */
ffn_status ffn_sparse_forward(ffn_plan *plan, const void *x, int32_t B, float *y,
                              const uint8_t *mask, int32_t *idx, int32_t *cnt, float *scores,
                              int32_t path, void *stream);

/*
 * The batch-1 decode path of ffn_sparse_forward without a plan and without a workspace, for
 * callers that cannot allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  It calls no hipMalloc / hipFree and no allocating routine, and creates
 * no plan: the descriptor and weights are checked on every call (as ffn_sparse_plan checks
 * them, max_batch bounding B), and the per-token scratch (predictor stage 1, the active
 * bitmap, |A| and the gather's partial sums of y) lives in a fixed device array inside the
 * library, 4 MiB + 64 KiB per GPU, held from the first call on that GPU until the process ends.
 * That covers every layer with d <= 4096 (the scratch grows with d); larger layers give
 * FFN_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   x, y, mask, idx, cnt: as ffn_sparse_forward (device pointers; y fully overwritten).  The B
 *   tokens run one after another through the batch-1 kernels (decode variant 0, no hot head),
 *   so each token's y and set equal those of ffn_sparse_forward on that token alone.
 * Every call on one GPU shares that GPU's scratch: calls on different streams that overlap in
 * time race and give unspecified results; calls ordered on one stream (or synchronised) are
 * safe.  The scratch's earlier contents never matter: every word a call reads, it wrote first.
 */
ffn_status ffn_sparse_forward_static(const ffn_layer_desc *desc, const ffn_layer_weights *weights,
                                     const void *x, int32_t B, float *y, const uint8_t *mask,
                                     int32_t *idx, int32_t *cnt, void *stream);

/*
 * Dense FFN (every neuron), y[B][d] fp32, through the MFMA GEMM kernels (the prefill path).
 * mask [B][ffn] uint8 or NULL: non-NULL zeroes h for inactive (token, neuron) pairs in the
 * epilogue, which equals the sparse result.
 */
ffn_status ffn_dense_forward(ffn_plan *plan, const void *x, int32_t B, float *y,
                             const uint8_t *mask, void *stream);

/* Crossover density for batch B: the union density above which AUTO takes the dense path
 * (batch buckets 1, 2-3, 4-7, ..., 4096).  The built-in table is described at ffn_sparse_plan;
 * calibration measures it, and a caller may set it. */
ffn_status ffn_plan_crossover(const ffn_plan *plan, int32_t B, float *density);
ffn_status ffn_plan_set_crossover(ffn_plan *plan, int32_t B, float density);

/* Device address (inside the plan's workspace, read-only for the caller) of the int32 in which
 * the device records the path it chose on the plan's last AUTO call of 64 tokens or more: 1 =
 * the dense GEMMs ran, 0 = the sparse passes ran.  Calls with another path, or fewer tokens,
 * leave it as it was; it is unspecified before the first such call.  FFN_ERR_UNSUPPORTED for a
 * plan without the dense GEMMs (fp16 layers with max_batch >= 64 have them). */
ffn_status ffn_plan_path_flag(const ffn_plan *plan, const int32_t **flag);

/*
 * Batch-1 decode variant (a tuning knob; results agree within rounding).  0: the predictor's
 * second stage and a rank-balanced gather are separate launches (the default); 1: one fused
 * launch in which every workgroup scores 64 neurons and gathers its own active ones (one launch
 * and one scan fewer, no balancing).  1 needs fp32 / fp16 rows of 64..1024 16-byte chunks and
 * a predictor (FFN_ERR_UNSUPPORTED otherwise); calls with a caller mask use variant 0.
 */
ffn_status ffn_plan_set_decode_variant(ffn_plan *plan, int32_t variant);

/*
 * Hot head (unite.ai PowerInfer, sections "Offline stage" and "Neuron placement and management":
 * an offline profile separates the few neurons that fire for almost every input from the rest,
 * and neurons are placed by that profile).  The caller orders the layer's neurons by profiled
 * firing frequency, hottest first (every per-neuron array permuted alike: rows of W_up, W_gate,
 * W_down_t and their int4 scales, b_up, b_gate, rows of P2, c2), and passes the head length
 * n_hot.  From then on, whenever the predictor picks the sets (mask == NULL), neurons
 * [0, n_hot) are always active and only [n_hot, ffn) are predicted: the head's P2 rows and c2
 * entries are never read and its scores are not written (their slots in `scores` keep what they
 * held).  The head's rows are contiguous, so the gather reads them as one dense block.  Calls
 * with a caller mask are unaffected.  n_hot must be a multiple of 32 in [0, ffn]
 * (FFN_ERR_INVALID_ARGUMENT otherwise); 0 (the default) turns the head off.
 */
ffn_status ffn_plan_set_hot_head(ffn_plan *plan, int32_t n_hot);

/*
 * Neuron cache for layers whose FFN rows live in host memory (citnews.com.cn PowerInfer-2
 * article, section "Dynamic neuron cache": an in-memory pool of neurons under LRU replacement,
 * segmented by weight type; neuron-cluster pipelining: neurons waiting for I/O overlap neurons
 * being computed).  Here the pool is `capacity` slots of HBM holding the up / gate / down rows
 * of recently used neurons; the predictor (p1, p2, c1, c2) and the biases stay device-resident
 * (the always-resident segment), and w_up / w_gate / w_down_t are pinned host memory
 * (hipHostMalloc; anything else gives FFN_ERR_INVALID_ARGUMENT), read over PCIe.
 *
 * Per token, after the active set is known: every active neuron found in the pool is read from
 * its slot, whose last use becomes the token's stamp (a counter starting at 1); the misses, in
 * ascending neuron order, are read from host memory and admitted to the free or least recently
 * used slots not used by this token (ascending (last use, slot)), evicting those slots' neurons;
 * misses beyond them are read without admission.  Neurons [0, n_pinned) are copied into slots
 * [0, n_pinned) at plan time and never evicted (pair with ffn_plan_set_hot_head).  y is
 * bit-identical to a plan over the same rows held in device memory.
 *
 * fp16 rows and tokens and a predictor are required (FFN_ERR_UNSUPPORTED otherwise); capacity is
 * a multiple of 32 in [32, min(ffn, 8192)] (FFN_ERR_INVALID_ARGUMENT otherwise); the plan takes
 * one token per call (max_batch is treated as 1) and is freed with ffn_plan_destroy; it cannot
 * be a mixture expert, and runs decode variant 0 only.  ffn_sparse_forward with path SPARSE or
 * AUTO (predicted sets or a caller mask) goes through the pool; path DENSE and ffn_dense_forward
 * read every row once straight from host memory and leave the pool as it was (a dense call
 * would only churn it).
 * The plan call initialises the pool on `stream` and synchronises it.  The pool's state lives
 * in the workspace: successive calls share it, so calls must stay ordered; a stamp wraps after
 * 2^32 - 1 tokens, which this library does not handle.
 */
ffn_status ffn_offload_workspace_size(const ffn_layer_desc *desc, int32_t capacity,
                                      size_t *bytes);
ffn_status ffn_offload_plan(const ffn_layer_desc *desc, const ffn_layer_weights *weights,
                            int32_t capacity, int32_t n_pinned, void *workspace,
                            size_t workspace_bytes, void *stream, ffn_plan **out);

/* Device pointers (inside the plan's workspace, read-only for the caller) to the pool's tables:
 * slot_of [ffn] (slot of each neuron, or -1), neuron_of [capacity] (or -1), last_use [capacity]
 * (stamp of the last token that used the slot; pinned slots 0xFFFFFFFF) and stats [8]: the
 * last call's hits, misses, admitted misses and |A|, then the same four summed over every call
 * since the plan was made (modulo 2^32).  Any output pointer may be NULL.
 * FFN_ERR_INVALID_ARGUMENT for a plan without a pool. */
ffn_status ffn_offload_tables(const ffn_plan *plan, const int32_t **slot_of,
                              const int32_t **neuron_of, const uint32_t **last_use,
                              const int32_t **stats);

ffn_status ffn_plan_destroy(ffn_plan *plan);

/*
 * Instrumentation, for a caller that times one kernel of a path on its own.  Stages:
 *   batch-1 decode (four kernels per token): FFN_STAGE_PRED_Z (predictor stage 1),
 *     FFN_STAGE_PRED_S (predictor stage 2, threshold and active bitmap), FFN_STAGE_GATHER (the
 *     active neurons' up, gate and transposed-down rows: activation and one row axpy per
 *     neuron into partials of y), FFN_STAGE_REDUCE (sum of the partials);
 *   batched passes (fp16, several tokens): FFN_STAGE_BATCH_UPGATE (union rows of up / gate and
 *     h on the matrix cores), FFN_STAGE_BATCH_DOWN (h times the union's transposed-down rows);
 *   dense GEMMs (fp16, 64 tokens or more): FFN_STAGE_DENSE_UP (X W_up^T [, X W_gate^T] and h),
 *     FFN_STAGE_DENSE_DOWN (H W_down_t), FFN_STAGE_DENSE_REDUCE (sum of its K slices).
 * While `start` and `stop` (hipEvent_t handles passed as void*, created with timing enabled)
 * are set for a stage, every launch of that stage's kernel on this plan carries the two events
 * on the dispatch itself, so hipEventElapsedTime(start, stop) afterwards is the last such
 * launch's execution time.  NULL, NULL turns it off.  Not meant for calls under graph capture.
 */
typedef enum {
    FFN_STAGE_PRED_Z = 0,
    FFN_STAGE_PRED_S = 1,
    FFN_STAGE_GATHER = 2,
    FFN_STAGE_REDUCE = 3,
    FFN_STAGE_BATCH_UPGATE = 4,
    FFN_STAGE_BATCH_DOWN = 5,
    FFN_STAGE_DENSE_UP = 6,
    FFN_STAGE_DENSE_DOWN = 7,
    FFN_STAGE_DENSE_REDUCE = 8,
    /* attention block (ffn_attn_set_timing_events; predictor stage 1 is FFN_STAGE_PRED_Z) */
    FFN_STAGE_ATTN_PROJ = 9,     /* head scores and set, query / key / value rows            */
    FFN_STAGE_ATTN_SCORES = 10,  /* scores, softmax and values per (active head, chunk)      */
    FFN_STAGE_ATTN_OUT = 11,     /* active heads' output-projection rows into partials of y  */
    FFN_STAGE_ATTN_REDUCE = 12   /* sum of the partials                                      */
} ffn_stage;

ffn_status ffn_plan_set_timing_events(ffn_plan *plan, int32_t stage, void *start, void *stop);

/* Fixed name of a status code ("FFN_OK", "FFN_ERR_INVALID_ARGUMENT", ...; "FFN_STATUS_UNKNOWN"
 * for a value outside the enum).  A static string: never NULL, never freed, safe from any thread. */
const char *ffn_status_string(ffn_status status);

/* Message of the last error on the calling thread ("" if none).  Never NULL. */
const char *ffn_last_error(void);

/* ---------------------------------------------------------------------------------------------
 * Mixture of experts (TurboSparse-Mixtral; nubint.ai PowerInfer-2 review, section on the models
 * it runs; citnews.com.cn PowerInfer-2 article): a router picks top_k experts per token and
 *   logits_e = R[e] . x ;  the top_k largest win, ties going to the lower expert index;
 *   w = softmax over the chosen logits;   y = sum_t w_t FFN_{e_t}(x),
 * each expert a sparse FFN (predictor, active set, rows) of its own.  Routing stays on the
 * device: the router kernel copies the chosen experts' weight pointers into per-slot records in
 * the mixture's workspace and the expert kernels read them there; the host never sees the
 * choice.  The weighted expert results are summed in slot order (no atomics).
 * Limits: 1 <= n_experts <= 16, 1 <= top_k <= min(n_experts, 4); every expert plan has the same
 * descriptor (shapes, dtypes, threshold, max_batch) and a predictor (rank > 0).
 */
typedef struct ffn_moe ffn_moe;

/* Bytes of device workspace the mixture needs (expert0 gives the shapes). */
ffn_status ffn_moe_workspace_size(int32_t n_experts, int32_t top_k, const ffn_plan *expert0,
                                  size_t *bytes);

/* w_router: device [n_experts][d] in the experts' x_dtype (fp16 for fp16 / int4 experts).
 * experts: host array of n_experts plans, which must outlive the mixture (only their weights and
 * shapes are used; their own workspaces are not touched).  workspace: device, >=
 * ffn_moe_workspace_size bytes, caller-owned, not shared with a plan used concurrently. */
ffn_status ffn_moe_plan(int32_t n_experts, int32_t top_k, const void *w_router,
                        ffn_plan *const *experts, void *workspace, size_t workspace_bytes,
                        ffn_moe **out);

/* B tokens x[B][d]; y[B][d] fp32 overwritten.  expert_idx [B][top_k] int32 and expert_w
 * [B][top_k] fp32 (device, each may be NULL) receive the routing decision, best expert first;
 * expert_cnt [B][top_k] int32 (device or NULL) the size of each chosen expert's active set. */
ffn_status ffn_moe_forward(ffn_moe *moe, const void *x, int32_t B, float *y,
                           int32_t *expert_idx, float *expert_w, int32_t *expert_cnt,
                           void *stream);
ffn_status ffn_moe_destroy(ffn_moe *moe);

/* ---------------------------------------------------------------------------------------------
 * Self-attention block with a head-level active set (unite.ai PowerInfer, section "Adaptive
 * sparse predictor": each layer has a second predictor, for its self-attention block; section
 * "Online stage": what is predicted inactive is not computed).  The pages do not name the
 * attention block's unit; here it is one head: its query rows, its scores over the cache and its
 * rows of the transposed output projection.  For one token x (d values, fp16) at position t:
 *   predictor  z = P1 x + c1 ;  s = P2 z + c2  (one score per head)
 *              A = { h : sigmoid(s_h) > threshold }, ascending
 *   cache      K[g][t] = fp16(W_k[g] x),  V[g][t] = fp16(W_v[g] x)  for EVERY key/value head g (a
 *              head skipped now may be active later, and its scores then need this position)
 *   heads      for h in A, g = h / (H / G):  q_h = W_q[h] x ;  a_j = q_h . K[g][j] / sqrt(e),
 *              j = 0..t ;  o_h = sum_j softmax(a)_j V[g][j]
 *   output     y = sum_{h in A} sum_{c < e} o_h[c] W_o_t[h e + c]
 * Row h e + c of W_q (and of W_o_t) is channel c of head h; W_o_t is the output projection stored
 * transposed, so an active head contributes e contiguous rows.  No positional rotation and no
 * biases are applied (the pages name neither).  Limits: d % 8 == 0, d <= 8192; 1 <= H <= 128;
 * G divides H; e in {64, 128}; rank % 8 == 0, rank <= 1024 (0: no predictor, forward calls then
 * need a mask); max_seq >= 1.  Everything is fp16 except the fp32 c1, c2, y and scores.
 * Conventions as above: every device pointer 16-byte aligned, nothing allocated or synchronised
 * by a forward call, one plan used by one stream at a time.
 */
typedef struct {
    int32_t d;          /* model width                                                       */
    int32_t heads;      /* H query heads                                                      */
    int32_t kv_heads;   /* G key / value heads                                                */
    int32_t head_dim;   /* e                                                                  */
    int32_t rank;       /* head-predictor rank                                                */
    int32_t max_seq;    /* S: positions of the caller's caches                                */
    float threshold;    /* tau in (0, 1]: head active iff sigmoid(s) > tau, strictly          */
} ffn_attn_desc;

typedef struct {                          /* device pointers, caller-owned                     */
    const void *w_q, *w_k, *w_v, *w_o_t;  /* fp16 [H e][d], [G e][d], [G e][d], [H e][d]        */
    const void *p1, *p2;                  /* fp16 [rank][d], [H][rank] (NULL when rank == 0)    */
    const float *c1, *c2;                 /* [rank], [H] fp32; may be NULL (= 0)                */
} ffn_attn_weights;

typedef struct ffn_attn ffn_attn;         /* opaque host object                                */

/* Bytes of device workspace a plan for `desc` needs. */
ffn_status ffn_attn_workspace_size(const ffn_attn_desc *desc, size_t *bytes);

/* Validate and return a plan over the caller's weights and workspace (device, >=
 * ffn_attn_workspace_size bytes, caller-owned, outliving the plan).  Enqueues nothing. */
ffn_status ffn_attn_plan(const ffn_attn_desc *desc, const ffn_attn_weights *weights,
                         void *workspace, size_t workspace_bytes, ffn_attn **out);

/*
 * One token x [d] (fp16, device) at position pos in [0, max_seq): writes position pos of the
 * caches k_cache, v_cache ([G][max_seq][e] fp16, device; positions 0..pos-1 must hold the
 * context's keys and values, positions past pos are neither read nor written) and y [d] (fp32,
 * fully overwritten).
 *   mask    [H] uint8 0/1 or NULL (NULL: the predictor picks the heads; needs rank > 0).
 *   idx     [H] int32 or NULL: the active heads, ascending, in idx[0 .. cnt).
 *   cnt     [1] int32 or NULL: |A|.
 *   scores  [H] fp32 or NULL: the predictor's scores s (written only when mask == NULL).
 * An empty set gives y = 0 (the caches are still written).
 * Errors: FFN_ERR_INVALID_ARGUMENT for NULL x / y / caches, misaligned pointers, pos out of
 * range, mask == NULL with rank == 0.
 */
ffn_status ffn_attn_forward(ffn_attn *plan, const void *x, int32_t pos, void *k_cache,
                            void *v_cache, float *y, const uint8_t *mask, int32_t *idx,
                            int32_t *cnt, float *scores, void *stream);

/* As ffn_plan_set_timing_events, for the stages FFN_STAGE_PRED_Z and FFN_STAGE_ATTN_*. */
ffn_status ffn_attn_set_timing_events(ffn_attn *plan, int32_t stage, void *start, void *stop);

ffn_status ffn_attn_destroy(ffn_attn *plan);

#ifdef __cplusplus
}
#endif

#endif /* FFN_SPARSE_H */
