/*
 * csf.h -- C ABI of the contextual-sparsity sparse FFN library for AMD Instinct MI355X (gfx950).
 *
 * The library computes one feed-forward block the contextual-sparsity way: a small low-rank
 * predictor scores every FFN neuron from the layer input, the top-k (or thresholded) scores
 * name the active neurons, and only the active rows of the gate/up projection and the matching
 * rows of the neuron-major down projection are read and computed.
 *
 * Sources (three web pages on the method):
 *   [DV] "Contextual Sparsity: Activation-Aware LLM Inference and the Deja Vu Paradigm"
 *   [CP] "Contextual Sparsity and Activation Predictors"
 *   [AS] "Activation sparsity" (wiki page)
 *
 * Conventions shared by every entry point
 *   Handle        Every call that enqueues work takes a csf_handle (csf_create) as its first
 *                 argument.  A handle belongs to one device, which must be the current device
 *                 when it is used; it holds that device's facts (queried once: the compute-unit
 *                 count the persistent grids and the batched chunking are sized from), the
 *                 gathered FFN's options, the per-kernel timing hook and the stack's events,
 *                 capture stream and captured graph.  It holds no tensor.  A handle may be used
 *                 by one thread at a time; calls on different handles are independent.  A call
 *                 that enqueues nothing (B == 0, L == 0) does not look at the handle; otherwise
 *                 the handle is checked after every other argument, and a NULL, destroyed or
 *                 other-device handle gives CSF_ERR_INVALID_ARG with nothing enqueued.
 *   Pointers      All tensor pointers are DEVICE pointers (hipMalloc or equivalent) unless a
 *                 comment says "host".  The caller allocates and frees every buffer, including
 *                 the workspace; the library never allocates device memory.
 *   Streams       `stream` is a hipStream_t passed as void* (NULL = the null stream).  Every call
 *                 only enqueues work on it and returns; nothing synchronises the device.
 *                 Data-dependent sizes (threshold counts, union sizes) stay in device memory.
 *   Layouts       Row-major, contiguous.  x[B][d], V[r][d], U[f][r], W1[f][d], Wup[f][d] and
 *                 W2T[f][d] (the down projection stored neuron-major: row j holds the d output
 *                 weights of neuron j).  Weights and x share one storage type (csf_dtype);
 *                 scores, the hidden activations h, biases and outputs y are float32.
 *   Alignment     Every pointer must be 16-byte aligned, and each weight row must be a multiple of
 *                 16 bytes long (d and r multiples of 8 for 16-bit types, of 4 for float32);
 *                 otherwise CSF_ERR_MISALIGNED / CSF_ERR_UNSUPPORTED.
 *   Index lists   Active lists are int32, ascending, one row of `idx_stride` entries per token.
 *   Errors        Every entry point validates all of its arguments on the host BEFORE it
 *                 enqueues anything: a non-zero status means nothing was enqueued, except
 *                 CSF_ERR_HIP, which reports a failed launch.  Device faults surface at the
 *                 caller's next synchronisation.  csf_last_error() gives a message (per thread).
 *                 Test hook: while the environment variable CSF_FAULT_INJECT holds "all" or a
 *                 comma-separated list of entry-point names (read on every call), those entry
 *                 points return CSF_ERR_HIP once their arguments pass the host checks, before the
 *                 handle check and before anything is enqueued (no device needed).
 *                 Inputs must be finite; NaN/Inf are not checked (a NaN score ranks below every
 *                 number in the top-k selections and never passes a threshold).
 *   Determinism   The same inputs give bitwise-identical outputs: no floating-point atomics, every
 *                 reduction runs in a fixed order.
 */
#ifndef CSF_H
#define CSF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    CSF_OK = 0,
    CSF_ERR_INVALID_ARG = 1,          /* a size, k, pointer or enum value is out of range       */
    CSF_ERR_UNSUPPORTED = 2,          /* a valid request the library does not implement         */
    CSF_ERR_MISALIGNED = 3,           /* a pointer or a row length breaks the 16-byte rule       */
    CSF_ERR_WORKSPACE_TOO_SMALL = 4,  /* ws_bytes < csf_workspace_size(...)                      */
    CSF_ERR_HIP = 5                   /* the HIP runtime reported an error at launch             */
} csf_status;

typedef enum { CSF_F32 = 0, CSF_F16 = 1, CSF_BF16 = 2 } csf_dtype;

/* CSF_ACT_RELU:   h_j = max(0, W1[j].x + b1_j)                      ([DV] "Kernel-Level
 *                 Implementation": dot product then max(acc, 0)).
 * CSF_ACT_REGLU:  h_j = max(0, W1[j].x + b1_j) * (Wup[j].x), with W1 the gate projection
 *                 ([DV] "The SiLU/GELU Challenge: TurboSparse", the ReLU-fied gated form).
 * CSF_ACT_SILU:   h_j = silu(W1[j].x + b1_j), silu(p) = p / (1 + e^-p)  ([DV] "The Prediction
 *                 Problem": the sparse sketch's activation).
 * CSF_ACT_SWIGLU: h_j = silu(W1[j].x + b1_j) * (Wup[j].x)  ([DV] "The SiLU/GELU Challenge":
 *                 the LLaMA-style block before ReLU-fication).
 * SiLU is never exactly zero: over a predicted set the SiLU forms approximate the dense layer
 * (functional sparsity, [DV] "The Empirical Foundation"); the ReLU forms are exact over any set
 * that holds every neuron with a positive gate.  The float32 exponential is the device
 * library's expf. */
typedef enum { CSF_ACT_RELU = 0, CSF_ACT_REGLU = 1, CSF_ACT_SILU = 2, CSF_ACT_SWIGLU = 3 } csf_act;

/* Operation codes for csf_workspace_size. */
typedef enum {
    CSF_OP_PREDICT = 0,
    CSF_OP_SELECT_TOPK = 1,
    CSF_OP_SELECT_THRESHOLD = 2,
    CSF_OP_SPARSE_FFN = 3,
    CSF_OP_DENSE_FFN = 4,
    CSF_OP_LAYER = 5,
    CSF_OP_BATCHED_UNION = 6,
    CSF_OP_BATCHED_LAYER = 7,
    CSF_OP_STACK = 8,
    CSF_OP_ATTN_DECODE = 9,      /* csf_attention_workspace_size only */
    CSF_OP_ATTN_LAYER = 10       /* csf_attention_workspace_size only */
} csf_op;

/* How csf_stack_forward schedules the predictor of each layer. */
typedef enum {
    CSF_STACK_SYNC = 0,      /* layer l's set is predicted from layer l's own input             */
    CSF_STACK_LOOKAHEAD = 1, /* layer l's set is predicted from layer l-1's input, on the side
                                stream while layer l-1 runs (layer 0: from its own input)       */
    CSF_STACK_GRAPH = 0x100  /* flag, OR'd into the mode: enqueue the whole stack as one HIP
                                graph launch.  The first call captures it (kept by the handle);
                                later calls with identical arguments (every pointer, size and
                                value, the layers array's contents, the streams) replay it.     */
} csf_stack_mode;

/* One block of a stack: predictor and FFN weights, shapes and layouts as for
 * csf_sparse_ffn_layer (Wup only for the gated forms, b1 optional). */
typedef struct {
    const void *V, *U, *W1, *Wup, *W2T;
    const float *b1;
} csf_layer_weights;

/* Which rows each token of a batched call uses (csf_sparse_ffn_batched_union). */
typedef enum {
    CSF_SEM_PER_TOKEN = 0,   /* token t keeps only its own active neurons (batch-invariant)    */
    CSF_SEM_UNION = 1        /* every token uses every neuron of the batch's union              */
} csf_union_sem;

/* Kernel family of csf_sparse_ffn_batched_union. */
typedef enum {
    CSF_PATH_AUTO = 0,       /* chosen from the batch size and dtype                             */
    CSF_PATH_GATHER = 1,     /* vector-ALU gather kernels, B accumulators per column             */
    CSF_PATH_MFMA = 2        /* matrix-core (MFMA) kernels; 16-bit types, d % 256 == 0           */
} csf_path;

/* ABI version of this header (bumped on any incompatible change). */
#define CSF_ABI_VERSION 2
int csf_abi_version(void);

/* An opaque library handle (see "Handle" above). */
typedef struct csf_context *csf_handle;

/* csf_create -- a handle for HIP device `device` (0 <= device < the device count).  Queries the
 * device's compute-unit count; creates no stream, event or device buffer (the stack creates its
 * events and capture stream on first use, owned by the handle).
 *   out     HOST, out: the new handle (NULL on failure)
 * CSF_ERR_INVALID_ARG for a bad device index or NULL out; CSF_ERR_HIP when the runtime fails. */
int csf_create(csf_handle *out, int device);

/* csf_destroy -- releases a handle and whatever it created (events, capture stream, graph).  NULL
 * is accepted (no-op).  The caller must have finished (synchronised) the work the handle
 * enqueued that could still use its events or graph. */
int csf_destroy(csf_handle h);

/* The device of a handle and the compute units it reports (either pointer may be NULL). */
int csf_get_device_info(csf_handle h, int *device, int *compute_units);

/* Static text for a status code (never NULL). */
const char *csf_status_string(int status);

/* Message describing the last failure on the calling thread ("" if none).  Host memory owned by
 * the library, valid until the next call on this thread. */
const char *csf_last_error(void);

/* Bytes of device workspace the operation needs for these sizes (0 if none).  `d`, `f`, `r`, `B`
 * are the sizes passed to the entry point; `max_count` is the longest active list (k for top-k,
 * f for threshold or dense).  Returns 0 for invalid sizes.  h: the handle the calls will use (the
 * batched union's chunking follows its device), or NULL for a size that fits any device. */
size_t csf_workspace_size(csf_handle h, int op, int B, int d, int f, int r, int max_count,
                          int dtype);

/* ---------------------------------------------------------------------------------------------
 * csf_predict_active -- predictor scores for every neuron of every token.
 * [DV] "The Prediction Problem": a bias-free two-layer network per layer,
 *      scores = sigmoid(up(relu(down(x)))), down: d -> r (the bottleneck), up: r -> f.
 * [AS] "Implementation sketch", predict_active: the scores feed a threshold (or top-k) test.
 *
 *   x       [B][d]  dtype      layer input of B tokens
 *   V       [r][d]  dtype      predictor down projection
 *   U       [f][r]  dtype      predictor up projection
 *   scores  [B][f]  float32    out: sigmoid scores in [0, 1]
 * The hidden activation relu(V x) is kept in float32; all sums accumulate in float32.  From 4
 * tokens on, 16-bit weights with d and r multiples of 128 take the matrix cores, where the hidden
 * activation enters the product with U as 16-bit terms: two for binary16 (about 22 significant
 * bits) and three for bfloat16 (24).  A token whose largest hidden value reaches 2^15 (binary16;
 * 2^127 for bfloat16) is scaled by a power of two 2^k before the split and its sums by 2^-k
 * before the sigmoid (exact), so large values stay finite.
 * Workspace: csf_workspace_size(h, CSF_OP_PREDICT, B, d, f, r, 0, dtype) bytes.
 * ------------------------------------------------------------------------------------------- */
int csf_predict_active(csf_handle h, const void *x, int B, int d, const void *V, int r, const void *U, int f,
                       int dtype, float *scores, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_select_topk -- the k highest scores of each token.
 * [DV] "The Prediction Problem": the k largest predictor scores form the active set.
 * Ties go to the lower neuron index; -0.0 and +0.0 are equal; the list is ascending.
 *
 *   scores  [B][f]       float32   finite scores
 *   k       0 <= k <= f            (f <= 65536)
 *   idx     [B][k]       int32     out: ascending active list per token
 *   count   [B]          int32     out, optional (NULL): set to k
 *   bitmap  [B][(f+31)/32] uint32  out, optional (NULL): bit j%32 of word j/32 set iff j selected
 * Workspace: csf_workspace_size(h, CSF_OP_SELECT_TOPK, B, 1, f, 0, k, dtype) bytes; it is non-zero
 * when a few tokens have many scores (then the selection of a token runs over many workgroups,
 * with the same result) and 0 otherwise (pass NULL, 0).
 * ------------------------------------------------------------------------------------------- */
int csf_select_topk(csf_handle h, const float *scores, int B, int f, int k, int32_t *idx, int32_t *count,
                    uint32_t *bitmap, void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_select_threshold -- every neuron with score >= tau.
 * [AS] "Implementation sketch", predict_active: active = scores >= threshold.
 *
 *   idx     [B][f]       int32     out: ascending active list; entries past count[t] undefined
 *   count   [B]          int32     out (required): list length per token, in device memory
 *   bitmap  optional, as for csf_select_topk
 * Workspace: none.
 * ------------------------------------------------------------------------------------------- */
int csf_select_threshold(csf_handle h, const float *scores, int B, int f, float tau, int32_t *idx,
                         int32_t *count, uint32_t *bitmap, void *ws, size_t ws_bytes,
                         void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn -- the FFN restricted to each token's active list.
 * [DV] "The Prediction Problem" (sparse_mlp_forward): gather the active gate rows and the
 *      matching down weights, compute only those; "Kernel-Level Implementation": one dot
 *      product per selected neuron with float32 accumulation, then the activation.
 *
 *   x        [B][d]  dtype
 *   W1       [f][d]  dtype     gate (ReLU: the up) projection
 *   b1       [f]     float32   optional (NULL = no bias)
 *   Wup      [f][d]  dtype     gated forms (CSF_ACT_REGLU, CSF_ACT_SWIGLU) only, else NULL
 *   W2T      [f][d]  dtype     down projection, neuron-major
 *   idx      [B][idx_stride] int32  active lists (ascending, values in [0, f))
 *   count    [B]     int32     optional device lengths; NULL = every list has max_count entries
 *   max_count                  0 <= max_count <= idx_stride; device counts are clamped to it
 *   h        [B][idx_stride] float32  out, optional: activation of each listed neuron
 *   y        [B][d]  float32   out: y_t = sum over the list of h_j * W2T[j]
 * Tokens are independent (each reads its own rows).  For one read of shared rows across a
 * batch use csf_sparse_ffn_batched_union.
 * Workspace: csf_workspace_size(h, CSF_OP_SPARSE_FFN, B, d, f, 0, max_count, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn(csf_handle hd, const void *x, int B, int d, int f, int act, int dtype, const void *W1,
                   const float *b1, const void *Wup, const void *W2T, const int32_t *idx,
                   int idx_stride, const int32_t *count, int max_count, float *h, float *y,
                   void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_dense_ffn -- the same FFN over every neuron; the reference the sparse step must beat
 * ([CP] "The predictor and its budget": the dense layer's bytes are the budget).
 *   X [B][d] dtype, Y [B][d] float32; other arguments as csf_sparse_ffn.
 *   H [B][f] float32, optional (NULL): the activation of every neuron.  Its non-zero entries are
 *   the true active set ([DV] "The Empirical Foundation": a ReLU neuron is either exactly zero
 *   or contributes), against which a predicted set's recall and precision are measured
 *   ([CP] "Precision, recall, and which error hurts").
 * Workspace: csf_workspace_size(h, CSF_OP_DENSE_FFN, B, d, f, 0, f, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_dense_ffn(csf_handle h, const void *X, int B, int d, int f, int act, int dtype, const void *W1,
                  const float *b1, const void *Wup, const void *W2T, float *H, float *Y, void *ws,
                  size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn_layer -- predict, select and the sparse FFN for one token in one enqueue.
 * [DV] "The Prediction Problem" (the whole sparse_mlp_forward path).
 *
 *   x [d], predictor V [r][d] / U [f][r], FFN W1, b1, Wup, W2T as above.
 *   k >= 0        top-k selection with this k
 *   k == -1       threshold selection with tau
 *   y [d] float32 out
 *   scores_out [f] float32, idx_out [k or f] int32, count_out [1] int32: optional outputs (NULL =
 *   kept in the workspace only).
 * Workspace: csf_workspace_size(h, CSF_OP_LAYER, 1, d, f, r, k >= 0 ? k : f, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn_layer(csf_handle h, const void *x, int d, int f, int r, int act, int dtype, const void *V,
                         const void *U, const void *W1, const float *b1, const void *Wup,
                         const void *W2T, int k, float tau, float *y, float *scores_out,
                         int32_t *idx_out, int32_t *count_out, void *ws, size_t ws_bytes,
                         void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn_layer_noalloc -- csf_sparse_ffn_layer without a caller workspace, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The same kernels and bits as csf_sparse_ffn_layer, with the
 * library's static device scratch (8 MiB per GPU, created when the library is loaded on the GPU
 * and held until the process ends) as the workspace.  The call allocates nothing.
 *   Arguments as csf_sparse_ffn_layer, without ws / ws_bytes.
 *   A layer whose workspace (csf_workspace_size(h, CSF_OP_LAYER, 1, d, f, r, k >= 0 ? k : f,
 *   dtype)) exceeds the scratch is refused with CSF_ERR_UNSUPPORTED before anything is enqueued.
 * Every call on one GPU shares that GPU's scratch (through every handle of the GPU): calls whose
 * work overlaps on one GPU -- on different streams, or from different threads -- race and give
 * undefined results.  Calls ordered on one stream are safe: each call's first kernel writes
 * every scratch word a later kernel of the call reads before it is read.
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn_layer_noalloc(csf_handle h, const void *x, int d, int f, int r, int act,
                                 int dtype, const void *V, const void *U, const void *W1,
                                 const float *b1, const void *Wup, const void *W2T, int k,
                                 float tau, float *y, float *scores_out, int32_t *idx_out,
                                 int32_t *count_out, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn_layer_hot -- one token through a layer whose neurons are ordered hot first: the
 * leading `hot` neurons are always computed (no prediction), the predictor scores only the cold
 * remainder, and the top-k_cold (k_cold >= 0) or thresholded (k_cold == -1, tau) cold neurons
 * are added.
 * [CP] "Static locality: hot and cold neurons": activation frequency follows a power law, a small
 *      set fires for almost every token; the static split decides where a neuron lives, the
 *      predictor whether this token needs it.  [AS] "Hot and cold neuron split with per-layer
 *      predictors": neurons ranked by firing frequency, the frequent ones kept resident, a
 *      predictor per layer for the rest.
 *
 *   V [r][d]; U_cold [f - hot][r]: row i scores neuron hot + i (the predictor's up rows of the cold
 *   neurons only, so its bytes shrink by hot / f).  W1, b1, Wup, W2T [f][...] as csf_sparse_ffn,
 *   with the hot neurons in rows 0 .. hot-1 (see the reordering helpers of the Python package).
 *   0 <= hot < f; 0 <= k_cold <= f - hot.
 *   scores_out [f - hot], idx_out [hot + k_cold, or f in threshold mode], count_out [1]: optional;
 *   the list is 0 .. hot-1 followed by the selected cold neurons, ascending.
 * Workspace: csf_workspace_size(h, CSF_OP_LAYER, 1, d, f, r, hot + (k_cold >= 0 ? k_cold : f - hot),
 * dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn_layer_hot(csf_handle h, const void *x, int d, int f, int r, int act, int dtype,
                             const void *V, const void *U_cold, const void *W1, const float *b1,
                             const void *Wup, const void *W2T, int hot, int k_cold, float tau,
                             float *y, float *scores_out, int32_t *idx_out, int32_t *count_out,
                             void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn_batched_union -- the sparse FFN of B tokens reading the union of their active
 * sets once.
 * [CP] "When it breaks": the tokens of a batch select different neurons, so the layer reads the
 *      union of their sets; [DV] "Kernel-Level Implementation": each token keeps its own list;
 *      [DV] "Implications for System Design": sparse batching has a crossover batch size.
 *
 *   X         [B][d]  dtype       inputs, 1 <= B <= 32 (B = 0 is a no-op)
 *   W1, b1, Wup, W2T, act, dtype  as csf_sparse_ffn
 *   bitmaps   [B][(f+31)/32] uint32  each token's active set (the bitmap output of
 *                                  csf_select_topk / csf_select_threshold); bits past f ignored
 *   semantics CSF_SEM_PER_TOKEN: y_t = sparse FFN of x_t over its own set (rows of the union that
 *             t did not select contribute exactly zero); CSF_SEM_UNION: over the whole union.
 *   path      CSF_PATH_AUTO, CSF_PATH_GATHER or CSF_PATH_MFMA (CSF_ERR_UNSUPPORTED if the
 *             matrix-core path is asked for float32 or d % 256 != 0).  The matrix-core path
 *             multiplies h as a pair of 16-bit values (hi + lo): about 22 significant bits of h
 *             for binary16 and 16 for bfloat16.  A token whose largest |h| reaches 2^15
 *             (binary16; 2^127 for bfloat16) has its h scaled by a power of two 2^k before the
 *             split and its outputs by 2^-k after it (exact), so any finite h gives finite,
 *             accurate outputs; a binary16 value under 2^-24 2^-k rounds to zero in the split.
 *   Y         [B][d]  float32     out
 *   union_count [1] int32         out, optional device copy of the union size
 *   path_taken  HOST int*         out, optional: CSF_PATH_GATHER or CSF_PATH_MFMA
 * Each union row is read from HBM once per call for all B tokens.  f <= 65536.
 * Workspace: csf_workspace_size(h, CSF_OP_BATCHED_UNION, B, d, f, 0, 0, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn_batched_union(csf_handle h, const void *X, int B, int d, int f, int act, int dtype,
                                 const void *W1, const float *b1, const void *Wup,
                                 const void *W2T, const uint32_t *bitmaps, int semantics,
                                 int path, float *Y, int32_t *union_count, int *path_taken,
                                 void *ws, size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_ffn_batched_layer -- predict, select and the batched union FFN for B tokens in one
 * enqueue: csf_predict_active, csf_select_topk (k >= 0) or csf_select_threshold (k == -1, tau)
 * with bitmap output, then csf_sparse_ffn_batched_union.  Sources as those three.
 *
 *   X [B][d] dtype (1 <= B <= 32), predictor V [r][d] / U [f][r], FFN weights as above.
 *   semantics, path, Y, union_count, path_taken as csf_sparse_ffn_batched_union.
 *   bitmaps_out [B][(f+31)/32] uint32, optional: each token's selected set.
 * A batch of one on the gather path (CSF_PATH_GATHER, or CSF_PATH_AUTO at B = 1) is the
 * single-token layer: csf_sparse_ffn_layer's kernels and bits (without the post-gate skip), its
 * count as the union size.
 * Workspace: csf_workspace_size(h, CSF_OP_BATCHED_LAYER, B, d, f, r, k >= 0 ? k : f, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_ffn_batched_layer(csf_handle h, const void *X, int B, int d, int f, int r, int act, int dtype,
                                 const void *V, const void *U, const void *W1, const float *b1,
                                 const void *Wup, const void *W2T, int k, float tau,
                                 int semantics, int path, float *Y, uint32_t *bitmaps_out,
                                 int32_t *union_count, int *path_taken, void *ws,
                                 size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_stack_forward -- L residual blocks, each a contextual-sparsity FFN, on a float32 stream.
 * [CP] "Contextual Sparsity and Activation Predictors", section "The predictor and its budget":
 *      a sequential predict-then-compute pipeline puts the predictor on the critical path of
 *      every layer; predicting layer l+1's set from layer l's input and running that prediction
 *      asynchronously hides it, because the residual stream changes slowly between blocks;
 *      section "When it breaks": early layers are where that look-ahead is weakest.
 *
 *   layers    HOST array [L] of per-layer weight pointers (device memory); shapes d, f, r shared.
 *   x         [B][d] float32  in: the stream entering layer 0; out: the stream after layer L-1.
 *             For l = 0..L-1:  xhat_l = round(x_l / sqrt(mean(x_l^2) + eps)) (norm = 1) or
 *             round(x_l) (norm = 0), in the weight type;  A_l = top-k (k >= 0) or threshold (k =
 *             -1, tau) selection of predictor_l(xhat_l) (CSF_STACK_SYNC) or of predictor_l(xhat_{l-1})
 *             (CSF_STACK_LOOKAHEAD, l >= 1);  x_{l+1} = x_l + sparse FFN_l(xhat_l over A_l).
 *   mode      CSF_STACK_SYNC or CSF_STACK_LOOKAHEAD, optionally | CSF_STACK_GRAPH.  Look-ahead
 *             needs a side stream distinct from `stream`; the call orders it with events, and all
 *             of its work is ordered before the end of `stream`'s work, so synchronising `stream`
 *             is enough.  With CSF_STACK_GRAPH the host enqueues one launch per call instead of
 *             about 7 kernels and 4 event operations per layer; the captured graph (kept by the
 *             runtime, one per handle) is replaced when the arguments change.
 *   x_log     [L][B][d] float32, optional: x_l at the input of each layer.
 *   xhat_log  [L][B][d] dtype, optional: xhat_l.
 *   idx_log   [L][B][k or f] int32, optional: each layer's ascending active list.
 *   count_log [L][B] int32, optional: each layer's list length.
 * B >= 0 tokens, each with its own sets.  The handle keeps 4 HIP events, and for
 * CSF_STACK_GRAPH a capture stream and the instantiated graph (all created on first use; no device
 * buffers of its own).
 * Workspace: csf_workspace_size(h, CSF_OP_STACK, B, d, f, r, k >= 0 ? k : f, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_stack_forward(csf_handle h, const csf_layer_weights *layers, int L, int d, int f, int r, int act,
                      int dtype, float *x, int B, int mode, int k, float tau, int norm, float eps,
                      float *x_log, void *xhat_log, int32_t *idx_log, int32_t *count_log,
                      void *ws, size_t ws_bytes, void *stream, void *side_stream);

/* ---------------------------------------------------------------------------------------------
 * csf_set_ffn_flags -- options of the gathered FFN for later calls with this handle
 * (csf_sparse_ffn, csf_dense_ffn, csf_sparse_ffn_layer, csf_sparse_ffn_layer_hot,
 * csf_stack_forward; not the batched union path).  0 (the default) restores the plain method.
 *   CSF_FFN_SKIP_ZERO_H  post-gate skip: the gate activation a_j = act(W1[j].x + b1_j) of each
 *                        listed neuron is computed first; a neuron with |a_j| <= gate_tau (see
 *                        csf_set_ffn_gate_threshold; default 0) gets h_j = 0, its up row (gated
 *                        forms) and its down row are not read, and any other neuron whose h_j
 *                        is exactly 0 is dropped before its down row is read.  With gate_tau = 0
 *                        the ReLU forms lose nothing (the skipped terms are zero), so y is the
 *                        same up to float32 summation order.  A predictor tuned for recall
 *                        over-predicts ([CP] "Precision, recall, and which error hurts": a false
 *                        positive costs bandwidth), so most of the skipped rows are its false
 *                        positives.
 * ------------------------------------------------------------------------------------------- */
#define CSF_FFN_SKIP_ZERO_H 1
int csf_set_ffn_flags(csf_handle h, int flags);

/* ---------------------------------------------------------------------------------------------
 * csf_set_ffn_gate_threshold -- the gate_tau of CSF_FFN_SKIP_ZERO_H for later calls with this
 * handle (0 by default).  tau > 0 applies the functional activity test of [DV] "The
 * Empirical Foundation" (measure_mlp_sparsity: a neuron counts when the magnitude of its
 * activation exceeds a threshold, 0.1 there) inside the FFN: a SiLU gate is never exactly zero
 * ([DV] "The SiLU/GELU Challenge"), so the listed neurons are cut to those with |a_j| > tau
 * before their up and down rows are read.  This approximates the layer: each dropped neuron
 * changes y by at most tau * |Wup[j].x| * |W2T[j]| per element (without the Wup factor for the
 * ungated forms).  The test is taken in float32 on the kernel's own a_j.
 *   tau   >= 0 and finite, else CSF_ERR_INVALID_ARG (the previous value is kept).
 * ------------------------------------------------------------------------------------------- */
int csf_set_ffn_gate_threshold(csf_handle h, float tau);

/* ---------------------------------------------------------------------------------------------
 * csf_set_trace_events -- per-kernel timing hook for csf_sparse_ffn_layer,
 * csf_sparse_ffn_batched_union, csf_sparse_ffn_batched_layer and the attention calls made with
 * this handle.
 * While n > 0 events are set, the i-th kernel such a call launches has the HIP runtime record
 * events[2i] when it starts and events[2i+1] when it ends (while 2i+1 < n), so
 * hipEventElapsedTime(events[2i], events[2i+1]) is that kernel's own duration.  The kernels, in
 * order -- csf_sparse_ffn_layer: predictor down-projection, predictor up-projection, selection
 * (two kernels, histogram then finishing pass, for top-k over 20000 or more scores; none of its
 * own for f <= 1024, where the up projection selects), gathered up/gate rows, gathered down rows
 * (partial sums), reduction of the partial sums;
 * csf_sparse_ffn_batched_union: union list, up/gate rows, down rows, reduction;
 * csf_sparse_ffn_batched_layer: the predictor's kernels (two; three -- down projection, hidden
 * terms, up projection -- on the matrix cores from 4 tokens), selection, then the union's four;
 * a batch of one on the gather path: csf_sparse_ffn_layer's list;
 * csf_sparse_attention_decode: projections (q, k, v of the list; with kv_all q of the list then
 * k, v of every head), attention blocks, combine, output-projection rows, reduction; csf_sparse_attention_layer: the predictor's two kernels and selection first.
 * The events are hipEvent_t handles (as void*) created and owned by the caller, at most 16;
 * n = 0 switches timing off.
 * ------------------------------------------------------------------------------------------- */
int csf_set_trace_events(csf_handle h, void *const *events, int n);

/* ---------------------------------------------------------------------------------------------
 * Attention-head sparsity: one decode step of multi-head attention for a set of heads.
 * [DV] opening section: for a given input a small set of attention heads (with the MLP neurons)
 *      approximates the dense layer; "The Empirical Foundation": a fifth to a third of the heads
 *      matter per token; "Implications for System Design": choosing heads per token saves
 *      attention work and key/value cache traffic and memory.
 * For each listed head h and the new token x (standard multi-head attention, no positional
 * rotation; the pages give no formulas):
 *   q = Wq_h x + bq_h,  k = Wk_h x + bk_h,  v = Wv_h x + bv_h   (rows h*dh .. h*dh + dh - 1)
 *   k and v are rounded to the storage type and written at position len[h] of the head's cache;
 *   a_t = q . K_h[t] / sqrt(dh) for t = 0 .. len[h] (the new token included), p = softmax(a);
 *   o_h = sum_t p_t V_h[t];   y = sum over the listed heads of sum_i o_h[i] * WoT[h*dh + i].
 * A head outside the list computes nothing.  kv_all = 0: it stores nothing either (its cache
 * and length stay as they are: the cache-memory saving of the pages); kv_all = 1: every head
 * appends its k and v, so the caches stay complete and only q, the attention and the output
 * projection are sparse.  Each head that stores the token has len[h] advanced by one.
 *
 *   x        [d]           dtype     the layer input of one token
 *   Wq, Wk, Wv [H*dh][d]   dtype     head-major projections (head h owns rows h*dh .. h*dh+dh-1)
 *   bq, bk, bv [H*dh]      float32   optional biases (NULL = none)
 *   WoT      [H*dh][d]     dtype     output projection stored head-dimension major (row h*dh + i
 *                                    holds the d output weights of dimension i of head h)
 *   Kc, Vc   [H][Tmax][dh] dtype     key and value caches (in/out)
 *   len      [H]           int32     device, in/out: cached positions per head
 *   heads    [max_heads]   int32     device: distinct head indices (ascending gives the
 *                                    documented summation order); NULL = every head, in order
 *                                    (then max_heads must be H and count NULL: the dense step)
 *   count    [1]           int32     device, optional: entries of `heads` to use (clamped to
 *                                    [0, max_heads]); NULL = max_heads
 *   o        [max_heads][dh] float32 out, optional: o_h of each list entry (0 for a skipped one)
 *   y        [d]           float32   out
 * Device-side rules: an entry outside [0, H), or a head whose cache is full (len[h] >= Tmax)
 * or whose len is negative, is skipped (contributes nothing, stores nothing).
 * Build limits (CSF_ERR_UNSUPPORTED): dh * element size in {32, 64, 128, 256, 512} bytes,
 * H * dh <= 65536, d as for the FFN.  The score arithmetic is float32 (expf), o and y are float32
 * and the summation orders are fixed, so results are deterministic.
 * Workspace: csf_attention_workspace_size(CSF_OP_ATTN_DECODE, d, H, dh, 0, Tmax, max_heads,
 * dtype).
 * ------------------------------------------------------------------------------------------- */
size_t csf_attention_workspace_size(int op, int d, int H, int dh, int r, int Tmax, int max_heads,
                                    int dtype);
int csf_sparse_attention_decode(csf_handle h, const void *x, int d, int H, int dh, int dtype, const void *Wq,
                                const void *Wk, const void *Wv, const float *bq, const float *bk,
                                const float *bv, const void *WoT, void *Kc, void *Vc, int Tmax,
                                int32_t *len, const int32_t *heads, const int32_t *count,
                                int max_heads, int kv_all, float *o, float *y, void *ws,
                                size_t ws_bytes, void *stream);

/* ---------------------------------------------------------------------------------------------
 * csf_sparse_attention_layer -- the head predictor, the head selection and
 * csf_sparse_attention_decode over the selected heads, for one token, in one enqueue.
 * [DV] "The Prediction Problem": the same bias-free two-layer predictor, scoring heads instead of
 * neurons: scores = sigmoid(Up relu(Vp x)) with Vp [r][d], Up [H][r]; the k best heads (ties to
 * the lower index), or every head with score >= tau when k = -1, in ascending order.
 *   scores_out [H] float32, heads_out [k, or H for a threshold] int32, count_out [1] int32:
 *   optional copies (NULL = workspace).  Other arguments as csf_sparse_attention_decode.
 * Workspace: csf_attention_workspace_size(CSF_OP_ATTN_LAYER, d, H, dh, r, Tmax,
 * k >= 0 ? k : H, dtype).
 * ------------------------------------------------------------------------------------------- */
int csf_sparse_attention_layer(csf_handle h, const void *x, int d, int H, int dh, int r, int dtype,
                               const void *Vp, const void *Up, const void *Wq, const void *Wk,
                               const void *Wv, const float *bq, const float *bk, const float *bv,
                               const void *WoT, void *Kc, void *Vc, int Tmax, int32_t *len, int k,
                               float tau, int kv_all, float *scores_out, int32_t *heads_out,
                               int32_t *count_out, float *o, float *y, void *ws, size_t ws_bytes,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* CSF_H */
