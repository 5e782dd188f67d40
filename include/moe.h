/*
 * moe.h -- C ABI of the MI355X (gfx950) routed Mixture-of-Experts FFN forward pass.
 *
 * The layer (Kimi K3 pages):
 *  - "Kimi K3: The Open Model That Just Cornered the AI Frontier", section
 *    "Mixture-of-Experts with Dynamic Load Balancing": each token's hidden
 *    vector goes through a linear gate to one logit per expert, a softmax over
 *    the experts, and a top-k that returns the selected values and indices.
 *  - "Kimi K3: Open Frontier Intelligence", section "Operational Execution
 *    Flow": a token's routed output is the sum over its selected experts of the
 *    gate probability times that expert's output; the expert FFNs have SwiGLU's
 *    form (the SiTU-GLU sentence names the SwiGLU regime it keeps).
 *  - same page, section "Systems Optimization, Load Balancing, and
 *    Post-Training Alignment": per-expert token counts vary from step to step,
 *    and waiting on them on the host stalls the device; nothing here reads
 *    counts back to the host. The same section gives Quantile Balancing, the
 *    router-bias update of moe_qb_route / moe_qb_histogram / moe_qb_update;
 *    moe_aux_loss is the first page's auxiliary balance loss.
 *
 * Conventions shared by every call
 *  - All tensors are dense, on the device, 16-byte aligned; activations and
 *    every other buffer row-major (C order), bf16 weight matrices in the packed
 *    layout below. bfloat16 values are passed as uint16_t bit patterns.
 *  - Weights are output-major, input-contiguous matrices (the layout of a linear
 *    layer's weight): w_router [E, d] float32; w_gate, w_up [E, h, d] bf16;
 *    w_down [E, d, h] bf16. So logits = x w_router^T, gate = x w_gate[e]^T.
 *    The bf16 matrices of the expert and projection passes are held in the
 *    library's packed layout (matrix-core fragment order, see moe_pack_weights):
 *    a row-major checkpoint is converted once with moe_pack_weights, as a
 *    quantised one would be quantised once. The router weight stays row-major.
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues kernels on it and returns; nothing is synchronised, nothing is
 *    copied to the host, nothing is allocated or freed by the library. The
 *    caller owns every buffer, including the workspace.
 *  - Arguments are checked on the host before any launch. On error nothing is
 *    launched and a status other than MOE_OK is returned; moe_last_error()
 *    gives a message (thread-local). T == 0 is a successful no-op.
 *  - Calls on different streams may overlap when their buffers are disjoint.
 *  - Shapes: T >= 0 tokens; hidden width d and expert width h are multiples
 *    of 128; 1 <= E <= 1024 experts; 1 <= k <= min(E, 64); T * k < 2^31.
 *  - Results are deterministic: the same inputs give bitwise the same outputs
 *    (no floating-point atomics anywhere).
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 10

typedef struct moe_shape {
    int64_t T; /* tokens in the batch */
    int32_t d; /* hidden width */
    int32_t E; /* routed experts */
    int32_t k; /* experts selected per token */
    int32_t h; /* hidden width of one SwiGLU expert */
} moe_shape_t;

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad shape */
    MOE_ERR_UNSUPPORTED = 2, /* valid but outside the sizes this build handles */
    MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than moe_workspace_bytes() */
    MOE_ERR_HIP = 4          /* a HIP launch failed (message from the runtime) */
} moe_status_t;

/* Which call a workspace size is asked for. */
typedef enum moe_call {
    MOE_CALL_PERMUTE = 0,
    MOE_CALL_EXPERT_FFN = 1,
    MOE_CALL_FORWARD = 2,
    MOE_CALL_ROUTE = 3,
    MOE_CALL_AUX_LOSS = 4,
    MOE_CALL_MX_FORWARD = 5
} moe_call_t;

/* Intermediates that moe_forward keeps in its workspace (see moe_forward_ws_offset). */
typedef enum moe_fwd_slot {
    MOE_FWD_LOGITS = 0,         /* float   [T, E]   */
    MOE_FWD_TOPK_IDX = 1,       /* int32   [T, k]   */
    MOE_FWD_TOPK_W = 2,         /* float   [T, k]   */
    MOE_FWD_EXPERT_OFFSETS = 3, /* int32   [E + 1]  */
    MOE_FWD_ROW_OF = 4,         /* int32   [T, k]   */
    MOE_FWD_ROW_SRC = 5,        /* int32   [T * k]  */
    MOE_FWD_H = 6,              /* bf16    [T * k, h] */
    MOE_FWD_Y = 7,              /* float   [T * k, d] */
    MOE_FWD_NUM_SLOTS = 8
} moe_fwd_slot_t;
/* moe_forward keeps no x_perm: its gate/up pass reads x through row_src. */

/* Version of this ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static text for a status code. Never NULL. */
const char* moe_status_str(int status);

/* Message of the last error on the calling thread ("" if none). */
const char* moe_last_error(void);

/* Bytes of workspace that `call` (a moe_call_t) needs for this shape; 0 when the
 * shape is invalid (moe_last_error() then says why). Workspace must be 256-byte aligned. */
size_t moe_workspace_bytes(const moe_shape_t* shape, int call);

/* Byte offset inside moe_forward's workspace of one intermediate (slot is a
 * moe_fwd_slot_t), so a caller can read what the forward pass computed.
 * Returns MOE_OK or MOE_ERR_INVALID_ARG. */
int moe_forward_ws_offset(const moe_shape_t* shape, int slot, size_t* offset);

/*
 * moe_route -- gate logits, softmax over experts, top-k, renormalised weights.
 * Gate: "Kimi K3: The Open Model That Just Cornered the AI Frontier", section
 * "Mixture-of-Experts with Dynamic Load Balancing" (linear gate, softmax, top-k).
 *
 *  x           [T, d]  bf16    token hidden vectors (read)
 *  w_router    [E, d]  float32 gate weight (read)
 *  router_bias [E]     float32 added to every token's logits, or NULL (read)
 *  logits      [T, E]  float32 out: x w_router^T + bias, float32 accumulation of
 *                      exact bf16 x float32 products
 *  topk_idx    [T, k]  int32   out: slot j = expert with the j-th largest logit;
 *                      equal logits (and -0.0 vs +0.0) go to the lower expert id
 *  topk_w      [T, k]  float32 out: softmax probabilities of the selected experts,
 *                      renormalised to sum to 1 (exp(l_j - l_0) / sum_i exp(l_i - l_0))
 *  ws, ws_bytes        workspace of at least moe_workspace_bytes(shape, MOE_CALL_ROUTE)
 *                      (w_router split exactly into three bf16 parts for the matrix cores;
 *                      for batches too small to fill the GPU, float32 partial sums over
 *                      up to 32 K ranges, added in range order, so the logits do not
 *                      depend on scheduling)
 * NaN logits are outside the contract; the ids written are still k distinct
 * experts in [0, E).
 */
int moe_route(const moe_shape_t* shape, const uint16_t* x, const float* w_router,
              const float* router_bias, float* logits, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/*
 * moe_topk_softmax -- the second half of moe_route on caller-supplied float32
 * logits: softmax over experts, top-k, renormalised weights, with the same
 * selection and tie rules as moe_route (same section of the same page).
 *
 *  logits   [T, E] float32 (read)
 *  topk_idx [T, k] int32   (written)
 *  topk_w   [T, k] float32 (written)
 */
int moe_topk_softmax(const moe_shape_t* shape, const float* logits, int32_t* topk_idx, float* topk_w,
                     void* stream);

/*
 * moe_permute -- group the T*k (token, slot) assignments by expert, stably, and
 * gather the token rows into expert order: the dispatch of each token to the
 * experts chosen for it ("Kimi K3: Open Frontier Intelligence", section
 * "Operational Execution Flow", tokens dispatched to their active routed
 * experts). The per-expert counts stay on the device (same page, section
 * "Systems Optimization, Load Balancing, and Post-Training Alignment": token
 * counts that change from batch to batch stall the device when the host has
 * to wait for them).
 *
 *  x              [T, d]   bf16  (read; may be NULL when x_perm is NULL)
 *  topk_idx       [T, k]   int32 expert of each assignment, in [0, E) (read);
 *                          an id outside [0, E) is skipped: its row_of entry is -1
 *  expert_offsets [E + 1]  int32 out: rows of expert e are expert_offsets[e] ..
 *                          expert_offsets[e+1]-1; expert_offsets[0] = 0
 *  row_of         [T, k]   int32 out: row that holds assignment (t, j)
 *  row_src        [T * k]  int32 out: token of each row
 *  x_perm         [T * k, d] bf16 out: x_perm[r] = x[row_src[r]]; NULL skips the
 *                          gather (a caller that passes x and row_src to
 *                          moe_expert_ffn needs no x_perm)
 *  ws, ws_bytes   workspace of at least moe_workspace_bytes(shape, MOE_CALL_PERMUTE)
 * Within an expert, rows follow the flattened assignment index t*k + j.
 */
int moe_permute(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_idx,
                int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm,
                void* ws, size_t ws_bytes, void* stream);

/*
 * moe_permute_noalloc -- moe_permute for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that forbid
 * allocation): the same arguments without the workspace, the same results bit
 * for bit. Its scratch (the per-expert, per-chunk counts) lives in a fixed array
 * of MOE_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; the call allocates nothing, on the device or the host. Every
 * valid shape fits (E <= 1024 experts times at most 32 chunks of int32); a
 * larger need would be rejected with MOE_ERR_UNSUPPORTED. Calls on one GPU share
 * that GPU's array, so two calls that overlap in time on the same GPU (on
 * different streams, or from different threads) race and may give wrong
 * results; calls in order on one stream are safe. Nothing in the array needs to
 * start at zero.
 */
#define MOE_NOALLOC_SCRATCH_BYTES 131072
int moe_permute_noalloc(const moe_shape_t* shape, const uint16_t* x, const int32_t* topk_idx,
                        int32_t* expert_offsets, int32_t* row_of, int32_t* row_src, uint16_t* x_perm, void* stream);

/*
 * moe_expert_ffn -- every expert's SwiGLU FFN on its rows (grouped GEMM on bf16
 * MFMA with float32 accumulation). "Kimi K3: Open Frontier Intelligence",
 * section "Operational Execution Flow" (SwiGLU-form experts).
 *
 *  a, a_rows      the rows grouped by expert (read), given one of two ways:
 *                 a_rows == NULL: a = x_perm [T * k, d] bf16, row r is a[r];
 *                 a_rows != NULL: a = x [T, d] bf16 and a_rows = row_src [T * k]
 *                 int32 from moe_permute, row r is a[a_rows[r]] (the dispatch
 *                 gather done inside the GEMM; ids are clamped to [0, T))
 *  expert_offsets [E + 1]    int32 as written by moe_permute (read; only the
 *                            device copy is used, the host never sees it)
 *  w_gate, w_up   [E, h, d]  bf16, packed (moe_pack_weights with E groups, N = h, K = d) (read)
 *  w_down         [E, d, h]  bf16, packed (E groups, N = d, K = h) (read)
 *  h_act          [T * k, h] bf16 out: silu(x w_gate[e]^T) * (x w_up[e]^T), rounded once
 *  y_rows         [T * k, d] float32 out: h_act w_down[e]^T (float32 accumulation)
 *  ws, ws_bytes   workspace of at least moe_workspace_bytes(shape, MOE_CALL_EXPERT_FFN)
 */
int moe_expert_ffn(const moe_shape_t* shape, const uint16_t* a, const int32_t* a_rows,
                   const int32_t* expert_offsets, const uint16_t* w_gate, const uint16_t* w_up,
                   const uint16_t* w_down, uint16_t* h_act, float* y_rows, void* ws,
                   size_t ws_bytes, void* stream);

/*
 * moe_expert_gate_up -- the first half of moe_expert_ffn on its own:
 * h_act[r] = silu(A_r w_gate[e]^T) * (A_r w_up[e]^T) for every row r of expert
 * e (A_r as in moe_expert_ffn), rounded once to bf16. Arguments as in
 * moe_expert_ffn; the workspace is the same size (MOE_CALL_EXPERT_FFN).
 */
int moe_expert_gate_up(const moe_shape_t* shape, const uint16_t* a, const int32_t* a_rows,
                       const int32_t* expert_offsets, const uint16_t* w_gate, const uint16_t* w_up,
                       uint16_t* h_act, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_expert_down -- the second half of moe_expert_ffn on its own:
 * y_rows[r] = h_act[r] w_down[e]^T (float32) for every row r of expert e.
 * Arguments as in moe_expert_ffn; workspace size MOE_CALL_EXPERT_FFN.
 */
int moe_expert_down(const moe_shape_t* shape, const uint16_t* h_act, const int32_t* expert_offsets,
                    const uint16_t* w_down, float* y_rows, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine -- out[t] = sum_{j=0}^{k-1} topk_w[t, j] * y_rows[row_of[t, j]],
 * float32 accumulation in slot order, no atomics. "Kimi K3: Open Frontier
 * Intelligence", section "Operational Execution Flow" (weighted sum of experts).
 *
 *  y_rows [T * k, d] float32 (read); row_of [T, k] int32 (read; -1 entries are
 *  skipped); topk_w [T, k] float32 (read); out [T, d] float32 (written).
 */
int moe_combine(const moe_shape_t* shape, const float* y_rows, const int32_t* row_of,
                const float* topk_w, float* out, void* stream);

/*
 * moe_forward -- the whole routed layer: the gate, softmax and top-k of "Kimi
 * K3: The Open Model That Just Cornered the AI Frontier", section
 * "Mixture-of-Experts with Dynamic Load Balancing", then the probability-weighted
 * sum of the selected SwiGLU experts' outputs of "Kimi K3: Open Frontier
 * Intelligence", section "Operational Execution Flow". It runs moe_route,
 * moe_permute (without x_perm), moe_expert_ffn (reading x through row_src) and
 * moe_combine in sequence on one stream, intermediates in the workspace at the
 * offsets moe_forward_ws_offset() gives.
 *
 *  x [T, d] bf16; w_router [E, d] f32; router_bias [E] f32 or NULL;
 *  w_gate, w_up [E, h, d] bf16 packed; w_down [E, d, h] bf16 packed (all read)
 *  out [T, d] float32 (written)
 *  ws, ws_bytes  workspace of at least moe_workspace_bytes(shape, MOE_CALL_FORWARD)
 */
int moe_forward(const moe_shape_t* shape, const uint16_t* x, const float* w_router,
                const float* router_bias, const uint16_t* w_gate, const uint16_t* w_up,
                const uint16_t* w_down, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_aux_loss -- the auxiliary load-balancing loss that the gating forward
 * pass returns ("Kimi K3: The Open Model That Just Cornered the AI Frontier",
 * section "Mixture-of-Experts with Dynamic Load Balancing"): each expert's
 * softmax probability averaged over the T tokens, and the sum over experts of
 * its squared distance from the uniform share 1/E. The loss weight belongs to
 * the training objective and is not applied.
 *
 *  logits    [T, E] float32 (read)
 *  prob_mean [E]    float32 out: mean_t softmax(logits[t])[e] (summed in float64)
 *  aux_loss  [1]    float32 out: sum_e (prob_mean[e] - 1/E)^2 (evaluated in float64)
 *  ws, ws_bytes  workspace of at least moe_workspace_bytes(shape, MOE_CALL_AUX_LOSS)
 * T == 0 is a no-op (outputs untouched: an empty batch has no mean). d and h
 * of the shape are checked but not used.
 */
int moe_aux_loss(const moe_shape_t* shape, const float* logits, float* prob_mean, float* aux_loss,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * Quantile Balancing ("Kimi K3: Open Frontier Intelligence", section "Systems
 * Optimization, Load Balancing, and Post-Training Alignment"): balancing as
 * the dual of the token-to-expert assignment problem. One step is three calls:
 *   moe_qb_route      top-(k+1) routing on the biased scores: the k chosen
 *                     experts and each token's cutoff alpha;
 *   moe_qb_histogram  per-expert histogram of the margins logits - alpha
 *                     (ranks that share the batch would add their histograms
 *                     here, one integer all-reduce);
 *   moe_qb_update     each expert's new bias, minus the (1 - k/E)-quantile of
 *                     its margins read off the histogram.
 * The score is the router logit; the bias moves the selection only. These
 * calls need k < E and k <= 63 (the cutoff is the (k+1)-th score); d and h
 * of the shape are checked but not used.
 *
 * moe_qb_route:
 *  logits   [T, E] float32 (read); qb_bias [E] float32 (read)
 *  topk_idx [T, k] int32 out: the k largest fl32(logits[t, e] + qb_bias[e]),
 *           largest first, ties to the lower id
 *  topk_w   [T, k] float32 out: softmax of the unbiased logits renormalised
 *           over the chosen k
 *  alpha    [T]    float32 out: the (k+1)-th largest biased score
 *
 * moe_qb_histogram: hist[e, b] = number of tokens whose margin
 *  fl32(logits[t, e] - alpha[t]) falls in bin b = floor(fl32(fl32(margin - lo) / width)),
 *  clamped to [0, n_bins - 1]: bin b covers [lo + b width, lo + (b+1) width)
 *  and margins outside the range count in the end bins.
 *  logits [T, E], alpha [T] float32 (read); hist [E, n_bins] int32 (overwritten).
 *  lo finite, width finite and > 0, 1 <= n_bins <= 4096. T == 0 gives zeros.
 *
 * moe_qb_update: for each expert e with m = sum_b hist[e, b] > 0, b is the
 *  first bin whose cumulative count C_b has C_b * E >= m * (E - k) (exact
 *  integers) and Q = lo + width * (b + (m (E - k) / E - C_{b-1}) / hist[e, b])
 *  in float64; bias_out[e] = -Q rounded to float32. A row with m == 0 copies
 *  bias_in[e].
 *  hist [E, n_bins] int32 (read; counts >= 0); bias_in [E] float32 (read);
 *  bias_out [E] float32 (written; may be bias_in itself). shape->T is not used.
 */
int moe_qb_route(const moe_shape_t* shape, const float* logits, const float* qb_bias,
                 int32_t* topk_idx, float* topk_w, float* alpha, void* stream);
int moe_qb_histogram(const moe_shape_t* shape, const float* logits, const float* alpha, float lo,
                     float width, int32_t n_bins, int32_t* hist, void* stream);
int moe_qb_update(const moe_shape_t* shape, const int32_t* hist, float lo, float width,
                  int32_t n_bins, const float* bias_in, float* bias_out, void* stream);

/*
 * ------------------------------------------------------------ packed weights
 * The library's weight format for bf16 matrices (the expert, shared-expert and
 * projection weights): matrix-core fragment order. A weight matrix [N, K] is
 * cut into tiles of 16 rows x 32 columns, 512 contiguous elements each, in
 * (row block, column block) order; inside a tile, element (r, c) sits at
 * (r + 16 * (c / 8)) * 8 + c % 8, which is the order in which the 64 lanes of a
 * wavefront hold one 16 x 32 MFMA operand (lane l: row l % 16, columns
 * 8 * (l / 16) .. + 7). One kilobyte of HBM then is one operand, loaded in one
 * contiguous run straight into LDS. The values are those of the row-major
 * matrix, only their order differs.
 *
 * moe_pack_weights: w [groups, N, K] bf16 row-major (read) -> w_packed, the same
 *  number of elements in packed order (written; must not overlap w). N a
 *  multiple of 16, K of 32 (w_gate/w_up: N = h, K = d; w_down: N = d, K = h).
 */
int moe_pack_weights(int64_t groups, int32_t N, int32_t K, const uint16_t* w, uint16_t* w_packed,
                     void* stream);

/*
 * ---------------------------------------------------------------- LatentMoE
 * The Stable LatentMoE layer ("Kimi K3: Open Frontier Intelligence", section
 * "Operational Execution Flow: From Native Multimodal Inputs to Sparse Channel
 * Activations"): shared experts read x at full width, while the routed path
 * projects x down to a latent z, routes z through the k experts the gate picks
 * (from x), sums them into u, normalises u with an RMSNorm and projects back up:
 *   out = W_up_proj RMSNorm(u) + sum_s SharedExpert_s(x),
 *   u = sum_{j<k} w[t, j] E_{idx[t, j]}(z),  z = W_down_proj x,
 *   RMSNorm(u) = g * u / sqrt(mean u^2 + eps).
 * Every expert is SwiGLU. z, every expert's SwiGLU activation and RMSNorm(u)
 * are rounded to bf16 (they are matrix-core operands); u, the expert outputs
 * and out are float32.
 */
typedef struct moe_latent_shape {
    int64_t T;        /* tokens */
    int32_t d;        /* model width: x, out, shared experts (multiple of 128) */
    int32_t l;        /* latent width of the routed path (multiple of 128, <= 8192) */
    int32_t E;        /* routed experts, acting on R^l */
    int32_t k;        /* experts per token */
    int32_t h;        /* hidden width of a routed expert (multiple of 128) */
    int32_t n_shared; /* shared experts, 0 .. 8 */
    int32_t h_shared; /* hidden width of a shared expert (multiple of 128; unused when n_shared = 0) */
} moe_latent_shape_t;

/* Intermediates moe_latent_forward leaves in its workspace (moe_latent_ws_offset). */
typedef enum moe_latent_slot {
    MOE_LAT_LOGITS = 0,         /* [T, E] float32 */
    MOE_LAT_TOPK_IDX = 1,       /* [T, k] int32 */
    MOE_LAT_TOPK_W = 2,         /* [T, k] float32 */
    MOE_LAT_EXPERT_OFFSETS = 3, /* [E + 1] int32 */
    MOE_LAT_ROW_OF = 4,         /* [T, k] int32 */
    MOE_LAT_ROW_SRC = 5,        /* [T * k] int32 */
    MOE_LAT_Z = 6,              /* [T, l] bf16: x W_down_proj^T */
    MOE_LAT_H = 7,              /* [T * k, h] bf16: routed SwiGLU activations */
    MOE_LAT_Y = 8,              /* [T * k, l] float32: routed expert outputs */
    MOE_LAT_R = 9,              /* [T, l] bf16: RMSNorm(u) */
    MOE_LAT_SHARED_H = 10,      /* [n_shared * T, h_shared] bf16 */
    MOE_LAT_SHARED_Y = 11,      /* [n_shared * T, d] float32: shared expert s on rows s*T .. s*T + T - 1 */
    MOE_LAT_NUM_SLOTS = 12
} moe_latent_slot_t;

/* Workspace bytes of moe_latent_forward (0 with moe_last_error() set on a bad shape). */
size_t moe_latent_workspace_bytes(const moe_latent_shape_t* shape);
int moe_latent_ws_offset(const moe_latent_shape_t* shape, int slot, size_t* offset);

/*
 * moe_latent_forward -- the whole LatentMoE layer on one stream.
 *  x [T, d] bf16; w_router [E, d] f32; router_bias [E] f32 or NULL
 *  every bf16 matrix packed (moe_pack_weights; the projections as one group each):
 *  w_proj_down [l, d]; w_gate, w_up [E, h, l]; w_down [E, l, h]; w_proj_up [d, l];
 *  shared_gate, shared_up [n_shared, h_shared, d]; shared_down [n_shared, d, h_shared]
 *    (the shared three may be NULL when n_shared = 0)
 *  rms_gain [l] f32; rms_eps >= 0 (finite)
 *  out [T, d] float32 (written)
 *  ws, ws_bytes  workspace of at least moe_latent_workspace_bytes(shape)
 * Sums: u in slot order; out = ((W_up_proj r) + shared_0) + shared_1 ...
 */
int moe_latent_forward(const moe_latent_shape_t* shape, const uint16_t* x, const float* w_router,
                       const float* router_bias, const uint16_t* w_proj_down, const uint16_t* w_gate,
                       const uint16_t* w_up, const uint16_t* w_down, const float* rms_gain, float rms_eps,
                       const uint16_t* w_proj_up, const uint16_t* shared_gate, const uint16_t* shared_up,
                       const uint16_t* shared_down, float* out, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine_rmsnorm -- the routed sum followed by the RMSNorm, in one pass
 * (same page and section): u[t] = sum_j topk_w[t, j] y_rows[row_of[t, j]]
 * (float32, slot order, as moe_combine), r[t] = bf16(u[t] / sqrt(mean u[t]^2 + eps) * gain).
 *  shape->d is the row width (the latent width l, <= 8192)
 *  y_rows [T * k, d] f32; row_of [T, k] int32 (-1 entries skipped); topk_w [T, k] f32;
 *  gain [d] f32; eps >= 0 (finite)  (all read)
 *  u_out [T, d] f32 (written; may be NULL); r_out [T, d] bf16 (written)
 */
int moe_combine_rmsnorm(const moe_shape_t* shape, const float* y_rows, const int32_t* row_of,
                        const float* topk_w, const float* gain, float eps, float* u_out, uint16_t* r_out,
                        void* stream);

/*
 * --------------------------------------------------------------- MX experts
 * The serving variant of the routed layer ("Kimi K3: Open Frontier
 * Intelligence", section "Systems Optimization, Load Balancing, and
 * Post-Training Alignment"): MoE weights in MXFP4, activations in MXFP8. The
 * formats are the OCP Microscaling v1.0 ones: blocks of 32 consecutive elements
 * along K (the contraction dimension) share an E8M0 scale byte (2^(byte - 127));
 * elements are E2M1 (MXFP4) or E4M3 (MXFP8). Conversion of a block:
 * s = floor(log2 max|v|) - emax (emax 2 for E2M1, 8 for E4M3; s = -127 for an
 * all-zero block, clamped to [-127, 127]); each element is v / 2^s rounded to
 * the nearest element value, ties to the even code, clamped to the largest
 * value (6 or 448); a value that rounds to zero keeps its sign.
 * The MX calls need d and h to be multiples of 512, and T * k * max(d, h) < 2^32
 * (the grouped GEMM addresses its MXFP8 rows with 32-bit offsets); other shapes
 * return MOE_ERR_UNSUPPORTED.
 *
 * Layouts:
 *  - MXFP4 weights of G matrices [N, K] (N a multiple of 16), in matrix-core
 *    order, rows n counted within a matrix:
 *    codes, G * N * K/2 bytes: the 16 bytes of block kb (32 elements, element
 *    2i in the low nibble of byte i) of row n sit at byte
 *    ((n/16) * (K/128) + kb/4) * 1024 + (n%16) * 64 + (kb%4) * 16, so each
 *    16-row x 128-column tile is one contiguous kilobyte;
 *    scales, G * N * K/32 bytes: the scale of block kb of row n sits at byte
 *    ((n/16) * (K/512) + kb/16) * 256 + (n%16) * 16 + (kb%4) * 4 + (kb/4)%4.
 *  - MXFP8 rows [R, K]: codes [R, K] bytes; scales [R, K/32] bytes in row order.
 */

/* Quantise bf16 weights w [groups, N, K] to MXFP4 (K a multiple of 512, N of 16). */
int moe_mx_quantize_weights(int64_t groups, int32_t N, int32_t K, const uint16_t* w, uint8_t* q,
                            uint8_t* scales, void* stream);

/* Quantise rows [rows, K] (bf16, or float32 when in_is_f32) to MXFP8 (K a multiple of 32). */
int moe_mx_quantize_rows(int64_t rows, int32_t K, const void* in, int32_t in_is_f32, uint8_t* q,
                         uint8_t* scales, void* stream);

/*
 * moe_mx_expert_ffn -- every expert's SwiGLU FFN on its rows with MX operands.
 *  a_q, a_s   MXFP8 rows: [T * k, d] and [T * k, d/32] when a_rows is NULL, else
 *             the token rows [T, d] / [T, d/32] read through a_rows (= row_src)
 *  expert_offsets [E + 1] int32 (as moe_permute writes them)
 *  wg_*, wu_* MXFP4 gate and up weights of [E, h, d]; wd_* MXFP4 down weights of [E, d, h]
 *  h_act  [T * k, h] float32 out: silu(gate) * up, float32 accumulation of the exact products
 *  h_q, h_s [T * k, h], [T * k, h/32] out: h_act quantised to MXFP8 (codes decided on h_act)
 *  y_rows [T * k, d] float32 out
 *  ws, ws_bytes  workspace of at least moe_workspace_bytes(shape, MOE_CALL_EXPERT_FFN)
 */
int moe_mx_expert_ffn(const moe_shape_t* shape, const uint8_t* a_q, const uint8_t* a_s,
                      const int32_t* a_rows, const int32_t* expert_offsets, const uint8_t* wg_q,
                      const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s, const uint8_t* wd_q,
                      const uint8_t* wd_s, float* h_act, uint8_t* h_q, uint8_t* h_s, float* y_rows,
                      void* ws, size_t ws_bytes, void* stream);

/* The two halves of moe_mx_expert_ffn (with the H quantisation, moe_mx_quantize_rows on
 * h_act, in between), for callers that time or overlap them; same arguments and workspace. */
int moe_mx_expert_gate_up(const moe_shape_t* shape, const uint8_t* a_q, const uint8_t* a_s,
                          const int32_t* a_rows, const int32_t* expert_offsets, const uint8_t* wg_q,
                          const uint8_t* wg_s, const uint8_t* wu_q, const uint8_t* wu_s, float* h_act,
                          void* ws, size_t ws_bytes, void* stream);
int moe_mx_expert_down(const moe_shape_t* shape, const uint8_t* h_q, const uint8_t* h_s,
                       const int32_t* expert_offsets, const uint8_t* wd_q, const uint8_t* wd_s,
                       float* y_rows, void* ws, size_t ws_bytes, void* stream);

/* Intermediates moe_mx_forward leaves in its workspace (moe_mx_forward_ws_offset). */
typedef enum moe_mx_slot {
    MOE_MX_LOGITS = 0,         /* [T, E] float32 */
    MOE_MX_TOPK_IDX = 1,       /* [T, k] int32 */
    MOE_MX_TOPK_W = 2,         /* [T, k] float32 */
    MOE_MX_EXPERT_OFFSETS = 3, /* [E + 1] int32 */
    MOE_MX_ROW_OF = 4,         /* [T, k] int32 */
    MOE_MX_ROW_SRC = 5,        /* [T * k] int32 */
    MOE_MX_X_Q = 6,            /* [T, d] MXFP8 codes of x */
    MOE_MX_X_S = 7,            /* [T, d/32] their scales */
    MOE_MX_H = 8,              /* [T * k, h] float32 */
    MOE_MX_H_Q = 9,            /* [T * k, h] MXFP8 codes of H */
    MOE_MX_H_S = 10,           /* [T * k, h/32] their scales */
    MOE_MX_Y = 11,             /* [T * k, d] float32 */
    MOE_MX_NUM_SLOTS = 12
} moe_mx_slot_t;

int moe_mx_forward_ws_offset(const moe_shape_t* shape, int slot, size_t* offset);

/*
 * moe_mx_forward -- the routed layer with MXFP4 experts: moe_route, moe_permute
 * (no gather), x quantised to MXFP8, moe_mx_expert_ffn reading x's codes through
 * row_src, moe_combine.
 *  x [T, d] bf16; w_router [E, d] f32; router_bias [E] f32 or NULL;
 *  wg_*, wu_*, wd_* MXFP4 expert weights (moe_mx_quantize_weights layouts)
 *  out [T, d] float32 (written)
 *  ws, ws_bytes  workspace of at least moe_workspace_bytes(shape, MOE_CALL_MX_FORWARD)
 */
int moe_mx_forward(const moe_shape_t* shape, const uint16_t* x, const float* w_router,
                   const float* router_bias, const uint8_t* wg_q, const uint8_t* wg_s, const uint8_t* wu_q,
                   const uint8_t* wu_s, const uint8_t* wd_q, const uint8_t* wd_s, float* out, void* ws,
                   size_t ws_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
