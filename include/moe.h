/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward library, libmoe.so.
 *
 * One GPU's share of a Mixture-of-Experts layer forward:
 *   gate GEMM -> top-k + softmax -> capacity-limited dispatch into
 *   expert-contiguous rows -> grouped expert FFN (Linear d->d_ff, erf GELU,
 *   Linear d_ff->d) -> routing-weighted combine -> per-expert counts and
 *   balance loss.
 *
 * Pages cited (title, then section):
 *   [PithTrain]  "Native MoE training system PithTrain: core optimisations from
 *                sparse communication to dynamic memory management"
 *   [PyTorchMoE] "PyTorch distributed MoE training: principles, implementation
 *                and optimisation"
 *   [EP]         "Expert Parallelism: Scaling Mixture-of-Experts Models"
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 * Pointers.  Every tensor pointer is a DEVICE pointer owned by the caller;
 *   the library never allocates or frees device memory and keeps no pointer
 *   after a call returns.  Tensor pointers must be 16-byte aligned.
 *   `stream` is a hipStream_t (NULL = the default stream).  All calls are
 *   asynchronous on `stream`; results are valid after the caller synchronises.
 *   Calls are thread-compatible: concurrent calls need distinct outputs and
 *   workspaces.
 * Layouts (all row-major, dense):
 *   x      [T, d]         dtype            (bf16 = raw uint16 bits, or fp32)
 *   Wg     [d, E]         fp32
 *   bg     [E]            fp32, may be NULL (no gate bias)
 *   W1     [E, d, d_ff]   dtype            expert e: h = x W1[e] + b1[e]
 *   b1     [E, d_ff]      fp32
 *   W2     [E, d_ff, d]   dtype            expert e: o = h W2[e] + b2[e]
 *   b2     [E, d]         fp32
 *   y      [T, d]         fp32
 *   logits [T, E]         fp32
 *   topk_idx [T, k] int32 / topk_w [T, k] fp32: the j-th choice of token t
 *   routed, counts [E] int32; offsets [E+1] int32
 *   perm   [max_rows] int32; slot [T, k] int32
 *   x_perm [max_rows, d] dtype; out_perm [max_rows, d] fp32
 * Routing semantics (the readings of the pages this library implements):
 *   - experts are ranked by descending fp32 logit, ties to the LOWER expert
 *     index (-0 equals +0); topk_idx[t, 0..k-1] is that order;
 *   - topk_w[t, j] = softmax over the k selected logits divided by
 *     temperature ([PithTrain] 4.1; [EP] 2.2 for the temperature and the
 *     hybrid coarse top-8);
 *   - capacity cap = min(T, ceil(capacity_factor*T*k/E)); capacity_factor <= 0
 *     means no limit (cap = T) ([PithTrain] 4.3 item 1);
 *   - slots are kept in token order (t, then j) until an expert holds cap;
 *     dropped slots contribute nothing and the kept weights are not
 *     renormalised; a token with every slot dropped gets y = 0;
 *   - expert e owns rows [offsets[e], offsets[e+1]) of the packed,
 *     expert-contiguous buffers ([EP] 4.2, the expert bucket pool), in
 *     increasing token order; S = offsets[E] rows are used;
 *     max_rows = min(T*k, E*cap).
 * Precision: the gate accumulates in fp32; the expert GEMMs take bf16 (or
 *   fp32) operands with fp32 accumulation; bias, GELU, routing weights and
 *   the combine are fp32; h is stored in the layer dtype (bf16 rounded to
 *   nearest even) ([EP] 5.5: route in fp32, experts in bf16).  GELU is the
 *   erf form u Phi(u); fp32 layers evaluate erf with the device library's
 *   erff, bf16 layers with Abramowitz & Stegun eq. 7.1.26 (absolute error
 *   <= 1.5e-7 on erf, far below the bf16 rounding of h).
 * Errors: every entry point validates its arguments on the host first.  On a
 *   validation failure it returns a non-zero moe_status, launches nothing and
 *   writes nothing; moe_last_error() then holds a message for the calling
 *   thread.  A launch failure returns MOE_ERR_HIP.  Faults inside kernels
 *   surface at the caller's next synchronisation.
 * Shape limits: T >= 1, 1 <= E <= 1024, 1 <= k <= E, d and d_ff
 *   positive multiples of 8 with d * d_ff <= 2^29, temperature > 0 and
 *   finite, T*k < 2^31.
 * Streams and graphs: the compute entry points only launch kernels on
 *   `stream` (no allocation, no memset, no synchronisation), so after one
 *   eager call with a shape (which caches device attributes) a call can be
 *   captured into a HIP graph and replayed; every replay overwrites the
 *   outputs and needs the same workspace contents as an eager call (none).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                   */
    MOE_ERR_SHAPE = 2,       /* shape or hyper-parameter outside the limits  */
    MOE_ERR_UNSUPPORTED = 3, /* valid request this build does not provide    */
    MOE_ERR_ALIGN = 4,       /* a tensor pointer is not 16-byte aligned      */
    MOE_ERR_WORKSPACE = 5,   /* workspace NULL or smaller than required      */
    MOE_ERR_HIP = 6          /* a HIP runtime call or launch failed          */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef struct {
    int64_t T;               /* tokens                                        */
    int64_t d;               /* model width                                   */
    int64_t E;               /* experts                                       */
    int64_t k;               /* experts per token                             */
    int64_t d_ff;            /* expert hidden width (4d on the pages)         */
    float capacity_factor;   /* <= 0: no capacity limit                       */
    float temperature;       /* softmax(l_sel / temperature)                  */
    float aux_lambda;        /* balance-loss weight lambda                    */
    int32_t dtype;           /* moe_dtype of x, W1, W2, x_perm and h          */
} moe_shape;

/* ---- sizes and diagnostics (host only, no device work) ----------------- */

/* Per-expert capacity, min(T, ceil(capacity_factor*T*k/E)), or T without a
 * limit ([PithTrain] 4.3 item 1).  Returns -1 if the shape is invalid. */
int64_t moe_capacity(const moe_shape* s);

/* Rows of the expert-contiguous buffers: min(T*k, E*cap).  -1 if invalid. */
int64_t moe_max_rows(const moe_shape* s);

/* Bytes of workspace every entry point below accepts for this shape (the
 * largest need, that of moe_layer_forward).  0 if the shape is invalid. */
size_t moe_workspace_size(const moe_shape* s);

/* Byte offset inside the workspace of an intermediate that
 * moe_layer_forward leaves there, for inspection after the call completes:
 * which = MOE_WS_PERM (int32 [max_rows]), MOE_WS_SLOT (int32 [T,k]),
 * MOE_WS_OFFSETS (int32 [E+1]), MOE_WS_XPERM (dtype [max_rows,d]; fp32
 * layers only: -1 for a bf16 layer, whose forward keeps x_perm only as
 * MOE_WS_XPT),
 * MOE_WS_XPT (bf16 layers: x_perm in the tile layout of MOE_WS_H below with
 * ceil(d/32) column tiles, the first GEMM's operand; padding rows are
 * undefined, columns d..32*ceil(d/32)-1 of the kept rows are zero),
 * MOE_WS_H (h; fp32 layers: [max_rows,d_ff] row-major; bf16 layers: 16-row x
 * 32-column tiles over expert segments that start at multiples of 16 rows --
 * expert e's local row i is padded row p = P[e] + i with P[e] the sum of the
 * earlier experts' counts rounded up to 16, and (p, c) is element
 * ((p/16)*ceil(d_ff/32) + c/32)*512 + (p%16)*32 + c%32; padding rows are
 * undefined, columns d_ff..32*ceil(d_ff/32)-1 are zero), MOE_WS_OUT (fp32
 * [max_rows,d], the expert outputs before the weighted sum).  -1 if
 * invalid. */
enum { MOE_WS_PERM = 0, MOE_WS_SLOT = 1, MOE_WS_OFFSETS = 2, MOE_WS_XPERM = 3, MOE_WS_H = 4,
       MOE_WS_OUT = 5, MOE_WS_XPT = 6 };
int64_t moe_workspace_offset(const moe_shape* s, int which);

const char* moe_status_string(int status);
/* Message of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);
/* Library version string. */
const char* moe_version(void);

/* ---- the hot path ---------------------------------------------------------
 * 1. Gate + top-k + softmax.  logits[t,e] = sum_i x[t,i] Wg[i,e] + bg[e],
 *    accumulated in fp32 ([PithTrain] 4.1: linear gate, top-k, softmax over
 *    the selected values; [PyTorchMoE] 3.2: the gate may carry a bias;
 *    [EP] 5.5: routing kept in fp32).  Writes topk_idx and topk_w; also the
 *    logits when `logits` is not NULL.  For bf16 x with E <= 256 and
 *    k <= 16 or k > 32 the gate runs on the matrix cores with Wg split exactly into
 *    three bf16 parts (kept in the workspace), which gives fp32-accurate
 *    products; otherwise on the vector ALUs in fp32.  Either way the same
 *    selection rule and weights.  For k <= 32 the selection runs inside the
 *    gate kernel; for k > 32 (the soft layer over every expert, [EP] 2.2)
 *    the gate writes the logits (to `logits`, else to the workspace) and a
 *    second kernel selects by rank: expert e is the r-th choice with r the
 *    number of experts whose logit is larger, or equal with a lower index.
 *    The logits must be finite (a NaN logit leaves the selection
 *    unspecified).  ws: at least moe_workspace_size bytes. */
int moe_route(const moe_shape* s, const void* x, const float* Wg, const float* bg,
              float* logits /* NULL ok */, int32_t* topk_idx, float* topk_w,
              void* ws, size_t ws_bytes, void* stream);

/* 1b. Top-k + softmax of given fp32 logits [T,E] (same selection and weights
 *     as moe_route; lets a caller route on logits it already holds). */
int moe_route_logits(const moe_shape* s, const float* logits, int32_t* topk_idx,
                     float* topk_w, void* stream);

/* 2. Capacity-limited dispatch ([PithTrain] 4.3 item 1; [EP] 4.1-4.2: rows
 *    are written straight into their expert's contiguous segment, with no
 *    concatenation step).  From topk_idx it writes routed[e] (all slots,
 *    NULL ok), counts[e] (kept slots), offsets[E+1], perm (rows >= S set to
 *    -1), slot[t,j] (row or -1) and x_perm[row] = x[perm[row]] for row < S
 *    (rows >= S of x_perm are left as they were).  Each token's k experts
 *    must be distinct and in [0, E), as moe_route produces them; other
 *    indices give unspecified (but in-bounds) results. */
int moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx,
                 int32_t* routed /* NULL ok */, int32_t* counts, int32_t* offsets,
                 int32_t* perm, int32_t* slot, void* x_perm,
                 void* ws, size_t ws_bytes, void* stream);

/* 2b. moe_dispatch without a workspace, for callers that cannot allocate
 *     device memory (code under stream capture, tight serving loops,
 *     harnesses that forbid hipMalloc).  Same arguments and outputs as
 *     moe_dispatch, bit for bit, minus ws: the per-block expert histogram
 *     (int32 [nblk][E], nblk = the dispatch's token blocks of at least 64
 *     tokens each) lives in a static device array of
 *     MOE_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds
 *     until the process ends.  Any shape with E * ceil(T/64) <= 2^20 fits;
 *     a shape whose histogram does not fit returns MOE_ERR_WORKSPACE and
 *     launches nothing.  The first call on a device looks up the array's
 *     address there (hipGetSymbolAddress); no call allocates device or host
 *     memory.  Every call on one GPU shares the array: calls that overlap on
 *     one GPU (other streams, other threads) race and give undefined
 *     results; calls ordered on one stream are safe. */
#define MOE_NOALLOC_SCRATCH_BYTES (4u << 20)
int moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* topk_idx,
                         int32_t* routed /* NULL ok */, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* slot, void* x_perm, void* stream);

/* 3. Grouped expert FFN over the packed rows: for every row r of expert e
 *    (offsets[e] <= r < offsets[e+1]),
 *      out_perm[r] = GELU(x_perm[r] W1[e] + b1[e]) W2[e] + b2[e]
 *    with the erf GELU of the precision note above ([PithTrain] 4.1 expert =
 *    Linear, GELU, Linear; [PyTorchMoE] 3.2 Expert with biases).  offsets must be non-decreasing
 *    with offsets[0] = 0 and offsets[E] <= max_rows.  Rows >= offsets[E] of
 *    out_perm are not written.  h lives in the workspace. */
int moe_grouped_ffn(const moe_shape* s, const void* x_perm, const int32_t* offsets,
                    const void* W1, const float* b1, const void* W2, const float* b2,
                    float* out_perm, void* ws, size_t ws_bytes, void* stream);

/* 4. Routing-weighted combine back to token order ([PithTrain] 4.1: each
 *    expert output, scaled by the token's weight for that expert, is added
 *    into the token's row):  y[t] = sum_{j: slot[t,j] >= 0} topk_w[t,j] *
 *    out_perm[slot[t,j]], summed in j order.  y is overwritten. */
int moe_combine(const moe_shape* s, const float* out_perm, const int32_t* slot,
                const float* topk_w, float* y, void* stream);

/* 5. Balance loss aux = lambda * sum_e (counts[e] / (T k)) * (1/E) with the
 *    kept counts ([EP] 2.3, taken as printed). */
int moe_aux_loss(const moe_shape* s, const int32_t* counts, float* aux, void* stream);

/* 1c. Router variants of [PyTorchMoE] on fp32 logits [T,E] (e.g. the logits
 *     moe_route wrote):
 *     mode MOE_ROUTER_TOPK: as moe_route_logits (top-k, softmax over the k
 *       selected logits divided by temperature);
 *     mode MOE_ROUTER_TOP1_FULL (k must be 1; sections 2.3 and 4.3): the
 *       expert of the largest logit (ties to the lower index) with, as its
 *       weight, its probability under a softmax over all E logits divided by
 *       temperature.
 *     noise (NULL ok, [T,E] fp32): the training-time exploration noise of the
 *       stable layer (section 4.3): the routed values are
 *       fp32(L + fp32(noise_scale * noise[t,e])), product and sum each
 *       rounded to fp32 as the page's fp32 code does (0.1 on the page);
 *       `noise` holds the caller's standard-normal draws.
 *     noisy_logits (NULL ok, [T,E]) receives the routed values.
 *     Writes topk_idx [T,k] and topk_w [T,k].  k <= 32 (MOE_ERR_SHAPE
 *     otherwise). */
enum { MOE_ROUTER_TOPK = 0, MOE_ROUTER_TOP1_FULL = 1 };
int moe_route_logits_ex(const moe_shape* s, int mode, const float* logits, const float* noise,
                        float noise_scale, int32_t* topk_idx, float* topk_w,
                        float* noisy_logits /* NULL ok */, void* stream);

/* 5b. Balance-loss variants over per-expert loads `load` [E] int32:
 *     mode MOE_LOSS_SHARE: lambda * sum_e (load[e] / (T k)) * (1/E), as
 *       moe_aux_loss ([EP] section 2.3; pass the kept counts);
 *     mode MOE_LOSS_VARIANCE: lambda * mean_e (load[e] - mean load)^2, the
 *       load-variance loss of [PyTorchMoE] section 3.3 item 1 (the stable
 *       layer of section 4.3 applies it, lambda 0.01, to the top-1 choices:
 *       pass routed), in fp64, stored as fp32. */
enum { MOE_LOSS_SHARE = 0, MOE_LOSS_VARIANCE = 1 };
int moe_aux_loss_ex(const moe_shape* s, int mode, const int32_t* load, float* aux, void* stream);

/* 5c. Balance loss over a sliding window of calls ([EP] section 2.3: the
 *     expert shares are averaged over the last W batches, W = 100 on the
 *     page, before the loss is taken).  `state` is caller-owned device
 *     memory of moe_window_state_bytes(E, W) bytes, all zero before the
 *     first call (the caller clears it, e.g. torch.zeros); it holds the call
 *     count, the per-expert window sums and the last W count vectors, and
 *     must not be shared by calls that are not ordered on one stream.  Each
 *     call appends `counts` [E] (the kept counts of this batch) and writes
 *       pbar[e] = (sum of counts[e] over the last min(n, W) calls, this one
 *                  included) / (min(n, W) * T * k)          (NULL ok, fp32)
 *       aux     = lambda * sum_e pbar[e] * (1/E)
 *     in fp64, stored as fp32.  1 <= W <= 2^20.  The state's size depends
 *     only on E and W; a shape with other E or W must use its own state. */
size_t moe_window_state_bytes(int64_t E, int64_t W);
int moe_aux_loss_window(const moe_shape* s, const int32_t* counts, void* state, int64_t W, float* aux,
                        float* pbar /* NULL ok, [E] */, void* stream);

/* 6. Routing heat map and load telemetry, from topk_idx [T,k] (as written by
 *    moe_route).  [EP] section 3.2 step 1: the experts' co-selection counts
 *    per batch, the input of affinity-aware expert placement; the page calls
 *    the matrix non-symmetric, read here as ordered pairs:
 *      H[i*E + j] = number of tokens t with topk_idx[t,a] = i and
 *                   topk_idx[t,b] = j for some a < b
 *    (i ranked above j; H + H^T counts the tokens that chose both experts;
 *    the diagonal is 0 for distinct experts).  routed[e] = number of slots
 *    (t, j) with topk_idx[t,j] = e, before capacity ([EP] section 2.1, the
 *    per-expert load).  stats (NULL ok) = {mean load, population variance
 *    of the loads ([PyTorchMoE] section 3.3 item 1), coefficient of
 *    variation std / mean ([EP] section 2.1)}, computed in fp64 and stored
 *    as fp32.  H (int32 [E,E]) and routed (int32 [E]) are overwritten.
 *    Indices outside [0, E) are skipped (in-bounds, not counted).  Counts
 *    are exact integers, independent of the order of the atomic updates. */
int moe_coactivation(const moe_shape* s, const int32_t* topk_idx, int32_t* H, int32_t* routed,
                     float* stats /* NULL ok, [3] */, void* stream);

/* The whole layer in one call: steps 1-5 on one stream (the balance loss is
 * produced by the dispatch step).  Writes y, counts and aux; routed,
 * topk_idx, topk_w and logits are optional outputs (NULL ok).  perm, slot,
 * offsets, x_perm, h and the expert outputs stay in the workspace (see
 * moe_workspace_offset).  Returns like the steps above.  The result is
 * bitwise reproducible: no step depends on the order of atomic updates. */
int moe_layer_forward(const moe_shape* s, const void* x, const float* Wg, const float* bg,
                      const void* W1, const float* b1, const void* W2, const float* b2,
                      float* y, int32_t* counts, float* aux,
                      int32_t* routed, int32_t* topk_idx, float* topk_w, float* logits,
                      void* ws, size_t ws_bytes, void* stream);

/* ---- backward ------------------------------------------------------------
 * Gradients of sum(dy * y) for one forward call, with its routing decisions
 * (selection, capacity, drops) fixed: they are piecewise constant.  The
 * layer is differentiated as autograd would differentiate [PithTrain]
 * section 4.1's layer: the combine y[t] += w[t,j] o[r], the expert FFN
 * o = GELU(x W1 + b1) W2 + b2 (erf GELU, derivative Phi(a) + a phi(a))
 * and the gate w = softmax(l_sel / temperature) with l = x Wg + bg; the
 * balance loss depends on integer counts only and has no gradient.  Experts
 * that received no row get zero weight and bias gradients ([EP] section
 * 4.3, expert-grained gradients).
 * Inputs from the forward call: topk_idx, topk_w, slot, offsets, x_perm
 * (dtype [max_rows,d], or NULL: the kept rows of x are then copied by slot
 * into this call's workspace) and out_perm (fp32 [max_rows,d], the expert
 * outputs before the weighted sum) -- the outputs of moe_route /
 * moe_dispatch / moe_grouped_ffn, or the regions MOE_WS_SLOT,
 * MOE_WS_OFFSETS, MOE_WS_OUT of a moe_layer_forward workspace with x_perm
 * = MOE_WS_XPERM (fp32 layers) or NULL (bf16 layers, whose forward keeps
 * x_perm only in the tile layout); pass the forward's topk_idx and topk_w
 * outputs.  dy [T,d] fp32.
 * Outputs (fp32, overwritten): dx [T,d], dWg [d,E], dbg [E], dW1
 * [E,d,d_ff], db1 [E,d_ff], dW2 [E,d_ff,d], db2 [E,d].
 * Arithmetic.  fp32 layers: every GEMM in fp32 on the vector ALUs.  bf16
 * layers: the expert GEMMs run on bf16 matrix cores with fp32
 * accumulation, so their operands are rounded to bf16 -- the expert-output
 * gradient w[t,j] dy[t] and da = dh GELU'(a) (2^-9 relative each, like h;
 * GELU'(a) is kept in bf16 between the two GEMMs that make and use it, so
 * da carries one more such rounding); h is recomputed from x_perm, W1, b1
 * and rounded to bf16 as the forward stores it, GELU and GELU' use the
 * forward's erf approximation; db1 and
 * db2 are fp32 column sums of those bf16 values.  The gate's gradients
 * (dWg, dbg and the gate's part of dx) are fp32 sums over the k selected
 * experts of each token, the only logits with a gradient (bf16 x widened
 * exactly): dWg[:, e] and dbg[e] sum over the tokens that selected e in
 * token order, the gate's part of dx[t] sums over j in order.  ws: moe_backward_workspace_size bytes (its own workspace; the
 * forward's may be read through x_perm / out_perm, so the two must not
 * overlap). */
size_t moe_backward_workspace_size(const moe_shape* s);
int moe_layer_backward(const moe_shape* s, const void* x, const float* Wg, const void* W1, const float* b1,
                       const void* W2, const float* dy, const int32_t* topk_idx, const float* topk_w,
                       const int32_t* slot, const int32_t* offsets, const void* x_perm, const float* out_perm,
                       float* dx, float* dWg, float* dbg, float* dW1, float* db1, float* dW2, float* db2,
                       void* ws, size_t ws_bytes, void* stream);

/* ---- measurement hook ------------------------------------------------------
 * Stages of moe_layer_forward, in launch order. */
int moe_num_stages(void);
const char* moe_stage_name(int i);
/* Arm per-stage timing for the NEXT moe_layer_forward call on this thread:
 * events[2i] / events[2i+1] (hipEvent_t, created by the caller; NULL entries
 * are skipped) are recorded on the call's stream right before / after stage
 * i.  n_events must be 2*moe_num_stages().  The hook disarms itself after
 * that one call. */
int moe_set_stage_events(void** events, int n_events);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
