/*
 * moe.h — C ABI of the sparse Mixture-of-Experts layer forward for AMD
 * Instinct MI355X (gfx950).
 *
 * The layer (page 1, "Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター",
 * STEP 1-12; nanoMoE slides, "nanoMoEの深層解剖：Mixture of Expertsにおける
 * 条件分岐を排除した並列演算実装", slides 11-40) computes, for every token row x_t:
 *
 *   s      = W_g x_t + noise_t                         (STEP 2-4; slide 11)
 *   I_t    = the k largest scores, in descending order  (STEP 5; slide 12)
 *   g_t,j  = softmax of the k kept scores               (STEP 6; slide 13)
 *   slot   = rank of (j, t) among all assignments to expert I_t[j], counted
 *            over every token's first choice in token order, then every
 *            second choice, ...; ranks >= C are dropped  (slides 14-23)
 *   y_t    = sum over kept j of g_t,j * W_down[e] ReLU(W_up[e] x_t),
 *            e = I_t[j]; 0 when every choice is dropped (STEP 7-12; slides 33-40)
 *
 * with capacity C = ceil(capacity_factor * k * N / E) for a call of N tokens
 * (slide 14's get_capacity(num_tokens); its body is not shown, this is the
 * plain reading).
 *
 * Conventions for every entry point:
 *  - All tensor data pointers are DEVICE pointers owned by the caller; the
 *    library never allocates, frees or retains device memory, and keeps no
 *    global mutable state (every value a call needs, the device's compute
 *    unit count and kernel occupancy included, is queried within the call),
 *    except the per-device address of moe_dispatch_noalloc's static scratch.
 *    Tensors are row-major and contiguous.
 *  - Work is enqueued on the given HIP stream (hipStream_t passed as void*;
 *    NULL = the default stream). Calls return without synchronising; the
 *    results are valid once the stream reaches them.
 *  - Arguments are validated on the host before anything is enqueued. On
 *    error nothing is enqueued and nothing is written; the return value is a
 *    negative MOE_ERR_* code (see moe_error_string). MOE_ERR_HIP reports a
 *    failed launch; earlier launches of the same call may already be queued.
 *  - Work on one stream is ordered; two calls sharing a workspace must not
 *    run concurrently on different streams.
 *  - Results are deterministic: no floating-point atomics, fixed summation
 *    orders; two calls on the same inputs give bitwise-identical outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* element types */
enum { MOE_F32 = 0, MOE_BF16 = 1 };

/* return codes */
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = -1,        /* a required pointer is NULL                      */
    MOE_ERR_SHAPE = -2,       /* tensor ranks or extents are inconsistent        */
    MOE_ERR_DTYPE = -3,       /* element type not allowed for this tensor        */
    MOE_ERR_ARG = -4,         /* k < 1, k > E, capacity_factor <= 0 or not finite, negative sizes */
    MOE_ERR_WORKSPACE = -5,   /* workspace smaller than moe_workspace_size()     */
    MOE_ERR_UNSUPPORTED = -6, /* outside the documented limits below             */
    MOE_ERR_ALIGN = -7,       /* pointer not aligned as required                 */
    MOE_ERR_HIP = -8          /* a HIP launch failed                             */
};

/* Limits (MOE_ERR_UNSUPPORTED beyond them): E <= 256 experts, k <= 16,
 * N * k < 2^31 assignments, E * min(C, N) < 2^31 slots. bf16 tensors need
 * d and d_ff to be multiples of 8 and 16-byte aligned data pointers. */
#define MOE_MAX_EXPERTS 256
#define MOE_MAX_TOPK 16

/* A tensor view: data (device), element type, rank and extents (row-major,
 * contiguous). A 3-D activation [B, T, d] is read as [B*T, d]. */
typedef struct {
    void *data;
    int32_t dtype;     /* MOE_F32 or MOE_BF16 */
    int32_t ndim;      /* 1..4 */
    int64_t shape[4];
} moe_tensor;

/* Launch context and optional exports of moe_forward.
 * Inputs:  stream, workspace (device, 256-byte aligned) and its size.
 * Optional device outputs (NULL = not exported; the library then keeps the
 * values in the workspace):
 *   topk_idx       int32 [N, k]  expert ids, highest score first
 *   topk_gate      fp32  [N, k]  gates of those experts (sum to 1 per token)
 *   slot           int32 [N, k]  capacity slot of each assignment, -1 = dropped
 *   used_capacity  int32 [E]     kept assignments per expert (= min(count, C))
 * Router statistics (optional device outputs, NULL = not computed). The
 * pages name load imbalance and capacity drops as what a router must be
 * watched for ("MoE（Mixture of Experts）とは？", section on MoE's weak
 * points; "게이팅 위기(Gating Crisis)", section on the load-balancing
 * challenge and its capacity-drop panel) and give no loss formula, so these
 * are the counts that define them, with used_capacity (nanoMoE slide 14):
 *   expert_demand    int32 [E]  assignments routed to expert e before the
 *                               capacity clip (count[e] of slide 14)
 *   expert_drops     int32 [E]  of those, the ones past the capacity
 *                               (= expert_demand - used_capacity)
 *   expert_gate_sum  fp32  [E]  sum of the gates of every assignment routed
 *                               to e (kept or dropped), fp32, summed in a
 *                               fixed order (identical on every run)
 * Host output: capacity (C), written before anything is enqueued.
 * aux_stream (input, moe_backward* only; ignored by the forward): a second
 * HIP stream of the same device, owned by the caller, that the backward may
 * run part of its work on (the router-weight and down-projection weight
 * gradients) while the rest runs on `stream`. The call forks it from and
 * joins it back to `stream` with two events it creates and destroys within
 * the call, so the call stays one stream-ordered operation on `stream` and
 * can be captured in a graph. NULL: everything runs on `stream`.
 * Dropped assignments per call = N*k - sum(used_capacity). */
typedef struct {
    void *stream;
    void *workspace;
    size_t workspace_bytes;
    int32_t *topk_idx;
    float *topk_gate;
    int32_t *slot;
    int32_t *used_capacity;
    int64_t capacity;
    int32_t *expert_demand;
    int32_t *expert_drops;
    float *expert_gate_sum;
    void *aux_stream;
} moe_stats;

/* The whole layer forward (page 1 STEP 1-12; nanoMoE slides 11-40).
 *   x      [N, d] (or [B, T, d])   MOE_F32 or MOE_BF16
 *   W_g    [E, d]                  MOE_F32 (the router runs in full precision, slide 11)
 *   noise  [N, E] MOE_F32, or NULL for sigma = 0. The caller draws it: it is
 *          sigma * eps with eps ~ N(0, 1) (STEP 3-4) plus any constant score
 *          offset; the library has no random number generator.
 *   W_up   [E, d_ff, d]            same dtype as x (row f of expert e is the
 *          f-th hidden neuron: z = W_up[e] x, STEP 8)
 *   W_down [E, d, d_ff]            same dtype as x (E_i(x) = W_down[e] h, STEP 10)
 *   k      experts per token, 1 <= k <= min(E, 16)
 *   capacity_factor  > 0, finite
 *   out    [N, d] (same shape as x) same dtype as x; every row is written
 *   stats  launch context and optional exports (required)
 * Numerics: scores, top-k and gates in fp32; expert products accumulate in
 * fp32 (bf16 inputs on matrix cores); the hidden activation is stored in
 * the dtype of x. Each expert's output row is stored in fp32 for an fp32
 * layer; for a bf16 layer it is stored compact in the workspace: every group
 * of 32 columns as fp16 values of y * 2^sh with one power-of-two shift sh
 * per group, chosen from the group's largest finite magnitude (relative
 * error at most 2^-11, no overflow at any magnitude). The combine
 * accumulates in fp32 in choice order and rounds once to the dtype of out
 * (round to nearest even).
 * N = 0 is valid: capacity is 0, used_capacity (if given) is zeroed. */
int moe_forward(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                const moe_tensor *W_up, const moe_tensor *W_down, int k,
                float capacity_factor, moe_tensor *out, moe_stats *stats);

/* The expert variant of the nanoMoE slides (slide 32: a bias after each
 * projection and GELU between them) for moe_forward_ex and moe_experts_ex.
 * activation: MOE_ACT_RELU (page 1 STEP 9) or MOE_ACT_GELU, x * Phi(x) with
 * Phi the standard normal distribution function (erf form), evaluated in
 * fp32 before H is rounded; MOE_ERR_ARG for any other value.
 * b_up:   [E, d_ff] MOE_F32 added to W_up[e] x before the activation, or NULL
 * b_down: [E, d]    MOE_F32 added to W_down[e] h, or NULL
 * Bias data are device pointers, 16-byte aligned (MOE_ERR_ALIGN), checked
 * for dtype and extents like every other tensor.
 * dropout: training-mode dropout on each expert output row (slide 32: the
 *   expert ends in a dropout), after b_down; 0 (the default of a
 *   zero-initialised struct) applies none; MOE_ERR_ARG outside [0, 1).
 *   Element i of the row of assignment a = t k + j is kept when its 32-bit
 *   random word is >= floor(dropout 2^32), and is then scaled by
 *   1 / (1 - dropout); dropped elements are 0. The words of elements
 *   8q .. 8q+7 are the Philox4x64-10 block (Salmon et al., SC 2011) at
 *   counter (q, a, dropout_offset, 0) under key (dropout_seed, 0): element
 *   i takes half i % 2 (low half first) of output word (i % 8) / 2. A call
 *   with the same seed and offset draws the same mask, so moe_backward_ex
 *   differentiates exactly the forward's dropped-out layer.
 * Zero-initialise the struct and set the fields used. */
enum { MOE_ACT_RELU = 0, MOE_ACT_GELU = 1 };
typedef struct {
    int32_t activation;
    const moe_tensor *b_up;
    const moe_tensor *b_down;
    float dropout;
    uint64_t dropout_seed;
    uint64_t dropout_offset;
} moe_expert_opts;

/* moe_forward with the expert variant above; opts NULL is moe_forward. */
int moe_forward_ex(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                   const moe_tensor *W_up, const moe_tensor *W_down,
                   const moe_expert_opts *opts, int k, float capacity_factor, moe_tensor *out,
                   moe_stats *stats);

/* Bytes of workspace moe_forward needs for these sizes (0 on invalid sizes). */
size_t moe_workspace_size(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                          float capacity_factor, int32_t dtype);

/* Per-expert capacity C = ceil(capacity_factor * k * N / E), in double
 * (nanoMoE slide 14, get_capacity of the call's token count). -1 on
 * invalid arguments; 0 when N = 0. */
int64_t moe_capacity(int64_t N, int64_t E, int k, float capacity_factor);

/* Static description of a return code. */
const char *moe_error_string(int code);

/* ---------------------------------------------------------------------------
 * The four stages moe_forward enqueues, exported for callers that run them
 * separately (and for per-stage testing). Same conventions as above.
 * ------------------------------------------------------------------------- */

/* Router (page 1 STEP 2-6; slides 11-13): fp32 scores s = W_g x + noise,
 * top-k in descending order (equal scores: lower expert id first), softmax
 * over the k kept scores. Writes topk_idx [N, k] int32 and topk_gate [N, k]
 * fp32 (device). x, W_g, noise as in moe_forward. workspace: device scratch
 * of moe_router_workspace_size() bytes, 256-byte aligned (may be NULL when
 * that size is 0). */
int moe_router(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
               int k, int32_t *topk_idx, float *topk_gate, void *workspace,
               size_t workspace_bytes, void *stream);

/* Bytes of router scratch for N tokens of width d and E experts (0 on invalid
 * sizes or when the dtype needs none). */
size_t moe_router_workspace_size(int64_t N, int64_t d, int64_t E, int32_t dtype);

/* Capacity-limited dispatch plan (slides 14-29). From topk_idx [N, k] and the
 * capacity C (moe_capacity), writes:
 *   slot        int32 [N, k]          rank among the expert's assignments in
 *                                     (choice, token) order, -1 if >= C
 *   used        int32 [E]             kept assignments per expert
 *   slot_token  int32 [E, min(C, N)]  for r < used[e]: the assignment id
 *                                     t*k + j holding slot r of expert e
 *                                     (rows past used[e] are left untouched)
 *   tiles       int32 [2*(E+1)]       prefix sums of ceil(used[e]/128) and
 *                                     ceil(used[e]/256): the expert kernels'
 *                                     tile schedule
 * and, each when not NULL, the router statistics of moe_stats:
 * expert_demand, expert_drops (int32 [E]) and expert_gate_sum (fp32 [E],
 * which reads topk_gate [N, k]; topk_gate may be NULL otherwise).
 * workspace: device scratch of moe_dispatch_workspace_size() bytes (256-byte
 * aligned; may be NULL when that size is 0, i.e. for N*k <= 4096). An id
 * outside [0, E) in topk_idx is not counted and its slot is -1. */
int moe_dispatch(int64_t N, int64_t E, int k, int64_t capacity, const int32_t *topk_idx,
                 const float *topk_gate, int32_t *slot, int32_t *used, int32_t *slot_token,
                 int32_t *tiles, int32_t *expert_demand, int32_t *expert_drops,
                 float *expert_gate_sum, void *workspace, size_t workspace_bytes,
                 void *stream);

/* Name of the kernel instantiation moe_forward launches for one expert
 * product of a layer of these sizes (product 0: the up product, 1: the down
 * product; dropout != 0: the down product's training-dropout variant), as a
 * profiler lists it, e.g. "expert_gemm_kernel<256, 256, 4, 4, 1, 64, 2, 0>".
 * Written to buf, NUL-terminated and truncated to len bytes; returns the
 * length of the full name, or a negative MOE_ERR_* code (N = 0 is
 * MOE_ERR_ARG: nothing is launched). For measurement tools that match
 * profiles to the layer's stages. */
int moe_expert_kernel_name(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                           float capacity_factor, int32_t dtype, int product, int dropout,
                           char *buf, size_t len);

/* moe_dispatch for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same plan, outputs and limits as moe_dispatch, but the per-chunk
 * scratch lives in a static device array of the library (4 MiB, held by
 * each GPU the library runs on until the process ends) instead of a
 * workspace argument, and the call allocates nothing. MOE_ERR_UNSUPPORTED
 * when moe_dispatch_workspace_size(N, E, k) exceeds 4 MiB (about 2 million
 * assignments at E = 256, more with fewer experts). The library keeps the
 * array's device address per device (taken once per device on its first
 * call there). Calls that overlap on one GPU (on different streams, or from
 * several host threads) share that GPU's array and race; calls ordered on
 * one stream do not (the array holds the last call's partials, which the
 * next call overwrites before it reads them). */
int moe_dispatch_noalloc(int64_t N, int64_t E, int k, int64_t capacity,
                         const int32_t *topk_idx, const float *topk_gate, int32_t *slot,
                         int32_t *used, int32_t *slot_token, int32_t *tiles,
                         int32_t *expert_demand, int32_t *expert_drops,
                         float *expert_gate_sum, void *stream);

/* Bytes of dispatch scratch for N tokens, E experts and top-k (0 on invalid
 * sizes or when a call needs none). */
size_t moe_dispatch_workspace_size(int64_t N, int64_t E, int k);

/* Grouped expert FFN (page 1 STEP 7-10; slides 32-37) over the dispatch plan.
 * For each expert e and r < used[e], with a = slot_token[e, r], t = a / k:
 *   H[e, r, :] = ReLU(W_up[e] x_t)      stored in the dtype of x   [E, min(C,N), d_ff]
 *   Y[a, :]    = W_down[e] H[e, r, :]   stored in fp32             [N*k, d]
 * Both products accumulate in fp32; H is rounded once to the dtype of x (the
 * slides' experts run under bf16 autocast), Y is kept in fp32 so that the
 * combine rounds each output once. The gather of token rows is fused into
 * the first product. Rows of Y whose assignment was dropped are not written.
 * H and Y are caller device buffers (16-byte aligned for bf16).
 * workspace: optional device scratch of workspace_bytes (256-byte aligned,
 * MOE_ERR_ALIGN otherwise) in which the bf16 path keeps fp32 partial tiles
 * when it cuts the K loop of a product's last, partly idle round of tiles
 * into ranges; NULL, or too few bytes for one partial tile per workgroup the
 * device runs at once, computes every tile whole (moe_expert_workspace_size()
 * bytes are enough on a device with up to 256 compute units). Either way the
 * result is deterministic; the two differ only in fp32 summation order.
 * Calls that share a workspace must not overlap. */
int moe_experts(const moe_tensor *x, const moe_tensor *W_up, const moe_tensor *W_down,
                int k, int64_t capacity, const int32_t *used, const int32_t *slot_token,
                const int32_t *tiles, void *H, void *Y, void *workspace,
                size_t workspace_bytes, void *stream);

/* moe_experts with the expert variant of moe_expert_opts (NULL: ReLU, no
 * biases). */
int moe_experts_ex(const moe_tensor *x, const moe_tensor *W_up, const moe_tensor *W_down,
                   const moe_expert_opts *opts, int k, int64_t capacity, const int32_t *used,
                   const int32_t *slot_token, const int32_t *tiles, void *H, void *Y,
                   void *workspace, size_t workspace_bytes, void *stream);

/* moe_expert_up and moe_expert_down with the expert variant of
 * moe_expert_opts: the up product adds b_up and applies the activation, the
 * down product adds b_down (b_up and the activation are ignored there). */
int moe_expert_up_ex(const moe_tensor *x, const moe_tensor *W_up, const moe_expert_opts *opts,
                     int k, int64_t capacity, const int32_t *used, const int32_t *slot_token,
                     const int32_t *tiles, void *H, void *workspace, size_t workspace_bytes,
                     void *stream);
int moe_expert_down_ex(int64_t N, const moe_tensor *W_down, const moe_expert_opts *opts, int k,
                       int64_t capacity, const int32_t *used, const int32_t *slot_token,
                       const int32_t *tiles, const void *H, void *Y, void *workspace,
                       size_t workspace_bytes, void *stream);

/* Bytes of expert scratch that enable the K-split on any device with up to
 * 256 compute units (0 for MOE_F32 and for an unknown dtype). */
size_t moe_expert_workspace_size(int32_t dtype);

/* The two halves of moe_experts, one product each (page 1 STEP 8-9 and STEP
 * 10): moe_expert_up writes H from x and W_up; moe_expert_down writes Y from
 * H and W_down ([E, d, d_ff]; H has W_down's dtype and [E, min(C,N), d_ff]
 * rows, Y is [N*k, d] fp32). workspace as for moe_experts. */
int moe_expert_up(const moe_tensor *x, const moe_tensor *W_up, int k, int64_t capacity,
                  const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                  void *H, void *workspace, size_t workspace_bytes, void *stream);
int moe_expert_down(int64_t N, const moe_tensor *W_down, int k, int64_t capacity,
                    const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                    const void *H, void *Y, void *workspace, size_t workspace_bytes,
                    void *stream);

/* moe_expert_down_ex writing Y compact, the form in which the fused entry
 * points of a bf16 layer keep it (see moe_forward's numerics): Y16 [N*k, d]
 * fp16 bits and Ysh [N][ceil(d / 32)][k] int8 shifts, assignment a = t*k + j
 * standing for y[a, c] = Y16[a, c] * 2^-Ysh[t][c / 32][j] (a token's k
 * shifts of one group adjacent). Y16 16-byte aligned. bf16 layers
 * only (MOE_ERR_DTYPE otherwise); rows of dropped assignments are not
 * written. Callers that time or check the fused layer's stages use it. */
int moe_expert_down_compact(int64_t N, const moe_tensor *W_down, const moe_expert_opts *opts,
                            int k, int64_t capacity, const int32_t *used,
                            const int32_t *slot_token, const int32_t *tiles, const void *H,
                            void *Y16, int8_t *Ysh, void *workspace, size_t workspace_bytes,
                            void *stream);

/* Combine (page 1 STEP 11-12; slides 38-40): out[t] = sum over j < k with
 * slot[t, j] >= 0 of topk_gate[t, j] * Y[t*k + j], accumulated in fp32 in
 * order j = 0..k-1, rounded once to out's dtype; rows with every choice
 * dropped become 0. Y is [N*k, d] MOE_F32 or MOE_BF16 (read as exact fp32
 * values), out is [N, d] MOE_F32 or MOE_BF16. */
int moe_combine(int64_t N, int64_t d, int k, const moe_tensor *Y, const float *topk_gate,
                const int32_t *slot, moe_tensor *out, void *stream);

/* moe_combine over compact rows (Y16, Ysh as moe_expert_down_compact writes
 * them), each value taken as Y16 * 2^-Ysh exactly; d % 8 == 0
 * (MOE_ERR_UNSUPPORTED otherwise), Y16 and out 16-byte aligned. */
int moe_combine_compact(int64_t N, int64_t d, int k, const void *Y16, const int8_t *Ysh,
                        const float *topk_gate, const int32_t *slot, moe_tensor *out,
                        void *stream);

/* Backward pass of the layer (the row after the forward: gradients through
 * the gates to the router and through the experts), for bf16 layers with
 * ReLU experts and no biases (moe_backward_ex: the GELU / bias / dropout
 * variants). For a loss whose
 * gradient with respect to out is dout, by the chain rule of moe_forward:
 *   combine: dy = g * dout, dg = <dout, y> (kept choices; dropped: 0);
 *   masked softmax over the kept scores: ds_j = g_j (dg_j - sum_l g_l dg_l),
 *   and no gradient through the top-k choice or to experts outside it;
 *   scores: dW_g = ds^T x, dx += ds W_g;
 *   experts: dZ = (dY W_down) where H > 0, dW_down = dY^T H, dW_up = dZ^T X,
 *   dx += the kept choices' dZ W_up rows, summed in choice order.
 * The forward state (routing, dispatch plan, H and the experts' output
 * rows, as the forward combined them) is recomputed from the inputs in
 * the workspace, so the call takes the forward's arguments plus:
 *   dout    [N, d]         same dtype as x (MOE_BF16)
 *   dx      [N, d]         MOE_F32, written
 *   dW_g    [E, d]         MOE_F32, written
 *   dW_up   [E, d_ff, d]   MOE_F32, written
 *   dW_down [E, d, d_ff]   MOE_F32, written
 *   stats   as for moe_forward, with moe_backward_workspace_size() bytes
 * Products run on the matrix cores with bf16 operands (dy and dZ are rounded
 * to bf16; fp32 ds is split exactly into three bf16 terms) and fp32
 * accumulation; every sum has a fixed order. MOE_ERR_UNSUPPORTED for fp32
 * layers. Device pointers 16-byte aligned (MOE_ERR_ALIGN).
 * Streams: with stats->aux_stream set, part of the work (the router-weight
 * gradient and dW_down) runs on that caller-owned stream, forked from and
 * joined to stats->stream inside the call (see moe_stats); with NULL every
 * launch goes to stats->stream. The results are the same bit for bit. */
int moe_backward(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                 const moe_tensor *W_up, const moe_tensor *W_down, int k, float capacity_factor,
                 const moe_tensor *dout, moe_tensor *dx, moe_tensor *dW_g, moe_tensor *dW_up,
                 moe_tensor *dW_down, moe_stats *stats);

/* moe_backward for the expert variants of moe_forward_ex (page 2, slide
 * 32): opts as there (NULL: ReLU, no biases, no dropout). With GELU,
 * dZ = dH gelu'(z), gelu'(z) = Phi(z) + z phi(z), on the bf16
 * pre-activations z the recomputed up product keeps. With dropout, the
 * same mask as the forward's (same seed and offset): dg = <dout, y m> and
 * dY = g dout m, m the dropout factor (1 / (1 - p) or 0) of each element. Bias gradients, fp32, written exactly when the layer has
 * that bias (else they must be NULL: MOE_ERR_ARG; a missing one:
 * MOE_ERR_NULL), each the sum over the expert's kept assignments in a fixed
 * order:
 *   db_up   [E, d_ff]   sum of the dZ rows
 *   db_down [E, d]      sum of the dY rows (g * dout)
 * Same workspace as moe_backward. */
int moe_backward_ex(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                    const moe_tensor *W_up, const moe_tensor *W_down,
                    const moe_expert_opts *opts, int k, float capacity_factor,
                    const moe_tensor *dout, moe_tensor *dx, moe_tensor *dW_g, moe_tensor *dW_up,
                    moe_tensor *dW_down, moe_tensor *db_up, moe_tensor *db_down,
                    moe_stats *stats);

/* Training step without recomputation: moe_forward_train is moe_forward_ex
 * for a bf16 layer (same arguments, same out bit for bit) that also leaves
 * the forward state the backward needs (routing, dispatch plan, H, the
 * experts' output rows and, for GELU, the pre-activations) in
 * stats->workspace, which must hold moe_backward_workspace_size() bytes
 * (and in stats' exported routing arrays when given).
 * moe_backward_after_forward then takes moe_backward_ex's arguments and
 * computes the same gradients from that state instead of recomputing it:
 * pass the same inputs, options and moe_stats (workspace and exported
 * arrays) as to the forward, with no other call on that workspace in
 * between. The state serves one backward call (the GELU pre-activations are
 * overwritten by dZ). For callers that keep activations between the passes
 * of a training step; it saves the two recomputed expert products. */
int moe_forward_train(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                      const moe_tensor *W_up, const moe_tensor *W_down,
                      const moe_expert_opts *opts, int k, float capacity_factor, moe_tensor *out,
                      moe_stats *stats);
int moe_backward_after_forward(const moe_tensor *x, const moe_tensor *W_g,
                               const moe_tensor *noise, const moe_tensor *W_up,
                               const moe_tensor *W_down, const moe_expert_opts *opts, int k,
                               float capacity_factor, const moe_tensor *dout, moe_tensor *dx,
                               moe_tensor *dW_g, moe_tensor *dW_up, moe_tensor *dW_down,
                               moe_tensor *db_up, moe_tensor *db_down, moe_stats *stats);

/* Bytes of workspace moe_backward needs (0 on invalid sizes or a dtype
 * other than MOE_BF16). */
size_t moe_backward_workspace_size(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                                   float capacity_factor, int32_t dtype);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
