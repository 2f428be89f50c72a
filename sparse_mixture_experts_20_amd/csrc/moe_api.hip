// C ABI of the MoE layer: argument validation, workspace layouts and the
// order of the stages of the forward (router -> dispatch plan -> grouped
// expert FFN -> combine) and of the backward. Every check runs on the host
// before anything is enqueued.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/moe.h"
#include "common.hpp"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t dtype_size(int32_t dt) { return dt == MOE_BF16 ? 2 : 4; }

bool valid_dtype(int32_t dt) { return dt == MOE_F32 || dt == MOE_BF16; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t capacity_of(int64_t N, int64_t E, int k, float cf) {
    if (N <= 0)
        return 0;
    return (int64_t)ceil((double)cf * (double)((int64_t)k * N) / (double)E);
}

// Sizes of one call, as validated.
struct Dims {
    int64_t N, d, E, d_ff;
    int k;
    int64_t C, ceff;
    int32_t dtype;
};

// Workspace regions (byte offsets from the base).
struct Layout {
    size_t idx, gate, slot, used, tiles, slot_token, H, Y, Ysh, router, dispatch, part, total;
};

// Expert output rows of the fused entry points: compact for bf16 layers (fp16
// values and one int8 exponent shift per kYGroup columns), fp32 otherwise.
size_t y_bytes(size_t nk, int64_t d, int32_t dtype) {
    return align_up(nk * (size_t)d * (dtype == MOE_BF16 ? 2 : 4));
}
size_t ysh_bytes(size_t nk, int64_t d, int32_t dtype) {
    return dtype == MOE_BF16
               ? align_up(nk * (size_t)((d + moe::kYGroup - 1) / moe::kYGroup))
               : 0;
}

// Router scratch: the bf16 split of W_g (and partial scores for many experts).
size_t router_bytes(int64_t N, int64_t d, int64_t E, int32_t dtype) {
    return dtype == MOE_BF16 ? align_up(moe::router_workspace_bytes(N, d, (int)E)) : 0;
}

// Expert scratch: fp32 partial tiles of the K-split last round (bf16 path).
size_t expert_bytes(int32_t dtype) {
    return dtype == MOE_BF16 ? align_up(moe::split_workspace_bytes()) : 0;
}

Layout layout_of(const Dims &m) {
    Layout L;
    size_t o = 0;
    const size_t nk = (size_t)m.N * m.k;
    L.idx = o;        o += align_up(nk * 4);
    L.gate = o;       o += align_up(nk * 4);
    L.slot = o;       o += align_up(nk * 4);
    L.used = o;       o += align_up((size_t)m.E * 4);
    L.tiles = o;      o += align_up((size_t)(2 * (m.E + 1)) * 4);
    L.slot_token = o; o += align_up((size_t)(m.E * m.ceff) * 4);
    L.H = o;          o += align_up((size_t)(m.E * m.ceff * m.d_ff) * dtype_size(m.dtype));
    L.Y = o;          o += y_bytes(nk, m.d, m.dtype);   // expert output rows
    L.Ysh = o;        o += ysh_bytes(nk, m.d, m.dtype);
    L.router = o;     o += router_bytes(m.N, m.d, m.E, m.dtype);
    L.dispatch = o;   o += align_up(moe::dispatch_workspace_bytes(m.N, (int)m.E, m.k));
    L.part = o;       o += expert_bytes(m.dtype);
    L.total = o;
    return L;
}

// Workspace of the backward pass (bf16 layers): the recomputed forward state
// and the gradient intermediates.
struct BwdLayout {
    size_t idx, gate, slot, used, tiles, slot_token, H, Y, Ysh, dY, ds, dZ, dXa, T1, T2, dsT3,
        xT3, gpart, router, dispatch, part, total;
    int64_t Kp, Tc, S;
};

// Token chunks of the router-weight product dW_g = ds^T x: Tc tokens (a
// multiple of 64) per chunk, enough chunks for ~512 product tiles, and the
// per-chunk fp32 partials within 32 MiB.
void dwg_chunks(int64_t N, int64_t E, int64_t d, int64_t &Tc, int64_t &S) {
    const int64_t tiles = ((E + 127) / 128) * ((d + 127) / 128);
    int64_t want = (512 + tiles - 1) / tiles;
    const int64_t cap = ((int64_t)32 << 20) / (E * d * 4);
    if (want > cap) want = cap;
    if (want > (N + 63) / 64) want = (N + 63) / 64;
    if (want < 1) want = 1;
    Tc = ((N + want - 1) / want + 63) / 64 * 64;
    if (Tc < 64) Tc = 64;
    S = (N + Tc - 1) / Tc;
}

BwdLayout bwd_layout_of(const Dims &m) {
    BwdLayout L;
    size_t o = 0;
    const size_t nk = (size_t)m.N * m.k;
    L.Kp = (m.ceff + 7) / 8 * 8;
    dwg_chunks(m.N, m.E, m.d, L.Tc, L.S);
    const size_t tok = (size_t)(L.S * L.Tc);     // chunked token columns
    L.idx = o;        o += align_up(nk * 4);
    L.gate = o;       o += align_up(nk * 4);
    L.slot = o;       o += align_up(nk * 4);
    L.used = o;       o += align_up((size_t)m.E * 4);
    L.tiles = o;      o += align_up((size_t)(2 * (m.E + 1)) * 4);
    L.slot_token = o; o += align_up((size_t)(m.E * m.ceff) * 4);
    L.H = o;          o += align_up((size_t)(m.E * m.ceff * m.d_ff) * 2);
    L.Y = o;          o += y_bytes(nk, m.d, m.dtype);   // compact expert output rows
    L.Ysh = o;        o += ysh_bytes(nk, m.d, m.dtype);
    L.dY = o;         o += align_up(nk * (size_t)m.d * 2);
    L.ds = o;         o += align_up(nk * 4);
    L.dZ = o;         o += align_up((size_t)(m.E * m.ceff * m.d_ff) * 2);
    L.dXa = o;        o += align_up(nk * (size_t)m.d * 4);
    // transposed operands of the weight products, only when an expert's rows
    // exceed what the products read K-major themselves
    const bool tr = m.ceff > moe::kGradMaxRows;
    L.T1 = o;         o += tr ? align_up((size_t)(m.E * m.d * L.Kp) * 2) : 0;
    L.T2 = o;         o += tr ? align_up((size_t)(m.E * m.d_ff * L.Kp) * 2) : 0;
    L.dsT3 = o;       o += align_up((size_t)m.E * 3 * tok * 2);
    L.xT3 = o;        o += align_up((size_t)m.d * 3 * tok * 2);
    L.gpart = o;      o += align_up((size_t)(L.S * m.E * m.d) * 4);
    L.router = o;     o += router_bytes(m.N, m.d, m.E, m.dtype);
    L.dispatch = o;   o += align_up(moe::dispatch_workspace_bytes(m.N, (int)m.E, m.k));
    L.part = o;       o += expert_bytes(m.dtype);   // split scratch of the expert products
    L.total = o;
    return L;
}

// An fp32 gradient tensor of the given extents.
int check_grad(const moe_tensor *g, int ndim, const int64_t *ext) {
    if (!g)
        return MOE_ERR_NULL;
    if (g->dtype != MOE_F32)
        return MOE_ERR_DTYPE;
    if (g->ndim != ndim)
        return MOE_ERR_SHAPE;
    for (int i = 0; i < ndim; ++i)
        if (g->shape[i] != ext[i])
            return MOE_ERR_SHAPE;
    return MOE_OK;
}

// Common size checks; fills C and ceff.
int check_sizes(Dims &m) {
    if (m.N < 0 || m.d <= 0 || m.E <= 0 || m.d_ff <= 0)
        return MOE_ERR_ARG;
    if (m.k < 1 || m.k > m.E)
        return MOE_ERR_ARG;
    if (m.E > MOE_MAX_EXPERTS || m.k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (m.d > INT32_MAX || m.d_ff > INT32_MAX || m.N * (int64_t)m.k >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (m.ceff * m.E >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (m.dtype == MOE_BF16 && ((m.d % 8) != 0 || (m.d_ff % 8) != 0))
        return MOE_ERR_UNSUPPORTED;
    return MOE_OK;
}

bool cf_ok(float cf) { return isfinite(cf) && cf > 0.f; }

// Rows of an activation tensor: [N, d] or [B, T, d] flattened.
bool act_rows(const moe_tensor *t, int64_t &N, int64_t &d) {
    if (t->ndim < 2 || t->ndim > 3)
        return false;
    d = t->shape[t->ndim - 1];
    N = 1;
    for (int i = 0; i < t->ndim - 1; ++i) {
        if (t->shape[i] < 0)
            return false;
        N *= t->shape[i];
    }
    return d > 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

// Expected kept rows per expert: min(C, ceil(N*k/E)).
int64_t rows_per_expert(int64_t N, int k, int64_t E, int64_t ceff) {
    const int64_t avg = (N * k + E - 1) / E;
    return avg < ceff ? avg : ceff;
}

#define MOE_TRY(expr)                         \
    do {                                      \
        hipError_t e_ = (expr);               \
        if (e_ != hipSuccess)                 \
            return MOE_ERR_HIP;               \
    } while (0)

int router_checked(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                   int64_t N, int64_t d, int64_t E, int k, int32_t *idx, float *gate,
                   void *ws, hipStream_t s) {
    const float *nz = noise ? static_cast<const float *>(noise->data) : nullptr;
    if (x->dtype == MOE_BF16)
        return hip_status(moe::launch_router_bf16(x->data, static_cast<const float *>(W_g->data),
                                                  nz, N, d, (int)E, k, idx, gate, ws, s));
    return hip_status(moe::launch_router_f32(static_cast<const float *>(x->data),
                                             static_cast<const float *>(W_g->data), nz, N, d,
                                             (int)E, k, idx, gate, s));
}

// Validates x, W_g, noise; returns N, d, E.
int check_router_args(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                      int k, int64_t &N, int64_t &d, int64_t &E) {
    if (!x || !W_g)
        return MOE_ERR_NULL;
    if (!act_rows(x, N, d))
        return MOE_ERR_SHAPE;
    if (N > 0 && !x->data)
        return MOE_ERR_NULL;
    if (!W_g->data)
        return MOE_ERR_NULL;
    if (!valid_dtype(x->dtype) || W_g->dtype != MOE_F32)
        return MOE_ERR_DTYPE;
    if (W_g->ndim != 2 || W_g->shape[1] != d || W_g->shape[0] <= 0)
        return MOE_ERR_SHAPE;
    E = W_g->shape[0];
    if (noise) {
        if (N > 0 && !noise->data)
            return MOE_ERR_NULL;
        if (noise->dtype != MOE_F32)
            return MOE_ERR_DTYPE;
        if (noise->ndim != 2 || noise->shape[0] != N || noise->shape[1] != E)
            return MOE_ERR_SHAPE;
    }
    if (k < 1 || k > E)
        return MOE_ERR_ARG;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK)
        return MOE_ERR_UNSUPPORTED;
    if (N * (int64_t)k >= ((int64_t)1 << 31) || d > INT32_MAX)
        return MOE_ERR_UNSUPPORTED;
    if (x->dtype == MOE_BF16) {
        if (d % 8 != 0)
            return MOE_ERR_UNSUPPORTED;
        if (!aligned(x->data, 16) || !aligned(W_g->data, 16))
            return MOE_ERR_ALIGN;
    }
    return MOE_OK;
}

// Expert variant options: activation and fp32 biases [E, d_ff] / [E, d].
struct ExpertOpts {
    int act = moe::kActRelu;
    const float *b_up = nullptr, *b_down = nullptr;
    moe::Dropout drop;
};

int check_bias(const moe_tensor *b, int64_t E, int64_t n, const float *&out) {
    out = nullptr;
    if (!b)
        return MOE_OK;
    if (b->dtype != MOE_F32)
        return MOE_ERR_DTYPE;
    if (b->ndim != 2 || b->shape[0] != E || b->shape[1] != n)
        return MOE_ERR_SHAPE;
    if (!b->data)
        return MOE_ERR_NULL;
    if (!aligned(b->data, 16))
        return MOE_ERR_ALIGN;
    out = static_cast<const float *>(b->data);
    return MOE_OK;
}

int check_opts(const moe_expert_opts *o, int64_t E, int64_t d, int64_t d_ff, ExpertOpts &r) {
    r = ExpertOpts{};
    if (!o)
        return MOE_OK;
    if (o->activation != MOE_ACT_RELU && o->activation != MOE_ACT_GELU)
        return MOE_ERR_ARG;
    r.act = o->activation == MOE_ACT_GELU ? moe::kActGelu : moe::kActRelu;
    if (!(o->dropout >= 0.f && o->dropout < 1.f))      // NaN fails too
        return MOE_ERR_ARG;
    if (o->dropout > 0.f) {
        const double p = o->dropout;
        r.drop.on = 1;
        r.drop.thresh = (uint32_t)floor(p * 4294967296.0);
        r.drop.scale = (float)(1.0 / (1.0 - p));
        r.drop.seed = o->dropout_seed;
        r.drop.offset = o->dropout_offset;
    }
    int rc = check_bias(o->b_up, E, d_ff, r.b_up);
    if (rc != MOE_OK)
        return rc;
    return check_bias(o->b_down, E, d, r.b_down);
}

// Optional expert scratch: NULL runs without the K-split; a non-NULL pointer
// must be 256-byte aligned.
int check_expert_ws(const void *ws) {
    if (ws && !aligned(ws, kAlign))
        return MOE_ERR_ALIGN;
    return MOE_OK;
}

}  // namespace

// The forward state the backward needs, in the backward's workspace layout:
// routing (into the exported arrays when given), dispatch plan, H, the
// experts' compact output rows Y (bias and dropout applied) and, for GELU, the
// bf16 pre-activations (in the dZ region, which the dZ product overwrites).
static int forward_state(const BwdLayout &L, char *ws, const moe_tensor *x,
                         const moe_tensor *W_g, const moe_tensor *noise, const moe_tensor *W_up,
                         const moe_tensor *W_down, const ExpertOpts &o, const Dims &m,
                         moe_stats *stats, hipStream_t s);

extern "C" {

const char *moe_error_string(int code) {
    switch (code) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "tensor ranks or extents are inconsistent";
    case MOE_ERR_DTYPE: return "element type not allowed for this tensor";
    case MOE_ERR_ARG: return "invalid argument (k, capacity factor or sizes)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_UNSUPPORTED: return "outside the documented limits";
    case MOE_ERR_ALIGN: return "pointer not aligned as required";
    case MOE_ERR_HIP: return "a HIP launch failed";
    default: return "unknown error code";
    }
}

int64_t moe_capacity(int64_t N, int64_t E, int k, float capacity_factor) {
    if (N < 0 || E <= 0 || k < 1 || k > E || !cf_ok(capacity_factor))
        return -1;
    return capacity_of(N, E, k, capacity_factor);
}

size_t moe_workspace_size(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                          float capacity_factor, int32_t dtype) {
    if (!valid_dtype(dtype) || !cf_ok(capacity_factor))
        return 0;
    Dims m{N, d, E, d_ff, k, 0, 0, dtype};
    if (N < 0 || E <= 0 || k < 1 || k > E)
        return 0;
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    if (check_sizes(m) != MOE_OK)
        return 0;
    return layout_of(m).total;
}

size_t moe_router_workspace_size(int64_t N, int64_t d, int64_t E, int32_t dtype) {
    if (!valid_dtype(dtype) || N < 0 || d <= 0 || E <= 0 || E > MOE_MAX_EXPERTS)
        return 0;
    return router_bytes(N, d, E, dtype);
}

size_t moe_expert_workspace_size(int32_t dtype) {
    return valid_dtype(dtype) ? expert_bytes(dtype) : 0;
}

int moe_router(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise, int k,
               int32_t *topk_idx, float *topk_gate, void *workspace, size_t workspace_bytes,
               void *stream) {
    int64_t N, d, E;
    int rc = check_router_args(x, W_g, noise, k, N, d, E);
    if (rc != MOE_OK)
        return rc;
    if (N == 0)
        return MOE_OK;
    if (!topk_idx || !topk_gate)
        return MOE_ERR_NULL;
    const size_t need = router_bytes(N, d, E, x->dtype);
    if (need > 0) {
        if (!workspace)
            return MOE_ERR_NULL;
        if (!aligned(workspace, kAlign))
            return MOE_ERR_ALIGN;
        if (workspace_bytes < need)
            return MOE_ERR_WORKSPACE;
    }
    return router_checked(x, W_g, noise, N, d, E, k, topk_idx, topk_gate, workspace,
                          static_cast<hipStream_t>(stream));
}

int moe_expert_kernel_name(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                           float capacity_factor, int32_t dtype, int product, int dropout,
                           char *buf, size_t len) {
    if (!buf && len > 0)
        return MOE_ERR_NULL;
    if (!valid_dtype(dtype))
        return MOE_ERR_DTYPE;
    if (!cf_ok(capacity_factor) || (product != 0 && product != 1) || N <= 0)
        return MOE_ERR_ARG;
    Dims m{N, d, E, d_ff, k, 0, 0, dtype};
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    const int rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    return moe::expert_kernel_name(dtype == MOE_BF16, product, d, d_ff, (int)E,
                                   rows_per_expert(N, k, E, m.ceff), dropout != 0, buf, len);
}

}  // extern "C"

// Scratch of moe_dispatch_noalloc: a file-scope device array (each GPU that
// runs the library holds its own copy until the process ends). Host code
// never uses the array's name as an address: the device address of each
// GPU's copy comes from hipGetSymbolAddress, taken once per device with that
// device current and kept in g_noalloc_scratch.
constexpr size_t kNoAllocScratchBytes = (size_t)4 << 20;
__device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kNoAllocDevices = 64;
static std::atomic<void *> g_noalloc_scratch[kNoAllocDevices];

// The current device's copy of `scratch` (NULL on failure).
static void *noalloc_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kNoAllocDevices)
        return nullptr;
    void *p = g_noalloc_scratch[dev].load(std::memory_order_acquire);
    if (p)
        return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_noalloc_scratch[dev].store(p, std::memory_order_release);   // same value in every racer
    return p;
}

extern "C" {

int moe_dispatch_noalloc(int64_t N, int64_t E, int k, int64_t capacity,
                         const int32_t *topk_idx, const float *topk_gate, int32_t *slot,
                         int32_t *used, int32_t *slot_token, int32_t *tiles,
                         int32_t *expert_demand, int32_t *expert_drops,
                         float *expert_gate_sum, void *stream) {
    if (N < 0 || E <= 0 || k < 1 || k > E || capacity < 0 || (N > 0 && capacity == 0))
        return MOE_ERR_ARG;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || N * (int64_t)k >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    const size_t need = moe::dispatch_workspace_bytes(N, (int)E, k);
    if (need > kNoAllocScratchBytes)
        return MOE_ERR_UNSUPPORTED;   // beyond the static scratch: use moe_dispatch
    void *ws = nullptr;
    if (need > 0 && !(ws = noalloc_scratch()))
        return MOE_ERR_HIP;
    return moe_dispatch(N, E, k, capacity, topk_idx, topk_gate, slot, used, slot_token, tiles,
                        expert_demand, expert_drops, expert_gate_sum, ws,
                        ws ? kNoAllocScratchBytes : 0, stream);
}

size_t moe_dispatch_workspace_size(int64_t N, int64_t E, int k) {
    if (N < 0 || E <= 0 || E > MOE_MAX_EXPERTS || k < 1 || k > E || k > MOE_MAX_TOPK ||
        N * (int64_t)k >= ((int64_t)1 << 31))
        return 0;
    return moe::dispatch_workspace_bytes(N, (int)E, k);
}

// Zeroes the router statistics a call exports when it has no tokens.
static int zero_router_stats(int64_t E, int32_t *demand, int32_t *drops, float *gate_sum,
                             hipStream_t s) {
    if (demand)
        MOE_TRY(moe::launch_fill_i32(demand, E, 0, s));
    if (drops)
        MOE_TRY(moe::launch_fill_i32(drops, E, 0, s));
    if (gate_sum)   // 0.0f has the bit pattern of integer 0
        MOE_TRY(moe::launch_fill_i32(reinterpret_cast<int32_t *>(gate_sum), E, 0, s));
    return MOE_OK;
}

int moe_dispatch(int64_t N, int64_t E, int k, int64_t capacity, const int32_t *topk_idx,
                 const float *topk_gate, int32_t *slot, int32_t *used, int32_t *slot_token,
                 int32_t *tiles, int32_t *expert_demand, int32_t *expert_drops,
                 float *expert_gate_sum, void *workspace, size_t workspace_bytes,
                 void *stream) {
    if (N < 0 || E <= 0 || k < 1 || k > E || capacity < 0 || (N > 0 && capacity == 0))
        return MOE_ERR_ARG;
    if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOPK || N * (int64_t)k >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    const int64_t ceff = capacity < N ? capacity : N;
    if (ceff * E >= ((int64_t)1 << 31))
        return MOE_ERR_UNSUPPORTED;
    if (!used || !tiles || (N > 0 && (!topk_idx || !slot || !slot_token)))
        return MOE_ERR_NULL;
    if (N > 0 && expert_gate_sum && !topk_gate)
        return MOE_ERR_NULL;
    const size_t need = moe::dispatch_workspace_bytes(N, (int)E, k);
    if (need > 0) {
        if (!workspace)
            return MOE_ERR_NULL;
        if (!aligned(workspace, kAlign))
            return MOE_ERR_ALIGN;
        if (workspace_bytes < need)
            return MOE_ERR_WORKSPACE;
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (N == 0) {
        MOE_TRY(moe::launch_fill_i32(used, E, 0, s));
        MOE_TRY(moe::launch_fill_i32(tiles, 2 * (E + 1), 0, s));
        return zero_router_stats(E, expert_demand, expert_drops, expert_gate_sum, s);
    }
    return hip_status(moe::launch_dispatch(topk_idx, topk_gate, N, (int)E, k, ceff, slot, used,
                                           slot_token, tiles, expert_demand, expert_drops,
                                           expert_gate_sum, workspace, s));
}

static int expert_up_impl(const moe_tensor *x, const moe_tensor *W_up, int k, int64_t capacity,
                          const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                          void *H, void *workspace, size_t workspace_bytes, void *stream,
                          const ExpertOpts &o) {
    if (!x || !W_up)
        return MOE_ERR_NULL;
    int64_t N, d;
    if (!act_rows(x, N, d))
        return MOE_ERR_SHAPE;
    if (!valid_dtype(x->dtype) || W_up->dtype != x->dtype)
        return MOE_ERR_DTYPE;
    if (W_up->ndim != 3 || W_up->shape[2] != d)
        return MOE_ERR_SHAPE;
    const int64_t E = W_up->shape[0], d_ff = W_up->shape[1];
    if (capacity < 0 || (N > 0 && capacity == 0))
        return MOE_ERR_ARG;
    Dims m{N, d, E, d_ff, k, capacity, capacity < N ? capacity : N, x->dtype};
    int rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    if (N == 0)
        return MOE_OK;
    if (!x->data || !W_up->data || !used || !slot_token || !tiles || !H)
        return MOE_ERR_NULL;
    const bool bf16 = x->dtype == MOE_BF16;
    if (bf16 && (!aligned(x->data, 16) || !aligned(W_up->data, 16) || !aligned(H, 16)))
        return MOE_ERR_ALIGN;
    rc = check_expert_ws(workspace);
    if (rc != MOE_OK)
        return rc;
    return hip_status(moe::launch_expert_up(bf16, x->data, W_up->data, d, d_ff, (int)E, k,
                                            m.ceff, used, slot_token, tiles, H,
                                            rows_per_expert(N, k, E, m.ceff), workspace,
                                            workspace ? workspace_bytes : 0, o.act, o.b_up,
                                            static_cast<hipStream_t>(stream)));
}

int moe_expert_up(const moe_tensor *x, const moe_tensor *W_up, int k, int64_t capacity,
                  const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                  void *H, void *workspace, size_t workspace_bytes, void *stream) {
    return expert_up_impl(x, W_up, k, capacity, used, slot_token, tiles, H, workspace,
                          workspace_bytes, stream, ExpertOpts{});
}

int moe_expert_up_ex(const moe_tensor *x, const moe_tensor *W_up, const moe_expert_opts *opts,
                     int k, int64_t capacity, const int32_t *used, const int32_t *slot_token,
                     const int32_t *tiles, void *H, void *workspace, size_t workspace_bytes,
                     void *stream) {
    if (!x || !W_up)
        return MOE_ERR_NULL;
    if (W_up->ndim != 3)
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    const int64_t d = W_up->shape[2];
    const int rc = check_opts(opts, W_up->shape[0], d, W_up->shape[1], o);
    if (rc != MOE_OK)
        return rc;
    return expert_up_impl(x, W_up, k, capacity, used, slot_token, tiles, H, workspace,
                          workspace_bytes, stream, o);
}

static int expert_down_impl(int64_t N, const moe_tensor *W_down, int k, int64_t capacity,
                            const int32_t *used, const int32_t *slot_token,
                            const int32_t *tiles, const void *H, void *Y, void *workspace,
                            size_t workspace_bytes, void *stream, const ExpertOpts &o,
                            int8_t *ysh = nullptr, bool compact = false) {
    if (!W_down)
        return MOE_ERR_NULL;
    if (!valid_dtype(W_down->dtype))
        return MOE_ERR_DTYPE;
    if (W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    const int64_t E = W_down->shape[0], d = W_down->shape[1], d_ff = W_down->shape[2];
    if (N < 0 || capacity < 0 || (N > 0 && capacity == 0))
        return MOE_ERR_ARG;
    Dims m{N, d, E, d_ff, k, capacity, capacity < N ? capacity : N, W_down->dtype};
    int rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    if (N == 0)
        return MOE_OK;
    if (!W_down->data || !used || !slot_token || !tiles || !H || !Y || (compact && !ysh))
        return MOE_ERR_NULL;
    const bool bf16 = W_down->dtype == MOE_BF16;
    if (compact && !bf16)
        return MOE_ERR_DTYPE;
    if (bf16 && (!aligned(W_down->data, 16) || !aligned(H, 16) || !aligned(Y, 16)))
        return MOE_ERR_ALIGN;
    rc = check_expert_ws(workspace);
    if (rc != MOE_OK)
        return rc;
    return hip_status(moe::launch_expert_down(bf16, H, W_down->data, d, d_ff, (int)E, k, m.ceff,
                                              used, slot_token, tiles, Y,
                                              rows_per_expert(N, k, E, m.ceff), workspace,
                                              workspace ? workspace_bytes : 0, o.b_down,
                                              static_cast<hipStream_t>(stream), o.drop,
                                              compact ? reinterpret_cast<signed char *>(ysh)
                                                      : nullptr));
}

int moe_expert_down_compact(int64_t N, const moe_tensor *W_down, const moe_expert_opts *opts,
                            int k, int64_t capacity, const int32_t *used,
                            const int32_t *slot_token, const int32_t *tiles, const void *H,
                            void *Y16, int8_t *Ysh, void *workspace, size_t workspace_bytes,
                            void *stream) {
    if (!W_down)
        return MOE_ERR_NULL;
    if (W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    const int rc = check_opts(opts, W_down->shape[0], W_down->shape[1], W_down->shape[2], o);
    if (rc != MOE_OK)
        return rc;
    return expert_down_impl(N, W_down, k, capacity, used, slot_token, tiles, H, Y16, workspace,
                            workspace_bytes, stream, o, Ysh, true);
}

int moe_expert_down(int64_t N, const moe_tensor *W_down, int k, int64_t capacity,
                    const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                    const void *H, void *Y, void *workspace, size_t workspace_bytes,
                    void *stream) {
    return expert_down_impl(N, W_down, k, capacity, used, slot_token, tiles, H, Y, workspace,
                            workspace_bytes, stream, ExpertOpts{});
}

int moe_expert_down_ex(int64_t N, const moe_tensor *W_down, const moe_expert_opts *opts, int k,
                       int64_t capacity, const int32_t *used, const int32_t *slot_token,
                       const int32_t *tiles, const void *H, void *Y, void *workspace,
                       size_t workspace_bytes, void *stream) {
    if (!W_down)
        return MOE_ERR_NULL;
    if (W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    const int rc = check_opts(opts, W_down->shape[0], W_down->shape[1], W_down->shape[2], o);
    if (rc != MOE_OK)
        return rc;
    return expert_down_impl(N, W_down, k, capacity, used, slot_token, tiles, H, Y, workspace,
                            workspace_bytes, stream, o);
}

int moe_experts_ex(const moe_tensor *x, const moe_tensor *W_up, const moe_tensor *W_down,
                   const moe_expert_opts *opts, int k, int64_t capacity, const int32_t *used,
                   const int32_t *slot_token, const int32_t *tiles, void *H, void *Y,
                   void *workspace, size_t workspace_bytes, void *stream) {
    if (!x || !W_up || !W_down)
        return MOE_ERR_NULL;
    int64_t N, d;
    if (!act_rows(x, N, d))
        return MOE_ERR_SHAPE;
    if (W_up->ndim != 3 || W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    if (W_down->dtype != W_up->dtype)
        return MOE_ERR_DTYPE;
    if (W_down->shape[0] != W_up->shape[0] || W_down->shape[1] != d ||
        W_down->shape[2] != W_up->shape[1])
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    int rc = check_opts(opts, W_up->shape[0], d, W_up->shape[1], o);
    if (rc != MOE_OK)
        return rc;
    // validate both halves before enqueuing either
    rc = expert_up_impl(x, W_up, k, capacity, used, slot_token, tiles, nullptr, nullptr, 0,
                        nullptr, o);
    if (rc != MOE_OK && rc != MOE_ERR_NULL)
        return rc;
    if (N > 0 && (!H || !Y))
        return MOE_ERR_NULL;
    rc = check_expert_ws(workspace);
    if (rc != MOE_OK)
        return rc;
    rc = expert_up_impl(x, W_up, k, capacity, used, slot_token, tiles, H, workspace,
                        workspace_bytes, stream, o);
    if (rc != MOE_OK)
        return rc;
    return expert_down_impl(N, W_down, k, capacity, used, slot_token, tiles, H, Y, workspace,
                            workspace_bytes, stream, o);
}

int moe_experts(const moe_tensor *x, const moe_tensor *W_up, const moe_tensor *W_down, int k,
                int64_t capacity, const int32_t *used, const int32_t *slot_token,
                const int32_t *tiles, void *H, void *Y, void *workspace,
                size_t workspace_bytes, void *stream) {
    return moe_experts_ex(x, W_up, W_down, nullptr, k, capacity, used, slot_token, tiles, H, Y,
                          workspace, workspace_bytes, stream);
}

int moe_combine(int64_t N, int64_t d, int k, const moe_tensor *Y, const float *topk_gate,
                const int32_t *slot, moe_tensor *out, void *stream) {
    if (!out || !Y)
        return MOE_ERR_NULL;
    if (N < 0 || d <= 0 || k < 1 || k > MOE_MAX_TOPK)
        return MOE_ERR_ARG;
    int64_t oN, od;
    if (!act_rows(out, oN, od) || oN != N || od != d)
        return MOE_ERR_SHAPE;
    if (Y->ndim != 2 || Y->shape[0] != N * k || Y->shape[1] != d)
        return MOE_ERR_SHAPE;
    if (!valid_dtype(out->dtype) || !valid_dtype(Y->dtype))
        return MOE_ERR_DTYPE;
    if (N == 0)
        return MOE_OK;
    if (!Y->data || !topk_gate || !slot || !out->data)
        return MOE_ERR_NULL;
    const bool vec = Y->dtype == MOE_BF16 ? d % 8 == 0 : d % 4 == 0;
    if (vec && (!aligned(Y->data, 16) || !aligned(out->data, out->dtype == MOE_BF16 ? 8 : 16)))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_combine(Y->data, Y->dtype == MOE_BF16 ? 1 : 0, topk_gate, slot,
                                          N, d, k, out->data, out->dtype,
                                          static_cast<hipStream_t>(stream)));
}

int moe_combine_compact(int64_t N, int64_t d, int k, const void *Y16, const int8_t *Ysh,
                        const float *topk_gate, const int32_t *slot, moe_tensor *out,
                        void *stream) {
    if (!out)
        return MOE_ERR_NULL;
    if (N < 0 || d <= 0 || k < 1 || k > MOE_MAX_TOPK)
        return MOE_ERR_ARG;
    int64_t oN, od;
    if (!act_rows(out, oN, od) || oN != N || od != d)
        return MOE_ERR_SHAPE;
    if (!valid_dtype(out->dtype))
        return MOE_ERR_DTYPE;
    if (d % 8 != 0)
        return MOE_ERR_UNSUPPORTED;
    if (N == 0)
        return MOE_OK;
    if (!Y16 || !Ysh || !topk_gate || !slot || !out->data)
        return MOE_ERR_NULL;
    if (!aligned(Y16, 16) || !aligned(out->data, 16))
        return MOE_ERR_ALIGN;
    return hip_status(moe::launch_combine_compact(Y16, reinterpret_cast<const signed char *>(Ysh),
                                                  topk_gate, slot, N, d, k, out->data,
                                                  out->dtype, static_cast<hipStream_t>(stream)));
}

int moe_forward_ex(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                   const moe_tensor *W_up, const moe_tensor *W_down,
                   const moe_expert_opts *opts, int k, float capacity_factor, moe_tensor *out,
                   moe_stats *stats) {
    if (!stats || !W_up || !W_down || !out)
        return MOE_ERR_NULL;
    int64_t N, d, E;
    int rc = check_router_args(x, W_g, noise, k, N, d, E);
    if (rc != MOE_OK)
        return rc;
    if (!cf_ok(capacity_factor))
        return MOE_ERR_ARG;
    if (W_up->dtype != x->dtype || W_down->dtype != x->dtype || out->dtype != x->dtype)
        return MOE_ERR_DTYPE;
    if (W_up->ndim != 3 || W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    const int64_t d_ff = W_up->shape[1];
    if (W_up->shape[0] != E || W_up->shape[2] != d || W_down->shape[0] != E ||
        W_down->shape[1] != d || W_down->shape[2] != d_ff)
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    rc = check_opts(opts, E, d, d_ff, o);
    if (rc != MOE_OK)
        return rc;
    int64_t oN, od;
    if (!act_rows(out, oN, od) || oN != N || od != d)
        return MOE_ERR_SHAPE;
    Dims m{N, d, E, d_ff, k, 0, 0, x->dtype};
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stats->stream);
    if (N == 0) {
        stats->capacity = 0;
        if (stats->used_capacity)
            MOE_TRY(moe::launch_fill_i32(stats->used_capacity, E, 0, s));
        return zero_router_stats(E, stats->expert_demand, stats->expert_drops,
                                 stats->expert_gate_sum, s);
    }
    if (!W_up->data || !W_down->data || !out->data)
        return MOE_ERR_NULL;
    if (!stats->workspace)
        return MOE_ERR_NULL;
    if (!aligned(stats->workspace, kAlign))
        return MOE_ERR_ALIGN;
    if (x->dtype == MOE_BF16 &&
        (!aligned(W_up->data, 16) || !aligned(W_down->data, 16) || !aligned(out->data, 16)))
        return MOE_ERR_ALIGN;
    if (x->dtype == MOE_F32 && !aligned(out->data, 16) && d % 4 == 0)
        return MOE_ERR_ALIGN;
    const Layout L = layout_of(m);
    if (stats->workspace_bytes < L.total)
        return MOE_ERR_WORKSPACE;

    char *ws = static_cast<char *>(stats->workspace);
    int32_t *idx = stats->topk_idx ? stats->topk_idx : reinterpret_cast<int32_t *>(ws + L.idx);
    float *gate = stats->topk_gate ? stats->topk_gate : reinterpret_cast<float *>(ws + L.gate);
    int32_t *slot = stats->slot ? stats->slot : reinterpret_cast<int32_t *>(ws + L.slot);
    int32_t *used = stats->used_capacity ? stats->used_capacity
                                         : reinterpret_cast<int32_t *>(ws + L.used);
    int32_t *tiles = reinterpret_cast<int32_t *>(ws + L.tiles);
    int32_t *slot_token = reinterpret_cast<int32_t *>(ws + L.slot_token);
    void *H = ws + L.H;
    void *Y = ws + L.Y;   // expert outputs: compact (bf16 layers) or fp32
    signed char *ysh = x->dtype == MOE_BF16 ? reinterpret_cast<signed char *>(ws + L.Ysh) : nullptr;
    stats->capacity = m.C;

    rc = router_checked(x, W_g, noise, N, d, E, k, idx, gate, ws + L.router, s);
    if (rc != MOE_OK)
        return rc;
    MOE_TRY(moe::launch_dispatch(idx, gate, N, (int)E, k, m.ceff, slot, used, slot_token, tiles,
                                 stats->expert_demand, stats->expert_drops,
                                 stats->expert_gate_sum, ws + L.dispatch, s));
    const bool bf16 = x->dtype == MOE_BF16;
    const int64_t rpe = rows_per_expert(N, k, E, m.ceff);
    void *part = ws + L.part;
    const size_t part_bytes = L.total - L.part;
    MOE_TRY(moe::launch_expert_up(bf16, x->data, W_up->data, d, d_ff, (int)E, k, m.ceff, used,
                                  slot_token, tiles, H, rpe, part, part_bytes, o.act, o.b_up, s));
    MOE_TRY(moe::launch_expert_down(bf16, H, W_down->data, d, d_ff, (int)E, k, m.ceff, used,
                                    slot_token, tiles, Y, rpe, part, part_bytes, o.b_down, s,
                                    o.drop, ysh));
    if (ysh)
        MOE_TRY(moe::launch_combine_compact(Y, ysh, gate, slot, N, d, k, out->data, out->dtype,
                                            s));
    else
        MOE_TRY(moe::launch_combine(Y, 0, gate, slot, N, d, k, out->data, out->dtype, s));
    return MOE_OK;
}

int moe_forward(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                const moe_tensor *W_up, const moe_tensor *W_down, int k, float capacity_factor,
                moe_tensor *out, moe_stats *stats) {
    return moe_forward_ex(x, W_g, noise, W_up, W_down, nullptr, k, capacity_factor, out, stats);
}

size_t moe_backward_workspace_size(int64_t N, int64_t d, int64_t E, int64_t d_ff, int k,
                                   float capacity_factor, int32_t dtype) {
    if (dtype != MOE_BF16 || !cf_ok(capacity_factor))
        return 0;
    if (N < 0 || E <= 0 || k < 1 || k > E)
        return 0;
    Dims m{N, d, E, d_ff, k, 0, 0, dtype};
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    if (check_sizes(m) != MOE_OK)
        return 0;
    return bwd_layout_of(m).total;
}

// The backward; with `saved`, the forward state is the one a
// moe_forward_train call left in the workspace (and in the exported routing
// arrays) instead of being recomputed.
// Fork of the backward's second branch onto the caller's aux stream: the
// router-weight gradient and the down-projection weight gradient need only
// the combine backward's outputs, so on a second stream their products fill
// the CUs the main chain's products leave idle in their last rounds. Two
// events created for the call fork the aux stream from the caller's stream
// and join it back; they are destroyed when the call returns (HIP releases an
// event whose record is still pending once it completes, and a wait already
// enqueued on it is unaffected), so nothing outlives the call. Under stream
// capture the record/wait pairs become the graph's fork and join edges.
// Without an aux stream the branch runs on the caller's stream.
struct Fork {
    hipStream_t s, s2;
    hipEvent_t ev[2] = {nullptr, nullptr};
    bool open = false;
    explicit Fork(hipStream_t main) : s(main), s2(main) {}
    int begin(void *aux) {
        if (!aux || static_cast<hipStream_t>(aux) == s)
            return MOE_OK;
        if (hipEventCreateWithFlags(&ev[0], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&ev[1], hipEventDisableTiming) != hipSuccess ||
            hipEventRecord(ev[0], s) != hipSuccess ||
            hipStreamWaitEvent(static_cast<hipStream_t>(aux), ev[0], 0) != hipSuccess)
            return MOE_ERR_HIP;
        s2 = static_cast<hipStream_t>(aux);
        open = true;
        return MOE_OK;
    }
    // join the aux stream back into the caller's stream (idempotent)
    int join() {
        if (!open)
            return MOE_OK;
        open = false;
        if (hipEventRecord(ev[1], s2) != hipSuccess || hipStreamWaitEvent(s, ev[1], 0) != hipSuccess)
            return MOE_ERR_HIP;
        return MOE_OK;
    }
    ~Fork() {
        (void)join();
        for (hipEvent_t e : ev)
            if (e)
                (void)hipEventDestroy(e);
    }
};

static int backward_call(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                         const moe_tensor *W_up, const moe_tensor *W_down,
                         const moe_expert_opts *opts, int k, float capacity_factor,
                         const moe_tensor *dout, moe_tensor *dx, moe_tensor *dW_g,
                         moe_tensor *dW_up, moe_tensor *dW_down, moe_tensor *db_up,
                         moe_tensor *db_down, moe_stats *stats, bool saved) {
    if (!stats || !W_up || !W_down || !dout)
        return MOE_ERR_NULL;
    int64_t N, d, E;
    int rc = check_router_args(x, W_g, noise, k, N, d, E);
    if (rc != MOE_OK)
        return rc;
    if (!cf_ok(capacity_factor))
        return MOE_ERR_ARG;
    if (x->dtype != MOE_BF16)
        return MOE_ERR_UNSUPPORTED;   // the backward runs on bf16 layers
    if (W_up->dtype != x->dtype || W_down->dtype != x->dtype || dout->dtype != x->dtype)
        return MOE_ERR_DTYPE;
    if (W_up->ndim != 3 || W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    const int64_t d_ff = W_up->shape[1];
    if (W_up->shape[0] != E || W_up->shape[2] != d || W_down->shape[0] != E ||
        W_down->shape[1] != d || W_down->shape[2] != d_ff)
        return MOE_ERR_SHAPE;
    int64_t gN, gd;
    if (!act_rows(dout, gN, gd) || gN != N || gd != d)
        return MOE_ERR_SHAPE;
    {
        const int64_t e_dx[2] = {N, d}, e_wg[2] = {E, d}, e_up[3] = {E, d_ff, d},
                      e_dn[3] = {E, d, d_ff};
        if (!dx || !dW_g || !dW_up || !dW_down)
            return MOE_ERR_NULL;
        int64_t xN, xd;
        if (dx->dtype != MOE_F32)
            return MOE_ERR_DTYPE;
        if (!act_rows(dx, xN, xd) || xN != e_dx[0] || xd != e_dx[1])
            return MOE_ERR_SHAPE;
        if ((rc = check_grad(dW_g, 2, e_wg)) != MOE_OK ||
            (rc = check_grad(dW_up, 3, e_up)) != MOE_OK ||
            (rc = check_grad(dW_down, 3, e_dn)) != MOE_OK)
            return rc;
    }
    ExpertOpts o;
    rc = check_opts(opts, E, d, d_ff, o);
    if (rc != MOE_OK)
        return rc;
    // a bias gradient exactly when the layer has that bias
    if ((o.b_up && !db_up) || (o.b_down && !db_down))
        return MOE_ERR_NULL;
    if ((!o.b_up && db_up) || (!o.b_down && db_down))
        return MOE_ERR_ARG;
    {
        const int64_t e_bu[2] = {E, d_ff}, e_bd[2] = {E, d};
        if (db_up && (rc = check_grad(db_up, 2, e_bu)) != MOE_OK)
            return rc;
        if (db_down && (rc = check_grad(db_down, 2, e_bd)) != MOE_OK)
            return rc;
        if ((db_up && !db_up->data) || (db_down && !db_down->data))
            return MOE_ERR_NULL;
        if ((db_up && !aligned(db_up->data, 16)) || (db_down && !aligned(db_down->data, 16)))
            return MOE_ERR_ALIGN;
    }
    Dims m{N, d, E, d_ff, k, 0, 0, x->dtype};
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    // the weight gradients are written even without tokens
    if (!dW_g->data || !dW_up->data || !dW_down->data)
        return MOE_ERR_NULL;
    if (!aligned(dW_g->data, 16) || !aligned(dW_up->data, 16) || !aligned(dW_down->data, 16))
        return MOE_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stats->stream);
    if (N == 0) {
        // no tokens: every gradient is zero
        // (fill kernels, not memset nodes: the call may be captured in a graph)
        stats->capacity = 0;
        MOE_TRY(moe::launch_fill_i32(static_cast<int32_t *>(dW_g->data), E * d, 0, s));
        MOE_TRY(moe::launch_fill_i32(static_cast<int32_t *>(dW_up->data), E * d_ff * d, 0, s));
        MOE_TRY(moe::launch_fill_i32(static_cast<int32_t *>(dW_down->data), E * d * d_ff, 0, s));
        if (db_up)
            MOE_TRY(moe::launch_fill_i32(static_cast<int32_t *>(db_up->data), E * d_ff, 0, s));
        if (db_down)
            MOE_TRY(moe::launch_fill_i32(static_cast<int32_t *>(db_down->data), E * d, 0, s));
        if (stats->used_capacity)
            MOE_TRY(moe::launch_fill_i32(stats->used_capacity, E, 0, s));
        return zero_router_stats(E, stats->expert_demand, stats->expert_drops,
                                 stats->expert_gate_sum, s);
    }
    if (!W_up->data || !W_down->data || !dout->data || !dx->data)
        return MOE_ERR_NULL;
    if (!stats->workspace)
        return MOE_ERR_NULL;
    if (!aligned(stats->workspace, kAlign))
        return MOE_ERR_ALIGN;
    if (!aligned(W_up->data, 16) || !aligned(W_down->data, 16) || !aligned(dout->data, 16) ||
        !aligned(dx->data, 16))
        return MOE_ERR_ALIGN;
    const BwdLayout L = bwd_layout_of(m);
    if (stats->workspace_bytes < L.total)
        return MOE_ERR_WORKSPACE;
    stats->capacity = m.C;

    char *ws = static_cast<char *>(stats->workspace);
    int32_t *idx = stats->topk_idx ? stats->topk_idx : reinterpret_cast<int32_t *>(ws + L.idx);
    float *gate = stats->topk_gate ? stats->topk_gate : reinterpret_cast<float *>(ws + L.gate);
    int32_t *slot = stats->slot ? stats->slot : reinterpret_cast<int32_t *>(ws + L.slot);
    int32_t *used = stats->used_capacity ? stats->used_capacity
                                         : reinterpret_cast<int32_t *>(ws + L.used);
    int32_t *tiles = reinterpret_cast<int32_t *>(ws + L.tiles);
    int32_t *st = reinterpret_cast<int32_t *>(ws + L.slot_token);
    void *H = ws + L.H, *Y = ws + L.Y, *dY = ws + L.dY, *dZ = ws + L.dZ;
    void *T1 = ws + L.T1, *T2 = ws + L.T2, *dsT3 = ws + L.dsT3, *xT3 = ws + L.xT3;
    float *ds = reinterpret_cast<float *>(ws + L.ds);
    float *dXa = reinterpret_cast<float *>(ws + L.dXa);
    float *gpart = reinterpret_cast<float *>(ws + L.gpart);
    const int64_t ceff = m.ceff, Kp = L.Kp, Tc = L.Tc, S = L.S;
    const int64_t rpe = rows_per_expert(N, k, E, ceff);
    const int Ei = (int)E;

    // forward state: routing, plan, H and the experts' output rows
    const bool gelu = o.act == moe::kActGelu;
    if (!saved) {
        rc = forward_state(L, ws, x, W_g, noise, W_up, W_down, o, m, stats, s);
        if (rc != MOE_OK)
            return rc;
    }
    // combine and softmax backward; router weights: dW_g = ds^T x, per token
    // chunk on the exact split of ds, then the chunks summed in order
    MOE_TRY(moe::launch_combine_backward(dout->data, Y,
                                         reinterpret_cast<const signed char *>(ws + L.Ysh), gate,
                                         slot, N, d, k, dY, ds, s, o.drop));
    // fork: the aux stream s2 takes the router-weight gradient and (when the
    // products read K-major) the down-projection weight gradient; both read
    // only the forward state, ds and dY, and write buffers of their own. The
    // fork is joined back when `fork` goes out of scope on every return path.
    Fork fork(s);
    rc = fork.begin(stats->aux_stream);
    if (rc != MOE_OK)
        return rc;
    const hipStream_t s2 = fork.s2;
    MOE_TRY(moe::launch_ds_split(ds, idx, N, Tc, S, Ei, k, dsT3, s2));
    MOE_TRY(moe::launch_transpose_rows(x->data, d, Tc, nullptr, N, nullptr, k, 0, Tc, 3, (int)S,
                                       xT3, s2));
    MOE_TRY(moe::launch_batched_gemm_bf16(dsT3, xT3, E, 3 * Tc, d, (int)S, E * 3 * Tc,
                                          d * 3 * Tc, E * d, gpart, s2));
    MOE_TRY(moe::launch_chunk_sum(gpart, S, E * d, static_cast<float *>(dW_g->data), s2));
    const bool kmajor = ceff <= moe::kGradMaxRows;
    if (kmajor) {
        MOE_TRY(moe::launch_weight_grad(dY, d, H, d_ff, Ei, ceff, used, st, 1, 0,
                                        static_cast<float *>(dW_down->data), s2));
        if (db_down)
            MOE_TRY(moe::launch_colsum_rows(dY, d, Ei, ceff, used, st, 1,
                                            static_cast<float *>(db_down->data), s2));
    }
    // experts, input side: dZ = (dY W_down) [H > 0]; dX = dZ W_up; dx
    // (the weights are read K-major by the products themselves)
    MOE_TRY(moe::launch_expert_dz(dY, W_down->data, gelu ? dZ : H, o.act, d, d_ff, Ei, k, ceff,
                                  used, st, tiles, dZ, rpe, s));
    MOE_TRY(moe::launch_expert_rows_f32(dZ, W_up->data, d_ff, d, Ei, k, ceff, used, st, tiles,
                                        dXa, rpe, s));
    MOE_TRY(moe::launch_dx(dXa, ds, idx, slot, static_cast<const float *>(W_g->data), N, d, Ei,
                           k, static_cast<float *>(dx->data), s));
    // experts, weight side: dW_down = dY^T H (on the side stream, above),
    // dW_up = dZ^T X over each expert's kept rows, read K-major by the
    // products themselves
    if (kmajor) {
        MOE_TRY(moe::launch_weight_grad(dZ, d_ff, x->data, d, Ei, ceff, used, st, k, 1,
                                        static_cast<float *>(dW_up->data), s));
        if (db_up)
            MOE_TRY(moe::launch_colsum_rows(dZ, d_ff, Ei, ceff, used, nullptr, 1,
                                            static_cast<float *>(db_up->data), s));
        return fork.join();
    }
    // (longer experts: through transposes, K = kept rows padded to Kp;
    // bias gradients: the row sums of the transposed dY and dZ)
    MOE_TRY(moe::launch_transpose_rows(dY, d, ceff, used, 0, st, k, 1, Kp, 1, Ei, T1, s));
    if (db_down)
        MOE_TRY(moe::launch_row_sums(T1, E * d, Kp, static_cast<float *>(db_down->data), s));
    MOE_TRY(moe::launch_transpose_rows(H, d_ff, ceff, used, 0, st, k, 0, Kp, 1, Ei, T2, s));
    MOE_TRY(moe::launch_batched_gemm_bf16(T1, T2, d, Kp, d_ff, Ei, d * Kp, d_ff * Kp, d * d_ff,
                                          static_cast<float *>(dW_down->data), s));
    MOE_TRY(moe::launch_transpose_rows(x->data, d, ceff, used, 0, st, k, 2, Kp, 1, Ei, T1, s));
    MOE_TRY(moe::launch_transpose_rows(dZ, d_ff, ceff, used, 0, st, k, 0, Kp, 1, Ei, T2, s));
    if (db_up)
        MOE_TRY(moe::launch_row_sums(T2, E * d_ff, Kp, static_cast<float *>(db_up->data), s));
    MOE_TRY(moe::launch_batched_gemm_bf16(T2, T1, d_ff, Kp, d, Ei, d_ff * Kp, d * Kp, d_ff * d,
                                          static_cast<float *>(dW_up->data), s));
    return fork.join();
}

int moe_backward_ex(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                    const moe_tensor *W_up, const moe_tensor *W_down,
                    const moe_expert_opts *opts, int k, float capacity_factor,
                    const moe_tensor *dout, moe_tensor *dx, moe_tensor *dW_g, moe_tensor *dW_up,
                    moe_tensor *dW_down, moe_tensor *db_up, moe_tensor *db_down,
                    moe_stats *stats) {
    return backward_call(x, W_g, noise, W_up, W_down, opts, k, capacity_factor, dout, dx, dW_g,
                         dW_up, dW_down, db_up, db_down, stats, false);
}

int moe_backward_after_forward(const moe_tensor *x, const moe_tensor *W_g,
                               const moe_tensor *noise, const moe_tensor *W_up,
                               const moe_tensor *W_down, const moe_expert_opts *opts, int k,
                               float capacity_factor, const moe_tensor *dout, moe_tensor *dx,
                               moe_tensor *dW_g, moe_tensor *dW_up, moe_tensor *dW_down,
                               moe_tensor *db_up, moe_tensor *db_down, moe_stats *stats) {
    return backward_call(x, W_g, noise, W_up, W_down, opts, k, capacity_factor, dout, dx, dW_g,
                         dW_up, dW_down, db_up, db_down, stats, true);
}

int moe_forward_train(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                      const moe_tensor *W_up, const moe_tensor *W_down,
                      const moe_expert_opts *opts, int k, float capacity_factor, moe_tensor *out,
                      moe_stats *stats) {
    if (!stats || !W_up || !W_down || !out)
        return MOE_ERR_NULL;
    int64_t N, d, E;
    int rc = check_router_args(x, W_g, noise, k, N, d, E);
    if (rc != MOE_OK)
        return rc;
    if (!cf_ok(capacity_factor))
        return MOE_ERR_ARG;
    if (x->dtype != MOE_BF16)
        return MOE_ERR_UNSUPPORTED;   // training runs on bf16 layers
    if (W_up->dtype != x->dtype || W_down->dtype != x->dtype || out->dtype != x->dtype)
        return MOE_ERR_DTYPE;
    if (W_up->ndim != 3 || W_down->ndim != 3)
        return MOE_ERR_SHAPE;
    const int64_t d_ff = W_up->shape[1];
    if (W_up->shape[0] != E || W_up->shape[2] != d || W_down->shape[0] != E ||
        W_down->shape[1] != d || W_down->shape[2] != d_ff)
        return MOE_ERR_SHAPE;
    ExpertOpts o;
    rc = check_opts(opts, E, d, d_ff, o);
    if (rc != MOE_OK)
        return rc;
    int64_t oN, od;
    if (!act_rows(out, oN, od) || oN != N || od != d)
        return MOE_ERR_SHAPE;
    Dims m{N, d, E, d_ff, k, 0, 0, x->dtype};
    m.C = capacity_of(N, E, k, capacity_factor);
    m.ceff = m.C < N ? m.C : N;
    rc = check_sizes(m);
    if (rc != MOE_OK)
        return rc;
    hipStream_t s = static_cast<hipStream_t>(stats->stream);
    if (N == 0) {
        stats->capacity = 0;
        if (stats->used_capacity)
            MOE_TRY(moe::launch_fill_i32(stats->used_capacity, E, 0, s));
        return zero_router_stats(E, stats->expert_demand, stats->expert_drops,
                                 stats->expert_gate_sum, s);
    }
    if (!W_up->data || !W_down->data || !out->data)
        return MOE_ERR_NULL;
    if (!stats->workspace)
        return MOE_ERR_NULL;
    if (!aligned(stats->workspace, kAlign))
        return MOE_ERR_ALIGN;
    if (!aligned(W_up->data, 16) || !aligned(W_down->data, 16) || !aligned(out->data, 16))
        return MOE_ERR_ALIGN;
    const BwdLayout L = bwd_layout_of(m);
    if (stats->workspace_bytes < L.total)
        return MOE_ERR_WORKSPACE;
    stats->capacity = m.C;
    char *ws = static_cast<char *>(stats->workspace);
    rc = forward_state(L, ws, x, W_g, noise, W_up, W_down, o, m, stats, s);
    if (rc != MOE_OK)
        return rc;
    const float *gate = stats->topk_gate ? stats->topk_gate
                                         : reinterpret_cast<const float *>(ws + L.gate);
    const int32_t *slot = stats->slot ? stats->slot : reinterpret_cast<const int32_t *>(ws + L.slot);
    return hip_status(moe::launch_combine_compact(
        ws + L.Y, reinterpret_cast<const signed char *>(ws + L.Ysh), gate, slot, N, d, k,
        out->data, out->dtype, s));
}

int moe_backward(const moe_tensor *x, const moe_tensor *W_g, const moe_tensor *noise,
                 const moe_tensor *W_up, const moe_tensor *W_down, int k, float capacity_factor,
                 const moe_tensor *dout, moe_tensor *dx, moe_tensor *dW_g, moe_tensor *dW_up,
                 moe_tensor *dW_down, moe_stats *stats) {
    return moe_backward_ex(x, W_g, noise, W_up, W_down, nullptr, k, capacity_factor, dout, dx,
                           dW_g, dW_up, dW_down, nullptr, nullptr, stats);
}

}  // extern "C"

static int forward_state(const BwdLayout &L, char *ws, const moe_tensor *x,
                         const moe_tensor *W_g, const moe_tensor *noise, const moe_tensor *W_up,
                         const moe_tensor *W_down, const ExpertOpts &o, const Dims &m,
                         moe_stats *stats, hipStream_t s) {
    int32_t *idx = stats->topk_idx ? stats->topk_idx : reinterpret_cast<int32_t *>(ws + L.idx);
    float *gate = stats->topk_gate ? stats->topk_gate : reinterpret_cast<float *>(ws + L.gate);
    int32_t *slot = stats->slot ? stats->slot : reinterpret_cast<int32_t *>(ws + L.slot);
    int32_t *used = stats->used_capacity ? stats->used_capacity
                                         : reinterpret_cast<int32_t *>(ws + L.used);
    int32_t *tiles = reinterpret_cast<int32_t *>(ws + L.tiles);
    int32_t *st = reinterpret_cast<int32_t *>(ws + L.slot_token);
    const int Ei = (int)m.E;
    const int64_t rpe = rows_per_expert(m.N, m.k, m.E, m.ceff);
    int rc = router_checked(x, W_g, noise, m.N, m.d, m.E, m.k, idx, gate, ws + L.router, s);
    if (rc != MOE_OK)
        return rc;
    MOE_TRY(moe::launch_dispatch(idx, gate, m.N, Ei, m.k, m.ceff, slot, used, st, tiles,
                                 stats->expert_demand, stats->expert_drops,
                                 stats->expert_gate_sum, ws + L.dispatch, s));
    const bool gelu = o.act == moe::kActGelu;
    // (the same launch configuration as moe_forward_ex, split included, so
    // the state and out are bit for bit the forward's)
    void *part = ws + L.part;
    const size_t part_bytes = L.total - L.part;
    MOE_TRY(moe::launch_expert_up(true, x->data, W_up->data, m.d, m.d_ff, Ei, m.k, m.ceff, used,
                                  st, tiles, ws + L.H, rpe, part, part_bytes, o.act, o.b_up, s,
                                  gelu ? ws + L.dZ : nullptr));
    MOE_TRY(moe::launch_expert_down(true, ws + L.H, W_down->data, m.d, m.d_ff, Ei, m.k, m.ceff,
                                    used, st, tiles, ws + L.Y, rpe, part, part_bytes, o.b_down, s,
                                    o.drop, reinterpret_cast<signed char *>(ws + L.Ysh)));
    return MOE_OK;
}
