// Private helpers shared by the gfx950 kernels of the MoE layer (not part of
// the C ABI). Wave size is 64 on CDNA; every kernel here assumes it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kMaxQ = kMaxExperts / kWave;   // router scores per lane
constexpr int kFusedMaxExperts = 32;          // larger routers use the GEMM path
constexpr int kActRelu = 0, kActGelu = 1;     // expert activations (values of the C ABI)
constexpr int kGradMaxRows = 3072;            // rows per expert of the K-major weight gradients

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// float -> bf16 bits, round to nearest even (NaN stays a quiet NaN), on
// gfx950's conversion instruction (v_cvt_pk_bf16_f32); a pair converts in
// one instruction, lo in the low half. (Checked bit for bit against the
// integer round-to-nearest-even formulation on 2^24 values: ties,
// denormals, infinities and NaNs included.)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
__device__ __forceinline__ unsigned short f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(unsigned short, (__bf16)f);
}

__device__ __forceinline__ float bf16_bits_to_f32(unsigned short b) {
    return __builtin_bit_cast(float, (unsigned int)b << 16);
}

// Compact expert output rows (the fused entry points of bf16 layers): each
// group of kYGroup columns of a row of Y is stored as the fp16 values of
// y * 2^sh with one exponent shift sh (int8) per group, sh chosen from the
// group's largest finite magnitude m so that m * 2^sh lies in [2^14, 2^15).
// Scaling by a power of two is exact, so every value keeps fp16's 11
// significant bits (relative error at most 2^-11, round to nearest even),
// none can overflow, and values below m * 2^-28 (fp16 subnormals) lose at
// most m * 2^-39. Infinities and NaNs pass through. y' = fp16 * 2^-sh.
constexpr int kYGroup = 32;
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
// 2^s as an fp32 bit pattern, s in [-126, 127]
__device__ __forceinline__ float pow2f(int s) {
    return __uint_as_float((unsigned)(127 + s) << 23);
}
// Shift of a group whose largest finite magnitude is m (>= 0): 141 - the
// biased exponent of m, at most 126 (m = 0 or below 2^-112), so that both
// 2^sh and 2^-sh are normal fp32 values.
__device__ __forceinline__ int yshift_of(float m) {
    const int sh = 141 - (int)((__float_as_uint(m) >> 23) & 0xffu);
    return sh > 126 ? 126 : sh;
}
// Shifts are stored per token, then per group, then per choice: the shift of
// assignment a = t*k + j's group g is at (t*G + g)*k + j (G groups per row),
// so a token's k shifts of one group are adjacent. Assignment indices fit in
// 31 bits (N*k < 2^31), so the token comes from a 32-bit division.
__device__ __forceinline__ int64_t yshift_index(int a, int k, int G, int g) {
    const unsigned t = (unsigned)a / (unsigned)k;
    return ((int64_t)t * G + g) * k + (a - (int)t * k);
}
// The same for a known token t and choice j.
__device__ __forceinline__ int64_t yshift_index(int64_t t, int j, int k, int G, int g) {
    return (t * G + g) * k + j;
}
// acc raised to |v| when v is finite (NaN and infinities are ignored).
__device__ __forceinline__ float finite_max(float acc, float v) {
    const float a = fabsf(v);
    return a < __builtin_inff() ? fmaxf(acc, a) : acc;
}
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2_t{lo, hi}, f16x2_t));
}
__device__ __forceinline__ f32x2_t unpack_f16x2(unsigned w) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2_t, w), f32x2_t);
}

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011): ten rounds on a 4 x 64-bit counter; a round
// takes the 128-bit products of counter words 0 and 2 with the two round
// multipliers and forms (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key
// words grow by their Weyl constants between rounds.
__device__ __forceinline__ void philox4x64_10(uint64_t c0, uint64_t c1, uint64_t c2,
                                              uint64_t c3, uint64_t k0, uint64_t k1,
                                              uint64_t (&out)[4]) {
    constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
    constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
    // The rounds stay a loop: unrolled, the generator is large enough to stop
    // the unrolling of the epilogue loops that call it, whose accumulators
    // would then be indexed at run time and leave the registers.
#pragma unroll 1
    for (int r = 0; r < 10; ++r) {
        const uint64_t hi0 = __umul64hi(M0, c0), lo0 = M0 * c0;
        const uint64_t hi1 = __umul64hi(M1, c2), lo1 = M1 * c2;
        c0 = hi1 ^ c1 ^ k0;
        c1 = lo1;
        c2 = hi0 ^ c3 ^ k1;
        c3 = lo0;
        k0 += W0;
        k1 += W1;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

// Training-mode dropout on the expert output rows (nanoMoE slides, slide 32:
// the expert ends in a dropout). Element i of the row of assignment a is
// kept when its 32-bit word is >= thresh = floor(p 2^32) and then scaled by
// `scale` = 1 / (1 - p); dropped elements become 0. The words of elements
// 8q .. 8q+7 are the Philox4x64-10 block at counter (q, a, offset, 0) under
// key (seed, 0): element i takes half i % 2 (low half first) of output word
// (i % 8) / 2.
struct Dropout {
    int on = 0;              // 0: no dropout
    uint32_t thresh = 0;
    float scale = 1.f;
    uint64_t seed = 0, offset = 0;
};

// Dropout factors (scale or 0) of the 8 elements 8q .. 8q+7 of row a.
__device__ __forceinline__ void dropout_factors8(const Dropout &dp, int64_t a, int64_t q,
                                                 float (&m)[8]) {
    uint64_t r[4];
    philox4x64_10((uint64_t)q, (uint64_t)a, dp.offset, 0ull, dp.seed, 0ull, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t w = (uint32_t)(i % 2 ? r[i / 2] >> 32 : r[i / 2]);
        m[i] = w >= dp.thresh ? dp.scale : 0.f;
    }
}

// 64-bit lane masks
__device__ __forceinline__ uint64_t lanemask_lt() {
    const unsigned lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe

// ---------------------------------------------------------------------------
// Launchers (one per stage). All return hipSuccess or the launch error.
// ---------------------------------------------------------------------------
namespace moe {

// ws: router_workspace_bytes(N, d, E) bytes of device scratch (256-aligned).
size_t router_workspace_bytes(int64_t N, int64_t d, int E);
hipError_t launch_router_bf16(const void *x, const float *wg, const float *noise,
                              int64_t N, int64_t d, int E, int k,
                              int32_t *idx, float *gate, void *ws, hipStream_t s);
hipError_t launch_router_f32(const float *x, const float *wg, const float *noise,
                             int64_t N, int64_t d, int E, int k,
                             int32_t *idx, float *gate, hipStream_t s);

// Dispatch plan; demand / drops / gate_sum (router statistics) may each be
// NULL; gate is read only for gate_sum. ws: dispatch_workspace_bytes()
// bytes of device scratch (256-aligned; none for a single 4096-assignment chunk).
size_t dispatch_workspace_bytes(int64_t N, int E, int k);
hipError_t launch_dispatch(const int32_t *idx, const float *gate, int64_t N, int E, int k,
                           int64_t ceff, int32_t *slot, int32_t *used, int32_t *slot_token,
                           int32_t *tiles, int32_t *demand, int32_t *drops, float *gate_sum,
                           void *ws, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s);

// Grouped expert products. mode 0: H = act(x[gather] W_up^T + b_up); mode 1:
// Y[scatter] = H W_down^T + b_down. H has the operands' dtype (bf16 or fp32),
// Y is fp32.
// bf16 != 0: bf16 operands on matrix cores; otherwise fp32 operands.
// rows_per_expert: the expected kept rows per expert (picks the tile shape).
// part/part_bytes: device scratch for the K-split of a product's last round
// of tiles (NULL, or smaller than one partial tile per resident workgroup:
// no split). split_workspace_bytes() is enough for every tile shape on a
// device with up to 256 CUs.
constexpr size_t kSplitWorkspaceBytes = (size_t)256 * 256 * 256 * sizeof(float);
size_t split_workspace_bytes();
// act: kActRelu or kActGelu (up product); b_up [E, d_ff] / b_down [E, d]
// fp32 biases or NULL. Z (bf16 layers): when not NULL, the pre-activations
// z = W_up x + b_up are stored there too, [E, ceff, d_ff] like H.
hipError_t launch_expert_up(bool bf16, const void *x, const void *w_up, int64_t d,
                            int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                            const int32_t *slot_token, const int32_t *tiles, void *H,
                            int64_t rows_per_expert, void *part, size_t part_bytes, int act,
                            const float *b_up, hipStream_t s, void *Z = nullptr);
// dp: training-mode dropout on the rows of Y (default: none). ysh (bf16
// layers): when not NULL, Y is written compact, fp16 [N*k, d] with the
// shifts in ysh [N][ceil(d / kYGroup)][k]; otherwise Y is fp32 [N*k, d].
hipError_t launch_expert_down(bool bf16, const void *H, const void *w_down, int64_t d,
                              int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                              const int32_t *slot_token, const int32_t *tiles, void *Y,
                              int64_t rows_per_expert, void *part, size_t part_bytes,
                              const float *b_down, hipStream_t s, Dropout dp = Dropout{},
                              signed char *ysh = nullptr);

// Name of the kernel instantiation the expert product `product` (0: up, 1:
// down, with or without the dropout) launches for these sizes, as a profiler
// shows it; snprintf's return value.
int expert_kernel_name(bool bf16, int product, int64_t d, int64_t d_ff, int E,
                       int64_t rows_per_expert, bool dropout, char *buf, size_t len);

// Backward products over the dispatch plan (bf16 operands, fp32 accumulate;
// the weights are read K-major, as stored):
// dZ[e, r, :] = (dY[slot_token[e, r]] W_down[e]) * act'(z[e, r, :]), W_down
// [E, d, d_ff], bf16 into [E, ceff, d_ff]; act_in is H for ReLU
// (act' = [H > 0]) and the stored pre-activations Z for GELU;
// out[slot_token[e, r], :] = A[e, r, :] W[e] (A dense [E, ceff, K], W
// [E, K, Nout]), fp32.
hipError_t launch_expert_dz(const void *dY, const void *w_down, const void *act_in, int act,
                            int64_t d, int64_t d_ff, int E, int k, int64_t ceff,
                            const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                            void *dZ, int64_t rows_per_expert, hipStream_t s);
hipError_t launch_expert_rows_f32(const void *A, const void *w, int64_t K, int64_t Nout, int E,
                                  int k, int64_t ceff, const int32_t *used,
                                  const int32_t *slot_token, const int32_t *tiles, float *out,
                                  int64_t rows_per_expert, hipStream_t s);
// Weight gradient of every expert, O[e] (fp32 [M, N]) = sum over the
// expert's kept rows r < used[e] of A_r^T B_r, where A_r (M wide) and B_r (N
// wide) are rows of A and B: the gathered one (gathered == 0: A, 1: B) at
// slot_token[e*ceff + r] / kdiv, the other at e*ceff + r. Both operands are
// read K-major (no transposes). Needs ceff <= kGradMaxRows and M, N
// multiples of 8.
hipError_t launch_weight_grad(const void *A, int64_t M, const void *B, int64_t N, int E,
                              int64_t ceff, const int32_t *used, const int32_t *slot_token,
                              int kdiv, int gathered, float *out, hipStream_t s);
// C[b] (fp32 [M, Nout]) = A[b] [M, K] * W[b] [Nout, K]^T for b < batch, with
// element strides sa, sb, sc between batches; bf16 operands, K % 8 == 0.
hipError_t launch_batched_gemm_bf16(const void *A, const void *W, int64_t M, int64_t K,
                                    int64_t Nout, int batch, int64_t sa, int64_t sb, int64_t sc,
                                    float *C, hipStream_t s);

// Backward element-wise and layout kernels (backward.hip).
// dY rows (bf16, kept choices) = gate * dout; ds [N, k] = gate * (dg - sum gate*dg)
// with dg = <dout, Y> (Y: the experts' outputs, assignment-major, fp32 or,
// with ysh, compact as launch_expert_down writes them). d % 8 == 0.
// With dropout, dY = gate * dout * (the dropout factor of each Y element).
hipError_t launch_combine_backward(const void *dout, const void *Y, const signed char *ysh,
                                   const float *gate, const int32_t *slot, int64_t N, int64_t d,
                                   int k, void *dY, float *ds, hipStream_t s,
                                   Dropout dp = Dropout{});
// dsT3 [S][E][3*Tc] bf16: exact three-term split of ds(s*Tc + i, e) at columns
// i, Tc + i, 2*Tc + i (tokens chunked by Tc).
hipError_t launch_ds_split(const float *ds, const int32_t *idx, int64_t N, int64_t Tc, int64_t S,
                           int E, int k, void *dsT3, hipStream_t s);
// out[e][c] = sum over r < used[e] of src[row(e, r)][c] (bf16 rows of C
// columns, fp32 sums in a fixed order): row(e, r) = slot_token[e*ceff + r] /
// kdiv when slot_token is given, else e*ceff + r. C % 8 == 0.
hipError_t launch_colsum_rows(const void *src, int64_t C, int E, int64_t ceff,
                              const int32_t *used, const int32_t *slot_token, int kdiv,
                              float *out, hipStream_t s);
// out[i] = sum over r < Kp (fixed order) of T[i * Kp + r], bf16 T, fp32 out.
hipError_t launch_row_sums(const void *T, int64_t rows, int64_t Kp, float *out, hipStream_t s);
// out[i] = sum over s < S (in order) of part[s * n + i].
hipError_t launch_chunk_sum(const float *part, int64_t S, int64_t n, float *out, hipStream_t s);
// out[b][c][q*Kp + r] = src row R(b, r), column c (0 past the batch's rows), for
// q < copies; map 0: b*ceff + r (without used: min(ceff, nrows - b*ceff) rows),
// 1: slot_token[b*ceff + r], 2: slot_token[...] / k. C % 8 == 0, Kp % 8 == 0.
hipError_t launch_transpose_rows(const void *src, int64_t C, int64_t ceff, const int32_t *used,
                                 int64_t nrows, const int32_t *slot_token, int k, int map,
                                 int64_t Kp, int copies, int batch, void *out, hipStream_t s);
// dx = sum of the kept choices' dX rows + sum_j ds[t, j] W_g[idx[t, j]] (fp32, d % 4 == 0);
// ids outside [0, E) contribute nothing.
hipError_t launch_dx(const float *dXa, const float *ds, const int32_t *idx, const int32_t *slot,
                     const float *Wg, int64_t N, int64_t d, int E, int k, float *dx,
                     hipStream_t s);

// Router scores for more than 32 experts: x [N, d] bf16 against the split
// weights wsp [Ep][3 d] bf16 (hi, mid and lo terms of each expert's row),
// all three terms accumulated into one fp32 score; the K dimension is cut
// into router_score_splits() ranges whose partial scores go to
// P [splits][N][Ep] fp32 (summed in range order by the ranking).
int router_score_splits(int64_t N, int64_t d, int64_t Ep);
// Whether the split weights interleave the three terms per 64 columns
// (row layout [d / 64][3][64]) rather than placing them one after the other.
bool router_terms_interleaved(int64_t d);
hipError_t launch_router_scores_bf16(const void *x, const void *wsp, int64_t N, int64_t d,
                                     int64_t Ep, float *P, hipStream_t s);

// Y: [N*k, d] rows of dtype y_dtype (0 fp32, 1 bf16); out of dtype out_dtype.
hipError_t launch_combine(const void *Y, int y_dtype, const float *gate, const int32_t *slot,
                          int64_t N, int64_t d, int k, void *out, int out_dtype,
                          hipStream_t s);
// The same over compact rows: Y fp16 [N*k, d] with shifts ysh [N][ceil(d /
// kYGroup)][k] (see yshift_index); d % 8 == 0.
hipError_t launch_combine_compact(const void *Y, const signed char *ysh, const float *gate,
                                  const int32_t *slot, int64_t N, int64_t d, int k, void *out,
                                  int out_dtype, hipStream_t s);

}  // namespace moe
