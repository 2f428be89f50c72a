// Grouped expert FFN over the dispatch plan.
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 7 (each token is copied only to its kept experts), STEP 8 (z = W_up x),
// STEP 9 (h = ReLU(z)), STEP 10 (E(x) = W_down h); nanoMoE slides 32-37 (the
// experts are batched: one product per expert over its packed token rows;
// slide 32 also gives the expert variant with biases and GELU).
//
//   up:   H[e, r, :] = act(W_up[e] x_t + b_up[e])  for r < used[e], t = slot_token[e, r] / k
//   down: Y[a, :]    = W_down[e] H[e, r, :] + b_down[e]  with a = slot_token[e, r], fp32
//
// Both are "NT" products: every operand row is contiguous along the
// reduction dimension (activation rows along d or d_ff, weight rows are
// output neurons), which is exactly the K-contiguous layout both operands of
// a CDNA matrix instruction want. The gather of token rows (dispatch) is
// fused into the up product's operand load, so no packed copy of the tokens
// is ever written; the down product scatters its rows straight into the
// assignment-ordered buffer the combine reads. Both accumulate in fp32; H is
// rounded once to bf16 in the epilogue, Y stays fp32 (the combine rounds the
// gate-weighted sum once).
//
// bf16 kernel: a BM x BN output tile per workgroup, K-step 64 (128 for the
// tile of two K sets), waves laid out WAVES_M x WAVES_N (times WAVES_K sets
// that share each K-step) with a 16x16x32 bf16 MFMA grid each. A and B K-tiles go
// from global memory straight into a two-stage LDS ring (direct 16-byte
// loads, no register round trip; 16-byte chunks XOR-swizzled per row so the
// operand reads of a wave hit distinct banks); the loads of step kt+1 are
// issued before the MFMAs of step kt and stay in flight across the barrier,
// which waits on LDS traffic only. Waves skip the MFMAs of 16-row strips
// that lie wholly past used[e]. The epilogue transposes each wave's 16-row
// strips through LDS so every lane stores 16 contiguous bytes.
//
// Scheduling: tiles exist only for rows that exist (the dispatch plan's
// prefix of ceil(used[e]/BM), read on the device, so no host sync). The tile
// index walks an expert's row tiles fastest, so the blocks in flight share
// each weight tile, and block b (placed on XCD b mod 8 by the dispatcher)
// takes tile (b mod 8) * T/8 + b/8: every XCD works through one contiguous
// range of tiles and the sharing happens inside its own L2. When the last
// round of tiles would leave most workgroups idle, its tiles are cut into
// K-ranges (split_plan below); when the tiles just overflow one round, the
// light last row tiles of the experts go last (partial_prefix below).
#include <stdio.h>

#include <algorithm>
#include <type_traits>

#include "common.hpp"

namespace moe {
namespace {

constexpr int kXcds = 8;

// Workgroup barrier that waits for this wave's LDS traffic only (no memory
// fence, so the compiler does not drain outstanding global loads here).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Wait until at most N of this wave's vector-memory operations are in flight.
template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// 32-bit LDS offset of a pointer into __shared__ memory.
__device__ __forceinline__ unsigned lds_off(const void *p) {
    return (unsigned)(uintptr_t)((__attribute__((address_space(3))) const void *)p);
}

// A K-major operand tile ([BKT rows of K][BN columns], 16-byte chunks) keeps
// chunk c of row r at position c ^ tr_swizzle(r). One transposing read
// touches 16 rows (4 rows in each of 4 lane groups g: rows 8g + 4h + 0..3)
// and an aligned pair of chunks in each. Rows of 16 or more chunks: the 16
// rows take 8 distinct even offsets, so the 64 lanes hit every bank at most
// twice. Rows of 8 chunks (two rows per 256-byte bank row): rows of equal
// parity must take distinct pairs, which bits 1 and 3 of r give (rows
// 8g + 4h + j of two lane groups g, g + 1).
__device__ __forceinline__ int tr_swizzle(int r, int chunks_per_row) {
    if (chunks_per_row == 8)
        return 2 * (((r >> 1) & 1) | (((r >> 3) & 1) << 1));
    const int h = (r & 3) | ((((r >> 3) ^ (r >> 2)) & 1) << 2);
    return (2 * h) & (chunks_per_row - 1);
}

// Transposing LDS read (gfx950 ds_read_b64_tr_b16): within each group of 16
// lanes, lane l receives element l % 4 of the 8 bytes that lane
// 4q + l / 4 addresses, as its element q (q = 0..3). With lane s of a group
// addressing row kb + s / 4, columns 4 (s % 4) .. +3 of a K-major tile,
// lane l gets column l of rows kb .. kb + 3: a quarter of an MFMA operand
// fragment.
typedef short v4i16 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i16 lds_read_tr16(const void *p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) v4i16 *)(p));
}

// GELU of the nanoMoE slides' expert (slide 32): z * Phi(z), Phi(z) =
// (1 + erf(z / sqrt 2)) / 2, with erf from Abramowitz and Stegun, Handbook of
// Mathematical Functions, formula 7.1.26: for u >= 0,
// 1 - erf(u) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-u^2),
// t = 1 / (1 + p u), with absolute error below 1.5e-7 (far below the bf16
// rounding of H that follows). For z < 0 the complement is used directly, so
// small GELU values keep their relative accuracy.
__device__ __forceinline__ float gelu(float z) {
    const float u = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
    const float poly =
        t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                         -0.284496736f),
                 0.254829592f);
    const float q = poly * __expf(-u * u);   // 1 - erf(u)
    return 0.5f * z * (z >= 0.f ? 2.0f - q : q);
}

// Its derivative Phi(z) + z phi(z): Phi from the same erf approximation,
// phi(z) = exp(-z^2 / 2) / sqrt(2 pi) from the same exponential.
__device__ __forceinline__ float gelu_grad(float z) {
    const float u = fabsf(z) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
    const float poly =
        t * fmaf(t, fmaf(t, fmaf(t, fmaf(t, 1.061405429f, -1.453152027f), 1.421413741f),
                         -0.284496736f),
                 0.254829592f);
    const float ex = __expf(-u * u);         // exp(-z^2 / 2)
    const float q = poly * ex;               // 1 - erf(u)
    const float Phi = 0.5f * (z >= 0.f ? 2.0f - q : q);
    return fmaf(z * 0.39894228040143268f, ex, Phi);
}

// Expert activation: ReLU (page 1 STEP 9) or GELU, chosen at compile time so
// that the ReLU epilogue carries no trace of the other.
template <bool GELU>
__device__ __forceinline__ float activate(float z) {
    if constexpr (GELU)
        return gelu(z);
    else
        return fmaxf(z, 0.f);
}

// Largest v over aligned groups of G (1, 2 or 4) adjacent lanes, by
// data-parallel moves within each quad of lanes (quad_perm: lane ^ 1, then
// lane ^ 2): no LDS round trip. Every lane of a group must be active.
template <int G>
__device__ __forceinline__ float quad_group_max(float v) {
    static_assert(G == 1 || G == 2 || G == 4, "groups within a quad");
    if constexpr (G >= 2)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF,
                                                               0xF, false)));   // [1,0,3,2]
    if constexpr (G == 4)
        v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF,
                                                               0xF, false)));   // [2,3,0,1]
    return v;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's bytes land at
// LDS offset m0 + 16*l (one wave moves 1 KB). Issued in asm so that the
// compiler's wait insertion does not treat every later LDS read as aliasing
// it; the waits are explicit (wait_vm).
__device__ __forceinline__ void dma16(unsigned lds_base, const void *g) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
                 ::"s"(lds_base), "v"(g)
                 : "memory", "m0");
}

// Work split of a grouped product with T output tiles of KT K-steps over P
// workgroups that can run at once. Whole tiles fill the full rounds. When
// the last round would leave most workgroups idle, its `tail` tiles are cut
// into nsplit K-ranges; each range's fp32 partial tile goes to a scratch
// slot and split_fixup_kernel adds the ranges of a tile in K order. The cut
// is taken only when it shortens the product by at least 15% on paper
// ((1 - 1/nsplit) of one round out of R + 1): with many full rounds the
// rounds blur (tiles differ in cost) and the partial-tile traffic eats the
// gain. The plan depends only on (T, KT, P), so it and the result are the
// same on every run.
struct SplitPlan {
    int Tdp;      // tiles computed whole
    int tail;     // tiles cut into K-ranges (the last `tail` tile indices)
    int nsplit;   // K-ranges per cut tile (1: no split)
};

constexpr int kSplitMinSteps = 8;   // K-steps of the shortest range

__device__ __forceinline__ SplitPlan split_plan(int T, int KT, int P) {
    SplitPlan p{T, 0, 1};
    if (P <= 0 || T < P)
        return p;
    const int R = T / P, tail = T % P;
    if (tail == 0)
        return p;
    int ns = P / tail;
    if (ns > KT / kSplitMinSteps)
        ns = KT / kSplitMinSteps;
    if (ns < 2 || 20 * (ns - 1) < 3 * (R + 1) * ns)
        return p;
    p.Tdp = T - tail;
    p.tail = tail;
    p.nsplit = ns;
    return p;
}

// Order of the grouped schedule's T = s_mt[E]*NT tiles (s_mt: prefix sums
// of each expert's row tiles, ceil(used/BM)): expert by expert, row tiles
// fastest. When all tiles do not fit in one round of resident workgroups
// but those with more than BM/2 kept rows do, those come first and the
// light last row tiles (at most BM/2 kept rows) follow, expert by expert,
// columns fastest: workgroups are dispatched in index order, so it is the
// light tiles (their padding rows skip the matrix instructions) that wait
// for the round to free a CU, not heavy ones. Otherwise the plain order
// stays: a light tile then runs beside the other tiles of its expert and
// column, on the same XCD, whose operands it shares in that XCD's L2.
// s_pp[e] (e <= E): experts before e whose last row tile is light.
// Needs at least 256 threads (E <= 256); ends with a barrier.
__device__ __forceinline__ void partial_prefix(const int32_t *__restrict__ used, int E, int BM,
                                               int nthr, int *s_pp, uint64_t *s_msk) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (w < kMaxExperts / 64) {
        const int e = w * 64 + lane;
        const int rm = e < E ? used[e] % BM : 0;
        const uint64_t m = __ballot(rm != 0 && 2 * rm <= BM);
        if (lane == 0)
            s_msk[w] = m;
    }
    __syncthreads();
    for (int i = tid; i <= E; i += nthr) {
        int c = 0;
        for (int ww = 0; ww < i / 64; ++ww)
            c += __popcll(s_msk[ww]);
        if (i % 64)
            c += __popcll(s_msk[i / 64] & (~0ull >> (64 - i % 64)));
        s_pp[i] = c;
    }
    __syncthreads();
}

// Largest e in [0, E) with f(e) <= v (f non-decreasing, f(0) <= v).
template <typename F>
__device__ __forceinline__ int last_at_most(F f, int E, int v) {
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (f(mid) <= v) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Whether the light tiles go last (see above), P resident workgroups; s_mt
// must be in LDS. The light-tile prefix is only computed (with s_msk, two
// barriers) when the order can change: at most one tile per expert and
// column is light, so with more than P + E*NT tiles the heavy ones overflow
// the round anyway.
__device__ __forceinline__ bool light_last(const int32_t *__restrict__ used, const int *s_mt,
                                          int E, int NT, int BM, int P, int nthr, int *s_pp,
                                          uint64_t *s_msk) {
    const int T = s_mt[E] * NT;
    if (T <= P || T - E * NT > P)
        return false;
    partial_prefix(used, E, BM, nthr, s_pp, s_msk);
    return s_pp[E] > 0 && (s_mt[E] - s_pp[E]) * NT <= P;
}

// s_mt[e] = sum over e' < e of ceil(used[e'] / BM), for e <= E: the row
// tiles of a tile height the dispatch plan has no table for (and used[e]
// itself in s_used when given). Needs nthr >= kMaxExperts; s_tmp holds one
// int per wave; ends with a barrier.
__device__ __forceinline__ void row_tile_prefix(const int32_t *__restrict__ used, int E, int BM,
                                                int *s_mt, int *s_tmp, int *s_used = nullptr) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int c = 0;
    if (tid < E) {
        const int u = used[tid];
        c = (u + BM - 1) / BM;
        if (s_used)
            s_used[tid] = u;
    }
    int inc = c;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(inc, off);
        if (lane >= off)
            inc += o;
    }
    if (w < kMaxExperts / 64 && lane == 63)
        s_tmp[w] = inc;
    __syncthreads();
    if (tid < kMaxExperts) {
        for (int ww = 0; ww < w; ++ww)
            inc += s_tmp[ww];
        if (tid < E)
            s_mt[tid + 1] = inc;
        if (tid == 0)
            s_mt[0] = 0;
    }
    __syncthreads();
}

// Expert e owning tile L of the schedule above, and its tile origin
// (s_pp = NULL: the plain order).
__device__ __forceinline__ void decode_tile(int L, const int *s_mt, const int *s_pp, int E,
                                            int NT, int BM, int BN, int &e, int &m0, int &n0) {
    if (!s_pp) {
        e = last_at_most([&](int x) { return s_mt[x] * NT; }, E, L);
        const int mte = s_mt[e + 1] - s_mt[e];
        const int local = L - s_mt[e] * NT;
        m0 = (local % mte) * BM;
        n0 = (local / mte) * BN;
        return;
    }
    // heavy row tiles before expert e: s_mt[e] - s_pp[e]
    const int TA = (s_mt[E] - s_pp[E]) * NT;
    if (L < TA) {
        e = last_at_most([&](int x) { return (s_mt[x] - s_pp[x]) * NT; }, E, L);
        const int f0 = s_mt[e] - s_pp[e];
        const int nf = s_mt[e + 1] - s_pp[e + 1] - f0;
        const int local = L - f0 * NT;
        m0 = (local % nf) * BM;
        n0 = (local / nf) * BN;
    } else {
        const int q = (L - TA) / NT;   // q-th expert with a light last tile
        e = last_at_most([&](int x) { return s_pp[x]; }, E, q);
        m0 = (s_mt[e + 1] - s_mt[e] - 1) * BM;
        n0 = ((L - TA) % NT) * BN;
    }
}

// Block b of a launch whose first T8 blocks take whole tiles: block b runs on
// XCD b mod 8, and takes index (b mod 8) * T8/8 + b/8, so every XCD works
// through one contiguous range of indices (sharing operands in its own L2).
__device__ __forceinline__ int xcd_index(int b, int T8) {
    return (b % kXcds) * (T8 / kXcds) + b / kXcds;
}

// BM x BN output tile, K-step BKT, S-stage LDS ring filled by direct loads.
// Each K-tile row is BKT bf16 = RB bytes of 16-byte chunks; chunk c of row r
// is stored at position c ^ ((r / RPB) % CPR) (RPB rows share one 256-byte
// bank row), so the 16 lanes that read 16 consecutive rows at one chunk hit
// 16 distinct bank groups.
// Two waves per SIMD (the LDS budget allows no more), so the compiler may use
// up to 256 registers per lane and schedule for latency rather than occupancy;
// a tile of 16 waves runs four per SIMD with up to 128 registers each.
// MODE 0: up product (gathered token rows, activation, bf16 H into O16);
// 1: down product (fp32 rows of Y scattered to their assignment, into O32);
// 2: plain product of ceff rows of A into fp32 rows of O32 (no gather, no
// schedule table, no split), batched over blockIdx.y with element strides
// bsa, bsb, bsc of A, W and O32;
// 3: backward of the down product through the activation, dZ = (dY W_down)
// times act'(z): A rows are assignment rows of dY gathered by slot_token, W
// is W_down, bf16 [E, ceff, Nout] into O16; for ReLU mask = H
// (act' = [H > 0]), for GELU mask = the stored pre-activations Z, which may
// be O16 itself (each element is read before the same thread overwrites it);
// 4: backward of the up product, dX = dZ W_up: A rows dense like MODE 1,
// fp32 rows scattered to their assignment into O32.
// In modes 3 and 4 the right operand is the weight matrix itself, read
// K-major: W[e] is [K][Nout] (Nout contiguous: W_down for MODE 3, W_up for
// MODE 4); its tiles are staged row by row and turned into MFMA fragments
// by transposing LDS reads.
// part: scratch for the split of the last round (NULL: no split), P: the
// number of workgroups of this kernel that fit on the device at once (0:
// unknown; it sizes the split and chooses the tile order).
// act: activation of the up product (kActRelu, kActGelu); bias: [E, Nout]
// fp32 added to the product before the activation (MODE 0) or to the output
// row (MODE 1), or NULL. K-range partials take neither (the fix-up does).
// Z16 (MODE 0): when not NULL, the bf16 pre-activations (product plus bias)
// are stored there too, [E, ceff, Nout] like H (by the fix-up for cut tiles).
// ysh (MODES 1, 5): when not NULL, the rows of Y are stored compact (fp16
// values into O16 and one exponent shift per kYGroup columns into ysh, at
// yshift_index) instead of fp32 into O32.
// 5: MODE 1 with training-mode dropout dp on the rows of Y, after the bias
// (its own instantiation, so that the plain down product's epilogue carries
// none of the generator's code or registers).
// 6: weight gradient of expert e = blockIdx.y, O32[e] (fp32 [M, Nout]) =
// sum over the expert's kept rows r < used[e] of A(r, :)^T B(r, :): both
// operands K-major rows, A rows of width M = bsa, B rows of width Nout; the
// row of r is slot_token[e*ceff + r] / k for the gathered operand (act == 0:
// A, act == 1: B) and e*ceff + r for the other; bsc = M*Nout. K is unused
// (each expert's K is used[e]; kGradMaxRows bounds ceff).
// 7: router scores, a plain product of ceff rows of A (x, rows of bsa = d)
// with W = the three-term split of the router weights, [Nout][K] with
// K = 3 d (row e: the hi, mid and lo terms of expert e's weights, either
// interleaved per 64 columns, bsb = 1, each 64 columns of x read three
// times in a row, or one term after the other, bsb = 0), A's column taken
// from the term's, so that all three terms of an expert accumulate into
// one fp32 score; K is cut into gridDim.y ranges of K-steps,
// range s writing its fp32 partial scores to O32 + s * bsc.
// WAVES_K > 1 (modes 0, 1, 2, 5): WAVES_K sets of WAVES_M x WAVES_N waves
// share each K-step, set w taking its 32-wide MFMA steps w, w + WAVES_K, ...;
// after the last step the sets add their partial tiles into set 0 through
// LDS, in set order, and set 0 runs the epilogue. Same LDS reads per MFMA as
// WAVES_K = 1, with WAVES_K times the waves to hide latency.
template <int BM, int BN, int WAVES_M, int WAVES_N, int WAVES_K, int BKT, int S, int MODE>
__global__ __launch_bounds__(WAVES_M * WAVES_N * WAVES_K * 64)
__attribute__((amdgpu_waves_per_eu(WAVES_M * WAVES_N * WAVES_K >= 16 ? 4 : 2,
                                   WAVES_M * WAVES_N * WAVES_K >= 16 ? 4 : 2)))
void expert_gemm_kernel(
    const unsigned short *__restrict__ A_src, const unsigned short *__restrict__ W, int K,
    int Nout, int E, int k, int ceff, const int32_t *__restrict__ used,
    const int32_t *__restrict__ slot_token, const int32_t *__restrict__ mt_off,
    unsigned short *__restrict__ O16, float *__restrict__ O32, float *__restrict__ part,
    int P, int act, const float *__restrict__ bias, const unsigned short *mask,
    unsigned short *__restrict__ Z16, Dropout dp, int64_t bsa, int64_t bsb, int64_t bsc,
    signed char *__restrict__ ysh) {
    constexpr int WMN = WAVES_M * WAVES_N;                   // waves of one K set
    constexpr int NW = WMN * WAVES_K;
    constexpr int NTHR = NW * 64;
    constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;   // wave tile
    constexpr int FM = WTM / 16, FN = WTN / 16;              // 16x16 MFMA tiles per wave
    constexpr int RB = BKT * 2;                              // bytes per K-tile row
    constexpr int CPR = BKT / 8;                             // 16-byte chunks per row
    constexpr int RPB = 256 / RB;                            // rows per 256-byte bank row
    constexpr int RPI = 1024 / RB;                           // rows per direct-load wave op
    constexpr bool AT = MODE == 6;                           // A read K-major
    constexpr bool BT = MODE == 3 || MODE == 4 || MODE == 6; // B read K-major
    constexpr bool RM = !AT && !BT;                          // both row-major
    // Row-major operands: the A and B rows of a stage form one space of TOT
    // direct-load ops (RPI rows each), op q filling LDS bytes [q KB, q KB +
    // 1 KB) of the stage: A rows first, then B rows, the stage's layout.
    // Wave w issues ops w*GC .. w*GC + GC - 1 that exist.
    constexpr int TOT = (BM + BN) / RPI;
    constexpr int GC = (TOT + NW - 1) / NW;
    // K-major operands: IA and IB ops per wave per stage
    constexpr int IA = RM ? 0 : BM / (RPI * NW), IB = RM ? 0 : BN / (RPI * NW);
    constexpr int G = RM ? GC : IA + IB;                     // ops per wave per stage (at most)
    constexpr int STAGE = (BM + BN) * RB;                    // bytes per stage
    static_assert(BKT % 32 == 0 && S >= 2, "K-step is a multiple of one MFMA K");
    static_assert(RM ? (BM % RPI == 0 && BN % RPI == 0 && (S == 2 || TOT % NW == 0))
                     : (BM % (RPI * NW) == 0 && BN % (RPI * NW) == 0),
                  "tile/waves mismatch");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "16x16 MFMA tiles; 4 lanes x 8k columns per row");
    static_assert(WMN * 16 * (WTN + 4) * 4 <= S * STAGE, "epilogue scratch");
    static_assert(WAVES_K == 1 || (MODE != 3 && MODE != 4 && MODE != 6), "K sets: row-major B");
    static_assert((WAVES_K & (WAVES_K - 1)) == 0, "K sets: a power of two");
    static_assert(MODE == 2 || MODE == 6 || MODE == 7 || NTHR >= kMaxExperts,
                  "schedule prefix: a lane per expert");
    static_assert(WAVES_K / 2 * WMN * FM * FN * 64 * 16 <= S * STAGE, "K-set reduction");
    __shared__ __attribute__((aligned(1024)))
    char smem[S * STAGE + (MODE == 6 ? kGradMaxRows * 4 : 0)];
    __shared__ int s_mt[kMaxExperts + 1];
    __shared__ int s_pp[kMaxExperts + 1];
    __shared__ int s_used[kMaxExperts];   // used[], read once per workgroup
    __shared__ uint64_t s_msk[kMaxExperts / 64];
    // MODE 0: token of each tile row; 1, 4, 5: the assignment row its output
    // goes to (read by the epilogue from LDS, so that its stores never wait
    // behind a global load)
    constexpr bool TOK = MODE == 0 || MODE == 1 || MODE == 4 || MODE == 5;
    __shared__ int s_tok[TOK ? BM : 1];
    int *s_rows = reinterpret_cast<int *>(smem + S * STAGE);   // MODE 6: row of each r

    const int tid = threadIdx.x;
    const int NT = (Nout + BN - 1) / BN;
    int Kr = K;            // reduction length (MODE 6: the expert's kept rows)
    int KT = (K + BKT - 1) / BKT;
    // Grouped products (modes 0, 1, 3, 4, 5): the schedule (row-tile prefix
    // of the experts, split plan, tile order) is set up once per workgroup.
    // Work items: whole tiles in two launch segments (heavy ones, then light
    // ones when those go last), each spread over the XCDs, then the K-ranges
    // of the cut tiles. With the 320-row tiles of the forward products the
    // launch is persistent: one workgroup per resident slot (a multiple of
    // the XCD count, so that items b, b + gridDim.x, ... stay on one XCD)
    // walks items b, b + gridDim.x, ..., and a tile's fixed costs (workgroup
    // start, schedule set-up) are paid once per workgroup; otherwise one
    // item per workgroup.
    constexpr bool GROUPED = MODE != 2 && MODE != 6 && MODE != 7;
    constexpr bool PERSIST = BM == 320 && (MODE == 0 || MODE == 1 || MODE == 5);
    SplitPlan sp{0, 0, 1};
    bool ll = false;
    int T1 = 0, T18 = 0, T28 = 0, np8 = 0;
    if constexpr (GROUPED) {
        if (mt_off) {
            for (int i = tid; i <= E; i += NTHR)
                s_mt[i] = mt_off[i];
            for (int i = tid; i < E; i += NTHR)
                s_used[i] = used[i];
            __syncthreads();
        } else {
            row_tile_prefix(used, E, BM, s_mt, reinterpret_cast<int *>(s_msk), s_used);
        }
        const int T = s_mt[E] * NT;
        sp = split_plan(T, KT, part ? P : 0);
        // (the 320-row tile holds every expert of up to 320 rows: a light
        // last tile is rare there and not worth the extra pass over used)
        ll = BM == 320 ? false : light_last(used, s_mt, E, NT, BM, P, NTHR, s_pp, s_msk);
        T1 = ll ? min((s_mt[E] - s_pp[E]) * NT, sp.Tdp) : sp.Tdp;
        T18 = (T1 + kXcds - 1) / kXcds * kXcds;
        T28 = (sp.Tdp - T1 + kXcds - 1) / kXcds * kXcds;
        np8 = (sp.tail * sp.nsplit + kXcds - 1) / kXcds * kXcds;
    }
    const int nitems = PERSIST ? T18 + T28 + np8 : 0;
    const int stride = PERSIST ? (int)gridDim.x : 0;
    // (one trip, known at compile time, unless persistent)
    for (int it = 0, b = blockIdx.x; PERSIST ? b < nitems : it < 1; ++it, b += stride) {
    int e, m0, n0, rows;
    int kb = 0, ke = KT;   // K-steps of this item
    int piece = -1;        // scratch slot of a K-range, or -1 for a whole tile
    if constexpr (MODE == 6) {
        e = blockIdx.y;
        const int M = (int)bsa;
        O32 += (int64_t)e * bsc;
        const int mte = (M + BM - 1) / BM;
        const int T = mte * NT;
        const int T8 = (T + kXcds - 1) / kXcds * kXcds;
        if (b >= T8)
            return;
        const int L = xcd_index(b, T8);
        if (L >= T)
            return;
        rows = M;
        m0 = (L % mte) * BM;
        n0 = (L / mte) * BN;
        Kr = used[e];
        KT = (Kr + BKT - 1) / BKT;
        ke = KT;
        const int32_t *stp = slot_token + (int64_t)e * ceff;
        for (int i = tid; i < Kr; i += NTHR)
            s_rows[i] = stp[i] / k;
        __syncthreads();
    } else if constexpr (MODE == 2 || MODE == 7) {
        // plain product over ceff rows, one "expert" (MODE 2) or K-range
        // (MODE 7) per blockIdx.y: no schedule table
        if constexpr (MODE == 2) {
            A_src += blockIdx.y * bsa;
            W += blockIdx.y * bsb;
        } else {
            kb = (int)((int64_t)blockIdx.y * KT / gridDim.y);
            ke = (int)((int64_t)(blockIdx.y + 1) * KT / gridDim.y);
        }
        O32 += blockIdx.y * bsc;
        const int mte = (ceff + BM - 1) / BM;
        const int T = mte * NT;
        const int T8 = (T + kXcds - 1) / kXcds * kXcds;
        if (b >= T8)
            return;
        const int L = xcd_index(b, T8);
        if (L >= T)
            return;
        e = 0;
        rows = ceff;
        m0 = (L % mte) * BM;
        n0 = (L / mte) * BN;
    } else {
        // (an item past the schedule's end: `continue` leaves the loop, or
        // goes on to this workgroup's next item, with every wave alike)
        int L;
        if (b < T18) {
            L = xcd_index(b, T18);
            if (L >= T1)
                continue;
        } else if (b < T18 + T28) {
            L = T1 + xcd_index(b - T18, T28);
            if (L >= sp.Tdp)
                continue;
        } else {
            const int np = sp.tail * sp.nsplit;
            if (b - T18 - T28 >= np8)
                continue;
            piece = xcd_index(b - T18 - T28, np8);
            if (piece >= np)
                continue;
            L = sp.Tdp + piece / sp.nsplit;
            const int s = piece % sp.nsplit;
            kb = (int)((int64_t)s * KT / sp.nsplit);
            ke = (int)((int64_t)(s + 1) * KT / sp.nsplit);
        }
        decode_tile(L, s_mt, ll ? s_pp : nullptr, E, NT, BM, BN, e, m0, n0);
        rows = s_used[e];
    }

    if constexpr ((MODE == 1 || MODE == 5) && BM == 320) {
        // Staggered start of the first round: its workgroups begin in 8
        // groups 4 us apart (by position within their XCD). Every tile of
        // this product ends by writing BM x BN fp32 output rows (320 KB);
        // when all CUs start together they all write at once and the write
        // phases add up, while spread out they overlap other CUs' products.
        // At most 28 us once per launch; every wave leaves the wait.
        if (b == (int)blockIdx.x && b < P && piece < 0) {
            const long long t0 = wall_clock64();   // 100 MHz
            const long long dt = (long long)((b / kXcds) % 8) * 400;
            while (wall_clock64() - t0 < dt)
                __builtin_amdgcn_s_sleep(8);
        }
    }
    const int lane = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wk = WAVES_K == 1 ? 0 : wv / WMN;   // K set
    const int wm = (wv % WMN) / WAVES_N, wn = wv % WAVES_N;

    // Direct-load sources of this lane: one row and one 16-byte chunk per op.
    // Rows past the tile edge read row 0 of the expert (their outputs are
    // never stored); the K tail is zeroed in LDS after the last step lands.
    const unsigned short *gc[RM ? GC : 1];
    int cc[RM ? GC : 1];
    const unsigned short *We = W + (int64_t)__builtin_amdgcn_readfirstlane(e) * Nout * K;
    // the tile's token rows (MODE 0) or assignment rows, one load per thread
    // rather than a chain of dependent loads per op or per strip. The
    // assignment rows are only read by the epilogue: they are loaded after
    // the first K-step's operand loads are issued, so that the two round
    // trips overlap, and published by the main loop's barriers.
    auto fill_tok = [&]() {
        for (int i = tid; i < BM; i += NTHR) {
            const int r = m0 + i;
            const int v = slot_token[(int64_t)e * ceff + (r < rows ? r : 0)];
            s_tok[i] = MODE == 0 ? v / k : v;
        }
    };
    if constexpr (MODE == 0) {
        fill_tok();
        __syncthreads();
    }
    if constexpr (RM) {
#pragma unroll
        for (int i = 0; i < GC; ++i) {
            const int q = min(wv * GC + i, TOT - 1);   // ops past TOT are not issued
            const bool isA = q * RPI < BM;              // the same for the whole op
            const int row = (isA ? q * RPI : q * RPI - BM) + lane / CPR;
            const int c = (lane % CPR) ^ ((row / RPB) % CPR);
            const int r = m0 + row, n = n0 + row;
            const int64_t srow = (int64_t)e * ceff + (r < rows ? r : 0);
            const int64_t asrc = MODE == 0 ? (int64_t)s_tok[min(row, BM - 1)] : srow;
            const int64_t src = isA ? asrc : (int64_t)(n < Nout ? n : 0);
            cc[i] = c;
            gc[i] = (isA ? A_src : We) + src * (MODE == 7 && isA ? (int)bsa : K);
        }
    }
    const unsigned short *ga[IA > 0 ? IA : 1];
    const unsigned short *gb[IB > 0 ? IB : 1];
    int ca[IA > 0 ? IA : 1], cb[IB > 0 ? IB : 1];
    // K-major left operand (MODE 6): like the right one below, with M
    // columns of width bsa
    constexpr int RBTA = BM * 2, CPRTA = BM / 8;
    static_assert(!AT || (BM & (BM - 1)) == 0, "K-major tiles are a power of two wide");
    int ak[AT ? IA : 1];
    const bool gatherA = MODE == 6 && act == 0, gatherB = MODE == 6 && act == 1;
#pragma unroll
    for (int i = 0; i < IA; ++i) {
        if constexpr (AT) {
            const int M = (int)bsa;
            const int q = (wv * IA + i) * 64 + lane;        // 16-byte slot in the tile
            const int row = q / CPRTA;
            const int c = (q % CPRTA) ^ tr_swizzle(row, CPRTA);
            const int m = m0 + 8 * c;
            ak[i] = row;
            ca[i] = 0;
            ga[i] = A_src + (m < M ? m : M - 8);
        } else {
            const int row = (wv * IA + i) * RPI + lane / CPR;
            ca[i] = (lane % CPR) ^ ((row / RPB) % CPR);
            const int r = m0 + row;
            const int64_t srow = (int64_t)e * ceff + (r < rows ? r : 0);
            const int64_t src = MODE == 0   ? (int64_t)(slot_token[srow] / k)
                                : MODE == 3 ? (int64_t)slot_token[srow]
                                            : srow;
            ga[i] = A_src + src * K;
        }
    }
    // K-major right operand: per op, the LDS row (k within the K-step) and a
    // pointer to its 8 columns in row 0 of W[e]; columns past Nout read the
    // last 8 (never stored), rows past K read row K - 1 (A's K tail is 0)
    constexpr int RBT = BN * 2, CPRT = BN / 8;   // bytes, 16-byte chunks per K-major row
    static_assert(!BT || (BN & (BN - 1)) == 0, "K-major tiles are a power of two wide");
    int bk[BT ? IB : 1];
#pragma unroll
    for (int i = 0; i < IB; ++i) {
        if constexpr (BT) {
            const int q = (wv * IB + i) * 64 + lane;        // 16-byte slot in the tile
            const int row = q / CPRT;
            const int c = (q % CPRT) ^ tr_swizzle(row, CPRT);
            const int n = n0 + 8 * c;
            bk[i] = row;
            cb[i] = 0;
            gb[i] = W + (MODE == 6 ? 0 : (int64_t)e * K * Nout) + (n < Nout ? n : Nout - 8);
        } else {
            const int row = (wv * IB + i) * RPI + lane / CPR;
            cb[i] = (lane % CPR) ^ ((row / RPB) % CPR);
            const int n = n0 + row;
            gb[i] = W + ((int64_t)e * Nout + (n < Nout ? n : 0)) * K;
        }
    }
    const unsigned smem_off = lds_off(smem);
    auto issue = [&](int kt) {
        const unsigned base = smem_off + (unsigned)((kt % S) * STAGE);
        if constexpr (RM) {
#pragma unroll
            for (int i = 0; i < GC; ++i) {
                if (TOT % NW == 0 || wv * GC + i < TOT) {
                    int kk = min(kt * BKT + cc[i] * 8, K - 8);
                    if (MODE == 7 && (wv * GC + i) * RPI < BM) {
                        // A's column of the term this chunk belongs to:
                        // terms interleaved per 64 columns (bsb = 1), or
                        // one after the other
                        const int d = (int)bsa;
                        kk = bsb ? (kk / 192) * 64 + kk % 64
                                 : kk >= 2 * d ? kk - 2 * d : kk >= d ? kk - d : kk;
                    }
                    dma16(base + (unsigned)((wv * GC + i) * 1024), gc[i] + kk);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < IA; ++i) {
            if constexpr (AT) {
                const int kr = min(kt * BKT + ak[i], Kr - 1);
                const int64_t gi = gatherA ? (int64_t)s_rows[kr] : (int64_t)e * ceff + kr;
                dma16(base + (unsigned)((wv * IA + i) * 1024), ga[i] + gi * bsa);
            } else {
                const int kk = min(kt * BKT + ca[i] * 8, K - 8);
                dma16(base + (unsigned)((wv * IA + i) * 1024), ga[i] + kk);
            }
        }
#pragma unroll
        for (int i = 0; i < IB; ++i) {
            if constexpr (BT) {
                const int kr = min(kt * BKT + bk[i], Kr - 1);
                const int64_t gi = MODE != 6 ? (int64_t)kr
                                   : gatherB ? (int64_t)s_rows[kr]
                                             : (int64_t)e * ceff + kr;
                dma16(base + (unsigned)(BM * RB + (wv * IB + i) * 1024), gb[i] + gi * Nout);
            } else {
                const int kk = min(kt * BKT + cb[i] * 8, K - 8);
                dma16(base + (unsigned)(BM * RB + (wv * IB + i) * 1024), gb[i] + kk);
            }
        }
    };

    // operand reads: row r, chunk c sits at r*RB + ((c ^ ((r/RPB)%CPR)) * 16);
    // for this lane's rows the swizzle term is the same for every 16-row tile
    const int ra0 = wm * WTM + (lane & 15), rb0 = wn * WTN + (lane & 15);
    const int xa = (ra0 / RPB) % CPR, xb = (rb0 / RPB) % CPR;
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    // 16-row strips of this wave that hold kept rows: the rest of the tile is
    // padding past used[e], whose products are never stored, so the last
    // row tile of an expert skips their matrix instructions.
    int nvf = (rows - m0 - wm * WTM + 15) / 16;
    nvf = __builtin_amdgcn_readfirstlane(nvf < 0 ? 0 : (nvf > FM ? FM : nvf));
    // Operand fragments of K-step ks (32 wide) of stage st; the next step's
    // fragments are read before the current step's MFMAs are issued.
    constexpr int KS = BKT / 32;
    static_assert(KS % WAVES_K == 0, "MFMA steps split evenly among the K sets");
    constexpr int KSW = KS / WAVES_K;      // MFMA steps of one K set per K-step
    auto read_frags = [&](int st, int ks, bf16x8 (&af)[FM], bf16x8 (&bfr)[FN]) {
        const char *As = smem + st * STAGE;
        const char *Bs = As + BM * RB;
        const int c = ks * 4 + (lane >> 4);
        if constexpr (AT) {
            const int s4 = lane & 15;
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                const int col = wm * WTM + i * 16 + 4 * (s4 & 3);
                v4i16 q[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = ks * 32 + 8 * (lane >> 4) + 4 * h + (s4 >> 2);
                    const int ch = (col >> 3) ^ tr_swizzle(row, CPRTA);
                    q[h] = lds_read_tr16(As + row * RBTA + ch * 16 + (col & 7) * 2);
                }
                const v4i16 lo = q[0], hi = q[1];
                af[i] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        } else {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *reinterpret_cast<const bf16x8 *>(As + (ra0 + i * 16) * RB +
                                                          ((c ^ xa) << 4));
        }
        if constexpr (BT) {
            // rows ks*32 + 8g + 4h + s/4 (g = lane group, h = half), columns
            // 4 (s % 4) .. +3 of this lane's 16-column block j
            const int s4 = lane & 15;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int col = wn * WTN + j * 16 + 4 * (s4 & 3);
                v4i16 q[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int row = ks * 32 + 8 * (lane >> 4) + 4 * h + (s4 >> 2);
                    const int ch = (col >> 3) ^ tr_swizzle(row, CPRT);
                    q[h] = lds_read_tr16(Bs + row * RBT + ch * 16 + (col & 7) * 2);
                }
                const v4i16 lo = q[0], hi = q[1];
                bfr[j] = __builtin_bit_cast(
                    bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
        } else {
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bfr[j] = *reinterpret_cast<const bf16x8 *>(Bs + (rb0 + j * 16) * RB +
                                                           ((c ^ xb) << 4));
        }
    };
    auto mma = [&](const bf16x8 (&af)[FM], const bf16x8 (&bfr)[FN], auto full) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            if (decltype(full)::value || i < nvf) {
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j],
                                                                         0, 0, 0);
            }
        }
    };
    // (the 256x256 weight-gradient tile reads one step's fragments at a time:
    // with both operands transposed, a second set would not fit in registers;
    // so does a tile of 16 waves, four per SIMD, whose 128 registers per lane
    // hold one set)
    constexpr bool kPrefetchFrags =
        !(MODE == 6 && BM * BN >= 256 * 256) && NW < 16 && FM * FN < 40;
    auto compute = [&](int st, auto full) {
        if constexpr (kPrefetchFrags) {
            bf16x8 af[2][FM], bfr[2][FN];
            read_frags(st, wk, af[0], bfr[0]);
#pragma unroll
            for (int u = 0; u < KSW; ++u) {
                if (u + 1 < KSW)
                    read_frags(st, wk + (u + 1) * WAVES_K, af[(u + 1) & 1], bfr[(u + 1) & 1]);
                mma(af[u & 1], bfr[u & 1], full);
            }
        } else {
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int u = 0; u < KSW; ++u) {
                read_frags(st, wk + u * WAVES_K, af, bfr);
                mma(af, bfr, full);
            }
        }
    };
    // zero the chunks of the last K-tile that lie past K (both operands; a
    // K-major right operand: its rows past K)
    auto zero_tail = [&](int kt) {
        char *st = smem + (kt % S) * STAGE;
        if constexpr (!AT) {
            for (int q = tid; q < (BT ? BM : BM + BN) * CPR; q += NTHR) {
                const int row = q / CPR, c = q % CPR;
                if (kt * BKT + c * 8 >= Kr)
                    *reinterpret_cast<u32x4 *>(st + row * RB +
                                               ((c ^ ((row / RPB) % CPR)) << 4)) =
                        u32x4{0u, 0u, 0u, 0u};
            }
        } else {
            for (int q = tid; q < BKT * CPRTA; q += NTHR)
                if (kt * BKT + q / CPRTA >= Kr)
                    *reinterpret_cast<u32x4 *>(st + q * 16) = u32x4{0u, 0u, 0u, 0u};
        }
        if constexpr (BT) {
            for (int q = tid; q < BKT * CPRT; q += NTHR)
                if (kt * BKT + q / CPRT >= Kr)
                    *reinterpret_cast<u32x4 *>(st + BM * RB + q * 16) = u32x4{0u, 0u, 0u, 0u};
        }
    };

    auto mainloop = [&](auto full) {
#pragma unroll
        for (int s = 0; s < S - 1; ++s)
            if (kb + s < ke)
                issue(kb + s);
        if constexpr (TOK && MODE != 0)
            fill_tok();   // (every workgroup has at least one K-step, so a barrier follows)
        for (int kt = kb; kt < ke; ++kt) {
            // step kt must have landed: later steps issued so far may stay in flight
            const int later = min(S - 2, ke - 1 - kt);
            if (later >= S - 2) {
                wait_vm<(S - 2) * G>();
            } else if constexpr (S > 2) {
                if (later == 0) wait_vm<0>();
                else if (later == 1) wait_vm<G>();
                else wait_vm<0>();
            }
            lds_barrier();
            if (kt + S - 1 < ke)
                issue(kt + S - 1);
            if (kt == KT - 1 && (Kr % BKT) != 0) {
                zero_tail(kt);
                lds_barrier();
            }
            compute(kt % S, full);
        }
    };
    if (nvf == FM)
        mainloop(std::true_type{});
    else
        mainloop(std::false_type{});
    lds_barrier();
    if constexpr (WAVES_K > 1) {
        // pairwise: at each level the upper half of the remaining K sets hands
        // its partial tiles (lane-interleaved 16-byte slots) to the lower half,
        // set w adding set w + h, until set 0 holds the sum
        f32x4 *red = reinterpret_cast<f32x4 *>(smem);
        const int wmn = wv % WMN;
#pragma unroll
        for (int h = WAVES_K / 2; h >= 1; h /= 2) {
            if (wk >= h && wk < 2 * h) {
                f32x4 *dst = red + ((wk - h) * WMN + wmn) * (FM * FN * 64) + lane;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        dst[(i * FN + j) * 64] = acc[i][j];
            }
            lds_barrier();
            if (wk < h) {
                const f32x4 *src = red + (wk * WMN + wmn) * (FM * FN * 64) + lane;
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] += src[(i * FN + j) * 64];
            }
            lds_barrier();   // the slots (and then the epilogue scratch) are reused
        }
        if (wk > 0)
            return;
    }

    // epilogue: per wave, one 16-row strip at a time through a private LDS
    // scratch, then 16-byte stores of CPL contiguous columns per lane.
    // acc[i][j][q] is wave row i*16 + 4*(lane/16) + q, column j*16 + lane%16.
    constexpr int SLD = WTN + 4;
    constexpr int CPL = WTN / 4;          // columns per lane on read-back
    float *scr = reinterpret_cast<float *>(smem) + wv * 16 * SLD;
    const int rr = lane >> 2;            // strip row read back by this lane
    const int cg = (lane & 3) * CPL;     // its first column
    // The loop over the strips is instantiated per (bias given, compact rows
    // of Y), so that no strip branches on them (the epilogue's vector
    // instructions are a visible share of a short tile's time).
    auto epilogue = [&](auto has_bias, auto compact_y) {
    constexpr bool HB = decltype(has_bias)::value;
    constexpr bool CY = decltype(compact_y)::value;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                scr[((lane >> 4) * 4 + q) * SLD + j * 16 + (lane & 15)] = acc[i][j][q];
        const int tr = wm * WTM + i * 16 + rr;   // row within the tile
        const int r = m0 + tr;
        const int tc = wn * WTN + cg;            // column within the tile
        const int nb = n0 + tc;
        f32x4 v[CPL / 4];
#pragma unroll
        for (int c = 0; c < CPL / 4; ++c)
            v[c] = *reinterpret_cast<const f32x4 *>(&scr[rr * SLD + cg + 4 * c]);
        if (r < rows) {
            const int64_t srow = (int64_t)e * ceff + r;
            if (piece >= 0) {
                // fp32 partial of a K-range, tile-local [BM][BN] slot
                float *dst = part + ((int64_t)piece * BM + tr) * BN + tc;
#pragma unroll
                for (int c = 0; c < CPL / 4; ++c)
                    if (nb + 4 * c + 4 <= Nout)
                        *reinterpret_cast<f32x4 *>(dst + 4 * c) = v[c];
            } else if (MODE == 0) {
                unsigned short *dst = O16 + srow * Nout + nb;
                const float *bp = HB ? bias + (int64_t)e * Nout + nb : nullptr;
                auto store_h = [&](auto use_gelu) {
#pragma unroll
                    for (int h = 0; h < CPL / 8; ++h) {
                        if (nb + 8 * h + 8 <= Nout) {
                            f32x4 z0 = v[2 * h], z1 = v[2 * h + 1];
                            if constexpr (HB) {
                                z0 += *reinterpret_cast<const f32x4 *>(bp + 8 * h);
                                z1 += *reinterpret_cast<const f32x4 *>(bp + 8 * h + 4);
                            }
                            u32x4 pk;
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const f32x4 &z = c < 2 ? z0 : z1;
                                const float lo = activate<decltype(use_gelu)::value>(z[(c % 2) * 2]);
                                const float hi =
                                    activate<decltype(use_gelu)::value>(z[(c % 2) * 2 + 1]);
                                pk[c] = pack_bf16x2(lo, hi);
                            }
                            *reinterpret_cast<u32x4 *>(dst + 8 * h) = pk;
                            if (Z16) {
                                u32x4 pz;
#pragma unroll
                                for (int c = 0; c < 4; ++c) {
                                    const f32x4 &z = c < 2 ? z0 : z1;
                                    pz[c] = pack_bf16x2(z[(c % 2) * 2], z[(c % 2) * 2 + 1]);
                                }
                                *reinterpret_cast<u32x4 *>(Z16 + srow * Nout + nb + 8 * h) = pz;
                            }
                        }
                    }
                };
                if (act == kActGelu)
                    store_h(std::true_type{});
                else
                    store_h(std::false_type{});
            } else if (MODE == 1 || MODE == 5) {
                // the row of Y at the assignment's position: fp32, or compact
                // (the lanes of a kYGroup-column group hold the same row, so
                // they all take this branch and agree on the group's shift)
                static_assert(!(MODE == 1 || MODE == 5) || kYGroup % CPL == 0,
                              "a lane's columns lie in one group of Y");
                const int64_t arow = (int64_t)s_tok[tr];
                const float *bp = HB ? bias + (int64_t)e * Nout + nb : nullptr;
                float amax = 0.f;
#pragma unroll
                for (int h = 0; h < CPL / 8; ++h) {
                    if (nb + 8 * h + 8 <= Nout) {
                        f32x4 z0 = v[2 * h], z1 = v[2 * h + 1];
                        if constexpr (HB) {
                            z0 += *reinterpret_cast<const f32x4 *>(bp + 8 * h);
                            z1 += *reinterpret_cast<const f32x4 *>(bp + 8 * h + 4);
                        }
                        if constexpr (MODE == 5) {
                            // columns nb + 8h .. +7 share one generator block
                            float m[8];
                            dropout_factors8(dp, arow, (nb + 8 * h) / 8, m);
                            z0 *= f32x4{m[0], m[1], m[2], m[3]};
                            z1 *= f32x4{m[4], m[5], m[6], m[7]};
                        }
                        v[2 * h] = z0;
                        v[2 * h + 1] = z1;
                        if constexpr (CY) {
                            // (max of magnitudes, NaN ignored; an infinity
                            // is taken out below, on the rare path)
#pragma unroll
                            for (int q = 0; q < 4; ++q)
                                amax = fmaxf(fmaxf(amax, fabsf(z0[q])), fabsf(z1[q]));
                        }
                    }
                }
                if constexpr (CY) {
                    amax = quad_group_max<kYGroup / CPL>(amax);
                    if (amax == __builtin_inff()) {
                        // the group holds an infinity: its largest finite
                        // magnitude instead (the whole group takes this path)
                        amax = 0.f;
#pragma unroll
                        for (int h = 0; h < CPL / 8; ++h)
                            if (nb + 8 * h + 8 <= Nout)
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    amax = finite_max(finite_max(amax, v[2 * h][q]),
                                                      v[2 * h + 1][q]);
                        amax = quad_group_max<kYGroup / CPL>(amax);
                    }
                    const int sh = yshift_of(amax);
                    const float sc = pow2f(sh);
                    unsigned short *dst = O16 + arow * Nout + nb;
#pragma unroll
                    for (int h = 0; h < CPL / 8; ++h) {
                        if (nb + 8 * h + 8 <= Nout) {
                            const f32x4 z0 = v[2 * h] * sc, z1 = v[2 * h + 1] * sc;
                            *reinterpret_cast<u32x4 *>(dst + 8 * h) =
                                u32x4{pack_f16x2(z0[0], z0[1]), pack_f16x2(z0[2], z0[3]),
                                      pack_f16x2(z1[0], z1[1]), pack_f16x2(z1[2], z1[3])};
                        }
                    }
                    if (nb % kYGroup == 0 && nb < Nout)   // (groups past Nout: none)
                        ysh[yshift_index((int)arow, k, (Nout + kYGroup - 1) / kYGroup,
                                         nb / kYGroup)] = (signed char)sh;
                } else {
                    float *dst = O32 + arow * Nout + nb;
#pragma unroll
                    for (int h = 0; h < CPL / 8; ++h) {
                        if (nb + 8 * h + 8 <= Nout) {
                            *reinterpret_cast<f32x4 *>(dst + 8 * h) = v[2 * h];
                            *reinterpret_cast<f32x4 *>(dst + 8 * h + 4) = v[2 * h + 1];
                        }
                    }
                }
            } else if (MODE == 3) {
                // dZ = dH act'(z), bf16 like H: ReLU passes dH where H > 0;
                // GELU scales it by gelu'(z) of the stored pre-activation
                unsigned short *dst = O16 + srow * Nout + nb;
                const unsigned short *hm = mask + srow * Nout + nb;
                auto store_dz = [&](auto use_gelu) {
#pragma unroll
                    for (int h = 0; h < CPL / 8; ++h) {
                        if (nb + 8 * h + 8 <= Nout) {
                            const u32x4 hb = *reinterpret_cast<const u32x4 *>(hm + 8 * h);
                            u32x4 pk;
#pragma unroll
                            for (int c = 0; c < 4; ++c) {
                                const f32x4 &z = c < 2 ? v[2 * h] : v[2 * h + 1];
                                const unsigned hl = hb[c] & 0xffffu, hh = hb[c] >> 16;
                                float lo, hi;
                                if constexpr (decltype(use_gelu)::value) {
                                    lo = z[(c % 2) * 2] * gelu_grad(bf16_bits_to_f32(hl));
                                    hi = z[(c % 2) * 2 + 1] * gelu_grad(bf16_bits_to_f32(hh));
                                } else {
                                    // a bf16 value > 0: sign clear and not zero
                                    lo = (hl - 1u) < 0x7fffu ? z[(c % 2) * 2] : 0.f;
                                    hi = (hh - 1u) < 0x7fffu ? z[(c % 2) * 2 + 1] : 0.f;
                                }
                                pk[c] = pack_bf16x2(lo, hi);
                            }
                            *reinterpret_cast<u32x4 *>(dst + 8 * h) = pk;
                        }
                    }
                };
                if (act == kActGelu)
                    store_dz(std::true_type{});
                else
                    store_dz(std::false_type{});
            } else {
                const int64_t orow = MODE == 4 ? (int64_t)s_tok[tr] : (int64_t)r;
                float *dst = O32 + orow * Nout + nb;
#pragma unroll
                for (int c = 0; c < CPL / 4; ++c)
                    if (nb + 4 * c + 4 <= Nout)
                        *reinterpret_cast<f32x4 *>(dst + 4 * c) = v[c];
            }
        }
    }
    };
    if constexpr (MODE == 0) {
        if (bias)
            epilogue(std::true_type{}, std::false_type{});
        else
            epilogue(std::false_type{}, std::false_type{});
    } else if constexpr (MODE == 1 || MODE == 5) {
        if (bias) {
            if (ysh)
                epilogue(std::true_type{}, std::true_type{});
            else
                epilogue(std::true_type{}, std::false_type{});
        } else {
            if (ysh)
                epilogue(std::false_type{}, std::true_type{});
            else
                epilogue(std::false_type{}, std::false_type{});
        }
    } else {
        epilogue(std::false_type{}, std::false_type{});
    }
    if constexpr (PERSIST)
        __syncthreads();   // the next item reuses the LDS (operand stages, epilogue scratch, s_tok)
    }   // items of this workgroup
}

// Sum of the K-range partials of the cut tiles, in K order, then the same
// epilogue as a whole tile (MODE 0: bias, activation, bf16 H; MODE 1: bias,
// dropout, the row of Y, fp32 or compact when ysh is given).
// One workgroup per 16-row strip of a cut tile; 4 columns per thread.
template <int BM, int BN, int BKT, int MODE>
__global__ __launch_bounds__(256) void split_fixup_kernel(
    int K, int Nout, int E, int ceff, const int32_t *__restrict__ used,
    const int32_t *__restrict__ slot_token, const int32_t *__restrict__ mt_off,
    const float *__restrict__ part, int P, unsigned short *__restrict__ O16,
    float *__restrict__ O32, int act, const float *__restrict__ bias, Dropout dp,
    unsigned short *__restrict__ Z16, signed char *__restrict__ ysh, int k) {
    constexpr int STRIPS = BM / 16;
    static_assert((BN / 4) % (kYGroup / 4) == 0, "a group of Y lies in one row of threads");
    __shared__ int s_mt[kMaxExperts + 1];
    __shared__ int s_pp[kMaxExperts + 1];
    __shared__ uint64_t s_msk[kMaxExperts / 64];
    if (mt_off) {
        for (int i = threadIdx.x; i <= E; i += 256)
            s_mt[i] = mt_off[i];
        __syncthreads();
    } else {
        row_tile_prefix(used, E, BM, s_mt, reinterpret_cast<int *>(s_msk));
    }
    const int NT = (Nout + BN - 1) / BN;
    const int KT = (K + BKT - 1) / BKT;
    const SplitPlan sp = split_plan(s_mt[E] * NT, KT, P);
    const int t = blockIdx.x / STRIPS, strip = blockIdx.x % STRIPS;
    if (sp.nsplit < 2 || t >= sp.tail)   // (the same for the whole workgroup)
        return;
    // (the same order as the product kernel: no light-last pass for 320 rows)
    const bool ll = BM == 320 ? false : light_last(used, s_mt, E, NT, BM, P, 256, s_pp, s_msk);
    int e, m0, n0;
    decode_tile(sp.Tdp + t, s_mt, ll ? s_pp : nullptr, E, NT, BM, BN, e, m0, n0);
    const int rows = used[e];
    static_assert((16 * (BN / 4)) % 256 == 0, "every thread takes every trip");
    for (int i = threadIdx.x; i < 16 * (BN / 4); i += 256) {
        const int rr = i / (BN / 4), c4 = i % (BN / 4);
        const int tr = strip * 16 + rr;
        const int r = m0 + tr;
        const int n = n0 + 4 * c4;
        const bool ok = r < rows && n + 4 <= Nout;
        if (MODE == 1 && ysh) {
            // compact row of Y: the kYGroup / 4 threads of a group (adjacent
            // lanes of one row) agree on its shift; all of them take part
            f32x4 v = {0.f, 0.f, 0.f, 0.f};
            int64_t orow = 0;
            if (ok) {
                const float *src = part + ((int64_t)t * sp.nsplit * BM + tr) * BN + 4 * c4;
                v = *reinterpret_cast<const f32x4 *>(src);
                for (int s = 1; s < sp.nsplit; ++s)
                    v += *reinterpret_cast<const f32x4 *>(src + (int64_t)s * BM * BN);
                if (bias)
                    v += *reinterpret_cast<const f32x4 *>(bias + (int64_t)e * Nout + n);
                orow = (int64_t)slot_token[(int64_t)e * ceff + r];
                if (dp.on) {
                    float m[8];
                    dropout_factors8(dp, orow, n / 8, m);
                    const int o = n % 8;
                    v *= f32x4{m[o], m[o + 1], m[o + 2], m[o + 3]};
                }
            }
            float amax = finite_max(finite_max(finite_max(finite_max(0.f, v[0]), v[1]), v[2]), v[3]);
#pragma unroll
            for (int o = 1; o < kYGroup / 4; o <<= 1)
                amax = fmaxf(amax, __shfl_xor(amax, o));
            if (ok) {
                const int sh = yshift_of(amax);
                const f32x4 z = v * pow2f(sh);
                *reinterpret_cast<u32x2 *>(O16 + orow * Nout + n) =
                    u32x2{pack_f16x2(z[0], z[1]), pack_f16x2(z[2], z[3])};
                if (n % kYGroup == 0)
                    ysh[yshift_index((int)orow, k, (Nout + kYGroup - 1) / kYGroup, n / kYGroup)] =
                        (signed char)sh;
            }
            continue;
        }
        if (!ok)
            continue;
        const float *src = part + ((int64_t)t * sp.nsplit * BM + tr) * BN + 4 * c4;
        f32x4 v = *reinterpret_cast<const f32x4 *>(src);
        for (int s = 1; s < sp.nsplit; ++s)
            v += *reinterpret_cast<const f32x4 *>(src + (int64_t)s * BM * BN);
        const int64_t srow = (int64_t)e * ceff + r;
        if (bias)
            v += *reinterpret_cast<const f32x4 *>(bias + (int64_t)e * Nout + n);
        int64_t orow = (int64_t)slot_token[srow];   // MODE 1: the row of Y
        if (MODE == 1 && dp.on) {
            float m[8];
            dropout_factors8(dp, orow, n / 8, m);
            const int o = n % 8;                      // 0 or 4
            v *= f32x4{m[o], m[o + 1], m[o + 2], m[o + 3]};
        }
        if (MODE == 0) {
            orow = srow;                              // the row of H
            if (Z16) {                                // the pre-activations too
                u32x2 pz;
                pz[0] = pack_bf16x2(v[0], v[1]);
                pz[1] = pack_bf16x2(v[2], v[3]);
                *reinterpret_cast<u32x2 *>(Z16 + orow * Nout + n) = pz;
            }
            if (act == kActGelu)
                v = f32x4{gelu(v[0]), gelu(v[1]), gelu(v[2]), gelu(v[3])};
            else
                v = f32x4{fmaxf(v[0], 0.f), fmaxf(v[1], 0.f), fmaxf(v[2], 0.f), fmaxf(v[3], 0.f)};
        }
        if (MODE == 1) {
            *reinterpret_cast<f32x4 *>(O32 + orow * Nout + n) = v;   // fp32 row of Y
            continue;
        }
        u32x2 pk;
        pk[0] = pack_bf16x2(v[0], v[1]);
        pk[1] = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<u32x2 *>(O16 + orow * Nout + n) = pk;
    }
}

// fp32 path (correctness-first, any shape): 64 x 64 tiles, K-step 16,
// 256 threads with 4 x 4 outputs each, fp32 FMA.
template <int MODE>
__global__ __launch_bounds__(256) void experts_f32_kernel(
    const float *__restrict__ A_src, const float *__restrict__ W, int K, int Nout, int k,
    int ceff, const int32_t *__restrict__ used, const int32_t *__restrict__ slot_token,
    float *__restrict__ H_out, float *__restrict__ Y_out, int act,
    const float *__restrict__ bias, Dropout dp) {
    constexpr int TM = 64, TN = 64, TK = 16;
    __shared__ float As[TK][TM + 4];
    __shared__ float Bs[TK][TN + 4];
    const int e = blockIdx.z;
    const int m0 = blockIdx.y * TM;
    const int n0 = blockIdx.x * TN;
    const int rows = used[e];
    if (m0 >= rows)
        return;
    const int tid = threadIdx.x;
    const int tr = tid / 16, tc = tid % 16;
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += TK) {
        for (int i = tid; i < TM * TK; i += 256) {
            const int r = i / TK, kk = i % TK;
            const int gr = m0 + r, gk = k0 + kk;
            float v = 0.f;
            if (gr < rows && gk < K) {
                const int64_t srow = (int64_t)e * ceff + gr;
                const int64_t src = MODE == 0 ? (int64_t)(slot_token[srow] / k) : srow;
                v = A_src[src * K + gk];
            }
            As[kk][r] = v;
            const int gn = n0 + r;
            float wv = 0.f;
            if (gn < Nout && gk < K)
                wv = W[((int64_t)e * Nout + gn) * K + gk];
            Bs[kk][r] = wv;
        }
        __syncthreads();
        for (int kk = 0; kk < TK; ++kk) {
            float a[4], bv[4];
            for (int i = 0; i < 4; ++i) {
                a[i] = As[kk][tr * 4 + i];
                bv[i] = Bs[kk][tc * 4 + i];
            }
            for (int i = 0; i < 4; ++i)
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = fmaf(a[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
    for (int i = 0; i < 4; ++i) {
        const int r = m0 + tr * 4 + i;
        if (r >= rows)
            continue;
        const int64_t srow = (int64_t)e * ceff + r;
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tc * 4 + j;
            if (n >= Nout)
                continue;
            const float z = bias ? acc[i][j] + bias[(int64_t)e * Nout + n] : acc[i][j];
            if (MODE == 0) {
                H_out[srow * Nout + n] = act == kActGelu ? gelu(z) : fmaxf(z, 0.f);
            } else {
                const int64_t arow = (int64_t)slot_token[srow];
                float f = 1.f;
                if (dp.on) {
                    float m[8];
                    dropout_factors8(dp, arow, n / 8, m);
                    f = m[n % 8];
                }
                Y_out[arow * Nout + n] = z * f;
            }
        }
    }
}

}  // namespace

namespace {

// Tile shapes (rows_per_expert = expected kept rows per expert):
//  - 256x256, one workgroup per CU: experts with >= 256 rows when that still
//    gives a full grid or the product is wide (16 waves of 64x64 for the
//    forward products, 8 of 128x64 for the backward's K-major ones);
//  - 128x128 in two K sets (16 waves: 2 x 4 of 64x32 per set, K-step 128,
//    one workgroup per CU): when 128x128 tiles give between 192 and 384
//    tiles, i.e. about one per CU (four waves per SIMD to hide latency);
//  - 128x64, 4 waves of 64x32: when 128x128 tiles would leave more CUs idle
//    (fewer than 192 tiles), trading operand reuse for parallelism;
//  - 128x128, 4 waves of 64x64, two workgroups per CU: otherwise.
// Products whose right operand is read K-major (modes 3, 4) take 128x64
// where the K-set tile would be picked.
enum class Tile { k128, k128x64, k256, k128k2, k320 };

constexpr int kBK = 64;    // K-step of the one-set tile shapes
constexpr int kBK2 = 128;  // K-step of the K-set tile: two 32-wide MFMA steps per set

Tile pick_tile(int64_t rows_per_expert, int64_t Nout, int E) {
    if (rows_per_expert >= 232 && rows_per_expert <= 288)
        return Tile::k320;
    const int64_t t256 = (int64_t)E * ((rows_per_expert + 255) / 256) * ((Nout + 255) / 256);
    if (rows_per_expert >= 256 && (t256 >= 256 || Nout >= 2048))
        return Tile::k256;
    const int64_t t128 = (int64_t)E * ((rows_per_expert + 127) / 128) * ((Nout + 127) / 128);
    if (t128 < 192)
        return Tile::k128x64;
    if (t128 < 384)
        return Tile::k128k2;
    return Tile::k128;
}

// Workgroups of `kernel` that run at once on the current device (-1 if
// unknown), queried on every launch (the library keeps no state between calls).
template <typename Kern>
int resident_blocks(Kern kernel, int threads) {
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
        cus * per_cu <= 0)
        return -1;
    return cus * per_cu;
}

// One bf16 grouped product on tile shape BM x BN, plus the fix-up of the
// split last round when the scratch `part` can hold it.
template <int BM, int BN, int WM, int WN, int WK, int BKT, int MODE, int S = 2>
hipError_t launch_tiles(const unsigned short *A, const unsigned short *W, int64_t K, int64_t Nout,
                        int E, int k, int64_t ceff, const int32_t *used,
                        const int32_t *slot_token, const int32_t *mt, unsigned short *O16,
                        float *part, size_t part_bytes, int act, const float *bias,
                        hipStream_t s, const unsigned short *mask = nullptr,
                        float *O32 = nullptr, unsigned short *Z16 = nullptr,
                        Dropout dp = Dropout{}, signed char *ysh = nullptr) {
    auto kern = expert_gemm_kernel<BM, BN, WM, WN, WK, BKT, S, MODE>;
    constexpr int NTHR = WM * WN * WK * 64;
    int P = resident_blocks(kern, NTHR);
    if (P < 0) {
        (void)hipGetLastError();   // a failed query leaves no error behind: plan without it
        P = 0;
    }
    const int64_t slot = (int64_t)BM * BN * sizeof(float);
    const int64_t KT = (K + BKT - 1) / BKT;
    const int64_t tmax = (int64_t)E * ((ceff + BM - 1) / BM) * ((Nout + BN - 1) / BN);
    // a split needs the scratch, at least two ranges of kSplitMinSteps, at
    // least one full round of tiles and (by the 15% rule of split_plan)
    // fewer than six
    const bool split = (MODE == 0 || MODE == 1 || MODE == 5) && part && P > 0 &&
                       (int64_t)P * slot <= (int64_t)part_bytes &&
                       KT >= 2 * kSplitMinSteps &&
                       tmax >= P && tmax < 6 * (int64_t)P;
    // whole tiles take two XCD-rounded segments (one more group of kXcds)
    int64_t grid = (tmax + kXcds - 1) / kXcds * kXcds + kXcds +
                   (split ? (int64_t)(P + kXcds - 1) / kXcds * kXcds : 0);
    // the 320-row tiles' persistent launch: one workgroup per resident slot,
    // a multiple of the XCD count (the kernel walks the items)
    if (BM == 320 && (MODE == 0 || MODE == 1 || MODE == 5) && P >= kXcds)
        grid = std::min<int64_t>(grid, P / kXcds * kXcds);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(NTHR), 0, s, A, W, (int)K, (int)Nout, E,
                       k, (int)ceff, used, slot_token, mt, O16, O32, split ? part : nullptr,
                       P, act, bias, mask, Z16, dp, (int64_t)0, (int64_t)0, (int64_t)0, ysh);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess || !split)
        return err;
    hipLaunchKernelGGL((split_fixup_kernel<BM, BN, BKT, MODE == 0 ? 0 : 1>),
                       dim3((unsigned)(P * (BM / 16))),
                       dim3(256), 0, s, (int)K, (int)Nout, E, (int)ceff, used, slot_token, mt,
                       (const float *)part, P, O16, O32, act, bias, dp, Z16, ysh, k);
    return hipGetLastError();
}

// Template arguments of the kernel a product of this mode runs on tile shape
// t: BM, BN, waves along rows, columns and K, K-step.
template <int BM_, int BN_, int WM_, int WN_, int WK_, int BKT_, int S_ = 2>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, WK = WK_, BKT = BKT_, S = S_;
};

// Calls f(TileCfg<...>{}, tiles) with the instantiation mode MODE runs for
// tile shape t and the dispatch plan's schedule table it uses (row tiles of
// 128 or of 256): the one place that maps a tile shape to a kernel, shared by
// the launch and by the kernel-name query.
template <int MODE, typename F>
auto with_tile(Tile t, const int32_t *tiles, int E, F f) {
    if (t == Tile::k320) {
        // forward products: 8 waves of 160x64 (two per SIMD); the schedule
        // table of 320-row tiles is computed by the kernel itself
        if constexpr (MODE == 0 || MODE == 1 || MODE == 5)
            return f(TileCfg<320, 256, 2, 4, 1, kBK>{}, (const int32_t *)nullptr);
        t = Tile::k256;
    }
    if (t == Tile::k128k2) {
        if constexpr (MODE == 0 || MODE == 1 || MODE == 5)
            return f(TileCfg<128, 128, 2, 4, 2, kBK2>{}, tiles);
        t = Tile::k128x64;   // K-major right operands: no K sets
    }
    if (t == Tile::k256) {
        // forward products: 16 waves of 64x64 (four per SIMD, more latency
        // hidden than the 8 waves of 128x64 save in LDS reads); the backward's
        // K-major products keep 8 waves (16 would spill there)
        if constexpr (MODE == 0 || MODE == 1 || MODE == 5)
            return f(TileCfg<256, 256, 4, 4, 1, kBK>{}, tiles + E + 1);
        else
            return f(TileCfg<256, 256, 2, 4, 1, kBK>{}, tiles + E + 1);
    }
    if (t == Tile::k128x64)
        return f(TileCfg<128, 64, 2, 2, 1, kBK>{}, tiles);
    return f(TileCfg<128, 128, 2, 2, 1, kBK>{}, tiles);
}

template <int MODE>
hipError_t launch_gemm(Tile t, const unsigned short *A, const unsigned short *W, int64_t K,
                       int64_t Nout, int E, int k, int64_t ceff, const int32_t *used,
                       const int32_t *slot_token, const int32_t *tiles, unsigned short *O16,
                       void *part, size_t part_bytes, int act, const float *bias,
                       hipStream_t s, const unsigned short *mask = nullptr,
                       float *O32 = nullptr, unsigned short *Z16 = nullptr,
                       Dropout dp = Dropout{}, signed char *ysh = nullptr) {
    float *pf = static_cast<float *>(part);
    return with_tile<MODE>(t, tiles, E, [&](auto c, const int32_t *tt) {
        using C = decltype(c);
        return launch_tiles<C::BM, C::BN, C::WM, C::WN, C::WK, C::BKT, MODE, C::S>(
            A, W, K, Nout, E, k, ceff, used, slot_token, tt, O16, pf, part_bytes, act, bias, s,
            mask, O32, Z16, dp, ysh);
    });
}

}  // namespace

size_t split_workspace_bytes() { return kSplitWorkspaceBytes; }

bool router_terms_interleaved(int64_t d) { return d % 64 == 0; }

int router_score_splits(int64_t N, int64_t d, int64_t Ep) {
    // about one round of 256x256 tiles (one workgroup per CU), ranges of at
    // least 8 K-steps
    const int64_t tiles = ((N + 255) / 256) * ((Ep + 255) / 256);
    const int64_t KT = (3 * d + kBK - 1) / kBK;
    int64_t ns = std::max<int64_t>(256 / std::max<int64_t>(tiles, 1), 1);
    ns = std::min<int64_t>(ns, std::max<int64_t>(KT / 8, 1));
    return (int)ns;
}

hipError_t launch_router_scores_bf16(const void *x, const void *wsp, int64_t N, int64_t d,
                                     int64_t Ep, float *P, hipStream_t s) {
    if (N == 0)
        return hipSuccess;
    const int ns = router_score_splits(N, d, Ep);
    const int64_t tiles = ((N + 255) / 256) * ((Ep + 255) / 256);
    const int64_t grid = (tiles + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((expert_gemm_kernel<256, 256, 4, 4, 1, kBK, 2, 7>),
                       dim3((unsigned)grid, (unsigned)ns), dim3(1024), 0, s,
                       static_cast<const unsigned short *>(x),
                       static_cast<const unsigned short *>(wsp), (int)(3 * d), (int)Ep, 1, 1,
                       (int)N, (const int32_t *)nullptr, (const int32_t *)nullptr,
                       (const int32_t *)nullptr, (unsigned short *)nullptr, P, (float *)nullptr,
                       0, kActRelu, (const float *)nullptr, (const unsigned short *)nullptr,
                       (unsigned short *)nullptr, Dropout{}, d,
                       (int64_t)router_terms_interleaved(d), N * Ep, (signed char *)nullptr);
    return hipGetLastError();
}

hipError_t launch_expert_up(bool bf16, const void *x, const void *w_up, int64_t d,
                            int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                            const int32_t *slot_token, const int32_t *tiles, void *H,
                            int64_t rows_per_expert, void *part, size_t part_bytes, int act,
                            const float *b_up, hipStream_t s, void *Z) {
    if (ceff == 0)
        return hipSuccess;
    if (bf16)
        return launch_gemm<0>(pick_tile(rows_per_expert, d_ff, E),
                              static_cast<const unsigned short *>(x),
                              static_cast<const unsigned short *>(w_up), d, d_ff, E, k, ceff,
                              used, slot_token, tiles, static_cast<unsigned short *>(H),
                              part, part_bytes, act, b_up, s, nullptr, nullptr,
                              static_cast<unsigned short *>(Z));
    if (Z)
        return hipErrorInvalidValue;   // pre-activations are kept for bf16 layers only
    hipLaunchKernelGGL(experts_f32_kernel<0>,
                       dim3((unsigned)((d_ff + 63) / 64), (unsigned)((ceff + 63) / 64), E),
                       dim3(256), 0, s, static_cast<const float *>(x),
                       static_cast<const float *>(w_up), (int)d, (int)d_ff, k, (int)ceff, used,
                       slot_token, static_cast<float *>(H), (float *)nullptr, act, b_up,
                       Dropout{});
    return hipGetLastError();
}

hipError_t launch_expert_down(bool bf16, const void *H, const void *w_down, int64_t d,
                              int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                              const int32_t *slot_token, const int32_t *tiles, void *Y,
                              int64_t rows_per_expert, void *part, size_t part_bytes,
                              const float *b_down, hipStream_t s, Dropout dp,
                              signed char *ysh) {
    if (ceff == 0)
        return hipSuccess;
    if (ysh && !bf16)
        return hipErrorInvalidValue;   // compact rows are for bf16 layers only
    // compact rows: fp16 values through O16, fp32 rows through O32
    unsigned short *y16 = ysh ? static_cast<unsigned short *>(Y) : nullptr;
    float *y32 = ysh ? nullptr : static_cast<float *>(Y);
    if (bf16 && dp.on)
        return launch_gemm<5>(pick_tile(rows_per_expert, d, E),
                              static_cast<const unsigned short *>(H),
                              static_cast<const unsigned short *>(w_down), d_ff, d, E, k, ceff,
                              used, slot_token, tiles, y16, part, part_bytes, kActRelu,
                              b_down, s, nullptr, y32, nullptr, dp, ysh);
    if (bf16)
        return launch_gemm<1>(pick_tile(rows_per_expert, d, E),
                              static_cast<const unsigned short *>(H),
                              static_cast<const unsigned short *>(w_down), d_ff, d, E, k, ceff,
                              used, slot_token, tiles, y16, part, part_bytes, kActRelu,
                              b_down, s, nullptr, y32, nullptr, Dropout{}, ysh);
    hipLaunchKernelGGL(experts_f32_kernel<1>,
                       dim3((unsigned)((d + 63) / 64), (unsigned)((ceff + 63) / 64), E),
                       dim3(256), 0, s, static_cast<const float *>(H),
                       static_cast<const float *>(w_down), (int)d_ff, (int)d, k, (int)ceff, used,
                       slot_token, (float *)nullptr, static_cast<float *>(Y), kActRelu, b_down,
                       dp);
    return hipGetLastError();
}

int expert_kernel_name(bool bf16, int product, int64_t d, int64_t d_ff, int E,
                       int64_t rows_per_expert, bool dropout, char *buf, size_t len) {
    if (!bf16)
        return snprintf(buf, len, "experts_f32_kernel<%d>", product);
    const int64_t nout = product == 0 ? d_ff : d;
    const int mode = product == 0 ? 0 : (dropout ? 5 : 1);
    auto name = [&](auto c, const int32_t *) {
        using C = decltype(c);
        return snprintf(buf, len, "expert_gemm_kernel<%d, %d, %d, %d, %d, %d, 2, %d>", C::BM,
                        C::BN, C::WM, C::WN, C::WK, C::BKT, mode);
    };
    const Tile t = pick_tile(rows_per_expert, nout, E);
    if (mode == 0)
        return with_tile<0>(t, nullptr, E, name);
    if (mode == 5)
        return with_tile<5>(t, nullptr, E, name);
    return with_tile<1>(t, nullptr, E, name);
}

// ---- backward-pass products (bf16 operands, fp32 accumulation) ----------

hipError_t launch_expert_dz(const void *dY, const void *w_down, const void *act_in, int act,
                            int64_t d, int64_t d_ff, int E, int k, int64_t ceff,
                            const int32_t *used, const int32_t *slot_token, const int32_t *tiles,
                            void *dZ, int64_t rows_per_expert, hipStream_t s) {
    if (ceff == 0)
        return hipSuccess;
    return launch_gemm<3>(pick_tile(rows_per_expert, d_ff, E),
                          static_cast<const unsigned short *>(dY),
                          static_cast<const unsigned short *>(w_down), d, d_ff, E, k, ceff,
                          used, slot_token, tiles, static_cast<unsigned short *>(dZ), nullptr, 0,
                          act, nullptr, s, static_cast<const unsigned short *>(act_in));
}

hipError_t launch_expert_rows_f32(const void *A, const void *w, int64_t K, int64_t Nout, int E,
                                  int k, int64_t ceff, const int32_t *used,
                                  const int32_t *slot_token, const int32_t *tiles, float *out,
                                  int64_t rows_per_expert, hipStream_t s) {
    if (ceff == 0)
        return hipSuccess;
    return launch_gemm<4>(pick_tile(rows_per_expert, Nout, E),
                          static_cast<const unsigned short *>(A),
                          static_cast<const unsigned short *>(w), K, Nout, E, k, ceff, used,
                          slot_token, tiles, nullptr, nullptr, 0, kActRelu, nullptr, s, nullptr,
                          out);
}

hipError_t launch_weight_grad(const void *A, int64_t M, const void *B, int64_t N, int E,
                              int64_t ceff, const int32_t *used, const int32_t *slot_token,
                              int kdiv, int gathered, float *out, hipStream_t s) {
    if (M == 0 || N == 0 || E == 0)
        return hipSuccess;
    if (ceff > kGradMaxRows || M % 8 != 0 || N % 8 != 0 || kdiv < 1)
        return hipErrorInvalidValue;
    const auto *a = static_cast<const unsigned short *>(A);
    const auto *w = static_cast<const unsigned short *>(B);
    // 256x256 tiles for large products (at least four rounds of them), else
    // 128x128
    const int64_t t256 = ((M + 255) / 256) * ((N + 255) / 256);
    if (M >= 512 && N >= 512 && t256 * E >= 1024) {
        const int64_t grid = (t256 + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL((expert_gemm_kernel<256, 256, 2, 4, 1, kBK, 2, 6>),
                           dim3((unsigned)grid, (unsigned)E), dim3(512), 0, s, a, w, 0, (int)N,
                           E, kdiv, (int)ceff, used, slot_token, (const int32_t *)nullptr,
                           (unsigned short *)nullptr, out, (float *)nullptr, 0, gathered,
                           (const float *)nullptr, (const unsigned short *)nullptr,
                           (unsigned short *)nullptr, Dropout{}, M, (int64_t)0, M * N,
                           (signed char *)nullptr);
        return hipGetLastError();
    }
    const int64_t grid = (((M + 127) / 128) * ((N + 127) / 128) + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((expert_gemm_kernel<128, 128, 2, 2, 1, kBK, 2, 6>),
                       dim3((unsigned)grid, (unsigned)E), dim3(256), 0, s, a, w, 0, (int)N, E,
                       kdiv, (int)ceff, used, slot_token, (const int32_t *)nullptr,
                       (unsigned short *)nullptr, out, (float *)nullptr, 0, gathered,
                       (const float *)nullptr, (const unsigned short *)nullptr,
                       (unsigned short *)nullptr, Dropout{}, M, (int64_t)0, M * N,
                           (signed char *)nullptr);
    return hipGetLastError();
}

hipError_t launch_batched_gemm_bf16(const void *A, const void *W, int64_t M, int64_t K,
                                    int64_t Nout, int batch, int64_t sa, int64_t sb, int64_t sc,
                                    float *C, hipStream_t s) {
    if (M == 0 || batch == 0)
        return hipSuccess;
    const auto *a = static_cast<const unsigned short *>(A);
    const auto *w = static_cast<const unsigned short *>(W);
    // 256x256 tiles for large products (at least four rounds of them), else
    // 128x128
    const int64_t t256 = ((M + 255) / 256) * ((Nout + 255) / 256);
    if (M >= 512 && Nout >= 512 && K >= 256 && t256 * batch >= 1024) {
        const int64_t grid = (t256 + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL((expert_gemm_kernel<256, 256, 2, 4, 1, kBK, 2, 2>),
                           dim3((unsigned)grid, (unsigned)batch), dim3(512), 0, s, a, w, (int)K,
                           (int)Nout, 1, 1, (int)M, (const int32_t *)nullptr,
                           (const int32_t *)nullptr, (const int32_t *)nullptr,
                           (unsigned short *)nullptr, C, (float *)nullptr, 0, kActRelu,
                           (const float *)nullptr, (const unsigned short *)nullptr,
                           (unsigned short *)nullptr, Dropout{}, sa, sb, sc, (signed char *)nullptr);
        return hipGetLastError();
    }
    const int64_t grid = (((M + 127) / 128) * ((Nout + 127) / 128) + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL((expert_gemm_kernel<128, 128, 2, 2, 1, kBK, 2, 2>),
                       dim3((unsigned)grid, (unsigned)batch), dim3(256), 0, s, a, w, (int)K,
                       (int)Nout, 1, 1, (int)M, (const int32_t *)nullptr,
                       (const int32_t *)nullptr, (const int32_t *)nullptr,
                       (unsigned short *)nullptr, C, (float *)nullptr, 0, kActRelu,
                       (const float *)nullptr, (const unsigned short *)nullptr,
                           (unsigned short *)nullptr, Dropout{}, sa, sb, sc, (signed char *)nullptr);
    return hipGetLastError();
}

}  // namespace moe
