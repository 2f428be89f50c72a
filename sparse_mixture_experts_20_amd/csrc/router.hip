// Router: scores s = W_g x + noise in fp32, top-k in descending order (equal
// scores: lower expert id first), softmax over the k kept scores.
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 2 (s_raw = W_g x), STEP 4 (s = s_raw + eps), STEP 5 (KeepTopK with a
// -inf mask), STEP 6 (softmax: masked experts get exactly 0, so only the k
// kept scores enter the sum); nanoMoE slides 11-13 (router in full precision,
// top-k then masked softmax).
//
// bf16 activations: the score product is a skinny GEMM [N, d] x [d, E]. It
// runs on the matrix cores without losing fp32 accuracy: every fp32 router
// weight w is split exactly into three bf16 terms w = hi + mid + lo (each
// residual is exact in fp32 and the last one fits in bf16's 8-bit
// significand), and a bf16 activation times a bf16 term is exact in the fp32
// accumulator. Three bf16 MFMAs per K-step therefore give an fp32-accumulated
// dot product of the exact inputs, at a fraction of the cost of fp32 MFMA.
// Up to 32 experts one fused kernel splits the weights in registers,
// computes the scores of 16 tokens and ranks them. With more experts the
// split is done once per call into the workspace (a [Ep][3 d] bf16 matrix
// whose row pi(e) holds hi, mid and lo of expert e one after the other;
// Ep = E rounded up to 16, or to 128 or 256 past 64 experts, padding rows
// zero;
// pi(e) = (e mod 64) Q + e / 64 with Q = Ep / 64 puts the Q experts a
// ranking lane holds, e, e + 64, ..., in adjacent score columns), the score
// product runs on the
// expert-product kernel with the token row read once per term, so that the
// three terms of an expert accumulate into one fp32 score, its K dimension
// cut into ranges that write partial scores, and a ranking kernel adds the
// ranges in order and finishes.
#include "common.hpp"

#include <float.h>
#include <limits.h>

namespace moe {
namespace {

constexpr int kTokTile = 16;   // tokens per block (one MFMA M-tile)
constexpr int kRankWaves = 4;  // waves that rank the block's tokens

// Exact three-term split of two fp32 weights, w = hi + mid + lo, by
// truncation: hi keeps the upper 16 bits of w (sign, exponent and the top 7
// stored significand bits), mid the upper 16 bits of the residual w - hi
// (exact, at most 16 significant bits), and lo = (w - hi) - mid, which is
// exact and has at most 8 significant bits, so it is a bf16 value too. A
// term's bf16 encoding is its upper 16 bits; the pair is packed with a in the
// low half, b in the high half (bf16 elements 2j and 2j+1 of a vector).
__device__ __forceinline__ void split3x2(float a, float b, unsigned &hi, unsigned &mid,
                                         unsigned &lo) {
    const unsigned ha = __float_as_uint(a) & 0xffff0000u, hb = __float_as_uint(b) & 0xffff0000u;
    const float ra = a - __uint_as_float(ha), rb = b - __uint_as_float(hb);
    const unsigned ma = __float_as_uint(ra) & 0xffff0000u, mb = __float_as_uint(rb) & 0xffff0000u;
    const float la = ra - __uint_as_float(ma), lb = rb - __uint_as_float(mb);
    hi = (ha >> 16) | hb;
    mid = (ma >> 16) | mb;
    lo = (__float_as_uint(la) >> 16) | (__float_as_uint(lb) & 0xffff0000u);
}

// Split of 8 consecutive weights (w0 = elements 0-3, w1 = elements 4-7).
__device__ __forceinline__ void split8(const f32x4 &w0, const f32x4 &w1, u32x4 &hi, u32x4 &mid,
                                       u32x4 &lo) {
    unsigned h[4], m[4], l[4];
    split3x2(w0[0], w0[1], h[0], m[0], l[0]);
    split3x2(w0[2], w0[3], h[1], m[1], l[1]);
    split3x2(w1[0], w1[1], h[2], m[2], l[2]);
    split3x2(w1[2], w1[3], h[3], m[3], l[3]);
    hi = u32x4{h[0], h[1], h[2], h[3]};
    mid = u32x4{m[0], m[1], m[2], m[3]};
    lo = u32x4{l[0], l[1], l[2], l[3]};
}

// Ranking key of (score, expert): ordered as the scores, descending, then the
// ids, ascending (NaN ranks as -inf; -0 as +0, which compare equal).
__device__ __forceinline__ uint64_t rank_key(float v, int e) {
    const float c = v != v ? -INFINITY : v + 0.f;
    const unsigned b = __float_as_uint(c);
    const unsigned o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)o << 32) | (uint64_t)(0xffffffffu - (unsigned)e);
}
__device__ __forceinline__ float key_score(uint64_t key) {
    const unsigned o = (unsigned)(key >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}
template <int CTRL, int ROWS = 0xf>
__device__ __forceinline__ uint64_t dpp_max(uint64_t x) {
    const int lo = (int)(unsigned)x, hi = (int)(unsigned)(x >> 32);
    const unsigned olo = (unsigned)__builtin_amdgcn_update_dpp(lo, lo, CTRL, ROWS, 0xf, false);
    const unsigned ohi = (unsigned)__builtin_amdgcn_update_dpp(hi, hi, CTRL, ROWS, 0xf, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > x ? o : x;
}
// The largest key of the wave, on every lane: within quads, rows of 16, then
// across rows; lane 63 ends with the maximum of all 64.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t x) {
    x = dpp_max<0xb1>(x);          // quad_perm [1,0,3,2]
    x = dpp_max<0x4e>(x);          // quad_perm [2,3,0,1]
    x = dpp_max<0x124>(x);         // row_ror:4
    x = dpp_max<0x128>(x);         // row_ror:8
    x = dpp_max<0x142, 0xa>(x);    // row_bcast:15 into rows 1 and 3
    x = dpp_max<0x143, 0xc>(x);    // row_bcast:31 into rows 2 and 3
    const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)x, 63);
    const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(unsigned)(x >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Top-k of one token's scores held by a whole wave (lane g holds experts g,
// g+64, ...), as topk_softmax_group below for G = 64: every round takes the
// wave's largest ranking key by DPP moves (no LDS shuffles) and the softmax
// sums the kept choices' terms in choice order from uniform reads.
template <int Q>
__device__ __forceinline__ void topk_softmax_wave(const float (&v)[Q], int E, int k, int64_t t,
                                                  bool active, int32_t *__restrict__ idx_out,
                                                  float *__restrict__ gate_out) {
    const int lane = __lane_id();
    uint64_t key[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = lane + 64 * q;
        key[q] = e < E ? rank_key(v[q], e) : 0ull;   // 0: no candidate
    }
    float my_v = -INFINITY, v0 = -INFINITY;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        uint64_t b = key[0];
#pragma unroll
        for (int q = 1; q < Q; ++q)
            b = key[q] > b ? key[q] : b;
        b = wave_max_key(b);
        const int be = (int)(0xffffffffu - (unsigned)b);
        const float bv = key_score(b);
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (be == lane + 64 * q)
                key[q] = 0ull;
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
        if (j == 0)
            v0 = bv;
    }
    const float ex = lane < k ? expf(my_v - v0) : 0.f;
    float den = 0.f;
    for (int j = 0; j < k; ++j)   // choice order
        den += __uint_as_float(
            (unsigned)__builtin_amdgcn_readlane((int)__float_as_uint(ex), j));
    if (active && lane < k) {
        idx_out[t * k + lane] = my_e;
        gate_out[t * k + lane] = ex / den;
    }
}

// Top-k of one token's scores held by a group of G lanes (lane g of the
// group holds experts g, g+G, ...; a wave ranks 64/G tokens at once) and the
// softmax of the kept scores. Every lane of a group ends with the same
// selection; lanes j < k of the group write choice j.
template <int G, int Q>
__device__ __forceinline__ void topk_softmax_group(const float (&v)[Q], int E, int k, int64_t t,
                                                   bool active, int32_t *__restrict__ idx_out,
                                                   float *__restrict__ gate_out) {
    if constexpr (G == 64) {
        topk_softmax_wave<Q>(v, E, k, t, active, idx_out, gate_out);
        return;
    }
    const int lane = __lane_id();
    const int lg = lane % G, gbase = lane - lg;
    unsigned taken = 0;
    float my_v = -INFINITY, v0 = -INFINITY;
    int my_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = INT_MAX;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = lg + G * q;
            // a NaN score ranks as -inf, so every lane of the group holds a
            // candidate in [0, E) while an untaken expert is left
            const float vq = v[q] != v[q] ? -INFINITY : v[q];
            if (e < E && !((taken >> q) & 1u)) {
                if (vq > bv || (vq == bv && e < be)) {
                    bv = vq;
                    be = e;
                }
            }
        }
        // group arg-max under the total order (score desc, id asc)
#pragma unroll
        for (int off = G / 2; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oe = __shfl_xor(be, off);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be % G) == lg)
            taken |= 1u << (be / G);
        if (lg == j) {
            my_v = bv;
            my_e = be;
        }
        if (j == 0)
            v0 = bv;
    }
    const float ex = lg < k ? expf(my_v - v0) : 0.f;
    float den = 0.f;
    for (int j = 0; j < k; ++j)   // choice order, identical on every lane of the group
        den += __shfl(ex, gbase + j);
    if (active && lg < k) {
        idx_out[t * k + lg] = my_e;
        gate_out[t * k + lg] = ex / den;
    }
}

// W_g [E, d] fp32 -> Wsp [Ep][3 d] bf16 (row pi(e): hi, mid, lo of expert e, per
// 64 columns when interleaved);
// 8 elements per thread.
__global__ __launch_bounds__(256) void split_router_weights_kernel(const float *__restrict__ wg,
                                                                   int E, int Ep, int d,
                                                                   bool inter,
                                                                   unsigned short *__restrict__ wsp) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // group of 8
    const int64_t groups = (int64_t)Ep * (d / 8);
    if (g >= groups)
        return;
    const int e = (int)(g / (d / 8));
    const int i = (int)(g - (int64_t)e * (d / 8)) * 8;
    f32x4 w0 = {0.f, 0.f, 0.f, 0.f}, w1 = {0.f, 0.f, 0.f, 0.f};
    if (e < E) {
        w0 = *reinterpret_cast<const f32x4 *>(wg + (int64_t)e * d + i);
        w1 = *reinterpret_cast<const f32x4 *>(wg + (int64_t)e * d + i + 4);
    }
    u32x4 hi, mid, lo;
    split8(w0, w1, hi, mid, lo);
    const int Q = Ep > 64 ? Ep / 64 : 1;
    unsigned short *row = wsp + (int64_t)((e % 64) * Q + e / 64) * 3 * d;
    // the terms of 64 columns one after the other, or each term's d columns
    const int64_t o = inter ? (int64_t)(i / 64) * 192 + i % 64 : i;
    const int64_t step = inter ? 64 : d;
    *reinterpret_cast<u32x4 *>(row + o) = hi;
    *reinterpret_cast<u32x4 *>(row + o + step) = mid;
    *reinterpret_cast<u32x4 *>(row + o + 2 * step) = lo;
}

// Ranking of one token per 64-lane wave from the partial scores of ns
// K-ranges, P [ns][N][Ep] (summed here in range order), plus noise. Lane g
// holds experts g + 64 q, q < Q, which the permuted columns place at
// g Q .. g Q + Q - 1: one load of Q scores per range.
template <int G, int Q>
__global__ __launch_bounds__(256) void rank_scores_kernel(const float *__restrict__ P, int ns,
                                                          const float *__restrict__ noise, int N,
                                                          int E, int Ep, int k,
                                                          int32_t *__restrict__ idx_out,
                                                          float *__restrict__ gate_out) {
    const int lane = threadIdx.x & 63;
    const int lg = lane % G;
    const int64_t t = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / G) + lane / G;
    const bool active = t < N;
    const int64_t tc = active ? t : 0;
    static_assert(G == 64 && (Q == 1 || Q == 2 || Q == 4), "one token per wave");
    float v[Q];
    const float *r = P + tc * Ep + (int64_t)lg * Q;
    auto load = [&](const float *p, float (&o)[Q]) {
        if constexpr (Q == 4) {
            const f32x4 t4 = *reinterpret_cast<const f32x4 *>(p);
            o[0] = t4[0]; o[1] = t4[1]; o[2] = t4[2]; o[3] = t4[3];
        } else if constexpr (Q == 2) {
            const f32x2_t t2 = *reinterpret_cast<const f32x2_t *>(p);
            o[0] = t2[0]; o[1] = t2[1];
        } else {
            o[0] = p[0];
        }
    };
    load(r, v);
    // the ranges' loads in batches of B in flight, added in range order
    constexpr int B = 8;
    for (int s0 = 1; s0 < ns; s0 += B) {
        float w[B][Q];
#pragma unroll
        for (int u = 0; u < B; ++u)
            if (s0 + u < ns)
                load(r + (int64_t)(s0 + u) * N * Ep, w[u]);
#pragma unroll
        for (int u = 0; u < B; ++u)
            if (s0 + u < ns)
#pragma unroll
                for (int q = 0; q < Q; ++q)
                    v[q] += w[u][q];
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int e = lg + G * q;
        float sc = -INFINITY;
        if (e < E) {
            sc = v[q];
            if (noise)
                sc += noise[tc * E + e];
            if (sc != sc)
                sc = -INFINITY;
        }
        v[q] = sc;
    }
    topk_softmax_group<G, Q>(v, E, k, t, active, idx_out, gate_out);
}

// One block = 16 tokens; wave w of NW accumulates K-chunks c = w, w+NW, ...
// with 16x16x32 bf16 MFMAs over NT tiles of 16 experts, then the NW partial
// score tiles are summed in wave order through LDS and the first four waves
// rank the tokens. Wide rows (d >= 2048) take 16 waves, so that a CU keeps
// four times the loads in flight.
template <int NT, int NW>
__global__ __launch_bounds__(NW * 64) void router_bf16_kernel(
    const unsigned short *__restrict__ x, const float *__restrict__ wg,
    const float *__restrict__ noise, int N, int d, int E, int k,
    int32_t *__restrict__ idx_out, float *__restrict__ gate_out) {
    constexpr int EP = NT * 16;
    constexpr int kWaves = NW;
    static_assert(NW >= kRankWaves, "four ranking waves");
    __shared__ float red[kWaves * kTokTile * EP];

    const int lane = threadIdx.x & 63;
    const int w = threadIdx.x >> 6;
    const int row = lane & 15;   // token row (A) / expert column (B) of this lane
    const int kg = lane >> 4;    // 8-element K group of this lane
    const int64_t t0 = (int64_t)blockIdx.x * kTokTile;
    const int64_t tok = t0 + row;
    const bool tok_ok = tok < N;
    const unsigned short *xrow = x + (tok_ok ? tok : 0) * (int64_t)d;

    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Ranking layout: groups of G lanes rank one token each, 64/G tokens per
    // pass, TPW/TPP passes for the 4 tokens 4w .. 4w+3 this wave ranks. Their
    // noise rows are loaded up front, overlapping the score product.
    constexpr int TPW = kTokTile / kRankWaves;
    constexpr int G = EP <= 16 ? 16 : (EP <= 32 ? 32 : 64);
    constexpr int QG = (EP + G - 1) / G;   // scores per lane
    constexpr int TPP = 64 / G;             // tokens per pass
    constexpr int PASSES = TPW / TPP;
    const int lg = lane % G;
    float nz[PASSES][QG];
    const bool ranker = w < kRankWaves;
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int64_t t = t0 + w * TPW + ps * TPP + lane / G;
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            const int e = lg + G * q;
            nz[ps][q] = (ranker && noise && t < N && e < E) ? noise[t * E + e] : 0.f;
        }
    }
    // K-chunks are processed in batches of U: all loads of a batch are issued
    // before any of its MFMAs (from clamped, always valid addresses; chunks
    // past d or experts past E are masked to zero afterwards), so a wave
    // waits for memory once per batch rather than once per chunk. Small
    // batches keep the registers few and the workgroups per CU many, which
    // hides the load latency better than deep batches (16 experts or fewer,
    // measured: batches of 2 against 8 take the nanoMoE router from 5.7 to
    // 4.8 us and the Mixtral-shaped one from 14.6 to 13.1 us). With at most
    // 32 experts the fp32 weights are split in registers (a few VALU
    // operations per weight), which saves a separate split kernel.
    constexpr int U = NT >= 2 ? 4 : 2;
    const int nchunks = (d + 31) / 32;
    for (int c0 = w; c0 < nchunks; c0 += kWaves * U) {
        u32x4 xa[U];
        f32x4 w0[U][NT], w1[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kof = (c0 + u * kWaves) * 32 + kg * 8;
            const int kc = kof < d ? kof : 0;   // d % 8 == 0: a group is all in or all out
            xa[u] = *reinterpret_cast<const u32x4 *>(xrow + kc);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int e = nt * 16 + row;
                const float *wp = wg + (int64_t)(e < E ? e : 0) * d + kc;
                w0[u][nt] = *reinterpret_cast<const f32x4 *>(wp);
                w1[u][nt] = *reinterpret_cast<const f32x4 *>(wp + 4);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool k_ok = (c0 + u * kWaves) * 32 + kg * 8 < d;
            const u32x4 z = {0u, 0u, 0u, 0u};
            const bf16x8 a = __builtin_bit_cast(bf16x8, (tok_ok && k_ok) ? xa[u] : z);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const bool w_ok = k_ok && (nt * 16 + row < E);
                const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
                u32x4 hi, mid, lo;
                split8(w_ok ? w0[u][nt] : zf, w_ok ? w1[u][nt] : zf, hi, mid, lo);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, hi), acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, mid), acc[nt], 0, 0, 0);
                acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, __builtin_bit_cast(bf16x8, lo), acc[nt], 0, 0, 0);
            }
        }
    }
    // acc[nt][i] holds the partial score of token 4*kg+i for expert nt*16+row
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            red[(w * kTokTile + 4 * kg + i) * EP + nt * 16 + row] = acc[nt][i];
    __syncthreads();
    if (!ranker)
        return;

#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
        const int m = w * TPW + ps * TPP + lane / G;
        const int64_t t = t0 + m;
        float v[QG];
#pragma unroll
        for (int q = 0; q < QG; ++q) {
            const int e = lg + G * q;
            float s = -INFINITY;
            if (e < E) {
                s = red[(0 * kTokTile + m) * EP + e];
#pragma unroll
                for (int ww = 1; ww < kWaves; ++ww)
                    s += red[(ww * kTokTile + m) * EP + e];
                if (noise)
                    s += nz[ps][q];
                if (s != s)
                    s = -INFINITY;   // a NaN score never outranks a number
            }
            v[q] = s;
        }
        topk_softmax_group<G, QG>(v, E, k, t, t < N, idx_out, gate_out);
    }
}

// fp32 activations: one wave per token, lanes stride over d, the wave then
// reduces each expert's partial sums in a fixed butterfly order.
__global__ __launch_bounds__(256) void router_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ wg, const float *__restrict__ noise,
    int N, int d, int E, int k, int32_t *__restrict__ idx_out, float *__restrict__ gate_out) {
    constexpr int Q = kMaxQ;
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= N)
        return;
    const float *xr = x + t * (int64_t)d;
    float v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q)
        v[q] = -INFINITY;
    for (int e = 0; e < E; ++e) {
        float p = 0.f;
        for (int i = lane; i < d; i += 64)
            p = fmaf(wg[(int64_t)e * d + i], xr[i], p);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1)
            p += __shfl_xor(p, off);
        p = __shfl(p, 0);   // every lane takes lane 0's sum
        if (noise)
            p += noise[t * E + e];
        if (p != p)
            p = -INFINITY;
#pragma unroll
        for (int q = 0; q < Q; ++q)
            if (e == lane + 64 * q)
                v[q] = p;
    }
    topk_softmax_group<64, Q>(v, E, k, t, true, idx_out, gate_out);
}

template <int NT>
hipError_t launch_fused(const void *x, const float *wg, const float *noise, int64_t N,
                        int64_t d, int E, int k, int32_t *idx, float *gate, hipStream_t s) {
    const int blocks = (int)((N + kTokTile - 1) / kTokTile);
    if (d >= 2048)
        hipLaunchKernelGGL((router_bf16_kernel<NT, 16>), dim3(blocks), dim3(1024), 0, s,
                           static_cast<const unsigned short *>(x), wg, noise, (int)N, (int)d, E,
                           k, idx, gate);
    else
        hipLaunchKernelGGL((router_bf16_kernel<NT, 4>), dim3(blocks), dim3(256), 0, s,
                           static_cast<const unsigned short *>(x), wg, noise, (int)N, (int)d, E,
                           k, idx, gate);
    return hipGetLastError();
}

template <int G, int Q>
hipError_t launch_rank(const float *P, int ns, const float *noise, int64_t N, int E, int Ep,
                       int k, int32_t *idx, float *gate, hipStream_t s) {
    const int64_t tokens_per_block = 4 * (64 / G);
    const int blocks = (int)((N + tokens_per_block - 1) / tokens_per_block);
    hipLaunchKernelGGL((rank_scores_kernel<G, Q>), dim3(blocks), dim3(256), 0, s, P, ns, noise,
                       (int)N, E, Ep, k, idx, gate);
    return hipGetLastError();
}

}  // namespace

int64_t router_padded_experts(int E) {
    // past 64 experts a ranking lane holds Q = Ep / 64 in {2, 4} scores
    return E <= 64 ? (E + 15) / 16 * 16 : E <= 128 ? 128 : 256;
}

size_t router_workspace_bytes(int64_t N, int64_t d, int E) {
    const int64_t Ep = router_padded_experts(E);
    if (Ep <= kFusedMaxExperts)
        return 0;
    const int64_t ns = router_score_splits(N, d, Ep);
    return (size_t)(3 * Ep * d * 2 + 255) / 256 * 256 + (size_t)(ns * N * Ep * 4 + 255) / 256 * 256;
}

hipError_t launch_router_bf16(const void *x, const float *wg, const float *noise, int64_t N,
                              int64_t d, int E, int k, int32_t *idx, float *gate, void *ws,
                              hipStream_t s) {
    if (N == 0)
        return hipSuccess;
    const int Ep = (int)router_padded_experts(E);
    if (Ep <= 16) return launch_fused<1>(x, wg, noise, N, d, E, k, idx, gate, s);
    if (Ep <= 32) return launch_fused<2>(x, wg, noise, N, d, E, k, idx, gate, s);
    unsigned short *wsp = static_cast<unsigned short *>(ws);
    const int64_t groups = (int64_t)Ep * (d / 8);
    hipLaunchKernelGGL(split_router_weights_kernel, dim3((unsigned)((groups + 255) / 256)),
                       dim3(256), 0, s, wg, E, Ep, (int)d, router_terms_interleaved(d), wsp);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    float *P = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                         (size_t)(3 * Ep * d * 2 + 255) / 256 * 256);
    err = launch_router_scores_bf16(x, wsp, N, d, Ep, P, s);
    if (err != hipSuccess)
        return err;
    const int ns = router_score_splits(N, d, Ep);
    if (Ep <= 64) return launch_rank<64, 1>(P, ns, noise, N, E, Ep, k, idx, gate, s);
    if (Ep <= 128) return launch_rank<64, 2>(P, ns, noise, N, E, Ep, k, idx, gate, s);
    return launch_rank<64, 4>(P, ns, noise, N, E, Ep, k, idx, gate, s);
}

hipError_t launch_router_f32(const float *x, const float *wg, const float *noise, int64_t N,
                             int64_t d, int E, int k, int32_t *idx, float *gate,
                             hipStream_t s) {
    if (N == 0)
        return hipSuccess;
    const int blocks = (int)((N + 3) / 4);
    hipLaunchKernelGGL(router_f32_kernel, dim3(blocks), dim3(256), 0, s, x, wg, noise, (int)N,
                       (int)d, E, k, idx, gate);
    return hipGetLastError();
}

}  // namespace moe
