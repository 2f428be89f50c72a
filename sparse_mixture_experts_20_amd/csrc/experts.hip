// Grouped expert FFN over the dispatch plan.
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 7 (each token is copied only to its kept experts), STEP 8 (z = W_up x),
// STEP 9 (h = ReLU(z)), STEP 10 (E(x) = W_down h); nanoMoE slides 32-37 (the
// experts are batched: one product per expert over its packed token rows).
//
//   up:   H[e, r, :] = ReLU(W_up[e] x_t)   for r < used[e], t = slot_token[e, r] / k
//   down: Y[a, :]    = W_down[e] H[e, r, :]  with a = slot_token[e, r]
//
// Both are "NT" products: every operand row is contiguous along the
// reduction dimension (activation rows along d or d_ff, weight rows are
// output neurons), which is exactly the K-contiguous layout both operands of
// a CDNA matrix instruction want. The gather of token rows (dispatch) is
// fused into the up product's operand load, so no packed copy of the tokens
// is ever written; the down product scatters its rows straight into the
// assignment-ordered buffer the combine reads.
//
// bf16 tile: 128 x 128 outputs, K-step 64, 256 threads = 2 x 2 waves of
// 64 x 64, each built from 16x16x32 bf16 MFMAs with fp32 accumulation; A and
// B tiles double-buffered in LDS (rows padded by 16 bytes so the 16-byte
// reads of a wave hit distinct banks). Tiles are enumerated only for rows that
// exist (the dispatch plan's prefix of ceil(used[e]/128)); consecutive tiles
// of one expert walk its row tiles fastest so the blocks in flight share each
// weight tile, and each XCD (blocks b with the same b % 8) receives one
// contiguous range of tiles so that sharing happens inside one L2.
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDK = BK + 8;            // padded LDS row (bf16 elements)
constexpr int kThreads = 256;
constexpr int kXcds = 8;

template <int MODE>   // 0: up (gather x rows, ReLU, store H in bf16); 1: down (fp32, scatter to Y)
__global__ __launch_bounds__(kThreads, 2) void experts_bf16_kernel(
    const unsigned short *__restrict__ A_src, const unsigned short *__restrict__ W, int K,
    int Nout, int E, int k, int ceff, const int32_t *__restrict__ used,
    const int32_t *__restrict__ slot_token, const int32_t *__restrict__ mt_off,
    unsigned short *__restrict__ H_out, float *__restrict__ Y_out) {
    __shared__ unsigned short As[2][BM * LDK];
    __shared__ unsigned short Bs[2][BN * LDK];
    __shared__ int s_mt[kMaxExperts + 1];

    const int tid = threadIdx.x;
    const int NT = (Nout + BN - 1) / BN;

    for (int i = tid; i <= E; i += kThreads)
        s_mt[i] = mt_off[i];
    __syncthreads();
    const int T = s_mt[E] * NT;
    const int T8 = (T + kXcds - 1) / kXcds * kXcds;
    const int b = blockIdx.x;
    if (b >= T8)
        return;
    const int L = (b % kXcds) * (T8 / kXcds) + b / kXcds;
    if (L >= T)
        return;
    // expert owning tile L: the last e with s_mt[e] * NT <= L
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_mt[mid] * NT <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int mte = s_mt[e + 1] - s_mt[e];
    const int local = L - s_mt[e] * NT;
    const int m0 = (local % mte) * BM;
    const int n0 = (local / mte) * BN;
    const int rows = used[e];

    // global -> LDS copy assignment: 8 threads per 64-element row, 32 rows per pass
    const int lrow = tid >> 3;
    const int lk = (tid & 7) * 8;
    const unsigned short *arow[4];
    const unsigned short *brow[4];
    bool aok[4], bok[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int r = m0 + p * 32 + lrow;
        aok[p] = r < rows;
        int64_t src = 0;
        if (aok[p]) {
            const int64_t srow = (int64_t)e * ceff + r;
            src = MODE == 0 ? (int64_t)(slot_token[srow] / k) : srow;
        }
        arow[p] = A_src + src * K;
        const int n = n0 + p * 32 + lrow;
        bok[p] = n < Nout;
        brow[p] = W + ((int64_t)e * Nout + (bok[p] ? n : 0)) * K;
    }

    const int lane = tid & 63;
    const int wv = tid >> 6;
    const int wm = wv >> 1, wn = wv & 1;

    f32x4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 ra[4], rb[4];
    auto gload = [&](int kt) {
        const int kk = kt * BK + lk;
        const bool kok = kk < K;   // K % 8 == 0
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            ra[p] = (aok[p] && kok) ? *reinterpret_cast<const u32x4 *>(arow[p] + kk)
                                    : u32x4{0u, 0u, 0u, 0u};
            rb[p] = (bok[p] && kok) ? *reinterpret_cast<const u32x4 *>(brow[p] + kk)
                                    : u32x4{0u, 0u, 0u, 0u};
        }
    };
    auto sstore = [&](int st) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            *reinterpret_cast<u32x4 *>(&As[st][(p * 32 + lrow) * LDK + lk]) = ra[p];
            *reinterpret_cast<u32x4 *>(&Bs[st][(p * 32 + lrow) * LDK + lk]) = rb[p];
        }
    };

    const int KT = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int st = kt & 1;
        if (kt + 1 < KT)
            gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < BK; ks += 32) {
            const int kof = ks + (lane >> 4) * 8;
            bf16x8 af[4], bfr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wm * 64 + i * 16 + (lane & 15);
                af[i] = *reinterpret_cast<const bf16x8 *>(&As[st][r * LDK + kof]);
                const int c = wn * 64 + i * 16 + (lane & 15);
                bfr[i] = *reinterpret_cast<const bf16x8 *>(&Bs[st][c * LDK + kof]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT)
            sstore(st ^ 1);
        __syncthreads();
    }

    // epilogue: acc[i][j][q] is row wm*64 + i*16 + 4*(lane/16) + q, column wn*64 + j*16 + lane%16
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = m0 + wm * 64 + i * 16 + (lane >> 4) * 4 + q;
            if (r >= rows)
                continue;
            const int64_t srow = (int64_t)e * ceff + r;
            if (MODE == 0) {
                unsigned short *dst = H_out + srow * Nout;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 64 + j * 16 + (lane & 15);
                    if (n < Nout)
                        dst[n] = f32_to_bf16_bits(fmaxf(acc[i][j][q], 0.f));
                }
            } else {
                float *dst = Y_out + (int64_t)slot_token[srow] * Nout;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int n = n0 + wn * 64 + j * 16 + (lane & 15);
                    if (n < Nout)
                        dst[n] = acc[i][j][q];
                }
            }
        }
    }
}

// fp32 path (correctness-first, any shape): 64 x 64 tiles, K-step 16,
// 256 threads with 4 x 4 outputs each, fp32 FMA.
template <int MODE>
__global__ __launch_bounds__(256) void experts_f32_kernel(
    const float *__restrict__ A_src, const float *__restrict__ W, int K, int Nout, int k,
    int ceff, const int32_t *__restrict__ used, const int32_t *__restrict__ slot_token,
    float *__restrict__ H_out, float *__restrict__ Y_out) {
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
            if (MODE == 0)
                H_out[srow * Nout + n] = fmaxf(acc[i][j], 0.f);
            else
                Y_out[(int64_t)slot_token[srow] * Nout + n] = acc[i][j];
        }
    }
}

}  // namespace

hipError_t launch_expert_up(bool bf16, const void *x, const void *w_up, int64_t d,
                            int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                            const int32_t *slot_token, const int32_t *tiles, void *H,
                            hipStream_t s) {
    if (ceff == 0)
        return hipSuccess;
    if (bf16) {
        const int64_t mt_max = (ceff + BM - 1) / BM;
        const int64_t nt = (d_ff + BN - 1) / BN;
        const int64_t grid = (E * mt_max * nt + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL(experts_bf16_kernel<0>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           static_cast<const unsigned short *>(x),
                           static_cast<const unsigned short *>(w_up), (int)d, (int)d_ff, E, k,
                           (int)ceff, used, slot_token, tiles,
                           static_cast<unsigned short *>(H), (float *)nullptr);
    } else {
        hipLaunchKernelGGL(experts_f32_kernel<0>,
                           dim3((unsigned)((d_ff + 63) / 64), (unsigned)((ceff + 63) / 64), E),
                           dim3(256), 0, s, static_cast<const float *>(x),
                           static_cast<const float *>(w_up), (int)d, (int)d_ff, k, (int)ceff,
                           used, slot_token, static_cast<float *>(H), (float *)nullptr);
    }
    return hipGetLastError();
}

hipError_t launch_expert_down(bool bf16, const void *H, const void *w_down, int64_t d,
                              int64_t d_ff, int E, int k, int64_t ceff, const int32_t *used,
                              const int32_t *slot_token, const int32_t *tiles, float *Y,
                              hipStream_t s) {
    if (ceff == 0)
        return hipSuccess;
    if (bf16) {
        const int64_t mt_max = (ceff + BM - 1) / BM;
        const int64_t nt = (d + BN - 1) / BN;
        const int64_t grid = (E * mt_max * nt + kXcds - 1) / kXcds * kXcds;
        hipLaunchKernelGGL(experts_bf16_kernel<1>, dim3((unsigned)grid), dim3(kThreads), 0, s,
                           static_cast<const unsigned short *>(H),
                           static_cast<const unsigned short *>(w_down), (int)d_ff, (int)d, E, k,
                           (int)ceff, used, slot_token, tiles, (unsigned short *)nullptr, Y);
    } else {
        hipLaunchKernelGGL(experts_f32_kernel<1>,
                           dim3((unsigned)((d + 63) / 64), (unsigned)((ceff + 63) / 64), E),
                           dim3(256), 0, s, static_cast<const float *>(H),
                           static_cast<const float *>(w_down), (int)d_ff, (int)d, k, (int)ceff,
                           used, slot_token, (float *)nullptr, Y);
    }
    return hipGetLastError();
}

}  // namespace moe
