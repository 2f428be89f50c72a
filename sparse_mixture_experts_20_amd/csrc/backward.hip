// Backward pass of the layer: gradients of a loss through the gates to the
// router and through the experts (ReLU or GELU experts, optional biases,
// optional training-mode dropout on the expert outputs).
// Chain rule of the forward in this library (page 1 STEP 2-12; nanoMoE
// slides 11-40), for an output gradient dout:
//   combine  out_t = sum_j g_tj y_tj (kept j)   -> dy_tj = g_tj dout_t,
//                                                 dg_tj = <dout_t, y_tj>
//   softmax over the kept scores                -> ds_j = g_j (dg_j - sum_l g_l dg_l)
//   scores   s = W_g x + noise                  -> dW_g = ds^T x, dx += ds W_g
//   experts  h = ReLU(W_up x), y = W_down h     -> dZ = (dY W_down) [H > 0],
//            dW_down = dY^T H, dW_up = dZ^T X, dX = dZ W_up
// The products run on the expert GEMM kernel (bf16 operands, fp32
// accumulation); this file holds the element-wise and layout kernels around
// them: the combine's backward, the dense split of ds for the router-weight
// product, transposes that make every product "NT", and the assembly of dx.
// Every sum has a fixed order, so the gradients are the same on every run.
#include "common.hpp"

namespace moe {
namespace {

// Exact split of an fp32 value into three bf16 terms (upper 16 bits of the
// value, then of the exact residual; the last residual has at most 8
// significant bits).
__device__ __forceinline__ void split3_bits(float a, unsigned short &hi, unsigned short &mid,
                                            unsigned short &lo) {
    const unsigned h = __float_as_uint(a) & 0xffff0000u;
    const float r = a - __uint_as_float(h);
    const unsigned m = __float_as_uint(r) & 0xffff0000u;
    const float l = r - __uint_as_float(m);
    hi = (unsigned short)(h >> 16);
    mid = (unsigned short)(m >> 16);
    lo = (unsigned short)(__float_as_uint(l) >> 16);
}

// One wave per token: dY rows (bf16, kept choices), dg by a wave reduction in
// a fixed butterfly order, then ds for every choice (dropped ones have dg 0
// but still took part in the softmax). Y holds the experts' outputs, the
// values the forward combined: fp32 rows, or (ysh not NULL) the compact fp16
// rows with one exponent shift per kYGroup columns; 8 columns per lane and
// load.
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const unsigned short *__restrict__ dout, const void *__restrict__ Y,
    const signed char *__restrict__ ysh, const float *__restrict__ gate,
    const int32_t *__restrict__ slot, int N, int d, int k, unsigned short *__restrict__ dY,
    float *__restrict__ ds, Dropout dp) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= N)
        return;
    const int chunks = d / 8;
    const unsigned short *go = dout + t * d;
    float dg[kMaxTopK];
    float gdg = 0.f;
    for (int j = 0; j < k; ++j) {
        const int64_t a = t * k + j;
        float p = 0.f;
        if (slot[a] >= 0) {
            const float g = gate[a];
            unsigned short *dyr = dY + a * d;
            for (int c = lane; c < chunks; c += 64) {
                const u32x4 ov = *reinterpret_cast<const u32x4 *>(go + 8 * c);
                f32x4 y0, y1;
                if (ysh) {
                    const u32x4 h = *reinterpret_cast<const u32x4 *>(
                        static_cast<const unsigned short *>(Y) + a * d + 8 * c);
                    const float sc = pow2f(-(int)ysh[yshift_index(
                        t, j, k, (d + kYGroup - 1) / kYGroup, 8 * c / kYGroup)]);
                    const f32x2_t p0 = unpack_f16x2(h[0]), p1 = unpack_f16x2(h[1]);
                    const f32x2_t p2 = unpack_f16x2(h[2]), p3 = unpack_f16x2(h[3]);
                    y0 = f32x4{p0[0], p0[1], p1[0], p1[1]} * sc;
                    y1 = f32x4{p2[0], p2[1], p3[0], p3[1]} * sc;
                } else {
                    const float *yr = static_cast<const float *>(Y) + a * d;
                    y0 = *reinterpret_cast<const f32x4 *>(yr + 8 * c);
                    y1 = *reinterpret_cast<const f32x4 *>(yr + 8 * c + 4);
                }
                // Y already carries the dropout; dY = g dout m
                float m[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
                if (dp.on)
                    dropout_factors8(dp, a, c, m);
                u32x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float o0 = __uint_as_float(ov[q] << 16);
                    const float o1 = __uint_as_float(ov[q] & 0xffff0000u);
                    const f32x4 &y = q < 2 ? y0 : y1;
                    p = fmaf(o0, y[(q % 2) * 2], p);
                    p = fmaf(o1, y[(q % 2) * 2 + 1], p);
                    w[q] = pack_bf16x2(g * o0 * m[2 * q], g * o1 * m[2 * q + 1]);
                }
                *reinterpret_cast<u32x4 *>(dyr + 8 * c) = w;
            }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1)
                p += __shfl_xor(p, off);
        }
        dg[j] = p;
        gdg = fmaf(gate[t * k + j], p, gdg);
    }
    if (lane < k) {
        float v = 0.f;
        for (int j = 0; j < k; ++j)
            if (j == lane)
                v = gate[t * k + j] * (dg[j] - gdg);
        ds[t * k + lane] = v;
    }
}

// Token-chunked operands of the router-weight product dW_g = ds^T x: chunk s
// holds tokens [s*Tc, (s+1)*Tc). dsT3[s][e][q*Tc + i] is term q of the exact
// three-term split of ds(s*Tc + i, e) (0 where that token did not choose e or
// lies past N).
__global__ __launch_bounds__(256) void ds_split_kernel(const float *__restrict__ ds,
                                                       const int32_t *__restrict__ idx, int N,
                                                       int Tc, int S, int E, int k,
                                                       unsigned short *__restrict__ dsT3) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)S * E * Tc)
        return;
    const int tt = (int)(i % Tc);
    const int64_t se = i / Tc;             // s * E + e
    const int e = (int)(se % E);
    const int t = (int)(se / E) * Tc + tt;
    float v = 0.f;
    if (t < N)
        for (int j = 0; j < k; ++j)
            if (idx[(int64_t)t * k + j] == e)
                v = ds[(int64_t)t * k + j];
    unsigned short h, m, l;
    split3_bits(v, h, m, l);
    unsigned short *row = dsT3 + se * 3 * Tc;
    row[tt] = h;
    row[Tc + tt] = m;
    row[2 * Tc + tt] = l;
}

// dW_g[e][c] = sum over chunks s (in order) of part[s][e][c].
__global__ __launch_bounds__(256) void chunk_sum_kernel(const float *__restrict__ part, int S,
                                                        int64_t n, float *__restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n)
        return;
    float acc = 0.f;
    int s = 0;
    for (; s + 8 <= S; s += 8) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            v[q] = part[(int64_t)(s + q) * n + i];
#pragma unroll
        for (int q = 0; q < 8; ++q)
            acc += v[q];
    }
    for (; s < S; ++s)
        acc += part[(int64_t)s * n + i];
    out[i] = acc;
}

// Column sums of an expert's rows: out[e][c] = sum over r < used[e] of
// src[row(e, r)][c]. A block takes 512 columns (8 per lane) of one expert;
// its 16 waves sum contiguous sixteenths of the rows in order, then the
// partial sums are added in wave order, so the result does not depend on
// timing.
constexpr int kColsumWaves = 16;
__global__ __launch_bounds__(kColsumWaves * 64) void colsum_rows_kernel(
    const unsigned short *__restrict__ src, int C, int64_t ceff, const int32_t *__restrict__ used,
    const int32_t *__restrict__ slot_token, int kdiv, float *__restrict__ out) {
    __shared__ float part[kColsumWaves][512];
    const int e = blockIdx.y;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c0 = blockIdx.x * 512 + lane * 8;
    const int R = used[e];
    const int r0 = (int)((int64_t)R * w / kColsumWaves);
    const int r1 = (int)((int64_t)R * (w + 1) / kColsumWaves);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c0 < C) {
#pragma unroll 8
        for (int r = r0; r < r1; ++r) {
            const int64_t sr = (int64_t)e * ceff + r;
            const int64_t row = slot_token ? (int64_t)(slot_token[sr] / kdiv) : sr;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(src + row * C + c0);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc[2 * q] += __uint_as_float(v[q] << 16);
                acc[2 * q + 1] += __uint_as_float(v[q] & 0xffff0000u);
            }
        }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q)
        part[w][lane * 8 + q] = acc[q];
    __syncthreads();
    for (int i = threadIdx.x; i < 512; i += kColsumWaves * 64) {
        const int c = blockIdx.x * 512 + i;
        if (c < C) {
            float v = 0.f;
#pragma unroll
            for (int q = 0; q < kColsumWaves; ++q)
                v += part[q][i];
            out[(int64_t)e * C + c] = v;
        }
    }
}

// out[i] = sum of the Kp bf16 values of row i of T (one wave per row; lane
// partial sums over a fixed stride, then a fixed butterfly).
__global__ __launch_bounds__(256) void row_sums_kernel(const unsigned short *__restrict__ T,
                                                       int64_t rows, int Kp,
                                                       float *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t i = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (i >= rows)
        return;
    const unsigned short *row = T + i * Kp;
    float acc = 0.f;
    for (int c = lane * 8; c < Kp; c += 512) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(row + c);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            acc += __uint_as_float(v[q] << 16) + __uint_as_float(v[q] & 0xffff0000u);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
        acc += __shfl_xor(acc, off);
    if (lane == 0)
        out[i] = acc;
}

// Tiled transpose through LDS: out[b][c][q*Kp + r] = src row R(b, r), column
// c, for r below the batch's row count, and 0 for the rest of the Kp columns,
// for each of `copies` copies q. Row map: 0: b*ceff + r (dense batches of
// ceff rows; without `used`, the batch holds min(ceff, nrows - b*ceff) rows);
// 1: slot_token[b*ceff + r] (assignment rows); 2: slot_token[...] / k (token
// rows); with `used`, batch b holds used[b] rows. 64 x 64 tiles, 256
// threads, 16-byte loads and stores (C and Kp multiples of 8).
__global__ __launch_bounds__(256) void transpose_rows_kernel(
    const unsigned short *__restrict__ src, int C, int64_t ceff, const int32_t *__restrict__ used,
    int64_t nrows, const int32_t *__restrict__ slot_token, int k, int map, int Kp, int copies,
    unsigned short *__restrict__ out) {
    constexpr int LD = 64 + 2;               // padded row of the LDS tile (u16)
    __shared__ unsigned short tile[64 * LD];
    const int b = blockIdx.z;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    int64_t rows;
    if (used)
        rows = used[b];
    else {
        rows = nrows - (int64_t)b * ceff;
        rows = rows < ceff ? rows : ceff;
    }
    const int tid = threadIdx.x;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int q = tid + 256 * p;
        const int rr = q >> 3, cc = (q & 7) * 8;
        const int r = r0 + rr, c = c0 + cc;
        u32x4 v = {0u, 0u, 0u, 0u};
        if (r < rows && c < C) {
            const int64_t sr = (int64_t)b * ceff + r;
            const int64_t row = map == 0 ? sr
                              : map == 1 ? (int64_t)slot_token[sr]
                                         : (int64_t)(slot_token[sr] / k);
            v = *reinterpret_cast<const u32x4 *>(src + row * C + c);
        }
        unsigned short *dst = tile + rr * LD + cc;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            dst[2 * h] = (unsigned short)(v[h] & 0xffffu);
            dst[2 * h + 1] = (unsigned short)(v[h] >> 16);
        }
    }
    __syncthreads();
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int q = tid + 256 * p;
        const int cc = q >> 3, rr = (q & 7) * 8;
        const int c = c0 + cc, r = r0 + rr;
        if (c < C && r < Kp) {
            u32x4 w;
#pragma unroll
            for (int h = 0; h < 4; ++h)
                w[h] = (unsigned)tile[(rr + 2 * h) * LD + cc] |
                       ((unsigned)tile[(rr + 2 * h + 1) * LD + cc] << 16);
            unsigned short *o = out + ((int64_t)b * C + c) * ((int64_t)copies * Kp) + r;
            for (int qq = 0; qq < copies; ++qq)
                *reinterpret_cast<u32x4 *>(o + (int64_t)qq * Kp) = w;
        }
    }
}

// dx[t] = sum over kept j of dXa[t*k + j] + sum over j of ds[t, j] W_g[idx[t, j]],
// in that order; one thread per 4 columns.
__global__ __launch_bounds__(256) void dx_kernel(const float *__restrict__ dXa,
                                                 const float *__restrict__ ds,
                                                 const int32_t *__restrict__ idx,
                                                 const int32_t *__restrict__ slot,
                                                 const float *__restrict__ Wg, int64_t N, int d,
                                                 int E, int k, float *__restrict__ dx) {
    const int cols = d / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= N * cols)
        return;
    const int64_t t = i / cols;
    const int c = (int)(i - t * cols) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int64_t a = t * k + j;
        if (slot[a] >= 0)
            acc += *reinterpret_cast<const f32x4 *>(dXa + a * d + c);
    }
    for (int j = 0; j < k; ++j) {
        const int64_t a = t * k + j;
        const int e = idx[a];
        if (e < 0 || e >= E)   // not an expert: no score, no gradient (as in the dispatch)
            continue;
        const float s = ds[a];
        const f32x4 w = *reinterpret_cast<const f32x4 *>(Wg + (int64_t)e * d + c);
        acc += s * w;
    }
    *reinterpret_cast<f32x4 *>(dx + t * d + c) = acc;
}

}  // namespace

hipError_t launch_combine_backward(const void *dout, const void *Y, const signed char *ysh,
                                   const float *gate, const int32_t *slot, int64_t N, int64_t d,
                                   int k, void *dY, float *ds, hipStream_t s, Dropout dp) {
    if (N == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_backward_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s,
                       static_cast<const unsigned short *>(dout), Y, ysh, gate, slot, (int)N,
                       (int)d, k, static_cast<unsigned short *>(dY), ds, dp);
    return hipGetLastError();
}

hipError_t launch_ds_split(const float *ds, const int32_t *idx, int64_t N, int64_t Tc, int64_t S,
                           int E, int k, void *dsT3, hipStream_t s) {
    const int64_t n = S * E * Tc;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(ds_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ds,
                       idx, (int)N, (int)Tc, (int)S, E, k, static_cast<unsigned short *>(dsT3));
    return hipGetLastError();
}

hipError_t launch_row_sums(const void *T, int64_t rows, int64_t Kp, float *out, hipStream_t s) {
    if (rows == 0)
        return hipSuccess;
    if (Kp % 8 != 0)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(row_sums_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s,
                       static_cast<const unsigned short *>(T), rows, (int)Kp, out);
    return hipGetLastError();
}

hipError_t launch_colsum_rows(const void *src, int64_t C, int E, int64_t ceff,
                              const int32_t *used, const int32_t *slot_token, int kdiv,
                              float *out, hipStream_t s) {
    if (C == 0 || E == 0)
        return hipSuccess;
    if (C % 8 != 0 || kdiv < 1)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(colsum_rows_kernel, dim3((unsigned)((C + 511) / 512), (unsigned)E),
                       dim3(kColsumWaves * 64), 0, s, static_cast<const unsigned short *>(src),
                       (int)C, ceff,
                       used, slot_token, kdiv, out);
    return hipGetLastError();
}

hipError_t launch_chunk_sum(const float *part, int64_t S, int64_t n, float *out, hipStream_t s) {
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(chunk_sum_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, part,
                       (int)S, n, out);
    return hipGetLastError();
}

hipError_t launch_transpose_rows(const void *src, int64_t C, int64_t ceff, const int32_t *used,
                                 int64_t nrows, const int32_t *slot_token, int k, int map,
                                 int64_t Kp, int copies, int batch, void *out, hipStream_t s) {
    if (Kp == 0 || C == 0 || batch == 0)
        return hipSuccess;
    if (C % 8 != 0 || Kp % 8 != 0 || map < 0 || map > 2)
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(transpose_rows_kernel,
                       dim3((unsigned)((Kp + 63) / 64), (unsigned)((C + 63) / 64),
                            (unsigned)batch),
                       dim3(256), 0, s, static_cast<const unsigned short *>(src), (int)C, ceff,
                       used, nrows, slot_token, k, map, (int)Kp, copies,
                       static_cast<unsigned short *>(out));
    return hipGetLastError();
}

hipError_t launch_dx(const float *dXa, const float *ds, const int32_t *idx, const int32_t *slot,
                     const float *Wg, int64_t N, int64_t d, int E, int k, float *dx,
                     hipStream_t s) {
    const int64_t n = N * (d / 4);
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(dx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dXa, ds,
                       idx, slot, Wg, N, (int)d, E, k, dx);
    return hipGetLastError();
}

}  // namespace moe
