// Backward pass of the layer: gradients of a loss through the gates to the
// router and through the experts (ReLU experts, no biases, dropout off).
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
// but still took part in the softmax).
__global__ __launch_bounds__(256) void combine_backward_kernel(
    const unsigned short *__restrict__ dout, const float *__restrict__ Yf,
    const float *__restrict__ gate, const int32_t *__restrict__ slot, int N, int d, int k,
    unsigned short *__restrict__ dY, float *__restrict__ ds) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= N)
        return;
    const unsigned short *go = dout + t * d;
    float dg[kMaxTopK];
    float gdg = 0.f;
    for (int j = 0; j < k; ++j) {
        const int64_t a = t * k + j;
        float p = 0.f;
        if (slot[a] >= 0) {
            const float g = gate[a];
            const float *yr = Yf + a * d;
            unsigned short *dyr = dY + a * d;
            for (int i = lane; i < d; i += 64) {
                const float o = bf16_bits_to_f32(go[i]);
                p = fmaf(o, yr[i], p);
                dyr[i] = f32_to_bf16_bits(g * o);
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

// dsT3 [E, 3*Np] bf16: row e holds the three bf16 terms of ds(t, e) at
// columns t, Np + t, 2*Np + t (0 where token t did not choose e or t >= N).
__global__ __launch_bounds__(256) void ds_split_kernel(const float *__restrict__ ds,
                                                       const int32_t *__restrict__ idx, int N,
                                                       int Np, int E, int k,
                                                       unsigned short *__restrict__ dsT3) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)E * Np)
        return;
    const int e = (int)(i / Np), t = (int)(i - (int64_t)e * Np);
    float v = 0.f;
    if (t < N)
        for (int j = 0; j < k; ++j)
            if (idx[(int64_t)t * k + j] == e)
                v = ds[(int64_t)t * k + j];
    unsigned short h, m, l;
    split3_bits(v, h, m, l);
    unsigned short *row = dsT3 + (int64_t)e * 3 * Np;
    row[t] = h;
    row[Np + t] = m;
    row[2 * Np + t] = l;
}

// Tiled transpose through LDS: out[e][c][r] = src row R(e, r), column c, for
// r < used[e] (used == NULL: every r < nrows), and 0 for the rest of the Kp
// columns. Row map: 0: e*ceff + r (dense [E, ceff, C]); 1: slot_token[e*ceff
// + r] (assignment rows); 2: slot_token[...] / k (token rows); 3: r (a plain
// [rows, C] matrix, one batch). out has `copies` copies side by side along
// the last dimension (row length copies * Kp). 64 x 64 tiles, 256 threads.
__global__ __launch_bounds__(256) void transpose_rows_kernel(
    const unsigned short *__restrict__ src, int C, int64_t ceff, const int32_t *__restrict__ used,
    int nrows, const int32_t *__restrict__ slot_token, int k, int map, int Kp, int copies,
    unsigned short *__restrict__ out) {
    __shared__ unsigned short tile[64][66];
    const int e = blockIdx.z;
    const int r0 = blockIdx.x * 64, c0 = blockIdx.y * 64;
    const int rows = used ? used[e] : nrows;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;   // 64 x 4
    for (int rr = ty; rr < 64; rr += 4) {
        const int r = r0 + rr, c = c0 + tx;
        unsigned short v = 0;
        if (r < rows && c < C) {
            int64_t row;
            const int64_t sr = (int64_t)e * ceff + r;
            if (map == 0) row = sr;
            else if (map == 1) row = slot_token[sr];
            else if (map == 2) row = slot_token[sr] / k;
            else row = r;
            v = src[row * C + c];
        }
        tile[rr][tx] = v;
    }
    __syncthreads();
    for (int cc = ty; cc < 64; cc += 4) {
        const int c = c0 + cc, r = r0 + tx;
        if (c < C && r < Kp) {
            const unsigned short v = tile[tx][cc];
            unsigned short *o = out + ((int64_t)e * C + c) * ((int64_t)copies * Kp) + r;
            for (int q = 0; q < copies; ++q)
                o[(int64_t)q * Kp] = v;
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
                                                 int k, float *__restrict__ dx) {
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
        const float s = ds[a];
        const f32x4 w = *reinterpret_cast<const f32x4 *>(Wg + (int64_t)idx[a] * d + c);
        acc += s * w;
    }
    *reinterpret_cast<f32x4 *>(dx + t * d + c) = acc;
}

}  // namespace

hipError_t launch_combine_backward(const void *dout, const float *Yf, const float *gate,
                                   const int32_t *slot, int64_t N, int64_t d, int k, void *dY,
                                   float *ds, hipStream_t s) {
    if (N == 0)
        return hipSuccess;
    hipLaunchKernelGGL(combine_backward_kernel, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s,
                       static_cast<const unsigned short *>(dout), Yf, gate, slot, (int)N, (int)d,
                       k, static_cast<unsigned short *>(dY), ds);
    return hipGetLastError();
}

hipError_t launch_ds_split(const float *ds, const int32_t *idx, int64_t N, int64_t Np, int E,
                           int k, void *dsT3, hipStream_t s) {
    const int64_t n = (int64_t)E * Np;
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(ds_split_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, ds,
                       idx, (int)N, (int)Np, E, k, static_cast<unsigned short *>(dsT3));
    return hipGetLastError();
}

hipError_t launch_transpose_rows(const void *src, int64_t C, int64_t ceff, const int32_t *used,
                                 int64_t nrows, const int32_t *slot_token, int k, int map,
                                 int64_t Kp, int copies, int batch, void *out, hipStream_t s) {
    if (Kp == 0 || C == 0 || batch == 0)
        return hipSuccess;
    hipLaunchKernelGGL(transpose_rows_kernel,
                       dim3((unsigned)((Kp + 63) / 64), (unsigned)((C + 63) / 64),
                            (unsigned)batch),
                       dim3(256), 0, s, static_cast<const unsigned short *>(src), (int)C, ceff,
                       used, (int)nrows, slot_token, k, map, (int)Kp, copies,
                       static_cast<unsigned short *>(out));
    return hipGetLastError();
}

hipError_t launch_dx(const float *dXa, const float *ds, const int32_t *idx, const int32_t *slot,
                     const float *Wg, int64_t N, int64_t d, int k, float *dx, hipStream_t s) {
    const int64_t n = N * (d / 4);
    if (n == 0)
        return hipSuccess;
    hipLaunchKernelGGL(dx_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, dXa, ds,
                       idx, slot, Wg, N, (int)d, k, dx);
    return hipGetLastError();
}

}  // namespace moe
