// Combine: out[t] = sum over kept choices j of g[t, j] * Y[t*k + j].
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 11 (each expert output is scaled by its gate) and STEP 12 (the scaled
// outputs are summed); nanoMoE slides 38-40 (the combine weights are the raw
// gates, so a dropped assignment contributes nothing and a token whose every
// choice was dropped gets 0).
//
// Each thread owns a VEC-wide column slice of one token row: it reads the k
// expert rows of that token (stored contiguously, assignment-major; bf16 or
// fp32), accumulates in fp32 in choice order and rounds once to the output
// type. A pure streaming kernel: k*d*sizeof(Y) bytes read per token and
// d*sizeof(out) bytes written. bf16 rows are read 8 columns (16 bytes) at a
// time. The slots and gates of up to kGroup choices are loaded together,
// then the rows of the kept ones together (two memory round trips per group
// rather than two per choice); a dropped assignment's row is neither read
// nor added.
#include "common.hpp"

namespace moe {
namespace {

template <int VEC>
__device__ __forceinline__ void load_row(const float *y, float (&v)[VEC]) {
    if constexpr (VEC % 4 == 0) {
#pragma unroll
        for (int q = 0; q < VEC / 4; ++q) {
            const f32x4 a = *reinterpret_cast<const f32x4 *>(y + 4 * q);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                v[4 * q + i] = a[i];
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            v[i] = y[i];
    }
}

template <int VEC>
__device__ __forceinline__ void load_row(const unsigned short *y, float (&v)[VEC]) {
    if constexpr (VEC == 8) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(y);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(a[i] << 16);
            v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < VEC; ++i)
            v[i] = bf16_bits_to_f32(y[i]);
    }
}

constexpr int kGroup = 4;   // choices whose loads are in flight together

template <typename YT, bool BF16, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ Y,
                                                      const float *__restrict__ gate,
                                                      const int32_t *__restrict__ slot,
                                                      int64_t N, int d, int k,
                                                      void *__restrict__ out) {
    const int cols = d / VEC;
    const int64_t total = N * cols;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = i / cols;
        const int c = (int)(i - t * cols) * VEC;
        float acc[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            acc[v] = 0.f;
        for (int j0 = 0; j0 < k; j0 += kGroup) {
            bool kept[kGroup];
            float g[kGroup], y[kGroup][VEC];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                // (past the token's last choice: its last assignment, not added)
                const int64_t a = t * k + (j0 + u < k ? j0 + u : k - 1);
                kept[u] = j0 + u < k && slot[a] >= 0;
                g[u] = gate[a];
            }
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (kept[u])
                    load_row<VEC>(Y + (t * k + j0 + u) * d + c, y[u]);
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (kept[u]) {
#pragma unroll
                    for (int v = 0; v < VEC; ++v)
                        acc[v] += g[u] * y[u][v];
                }
        }
        if (BF16) {
            unsigned short *o = static_cast<unsigned short *>(out) + t * d + c;
            if constexpr (VEC % 4 == 0) {
#pragma unroll
                for (int q = 0; q < VEC / 4; ++q) {
                    u32x2 pk;
                    pk[0] = pack_bf16x2(acc[4 * q], acc[4 * q + 1]);
                    pk[1] = pack_bf16x2(acc[4 * q + 2], acc[4 * q + 3]);
                    *reinterpret_cast<u32x2 *>(o + 4 * q) = pk;
                }
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    o[v] = f32_to_bf16_bits(acc[v]);
            }
        } else {
            float *o = static_cast<float *>(out) + t * d + c;
#pragma unroll
            for (int v = 0; v < VEC; ++v)
                o[v] = acc[v];
        }
    }
}

template <typename YT, bool BF16, int VEC>
hipError_t launch(const void *Y, const float *gate, const int32_t *slot, int64_t N, int64_t d,
                  int k, void *out, hipStream_t s) {
    const int64_t total = N * (d / VEC);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL((combine_kernel<YT, BF16, VEC>), dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<const YT *>(Y), gate, slot, N, (int)d, k, out);
    return hipGetLastError();
}

template <typename YT, int VEC>
hipError_t launch_out(const void *Y, const float *gate, const int32_t *slot, int64_t N, int64_t d,
                      int k, void *out, int out_dtype, hipStream_t s) {
    return out_dtype == 1 ? launch<YT, true, VEC>(Y, gate, slot, N, d, k, out, s)
                          : launch<YT, false, VEC>(Y, gate, slot, N, d, k, out, s);
}

}  // namespace

hipError_t launch_combine(const void *Y, int y_dtype, const float *gate, const int32_t *slot,
                          int64_t N, int64_t d, int k, void *out, int out_dtype, hipStream_t s) {
    if (N == 0 || d == 0)
        return hipSuccess;
    if (y_dtype == 1) {
        if (d % 8 == 0)
            return launch_out<unsigned short, 8>(Y, gate, slot, N, d, k, out, out_dtype, s);
        return launch_out<unsigned short, 1>(Y, gate, slot, N, d, k, out, out_dtype, s);
    }
    if (d % 4 == 0)
        return launch_out<float, 4>(Y, gate, slot, N, d, k, out, out_dtype, s);
    return launch_out<float, 1>(Y, gate, slot, N, d, k, out, out_dtype, s);
}

}  // namespace moe
