// Combine: out[t] = sum over kept choices j of g[t, j] * Y[t*k + j].
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 11 (each expert output is scaled by its gate) and STEP 12 (the scaled
// outputs are summed); nanoMoE slides 38-40 (the combine weights are the raw
// gates, so a dropped assignment contributes nothing and a token whose every
// choice was dropped gets 0).
//
// Each thread owns a 4-wide column slice of one token row: it reads the k
// fp32 expert rows of that token (stored contiguously, assignment-major),
// accumulates in fp32 in choice order and rounds once to the output type.
// A pure streaming kernel: k*d*4 bytes read per token (kept rows only) and
// d * sizeof(out) bytes written.
#include "common.hpp"

namespace moe {
namespace {

template <bool BF16, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ Y,
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
        for (int j = 0; j < k; ++j) {
            const int64_t a = t * k + j;
            if (slot[a] < 0)
                continue;
            const float g = gate[a];
            const float *yr = Y + a * d + c;
            if (VEC == 4) {
                const f32x4 y = *reinterpret_cast<const f32x4 *>(yr);
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[v] += g * y[v];
            } else {
#pragma unroll
                for (int v = 0; v < VEC; ++v)
                    acc[v] += g * yr[v];
            }
        }
        if (BF16) {
            unsigned short *o = static_cast<unsigned short *>(out) + t * d + c;
            if (VEC == 4) {
                u32x2 pk;
                pk[0] = (unsigned)f32_to_bf16_bits(acc[0]) | ((unsigned)f32_to_bf16_bits(acc[1]) << 16);
                pk[1] = (unsigned)f32_to_bf16_bits(acc[2]) | ((unsigned)f32_to_bf16_bits(acc[3]) << 16);
                *reinterpret_cast<u32x2 *>(o) = pk;
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

template <bool BF16, int VEC>
hipError_t launch(const float *Y, const float *gate, const int32_t *slot, int64_t N, int64_t d,
                  int k, void *out, hipStream_t s) {
    const int64_t total = N * (d / VEC);
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL((combine_kernel<BF16, VEC>), dim3((unsigned)blocks), dim3(256), 0, s, Y,
                       gate, slot, N, (int)d, k, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const float *Y, const float *gate, const int32_t *slot, int64_t N,
                          int64_t d, int k, void *out, int out_dtype, hipStream_t s) {
    if (N == 0 || d == 0)
        return hipSuccess;
    const bool vec4 = (d % 4) == 0;
    if (out_dtype == 1)
        return vec4 ? launch<true, 4>(Y, gate, slot, N, d, k, out, s)
                    : launch<true, 1>(Y, gate, slot, N, d, k, out, s);
    return vec4 ? launch<false, 4>(Y, gate, slot, N, d, k, out, s)
                : launch<false, 1>(Y, gate, slot, N, d, k, out, s);
}

}  // namespace moe
