// Combine: out[t] = sum over kept choices j of g[t, j] * Y[t*k + j].
// Page 1 ("Mixture of Experts (MoE) 12段階極小ビジュアル解剖シミュレーター"),
// STEP 11 (each expert output is scaled by its gate) and STEP 12 (the scaled
// outputs are summed); nanoMoE slides 38-40 (the combine weights are the raw
// gates, so a dropped assignment contributes nothing and a token whose every
// choice was dropped gets 0).
//
// Each thread owns a VEC-wide column slice of one token row: it reads the k
// expert rows of that token (stored contiguously, assignment-major; bf16,
// fp32, or the compact fp16 rows with a shift per group of columns that the
// fused layer writes), accumulates in fp32 in choice order and rounds once to the output
// type. A pure streaming kernel: k*d*sizeof(Y) bytes read per token and
// d*sizeof(out) bytes written. Rows are read 8 columns at a time (16 bytes of
// bf16, 32 of fp32). The slots and gates of a group of choices (8 for fp32
// rows, 4 for bf16) are loaded together, then the rows of the kept ones
// together (two memory round trips per group rather than two per choice); a
// dropped assignment's row is neither read nor added.
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

// choices whose loads are in flight together: 4 rows of 16 bytes for bf16
// rows, 8 rows of 32 bytes for fp32 rows (the layer's expert outputs)
template <typename YT>
constexpr int group_of() { return sizeof(YT) == 4 ? 8 : 4; }

template <typename YT, bool BF16, int VEC>
__global__ __launch_bounds__(256) void combine_kernel(const YT *__restrict__ Y,
                                                      const float *__restrict__ gate,
                                                      const int32_t *__restrict__ slot,
                                                      int64_t N, int d, int k,
                                                      void *__restrict__ out) {
    constexpr int kGroup = group_of<YT>();
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

// The same combine over compact rows of Y (the fused layer's own format):
// VEC columns per thread (16: as many bytes per choice as 8 fp32 columns),
// the slots and gates of 8 choices loaded together, then their kept rows
// and shifts, accumulated in choice order. The rows stay fp16 in registers
// until they are added (half the registers of fp32 rows).
template <bool BF16, int VEC, bool OFF32, bool SH8>
__global__ __launch_bounds__(256) void combine_compact_kernel(
    const unsigned short *__restrict__ Y, const signed char *__restrict__ ysh,
    const float *__restrict__ gate, const int32_t *__restrict__ slot, int64_t N, int d, int k,
    void *__restrict__ out) {
    static_assert(VEC % 8 == 0 && kYGroup % VEC == 0, "16-byte loads within one group");
    constexpr int kGroup = 8;
    const int cols = d / VEC;
    const int G = (d + kYGroup - 1) / kYGroup;
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
            float g[kGroup], sc[kGroup];
            u32x4 raw[kGroup][VEC / 8];
#pragma unroll
            for (int u = 0; u < kGroup; ++u) {
                const int64_t a = t * k + (j0 + u < k ? j0 + u : k - 1);
                kept[u] = j0 + u < k && slot[a] >= 0;
                g[u] = gate[a];
            }
            // the shifts of these choices' group are adjacent (token, group,
            // choice order): with k a multiple of 8, one 8-byte load (SH8)
            const int64_t sbase = (t * G + c / kYGroup) * k + j0;
            uint64_t sh8 = 0;
            if constexpr (SH8)
                sh8 = *reinterpret_cast<const uint64_t *>(ysh + sbase);
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (kept[u]) {
                    const int64_t a = t * k + j0 + u;
                    // (OFF32: every offset fits in 32 bits, so a load takes a
                    // 32-bit offset from the uniform base: fewer registers)
                    const unsigned short *yr;
                    if constexpr (OFF32)
                        yr = Y + (uint32_t)((uint32_t)a * (uint32_t)d + (uint32_t)c);
                    else
                        yr = Y + a * d + c;
#pragma unroll
                    for (int q = 0; q < VEC / 8; ++q)
                        raw[u][q] = *reinterpret_cast<const u32x4 *>(yr + 8 * q);
                    const int sh = SH8 ? (int)(signed char)(sh8 >> (8 * u)) : (int)ysh[sbase + u];
                    sc[u] = pow2f(-sh);
                }
#pragma unroll
            for (int u = 0; u < kGroup; ++u)
                if (kept[u]) {
#pragma unroll
                    for (int q = 0; q < VEC / 8; ++q)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const f32x2_t p = unpack_f16x2(raw[u][q][i]);
                            acc[8 * q + 2 * i] += g[u] * (p[0] * sc[u]);
                            acc[8 * q + 2 * i + 1] += g[u] * (p[1] * sc[u]);
                        }
                }
        }
#pragma unroll
        for (int q = 0; q < VEC / 8; ++q) {
            const float *a8 = acc + 8 * q;
            if (BF16) {
                unsigned short *o = static_cast<unsigned short *>(out) + t * d + c + 8 * q;
                *reinterpret_cast<u32x4 *>(o) =
                    u32x4{pack_bf16x2(a8[0], a8[1]), pack_bf16x2(a8[2], a8[3]),
                          pack_bf16x2(a8[4], a8[5]), pack_bf16x2(a8[6], a8[7])};
            } else {
                float *o = static_cast<float *>(out) + t * d + c + 8 * q;
                *reinterpret_cast<f32x4 *>(o) = f32x4{a8[0], a8[1], a8[2], a8[3]};
                *reinterpret_cast<f32x4 *>(o + 4) = f32x4{a8[4], a8[5], a8[6], a8[7]};
            }
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

hipError_t launch_combine_compact(const void *Y, const signed char *ysh, const float *gate,
                                  const int32_t *slot, int64_t N, int64_t d, int k, void *out,
                                  int out_dtype, hipStream_t s) {
    if (N == 0 || d == 0)
        return hipSuccess;
    if (d % 8 != 0)
        return hipErrorInvalidValue;
    auto go = [&](auto kern, int vec) {
        int64_t blocks = (N * (d / vec) + 255) / 256;
        if (blocks > 65536)
            blocks = 65536;
        hipLaunchKernelGGL(kern, dim3((unsigned)blocks), dim3(256), 0, s,
                           static_cast<const unsigned short *>(Y), ysh, gate, slot, N, (int)d, k,
                           out);
        return hipGetLastError();
    };
    // 32-bit element offsets when the rows of Y fit; the shifts of 8 choices
    // in one load when k is a multiple of 8 and they are 8-byte aligned
    const bool off32 = N * k * d < ((int64_t)1 << 32);
    const bool sh8 = k % 8 == 0 && reinterpret_cast<uintptr_t>(ysh) % 8 == 0;
    if (off32 && sh8 && d % 16 == 0)
        return out_dtype == 1 ? go(combine_compact_kernel<true, 16, true, true>, 16)
                              : go(combine_compact_kernel<false, 16, true, true>, 16);
    if (off32 && d % 16 == 0)
        return out_dtype == 1 ? go(combine_compact_kernel<true, 16, true, false>, 16)
                              : go(combine_compact_kernel<false, 16, true, false>, 16);
    if (d % 16 == 0)
        return out_dtype == 1 ? go(combine_compact_kernel<true, 16, false, false>, 16)
                              : go(combine_compact_kernel<false, 16, false, false>, 16);
    return out_dtype == 1 ? go(combine_compact_kernel<true, 8, false, false>, 8)
                          : go(combine_compact_kernel<false, 8, false, false>, 8);
}

hipError_t launch_combine(const void *Y, int y_dtype, const float *gate, const int32_t *slot,
                          int64_t N, int64_t d, int k, void *out, int out_dtype, hipStream_t s) {
    if (N == 0 || d == 0)
        return hipSuccess;
    if (y_dtype == 1) {
        if (d % 8 == 0)
            return launch_out<unsigned short, 8>(Y, gate, slot, N, d, k, out, out_dtype, s);
        return launch_out<unsigned short, 1>(Y, gate, slot, N, d, k, out, out_dtype, s);
    }
    if (d % 8 == 0)
        return launch_out<float, 8>(Y, gate, slot, N, d, k, out, out_dtype, s);
    if (d % 4 == 0)
        return launch_out<float, 4>(Y, gate, slot, N, d, k, out, out_dtype, s);
    return launch_out<float, 1>(Y, gate, slot, N, d, k, out, out_dtype, s);
}

}  // namespace moe
