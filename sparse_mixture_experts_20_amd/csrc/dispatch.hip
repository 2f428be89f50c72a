// Capacity-limited dispatch plan: the slot of every (choice j, token t)
// assignment is its rank among the assignments to the same expert, counted
// over every token's first choice in token order, then every second choice,
// and so on; ranks at or past the capacity C are dropped.
// nanoMoE slides ("nanoMoEの深層解剖：Mixture of Expertsにおける条件分岐を排除した
// 並列演算実装") 14-23: one-hot of the top-k ids laid out top-1 block first, a
// running count per expert, minus one, masked by rank < capacity; slide 19:
// the top-1 block comes first so first choices have priority.
//
// The running count is never materialised as a [k*N, E] one-hot matrix.
// Assignments are taken in (j, t) order in chunks of 4096, one workgroup per
// chunk. A workgroup first counts, per expert, the assignments of all earlier
// chunks (a histogram: integer counts, so the order of the additions does not
// matter), then ranks its own chunk: each wave ranks its 4 x 64 assignments
// against the lanes holding the same id, found with one ballot per id bit,
// the per-wave counts are turned into exclusive prefixes across the 16 waves
// in LDS, and the rank is the earlier chunks' count plus the rank inside the
// chunk. Ranks are positional, never taken from atomics, so the plan is the
// same on every run. The last workgroup also writes used[] and the GEMM tile
// schedule. (Re-counting earlier chunks costs the last workgroup one pass
// over k*N ids; it replaces a second kernel and a global scratch.)
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / kWave;   // 16
constexpr int kItems = 4;                           // 64-assignment groups per wave per chunk
constexpr int kPhase = kThreads * kItems;           // 4096 assignments per chunk

// Lanes of the wave holding the same expert id as this lane (among lanes
// with valid ids): one ballot per id bit, O(log E) with no memory traffic.
__device__ __forceinline__ uint64_t match_ids(int e, bool valid, int nbits) {
    uint64_t m = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
        const bool bit = valid && ((e >> b) & 1);
        const uint64_t ones = __ballot(bit);
        m &= bit ? ones : ~ones;
    }
    return valid ? m : 0ull;
}

__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ idx, int N, int E, int k, int ceff,
    int32_t *__restrict__ slot, int32_t *__restrict__ used, int32_t *__restrict__ slot_token,
    int32_t *__restrict__ tiles) {
    __shared__ int base[kMaxExperts];                     // assignments of earlier chunks
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];    // per-wave counts, then prefixes

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int total = N * k;   // < 2^31
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
    const int64_t p0 = (int64_t)blockIdx.x * kPhase;   // this workgroup's chunk

    // (choice, token) order: p = j*N + t; assignment id a = t*k + j
    auto assignment = [&](int p) {
        const int j = p / N;
        return (p - j * N) * k + j;
    };

    // this chunk's ids, loaded first so that they arrive during the count
    int cur_e[kItems], cur_a[kItems];
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
        const int64_t p = p0 + w * (kItems * 64) + s * 64 + lane;
        cur_a[s] = assignment(p < total ? (int)p : 0);
        cur_e[s] = idx[cur_a[s]];
    }

    for (int e = tid; e < E; e += kThreads)
        base[e] = 0;
    for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
        wcnt[i] = 0;
    __syncthreads();
    // histogram of the earlier chunks, 8 ids per thread in flight at a time;
    // with few experts one LDS add per distinct id per wave (adds to one bin
    // would serialise), with many a plain add per id
    constexpr int U = 8;
    for (int p = tid; p < (int)p0; p += kThreads * U) {
        int ev[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int pp = p + u * kThreads;
            ev[u] = pp < (int)p0 ? idx[assignment(pp)] : -1;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = ev[u];
            const bool ok = e >= 0 && e < E;
            if (E > 64) {
                if (ok)
                    atomicAdd(&base[e], 1);
            } else {
                const uint64_t m = match_ids(e, ok, nbits);
                if (ok && __popcll(m & lt) == 0)
                    atomicAdd(&base[e], __popcll(m));
            }
        }
    }

    // rank of each assignment among the wave's earlier ones with its id
    int my_r[kItems];
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
        const int64_t p = p0 + w * (kItems * 64) + s * 64 + lane;
        int e = -1;
        if (p < total) {
            e = cur_e[s];
            if (e < 0 || e >= E) {   // not an expert id: the assignment is dropped
                slot[cur_a[s]] = -1;
                e = -1;
            }
        }
        const uint64_t m = match_ids(e, e >= 0, nbits);
        const int before = __popcll(m & lt);
        my_r[s] = e >= 0 ? wcnt[w * E + e] + before : 0;
        if (e >= 0 && before == 0)
            wcnt[w * E + e] += __popcll(m);   // one lane per distinct id
        cur_e[s] = e;
    }
    __syncthreads();
    // per expert: exclusive prefix over the waves, starting at the base; the
    // wave counts of an expert sit on kWavesPerBlock lanes of one wave and are
    // scanned with shuffles (kThreads / kWavesPerBlock experts per pass)
    static_assert((kWavesPerBlock & (kWavesPerBlock - 1)) == 0 && kWavesPerBlock <= kWave,
                  "one power-of-two lane group per expert");
    for (int e0 = 0; e0 < E; e0 += kThreads / kWavesPerBlock) {
        const int e = e0 + tid / kWavesPerBlock, ww = tid % kWavesPerBlock;
        const int c = e < E ? wcnt[ww * E + e] : 0;
        const int b0 = e < E ? base[e] : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < kWavesPerBlock; off <<= 1) {
            const int o = __shfl_up(incl, off, kWavesPerBlock);
            if (ww >= off)
                incl += o;
        }
        if (e < E) {
            wcnt[ww * E + e] = b0 + incl - c;
            if (ww == kWavesPerBlock - 1)
                base[e] = b0 + incl;   // assignments up to the end of this chunk
        }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
        const int e = cur_e[s];
        if (e < 0)
            continue;
        const int r = wcnt[w * E + e] + my_r[s];
        const int a = cur_a[s];
        const bool kept = r < ceff;   // r < N always, so r < C <=> r < min(C, N)
        slot[a] = kept ? r : -1;
        if (kept)
            slot_token[(int64_t)e * ceff + r] = a;
    }

    if (blockIdx.x != gridDim.x - 1)
        return;
    for (int e = tid; e < E; e += kThreads)
        used[e] = base[e] < ceff ? base[e] : ceff;
    if (tid < kWave) {
        // tile schedule of the expert kernels: exclusive prefix sums of row
        // tiles of 128 and 256 over the experts, 4 experts per lane of wave 0
        constexpr int Q = kMaxExperts / kWave;
        int c128[Q], c256[Q], s128 = 0, s256 = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = tid * Q + q;
            const int u = e < E ? (base[e] < ceff ? base[e] : ceff) : 0;
            c128[q] = (u + 127) / 128;
            c256[q] = (u + 255) / 256;
            s128 += c128[q];
            s256 += c256[q];
        }
        int i128 = s128, i256 = s256;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o128 = __shfl_up(i128, off), o256 = __shfl_up(i256, off);
            if (lane >= off) {
                i128 += o128;
                i256 += o256;
            }
        }
        int x128 = i128 - s128, x256 = i256 - s256;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = tid * Q + q;
            if (e < E) {
                tiles[e] = x128;
                tiles[E + 1 + e] = x256;
            }
            x128 += c128[q];
            x256 += c256[q];
        }
        if (lane == kWave - 1) {
            tiles[E] = i128;
            tiles[2 * E + 1] = i256;
        }
    }
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

}  // namespace

hipError_t launch_dispatch(const int32_t *idx, int64_t N, int E, int k, int64_t ceff,
                           int32_t *slot, int32_t *used, int32_t *slot_token, int32_t *tiles,
                           hipStream_t s) {
    const int64_t chunks = (N * k + kPhase - 1) / kPhase;
    hipLaunchKernelGGL(dispatch_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, s, idx, (int)N,
                       E, k, (int)ceff, slot, used, slot_token, tiles);
    return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int64_t n, int32_t v, hipStream_t s) {
    if (n <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(fill_i32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, n,
                       v);
    return hipGetLastError();
}

}  // namespace moe
