// Capacity-limited dispatch plan: the slot of every (choice j, token t)
// assignment is its rank among the assignments to the same expert, counted
// over every token's first choice in token order, then every second choice,
// and so on; ranks at or past the capacity C are dropped.
// nanoMoE slides ("nanoMoEの深層解剖：Mixture of Expertsにおける条件分岐を排除した
// 並列演算実装") 14-23: one-hot of the top-k ids laid out top-1 block first, a
// running count per expert, minus one, masked by rank < capacity; slide 19:
// the top-1 block comes first so first choices have priority.
//
// The running count is never materialised as a [k*N, E] one-hot matrix. One
// workgroup walks the k*N assignments in (j, t) order, 4096 per phase: each
// wave ranks its 4 x 64 assignments with ballots (one ballot per distinct
// expert among the 64 lanes), the per-wave counts are prefix-summed across
// the 16 waves in LDS, and a running per-expert base carries the count into
// the next phase. Ranks are positional, never taken from atomics, so the
// plan is the same on every run.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / kWave;   // 16
constexpr int kItems = 4;                           // 64-assignment groups per wave per phase
constexpr int kPhase = kThreads * kItems;           // 4096 assignments per phase

__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ idx, int N, int E, int k, int ceff,
    int32_t *__restrict__ slot, int32_t *__restrict__ used, int32_t *__restrict__ slot_token,
    int32_t *__restrict__ tiles) {
    __shared__ int base[kMaxExperts];                     // kept+dropped count so far
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];    // per-wave count in this phase

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int64_t total = (int64_t)N * k;

    for (int e = tid; e < E; e += kThreads)
        base[e] = 0;

    for (int64_t p0 = 0; p0 < total; p0 += kPhase) {
        for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
            wcnt[i] = 0;
        __syncthreads();

        int my_e[kItems], my_r[kItems];
#pragma unroll
        for (int s = 0; s < kItems; ++s) {
            const int64_t p = p0 + (int64_t)w * (kItems * 64) + s * 64 + lane;
            int e = -1;
            if (p < total) {
                const int j = (int)(p / N);
                const int64_t t = p - (int64_t)j * N;
                e = idx[t * k + j];
                if (e < 0 || e >= E) {   // not an expert id: the assignment is dropped
                    slot[t * k + j] = -1;
                    e = -1;
                }
            }
            int r = 0;
            uint64_t rem = __ballot(e >= 0);
            while (rem) {
                const int leader = __ffsll((unsigned long long)rem) - 1;
                const int v = __shfl(e, leader);
                const uint64_t m = __ballot(e == v) & rem;
                if (e == v)
                    r = wcnt[w * E + v] + __popcll(m & lt);
                if (lane == leader)
                    wcnt[w * E + v] += __popcll(m);
                rem &= ~m;
            }
            my_e[s] = e;
            my_r[s] = r;
        }
        __syncthreads();

#pragma unroll
        for (int s = 0; s < kItems; ++s) {
            const int e = my_e[s];
            if (e < 0)
                continue;
            int off = base[e];
            for (int ww = 0; ww < w; ++ww)
                off += wcnt[ww * E + e];
            const int r = off + my_r[s];
            const int64_t p = p0 + (int64_t)w * (kItems * 64) + s * 64 + lane;
            const int j = (int)(p / N);
            const int64_t t = p - (int64_t)j * N;
            const int a = (int)(t * k + j);
            const bool kept = r < ceff;   // r < N always, so r < C <=> r < min(C, N)
            slot[a] = kept ? r : -1;
            if (kept)
                slot_token[(int64_t)e * ceff + r] = a;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kThreads) {
            int c = base[e];
            for (int ww = 0; ww < kWavesPerBlock; ++ww)
                c += wcnt[ww * E + e];
            base[e] = c;
        }
        __syncthreads();
    }

    for (int e = tid; e < E; e += kThreads)
        used[e] = base[e] < ceff ? base[e] : ceff;
    __syncthreads();
    if (tid == 0) {
        // tile schedule of the expert kernels: prefix sums of row tiles of 128 and 256
        int a128 = 0, a256 = 0;
        for (int e = 0; e < E; ++e) {
            tiles[e] = a128;
            tiles[E + 1 + e] = a256;
            const int u = base[e] < ceff ? base[e] : ceff;
            a128 += (u + 127) / 128;
            a256 += (u + 255) / 256;
        }
        tiles[E] = a128;
        tiles[2 * E + 1] = a256;
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
    hipLaunchKernelGGL(dispatch_kernel, dim3(1), dim3(kThreads), 0, s, idx, (int)N, E, k,
                       (int)ceff, slot, used, slot_token, tiles);
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
