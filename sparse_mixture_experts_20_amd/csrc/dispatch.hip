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
// workgroup walks the k*N assignments in (j, t) order, 4096 per phase (the
// next phase's ids are loaded while the current one is ranked): each wave
// ranks its 4 x 64 assignments against the lanes holding the same id, found
// with one ballot per id bit, the per-wave counts are turned into exclusive
// prefixes across the 16 waves in LDS, and a running per-expert base carries
// the count into the next phase. Ranks are positional, never taken from
// atomics, so the plan is the same on every run.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / kWave;   // 16
constexpr int kItems = 4;                           // 64-assignment groups per wave per phase
constexpr int kPhase = kThreads * kItems;           // 4096 assignments per phase

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
    __shared__ int base[kMaxExperts];                     // assignments counted so far
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];    // per-wave counts, then prefixes

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int total = N * k;   // < 2^31
    const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;

    for (int e = tid; e < E; e += kThreads)
        base[e] = 0;

    // (choice, token) order: p = j*N + t; assignment id a = t*k + j
    auto load_phase = [&](int64_t p0, int (&ids)[kItems], int (&as)[kItems]) {
#pragma unroll
        for (int s = 0; s < kItems; ++s) {
            const int64_t p = p0 + w * (kItems * 64) + s * 64 + lane;
            const int pc = p < total ? (int)p : 0;
            const int j = pc / N;
            as[s] = (pc - j * N) * k + j;
            ids[s] = idx[as[s]];
        }
    };
    int cur_e[kItems], cur_a[kItems];
    load_phase(0, cur_e, cur_a);

    for (int64_t p0 = 0; p0 < total; p0 += kPhase) {
        int nxt_e[kItems], nxt_a[kItems];
        const bool more = p0 + kPhase < total;
        if (more)
            load_phase(p0 + kPhase, nxt_e, nxt_a);   // in flight during this phase

        for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
            wcnt[i] = 0;
        __syncthreads();

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
        // per expert: exclusive prefix over the waves, starting at the base
        for (int e = tid; e < E; e += kThreads) {
            int run = base[e];
            for (int ww = 0; ww < kWavesPerBlock; ++ww) {
                const int c = wcnt[ww * E + e];
                wcnt[ww * E + e] = run;
                run += c;
            }
            base[e] = run;
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
        __syncthreads();
        if (more) {
#pragma unroll
            for (int s = 0; s < kItems; ++s) {
                cur_e[s] = nxt_e[s];
                cur_a[s] = nxt_a[s];
            }
        }
    }

    for (int e = tid; e < E; e += kThreads)
        used[e] = base[e] < ceff ? base[e] : ceff;
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
