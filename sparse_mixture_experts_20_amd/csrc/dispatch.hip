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
// Assignments are taken in (j, t) order. A call of at most 4096 of them is
// one chunk, planned by one workgroup (dispatch_kernel<4>): each wave ranks
// its 4 x 64 assignments against the lanes holding the same id (found with
// one ballot per id bit), the per-wave counts become exclusive prefixes
// across the 16 waves, and the workgroup finishes the plan. Larger calls
// take chunks of 1024 (one assignment per thread) in two passes:
//  1. chunk_hist_kernel: per chunk, the count of assignments to each expert
//     (integer adds, so their order does not matter) and, when asked for, the
//     sum of their gates in a fixed order;
//  2. dispatch_kernel<1>: per chunk, the count of each expert's assignments
//     in the earlier chunks (the sum of their counts, four ranges of chunks
//     added by four threads per expert; integers, so the order does not
//     matter), then the ranking of its chunk as above; the last workgroup
//     finishes the plan: used[], the router statistics and the GEMM tile
//     schedule.
// Past 128 chunks the earlier chunks' counts come from chunk_scan_kernel,
// one thread per expert adding the chunks in order, between the two passes.
// Ranks are positional, never taken from atomics, so the plan is the same on
// every run.
#include "common.hpp"

namespace moe {
namespace {

constexpr int kThreads = 1024;
constexpr int kWavesPerBlock = kThreads / kWave;   // 16
constexpr int kOneChunk = kThreads * 4;             // a call planned by one workgroup
constexpr int kChunk = kThreads;                    // assignments per chunk of larger calls
constexpr int kInlineChunks = 128;                  // the ranking pass sums earlier chunks itself

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

__device__ __forceinline__ int id_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// (choice, token) order: p = j*N + t; assignment id a = t*k + j
__device__ __forceinline__ int assignment_of(int p, int N, int k) {
    const int j = p / N;
    return (p - j * N) * k + j;
}

// This thread's assignments of the chunk starting at p0 (item s: wave w's
// group s, lane), with their expert ids (-1: past the end or not an id).
template <int ITEMS>
__device__ __forceinline__ void load_chunk(const int32_t *__restrict__ idx, int64_t p0, int total,
                                           int N, int k, int E, int (&cur_a)[ITEMS],
                                           int (&cur_e)[ITEMS]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int64_t p = p0 + w * (ITEMS * 64) + s * 64 + lane;
        cur_a[s] = p < total ? assignment_of((int)p, N, k) : -1;
        const int e = cur_a[s] >= 0 ? idx[cur_a[s]] : -1;
        cur_e[s] = (e >= 0 && e < E) ? e : -1;
    }
}

// Count of each expert's assignments in this chunk into cnt[e] (LDS, zeroed
// by the caller), and, with gate != NULL, the sum of their gates into
// gsum[e] in a fixed order: lanes in order within each 64-assignment group
// (summed by the group's first lane with that id), groups in order within a
// wave, then the waves in order. wsum: LDS scratch [16][E] floats, wg: [16][64].
template <int ITEMS>
__device__ void chunk_counts(const int (&cur_a)[ITEMS], const int (&cur_e)[ITEMS], int E,
                             const float *__restrict__ gate, int *cnt, float *gsum,
                             float *wsum, float *wg) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int nbits = id_bits(E);
    if (gate)
        for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
            wsum[i] = 0.f;
    __syncthreads();
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int e = cur_e[s];
        const uint64_t m = match_ids(e, e >= 0, nbits);
        const bool lead = e >= 0 && __popcll(m & lt) == 0;
        if (lead)
            atomicAdd(&cnt[e], __popcll(m));
        if (gate) {
            wg[w * 64 + lane] = e >= 0 ? gate[cur_a[s]] : 0.f;
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            if (lead) {
                float acc = 0.f;
                for (uint64_t mm = m; mm; mm &= mm - 1)
                    acc += wg[w * 64 + __ffsll((unsigned long long)mm) - 1];
                wsum[w * E + e] += acc;
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            __builtin_amdgcn_wave_barrier();
        }
    }
    __syncthreads();
    if (gate)
        for (int e = tid; e < E; e += kThreads) {
            float acc = 0.f;
            for (int ww = 0; ww < kWavesPerBlock; ++ww)
                acc += wsum[ww * E + e];
            gsum[e] = acc;
        }
    __syncthreads();
}

// The plan's totals from the per-expert counts cnt[] (LDS, complete): used[],
// the router statistics (each NULL when not asked for; gsum[] in LDS when
// gate_sum is) and the tile schedule of the expert kernels: exclusive prefix
// sums of row tiles of 128 and 256 over the experts, 4 experts per lane of
// wave 0. Any block size >= 64 threads.
__device__ void finish_plan(const int *cnt, const float *gsum, int E, int ceff,
                            int32_t *__restrict__ used, int32_t *__restrict__ tiles,
                            int32_t *__restrict__ demand, int32_t *__restrict__ drops,
                            float *__restrict__ gate_sum) {
    const int tid = threadIdx.x, lane = tid & 63;
    for (int e = tid; e < E; e += blockDim.x) {
        const int c = cnt[e], u = c < ceff ? c : ceff;
        used[e] = u;
        if (demand)
            demand[e] = c;
        if (drops)
            drops[e] = c - u;
        if (gate_sum)
            gate_sum[e] = gsum[e];
    }
    if (tid < kWave) {
        constexpr int Q = kMaxExperts / kWave;
        int c128[Q], c256[Q], s128 = 0, s256 = 0;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int e = tid * Q + q;
            const int u = e < E ? (cnt[e] < ceff ? cnt[e] : ceff) : 0;
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

// Pass 1: per chunk c, hist[c][e] = its assignments to expert e and, with
// gate, gpart[c][e] = the sum of their gates.
__global__ __launch_bounds__(kThreads) void chunk_hist_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ gate, int N, int E, int k,
    int32_t *__restrict__ hist, float *__restrict__ gpart) {
    __shared__ int cnt[kMaxExperts];
    __shared__ float gsum[kMaxExperts];
    __shared__ float wsum[kWavesPerBlock * kMaxExperts];
    __shared__ float wg[kWavesPerBlock * 64];
    const int total = N * k;
    const int64_t p0 = (int64_t)blockIdx.x * kChunk;
    int cur_a[1], cur_e[1];
    load_chunk<1>(idx, p0, total, N, k, E, cur_a, cur_e);
    for (int e = threadIdx.x; e < E; e += kThreads)
        cnt[e] = 0;
    chunk_counts<1>(cur_a, cur_e, E, gate, cnt, gsum, wsum, wg);
    for (int e = threadIdx.x; e < E; e += kThreads) {
        hist[(int64_t)blockIdx.x * E + e] = cnt[e];
        if (gate)
            gpart[(int64_t)blockIdx.x * E + e] = gsum[e];
    }
}

// Between the passes, past kInlineChunks chunks (one workgroup of 256
// threads): hist[c][e] becomes the exclusive prefix over chunks c' < c, in
// chunk order.
__global__ __launch_bounds__(256) void chunk_scan_kernel(int32_t *__restrict__ hist, int chunks,
                                                         int E) {
    const int e = threadIdx.x;
    if (e >= E)
        return;
    constexpr int U = 8;   // loads of U chunks in flight
    int run = 0;
    for (int c0 = 0; c0 < chunks; c0 += U) {
        int h[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            h[u] = c0 + u < chunks ? hist[(int64_t)(c0 + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c0 + u < chunks) {
                hist[(int64_t)(c0 + u) * E + e] = run;
                run += h[u];
            }
        }
    }
}

// The slots of one chunk (ITEMS = 4: a call of one chunk of up to 4096
// assignments, which also counts itself and finishes the plan; ITEMS = 1:
// chunk blockIdx.x of 1024 of a larger call, after pass 1). hist: the
// per-chunk counts of pass 1 (the ranking sums those of the earlier chunks),
// or, with scanned, their exclusive prefixes; gpart: the per-chunk gate sums
// of pass 1 (read by the last workgroup when gate_sum is asked for).
template <int ITEMS>
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ gate, int N, int E, int k,
    int ceff, const int32_t *__restrict__ hist, const float *__restrict__ gpart, int scanned,
    int32_t *__restrict__ slot, int32_t *__restrict__ used, int32_t *__restrict__ slot_token,
    int32_t *__restrict__ tiles, int32_t *__restrict__ demand, int32_t *__restrict__ drops,
    float *__restrict__ gate_sum) {
    constexpr int kParts = kThreads / kMaxExperts;        // threads per expert in the sums
    __shared__ int base[kMaxExperts];                     // assignments of earlier chunks
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];    // per-wave counts, then prefixes
    __shared__ int cnt[kMaxExperts];                      // totals up to this chunk's end
    __shared__ float gsum[kMaxExperts];
    __shared__ float wg[kWavesPerBlock * 64];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int total = N * k;   // < 2^31
    const int nbits = id_bits(E);
    const int c = blockIdx.x;
    const int64_t p0 = (int64_t)c * (ITEMS * kThreads);   // this workgroup's chunk
    const bool last = c == (int)gridDim.x - 1;

    int cur_a[ITEMS], cur_e[ITEMS];
    load_chunk<ITEMS>(idx, p0, total, N, k, E, cur_a, cur_e);
    for (int e = tid; e < E; e += kThreads)
        cnt[e] = 0;
    if constexpr (ITEMS == 1) {
        // the earlier chunks' counts: kParts consecutive ranges of chunks,
        // one thread each, added into base (integers: any order)
        int *part = wcnt;   // [kParts][kMaxExperts], zeroed again below
        const int e = tid % kMaxExperts, q = tid / kMaxExperts;
        if (e < E) {
            int acc = 0;
            if (scanned) {
                if (q == 0)
                    acc = hist[(int64_t)c * E + e];
            } else {
                const int c0 = q * c / kParts, c1 = (q + 1) * c / kParts;
                constexpr int U = 16;
                for (int cc = c0; cc < c1; cc += U) {
                    int h[U];
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        h[u] = cc + u < c1 ? hist[(int64_t)(cc + u) * E + e] : 0;
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        acc += h[u];
                }
            }
            part[q * kMaxExperts + e] = acc;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kThreads) {
            int b = 0;
#pragma unroll
            for (int qq = 0; qq < kParts; ++qq)
                b += part[qq * kMaxExperts + ee];
            base[ee] = b;
        }
        __syncthreads();
    } else {
        for (int e = tid; e < E; e += kThreads)
            base[e] = 0;
        // one chunk: its counts and gate sums finish the plan (wsum borrows
        // wcnt, which is zeroed again below)
        chunk_counts<ITEMS>(cur_a, cur_e, E, gate_sum ? gate : nullptr, cnt, gsum,
                            reinterpret_cast<float *>(wcnt), wg);
        finish_plan(cnt, gsum, E, ceff, used, tiles, demand, drops, gate_sum);
    }
    for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
        wcnt[i] = 0;
    __syncthreads();

    // rank of each assignment among the wave's earlier ones with its id
    int my_r[ITEMS];
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
        const int e = cur_e[s];
        if (cur_a[s] >= 0 && e < 0)   // not an expert id: the assignment is dropped
            slot[cur_a[s]] = -1;
        const uint64_t m = match_ids(e, e >= 0, nbits);
        const int before = __popcll(m & lt);
        my_r[s] = e >= 0 ? wcnt[w * E + e] + before : 0;
        if (e >= 0 && before == 0)
            wcnt[w * E + e] += __popcll(m);   // one lane per distinct id
    }
    __syncthreads();
    // per expert: exclusive prefix over the waves, starting at the base; the
    // wave counts of an expert sit on kWavesPerBlock lanes of one wave and are
    // scanned with shuffles (kThreads / kWavesPerBlock experts per pass)
    static_assert((kWavesPerBlock & (kWavesPerBlock - 1)) == 0 && kWavesPerBlock <= kWave,
                  "one power-of-two lane group per expert");
    for (int e0 = 0; e0 < E; e0 += kThreads / kWavesPerBlock) {
        const int e = e0 + tid / kWavesPerBlock, ww = tid % kWavesPerBlock;
        const int cw = e < E ? wcnt[ww * E + e] : 0;
        const int b0 = e < E ? base[e] : 0;
        int incl = cw;
#pragma unroll
        for (int off = 1; off < kWavesPerBlock; off <<= 1) {
            const int o = __shfl_up(incl, off, kWavesPerBlock);
            if (ww >= off)
                incl += o;
        }
        if (e < E) {
            wcnt[ww * E + e] = b0 + incl - cw;
            if (ITEMS == 1 && ww == kWavesPerBlock - 1)
                cnt[e] = b0 + incl;   // assignments up to the end of this chunk
        }
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < ITEMS; ++s) {
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
    if (ITEMS != 1 || !last)
        return;
    if (gate_sum) {
        // gate sums of all chunks: kParts consecutive ranges, each in chunk
        // order, then the ranges in order
        float *gp = reinterpret_cast<float *>(wcnt);   // ranking done: free
        __syncthreads();
        const int e = tid % kMaxExperts, q = tid / kMaxExperts;
        const int nc = (int)gridDim.x;
        if (e < E) {
            float acc = 0.f;
            const int c0 = q * nc / kParts, c1 = (q + 1) * nc / kParts;
            constexpr int U = 8;   // loads in flight, added in chunk order
            for (int cc = c0; cc < c1; cc += U) {
                float h[U];
#pragma unroll
                for (int u = 0; u < U; ++u)
                    h[u] = cc + u < c1 ? gpart[(int64_t)(cc + u) * E + e] : 0.f;
#pragma unroll
                for (int u = 0; u < U; ++u)
                    if (cc + u < c1)
                        acc += h[u];
            }
            gp[q * kMaxExperts + e] = acc;
        }
        __syncthreads();
        for (int ee = tid; ee < E; ee += kThreads) {
            float g = gp[ee];
#pragma unroll
            for (int qq = 1; qq < kParts; ++qq)
                g += gp[qq * kMaxExperts + ee];
            gsum[ee] = g;
        }
    }
    __syncthreads();
    finish_plan(cnt, gsum, E, ceff, used, tiles, demand, drops, gate_sum);
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

}  // namespace

int64_t dispatch_chunks(int64_t N, int k) {
    const int64_t total = N * k;
    return total <= kOneChunk ? (total > 0 ? 1 : 0) : (total + kChunk - 1) / kChunk;
}

size_t dispatch_workspace_bytes(int64_t N, int E, int k) {
    const int64_t chunks = dispatch_chunks(N, k);
    if (chunks <= 1)
        return 0;
    return 2 * ((size_t)(chunks * E * 4 + 255) / 256 * 256);
}

hipError_t launch_dispatch(const int32_t *idx, const float *gate, int64_t N, int E, int k,
                           int64_t ceff, int32_t *slot, int32_t *used, int32_t *slot_token,
                           int32_t *tiles, int32_t *demand, int32_t *drops, float *gate_sum,
                           void *ws, hipStream_t s) {
    const int64_t chunks = dispatch_chunks(N, k);
    if (chunks == 0)
        return hipSuccess;
    const float *g = gate_sum ? gate : nullptr;
    if (chunks == 1) {
        hipLaunchKernelGGL(dispatch_kernel<4>, dim3(1), dim3(kThreads), 0, s, idx, g, (int)N, E,
                           k, (int)ceff, (const int32_t *)nullptr, (const float *)nullptr, 0,
                           slot, used, slot_token, tiles, demand, drops, gate_sum);
        return hipGetLastError();
    }
    int32_t *hist = static_cast<int32_t *>(ws);
    float *gpart = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                             (size_t)(chunks * E * 4 + 255) / 256 * 256);
    hipLaunchKernelGGL(chunk_hist_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, s, idx, g,
                       (int)N, E, k, hist, gpart);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess)
        return err;
    const int scanned = chunks > kInlineChunks;
    if (scanned) {
        hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(256), 0, s, hist, (int)chunks, E);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(dispatch_kernel<1>, dim3((unsigned)chunks), dim3(kThreads), 0, s, idx, g,
                       (int)N, E, k, (int)ceff, (const int32_t *)hist, (const float *)gpart,
                       scanned, slot, used, slot_token, tiles, demand, drops, gate_sum);
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
