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
// Assignments are taken in (j, t) order in chunks of 4096, in three passes:
//  1. chunk_hist_kernel: per chunk, the count of assignments to each expert
//     (integer adds, so their order does not matter) and, when asked for, the
//     sum of their gates in a fixed order;
//  2. chunk_scan_kernel: one thread per expert turns the counts into
//     exclusive prefixes over the chunks, in chunk order, and finishes the
//     plan: used[], the router statistics and the GEMM tile schedule;
//  3. dispatch_kernel: per chunk, each wave ranks its 4 x 64 assignments
//     against the lanes holding the same id (found with one ballot per id
//     bit), the per-wave counts become exclusive prefixes across the 16 waves,
//     and the slot is the earlier chunks' count plus the rank in the chunk.
// A call with a single chunk runs pass 3 alone (it finishes the plan itself);
// one with at most 32 chunks and no gate sums asked for runs a single pass
// (dispatch_fused_kernel) in which every workgroup recounts the earlier
// chunks.
// Ranks are positional, never taken from atomics, so the plan is the same on
// every run.
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

__device__ __forceinline__ int id_bits(int E) { return E > 1 ? 32 - __clz(E - 1) : 0; }

// (choice, token) order: p = j*N + t; assignment id a = t*k + j
__device__ __forceinline__ int assignment_of(int p, int N, int k) {
    const int j = p / N;
    return (p - j * N) * k + j;
}

// This thread's assignments of chunk p0 (item s: wave w's group s, lane),
// with their expert ids (-1: past the end or not an expert id).
__device__ __forceinline__ void load_chunk(const int32_t *__restrict__ idx, int64_t p0, int total,
                                           int N, int k, int E, int (&cur_a)[kItems],
                                           int (&cur_e)[kItems]) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
        const int64_t p = p0 + w * (kItems * 64) + s * 64 + lane;
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
__device__ void chunk_counts(const int (&cur_a)[kItems], const int (&cur_e)[kItems], int E,
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
    for (int s = 0; s < kItems; ++s) {
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
    const int64_t p0 = (int64_t)blockIdx.x * kPhase;
    int cur_a[kItems], cur_e[kItems];
    load_chunk(idx, p0, total, N, k, E, cur_a, cur_e);
    for (int e = threadIdx.x; e < E; e += kThreads)
        cnt[e] = 0;
    chunk_counts(cur_a, cur_e, E, gate, cnt, gsum, wsum, wg);
    for (int e = threadIdx.x; e < E; e += kThreads) {
        hist[(int64_t)blockIdx.x * E + e] = cnt[e];
        if (gate)
            gpart[(int64_t)blockIdx.x * E + e] = gsum[e];
    }
}

// Pass 2 (one workgroup of 256 threads): hist[c][e] becomes the exclusive
// prefix over chunks c' < c, in chunk order; the totals finish the plan.
__global__ __launch_bounds__(256) void chunk_scan_kernel(
    int32_t *__restrict__ hist, const float *__restrict__ gpart, int chunks, int E, int ceff,
    int32_t *__restrict__ used, int32_t *__restrict__ tiles, int32_t *__restrict__ demand,
    int32_t *__restrict__ drops, float *__restrict__ gate_sum) {
    __shared__ int cnt[kMaxExperts];
    __shared__ float gsum[kMaxExperts];
    const int e = threadIdx.x;
    if (e < E) {
        constexpr int U = 8;   // loads of U chunks in flight
        int run = 0;
        float gs = 0.f;
        for (int c0 = 0; c0 < chunks; c0 += U) {
            int h[U];
            float g[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                h[u] = c0 + u < chunks ? hist[(int64_t)(c0 + u) * E + e] : 0;
                g[u] = (gate_sum && c0 + u < chunks) ? gpart[(int64_t)(c0 + u) * E + e] : 0.f;
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (c0 + u < chunks) {
                    hist[(int64_t)(c0 + u) * E + e] = run;
                    run += h[u];
                    gs += g[u];
                }
            }
        }
        cnt[e] = run;
        gsum[e] = gs;
    }
    __syncthreads();
    finish_plan(cnt, gsum, E, ceff, used, tiles, demand, drops, gate_sum);
}

// Pass 3: the slots of chunk c. excl: the exclusive prefixes of pass 2 (NULL
// for a single chunk, which then also finishes the plan).
__global__ __launch_bounds__(kThreads) void dispatch_kernel(
    const int32_t *__restrict__ idx, const float *__restrict__ gate, int N, int E, int k,
    int ceff, const int32_t *__restrict__ excl, int32_t *__restrict__ slot,
    int32_t *__restrict__ used, int32_t *__restrict__ slot_token, int32_t *__restrict__ tiles,
    int32_t *__restrict__ demand, int32_t *__restrict__ drops, float *__restrict__ gate_sum) {
    __shared__ int base[kMaxExperts];                     // assignments of earlier chunks
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];    // per-wave counts, then prefixes
    __shared__ int cnt[kMaxExperts];                      // single chunk: its counts
    __shared__ float gsum[kMaxExperts];
    __shared__ float wg[kWavesPerBlock * 64];

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int total = N * k;   // < 2^31
    const int nbits = id_bits(E);
    const int64_t p0 = (int64_t)blockIdx.x * kPhase;   // this workgroup's chunk

    int cur_a[kItems], cur_e[kItems];
    load_chunk(idx, p0, total, N, k, E, cur_a, cur_e);
    for (int e = tid; e < E; e += kThreads) {
        base[e] = excl ? excl[(int64_t)blockIdx.x * E + e] : 0;
        cnt[e] = 0;
    }
    for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
        wcnt[i] = 0;
    if (!excl) {
        // single chunk: its counts and gate sums finish the plan (wsum
        // borrows wcnt, which is zeroed again below)
        chunk_counts(cur_a, cur_e, E, gate_sum ? gate : nullptr, cnt, gsum,
                     reinterpret_cast<float *>(wcnt), wg);
        finish_plan(cnt, gsum, E, ceff, used, tiles, demand, drops, gate_sum);
        for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
            wcnt[i] = 0;
    }
    __syncthreads();

    // rank of each assignment among the wave's earlier ones with its id
    int my_r[kItems];
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
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
        const int c = e < E ? wcnt[ww * E + e] : 0;
        const int b0 = e < E ? base[e] : 0;
        int incl = c;
#pragma unroll
        for (int off = 1; off < kWavesPerBlock; off <<= 1) {
            const int o = __shfl_up(incl, off, kWavesPerBlock);
            if (ww >= off)
                incl += o;
        }
        if (e < E)
            wcnt[ww * E + e] = b0 + incl - c;
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
}

__global__ void fill_i32_kernel(int32_t *p, int64_t n, int32_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = v;
}

// One-launch plan for at most kFusedChunks chunks when no gate sums are
// asked for: every workgroup counts, per expert, the assignments of the
// earlier chunks itself (reading the ids in their [N, k] layout, 4 per load,
// and keeping those whose (choice, token) position lies before its chunk;
// integer adds, so their order does not matter), then ranks its chunk as
// dispatch_kernel does; the last workgroup, which also counts its own chunk,
// finishes the plan. The slots, used counts and tile schedule are those of
// the three-pass plan.
constexpr int kFusedChunks = 32;

__global__ __launch_bounds__(kThreads) void dispatch_fused_kernel(
    const int32_t *__restrict__ idx, int N, int E, int k, int ceff, int32_t *__restrict__ slot,
    int32_t *__restrict__ used, int32_t *__restrict__ slot_token, int32_t *__restrict__ tiles,
    int32_t *__restrict__ demand, int32_t *__restrict__ drops) {
    __shared__ int base[kMaxExperts];
    __shared__ int wcnt[kWavesPerBlock * kMaxExperts];
    __shared__ int cnt[kMaxExperts];
    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const uint64_t lt = lanemask_lt();
    const int total = N * k;
    const int nbits = id_bits(E);
    const int64_t p0 = (int64_t)blockIdx.x * kPhase;
    const bool last = blockIdx.x == gridDim.x - 1;
    int cur_a[kItems], cur_e[kItems];
    load_chunk(idx, p0, total, N, k, E, cur_a, cur_e);
    for (int e = tid; e < E; e += kThreads) {
        base[e] = 0;
        cnt[e] = 0;
    }
    for (int i = tid; i < kWavesPerBlock * E; i += kThreads)
        wcnt[i] = 0;
    __syncthreads();
    // earlier chunks: assignments a = t*k + j with j*N + t < p0 (p0 > 0 only)
    if (p0 > 0) {
        const bool vec = ((uintptr_t)idx & 15) == 0;
        for (int a0 = tid * 4; a0 < total; a0 += kThreads * 4) {
            int ev[4];
            if (vec && a0 + 4 <= total) {
                const u32x4 v = *reinterpret_cast<const u32x4 *>(idx + a0);
                ev[0] = (int)v[0]; ev[1] = (int)v[1]; ev[2] = (int)v[2]; ev[3] = (int)v[3];
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    ev[q] = a0 + q < total ? idx[a0 + q] : -1;
            }
            int t = a0 / k, j = a0 - t * k;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = ev[q];
                if (a0 + q < total && e >= 0 && e < E && (int64_t)j * N + t < p0)
                    atomicAdd(&base[e], 1);
                if (++j == k) {
                    j = 0;
                    ++t;
                }
            }
        }
    }
    __syncthreads();
    // rank of each assignment among the wave's earlier ones with its id
    int my_r[kItems];
#pragma unroll
    for (int s = 0; s < kItems; ++s) {
        const int e = cur_e[s];
        if (cur_a[s] >= 0 && e < 0)
            slot[cur_a[s]] = -1;
        const uint64_t m = match_ids(e, e >= 0, nbits);
        const int before = __popcll(m & lt);
        my_r[s] = e >= 0 ? wcnt[w * E + e] + before : 0;
        if (e >= 0 && before == 0)
            wcnt[w * E + e] += __popcll(m);
    }
    __syncthreads();
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
                cnt[e] = b0 + incl;   // assignments up to the end of this chunk
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
        const bool kept = r < ceff;
        slot[a] = kept ? r : -1;
        if (kept)
            slot_token[(int64_t)e * ceff + r] = a;
    }
    if (last)
        finish_plan(cnt, nullptr, E, ceff, used, tiles, demand, drops, nullptr);
}

}  // namespace

int64_t dispatch_chunks(int64_t N, int k) { return (N * k + kPhase - 1) / kPhase; }

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
    if (chunks <= kFusedChunks && !gate_sum) {
        hipLaunchKernelGGL(dispatch_fused_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, s,
                           idx, (int)N, E, k, (int)ceff, slot, used, slot_token, tiles, demand,
                           drops);
        return hipGetLastError();
    }
    int32_t *hist = nullptr;
    if (chunks > 1) {
        hist = static_cast<int32_t *>(ws);
        float *gpart = reinterpret_cast<float *>(static_cast<char *>(ws) +
                                                 (size_t)(chunks * E * 4 + 255) / 256 * 256);
        hipLaunchKernelGGL(chunk_hist_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, s, idx,
                           g, (int)N, E, k, hist, gpart);
        hipError_t err = hipGetLastError();
        if (err != hipSuccess)
            return err;
        hipLaunchKernelGGL(chunk_scan_kernel, dim3(1), dim3(256), 0, s, hist,
                           (const float *)gpart, (int)chunks, E, (int)ceff, used, tiles, demand,
                           drops, gate_sum);
        err = hipGetLastError();
        if (err != hipSuccess)
            return err;
    }
    hipLaunchKernelGGL(dispatch_kernel, dim3((unsigned)chunks), dim3(kThreads), 0, s, idx, g,
                       (int)N, E, k, (int)ceff, (const int32_t *)hist, slot, used, slot_token,
                       tiles, demand, drops, gate_sum);
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
