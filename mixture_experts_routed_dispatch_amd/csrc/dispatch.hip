// dispatch.hip -- deterministic expert-major dispatch on gfx950.
//
// Computes what the nvfp4moe README ("Grouped GEMM", "Training") calls the
// dispatch metadata: per-expert counts, m_indptr [E+1] (empty experts valid),
// gather (routed row -> token), slots ((t, j) -> routed row) and probs (scores
// moved to their rows).  Rows of one expert are ordered by ascending token,
// i.e. a stable counting sort of the flattened (t, j) list by expert id.
//
// Two launches, no global atomics on the ordering, so the result is
// bit-identical run to run:
//   1. count: each workgroup owns a chunk of kDispatchChunk consecutive
//      entries and writes its per-expert histogram (LDS atomics; only counts,
//      so their order does not matter).
//   2. place: each workgroup re-derives the global exclusive scan and the
//      number of earlier-chunk entries of every expert from the histograms,
//      splits its chunk over its four waves (a second, per-wave histogram
//      gives every wave its starting row per expert), and each wave walks its
//      entries 64 at a time: lanes with the same expert find each other with
//      8 ballots over the bits of the id, the rank among them is a popcount
//      of the lower lanes, and the highest such lane advances the wave's
//      running count.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kPerWave = kDispatchChunk / kWaves;      // entries per wave
constexpr int kSteps = kPerWave / MOE_WAVE;             // 64-entry steps per wave
static_assert(kPerWave % MOE_WAVE == 0, "chunk split");

__global__ __launch_bounds__(kThreads) void dispatch_count(const int32_t* __restrict__ ids, int T,
                                                           int k, int E, int32_t* __restrict__ hist,
                                                           int32_t* __restrict__ status) {
    __shared__ int h[256];
    __shared__ int sid[kDispatchChunk];   // the chunk's ids, for the repeated-id check
    for (int e = threadIdx.x; e < 256; e += kThreads) h[e] = 0;
    const int64_t R = (int64_t)T * k;
    const int64_t q0 = (int64_t)blockIdx.x * kDispatchChunk;
    const int64_t q1 = q0 + kDispatchChunk < R ? q0 + kDispatchChunk : R;
    const int n = (int)(q1 - q0);
    // all loads of the chunk in flight at once (a loop whose trip count the compiler
    // cannot see would wait for each one)
    int ev[kDispatchChunk / kThreads];
#pragma unroll
    for (int s = 0; s < kDispatchChunk / kThreads; ++s) {
        const int i = s * kThreads + (int)threadIdx.x;
        ev[s] = i < n ? ids[q0 + i] : 0;
    }
#pragma unroll
    for (int s = 0; s < kDispatchChunk / kThreads; ++s) {
        const int i = s * kThreads + (int)threadIdx.x;
        if (i < n) sid[i] = ev[s];
    }
    __syncthreads();
    int bad = 0;
#pragma unroll
    for (int s = 0; s < kDispatchChunk / kThreads; ++s) {
        const int i = s * kThreads + (int)threadIdx.x;
        if (i >= n) continue;
        const int64_t q = q0 + i;
        const int e = ev[s];
        if ((unsigned)e >= (unsigned)E) {
            bad |= 1;
            continue;
        }
        const int64_t t = q / k;
        const int j = (int)(q - t * k);
        for (int jj = 0; jj < j; ++jj) {
            const int64_t qq = t * k + jj;          // an earlier entry of the same token
            const int e2 = qq >= q0 ? sid[qq - q0] : ids[qq];
            if (e2 == e) bad |= 2;
        }
        atomicAdd(&h[e], 1);
    }
    if (bad) atomicOr(status, bad);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads) hist[(int64_t)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(kThreads) void dispatch_place(
    const int32_t* __restrict__ ids, const float* __restrict__ scores, int T, int k, int E,
    int nchunks, const int32_t* __restrict__ hist, int32_t* __restrict__ m_indptr,
    int32_t* __restrict__ gather, int32_t* __restrict__ slots, float* __restrict__ probs) {
    __shared__ int start[kWaves][256];   // first row of each wave's entries, per expert
    __shared__ int wsum[kWaves];
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int64_t R = (int64_t)T * k;

    // 1. per expert: total count and count in earlier chunks (thread e owns expert e)
    int tot = 0, before = 0;
    if (tid < E) {
        // eight chunk histograms in flight at a time
        for (int b0 = 0; b0 < nchunks; b0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = b0 + u < nchunks ? hist[(int64_t)(b0 + u) * E + tid] : 0;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                tot += v[u];
                before += (b0 + u < (int)blockIdx.x) ? v[u] : 0;
            }
        }
    }
    // 2. exclusive scan of the totals over experts (wave scan + wave offsets)
    int incl = tot;
    for (int off = 1; off < MOE_WAVE; off <<= 1) {
        const int v = __shfl_up(incl, off, MOE_WAVE);
        if (lane >= off) incl += v;
    }
    if (lane == MOE_WAVE - 1) wsum[wave] = incl;
    __syncthreads();
    int wpre = 0;
    for (int w = 0; w < wave; ++w) wpre += wsum[w];
    const int excl = wpre + incl - tot;
    if (blockIdx.x == 0) {
        if (tid < E) m_indptr[tid] = excl;
        if (tid == E - 1) m_indptr[E] = excl + tot;
    }

    // 3. per-wave histograms of this chunk (entries preloaded into registers)
    for (int e = tid; e < kWaves * 256; e += kThreads) (&start[0][0])[e] = 0;
    __syncthreads();
    const int64_t qw = (int64_t)blockIdx.x * kDispatchChunk + (int64_t)wave * kPerWave;
    int ev[kSteps];
    float sv[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {                   // all loads first, then the counts
        const int64_t q = qw + s * MOE_WAVE + lane;
        ev[s] = q < R ? ids[q] : -1;
        sv[s] = q < R ? scores[q] : 0.f;
    }
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        if ((unsigned)ev[s] >= (unsigned)E) ev[s] = -1;
        if (ev[s] >= 0) atomicAdd(&start[wave][ev[s]], 1);
    }
    __syncthreads();
    // 4. turn the per-wave counts into per-wave starting rows
    if (tid < E) {
        int run = excl + before;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const int c = start[w][tid];
            start[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    // 5. stable ranks inside each wave, 64 entries per step, in entry order
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t q = qw + s * MOE_WAVE + lane;
        const int e = ev[s];
        const bool valid = e >= 0;
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool b = valid && ((e >> bit) & 1);
            const uint64_t m = __ballot(b);
            peers &= b ? m : ~m;
        }
        if (valid) {
            const int rank = __popcll(peers & lanemask_lt());
            const int pos = start[wave][e] + rank;
            gather[pos] = (int32_t)(q / k);
            probs[pos] = sv[s];
            slots[q] = pos;
            if (lane == 63 - __clzll(peers)) start[wave][e] += __popcll(peers);
        } else if (q < R) {
            slots[q] = 0;   // invalid id: keep later reads in bounds; status already flagged
        }
    }
}

// Rows already in expert order: workgroup 0 checks the caller's m_indptr (entry 0 is
// 0, every entry at least the one before and at most R) and copies it, or zeros when it
// fails; every workgroup writes part of the identity gather, so that the gathered
// products read row r of the caller's rows for routed row r.
__global__ __launch_bounds__(kThreads) void routed_prep(const int32_t* __restrict__ m_in, int E, int64_t R,
                                                        int32_t* __restrict__ m_out,
                                                        int32_t* __restrict__ gather,
                                                        int32_t* __restrict__ status) {
    if (blockIdx.x == 0) {
        __shared__ int bad;
        if (threadIdx.x == 0) bad = 0;
        __syncthreads();
        for (int i = threadIdx.x; i <= E; i += kThreads) {
            const int v = m_in[i];
            const bool ok = (i == 0) ? v == 0 : (v >= m_in[i - 1] && (int64_t)v <= R);
            if (!ok) atomicOr(&bad, 1);
        }
        __syncthreads();
        const bool b = bad != 0;
        for (int i = threadIdx.x; i <= E; i += kThreads) m_out[i] = b ? 0 : m_in[i];
        if (b && threadIdx.x == 0) atomicOr(status, kDevBadIndptr);
    }
    for (int64_t r = (int64_t)blockIdx.x * kThreads + threadIdx.x; r < R; r += (int64_t)gridDim.x * kThreads)
        gather[r] = (int32_t)r;
}

}  // namespace

hipError_t launch_routed_prep(const int32_t* m_in, int E, int64_t R, int32_t* m_out, int32_t* gather,
                              int32_t* status, hipStream_t s) {
    int64_t grid = (R + kThreads - 1) / kThreads;
    if (grid < 1) grid = 1;
    if (grid > 1024) grid = 1024;
    hipLaunchKernelGGL(routed_prep, dim3((unsigned)grid), dim3(kThreads), 0, s, m_in, E, R, m_out, gather, status);
    return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* ids, const float* scores, int T, int k, int E,
                           int32_t* hist, int32_t* m_indptr, int32_t* gather, int32_t* slots,
                           float* probs, int32_t* status, hipStream_t s) {
    const int64_t R = (int64_t)T * k;
    int nchunks = dispatch_chunks(R);
    if (nchunks > 0) {
        hipLaunchKernelGGL(dispatch_count, dim3(nchunks), dim3(kThreads), 0, s, ids, T, k, E, hist,
                           status);
    }
    const int nplace = nchunks > 0 ? nchunks : 1;
    hipLaunchKernelGGL(dispatch_place, dim3(nplace), dim3(kThreads), 0, s, ids, scores, T, k, E,
                       nchunks, hist, m_indptr, gather, slots, probs);
    return hipGetLastError();
}

}  // namespace moe
