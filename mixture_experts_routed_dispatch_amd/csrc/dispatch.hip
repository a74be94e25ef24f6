// dispatch.hip -- deterministic expert-major dispatch on gfx950.
//
// Computes what the nvfp4moe README ("Grouped GEMM", "Training") calls the
// dispatch metadata: per-expert counts, m_indptr [E+1] (empty experts valid),
// gather (routed row -> token), slots ((t, j) -> routed row) and probs (scores
// moved to their rows).  Rows of one expert are ordered by ascending token,
// i.e. a stable counting sort of the flattened (t, j) list by expert id.
//
// One launch, no global atomics on the ordering and no wait between workgroups, so
// the result is bit-identical run to run.  Workgroup c owns the chunk of
// kDispatchChunk consecutive entries starting at c * kDispatchChunk:
//   1. it counts, per expert, all R entries and those before its chunk (every
//      workgroup reads the whole id list, R * 4 bytes that stay in L2, with 16-byte
//      loads eight per lane in flight: cheaper than a second launch or a wait on the
//      other workgroups' counts);
//   2. the exclusive scan of the totals over experts gives m_indptr (written by
//      workgroup 0) and, plus the earlier-chunk counts, the chunk's first row per
//      expert;
//   3. its sixteen waves split the chunk; a per-wave histogram gives every wave its
//      starting row per expert, and each wave walks its entries 64 at a time: lanes
//      with the same expert find each other with 8 ballots over the bits of the id,
//      the rank among them is a popcount of the lower lanes, and the highest such lane
//      advances the wave's running count.
// The chunk's ids are also checked (in range, distinct within a token) into the
// sticky status word.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;                            // routed_prep
constexpr int kDThreads = 1024;                          // dispatch
constexpr int kDWaves = kDThreads / MOE_WAVE;
constexpr int kPerWave = kDispatchChunk / kDWaves;       // chunk entries per wave
constexpr int kSteps = kPerWave / MOE_WAVE;              // 64-entry steps per wave
constexpr int kCountUnroll = 8;                          // count groups with loads in flight together
static_assert(kPerWave % MOE_WAVE == 0, "chunk split");
static_assert(kDispatchChunk % 256 == 0, "count groups of 256 entries never straddle a chunk start");

// mask of the lanes whose value equals this lane's (valid lanes only; 8-bit values)
__device__ __forceinline__ uint64_t same_lanes(int e, bool valid) {
    uint64_t peers = __ballot(valid);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
        const bool b = valid && ((e >> bit) & 1);
        const uint64_t m = __ballot(b);
        peers &= b ? m : ~m;
    }
    return peers;
}

__global__ __launch_bounds__(kDThreads) void dispatch_kernel(
    const int32_t* __restrict__ ids, const float* __restrict__ scores, int T, int k, int E,
    int32_t* __restrict__ m_indptr, int32_t* __restrict__ gather, int32_t* __restrict__ slots,
    float* __restrict__ probs, int32_t* __restrict__ status) {
    __shared__ int cnt[2][kDWaves][256];    // per wave: entries before the chunk, and the rest
    __shared__ int start[kDWaves][256];     // first row of each wave's chunk entries, per expert
    __shared__ int sid[kDispatchChunk];     // the chunk's ids, for the repeated-id check
    __shared__ int wsum[kDWaves];
    const int tid = threadIdx.x;
    const int wave = tid / MOE_WAVE;
    const int lane = tid % MOE_WAVE;
    const int64_t R = (int64_t)T * k;
    const int64_t q0 = (int64_t)blockIdx.x * kDispatchChunk;
    for (int i = tid; i < 2 * kDWaves * 256; i += kDThreads) (&cnt[0][0][0])[i] = 0;
    __syncthreads();

    // 1. counts over all entries: wave w takes the groups of 256 consecutive entries
    // w, w + 16, ..., a lane 4 of them with one 16-byte load, eight groups' loads in
    // flight at once; a group lies wholly before the chunk or not (chunks are multiples
    // of 256 entries).  Counts go into the wave's own histograms with LDS adds (grouping
// equal ids with ballots first, as the placement does, was 2.5x slower here).
    const int64_t ngroup = (R + 255) / 256;
    const bool vec = ((uintptr_t)ids & 15) == 0;
    for (int64_t g0 = wave; g0 < ngroup; g0 += (int64_t)kDWaves * kCountUnroll) {
        int4 ev[kCountUnroll];
#pragma unroll
        for (int u = 0; u < kCountUnroll; ++u) {
            const int64_t q = (g0 + (int64_t)u * kDWaves) * 256 + 4 * lane;
            if (vec && q + 3 < R) {
                ev[u] = *reinterpret_cast<const int4*>(ids + q);
            } else {
                ev[u].x = q < R ? ids[q] : -1;
                ev[u].y = q + 1 < R ? ids[q + 1] : -1;
                ev[u].z = q + 2 < R ? ids[q + 2] : -1;
                ev[u].w = q + 3 < R ? ids[q + 3] : -1;
            }
        }
#pragma unroll
        for (int u = 0; u < kCountUnroll; ++u) {
            const int64_t gi = g0 + (int64_t)u * kDWaves;
            int* h = &cnt[gi * 256 < q0 ? 0 : 1][wave][0];
            const int e4[4] = {ev[u].x, ev[u].y, ev[u].z, ev[u].w};
#pragma unroll
            for (int c = 0; c < 4; ++c)
                if ((unsigned)e4[c] < (unsigned)E) atomicAdd(&h[e4[c]], 1);
        }
    }
    __syncthreads();

    // 2. per expert: total and earlier-chunk counts, exclusive scan over experts
    int tot = 0, before = 0;
    if (tid < E) {
#pragma unroll
        for (int w = 0; w < kDWaves; ++w) {
            before += cnt[0][w][tid];
            tot += cnt[0][w][tid] + cnt[1][w][tid];
        }
    }
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

    // 3. the chunk: its ids (checked), per-wave histograms, per-wave starting rows
    for (int i = tid; i < kDWaves * 256; i += kDThreads) (&start[0][0])[i] = 0;
    const int64_t qw = q0 + (int64_t)wave * kPerWave;
    int ev[kSteps];
    float sv[kSteps];
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {                   // all loads first, then the counts
        const int64_t q = qw + s * MOE_WAVE + lane;
        ev[s] = q < R ? ids[q] : -1;
        sv[s] = q < R ? scores[q] : 0.f;
        if (q < R) sid[q - q0] = ev[s];
    }
    __syncthreads();
    int bad = 0;
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t q = qw + s * MOE_WAVE + lane;
        if (q >= R) continue;
        const int e = ev[s];
        if ((unsigned)e >= (unsigned)E) {
            bad |= 1;
            ev[s] = -1;
            continue;
        }
        const int64_t t = q / k;
        const int j = (int)(q - t * k);
        for (int jj = 0; jj < j; ++jj) {
            const int64_t qq = t * k + jj;          // an earlier entry of the same token
            const int e2 = qq >= q0 ? sid[qq - q0] : ids[qq];
            if (e2 == e) bad |= 2;
        }
        atomicAdd(&start[wave][e], 1);
    }
    if (bad) atomicOr(status, bad);
    __syncthreads();
    if (tid < E) {
        int run = excl + before;
#pragma unroll
        for (int w = 0; w < kDWaves; ++w) {
            const int c = start[w][tid];
            start[w][tid] = run;
            run += c;
        }
    }
    __syncthreads();
    // 4. stable ranks inside each wave, 64 entries per step, in entry order
#pragma unroll
    for (int s = 0; s < kSteps; ++s) {
        const int64_t q = qw + s * MOE_WAVE + lane;
        const int e = ev[s];
        const bool valid = e >= 0;
        const uint64_t peers = same_lanes(e, valid);
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
                           int32_t* m_indptr, int32_t* gather, int32_t* slots, float* probs,
                           int32_t* status, hipStream_t s) {
    if (E <= 0 || E > 256) return hipErrorInvalidValue;
    const int64_t R = (int64_t)T * k;
    const int nchunks = dispatch_chunks(R);
    hipLaunchKernelGGL(dispatch_kernel, dim3(nchunks > 0 ? nchunks : 1), dim3(kDThreads), 0, s, ids, scores, T, k, E,
                       m_indptr, gather, slots, probs, status);
    return hipGetLastError();
}

}  // namespace moe
