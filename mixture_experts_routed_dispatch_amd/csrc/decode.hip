// decode.hip -- weight-streaming path of the routed expert layer for small batches.
//
// The nvfp4moe README ("MoE layer") gives batch-one and small-batch decode its
// own launch grid and fuses dispatch into it when top-k is at most 32.  With
// T*k <= 256 routed rows every active expert owns only a few rows, so the two
// expert products are matrix-vector-like and the time is the time to stream
// each active expert's W13 and W2 from HBM once.
//
// Three launches:
//   decode_w13: work items (active expert, block of 8 intermediate indices).  An
//     item streams the 8 gate and 8 up rows of W13_e once and writes
//     a[t*k + j][i] = silu(g) * u in BF16 for every routed entry of the expert.
//     With one token the experts are the k ids themselves (distinct by the
//     layer's precondition), so an item reads its expert id and starts streaming
//     at once; with more tokens every workgroup first re-derives the routing from
//     ids in LDS (a few hundred entries: counts, the active experts in ascending
//     id, and the entries of one expert in ascending (t, j) order).
//   decode_w2: items (active expert, block of 16 output features) stream 16 rows
//     of W2_e and write o[t*k + j][n] in BF16.
//   combine: y[t] = sum_j s[t][j] * o[t*k + j], FP32, j ascending from +0.0 (the
//     prefill combine kernel, reading the rows in entry order).
//
// Both products use v_mfma_f32_16x16x32_bf16 with the weight rows as the 16
// columns and up to 16 routed rows as the 16 rows of one MFMA; lane l loads 16
// contiguous bytes of weight row (l & 15) at K offset 32 s + 8 (l >> 4), so a
// wave's load covers 64 contiguous bytes of 16 rows.  The K range is split over
// the four waves (step s goes to wave s & 3) and the partial accumulators are
// added in wave order through LDS, so the result does not depend on timing.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kBatch = 16;         // K steps of 32 per wave held in registers at once

struct DecodeSmem {
    int ids[kMaxDecodeRows];       // expert of entry q = t*k + j (-1 when invalid)
    int cnt[256];                  // routed rows per expert
    int slot_expert[256];          // i-th active expert (ascending id)
    int list[kMaxDecodeRows];      // entries of the current expert, ascending
    int wcnt[kWaves];
    int n_active;
    int M;
    f32x4_t red[kWaves][MOE_WAVE]; // per-wave partial accumulators
};

// Counts, active-expert list and routing flags, from ids; every workgroup runs it.
__device__ void decode_setup(DecodeSmem& sm, const int32_t* __restrict__ ids, int T, int k, int E,
                             int32_t* status, bool report) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int R = T * k;
    for (int e = tid; e < 256; e += kThreads) sm.cnt[e] = 0;
    __syncthreads();
    if (tid < R) {
        const int e = ids[tid];
        const bool ok = (unsigned)e < (unsigned)E;
        sm.ids[tid] = ok ? e : -1;
        if (ok) atomicAdd(&sm.cnt[e], 1);
        if (report) {
            int bad = ok ? 0 : kDevIdOutOfRange;
            const int t = tid / k, j = tid - t * k;
            for (int jj = 0; jj < j; ++jj)
                if (ok && ids[t * k + jj] == e) bad |= kDevIdDuplicate;
            if (bad) atomicOr(status, bad);
        }
    }
    __syncthreads();
    // active experts in ascending id: ballot ranks inside a wave, wave prefix via LDS
    const bool active = tid < E && sm.cnt[tid] > 0;
    const uint64_t b = __ballot(active);
    if (lane == 0) sm.wcnt[wave] = __popcll(b);
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += sm.wcnt[w];
    if (active) sm.slot_expert[pre + __popcll(b & lanemask_lt())] = tid;
    if (tid == 0) sm.n_active = sm.wcnt[0] + sm.wcnt[1] + sm.wcnt[2] + sm.wcnt[3];
    __syncthreads();
}

// sm.list[0 .. sm.M) = entries routed to expert e, ascending.
__device__ void decode_rows_of(DecodeSmem& sm, int e, int R) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __syncthreads();                       // previous item is done with list / wcnt
    const bool match = tid < R && sm.ids[tid] == e;
    const uint64_t b = __ballot(match);
    if (lane == 0) sm.wcnt[wave] = __popcll(b);
    __syncthreads();
    int pre = 0;
    for (int w = 0; w < wave; ++w) pre += sm.wcnt[w];
    if (match) sm.list[pre + __popcll(b & lanemask_lt())] = tid;
    if (tid == 0) sm.M = sm.wcnt[0] + sm.wcnt[1] + sm.wcnt[2] + sm.wcnt[3];
    __syncthreads();
}

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
}

// acc(16 rows x 16 cols) += A(rows: routed rows src_row[m]) * B(cols: weight rows), K = Ksz.
// Lane l: B column (l & 15) from wrow_ptr (already offset by 8 (l >> 4)); A row (l & 15)
// from arow_ptr (same K offset), or zeros when the row is absent.  Returns this wave's
// partial sum over its K steps (s = wave, wave + 4, ...).
__device__ __forceinline__ f32x4_t decode_mma(const uint16_t* wrow_ptr, const uint16_t* arow_ptr,
                                              bool arow_valid, int nsteps) {
    const int wave = threadIdx.x >> 6;
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    const bf16x8_t zero = {};
    for (int base = 0; base < nsteps; base += kWaves * kBatch) {
        bf16x8_t wb[kBatch], xa[kBatch];
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = base + wave + kWaves * j;
            if (s < nsteps) {
                wb[j] = ld_bf16x8(wrow_ptr + 32 * s);
                xa[j] = arow_valid ? ld_bf16x8(arow_ptr + 32 * s) : zero;
            }
        }
#pragma unroll
        for (int j = 0; j < kBatch; ++j) {
            const int s = base + wave + kWaves * j;
            if (s < nsteps) acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[j], wb[j], acc, 0, 0, 0);
        }
    }
    return acc;
}

// Sum of the four waves' partial accumulators, in wave order; valid in wave 0.
__device__ __forceinline__ f32x4_t decode_reduce(DecodeSmem& sm, f32x4_t acc) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    sm.red[wave][lane] = acc;
    __syncthreads();
    f32x4_t s = sm.red[0][lane];
    if (wave == 0) {
#pragma unroll
        for (int w = 1; w < kWaves; ++w) {
            const f32x4_t v = sm.red[w][lane];
            s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
        }
    }
    __syncthreads();
    return s;
}

// Routing flags for the one-token path (block 0 only): ids out of range or repeated.
__device__ void decode_flags_one_token(const DecodeArgs& g) {
    const int j = threadIdx.x;
    if (j < g.k) {
        const int e = g.ids[j];
        int bad = (unsigned)e < (unsigned)g.E ? 0 : kDevIdOutOfRange;
        for (int jj = 0; jj < j; ++jj)
            if (bad == 0 && g.ids[jj] == e) bad |= kDevIdDuplicate;
        if (bad) atomicOr(g.status, bad);
    }
}

// One W13 item: expert e, intermediate block i0 .. i0+7, routed entries entry(0 .. M-1).
template <class EntryOf>
__device__ __forceinline__ void w13_item(const DecodeArgs& g, DecodeSmem& sm, int e, int M,
                                         EntryOf entry, int i0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I;
    // columns 0..7: gate rows i0..i0+7; columns 8..15: up rows I+i0..I+i0+7
    const int wrow = (n < 8) ? (i0 + n) : (I + i0 + n - 8);
    const uint16_t* wp = g.w13 + ((size_t)e * 2 * I + wrow) * d + 8 * kq;
    for (int g0 = 0; g0 < M; g0 += 16) {
        const int m = g0 + (lane & 15);
        const bool mv = m < M;
        const int tok = mv ? entry(m) / g.k : 0;
        const uint16_t* xp = g.x + (size_t)tok * d + 8 * kq;
        f32x4_t acc = decode_mma(wp, xp, mv, d / 32);
        acc = decode_reduce(sm, acc);
        // lane l of wave 0 holds rows 4 (l >> 4) + z of column l & 15; the up value of
        // gate column c < 8 sits in lane l + 8 of the same 16-lane group
        float up[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) up[z] = __shfl_down(acc[z], 8, 16);
        if (wave == 0 && n < 8) {
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int mm = g0 + 4 * kq + z;
                if (mm < M) {
                    const float av = silu_f(acc[z]) * up[z];
                    g.a[(size_t)entry(mm) * I + i0 + n] = (uint16_t)f32_to_bf16(av);
                }
            }
        }
    }
}

// One W2 item: expert e, output features n0 .. n0+15, routed entries entry(0 .. M-1).
template <class EntryOf>
__device__ __forceinline__ void w2_item(const DecodeArgs& g, DecodeSmem& sm, int e, int M,
                                        EntryOf entry, int n0) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I;
    const uint16_t* wp = g.w2 + ((size_t)e * d + n0 + n) * I + 8 * kq;
    for (int g0 = 0; g0 < M; g0 += 16) {
        const int m = g0 + (lane & 15);
        const bool mv = m < M;
        const uint16_t* ap = g.a + (size_t)(mv ? entry(m) : 0) * I + 8 * kq;
        f32x4_t acc = decode_mma(wp, ap, mv, I / 32);
        acc = decode_reduce(sm, acc);
        if (wave == 0) {
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int mm = g0 + 4 * kq + z;
                if (mm < M) g.o[(size_t)entry(mm) * d + n0 + n] = (uint16_t)f32_to_bf16(acc[z]);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads, 3) void decode_w13(DecodeArgs g) {
    __shared__ DecodeSmem sm;
    const int nIB = g.I / 8;
    if (g.T == 1) {
        if (blockIdx.x == 0) decode_flags_one_token(g);
        const int items = g.k * nIB;
        for (int item = blockIdx.x; item < items; item += gridDim.x) {
            const int slot = item / nIB, ib = item - slot * nIB;
            const int e = g.ids[slot];
            if ((unsigned)e >= (unsigned)g.E) continue;
            w13_item(g, sm, e, 1, [slot](int) { return slot; }, ib * 8);
        }
        return;
    }
    const int R = g.T * g.k;
    decode_setup(sm, g.ids, g.T, g.k, g.E, g.status, blockIdx.x == 0);
    const int items = sm.n_active * nIB;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int slot = item / nIB, ib = item - slot * nIB;
        const int e = sm.slot_expert[slot];
        decode_rows_of(sm, e, R);
        w13_item(g, sm, e, sm.M, [lst = sm.list](int m) { return lst[m]; }, ib * 8);
    }
}

__global__ __launch_bounds__(kThreads, 3) void decode_w2(DecodeArgs g) {
    __shared__ DecodeSmem sm;
    const int nNB = g.d / 16;
    if (g.T == 1) {
        const int items = g.k * nNB;
        for (int item = blockIdx.x; item < items; item += gridDim.x) {
            const int slot = item / nNB, nb = item - slot * nNB;
            const int e = g.ids[slot];
            if ((unsigned)e >= (unsigned)g.E) continue;
            w2_item(g, sm, e, 1, [slot](int) { return slot; }, nb * 16);
        }
        return;
    }
    const int R = g.T * g.k;
    decode_setup(sm, g.ids, g.T, g.k, g.E, g.status, false);
    const int items = sm.n_active * nNB;
    for (int item = blockIdx.x; item < items; item += gridDim.x) {
        const int slot = item / nNB, nb = item - slot * nNB;
        const int e = sm.slot_expert[slot];
        decode_rows_of(sm, e, R);
        w2_item(g, sm, e, sm.M, [lst = sm.list](int m) { return lst[m]; }, nb * 16);
    }
}

}  // namespace

hipError_t launch_decode_w13(const DecodeArgs& g, int num_cu, hipStream_t s) {
    const int R = g.T * g.k;
    if (R <= 0) return hipSuccess;
    const int slots = R < g.E ? R : g.E;                  // active experts at most
    const int cap = 3 * num_cu;                           // resident workgroups
    int grid = slots * (g.I / 8);
    grid = grid < cap ? grid : cap;
    hipLaunchKernelGGL(decode_w13, dim3(grid), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_decode_w2(const DecodeArgs& g, int num_cu, hipStream_t s) {
    const int R = g.T * g.k;
    if (R <= 0) return hipSuccess;
    const int slots = R < g.E ? R : g.E;
    const int cap = 3 * num_cu;
    int grid = slots * (g.d / 16);
    grid = grid < cap ? grid : cap;
    hipLaunchKernelGGL(decode_w2, dim3(grid), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

}  // namespace moe
