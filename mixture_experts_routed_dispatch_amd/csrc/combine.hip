// combine.hip -- score-weighted deterministic combine and its gradients on gfx950.
//
// nvfp4moe README, "MoE layer": the timed path ends with probability weighting
// and a deterministic combine; "Training": router gradients.  Both are
// HBM-streaming gathers: each thread owns 8 consecutive features (one 16-byte
// load per routed row, non-temporal in the combine: 53.5 against 57 us at the
// prefill size) and sums the k rows of its token in FP32 with j ascending from
// +0.0, so the result does not depend on the launch shape.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

// A gathered row piece, read non-temporally: each routed row is read once (by its
// token), and the producers stream these rows out with non-temporal stores.
__device__ __forceinline__ uint4 ld_row_nt(const uint16_t* p) {
    const u32x4_t w = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint16_t* __restrict__ src,
                                                           const int32_t* __restrict__ slots,
                                                           const float* __restrict__ w, int T, int k,
                                                           int d, uint16_t* __restrict__ y) {
    const int t = blockIdx.y;
    const int n = (blockIdx.x * kThreads + threadIdx.x) * 8;
    if (n >= d) return;
    float acc[8];
#pragma unroll
    for (int z = 0; z < 8; ++z) acc[z] = 0.0f;
    const int32_t* sl = slots ? slots + (size_t)t * k : nullptr;
    const float* wt = w ? w + (size_t)t * k : nullptr;
    auto row = [&](int j) { return sl ? (size_t)sl[j] : (size_t)t * k + j; };
    int j = 0;
    for (; j + 4 <= k; j += 4) {       // four rows in flight per step; summation order unchanged
        uint4 v[4];
        float s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            v[u] = ld_row_nt(src + row(j + u) * d + n);
            s[u] = wt ? wt[j + u] : 1.0f;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const uint32_t ww[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                acc[2 * z] = __builtin_fmaf(s[u], bf16lo(ww[z]), acc[2 * z]);
                acc[2 * z + 1] = __builtin_fmaf(s[u], bf16hi(ww[z]), acc[2 * z + 1]);
            }
        }
    }
    for (; j < k; ++j) {
        const uint4 v = ld_row_nt(src + row(j) * d + n);
        const float s = wt ? wt[j] : 1.0f;
        const uint32_t ww[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int z = 0; z < 4; ++z) {
            acc[2 * z] = __builtin_fmaf(s, bf16lo(ww[z]), acc[2 * z]);
            acc[2 * z + 1] = __builtin_fmaf(s, bf16hi(ww[z]), acc[2 * z + 1]);
        }
    }
    uint4 o;
    o.x = pack_bf16(acc[0], acc[1]);
    o.y = pack_bf16(acc[2], acc[3]);
    o.z = pack_bf16(acc[4], acc[5]);
    o.w = pack_bf16(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + (size_t)t * d + n) = o;
}

// ds[t][j] = <dy[t], o[slots[t][j]]>: one workgroup per token, fixed reduction tree.
// The token's rows are taken 8 at a time with all their loads in flight (indices past
// k clamp to row k - 1 and are not used); each j keeps its own chain of FMAs over n, so
// the sums are those of one row at a time.
constexpr int kMaxK = 32;
constexpr int kRowsInFlight = 8;

__global__ __launch_bounds__(kThreads) void score_grad_kernel(const uint16_t* __restrict__ dy,
                                                              const uint16_t* __restrict__ o,
                                                              const int32_t* __restrict__ slots,
                                                              int T, int k, int d,
                                                              float* __restrict__ ds) {
    __shared__ float part[kThreads / MOE_WAVE][kMaxK];
    const int t = blockIdx.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int32_t* sl = slots + (size_t)t * k;
    for (int j0 = 0; j0 < k; j0 += kRowsInFlight) {
        size_t r[kRowsInFlight];
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) r[u] = (size_t)sl[j0 + u < k ? j0 + u : k - 1];
        float acc[kRowsInFlight];
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) acc[u] = 0.0f;
        for (int n = threadIdx.x * 8; n < d; n += kThreads * 8) {
            const uint4 a = *reinterpret_cast<const uint4*>(dy + (size_t)t * d + n);
            uint4 b[kRowsInFlight];
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) b[u] = ld_row_nt(o + r[u] * d + n);
            const uint32_t aw[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int u = 0; u < kRowsInFlight; ++u) {
                const uint32_t bw[4] = {b[u].x, b[u].y, b[u].z, b[u].w};
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    acc[u] = __builtin_fmaf(bf16lo(aw[z]), bf16lo(bw[z]), acc[u]);
                    acc[u] = __builtin_fmaf(bf16hi(aw[z]), bf16hi(bw[z]), acc[u]);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kRowsInFlight; ++u) {
            float v = acc[u];
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) v += __shfl_down(v, off, MOE_WAVE);
            if (lane == 0 && j0 + u < k) part[wave][j0 + u] = v;
        }
    }
    __syncthreads();
    if (threadIdx.x < k) {
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kThreads / MOE_WAVE; ++w) s += part[w][threadIdx.x];
        ds[(size_t)t * k + threadIdx.x] = s;
    }
}

// The router gradient from the partials the W2 data-gradient product leaves: <dy[t], o>
// with o = W2 a equals sum_i (dy[t] W2)[i] a[i], which that product's epilogue has at
// hand (its accumulators before the probs scaling, and a from the saved h), in pieces of
// 64 columns.  Entry q (= t k + j) adds its row's pieces in slot order, from +0.0, so
// the result does not depend on the launch.
__global__ __launch_bounds__(kThreads) void score_grad_sum_kernel(const float* __restrict__ part,
                                                                  const int32_t* __restrict__ slots,
                                                                  int R, int nslots, float* __restrict__ ds) {
    const int q = blockIdx.x * kThreads + threadIdx.x;
    if (q >= R) return;
    const float* p = part + (size_t)slots[q] * nslots;
    float s = 0.0f;
    for (int i = 0; i < nslots; ++i) s += p[i];
    ds[q] = s;
}

// Row-major operands of the weight-gradient products: xg[r] = x[gather[r]] and
// dys[r] = bf16(probs[r] * dy[gather[r]]) for routed rows r.  Token-major: one
// workgroup per token t (grid-strided) reads x[t] and dy[t] once, one 16-byte chunk
// of each per thread, and writes them to the token's routed rows r = slots[t][j].  A
// row is written only when gather[r] == t: an entry with an invalid expert id has slot
// 0, and passes that test only if row 0 is the same token's, where it writes what row
// 0's own entry writes.  Rows past the routed count stay unwritten; the products read
// only the rows of their experts.  (Row-major in r, the k reads of each token lay far
// apart in time and missed in L2: 537 MB fetched for 67 MB of x and dy.)
__global__ __launch_bounds__(kThreads) void wgrad_rows_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ dy,
                                                              const int32_t* __restrict__ slots,
                                                              const int32_t* __restrict__ gather,
                                                              const float* __restrict__ probs,
                                                              int T, int k, int d,
                                                              uint16_t* __restrict__ xg,
                                                              uint16_t* __restrict__ dys) {
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        for (int n = threadIdx.x * 8; n < d; n += kThreads * 8) {
            const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * d + n);
            const uint4 gv = *reinterpret_cast<const uint4*>(dy + (size_t)t * d + n);
            const uint32_t gw[4] = {gv.x, gv.y, gv.z, gv.w};
            for (int j = 0; j < k; ++j) {
                const int r = slots[(size_t)t * k + j];
                if (gather[r] != t) continue;
                const float sc = probs[r];
                uint32_t ow[4];
#pragma unroll
                for (int z = 0; z < 4; ++z) ow[z] = pack_bf16(sc * bf16lo(gw[z]), sc * bf16hi(gw[z]));
                *reinterpret_cast<uint4*>(xg + (size_t)r * d + n) = xv;
                *reinterpret_cast<uint4*>(dys + (size_t)r * d + n) = make_uint4(ow[0], ow[1], ow[2], ow[3]);
            }
        }
    }
}

}  // namespace

hipError_t launch_wgrad_rows(const uint16_t* x, const uint16_t* dy, int T, int k, const int32_t* slots,
                             const int32_t* gather, const float* probs, int d, uint16_t* xg, uint16_t* dys,
                             hipStream_t s) {
    if (T == 0 || k == 0) return hipSuccess;
    if (T < 0 || k < 0 || d % 8 != 0) return hipErrorInvalidValue;
    const int grid = T < 65536 ? T : 65536;
    hipLaunchKernelGGL(wgrad_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, x, dy, slots, gather,
                       probs, T, k, d, xg, dys);
    return hipGetLastError();
}

hipError_t launch_combine(const uint16_t* src, const int32_t* slots, const float* w, int T, int k,
                          int d, uint16_t* y, hipStream_t s) {
    if (T == 0) return hipSuccess;
    const dim3 grid((d / 8 + kThreads - 1) / kThreads, T);
    hipLaunchKernelGGL(combine_kernel, grid, dim3(kThreads), 0, s, src, slots, w, T, k, d, y);
    return hipGetLastError();
}

hipError_t launch_score_grad_sum(const float* part, const int32_t* slots, int R, int nslots, float* ds,
                                 hipStream_t s) {
    if (R == 0) return hipSuccess;
    hipLaunchKernelGGL(score_grad_sum_kernel, dim3((R + kThreads - 1) / kThreads), dim3(kThreads), 0, s,
                       part, slots, R, nslots, ds);
    return hipGetLastError();
}

hipError_t launch_score_grad(const uint16_t* dy, const uint16_t* o, const int32_t* slots, int T,
                             int k, int d, float* ds, hipStream_t s) {
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(score_grad_kernel, dim3(T), dim3(kThreads), 0, s, dy, o, slots, T, k, d, ds);
    return hipGetLastError();
}

}  // namespace moe
