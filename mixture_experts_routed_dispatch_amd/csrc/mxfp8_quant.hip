// mxfp8_quant.hip -- OCP MXFP8 (E4M3 elements, E8M0 scale per 32) conversion on gfx950.
//
// The blog post ("What it is selling") names MXFP8 E4M3 with prepared weights
// and activations quantized after routing.  Per OCP MX v1.0 block of 32 values along
// K, the shared scale is the smallest power of two 2^s with max|v| / 2^s <= 448
// (E4M3's largest normal: s = ceil(log2(max|v| / 448))), stored biased by 127 and
// clamped to [0, 254] (0 for an all-zero block); each element is v / 2^s rounded to
// nearest even on the E4M3 grid (no element saturates; the clamp to +-448 stays for
// non-finite input).  Inputs are BF16, so v / 2^s is exact in FP32 and the codes are a
// deterministic function of the input bits.
//
// Scales are stored row-major ([rows, K/32]) or block-major: the four bytes of blocks
// 4 g .. 4 g + 3 of a row form one word, and word (g, row) sits at (g * rows + row) * 4,
// so that the words of consecutive rows for one group of 128 K elements are contiguous
// (the MXFP8 GEMMs copy them 64 rows at a time).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void quantize_kernel(const uint16_t* __restrict__ v,
                                                            int64_t nblocks, int kb_row, int64_t rows,
                                                            const int32_t* __restrict__ rows_dev,
                                                            bool block_major,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
    if (rows_dev) {                       // only the first *rows_dev rows (at most rows)
        const int64_t n = *rows_dev;
        if (n < rows) nblocks = (n > 0 ? n : 0) * kb_row;
    }
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblocks;
         b += (int64_t)gridDim.x * kThreads) {
        const uint4* src = reinterpret_cast<const uint4*>(v + b * 32);
        uint32_t w[16];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 q = src[c];
            w[4 * c] = q.x; w[4 * c + 1] = q.y; w[4 * c + 2] = q.z; w[4 * c + 3] = q.w;
        }
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
            amax = __builtin_fmaxf(amax, __builtin_fmaxf(__builtin_fabsf(bf16lo(w[i])), __builtin_fabsf(bf16hi(w[i]))));
        const uint32_t sb = e8m0_scale(amax);
        const int sh = 127 - (int)sb;
        uint32_t out[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            out[i] = e4m3_pack4(__builtin_ldexpf(bf16lo(w[2 * i]), sh), __builtin_ldexpf(bf16hi(w[2 * i]), sh),
                                __builtin_ldexpf(bf16lo(w[2 * i + 1]), sh), __builtin_ldexpf(bf16hi(w[2 * i + 1]), sh));
        }
        uint4* dst = reinterpret_cast<uint4*>(codes + b * 32);
        dst[0] = make_uint4(out[0], out[1], out[2], out[3]);
        dst[1] = make_uint4(out[4], out[5], out[6], out[7]);
        int64_t si = b;
        if (block_major) {
            const int64_t row = b / kb_row;
            const int kb = (int)(b - row * kb_row);
            si = ((int64_t)(kb >> 2) * rows + row) * 4 + (kb & 3);
        }
        scales[si] = (uint8_t)sb;
    }
}

// Scales of gathered rows, block-major: word (g, r) of out, the four scale bytes of K
// group g (blocks 4 g .. 4 g + 3) of routed row r, is word g of source row gather[r].
// A workgroup transposes 256 routed rows x 16 groups through LDS: 16 lanes read the 64
// bytes of one source row, and each store of a wave covers 64 consecutive words of one
// group.  Row stride 17 words in LDS: the column reads hit 64 different banks.
// Entries of gather past the routed count (left unwritten by the dispatch when routes
// carry invalid expert ids) are read clamped to row 0; no product reads their words.
constexpr int kRouteRows = 256, kRouteGroups = 16;
__global__ void __launch_bounds__(kThreads) route_scales_kernel(const uint32_t* __restrict__ src,
                                                                const int32_t* __restrict__ gather,
                                                                int64_t R, int groups, uint32_t src_rows,
                                                                uint32_t* __restrict__ out) {
    static_assert(kThreads == kRouteRows, "one thread per routed row in the stores");
    __shared__ uint32_t tile[kRouteRows * (kRouteGroups + 1)];
    const int t = threadIdx.x;
    const int g0 = blockIdx.y * kRouteGroups;
    const int w = t % kRouteGroups;
    for (int64_t r0 = (int64_t)blockIdx.x * kRouteRows; r0 < R; r0 += (int64_t)gridDim.x * kRouteRows) {
#pragma unroll
        for (int i = 0; i < kRouteGroups; ++i) {
            const int row = t / kRouteGroups + i * (kThreads / kRouteGroups);
            if (r0 + row < R && g0 + w < groups) {
                uint32_t tok = (uint32_t)gather[r0 + row];
                if (tok >= src_rows) tok = 0;
                tile[row * (kRouteGroups + 1) + w] = src[(int64_t)tok * groups + g0 + w];
            }
        }
        __syncthreads();
        if (r0 + t < R) {
            for (int gi = 0; gi < kRouteGroups && g0 + gi < groups; ++gi)
                out[(int64_t)(g0 + gi) * R + r0 + t] = tile[t * (kRouteGroups + 1) + gi];
        }
        __syncthreads();
    }
}

// One MX block of 32 FP32 values: E8M0 scale byte and 32 E4M3 codes (8 words).
__device__ __forceinline__ uint32_t quant_block32(const float* v, uint32_t out[8]) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
    const uint32_t sb = e8m0_scale(amax);
    const int sh = 127 - (int)sb;
#pragma unroll
    for (int i = 0; i < 8; ++i)
        out[i] = e4m3_pack4(__builtin_ldexpf(v[4 * i], sh), __builtin_ldexpf(v[4 * i + 1], sh),
                            __builtin_ldexpf(v[4 * i + 2], sh), __builtin_ldexpf(v[4 * i + 3], sh));
    return sb;
}

__device__ __forceinline__ void store_codes32(uint8_t* dst, const uint32_t w[8]) {
    uint4* d = reinterpret_cast<uint4*>(dst);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// Byte of block kb of routed row r in the block-major layout [K/128][R][4].
__device__ __forceinline__ int64_t bm_index(int64_t R, int64_t r, int kb) {
    return ((int64_t)(kb >> 2) * R + r) * 4 + (kb & 3);
}

// dO of the MXFP8 backward: rows r of probs[r] * dy[gather[r]] (FP32) quantized along d.
// Token-major: one wave per token t (grid-strided), lane = block of 32 along d, reads dy[t]
// once and quantizes it for each of the token's routed rows r = slots[t][j] with
// gather[r] == t (an entry with an invalid expert id has slot 0 and passes only if row 0
// is the same token's, where it writes what row 0's own entry writes).  Rows past the
// routed count stay unwritten; the products read only the rows of their experts.
// (Row-major, the k reads of each token lay far apart in time and missed in L2.)
__global__ __launch_bounds__(kThreads) void mx_scaled_rows_kernel(const uint16_t* __restrict__ dy, int T, int k,
                                                                  const int32_t* __restrict__ slots,
                                                                  const int32_t* __restrict__ gather,
                                                                  const float* __restrict__ probs, int64_t R, int d,
                                                                  uint8_t* __restrict__ codes,
                                                                  uint8_t* __restrict__ scales) {
    const int kb_row = d / 32;
    const int lane = threadIdx.x % MOE_WAVE;
    const int nw = gridDim.x * (kThreads / MOE_WAVE);
    for (int t = blockIdx.x * (kThreads / MOE_WAVE) + (int)(threadIdx.x / MOE_WAVE); t < T; t += nw) {
        for (int kb = lane; kb < kb_row; kb += MOE_WAVE) {
            const uint4* src = reinterpret_cast<const uint4*>(dy + (int64_t)t * d + 32 * kb);
            uint32_t w[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 q = src[c];
                w[4 * c] = q.x; w[4 * c + 1] = q.y; w[4 * c + 2] = q.z; w[4 * c + 3] = q.w;
            }
            for (int j = 0; j < k; ++j) {
                const int64_t r = slots[(int64_t)t * k + j];
                if (gather[r] != t) continue;
                const float pr = probs[r];
                float v[32];
#pragma unroll
                for (int z = 0; z < 16; ++z) {
                    v[2 * z] = pr * bf16lo(w[z]);
                    v[2 * z + 1] = pr * bf16hi(w[z]);
                }
                uint32_t out[8];
                const uint32_t sb = quant_block32(v, out);
                store_codes32(codes + r * d + 32 * kb, out);
                scales[bm_index(R, r, kb)] = (uint8_t)sb;
            }
        }
    }
}

// The gated activation's backward of the MXFP8 backward: one thread per (row, block of 32
// intermediate columns): dg = dA u f'(g) and du = dA f(g) from BF16 dA and h; dh in BF16
// and both blocks quantized along 2I
template <int kAct>
__global__ __launch_bounds__(kThreads) void mx_act_backward_kernel(const uint16_t* __restrict__ dA,
                                                                   const uint16_t* __restrict__ h, int64_t R, int I,
                                                                   uint16_t* __restrict__ dh,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales) {
    const int kb_row = I / 32;
    const int64_t nb = R * kb_row;
    for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nb; b += (int64_t)gridDim.x * kThreads) {
        const int64_t r = b / kb_row;
        const int kb = (int)(b - r * kb_row);
        const int i0 = 32 * kb;
        float dg[32], du[32];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint4 a4 = reinterpret_cast<const uint4*>(dA + r * I + i0)[c];
            const uint4 g4 = reinterpret_cast<const uint4*>(h + r * 2 * I + i0)[c];
            const uint4 u4 = reinterpret_cast<const uint4*>(h + r * 2 * I + I + i0)[c];
            const uint32_t aw[4] = {a4.x, a4.y, a4.z, a4.w};
            const uint32_t gw[4] = {g4.x, g4.y, g4.z, g4.w};
            const uint32_t uw[4] = {u4.x, u4.y, u4.z, u4.w};
#pragma unroll
            for (int z = 0; z < 4; ++z)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    const float a = hh ? bf16hi(aw[z]) : bf16lo(aw[z]);
                    const float gv = hh ? bf16hi(gw[z]) : bf16lo(gw[z]);
                    const float uv = hh ? bf16hi(uw[z]) : bf16lo(uw[z]);
                    float f, df;
                    act_f_df<kAct>(gv, f, df);
                    dg[8 * c + 2 * z + hh] = a * uv * df;
                    du[8 * c + 2 * z + hh] = a * f;
                }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            uint4 og, ou;
            og.x = pack_bf16(dg[8 * c], dg[8 * c + 1]); og.y = pack_bf16(dg[8 * c + 2], dg[8 * c + 3]);
            og.z = pack_bf16(dg[8 * c + 4], dg[8 * c + 5]); og.w = pack_bf16(dg[8 * c + 6], dg[8 * c + 7]);
            ou.x = pack_bf16(du[8 * c], du[8 * c + 1]); ou.y = pack_bf16(du[8 * c + 2], du[8 * c + 3]);
            ou.z = pack_bf16(du[8 * c + 4], du[8 * c + 5]); ou.w = pack_bf16(du[8 * c + 6], du[8 * c + 7]);
            reinterpret_cast<uint4*>(dh + r * 2 * I + i0)[c] = og;
            reinterpret_cast<uint4*>(dh + r * 2 * I + I + i0)[c] = ou;
        }
        uint32_t out[8];
        uint32_t sb = quant_block32(dg, out);
        store_codes32(codes + r * 2 * I + i0, out);
        scales[bm_index(R, r, kb)] = (uint8_t)sb;
        sb = quant_block32(du, out);
        store_codes32(codes + r * 2 * I + I + i0, out);
        scales[bm_index(R, r, kb_row + kb)] = (uint8_t)sb;
    }
}

// Transposing quantization (see launch_mx_transpose_quant).  A workgroup takes 128 source
// rows (one group of four MX blocks along the rows) and walks every gridDim.y-th tile of
// 64 columns, the next tile's loads in flight while the current one is converted:
//   1. two threads per row copy the row's 64 columns (128 contiguous bytes) into LDS as
//      FP32, [row][65] (scaled by probs, zero past the segment's rows);
//   2. thread (column f = t / 4, block b = t % 4) quantizes rows 32 b .. 32 b + 31 of
//      column f and writes their 32 codes, so that the four threads of a column write
//      its 128 contiguous code bytes and its scale word together.
// The row tile's segment, source rows and scores are looked up once per workgroup.
// Token layout: the tiles of all segments are numbered in segment order (segment e has
// kp_e / 128 of them), gridDim.x covers the largest possible total, and workgroups past
// the actual one exit.  Weight layout: blockIdx.z is the matrix, blockIdx.x its tile.
constexpr int kTqRows = 128, kTqCols = 64, kTqLd = kTqCols + 1;

__global__ __launch_bounds__(kThreads) void mx_transpose_quant_kernel(const uint16_t* __restrict__ src, int segs,
                                                                      int K, int N,
                                                                      const int32_t* __restrict__ m_indptr,
                                                                      const int32_t* __restrict__ gather,
                                                                      const float* __restrict__ probs, int T,
                                                                      bool weights, uint8_t* __restrict__ codes,
                                                                      uint8_t* __restrict__ scales) {
    __shared__ float tile[kTqRows * kTqLd];
    __shared__ int wsum[kThreads / 64];
    __shared__ int info[4];            // segment, tile within it, first routed row, rows
    const int tid = threadIdx.x;
    int e, kt, r0, rows, kp;
    int64_t koff;
    if (weights) {
        e = blockIdx.z;
        kt = blockIdx.x;
        r0 = 0;
        rows = K;
        kp = K;
        koff = (int64_t)e * K;
    } else {
        // tiles per segment and their prefix, then the segment holding tile blockIdx.x
        int nt = 0, rs = 0, mb = 0;
        if (tid < segs) {
            mb = m_indptr[tid];
            rs = m_indptr[tid + 1] - mb;
            nt = ((rs > 0 ? rs : 1) + kMxWgradPad - 1) / kMxWgradPad;
        }
        int incl = nt;
        const int lane = tid & 63, wave = tid >> 6;
        for (int off = 1; off < 64; off <<= 1) {
            const int v = __shfl_up(incl, off, 64);
            if (lane >= off) incl += v;
        }
        if (lane == 63) wsum[wave] = incl;
        if (tid == 0) info[0] = -1;
        __syncthreads();
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += wsum[w];
        const int first = pre + incl - nt;
        const int j = blockIdx.x;
        if (tid < segs && j >= first && j < first + nt) {
            info[0] = tid;
            info[1] = j - first;
            info[2] = mb;
            info[3] = rs;
        }
        // koff of the segment = 128 * (tiles before it): kept by the owning thread
        __syncthreads();
        e = info[0];
        if (e < 0) return;                         // past the last tile
        kt = info[1];
        r0 = info[2];
        rows = info[3];
        __syncthreads();
        if (tid == e) info[0] = first;
        __syncthreads();
        koff = (int64_t)info[0] * kMxWgradPad;
        kp = ((rows > 0 ? rows : 1) + kMxWgradPad - 1) / kMxWgradPad * kMxWgradPad;   // row stride of the codes
    }
    // the thread's source row (two threads per row, 32 columns each), loaded once
    const int row = tid >> 1, half = tid & 1;
    const int kr = kt * kTqRows + row;
    const bool live = kr < rows;
    int64_t srow = 0;
    float sc = 1.0f;
    if (live) {
        if (weights) {
            srow = (int64_t)e * K + kr;
        } else {
            srow = r0 + kr;
            if (probs) sc = probs[srow];
            if (gather) {
                const uint32_t t = (uint32_t)gather[srow];
                srow = t < (uint32_t)T ? t : 0;
            }
        }
    }
    const uint16_t* rowp = src + srow * N + 32 * half;
    auto load = [&](int ft, uint4 q[4]) {
        const uint4* p = reinterpret_cast<const uint4*>(rowp + (int64_t)ft * kTqCols);
#pragma unroll
        for (int c = 0; c < 4; ++c) q[c] = live ? p[c] : make_uint4(0, 0, 0, 0);
    };
    const int nft = N / kTqCols;
    uint4 cur[4];
    load(blockIdx.y, cur);
    for (int ft = blockIdx.y; ft < nft; ft += gridDim.y) {
        // the next column tile's loads go out before this one is converted
        uint4 nxt[4];
        if (ft + (int)gridDim.y < nft) load(ft + gridDim.y, nxt);
        __syncthreads();                            // the previous tile's readers are done
        // 1. the row's 32 columns into LDS as FP32 (times probs; zero past the rows)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t w[4] = {cur[c].x, cur[c].y, cur[c].z, cur[c].w};
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                tile[row * kTqLd + 32 * half + 8 * c + 2 * z] = sc * bf16lo(w[z]);
                tile[row * kTqLd + 32 * half + 8 * c + 2 * z + 1] = sc * bf16hi(w[z]);
            }
        }
        __syncthreads();
        // 2. column f, rows 32 b .. 32 b + 31 of the tile
        {
            const int f = tid >> 2, b = tid & 3;
            float v[32];
#pragma unroll
            for (int j = 0; j < 32; ++j) v[j] = tile[(32 * b + j) * kTqLd + f];
            uint32_t out[8];
            const uint32_t sb = quant_block32(v, out);
            const int n = ft * kTqCols + f;
            const int kb = kt * 4 + b;                  // MX block along the rows
            if (weights) {
                store_codes32(codes + ((int64_t)e * N + n) * K + 32 * kb, out);
                scales[((int64_t)kt * segs * N + (int64_t)e * N + n) * 4 + b] = (uint8_t)sb;
            } else {
                store_codes32(codes + koff * N + (int64_t)n * kp + 32 * kb, out);
                scales[koff * N / 32 + ((int64_t)kt * N + n) * 4 + b] = (uint8_t)sb;
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) cur[c] = nxt[c];
    }
}

}  // namespace

hipError_t launch_route_scales(const uint8_t* scales, int64_t rows, const int32_t* gather, int64_t R,
                               int K, uint8_t* out, hipStream_t s) {
    if (K % 128 != 0 || rows <= 0 || rows > 0xFFFFFFFFll) return hipErrorInvalidValue;
    if (R == 0) return hipSuccess;
    const int chunks = (K / 128 + kRouteGroups - 1) / kRouteGroups;
    if (chunks > 65535) return hipErrorInvalidValue;
    int64_t grid = (R + kRouteRows - 1) / kRouteRows;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(route_scales_kernel, dim3((unsigned)grid, (unsigned)chunks), dim3(kThreads), 0, s,
                       reinterpret_cast<const uint32_t*>(scales), gather, R, K / 128, (uint32_t)rows,
                       reinterpret_cast<uint32_t*>(out));
    return hipGetLastError();
}

hipError_t launch_quantize_mxfp8(const uint16_t* v, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, bool block_major, hipStream_t s,
                                 const int32_t* rows_dev) {
    if (block_major && K % 128 != 0) return hipErrorInvalidValue;
    const int64_t nblocks = rows * (K / 32);
    if (nblocks == 0) return hipSuccess;
    int64_t grid = (nblocks + kThreads - 1) / kThreads;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, v, nblocks, K / 32,
                       rows, rows_dev, block_major, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_scaled_rows(const uint16_t* dy, int T, int k, const int32_t* slots, const int32_t* gather,
                                 const float* probs, int64_t R, int d, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s) {
    if (d % 128 != 0 || T < 0 || k < 0) return hipErrorInvalidValue;
    if (T == 0 || k == 0 || R == 0) return hipSuccess;
    constexpr int kWavesPerBlock = kThreads / MOE_WAVE;
    int64_t grid = ((int64_t)T + kWavesPerBlock - 1) / kWavesPerBlock;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(mx_scaled_rows_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, dy, T, k, slots, gather,
                       probs, R, d, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_act_backward(const uint16_t* dA, const uint16_t* h, int64_t R, int I, int act,
                                  uint16_t* dh, uint8_t* codes, uint8_t* scales, hipStream_t s) {
    if (I % 64 != 0) return hipErrorInvalidValue;
    const int64_t nb = R * (I / 32);
    if (nb == 0) return hipSuccess;
    int64_t grid = (nb + kThreads - 1) / kThreads;
    if (grid > 65536) grid = 65536;
    const dim3 gd((unsigned)grid), bd(kThreads);
    if (act == kActGeGLU) hipLaunchKernelGGL(mx_act_backward_kernel<kActGeGLU>, gd, bd, 0, s, dA, h, R, I, dh, codes, scales);
    else if (act == kActReGLU) hipLaunchKernelGGL(mx_act_backward_kernel<kActReGLU>, gd, bd, 0, s, dA, h, R, I, dh, codes, scales);
    else hipLaunchKernelGGL(mx_act_backward_kernel<kActSwiGLU>, gd, bd, 0, s, dA, h, R, I, dh, codes, scales);
    return hipGetLastError();
}

hipError_t launch_mx_transpose_quant(const uint16_t* src, int segs, int K, int N, const int32_t* m_indptr,
                                     const int32_t* gather, const float* probs, int T, bool weights,
                                     uint8_t* codes, uint8_t* scales, hipStream_t s) {
    if (segs <= 0 || segs > kThreads || N <= 0 || N % kTqCols != 0) return hipErrorInvalidValue;
    if (weights && (K <= 0 || K % kTqRows != 0)) return hipErrorInvalidValue;
    if (!weights && (!m_indptr || K < 0 || (gather && T <= 0))) return hipErrorInvalidValue;
    // token layout: K is the number of routed rows; the tiles number at most
    // K / 128 + segs (each segment rounds up to a multiple of 128, at least 128)
    const int64_t tiles = weights ? K / kTqRows : (int64_t)K / kTqRows + segs;
    if (tiles > 0x7FFFFFFF) return hipErrorInvalidValue;
    // column tiles of 64 split over up to 4 workgroups per row tile, each walking its share
    const int ngrp = N / kTqCols < 4 ? N / kTqCols : 4;
    const dim3 gd((unsigned)tiles, (unsigned)ngrp, weights ? (unsigned)segs : 1u);
    hipLaunchKernelGGL(mx_transpose_quant_kernel, gd, dim3(kThreads), 0, s, src, segs, K, N, m_indptr, gather, probs,
                       T, weights, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
