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

}  // namespace moe
