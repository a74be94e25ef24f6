// mxfp8_quant.hip -- OCP MXFP8 (E4M3 elements, E8M0 scale per 32) conversion on gfx950.
//
// The blog post ("What it is selling") names MXFP8 E4M3 with prepared weights
// and activations quantized after routing.  The conversion rule is the OCP MX
// v1.0 one: per block of 32 values along K, the shared exponent is
// floor(log2(max|v|)) - 8 (8 = largest E4M3 exponent), stored biased by 127
// and clamped to [0, 254] (0 for an all-zero block); each element is
// v / 2^(shared) rounded to nearest even on the E4M3 grid and clamped to
// +-448.  Inputs are BF16, so v / 2^(shared) is exact in FP32 and the
// codes are a deterministic function of the input bits.
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
                                                            bool block_major,
                                                            uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ scales) {
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
            const uint32_t c0 = e4m3_code(__builtin_ldexpf(bf16lo(w[2 * i]), sh));
            const uint32_t c1 = e4m3_code(__builtin_ldexpf(bf16hi(w[2 * i]), sh));
            const uint32_t c2 = e4m3_code(__builtin_ldexpf(bf16lo(w[2 * i + 1]), sh));
            const uint32_t c3 = e4m3_code(__builtin_ldexpf(bf16hi(w[2 * i + 1]), sh));
            out[i] = c0 | (c1 << 8) | (c2 << 16) | (c3 << 24);
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

}  // namespace

hipError_t launch_quantize_mxfp8(const uint16_t* v, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, bool block_major, hipStream_t s) {
    if (block_major && K % 128 != 0) return hipErrorInvalidValue;
    const int64_t nblocks = rows * (K / 32);
    if (nblocks == 0) return hipSuccess;
    int64_t grid = (nblocks + kThreads - 1) / kThreads;
    if (grid > 65536) grid = 65536;
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, s, v, nblocks, K / 32,
                       rows, block_major, codes, scales);
    return hipGetLastError();
}

}  // namespace moe
