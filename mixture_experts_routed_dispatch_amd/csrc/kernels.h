// kernels.h -- host-side launchers of the gfx950 kernels (internal to libmoe).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// Device status bits (the MOE_DEV_* values of moe.h).
constexpr int kDevIdOutOfRange = 1;
constexpr int kDevIdDuplicate = 2;
constexpr int kDevBadIndptr = 4;

// Entries (t, j) handled by one dispatch workgroup.
constexpr int kDispatchChunk = 2048;

inline int dispatch_chunks(int64_t R) { return (int)((R + kDispatchChunk - 1) / kDispatchChunk); }

// dispatch (one launch, no scratch); status is the sticky flag word.  E <= 256.
hipError_t launch_dispatch(const int32_t* ids, const float* scores, int T, int k, int E,
                           int32_t* m_indptr, int32_t* gather, int32_t* slots, float* probs,
                           int32_t* status, hipStream_t s);

// Pre-dispatched rows: validates a caller's m_indptr [E+1] into m_out (all zeros and
// kDevBadIndptr when it does not rise from 0 or passes R) and writes gather[r] = r, r < R.
hipError_t launch_routed_prep(const int32_t* m_in, int E, int64_t R, int32_t* m_out, int32_t* gather,
                              int32_t* status, hipStream_t s);

enum GemmMode { FWD_W13 = 0, FWD_W2 = 1, DGRAD_W2 = 2, DGRAD_W13 = 3, WGRAD_W2 = 4, WGRAD_W13 = 5 };

struct GemmArgs {
    int T, d, I, E, k;
    const int32_t* m_indptr;
    const int32_t* gather;
    const float* probs;
    const uint16_t* x;    // [T, d]
    const uint16_t* w13;  // [E, 2I, d]
    const uint16_t* w2;   // [E, d, I]
    const uint16_t* a;    // [R, I]   SwiGLU output
    const uint16_t* h;    // [R, 2I]  saved gate/up pre-activations
    const uint16_t* dy;   // [T, d]
    const uint16_t* dh;   // [R, 2I]  gradient w.r.t. (gate, up)
    const uint16_t* xg;   // [R, d]   x[gather[r]]              (weight gradients)
    const uint16_t* dys;  // [R, d]   bf16(probs[r] * dy[gather[r]])  (weight gradients)
    uint16_t* out;        // mode output
    uint16_t* out_h;      // FWD_W13 with save: h
    float* part;          // [kMaxPieces, 256 * 256] FP32 partial sums of split weight-gradient tiles
    int4* split;          // [kMaxPieces / 2] split tiles: (e, qt << 16 | pt, pieces, slot0 << 16 | stride)
    int32_t* nsplit;      // number of split tiles of the last weight-gradient launch
    int accumulate;       // weight gradients: add into out instead of overwriting
    int act;              // gated activation (kActSwiGLU / kActGeGLU / kActReGLU)
    // DGRAD_W2, when set: [R, ds_slots] FP32 partial router gradients, slot 4 pt + 2 wp + ah
    // of row r = sum over the 64 columns i of column tile pt, quarter 2 wp + ah, of
    // (dy W2)[r][i] a[r][i]
    float* ds_part;
    int ds_slots;
};

// Pieces of split weight-gradient tiles in one launch (sizes their FP32 partial sums).
constexpr int kMaxPieces = 512;
constexpr size_t kGemmPartBytes = (size_t)kMaxPieces * 256 * 256 * sizeof(float);

hipError_t launch_gemm(GemmMode mode, const GemmArgs& g, int num_cu, hipStream_t s);

// MXFP8 forward products (OCP E4M3 codes, E8M0 scale per 32 along K).
// MX_PLAIN_W13 / MX_WGRAD_W13: MX_PLAIN / MX_WGRAD as a kernel instance of their own (the
// W13-side backward products), so that traces tell them from the W2 side.
enum MxMode { MX_W13 = 0, MX_W2 = 1, MX_PLAIN = 2, MX_WGRAD = 3, MX_PLAIN_W13 = 4, MX_WGRAD_W13 = 5 };

struct MxGemmArgs {
    int T, d, I, E, k;
    const int32_t* m_indptr;
    const int32_t* gather;
    const uint8_t* xq;    // [T, d]      codes of x
    const uint8_t* xs;    // scales of x[gather], block-major words: (g, r) at (g * R + r) * 4
    const uint8_t* w13q;  // [E, 2I, d]
    const uint8_t* w13s;  // block-major words: (g, row) at (g * E 2I + row) * 4, row = e 2I + n
    const uint8_t* w2q;   // [E, d, I]
    const uint8_t* w2s;   // block-major words: (g, row) at (g * E d + row) * 4, row = e d + n
    uint8_t* aq;          // [R, I]      SwiGLU output, re-quantized (MX_W13 output, MX_W2 input)
    uint8_t* as;          // block-major words: (g, r) at (g * R + r) * 4
    uint16_t* o;          // [R, d]      BF16 expert outputs (MX_W2 output)
    int act;              // gated activation of the W13 epilogue
    // MX_W13 of a training forward: BF16 copies kept for the backward (NULL otherwise)
    uint16_t* h_out;      // [R, 2I]     (g, u)
    uint16_t* a_out;      // [R, I]      a before its re-quantization
    // MX_PLAIN (the input-gradient products): D[r][n] = sum_k P_e[n][k] Q[r][k]
    //   P: weight layout, codes [E][Np][Kp], block-major scales [Kp/128][E*Np][4]
    //   Q: routed rows, codes [R][Kp], block-major scales [Kp/128][R][4]
    //   out: BF16 [R][Np]
    // MX_WGRAD (the weight gradients): D_e[q][p] = sum_r Q_e[q][r] P_e[p][r] over the
    // routed rows of expert e, the operands in the token layout: expert e's rows padded to
    // kp_e = roundup(max(rows_e, 1), 128) and prefixed koff_e = sum of kp over the experts
    // before it; codes [N][kp_e] at koff_e * N, scales block-major [kp_e/128][N][4] at
    // byte koff_e * N / 32 (N = Np for P, Nq for Q); out: BF16 [E][Nq][Np], overwritten
    int Kp, Np, Nq;
    const uint8_t* pq;
    const uint8_t* ps;
    const uint8_t* qq;
    const uint8_t* qs;
    uint16_t* out;
    int accumulate;       // MX_WGRAD: out = bf16(out + bf16(D)) instead of bf16(D)
};

hipError_t launch_gemm_mxfp8(MxMode mode, const MxGemmArgs& g, int num_cu, hipStream_t s);

// Token-layout padding of MX_WGRAD operands: kp_e = roundup(max(rows_e, 1), 128); the
// sum over experts is at most R + 128 E.
constexpr int kMxWgradPad = 128;

// MXFP8 quantization for the backward (OCP MX blocks of 32, the same scale rule as
// launch_quantize_mxfp8):
// the routed rows r = slots[t][j] (valid entries: gather[r] == t) of probs[r] *
// dy[gather[r]] along d: codes [R][d], block-major scales [d/128][R][4]; other rows are
// left as they are
hipError_t launch_mx_scaled_rows(const uint16_t* dy, int T, int k, const int32_t* slots, const int32_t* gather,
                                 const float* probs, int64_t R, int d, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
// SwiGLU (GeGLU, ReGLU) backward of MXFP8 training: dg = dA u f'(g), du = dA f(g) from dA
// [R][I] and h = (g, u) [R][2I] (BF16); dh = (dg, du) in BF16 [R][2I] and quantized along
// 2I: codes [R][2I], block-major scales [2I/128][R][4]
hipError_t launch_mx_act_backward(const uint16_t* dA, const uint16_t* h, int64_t R, int I, int act,
                                  uint16_t* dh, uint8_t* codes, uint8_t* scales, hipStream_t s);
// Transposing quantization.  Weight layout (weights != 0): `segs` matrices src + e*K*N of
// K rows x N columns (BF16) become codes [e][N][K] (the transpose, quantized along K) with
// block-major scales [K/128][segs*N][4]; K a multiple of 128.  Token layout (weights == 0):
// segment e is the routed rows m_indptr[e] .. m_indptr[e+1] and becomes codes [N][kp_e]
// at koff_e * N (rows past the segment as zeros) with scales [kp_e/128][N][4] at byte
// koff_e * N / 32 (kp_e, koff_e as for MX_WGRAD); routed row r is src row r, or with
// gather the token row gather[r] of src [T, N] (entries outside [0, T) read row 0), times
// probs[r] when probs is given; K is then the number of routed rows (sizes the grid).
// segs <= 256, N a multiple of 64.
hipError_t launch_mx_transpose_quant(const uint16_t* src, int segs, int K, int N, const int32_t* m_indptr,
                                     const int32_t* gather, const float* probs, int T, bool weights,
                                     uint8_t* codes, uint8_t* scales, hipStream_t s);

// y[t] = sum_j w[t][j] * src[slots[t][j]] (w = NULL means weight 1; slots = NULL means
// row t*k + j), FP32, j ascending.
hipError_t launch_combine(const uint16_t* src, const int32_t* slots, const float* w, int T, int k,
                          int d, uint16_t* y, hipStream_t s);
// ds[t][j] = <dy[t], o[slots[t][j]]> in FP32.
// dS[q] = sum of the nslots partials of q's routed row slots[q], in slot order.
hipError_t launch_score_grad_sum(const float* part, const int32_t* slots, int R, int nslots, float* ds,
                                 hipStream_t s);
hipError_t launch_score_grad(const uint16_t* dy, const uint16_t* o, const int32_t* slots, int T,
                             int k, int d, float* ds, hipStream_t s);

// Operands of the weight gradients: xg[r] = x[gather[r]], dys[r] = bf16(probs[r] *
// dy[gather[r]]), both [R, d], for the routed rows r = slots[t][j] of valid entries
// (gather[r] == t); other rows are left as they are.
hipError_t launch_wgrad_rows(const uint16_t* x, const uint16_t* dy, int T, int k, const int32_t* slots,
                             const int32_t* gather, const float* probs, int d, uint16_t* xg, uint16_t* dys,
                             hipStream_t s);

// Small-batch (decode) path: T*k <= kMaxDecodeRows routed entries, E <= 256.
constexpr int kMaxDecodeRows = 256;

struct DecodeArgs {
    int T, d, I, E, k;
    const int32_t* ids;    // [T, k]
    const float* scores;   // [T, k]
    const uint16_t* x;     // [T, d]
    const uint16_t* w13;   // [E, 2I, d]
    const uint16_t* w2;    // [E, d, I]
    uint16_t* a;           // [T*k, I]  SwiGLU output of entry t*k + j
    uint16_t* o;           // [T*k, d]  expert output of entry t*k + j
    uint16_t* y;           // [T, d]
    int32_t* status;       // sticky routing flags
    int act;               // gated activation of decode W13
};

hipError_t launch_decode_w13(const DecodeArgs& g, int num_cu, hipStream_t s);
hipError_t launch_decode_w2(const DecodeArgs& g, int num_cu, hipStream_t s);
// One token: W2 of all k experts and the score-weighted combine into y (a launch in place
// of decode_w2 and combine).
constexpr int kMaxTopK = 32;
hipError_t launch_decode_w2_one(const DecodeArgs& g, int num_cu, hipStream_t s);
// "Mega" decode: W13 + activation + W2 chunked over I in one launch (chunks of
// mega_chunk(T, k) = 32 intermediate columns), FP32 partial expert outputs in part
// [T*k, I / chunk, d], then a combine launch into y.
int mega_chunk(int T, int k);
hipError_t launch_mega_decode(const DecodeArgs& g, float* part, int num_cu, hipStream_t s);

// block_major: scale word (g, row) (bytes of blocks 4 g .. 4 g + 3) at (g * rows + row) * 4
// (K a multiple of 128); else scales [rows, K/32].
// rows_dev (optional, device): convert only the first min(rows, *rows_dev) rows; the
// block-major layout keeps `rows` as its plane stride
hipError_t launch_quantize_mxfp8(const uint16_t* v, int64_t rows, int K, uint8_t* codes,
                                 uint8_t* scales, bool block_major, hipStream_t s,
                                 const int32_t* rows_dev = nullptr);
// block-major scale words of the routed rows x[gather[r]], r < R, from row-major
// [rows, K/32] scales; K a multiple of 128; gather entries outside [0, rows) read row 0
hipError_t launch_route_scales(const uint8_t* scales, int64_t rows, const int32_t* gather, int64_t R,
                               int K, uint8_t* out, hipStream_t s);

// Scratch for moe_forward_static: one array of kStaticScratchBytes per device (the size
// moe.h states as MOE_STATIC_SCRATCH_BYTES).  static_scratch returns the current device's
// copy (looked up once per device) and its compute-unit count.
constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
hipError_t static_scratch(void** ptr, int* num_cu);
// p[0 .. n) = v, as a kernel (no memset node when the caller captures the stream)
hipError_t launch_fill_i32(int32_t* p, int n, int32_t v, hipStream_t s);

}  // namespace moe
