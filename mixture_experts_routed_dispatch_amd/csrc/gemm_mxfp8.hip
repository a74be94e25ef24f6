// gemm_mxfp8.hip -- grouped MXFP8 GEMMs of the routed expert layer's forward on gfx950.
//
// The blog post ("What it is selling") lists an MXFP8 E4M3 mode: activations are
// quantized after routing and the weights are prepared beforehand.  Both expert
// products then run on OCP MXFP8 operands (E4M3 codes with one E8M0 scale per 32
// consecutive K elements) with FP32 accumulation, using the block-scaled MFMA
// v_mfma_scale_f32_32x32x64_f8f6f4:
//
//   mode      P (p, k)                  Q (q, k)                K     output
//   MX_W13    W13_e rows, gate/up pairs xq[gather[r]], xs       d     a = silu(g)*u re-quantized to
//                                                                     MXFP8 along I: aq [R, I], as [R, I/32]
//                                                                     (training: also h and a in BF16)
//   MX_W2     W2_e rows                 aq[r], as               I     o [R, d] BF16
//   MX_PLAIN  weight-layout rows        routed rows             Kp    BF16 [R, Np]: the input gradients
//             (W2 or W13 prepared transposed)                         dA = W2^T dO, dXp = W13^T dh
//   MX_WGRAD  token-layout rows of      token-layout rows of    rows  BF16 [E, Nq, Np]: the weight
//             a^T or x[gather]^T        dO^T or dh^T            of e  gradients dW2, dW13
//
// MX_WGRAD runs K over an expert's routed rows, quantized in blocks of 32 rows and padded
// to a multiple of 128 (an expert with no row gets 128 zero rows, so its gradient is
// written as +0); its experts are taken in decreasing order of rows, so that the longest
// tiles start first.
// The structure is the BF16 kernel's (workgroup tile 256 x 256, four waves of
// 128 x 128, a ring of four 32 KiB LDS buffers, direct global-to-LDS copies issued
// three stages ahead, one continuous stream of stages per workgroup); a stage is
// 64 K elements = 64 bytes per row = two MX blocks, consumed by one MFMA per
// (row block, column block).  Lane l of an MFMA supplies row l & 31: codes
// 16 (l >> 5) .. + 15 of each of the stage's two MX blocks, and the scale byte of MX
// block (l >> 5) of that row (the instruction applies lane half h's scale to block h
// of the row, whichever lane half holds its codes).
//
// Scales travel as direct copies too: the 4 bytes (blocks 2 kt .. 2 kt + 3) of a
// row cover a pair of stages; per stage pair, each wave copies the words of 64 P
// rows and 64 Q rows into one of three 2 KiB scale slots, together with the data
// copies of the pair's first stage.  The weight scales and the scales of a are
// stored block-major (the words of one stage pair for consecutive rows are
// contiguous), so those copies read 256 contiguous bytes; the scales of x are gathered
// by token, a word per row.  A lane then reads the words of its four row
// blocks once per pair and shifts them by 8 (lane >> 5) bits, so that byte 0 holds
// its scale for the first stage of the pair and byte 2 for the second (the MFMA's
// op_sel picks the byte).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TP = 256, TQ = 256, TKB = 64;   // TKB: K elements (bytes) per stage
constexpr int NBUF = 4;
constexpr int NTHR = 256;
constexpr int OPB = TP * TKB;                 // one operand of one stage: 16 KiB
constexpr int BUFB = 2 * OPB;                 // one stage buffer (P then Q): 32 KiB
constexpr int SCB = 2048;                     // one scale slot: P words then Q words
constexpr int NSC = 3;

typedef int i32x8_t __attribute__((ext_vector_type(8)));

// 64-byte rows, chunk slot c ^ swz(r): conflict-free reads of one chunk of 16 (or 8)
// consecutive rows (see the BF16 kernel).
__device__ __forceinline__ int swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }
__device__ __forceinline__ int lofs(int r, int c) { return r * 64 + ((c ^ swz(r)) << 4); }

// Order of an expert's tiles: groups of kQGroup q-tiles (token rows), and inside a
// group the p-tiles (weight rows) with the group's q-tiles fastest.  The 32 tiles one
// XCD runs at a time (consecutive ids) then span about 6 q-tiles x 5 p-tiles, which
// share far more operand data in that XCD's L2 than 32 tiles of one q-tile row or
// one p-tile column.
constexpr int kQGroup = 6;
__device__ __forceinline__ void tile_order(int local, int nQt, int nPt, int& pt, int& qt) {
    const int gi = local / (kQGroup * nPt);
    const int rem = local - gi * kQGroup * nPt;
    const int left = nQt - gi * kQGroup;
    const int gsz = left < kQGroup ? left : kQGroup;
    pt = rem / gsz;
    qt = gi * kQGroup + (rem - pt * gsz);
}

struct TileCtx {
    int e, mb, rows, pt, qt, nk;
    int koff, kp;                      // MX_WGRAD: the expert's token-layout offset and padded rows
};

// kProd only names the instance (1: the W13-side product of MX_PLAIN / MX_WGRAD), so that
// per-kernel traces and counters tell the two backward products of a mode apart.
template <int MODE, int kAct = kActSwiGLU, bool kSave = false, int kProd = 0>
__global__ __launch_bounds__(NTHR, 1) void grouped_gemm_mx(MxGemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char lds[NBUF * BUFB];
    __shared__ __attribute__((aligned(1024))) char lsc[NSC * SCB];
    __shared__ int cum[257];
    __shared__ int mptr[257];          // m_indptr, so that the tile walk reads no global memory
    __shared__ int gsrc[2][TQ];        // token ids (MX_W13) of the next two load-cursor tiles
    __shared__ int wtot[NTHR / MOE_WAVE];
    __shared__ int worder[256], wkp[256], wkoff[256];   // MX_WGRAD: work order, padded rows, offsets
    constexpr bool kWgrad = MODE == MX_WGRAD;
    // W13 and the weight gradients: the next tile's first stage skips its wait (below)
    constexpr bool kEarlyWait = MODE == MX_W13 || MODE == MX_WGRAD;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The lane id recomputed on the spot (inline mbcnt, which the compiler cannot fold
    // into `lane`), for the code that runs once per tile: lane-dependent offsets hoisted
    // out of the tile loop would be spilled, and a scratch reload waits on vmcnt, i.e.
    // on every copy in flight.
    auto fresh_lane = []() {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        return l;
    };
    const int wp = wave & 1, wq = wave >> 1;
    const int E = g.E;
    // K of the product (bytes per row; MX_WGRAD: per expert, in the tile context)
    const int K = MODE == MX_W13 ? g.d : (MODE == MX_W2 ? g.I : g.Kp);
    const size_t R = (size_t)g.T * g.k;                // routed rows
    const int nPt = MODE == MX_W13 ? g.I / 128 : (MODE == MX_W2 ? g.d / TP : (g.Np + TP - 1) / TP);
    const int nQt = kWgrad ? (g.Nq + TQ - 1) / TQ : 0; // MX_WGRAD: q-tiles per expert

    // exclusive prefix over threads 0 .. E-1 of v into out[1 .. E], out[0] = 0 (ends with a barrier)
    auto block_scan = [&](int v, int* out) {
        int incl = v;
        for (int off = 1; off < MOE_WAVE; off <<= 1) {
            const int u = __shfl_up(incl, off, MOE_WAVE);
            if (lane >= off) incl += u;
        }
        if (lane == MOE_WAVE - 1) wtot[wave] = incl;
        __syncthreads();
        int pre = 0;
        for (int w = 0; w < wave; ++w) pre += wtot[w];
        if (tid < E) out[tid + 1] = pre + incl;
        if (tid == 0) out[0] = 0;
        __syncthreads();
    };
    // ---- tile list: tiles of expert e (MX_WGRAD: of work position e) are cum[e] .. cum[e+1]-1
    for (int i = tid; i <= E; i += NTHR) mptr[i] = g.m_indptr[i];
    __syncthreads();
    if constexpr (kWgrad) {
        // padded rows and token-layout offsets in expert order, then the work order:
        // decreasing padded rows, then expert id
        const int kp = tid < E ? ((mptr[tid + 1] - mptr[tid] > 0 ? mptr[tid + 1] - mptr[tid] : 1) + kMxWgradPad - 1) /
                                     kMxWgradPad * kMxWgradPad
                               : 0;
        block_scan(kp, cum);
        if (tid < E) { wkp[tid] = kp; wkoff[tid] = cum[tid]; }
        __syncthreads();
        if (tid < E) {
            int rank = 0;
            for (int e2 = 0; e2 < E; ++e2) rank += (wkp[e2] > kp || (wkp[e2] == kp && e2 < tid)) ? 1 : 0;
            worder[rank] = tid;
        }
        __syncthreads();
        block_scan(tid < E ? nQt * nPt : 0, cum);
    } else {
        int cnt = 0;
        if (tid < E) {
            const int rows = mptr[tid + 1] - mptr[tid];
            cnt = ((rows + TQ - 1) / TQ) * nPt;
        }
        block_scan(cnt, cum);
    }
    const int total = cum[E];
    const int G = gridDim.x;
    const int vid = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    if (vid >= total) return;

    auto coords = [&](int tile) {
        // largest e with cum[e] <= tile = number of e in [1, E) with cum[e] <= tile
        const int fl = fresh_lane();
        int lo = 0;
#pragma unroll
        for (int base = 1; base < 257; base += 64) {
            const int e = base + fl;
            lo += __builtin_popcountll(__ballot(e < E && cum[e] <= tile));
        }
        lo = __builtin_amdgcn_readfirstlane(lo);
        TileCtx c;
        const int local = tile - cum[lo];
        if constexpr (kWgrad) {
            c.e = __builtin_amdgcn_readfirstlane(worder[lo]);
            c.mb = 0;
            c.rows = g.Nq;                            // q rows of the tile are features
            c.qt = local / nPt;
            c.pt = local - c.qt * nPt;
            c.kp = __builtin_amdgcn_readfirstlane(wkp[c.e]);
            c.koff = __builtin_amdgcn_readfirstlane(wkoff[c.e]);
            c.nk = c.kp / TKB;                        // even: kp is a multiple of 128
        } else {
            c.e = lo;
            c.mb = mptr[lo];
            c.rows = mptr[lo + 1] - c.mb;
            tile_order(local, (c.rows + TQ - 1) / TQ, nPt, c.pt, c.qt);
            c.nk = K / TKB;                           // even: K is a multiple of 128
            c.kp = K;
            c.koff = 0;
        }
        return c;
    };

    // row of the P operand (weight row of expert e) behind P tile row r
    auto p_row = [&](const TileCtx& c, int r) {
        if constexpr (MODE == MX_W13) {
            // 32-row block j of the tile: gate rows i0 + 16 j + (0..15), then the up rows of
            // the same i, so that an MFMA tile holds both halves of its 16 outputs
            int ii = c.pt * 128 + (r >> 5) * 16 + (r & 15);
            if (ii >= g.I) ii = g.I - 1;
            return (r & 16) ? g.I + ii : ii;
        } else if constexpr (MODE == MX_W2) {
            const int pr = c.pt * TP + r;
            return pr < g.d ? pr : g.d - 1;
        } else {
            const int pr = c.pt * TP + r;
            return pr < g.Np ? pr : g.Np - 1;
        }
    };
    // row of the Q operand (token of xq, or routed row of aq) behind Q tile row r, for
    // the rows r = 64 w .. 64 w + 63 of wave w only: the token ids come from gsrc[slot],
    // where gather_dma put them
    auto routed_row = [&](const TileCtx& c, int r) {
        int rr = c.qt * TQ + r;
        if (rr >= c.rows) rr = c.rows - 1;            // ragged tail: a row of the expert
        return c.mb + rr;
    };
    auto q_row = [&](const TileCtx& c, int slot, int r) {
        if constexpr (MODE == MX_W13) return gsrc[slot][r];
        else return routed_row(c, r);                 // MX_WGRAD: the feature row (mb = 0, rows = Nq)
    };
    // Token ids of tile c into gsrc[slot]: wave w copies entries 64 w .. 64 w + 63 (the
    // rows of its own data and scale copies) with one global_load_lds_dword, issued a
    // tile ahead and counted like the stage copies; a plain load would make the
    // compiler wait for every copy in flight.
    auto gather_dma = [&](const TileCtx& c, int slot) {
        if constexpr (MODE == MX_W13) {
            int rr = c.qt * TQ + 64 * wave + fresh_lane();
            if (rr >= c.rows) rr = c.rows - 1;                    // tiles exist only for rows >= 1
            const uint32_t voff = (uint32_t)(c.mb + rr) * 4u;
            const uint32_t dst = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int*)&gsrc[slot][64 * wave];
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                         :: "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(g.gather) : "memory");
        }
    };
    const uint8_t* pdata = MODE == MX_W13 ? g.w13q : (MODE == MX_W2 ? g.w2q : g.pq);
    const uint8_t* pscale = MODE == MX_W13 ? g.w13s : (MODE == MX_W2 ? g.w2s : g.ps);
    const uint8_t* qdata = MODE == MX_W13 ? g.xq : (MODE == MX_W2 ? g.aq : g.qq);
    const uint8_t* qscale = MODE == MX_W13 ? g.xs : (MODE == MX_W2 ? g.as : g.qs);
    // P rows per expert
    const size_t prows_e = MODE == MX_W13 ? (size_t)2 * g.I : (MODE == MX_W2 ? (size_t)g.d : (size_t)g.Np);

    // ------------------------------------------------------------ direct copies
    // Data: wave w copies the 1 KiB blocks 4w .. 4w+3 of each operand of a stage;
    // lane L fetches 16 bytes that land at (block start + 16 L) = row 16 blk + L/4,
    // chunk slot L%4, i.e. logical chunk (L%4) ^ swz(row).
    // Scales: wave w copies the 4-byte words (blocks 2 kt .. 2 kt+3) of P and Q tile
    // rows 64 w + L to (slot + 256 w + 4 L) and (slot + 1024 + 256 w + 4 L).
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
    const uint32_t lsc0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lsc;
    uint32_t dvoff[8];
    uint32_t svoffP = 0, svoffQ = 0;
    const char* pbase_e = nullptr;
    const char* psbase_e = nullptr;
    const char* qbase_e = reinterpret_cast<const char*>(qdata);     // per expert in MX_WGRAD
    const char* qsbase_e = reinterpret_cast<const char*>(qscale);
    // bytes between the scale words of consecutive 128-element K groups
    size_t pscale_stride = (size_t)E * prows_e * 4, qscale_stride = R * 4;
    auto copy_offsets = [&](const TileCtx& c, int slot) {
        const int fl = fresh_lane();
        const int Kt = c.kp;                                    // this tile's K (bytes per row)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (4 * wave + j) * 16 + (fl >> 2);
            const int cl = (fl & 3) ^ swz(r);
            dvoff[j] = (uint32_t)(p_row(c, r) * Kt + 16 * cl);
            dvoff[4 + j] = (uint32_t)(q_row(c, slot, r) * Kt + 16 * cl);
        }
        const int rs = 64 * wave + fl;
        svoffP = (uint32_t)(p_row(c, rs) * 4);
        svoffQ = (uint32_t)(routed_row(c, rs) * 4);          // Q scales are in routed (feature) order
        if constexpr (kWgrad) {
            pbase_e = reinterpret_cast<const char*>(pdata + (size_t)c.koff * g.Np);
            psbase_e = reinterpret_cast<const char*>(pscale + (size_t)c.koff * g.Np / 32);
            qbase_e = reinterpret_cast<const char*>(qdata + (size_t)c.koff * g.Nq);
            qsbase_e = reinterpret_cast<const char*>(qscale + (size_t)c.koff * g.Nq / 32);
            pscale_stride = (size_t)g.Np * 4;
            qscale_stride = (size_t)g.Nq * 4;
        } else {
            pbase_e = reinterpret_cast<const char*>(pdata + (size_t)c.e * prows_e * K);
            psbase_e = reinterpret_cast<const char*>(pscale + (size_t)c.e * prows_e * 4);
        }
    };
    auto dma16 = [&](uint32_t lds_addr, uint32_t voff, const char* base) {
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(base) : "memory");
    };
    auto dma4 = [&](uint32_t lds_addr, uint32_t voff, const char* base) {
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(base) : "memory");
    };
    // data copy j (0..3 P, 4..7 Q) of stage kt into ring buffer buf
    auto dma_data = [&](int kt, int buf, int j) {
        const uint32_t dst = lds0 + buf * BUFB + (4 * wave) * 1024;
        if (j < 4) dma16(dst + j * 1024, dvoff[j], pbase_e + kt * TKB);
        else dma16(dst + OPB + (j - 4) * 1024, dvoff[j], qbase_e + kt * TKB);
    };
    // scale words of the stage pair holding stage kt (blocks 2 (kt & ~1) .. +3) into
    // scale slot `slot`
    auto dma_scales = [&](int kt, int slot) {
        const uint32_t dst = lsc0 + slot * SCB + 256 * wave;
        const size_t kp = (size_t)(kt >> 1);                  // stage pair = group of 4 blocks
        dma4(dst, svoffP, psbase_e + kp * pscale_stride);
        dma4(dst + 1024, svoffQ, qsbase_e + kp * qscale_stride);
    };

    // ------------------------------------------------------------ fragments and scales
    // fragment b of P (Q): row wp*128 + 32 b + (lane & 31) (wq*128 + ...). The scaled
    // 32x32x64 fp8 MFMA takes, in lane half g = lane >> 5, bytes 16g..16g+15 of both MX
    // blocks of the stage: block 0 in registers 0-3, block 1 in registers 4-7 (chunks g
    // and 2 + g of the 64-byte row); the scale of (row, block h) sits in lane half h
    // (recomputed after every epilogue from the lane id read afresh, so that they are not
    // held across it: the epilogue of the training forward, which also stores h and a,
    // runs short of registers)
    int fragP[4][2], fragQ[4][2];
    auto frag_offsets = [&]() {
        const int fl = fresh_lane();
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                fragP[b][h] = lofs(wp * 128 + b * 32 + (fl & 31), (fl >> 5) + 2 * h);
                fragQ[b][h] = OPB + lofs(wq * 128 + b * 32 + (fl & 31), (fl >> 5) + 2 * h);
            }
    };
    frag_offsets();
    auto read_frag = [&](const char* base, int off0, int off1) {
        const uint4 x = *reinterpret_cast<const uint4*>(base + off0);
        const uint4 y = *reinterpret_cast<const uint4*>(base + off1);
        i32x8_t v;
        v[0] = (int)x.x; v[1] = (int)x.y; v[2] = (int)x.z; v[3] = (int)x.w;
        v[4] = (int)y.x; v[5] = (int)y.y; v[6] = (int)y.z; v[7] = (int)y.w;
        return v;
    };
    // this lane's scale words of its four P and four Q row blocks, from scale slot
    // `slot`, shifted so that byte 0 / byte 2 are its blocks of the pair's two stages
    auto read_scales = [&](int slot, int sp[4], int sq[4]) {
        const char* base = lsc + slot * SCB;
        const int sh = 8 * (lane >> 5);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            sp[b] = (int)(*reinterpret_cast<const uint32_t*>(base + 4 * (wp * 128 + b * 32 + (lane & 31))) >> sh);
            sq[b] = (int)(*reinterpret_cast<const uint32_t*>(base + 1024 + 4 * (wq * 128 + b * 32 + (lane & 31))) >> sh);
        }
    };

    f32x16_t acc[4][4];
    // One stage: 16 scaled MFMAs in four groups (row block a); each group also reads
    // P and Q fragment a of the next stage (from ring buffer nbuf) and issues data copies
    // 2a and 2a + 1 of the stage being prefetched.  OPSEL picks the scale byte.
    auto stage = [&](auto opsel_tag, const i32x8_t pf[4], const i32x8_t qf[4], const int sp[4], const int sq[4],
                     int nbuf, i32x8_t npf[4], i32x8_t nqf[4], int dma_kt, int dma_buf) {
        constexpr int OPSEL = decltype(opsel_tag)::value;
        const char* nb = lds + nbuf * BUFB;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            // The scaled MFMAs have no ordering edge to anything here, and instruction
            // selection would otherwise emit all of them after the stage's reads and
            // copies; an empty asm that takes the accumulators just written keeps them
            // in front of the next copy.  One copy after every two MFMAs: copies issued
            // back to back queue in the texture unit and hold up the MFMA issue.
            acc[a][0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pf[a], qf[0], acc[a][0], 0, 0, OPSEL, sp[a], OPSEL, sq[0]);
            npf[a] = read_frag(nb, fragP[a][0], fragP[a][1]);
            acc[a][1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pf[a], qf[1], acc[a][1], 0, 0, OPSEL, sp[a], OPSEL, sq[1]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            asm volatile("" :: "a"(acc[a][0]), "a"(acc[a][1]));
            dma_data(dma_kt, dma_buf, 2 * a);
            __builtin_amdgcn_sched_barrier(0);
            nqf[a] = read_frag(nb, fragQ[a][0], fragQ[a][1]);
            acc[a][2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pf[a], qf[2], acc[a][2], 0, 0, OPSEL, sp[a], OPSEL, sq[2]);
            acc[a][3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(pf[a], qf[3], acc[a][3], 0, 0, OPSEL, sp[a], OPSEL, sq[3]);
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            asm volatile("" :: "a"(acc[a][2]), "a"(acc[a][3]));
            dma_data(dma_kt, dma_buf, 2 * a + 1);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ------------------------------------------------------------ epilogue
    auto epilogue = [&](const TileCtx& c, int buf) {
        const int ln = fresh_lane();
        const int q_in = ln & 31, p_sub = 4 * (ln >> 5);
        if constexpr (MODE == MX_W13) {
            // a = silu(g) * u for i = pt*128 + wp*64 + 32 m + (0..31): one MX block per
            // (row, m), from MFMA tiles a = 2 m and 2 m + 1, whose element groups 0, 1 hold
            // gate values and 2, 3 the matching up values (outputs 16 a + 8 grp + p_sub + z),
            // split over lanes l and l ^ 32; amax, E8M0 scale and E4M3 codes
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                __builtin_amdgcn_sched_barrier(0);
                const int rr = c.qt * TQ + wq * 128 + b * 32 + q_in;
                const bool live = rr < c.rows;
                const size_t r = (size_t)c.mb + (live ? rr : 0);
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    float av[16];
                    float amax = 0.0f;
#pragma unroll
                    for (int h = 0; h < 2; ++h)
#pragma unroll
                        for (int grp = 0; grp < 2; ++grp)
#pragma unroll
                            for (int z = 0; z < 4; ++z) {
                                const float gv = acc[2 * m + h][b][4 * grp + z];
                                const float uv = acc[2 * m + h][b][4 * (grp + 2) + z];
                                const float v = act_f<kAct>(gv) * uv;
                                av[8 * h + 4 * grp + z] = v;
                                amax = __builtin_fmaxf(amax, __builtin_fabsf(v));
                                if constexpr (kSave) {
                                    // the training forward keeps h = (g, u) in BF16, staged
                                    // through this wave's 8 KiB of the stage buffer just
                                    // consumed: row q_in (256 bytes) holds its 64 gate values
                                    // (16-byte chunks 0..7) and 64 up values (chunks 8..15)
                                    if (z & 1) {
                                        const float gp = acc[2 * m + h][b][4 * grp + z - 1];
                                        const float up = acc[2 * m + h][b][4 * (grp + 2) + z - 1];
                                        const int cg = 2 * (2 * m + h) + grp;
                                        char* srow = lds + buf * BUFB + wave * 8192 + q_in * 256 + (p_sub << 1) +
                                                     ((z >> 1) << 2);
                                        *reinterpret_cast<uint32_t*>(srow + ((cg ^ (q_in & 15)) << 4)) = pack_bf16(gp, gv);
                                        *reinterpret_cast<uint32_t*>(srow + (((8 + cg) ^ (q_in & 15)) << 4)) = pack_bf16(up, uv);
                                    }
                                }
                            }
                    amax = __builtin_fmaxf(amax, __shfl_xor(amax, 32, 64));
                    const uint32_t sb = e8m0_scale(amax);
                    const int sh = 127 - (int)sb;
                    const int i0 = c.pt * 128 + wp * 64 + m * 32;
                    if (live && i0 < g.I) {
#pragma unroll
                        for (int h = 0; h < 2; ++h)
#pragma unroll
                            for (int grp = 0; grp < 2; ++grp) {
                                const float* q = &av[8 * h + 4 * grp];
                                const uint32_t w = e4m3_pack4(__builtin_ldexpf(q[0], sh), __builtin_ldexpf(q[1], sh),
                                                              __builtin_ldexpf(q[2], sh), __builtin_ldexpf(q[3], sh));
                                const int i = i0 + 16 * h + 8 * grp + p_sub;
                                *reinterpret_cast<uint32_t*>(g.aq + r * g.I + i) = w;
                                if constexpr (kSave) {
                                    // and a before its re-quantization, in BF16
                                    uint2 av2;
                                    av2.x = pack_bf16(q[0], q[1]); av2.y = pack_bf16(q[2], q[3]);
                                    *reinterpret_cast<uint2*>(g.a_out + r * g.I + i) = av2;
                                }
                            }
                        if (ln < 32) g.as[((size_t)(i0 >> 7) * R + r) * 4 + ((i0 >> 5) & 3)] = (uint8_t)sb;
                    }
                }
                if constexpr (kSave) {
                    // the staged h rows go out as two 128-byte segments each (g, then u)
                    __builtin_amdgcn_s_waitcnt(0xc07f);
                    const char* stg = lds + buf * BUFB + wave * 8192;
                    const int ibase = c.pt * 128 + wp * 64;
#pragma unroll
                    for (int it = 0; it < 8; ++it) {
                        const int row = 4 * it + (ln >> 4);
                        const int c16 = ln & 15;
                        const uint4 v = *reinterpret_cast<const uint4*>(stg + row * 256 + ((c16 ^ (row & 15)) << 4));
                        const int rr2 = c.qt * TQ + wq * 128 + b * 32 + row;
                        const int i = ibase + 8 * (c16 & 7);
                        if (rr2 < c.rows && i < g.I)
                            *reinterpret_cast<uint4*>(g.h_out + ((size_t)c.mb + rr2) * 2 * g.I + (c16 >> 3) * g.I + i) = v;
                    }
                    __builtin_amdgcn_s_waitcnt(0xc07f);
                }
            }
        } else {
            // o [R, d] (MX_PLAIN: [R, Np]; MX_WGRAD: expert e's [Nq, Np]) in BF16 through
            // LDS (this wave's 8 KiB of the stage buffer just consumed), stored as whole
            // 256-byte row segments with non-temporal stores (ordinary ones evict the
            // operands the XCD's workgroups share in L2)
            uint16_t* obase = MODE == MX_W2 ? g.o : g.out;
            const int ld = MODE == MX_W2 ? g.d : g.Np;
            if constexpr (kWgrad) obase += (size_t)c.e * g.Nq * g.Np;
            char* stg = lds + buf * BUFB + wave * 8192;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int grp = 0; grp < 4; ++grp) {
                        const int c16 = 4 * a + grp;
                        uint2 v;
                        v.x = pack_bf16(acc[a][b][4 * grp + 0], acc[a][b][4 * grp + 1]);
                        v.y = pack_bf16(acc[a][b][4 * grp + 2], acc[a][b][4 * grp + 3]);
                        *reinterpret_cast<uint2*>(stg + q_in * 256 + ((c16 ^ (q_in & 15)) << 4) + (p_sub << 1)) = v;
                    }
                __builtin_amdgcn_s_waitcnt(0xc07f);
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const int row = 4 * it + (ln >> 4);
                    const int c16 = ln & 15;
                    const uint4 v = *reinterpret_cast<const uint4*>(stg + row * 256 + ((c16 ^ (row & 15)) << 4));
                    const int rr = c.qt * TQ + wq * 128 + b * 32 + row;
                    const int p = c.pt * TP + wp * 128 + 8 * c16;
                    if (rr < c.rows && p < ld) {
                        uint16_t* dst = obase + ((size_t)c.mb + rr) * ld + p;
                        if (kWgrad && g.accumulate) {
                            // in-place accumulation: the BF16 gradient added to the value
                            // there in FP32, one rounding
                            const uint4 o = *reinterpret_cast<const uint4*>(dst);
                            const uint32_t ov[4] = {o.x, o.y, o.z, o.w}, nv[4] = {v.x, v.y, v.z, v.w};
                            uint32_t sv[4];
#pragma unroll
                            for (int z = 0; z < 4; ++z)
                                sv[z] = pack_bf16(bf16lo(ov[z]) + bf16lo(nv[z]), bf16hi(ov[z]) + bf16hi(nv[z]));
                            store_nt(dst, make_uint4(sv[0], sv[1], sv[2], sv[3]));
                        } else {
                            store_nt(dst, v);
                        }
                    }
                }
                __builtin_amdgcn_s_waitcnt(0xc07f);
            }
        }
    };

    // ------------------------------------------------------------ stage stream
    // As in the BF16 kernel: during stage s the data copies of stage s + 3 are issued
    // (and, when s + 3 starts a stage pair, its scale words first), the barrier ending
    // stage s publishes stage s + 2.  Copies issued after those of stage s + 2 are the
    // 8 data copies of stage s + 3, plus the 2 scale copies when s is odd.
    int l_tile = vid, l_kt = 0;
    TileCtx lc = coords(l_tile);
    TileCtx nc = lc;                   // coordinates of the load cursor's next tile
    int gslot = 0;                     // gsrc slot of the load cursor's tile
    gather_dma(lc, 0);
    if (l_tile + G < total) { nc = coords(l_tile + G); gather_dma(nc, 1); }
    if constexpr (MODE == MX_W13) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    copy_offsets(lc, 0);
    // The token ids of a new tile were copied at the previous switch, a whole tile of
    // at least 2 stages earlier (K is a multiple of 128), and every stage ends with a
    // wait that retires all copies issued before the previous stage.
    auto advance_load = [&]() {
        if (++l_kt < lc.nk) return;
        if (l_tile + G >= total) { l_kt = lc.nk - 1; return; }   // past the end: repeat the last stage
        if constexpr (MODE == MX_W13) if (lc.nk < 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        l_kt = 0;
        l_tile += G;
        gslot ^= 1;
        lc = nc;
        copy_offsets(lc, gslot);
        if (l_tile + G < total) { nc = coords(l_tile + G); gather_dma(nc, gslot ^ 1); }
    };
    auto issue_stage = [&](int buf, int pair_slot) {
        if (pair_slot >= 0) dma_scales(l_kt, pair_slot);
#pragma unroll
        for (int j = 0; j < 8; ++j) dma_data(l_kt, buf, j);
    };

    // prologue: stages 0, 1, 2, with the scale words of pairs 0 and 1
    issue_stage(0, 0);
    advance_load();
    issue_stage(1, -1);
    advance_load();
    issue_stage(2, 1);
    advance_load();
    asm volatile("s_waitcnt vmcnt(10)" ::: "memory");   // stages 0, 1 and pair 0's scales landed
    __syncthreads();

    i32x8_t pa[4], qa[4], pb[4], qb[4];
    int spa[4], sqa[4], spb[4], sqb[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        pa[b] = read_frag(lds, fragP[b][0], fragP[b][1]);
        qa[b] = read_frag(lds, fragQ[b][0], fragQ[b][1]);
    }
    read_scales(0, spa, sqa);

    int c_tile = vid;
    TileCtx cc = coords(c_tile);
    int gs = 0;
    while (true) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
        for (int kt = 0; kt < cc.nk; kt += 2, gs += 2) {
            const int pair = gs >> 1;
            // even stage gs: fragments (pa, qa), scale byte 0; copies of stage gs + 3
            // (odd: no scales)
            stage(std::integral_constant<int, 0>(), pa, qa, spa, sqa, (gs + 1) & 3, pb, qb, l_kt, (gs + 3) & 3);
            advance_load();
            // stage gs + 2 has landed; in a tile's first stage it already had (kEarlyWait)
            if (!kEarlyWait || kt != 0 || c_tile == vid) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
            __syncthreads();
            // odd stage gs + 1: fragments (pb, qb), scale byte 2; copies of stage gs + 4
            // after the scale words of the pair it starts; the next pair's scale words
            // (copied one pair ahead) are read for the next even stage
            read_scales((pair + 1) % NSC, spb, sqb);
            dma_scales(l_kt, (pair + 2) % NSC);
            stage(std::integral_constant<int, 2>(), pb, qb, spa, sqa, (gs + 2) & 3, pa, qa, l_kt, (gs + 4) & 3);
            advance_load();
            asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
            __syncthreads();
#pragma unroll
            for (int b = 0; b < 4; ++b) { spa[b] = spb[b]; sqa[b] = sqb[b]; }
        }
        // kEarlyWait: every copy issued so far lands before the epilogue's first store, so
        // that the next tile's first stage need not wait: its wait would count the
        // epilogue's stores and hold the stage until they are written
        if constexpr (kEarlyWait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        epilogue(cc, (gs - 1) & 3);
        c_tile += G;
        if (c_tile >= total) break;
        __syncthreads();               // the staging slots are copied into again from the next stage
        cc = coords(c_tile);
        frag_offsets();
        // the next tile's first stage again, from its ring buffer and scale slot (neither
        // is written before that stage runs), so that its fragments are not held in
        // registers across the epilogue
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            pa[b] = read_frag(lds + (gs & 3) * BUFB, fragP[b][0], fragP[b][1]);
            qa[b] = read_frag(lds + (gs & 3) * BUFB, fragQ[b][0], fragQ[b][1]);
        }
        read_scales((gs >> 1) % NSC, spa, sqa);
    }
}

template <int MODE, int kAct, int kProd>
hipError_t launch_mx_act(const MxGemmArgs& g, dim3 grid, hipStream_t s) {
    if constexpr (MODE == MX_W13)
        if (g.h_out) {
            hipLaunchKernelGGL((grouped_gemm_mx<MODE, kAct, true, kProd>), grid, dim3(NTHR), 0, s, g);
            return hipGetLastError();
        }
    hipLaunchKernelGGL((grouped_gemm_mx<MODE, kAct, false, kProd>), grid, dim3(NTHR), 0, s, g);
    return hipGetLastError();
}

template <int MODE, int kProd = 0>
hipError_t launch_mx_mode(const MxGemmArgs& g, int num_cu, hipStream_t s) {
    const int64_t R = (int64_t)g.T * g.k;
    int64_t tiles;
    if constexpr (MODE == MX_W13) tiles = (R / TQ + g.E) * (g.I / 128);
    else if constexpr (MODE == MX_W2) tiles = (R / TQ + g.E) * (g.d / TP);
    else if constexpr (MODE == MX_PLAIN) tiles = (R / TQ + g.E) * ((g.Np + TP - 1) / TP);
    else tiles = (int64_t)g.E * ((g.Np + TP - 1) / TP) * ((g.Nq + TQ - 1) / TQ);
    int64_t grid = tiles < num_cu ? tiles : num_cu;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    const dim3 gd((unsigned)grid);
    if constexpr (MODE == MX_W13) {
        if (g.act == kActGeGLU) return launch_mx_act<MODE, kActGeGLU, kProd>(g, gd, s);
        if (g.act == kActReGLU) return launch_mx_act<MODE, kActReGLU, kProd>(g, gd, s);
    }
    return launch_mx_act<MODE, kActSwiGLU, kProd>(g, gd, s);
}

}  // namespace

hipError_t launch_gemm_mxfp8(MxMode mode, const MxGemmArgs& g, int num_cu, hipStream_t s) {
    switch (mode) {
        case MX_W13: return launch_mx_mode<MX_W13>(g, num_cu, s);
        case MX_W2: return launch_mx_mode<MX_W2>(g, num_cu, s);
        case MX_PLAIN: return launch_mx_mode<MX_PLAIN>(g, num_cu, s);
        case MX_WGRAD: return launch_mx_mode<MX_WGRAD>(g, num_cu, s);
        case MX_PLAIN_W13: return launch_mx_mode<MX_PLAIN, 1>(g, num_cu, s);
        case MX_WGRAD_W13: return launch_mx_mode<MX_WGRAD, 1>(g, num_cu, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
