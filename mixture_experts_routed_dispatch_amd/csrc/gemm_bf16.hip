// gemm_bf16.hip -- grouped BF16 GEMMs of the routed expert layer on gfx950 MFMA.
//
// One persistent kernel template covers the six expert products of forward
// (FPROP) and backward (DGRAD, WGRAD) (blog post "What it is selling"; nvfp4moe
// README "Grouped GEMM": expert-major rows, m_indptr of length E+1, empty
// experts valid; "Supported kernel surface": fused SwiGLU FC1 epilogue,
// grouped input- and weight-gradient kernels).
//
// Every product is written as   D[q][p] = sum_k Q[q][k] * P[p][k]
// where p runs along the contiguous dimension of the output and q along its
// rows.  The MFMA v_mfma_f32_32x32x16_bf16 takes P as its A operand and Q as
// its B operand, so a lane ends up holding 4 consecutive p of one output row.
//
//   mode       P (p, k)                     Q (q, k)                  K      output
//   FWD_W13    W13_e rows, gate/up paired   x[gather[r]]  (K-major)   d      a = silu(g)*u [R, I] (+h)
//   FWD_W2     W2_e rows                    a[r]                      I      o [R, d]
//   DGRAD_W2   W2_e^T  (MN-major)           dy[gather[r]]             d      dh = SwiGLU'(h) * probs * W2^T dy
//   DGRAD_W13  W13_e^T (MN-major)           dh[r]                     2I     dxp [R, d]
//   WGRAD_W2   a^T     (MN-major)           dys^T (MN-major)          R_e    dW2_e [d, I]
//   WGRAD_W13  xg^T    (MN-major)           dh^T  (MN-major)          R_e    dW13_e [2I, d]
//
// (xg = x[gather], dys = bf16(probs * dy[gather]): row-major copies made once before
// the weight gradients, so that every operand is a plain slab the copies can move.)
//
// Workgroup tile 256 (p) x 256 (q), four waves of 128 x 128 (4 x 4 MFMA blocks
// of 32 x 32, 256 FP32 accumulators per lane), one workgroup per CU, persistent
// over a tile list built on the device from m_indptr (the host never reads routing
// counts).  K advances in stages of 32 through a ring of four LDS buffers (32 KiB
// each: both operands, rows of 64 bytes whose 16-byte chunks are XOR-swizzled so
// fragment reads and chunk writes are bank-conflict free).  A workgroup walks its
// tiles as one continuous stream of stages; during stage s it
//   * computes stage s from buffer s % 4: two k steps of 16 MFMAs, the fragments of
//     the second step read in the shadow of the first step's MFMAs, those of stage
//     s + 1's first step in the shadow of the second step's;
//   * issues the direct global-to-LDS copies of stage s + 3, one 1 KiB copy after
//     each group of four MFMAs (a burst of copies stalls the MFMA issue), waited for
//     with explicit vmcnt counts one stage later;
// and ends with one barrier.  K-major operands are staged as rows of K; MN-major
// operands (the transposed products of backward) as rows of M or N, read into MFMA
// fragments with the transposing LDS read ds_read_b64_tr_b16.  The tile walk keeps
// the expert offsets and the next tiles' gather indices in LDS (the latter fetched by
// an LDS copy a tile ahead), so the main loop issues no global load the compiler would
// have to wait for: such a wait would also wait for every copy in flight.  Consecutive
// work items go to workgroups of one XCD so that the operand slices they share stay
// in its L2.  The weight gradients order and cut their tiles for balance (see the
// work list below) and add split tiles up in wgrad_fixup.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int TP = 256, TQ = 256, TK = 32;
constexpr int NBUF = 4;
constexpr int NTHR = 256;
constexpr int OPB = TP * TK * 2;          // one operand of one stage: 16 KiB
constexpr int BUFB = 2 * OPB;             // one stage buffer (P then Q): 32 KiB

// Byte offset of logical 16-byte chunk c (k = 8c .. 8c+7 of the stage) of row r in
// an operand tile: 64-byte rows, chunk slot c ^ swz(r).  swz maps bits (2, 3) of r
// one-to-one for fixed bits (0, 1), and bits (1, 2) one-to-one for fixed bits
// (0, 3), so the same chunk of 16 consecutive rows covers all sixteen 16-byte slots
// of a 256-byte bank line, and of 8 consecutive rows all eight slots of a 128-byte
// line: fragment reads are free of bank conflicts with 64 or 32 banks.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) ^ (r >> 3)) & 1) | ((r >> 1) & 2); }
__device__ __forceinline__ int lofs(int r, int c) { return r * 64 + ((c ^ swz(r)) << 4); }

// Order of an expert's tiles: groups of kQGroup q-tiles (token rows), and inside a
// group the p-tiles (weight rows) with the group's q-tiles fastest.  The 32 tiles one
// XCD runs at a time (consecutive ids) then span about 6 q-tiles x 5 p-tiles, which
// share far more operand data in that XCD's L2 than 32 tiles of one q-tile row or
// one p-tile column.
constexpr int kQGroup = 6;
// Longest weight-gradient tile (in K stages) computed in one piece.
#ifndef MOE_WGRAD_CHUNK
#define MOE_WGRAD_CHUNK 192
#endif
constexpr int kChunk = MOE_WGRAD_CHUNK;
__device__ __forceinline__ void tile_order(int local, int nQt, int nPt, int& pt, int& qt) {
    const int gi = local / (kQGroup * nPt);
    const int rem = local - gi * kQGroup * nPt;
    const int left = nQt - gi * kQGroup;
    const int gsz = left < kQGroup ? left : kQGroup;
    pt = rem / gsz;
    qt = gi * kQGroup + (rem - pt * gsz);
}

template <int MODE> struct Traits;
template <> struct Traits<FWD_W13>   { static constexpr bool kP_kmajor = true,  kQ_kmajor = true,  kRaggedK = false; };
template <> struct Traits<FWD_W2>    { static constexpr bool kP_kmajor = true,  kQ_kmajor = true,  kRaggedK = false; };
template <> struct Traits<DGRAD_W2>  { static constexpr bool kP_kmajor = false, kQ_kmajor = true,  kRaggedK = false; };
template <> struct Traits<DGRAD_W13> { static constexpr bool kP_kmajor = false, kQ_kmajor = true,  kRaggedK = false; };
template <> struct Traits<WGRAD_W2>  { static constexpr bool kP_kmajor = false, kQ_kmajor = false, kRaggedK = true; };
template <> struct Traits<WGRAD_W13> { static constexpr bool kP_kmajor = false, kQ_kmajor = false, kRaggedK = true; };

// number of p-tiles; q-tiles of the fixed-size q dimension (weight gradients)
template <int MODE> __device__ __forceinline__ int num_p_tiles(const GemmArgs& g) {
    if constexpr (MODE == FWD_W13) return (g.I + 127) / 128;
    else if constexpr (MODE == FWD_W2 || MODE == DGRAD_W13 || MODE == WGRAD_W13) return (g.d + TP - 1) / TP;
    else return (g.I + TP - 1) / TP;   // DGRAD_W2, WGRAD_W2
}
template <int MODE> __device__ __forceinline__ int num_q_tiles_fixed(const GemmArgs& g) {
    if constexpr (MODE == WGRAD_W2) return (g.d + TQ - 1) / TQ;
    else return (2 * g.I + TQ - 1) / TQ;  // WGRAD_W13
}
template <int MODE> __device__ __forceinline__ int k_size(const GemmArgs& g, int rows_e) {
    if constexpr (MODE == FWD_W13 || MODE == DGRAD_W2) return g.d;
    else if constexpr (MODE == FWD_W2) return g.I;
    else if constexpr (MODE == DGRAD_W13) return 2 * g.I;
    else return rows_e;
}

// One work item of a workgroup: stages k0 .. k0 + nk - 1 of tile (e, pt, qt).  A
// weight-gradient tile cut into np > 1 pieces along K has its pieces' partial sums in
// slots pslot0 + i * pstride (i = 0 .. np - 1; this piece's is `slot`) and its piece
// counter at cslot.
struct TileCtx {
    int e, mb, rows, pt, qt;
    int k0, nk;
    int np, slot, pslot0, pstride, cslot;
};

// kSaveH (FWD_W13 only): also store h = (g, u) for backward.  A separate instantiation
// rather than a runtime branch: accumulators live into two branches of the epilogue
// are copied out to scratch by the register allocator.
// kAct (FWD_W13 and DGRAD_W2): the gated activation, a template parameter so that the
// SwiGLU kernels stay as they are.
// v summed over each group of 8 consecutive lanes, the total in all 8: lane pairs
// (xor 1), then quads (xor 2), then the two quads (row_half_mirror pairs lane i with
// 7 - i, which holds the other quad's sum), all through DPP.  Every lane of a group
// ends with the same bits.  All 64 lanes must be active.
template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, true));
}
__device__ __forceinline__ float sum_lanes8(float v) {
    v += dpp_f32<0xB1>(v);      // quad_perm [1, 0, 3, 2]
    v += dpp_f32<0x4E>(v);      // quad_perm [2, 3, 0, 1]
    v += dpp_f32<0x141>(v);     // row_half_mirror
    return v;
}

template <int MODE, bool kSaveH = false, int kAct = kActSwiGLU>
__global__ __launch_bounds__(NTHR, 1) void grouped_gemm(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) char lds[NBUF * BUFB];
    __shared__ int cum[257];           // prefix over experts of their tiles (work items)
    __shared__ int mptr[257];          // m_indptr, so that the tile walk reads no global memory
    // weight gradients only: experts in work order, their K stages and chunk counts, and
    // prefixes (in work order) of partial-sum slots and split tiles
    __shared__ int worder[256], wnk[256], wnch[256], pcum[257], tcum[257];
    __shared__ int gsrc[2][TQ];        // gather indices of the next two load-cursor tiles
    __shared__ int wtot[NTHR / MOE_WAVE];

    const int tid = threadIdx.x, lane = tid & 63;
    // The lane id recomputed on the spot (inline mbcnt, which the compiler cannot fold
    // into `lane`).  Code that runs once per tile (copy offsets, epilogue) derives its
    // lane-dependent offsets from it, so that none of them is hoisted out of the tile
    // loop: held across the main loop they would be spilled, and a scratch reload waits
    // on vmcnt, i.e. on every copy still in flight.
    auto fresh_lane = []() {
        int l;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
        return l;
    };
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wp = wave & 1, wq = wave >> 1;
    const int E = g.E;
    const int nPt = num_p_tiles<MODE>(g);
    constexpr bool kPk = Traits<MODE>::kP_kmajor, kQk = Traits<MODE>::kQ_kmajor;

    // ---- work list
    // Tiles are numbered expert by expert; workgroup v takes items v, v + G, ... (the
    // weight gradients snake: odd rounds run v = G - 1 .. 0).  Consecutive items run at
    // the same time on consecutive workgroups of one XCD, so the tiles of one expert
    // share their operand slices in its L2.
    // The weight gradients' K is the expert's routed rows, which skewed routing makes a
    // hundred times larger for some experts than for others.  There the experts are
    // taken in decreasing order of work per tile, and a tile longer than C stages is cut
    // into ceil(nk / C) equal pieces along K (C = kChunk stages, doubled until at most
    // kMaxPieces pieces result), each piece a work item of its own: all pieces i of an
    // expert's tiles follow each other in the list (they share K, like whole tiles).
    // Each piece stores its FP32 partial sums; the last piece of a tile to finish adds
    // them up in piece order (a fixed order: the result does not depend on timing).
    constexpr bool kRagged = Traits<MODE>::kRaggedK;
    const int kTPE = kRagged ? nPt * num_q_tiles_fixed<MODE>(g) : 0;   // tiles per expert (weight gradients)
    auto nk_of = [&](int rows) {
        const int nk = (k_size<MODE>(g, rows) + TK - 1) / TK;
        return nk > 0 ? nk : 1;                   // an empty expert still runs one all-zero stage
    };
    // exclusive prefix over threads 0 .. E-1 of v (threads >= E pass 0); returns the
    // block total.  Ends with a barrier.
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
        const int tot = wtot[0] + wtot[1] + wtot[2] + wtot[3];
        __syncthreads();
        return tot;
    };
    for (int i = tid; i <= E; i += NTHR) mptr[i] = g.m_indptr[i];
    __syncthreads();
    if constexpr (kRagged) {
        const int nk = tid < E ? nk_of(mptr[tid + 1] - mptr[tid]) : 0;
        // chunk size C = kChunk << ci: the smallest with at most kMaxPieces pieces
        int ci = 0;
        for (; ci < 7; ++ci) {
            const int C = kChunk << ci;
            const int pc = (tid < E && nk > C) ? kTPE * ((nk + C - 1) / C) : 0;
            if (block_scan(pc, pcum) <= kMaxPieces) break;
        }
        const int C = kChunk << ci;
        const int nch = tid < E ? (nk + C - 1) / C : 0;
        const int csz = tid < E ? (nk + nch - 1) / nch : 0;
        if (tid < E) { wnk[tid] = nk; wnch[tid] = csz; }
        __syncthreads();
        // work order: decreasing piece length, then expert id
        int rank = 0;
        if (tid < E)
            for (int e2 = 0; e2 < E; ++e2) rank += (wnch[e2] > csz || (wnch[e2] == csz && e2 < tid)) ? 1 : 0;
        __syncthreads();
        if (tid < E) { worder[rank] = tid; wnch[tid] = nch; }
        __syncthreads();
        const int e = tid < E ? worder[tid] : 0;            // expert at work position tid
        const int nche = tid < E ? wnch[e] : 0;
        block_scan(tid < E ? nche * kTPE : 0, cum);
        block_scan((tid < E && nche > 1) ? nche * kTPE : 0, pcum);
        block_scan((tid < E && nche > 1) ? kTPE : 0, tcum);
    } else {
        const int rows = tid < E ? mptr[tid + 1] - mptr[tid] : 0;
        block_scan(tid < E ? ((rows + TQ - 1) / TQ) * nPt : 0, cum);
    }
    const int G = gridDim.x;
    const int vid = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    const int total = cum[E];
    int n_items;
    {
        const int F = total / G, rem = total - F * G;
        const int pos = (kRagged && (F & 1)) ? G - 1 - vid : vid;
        n_items = F + (pos < rem ? 1 : 0);
    }
    if (n_items == 0) return;
    // largest s with cum[s] <= x: cum is non-decreasing and cum[0] = 0, so it is the
    // number of s in [1, E) with cum[s] <= x (one ballot per 64 entries)
    auto expert_at = [&](int x) {
        const int fl = fresh_lane();
        int lo = 0;
#pragma unroll
        for (int base = 1; base < 257; base += 64) {
            const int e = base + fl;
            lo += __builtin_popcountll(__ballot(e < E && cum[e] <= x));
        }
        return __builtin_amdgcn_readfirstlane(lo);
    };
    // work item k of this workgroup
    auto coords = [&](int k) {
        const int item = k * G + ((kRagged && (k & 1)) ? G - 1 - vid : vid);
        TileCtx c;
        const int sp = expert_at(item);
        const int local = item - cum[sp];
        if constexpr (kRagged) {
            const int e = worder[sp];
            const int nk = wnk[e], nch = wnch[e];
            const int ch = local / kTPE, j = local - ch * kTPE;
            c.e = e;
            c.qt = j / nPt;
            c.pt = j - c.qt * nPt;
            c.k0 = nk * ch / nch;
            c.nk = nk * (ch + 1) / nch - c.k0;
            c.np = nch;
            c.pslot0 = pcum[sp] + j;
            c.pstride = kTPE;
            c.slot = c.pslot0 + ch * kTPE;
            c.cslot = tcum[sp] + j;
        } else {
            c.e = sp;
            tile_order(local, (mptr[sp + 1] - mptr[sp] + TQ - 1) / TQ, nPt, c.pt, c.qt);
            c.k0 = 0;
            c.nk = nk_of(0);
            c.np = 1;
            c.pslot0 = c.pstride = c.slot = c.cslot = 0;
        }
        // uniform: kept in SGPRs
        c.mb = __builtin_amdgcn_readfirstlane(mptr[c.e]);
        c.rows = __builtin_amdgcn_readfirstlane(mptr[c.e + 1]) - c.mb;
        return c;
    };

    // ------------------------------------------------------------ K-major operands: direct copies
    // A K-major operand tile of one stage is 16 blocks of 1 KiB (16 rows x 64 bytes).
    // Wave w copies blocks 4w .. 4w+3 of each K-major operand with
    // global_load_lds_dwordx4: lane L fetches 16 bytes from global memory and the
    // hardware writes them to LDS at (block start + 16 L), i.e. row 16 blk + L/4,
    // chunk slot L%4, which holds logical chunk (L%4) ^ ((row >> 1) & 3).  The copies
    // bypass registers; they are issued three stages ahead and waited for with
    // explicit vmcnt counts (issued as inline assembly, so the compiler neither
    // tracks nor waits for them: loads complete in issue order, and the wait before a
    // barrier leaves exactly the younger copies outstanding).
    // MN-major operands (the transposed products of backward) are copied the same way
    // into MN-major stages: 32 rows (k) x 256 columns, read as MFMA fragments with
    // transposing LDS reads (read_tr below).
    constexpr bool kPmn = !kPk, kQmn = !kQk;
    // row length (elements) of an MN-major operand, which is also its column count:
    // P = W2_e [d, I] (DGRAD_W2), W13_e [2I, d] (DGRAD_W13), a [R, I] (WGRAD_W2),
    // xg [R, d] (WGRAD_W13); Q = dys [R, d] (WGRAD_W2), dh [R, 2I] (WGRAD_W13)
    const int pmn_ld = (MODE == DGRAD_W2 || MODE == WGRAD_W2) ? g.I : g.d;
    const int qmn_ld = MODE == WGRAD_W13 ? 2 * g.I : g.d;
    const uint32_t lds0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds;
    // byte offsets of this lane's rows: P blocks (j = 0..3), then Q blocks
    uint32_t dvoff[8];
    const char* pbase_e = nullptr;        // P base of the load cursor's expert
    const char* qbase_e = nullptr;        // Q base of the load cursor's expert (weight gradients)
    int lc_rows = 0;                      // routed rows of the load cursor's expert
    // MN-major copy j of wave w fills stage rows 8 w + 2 j + L / 32, 16-byte slot L % 32,
    // which holds logical chunk (L % 32) ^ ((row & 3) << 2), i.e. columns
    // col0 + 8 chunk .. + 7 of that k row; columns past the matrix read any valid column
    auto mn_offset = [&](int j, int col0, int ld) {
        const int L = fresh_lane();
        const int kr = 8 * wave + 2 * j + (L >> 5);
        const int ch = (L & 31) ^ ((kr & 3) << 2);
        int col = col0 + 8 * ch;
        if (col > ld - 8) col = ld - 8;
        return (uint32_t)(kr * ld + col) * 2u;
    };
    auto dma_offsets = [&](const TileCtx& c, const int src[4]) {
        lc_rows = c.rows;
        const int drow_in_blk = fresh_lane() >> 2;
        const int lane = drow_in_blk * 4 + (fresh_lane() & 3);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = (4 * wave + j) * 16 + drow_in_blk;       // row of the stage tile
            const int cl = (lane & 3) ^ swz(r);                   // logical chunk it holds
            if constexpr (MODE == FWD_W13) {
                // 32-row block j of the tile: gate rows i0 + 16 j + (0..15), then the up rows of
                // the same i, so that an MFMA tile holds both halves of its 16 outputs
                int ii = c.pt * 128 + (r >> 5) * 16 + (r & 15);
                if (ii >= g.I) ii = g.I - 1;
                const int wrow = (r & 16) ? g.I + ii : ii;
                dvoff[j] = (uint32_t)(wrow * g.d + 8 * cl) * 2u;
            } else if constexpr (MODE == FWD_W2) {
                int pr = c.pt * TP + r;
                if (pr >= g.d) pr = g.d - 1;
                dvoff[j] = (uint32_t)(pr * g.I + 8 * cl) * 2u;
            } else {
                dvoff[j] = mn_offset(j, c.pt * TP, pmn_ld);
            }
            if constexpr (kQmn) {
                dvoff[4 + j] = mn_offset(j, c.qt * TQ, qmn_ld);
            } else {
                const int qs = src[j];
                if constexpr (MODE == FWD_W13 || MODE == DGRAD_W2) dvoff[4 + j] = (uint32_t)(qs * g.d + 8 * cl) * 2u;
                else if constexpr (MODE == FWD_W2) dvoff[4 + j] = (uint32_t)(qs * g.I + 8 * cl) * 2u;
                else dvoff[4 + j] = (uint32_t)(qs * 2 * g.I + 8 * cl) * 2u;   // DGRAD_W13
            }
        }
        if constexpr (MODE == FWD_W13) pbase_e = reinterpret_cast<const char*>(g.w13 + (size_t)c.e * 2 * g.I * g.d);
        if constexpr (MODE == FWD_W2 || MODE == DGRAD_W2) pbase_e = reinterpret_cast<const char*>(g.w2 + (size_t)c.e * g.d * g.I);
        if constexpr (MODE == DGRAD_W13) pbase_e = reinterpret_cast<const char*>(g.w13 + (size_t)c.e * 2 * g.I * g.d);
        if constexpr (MODE == WGRAD_W2) {
            pbase_e = reinterpret_cast<const char*>(g.a + (size_t)c.mb * g.I);
            qbase_e = reinterpret_cast<const char*>(g.dys + (size_t)c.mb * g.d);
        }
        if constexpr (MODE == WGRAD_W13) {
            pbase_e = reinterpret_cast<const char*>(g.xg + (size_t)c.mb * g.d);
            qbase_e = reinterpret_cast<const char*>(g.dh + (size_t)c.mb * 2 * g.I);
        }
    };
    // byte offset of stage kt inside the P rows of the load cursor's expert
    auto p_stage_bytes = [&](int kt) {
        if constexpr (kPmn) return (size_t)kt * TK * pmn_ld * 2;
        else return (size_t)kt * TK * 2;
    };
    const char* qbase = nullptr;
    if constexpr (MODE == FWD_W13) qbase = reinterpret_cast<const char*>(g.x);
    if constexpr (MODE == DGRAD_W2) qbase = reinterpret_cast<const char*>(g.dy);
    if constexpr (MODE == FWD_W2) qbase = reinterpret_cast<const char*>(g.a);
    if constexpr (MODE == DGRAD_W13) qbase = reinterpret_cast<const char*>(g.dh);
    // source rows (token or routed row) of this lane's 4 Q block rows in tile c; the
    // gathered modes take the token ids from gsrc[slot], where gather_dma put them
    constexpr bool kGather = (MODE == FWD_W13 || MODE == DGRAD_W2);
    auto q_src = [&](const TileCtx& c, int slot, int src[4]) {
        if constexpr (kQk) {
            const int drow_in_blk = fresh_lane() >> 2;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (kGather) {
                    src[j] = gsrc[slot][(4 * wave + j) * 16 + drow_in_blk];
                } else {
                    int rr = c.qt * TQ + (4 * wave + j) * 16 + drow_in_blk;
                    if (rr >= c.rows) rr = c.rows > 0 ? c.rows - 1 : 0;   // ragged tail: a row of the expert
                    src[j] = c.mb + rr;
                }
            }
        }
    };
    // Gather indices of tile c into gsrc[slot]: wave w copies entries 64 w .. 64 w + 63
    // (the rows of its own copy blocks, so it later reads only what it copied itself)
    // with one global_load_lds_dword, issued a tile ahead and counted like the stage
    // copies; a plain load would make the compiler wait for every copy in flight.
    auto gather_dma = [&](const TileCtx& c, int slot) {
        if constexpr (kGather) {
            int rr = c.qt * TQ + 64 * wave + fresh_lane();
            if (rr >= c.rows) rr = c.rows - 1;                    // tiles exist only for rows >= 1
            const uint32_t voff = (uint32_t)(c.mb + rr) * 4u;
            const uint32_t dst = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) int*)&gsrc[slot][64 * wave];
            asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dword %1, %2"
                         :: "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(g.gather) : "memory");
        }
    };
    auto dma1 = [&](uint32_t lds_addr, uint32_t voff, const char* base) {
        asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(base) : "memory");
    };
    // The weight gradients run K over an expert's routed rows, which end at any row:
    // their copies are buffer loads whose resource covers only the stage's rows inside
    // the expert, so that the rows past its end land in LDS as zeros.
    auto bcopy = [&](uint32_t lds_addr, uint32_t voff, __amdgpu_buffer_rsrc_t rs) {
        asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                     :: "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rs) : "memory");
    };
    auto stage_rsrc = [&](const char* base_e, int ld, int kt) {
        const int left = lc_rows - kt * TK;
        const int n = left < 0 ? 0 : (left > TK ? TK : left);
        // the values are uniform; say so, so that the resource is built in SGPRs
        const uint64_t b = (uint64_t)(uintptr_t)(base_e + (size_t)kt * TK * ld * 2);
        const uint64_t bu = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
        return __builtin_amdgcn_make_buffer_rsrc((void*)(uintptr_t)bu, (short)0,
                                                 __builtin_amdgcn_readfirstlane(n * ld * 2), 0x00020000);
    };
    // copy j of stage kt of the load cursor's tile into ring buffer buf (j < 4: P
    // block j, else Q block j - 4)
    auto dma_one = [&](int kt, int buf, int j) {
        const uint32_t dst = lds0 + buf * BUFB + (4 * wave) * 1024 + (j < 4 ? j * 1024 : OPB + (j - 4) * 1024);
        if constexpr (kRagged) {
            if (j < 4) bcopy(dst, dvoff[j], stage_rsrc(pbase_e, pmn_ld, kt));
            else bcopy(dst, dvoff[j], stage_rsrc(qbase_e, qmn_ld, kt));
        } else {
            if (j < 4) dma1(dst, dvoff[j], pbase_e + p_stage_bytes(kt));
            else dma1(dst, dvoff[j], qbase + kt * TK * 2);
        }
    };
    auto dma_stage = [&](int kt, int buf) {
#pragma unroll
        for (int j = 0; j < 8; ++j) dma_one(kt, buf, j);
    };
    // wait until at most one stage (8 copies) of this wave's copies is outstanding
    auto wait_dma = [&]() { asm volatile("s_waitcnt vmcnt(8)" ::: "memory"); };
    constexpr bool kEarlyWait = MODE == FWD_W13 || MODE == DGRAD_W2 || MODE == WGRAD_W2 ||
                                MODE == WGRAD_W13;                     // see the stage stream
    // Q is the routed rows (tiles end at an expert's last row), and the registers allow
    // the partial-tile copies of the stage loop (W13 holds 512 per lane already)
    constexpr bool kRowsQ = MODE == FWD_W2 || MODE == DGRAD_W2 || MODE == DGRAD_W13;
    // ------------------------------------------------------------ fragments
    // fragment b of P (Q): rows wp*128 + 32 b + (lane & 31) (wq*128 + ...), k chunk (lane >> 5)
    // for k step 0 of a stage; k step 1 is chunk + 2, i.e. the byte offset ^ 32.
    // (recomputed at every tile start from the lane id read afresh, so that they are not
    // held across the epilogue, where the kernels that save h run short of registers)
    int fragP[4], fragQ[4];
    auto frag_offsets = [&]() {
        const int fl = fresh_lane();
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            fragP[b] = lofs(wp * 128 + b * 32 + (fl & 31), fl >> 5);
            fragQ[b] = OPB + lofs(wq * 128 + b * 32 + (fl & 31), fl >> 5);
        }
    };
    frag_offsets();
    // MN-major fragments with ds_read_b64_tr_b16: within a 16-lane group, lane j reads 4
    // consecutive columns of row k0 + j / 4 at column n0 + 4 (j % 4), and lane i
    // receives rows k0 .. k0 + 3 of column n0 + i.  Lane l = 16 g + j of fragment a, k
    // step ks, read t (k 4t .. 4t + 3 of its 8) takes row 16 ks + 8 (g >> 1) + 4 t +
    // (j >> 2) and column c0 + 16 (g & 1) + 4 (j & 3), c0 = 128 wp (P) or 128 wq (Q)
    // + 32 a: the result is the MFMA operand (column l & 31, k = 8 (l >> 5) ..), as a
    // K-major fragment read would give it.  The chunk swizzle puts the 32 (row, chunk)
    // pairs one read touches on every bank group exactly twice.
    int trbase = 0, trbaseQ = OPB, trxa[4] = {0, 0, 0, 0};
    if constexpr (kPmn || kQmn) {
        const int gq = lane >> 4, jj = lane & 15;
        const int rowpart = (8 * (gq >> 1) + (jj >> 2)) * 512 + (2 * (gq & 1) + ((jj & 3) >> 1)) * 16 + (jj & 1) * 8;
        trbase = rowpart + wp * 16 * 16;
        trbaseQ = OPB + rowpart + wq * 16 * 16;
#pragma unroll
        for (int a = 0; a < 4; ++a) trxa[a] = (a ^ (jj >> 2)) << 6;
    }
    auto read_tr = [&](const char* base, int tb, int a, int ks) {
        typedef short i16x4_t __attribute__((ext_vector_type(4)));
        typedef short i16x8_t __attribute__((ext_vector_type(8)));
        typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;
        const char* p0 = base + tb + trxa[a] + ks * 16 * 512;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) char*)p0);
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) char*)(p0 + 4 * 512));
        const i16x8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8_t, v);
    };
    auto read_frags = [&](int buf, int ks, bf16x8_t pf[4], bf16x8_t qf[4]) {
        const char* base = lds + buf * BUFB;
        const int x = ks ? 32 : 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if constexpr (kPmn) pf[b] = read_tr(base, trbase, b, ks);
            else pf[b] = *reinterpret_cast<const bf16x8_t*>(base + (fragP[b] ^ x));
            if constexpr (kQmn) qf[b] = read_tr(base, trbaseQ, b, ks);
            else qf[b] = *reinterpret_cast<const bf16x8_t*>(base + (fragQ[b] ^ x));
        }
    };

    f32x16_t acc[4][4];
    // One k step: 16 MFMAs on (pf, qf) in four groups of four (row block a).  Into
    // each group go two LDS fragment reads of the next k step (from ring buffer rbuf, k
    // step rks, into npf / nqf) and, after them, copy `dma_first + a` of the stage being
    // prefetched, so that reads and copies are spread over the MFMAs instead of queueing
    // up together.  The reads go in the order the next step consumes them: its first
    // group takes P fragment 0 with all four Q fragments, so the Q fragments are read
    // first (groups 0 and 1) and P fragments 0 .. 3 after them (groups 2 and 3); read in
    // pairs (P a, Q a) instead, the Q fragment read last was needed by the next step's
    // fourth MFMA, a few MFMAs after its read was issued.  The scheduling fences keep that
    // order (the copies are inline assembly, which the MFMAs could otherwise drift across).
    auto read_item = [&](const char* rbase, int x, int rks, int i, bf16x8_t npf[4], bf16x8_t nqf[4]) {
        if (i < 4) {
            if constexpr (kQmn) nqf[i] = read_tr(rbase, trbaseQ, i, rks);
            else nqf[i] = *reinterpret_cast<const bf16x8_t*>(rbase + (fragQ[i] ^ x));
        } else {
            if constexpr (kPmn) npf[i - 4] = read_tr(rbase, trbase, i - 4, rks);
            else npf[i - 4] = *reinterpret_cast<const bf16x8_t*>(rbase + (fragP[i - 4] ^ x));
        }
    };
    auto mfma_step = [&](const bf16x8_t pf[4], const bf16x8_t qf[4], int rbuf, int rks,
                         bf16x8_t npf[4], bf16x8_t nqf[4], int dma_kt, int dma_buf, int dma_first) {
        const char* rbase = lds + rbuf * BUFB;
        const int x = rks ? 32 : 0;
        constexpr int kQreads = kQmn ? 2 : 1, kPreads = kPmn ? 2 : 1;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            acc[a][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[a], qf[0], acc[a][0], 0, 0, 0);
            read_item(rbase, x, rks, 2 * a, npf, nqf);
            acc[a][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[a], qf[1], acc[a][1], 0, 0, 0);
            read_item(rbase, x, rks, 2 * a + 1, npf, nqf);
            acc[a][2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[a], qf[2], acc[a][2], 0, 0, 0);
            acc[a][3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[a], qf[3], acc[a][3], 0, 0, 0);
            if (a < 2) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, kQreads, 0);   // LDS read(s) of a Q fragment
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, kQreads, 0);
            } else {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, kPreads, 0);   // LDS read(s) of a P fragment
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x100, kPreads, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            dma_one(dma_kt, dma_buf, dma_first + a);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // A k step of a wave whose tile rows end inside its 128 Q rows (a ragged tail of an
    // expert): the MFMAs of Q blocks b < L only (the others would feed rows that are never
    // stored), with the same fragment reads and copies as mfma_step.
    auto mfma_step_part = [&](auto live_tag, const bf16x8_t pf[4], const bf16x8_t qf[4], int rbuf, int rks,
                              bf16x8_t npf[4], bf16x8_t nqf[4], int dma_kt, int dma_buf, int dma_first) {
        constexpr int L = decltype(live_tag)::value;
        const char* rbase = lds + rbuf * BUFB;
        const int x = rks ? 32 : 0;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
#pragma unroll
            for (int b = 0; b < L; ++b)
                acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pf[a], qf[b], acc[a][b], 0, 0, 0);
            read_item(rbase, x, rks, 2 * a, npf, nqf);
            read_item(rbase, x, rks, 2 * a + 1, npf, nqf);
            dma_one(dma_kt, dma_buf, dma_first + a);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // ------------------------------------------------------------ epilogue
    // lane holds D[q][p .. p+3] for q = q0 + 32 b + (lane & 31), p = p0 + 32 a + 8 grp + p_sub.
    // The epilogue computes its lane index `ln` afresh (mbcnt, as inline assembly the
    // compiler cannot fold into the kernel's lane id), so that none of the lane-derived offsets is hoisted out of the tile
    // loop: held across the main loop they would be spilled, and each scratch reload
    // waits on vmcnt, i.e. on every copy still in flight for the next stages.
    // Plain BF16 outputs go through LDS (this wave's 8 KiB of the stage buffer just
    // consumed) so that each store instruction writes whole 256-byte row segments:
    // per block b, 32 rows x 128 columns are written as 8-byte pieces (16-byte chunk
    // slot c ^ (row & 15)), read back as 16-byte chunks and stored row-contiguously.
    // These outputs (o, dxp, the weight gradients) are streamed out with non-temporal
    // stores of whole lines: written as ordinary stores they evicted the operand slices
    // the XCD's workgroups share in L2 (W2 main loop 31k cycles per tile without its
    // stores, 38-45k with ordinary ones).  a and dh, read back by the next product while
    // still cached, are stored normally, and so are stores of 8-byte pieces (the saved
    // h): non-temporal partial lines are written one by one, which made W13 35 % slower.
    // The staged rows are read back all at once and then stored: the empty asm consumes
    // every loaded value before the stores' bounds checks, so that the compiler issues the
    // reads together and waits once, instead of sinking each read into its store's branch
    // (a read, a wait and a store per row piece, one LDS latency each).  Once the values
    // are in registers the staging slot may be rewritten.
    auto lds_values_ready = [](auto& v) {
#pragma unroll
        for (auto& x : v) asm volatile("" : "+v"(x));
    };
    auto store_rows_bf16 = [&](int ln, char* stg, int b, uint16_t* out, size_t ld, int q_first, int q_limit,
                               int p_first, int p_limit) {
        const int q_in = ln & 31, p_sub = 4 * (ln >> 5);
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
        __builtin_amdgcn_s_waitcnt(0xc07f);      // lgkmcnt(0): the wave's own LDS writes are done
        u32x4_t v[8];
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int row = 4 * it + (ln >> 4);
            v[it] = *reinterpret_cast<const u32x4_t*>(stg + row * 256 + (((ln & 15) ^ (row & 15)) << 4));
        }
        lds_values_ready(v);
        if constexpr (MODE == WGRAD_W2 || MODE == WGRAD_W13) {
            // accumulate: out = bf16(out + bf16(gradient)); the old values are loaded at
            // clamped (always valid) addresses, all before the first add
            if (g.accumulate) {
                u32x4_t old[8];
#pragma unroll
                for (int it = 0; it < 8; ++it) {
                    const int q = q_first + 4 * it + (ln >> 4);
                    const int p = p_first + 8 * (ln & 15);
                    const int qc = q < q_limit ? q : q_limit - 1, pc = p < p_limit ? p : p_limit - 8;
                    old[it] = *reinterpret_cast<const u32x4_t*>(out + (size_t)qc * ld + pc);
                }
#pragma unroll
                for (int it = 0; it < 8; ++it)
#pragma unroll
                    for (int z = 0; z < 4; ++z)
                        v[it][z] = pack_bf16(bf16lo(old[it][z]) + bf16lo(v[it][z]), bf16hi(old[it][z]) + bf16hi(v[it][z]));
            }
        }
#pragma unroll
        for (int it = 0; it < 8; ++it) {
            const int q = q_first + 4 * it + (ln >> 4);
            const int p = p_first + 8 * (ln & 15);
            if (q < q_limit && p < p_limit) store_nt(out + (size_t)q * ld + p, make_uint4(v[it][0], v[it][1], v[it][2], v[it][3]));
        }
    };
    auto epilogue = [&](const TileCtx& c, int buf) {
        char* stg = lds + buf * BUFB + wave * 8192;
        const int ln = fresh_lane();
        const int q_in = ln & 31, p_sub = 4 * (ln >> 5);
        if constexpr (MODE == FWD_W13) {
            // a[r][i] for i = pt*128 + wp*64 + (0..63): 64 columns, 128-byte row segments.
            // MFMA tile (a, b) holds gate values in element groups 0, 1 and the matching up
            // values in groups 2, 3: outputs i = 16 a + 8 grp + p_sub + z of the wave's 64.
            // One row block b at a time (the fences keep the scheduler from overlapping
            // the blocks).
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                __builtin_amdgcn_sched_barrier(0);
                // saved h: one row pointer per block (the wave's 64 columns are all inside
                // I or all past it, I being a multiple of 64), constant offsets per store
                const int hr = c.qt * TQ + wq * 128 + b * 32 + q_in;
                const bool hlive = kSaveH && hr < c.rows && c.pt * 128 + wp * 64 < g.I;
                uint16_t* hrow = kSaveH ? g.out_h + ((size_t)c.mb + (hlive ? hr : 0)) * 2 * g.I + c.pt * 128 + wp * 64 + p_sub
                                        : nullptr;
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int grp = 0; grp < 2; ++grp) {
                        const int c8 = 2 * a + grp;
                        float gv[4], uv[4], av[4];
#pragma unroll
                        for (int z = 0; z < 4; ++z) {
                            gv[z] = acc[a][b][4 * grp + z];
                            uv[z] = acc[a][b][4 * (grp + 2) + z];
                            av[z] = act_f<kAct>(gv[z]) * uv[z];
                        }
                        uint2 v;
                        v.x = pack_bf16(av[0], av[1]);
                        v.y = pack_bf16(av[2], av[3]);
                        *reinterpret_cast<uint2*>(stg + q_in * 128 + ((c8 ^ (q_in & 7)) << 4) + (p_sub << 1)) = v;
                        if constexpr (kSaveH) {
                            if (hlive) {
                                uint2 hg, hu;
                                hg.x = pack_bf16(gv[0], gv[1]); hg.y = pack_bf16(gv[2], gv[3]);
                                hu.x = pack_bf16(uv[0], uv[1]); hu.y = pack_bf16(uv[2], uv[3]);
                                *reinterpret_cast<uint2*>(hrow + a * 16 + 8 * grp) = hg;
                                *reinterpret_cast<uint2*>(hrow + g.I + a * 16 + 8 * grp) = hu;
                            }
                        }
                    }
                __builtin_amdgcn_s_waitcnt(0xc07f);
                u32x4_t v[4];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = 8 * it + (ln >> 3);
                    v[it] = *reinterpret_cast<const u32x4_t*>(stg + row * 128 + (((ln & 7) ^ (row & 7)) << 4));
                }
                lds_values_ready(v);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int rr = c.qt * TQ + wq * 128 + b * 32 + 8 * it + (ln >> 3);
                    const int i = c.pt * 128 + wp * 64 + 8 * (ln & 7);
                    if (rr < c.rows && i < g.I)
                        *reinterpret_cast<u32x4_t*>(g.out + ((size_t)c.mb + rr) * g.I + i) = v[it];
                }
            }
        } else if constexpr (MODE == FWD_W2 || MODE == DGRAD_W13) {
            // o [R, d] or dxp [R, d]
#pragma unroll
            for (int b = 0; b < 4; ++b)
                store_rows_bf16(ln, stg, b, g.out + (size_t)c.mb * g.d, g.d, c.qt * TQ + wq * 128 + b * 32,
                                c.rows, c.pt * TP + wp * 128, g.d);
        } else if constexpr (MODE == DGRAD_W2) {
            // dA = probs[r] * acc; dg = dA u s(g)(1 + g(1 - s(g))), du = dA g s(g).  Per half
            // row block (32 rows x 64 columns of the wave) the FP32 accumulators go through
            // LDS (16-byte chunk c of row q at slot c ^ (q & 15)) so that each lane then owns
            // 8 consecutive columns of one row: h is read and dh written in 16-byte row
            // pieces (8-byte pieces of 32 rows per instruction cost about 40k cycles per
            // tile each way).  The h loads (and probs) of the next half block are issued
            // before the current one is staged, computed and stored, so that the eight
            // half blocks do not wait for eight memory round trips in turn.
            auto load_h = [&](int hb, uint4 hg[4], uint4 hu[4], float sc[4]) {
                const int b = hb >> 1, ah = hb & 1;
                const int i0 = c.pt * TP + wp * 128 + 64 * ah + 8 * (ln & 7);
                const int ic = i0 < g.I ? i0 : g.I - 8;
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int rr = c.qt * TQ + wq * 128 + b * 32 + 8 * it + (ln >> 3);
                    const size_t r = (size_t)c.mb + (rr < c.rows ? rr : c.rows - 1);
                    hg[it] = *reinterpret_cast<const uint4*>(g.h + r * 2 * g.I + ic);
                    hu[it] = *reinterpret_cast<const uint4*>(g.h + r * 2 * g.I + g.I + ic);
                    sc[it] = g.probs[r];
                }
            };
            // With g.ds_part, each half block also leaves the router gradient's piece of its
            // rows: the sum over its 64 columns of acc (dy W2, before the probs scaling)
            // times a = f(g) u from the saved h (columns past I add nothing), once the
            // row's dh is stored; the eight lanes of a row add their pieces (a fixed tree)
            // and the first stores it in slot 4 pt + 2 wp + ah.  (One piece over both half
            // blocks of a row block, held across the next one's loads, spills.)
            auto half_block = [&](int hb, const uint4 hg[4], const uint4 hu[4], const float sc[4]) {
                const int b = hb >> 1, ah = hb & 1;
                float dsum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                const int i0 = c.pt * TP + wp * 128 + 64 * ah + 8 * (ln & 7);   // this lane's 8 columns
#pragma unroll
                for (int a2 = 0; a2 < 2; ++a2)
#pragma unroll
                    for (int grp = 0; grp < 4; ++grp) {
                        const int c16 = (32 * a2 + 8 * grp + p_sub) >> 2;
                        const int a = 2 * ah + a2;
                        f32x4_t v = {acc[a][b][4 * grp], acc[a][b][4 * grp + 1], acc[a][b][4 * grp + 2], acc[a][b][4 * grp + 3]};
                        *reinterpret_cast<f32x4_t*>(stg + q_in * 256 + ((c16 ^ (q_in & 15)) << 4)) = v;
                    }
                __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): the wave's own LDS writes are done
                f32x4_t sv[8];
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = 8 * it + (ln >> 3), c8 = ln & 7;
                    sv[2 * it] = *reinterpret_cast<const f32x4_t*>(stg + row * 256 + (((2 * c8) ^ (row & 15)) << 4));
                    sv[2 * it + 1] = *reinterpret_cast<const f32x4_t*>(stg + row * 256 + (((2 * c8 + 1) ^ (row & 15)) << 4));
                }
                lds_values_ready(sv);
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const int row = 8 * it + (ln >> 3);
                    const f32x4_t v0 = sv[2 * it], v1 = sv[2 * it + 1];
                    const float av[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
                    const uint32_t gw[4] = {hg[it].x, hg[it].y, hg[it].z, hg[it].w};
                    const uint32_t uw[4] = {hu[it].x, hu[it].y, hu[it].z, hu[it].w};
                    uint32_t og[4], ou[4];
                    float fv[8];                          // f(g) of the lane's 8 columns
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        float dg2[2], du2[2];
#pragma unroll
                        for (int h2 = 0; h2 < 2; ++h2) {
                            const float gv = h2 ? bf16hi(gw[z]) : bf16lo(gw[z]);
                            const float uv = h2 ? bf16hi(uw[z]) : bf16lo(uw[z]);
                            const float dA = sc[it] * av[2 * z + h2];
                            if constexpr (kAct == kActSwiGLU) {
                                const float sg = sigmoid_f(gv);
                                dg2[h2] = dA * uv * sg * (1.0f + gv * (1.0f - sg));
                                du2[h2] = dA * gv * sg;
                                fv[2 * z + h2] = gv * sg;
                            } else {
                                float f, df;
                                act_f_df<kAct>(gv, f, df);
                                dg2[h2] = dA * uv * df;
                                du2[h2] = dA * f;
                                fv[2 * z + h2] = f;
                            }
                        }
                        og[z] = pack_bf16(dg2[0], dg2[1]);
                        ou[z] = pack_bf16(du2[0], du2[1]);
                    }
                    const int rr = c.qt * TQ + wq * 128 + b * 32 + row;
                    if (rr < c.rows && i0 < g.I) {
                        const size_t r = (size_t)c.mb + rr;
                        *reinterpret_cast<uint4*>(g.out + r * 2 * g.I + i0) = make_uint4(og[0], og[1], og[2], og[3]);
                        *reinterpret_cast<uint4*>(g.out + r * 2 * g.I + g.I + i0) = make_uint4(ou[0], ou[1], ou[2], ou[3]);
                    }
                    float dl = 0.0f;
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        dl = __builtin_fmaf(av[2 * z], fv[2 * z] * bf16lo(uw[z]), dl);
                        dl = __builtin_fmaf(av[2 * z + 1], fv[2 * z + 1] * bf16hi(uw[z]), dl);
                    }
                    dsum[it] += i0 < g.I ? dl : 0.0f;
                }
#pragma unroll
                for (int it = 0; it < 4; ++it) {
                    const float v = sum_lanes8(dsum[it]);
                    const int rr = c.qt * TQ + wq * 128 + b * 32 + 8 * it + (ln >> 3);
                    if (g.ds_part != nullptr && (ln & 7) == 0 && rr < c.rows)
                        g.ds_part[((size_t)c.mb + rr) * g.ds_slots + 4 * c.pt + 2 * wp + ah] = v;
                }
            };
            uint4 hg0[4], hu0[4], hg1[4], hu1[4];
            float sc0[4], sc1[4];
            load_h(0, hg0, hu0, sc0);
#pragma unroll
            for (int hb = 0; hb < 8; hb += 2) {
                __builtin_amdgcn_sched_barrier(0);
                load_h(hb + 1, hg1, hu1, sc1);
                half_block(hb, hg0, hu0, sc0);
                __builtin_amdgcn_sched_barrier(0);
                if (hb + 2 < 8) load_h(hb + 2, hg0, hu0, sc0);
                half_block(hb + 1, hg1, hu1, sc1);
            }
        } else {
            // weight gradients: out[e][q][p], q < Qsz rows, p < Psz columns
            const int Psz = (MODE == WGRAD_W2) ? g.I : g.d;
            const int Qsz = (MODE == WGRAD_W2) ? g.d : 2 * g.I;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                store_rows_bf16(ln, stg, b, g.out + (size_t)c.e * Qsz * Psz, Psz, c.qt * TQ + wq * 128 + b * 32,
                                Qsz, c.pt * TP + wp * 128, Psz);
        }
    };

    // ------------------------------------------------------------ stage stream
    // Stage s of the stream lives in ring buffer s % 4.  During stage s the copies
    // of stage s + 3 are issued; the barrier ending stage s publishes stage s + 2 (its
    // copies, issued during stage s - 1, are waited for) and ring buffer s + 1 was
    // published one barrier earlier, so the first fragments of stage s + 1 are read
    // before it.  The load cursor runs three stages ahead of the compute cursor;
    // once the stream is exhausted it repeats its last stage into buffers no later
    // stage reads.
    int l_item = 0, l_kt = 0;          // load cursor: work item, stage within it
    TileCtx lc = coords(0);
    int gslot = 0;                     // gsrc slot of the load cursor's tile
    TileCtx nc = lc;                   // coordinates of the load cursor's next item
    gather_dma(lc, 0);
    if (n_items > 1) { nc = coords(1); gather_dma(nc, 1); }
    if constexpr (kGather) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    {
        int src[4] = {0, 0, 0, 0};
        q_src(lc, 0, src);
        dma_offsets(lc, src);
    }
    auto advance_load = [&]() {
        if (++l_kt < lc.nk) return;
        if (l_item + 1 >= n_items) { l_kt = lc.nk - 1; return; }
        // the indices of the new tile were copied at the previous switch, lc.nk stages
        // ago; with fewer than 3 stages per tile the stage waits need not cover them
        if constexpr (kGather) if (lc.nk < 3) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        l_kt = 0;
        ++l_item;
        gslot ^= 1;
        lc = nc;
        int src[4] = {0, 0, 0, 0};
        q_src(lc, gslot, src);
        dma_offsets(lc, src);
        if (l_item + 1 < n_items) { nc = coords(l_item + 1); gather_dma(nc, gslot ^ 1); }
    };

    // prologue: stages 0, 1, 2
    dma_stage(lc.k0 + l_kt, 0);
    advance_load();
    dma_stage(lc.k0 + l_kt, 1);
    advance_load();
    dma_stage(lc.k0 + l_kt, 2);
    advance_load();
    wait_dma();                        // stages 0 and 1 copied (stage 2 may be in flight)
    __syncthreads();

    bf16x8_t fa[4], fb[4], fc[4], fd[4];
    read_frags(0, 0, fa, fc);

    // A piece of a split weight-gradient tile stores its partial sums: thread t, float4
    // j at (j * 256 + t) * 4 of its slot, j = (a * 4 + b) * 4 + z holding acc[a][b][4 z ..
    // 4 z + 3].  The first piece also describes the tile for wgrad_fixup, which adds up
    // the pieces after this kernel (the kernel boundary makes them visible; a device-wide
    // fence per piece would write back and invalidate an XCD's whole L2).
    constexpr int kPartFloats = NTHR * 256;
    auto store_piece = [&](const TileCtx& c) {
        const int t = fresh_lane() + 64 * wave;
        float* mine = g.part + (size_t)c.slot * kPartFloats;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const int j = (a * 4 + b) * 4 + z;
                    const f32x4_t v = {acc[a][b][4 * z], acc[a][b][4 * z + 1], acc[a][b][4 * z + 2], acc[a][b][4 * z + 3]};
                    *reinterpret_cast<f32x4_t*>(mine + ((size_t)j * NTHR + t) * 4) = v;
                }
        if (t == 0 && c.slot == c.pslot0) {
            int4 dsc;
            dsc.x = c.e; dsc.y = c.qt * 65536 + c.pt; dsc.z = c.np; dsc.w = c.pslot0 * 65536 + c.pstride;
            g.split[c.cslot] = dsc;
        }
    };
    if constexpr (kRagged)
        if (vid == 0 && tid == 0) *g.nsplit = tcum[E];

    int c_item = 0;
    TileCtx cc = coords(0);
    int gs = 0;
    while (true) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
        if constexpr (kRowsQ) {
            // the stages of the tile; L < 4: this wave's live Q blocks (rows past the
            // expert's end are never stored, so their MFMAs are skipped)
            auto stages = [&](auto live_tag) {
                constexpr int L = decltype(live_tag)::value;
                for (int kt = 0; kt < cc.nk; ++kt, ++gs) {
                    // k step 0: MFMAs on (fa, fc) while reading step 1's fragments (fb, fd) and
                    // issuing the first half of the copies of stage gs + 3
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (L == 4) mfma_step(fa, fc, gs & 3, 1, fb, fd, lc.k0 + l_kt, (gs + 3) & 3, 0);
                    else mfma_step_part(live_tag, fa, fc, gs & 3, 1, fb, fd, lc.k0 + l_kt, (gs + 3) & 3, 0);
                    // k step 1: MFMAs on (fb, fd) while reading stage gs + 1's first fragments and
                    // issuing the rest of the copies of stage gs + 3
                    __builtin_amdgcn_sched_barrier(0);
                    if constexpr (L == 4) mfma_step(fb, fd, (gs + 1) & 3, 0, fa, fc, lc.k0 + l_kt, (gs + 3) & 3, 4);
                    else mfma_step_part(live_tag, fb, fd, (gs + 1) & 3, 0, fa, fc, lc.k0 + l_kt, (gs + 3) & 3, 4);
                    advance_load();
                    // this wave's copies of stage gs + 2 have landed.  kEarlyWait modes: in the
                    // first stage of a tile they already had, since they were issued before the
                    // previous tile's epilogue, which waits for every copy before it starts; a
                    // wait here would count the epilogue's stores too and hold the stage until
                    // they are written (DGRAD_W2 313 -> 274 us at the training shape, the weight
                    // gradients 1-4 us; FWD_W2 and DGRAD_W13 gain nothing).
                    if (!kEarlyWait || kt != 0 || c_item == 0) wait_dma();
                    __syncthreads();
                }
            };
            const int left = cc.rows - cc.qt * TQ - wq * 128;          // this wave's rows in the tile
            const int live = left <= 0 ? 0 : (left >= 128 ? 4 : (left + 31) / 32);
            if (live == 4) stages(std::integral_constant<int, 4>{});
            else if (live == 3) stages(std::integral_constant<int, 3>{});
            else if (live == 2) stages(std::integral_constant<int, 2>{});
            else if (live == 1) stages(std::integral_constant<int, 1>{});
            else stages(std::integral_constant<int, 0>{});
        } else {
            // the same loop written out (as a lambda call it costs the W13 kernels spills)
            for (int kt = 0; kt < cc.nk; ++kt, ++gs) {
                __builtin_amdgcn_sched_barrier(0);
                mfma_step(fa, fc, gs & 3, 1, fb, fd, lc.k0 + l_kt, (gs + 3) & 3, 0);
                __builtin_amdgcn_sched_barrier(0);
                mfma_step(fb, fd, (gs + 1) & 3, 0, fa, fc, lc.k0 + l_kt, (gs + 3) & 3, 4);
                advance_load();
                if (!kEarlyWait || kt != 0 || c_item == 0) wait_dma();
                __syncthreads();
            }
        }
        if constexpr (kEarlyWait) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (!kRagged || cc.np == 1) epilogue(cc, (gs - 1) & 3);
        else store_piece(cc);
        if (++c_item >= n_items) break;
        __syncthreads();               // the staging slots are copied into again from the next stage
        cc = coords(c_item);
        frag_offsets();
        // the next stage's first fragments again, from its ring buffer (not written before
        // that stage runs), so that they are not held in registers across the epilogue
        read_frags(gs & 3, 0, fa, fc);
    }
}

// Weight-gradient tiles cut into pieces along K: out = ((piece 0 + piece 1) + ...) in
// BF16 (accumulate: out = bf16(out + that)), one workgroup per quarter of a tile.  Thread t of the tile owns the elements thread t of
// grouped_gemm held (wave w = t / 64 covers p in [128 (w & 1), +128), q in
// [128 (w >> 1), +128) of the tile).
template <int MODE>
__global__ __launch_bounds__(NTHR) void wgrad_fixup(GemmArgs g) {
    constexpr int kPartFloats = NTHR * 256;
    const int n = *g.nsplit;
    const int t = threadIdx.x, ln = t & 63, wave = t >> 6, wp = wave & 1, wq = wave >> 1;
    const int Psz = (MODE == WGRAD_W2) ? g.I : g.d;
    const int Qsz = (MODE == WGRAD_W2) ? g.d : 2 * g.I;
    for (int bi = blockIdx.x; bi < 4 * n; bi += gridDim.x) {
        const int ts = bi >> 2, j0 = 16 * (bi & 3);     // tile, quarter of its elements
        const int4 dsc = g.split[ts];
        const int e = dsc.x, qt = dsc.y >> 16, pt = dsc.y & 0xFFFF, np = dsc.z;
        const int pslot0 = dsc.w >> 16, pstride = dsc.w & 0xFFFF;
        // element (a, b, z, 0..3): q = q0 + 32 b + (ln & 31), p = p0 + 32 a + 8 z + 4 (ln >> 5)
        const int q0 = qt * TQ + wq * 128 + (ln & 31), p0 = pt * TP + wp * 128 + 4 * (ln >> 5);
        uint16_t* out = g.out + (size_t)e * Qsz * Psz;
        {
            f32x4_t sum[16];
#pragma unroll
            for (int i = 0; i < 16; ++i)
                sum[i] = *reinterpret_cast<const f32x4_t*>(g.part + (size_t)pslot0 * kPartFloats + ((size_t)(j0 + i) * NTHR + t) * 4);
            for (int w = 1; w < np; ++w) {
                const float* src = g.part + (size_t)(pslot0 + w * pstride) * kPartFloats;
                f32x4_t v[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const f32x4_t*>(src + ((size_t)(j0 + i) * NTHR + t) * 4);
#pragma unroll
                for (int i = 0; i < 16; ++i) sum[i] += v[i];
            }
            // accumulate: the old values, loaded at clamped addresses before any store
            uint2 old[16];
            if (g.accumulate) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int j = j0 + i, a = j >> 4, b = (j >> 2) & 3, z = j & 3;
                    const int q = q0 + 32 * b, p = p0 + 32 * a + 8 * z;
                    const int qc = q < Qsz ? q : Qsz - 1, pc = p < Psz ? p : Psz - 4;
                    old[i] = *reinterpret_cast<const uint2*>(out + (size_t)qc * Psz + pc);
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int j = j0 + i, a = j >> 4, b = (j >> 2) & 3, z = j & 3;
                const int q = q0 + 32 * b, p = p0 + 32 * a + 8 * z;
                if (q < Qsz && p < Psz) {
                    uint2 o;
                    o.x = pack_bf16(sum[i][0], sum[i][1]);
                    o.y = pack_bf16(sum[i][2], sum[i][3]);
                    if (g.accumulate) {
                        o.x = pack_bf16(bf16lo(old[i].x) + bf16lo(o.x), bf16hi(old[i].x) + bf16hi(o.x));
                        o.y = pack_bf16(bf16lo(old[i].y) + bf16lo(o.y), bf16hi(old[i].y) + bf16hi(o.y));
                    }
                    *reinterpret_cast<uint2*>(out + (size_t)q * Psz + p) = o;
                }
            }
        }
    }
}

template <int MODE>
hipError_t launch_mode(const GemmArgs& g, int num_cu, hipStream_t s) {
    // upper bound on the tile count; the kernel walks the exact list itself
    const int64_t R = (int64_t)g.T * g.k;
    int64_t tiles;
    if constexpr (MODE == FWD_W13) tiles = (R / TQ + g.E) * ((g.I + 127) / 128);
    else if constexpr (MODE == FWD_W2 || MODE == DGRAD_W13) tiles = (R / TQ + g.E) * ((g.d + TP - 1) / TP);
    else if constexpr (MODE == DGRAD_W2) tiles = (R / TQ + g.E) * ((g.I + TP - 1) / TP);
    else if constexpr (MODE == WGRAD_W2) tiles = (int64_t)g.E * ((g.I + TP - 1) / TP) * ((g.d + TQ - 1) / TQ);
    else tiles = (int64_t)g.E * ((g.d + TP - 1) / TP) * ((2 * g.I + TQ - 1) / TQ);
    int64_t grid = tiles < num_cu ? tiles : num_cu;
    if (grid >= 8) grid -= grid % 8;
    if (grid < 1) grid = 1;
    const dim3 gd((unsigned)grid), bd(NTHR);
    if constexpr (MODE == FWD_W13) {
        if (g.out_h) {
            if (g.act == kActGeGLU) hipLaunchKernelGGL((grouped_gemm<MODE, true, kActGeGLU>), gd, bd, 0, s, g);
            else if (g.act == kActReGLU) hipLaunchKernelGGL((grouped_gemm<MODE, true, kActReGLU>), gd, bd, 0, s, g);
            else hipLaunchKernelGGL((grouped_gemm<MODE, true>), gd, bd, 0, s, g);
            return hipGetLastError();
        }
    }
    if constexpr (MODE == FWD_W13 || MODE == DGRAD_W2) {
        if (g.act == kActGeGLU) {
            hipLaunchKernelGGL((grouped_gemm<MODE, false, kActGeGLU>), gd, bd, 0, s, g);
            return hipGetLastError();
        }
        if (g.act == kActReGLU) {
            hipLaunchKernelGGL((grouped_gemm<MODE, false, kActReGLU>), gd, bd, 0, s, g);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((grouped_gemm<MODE, false>), gd, bd, 0, s, g);
    if constexpr (MODE == WGRAD_W2 || MODE == WGRAD_W13) {
        if (hipGetLastError() != hipSuccess) return hipErrorLaunchFailure;
        hipLaunchKernelGGL((wgrad_fixup<MODE>), dim3(2 * kMaxPieces), dim3(NTHR), 0, s, g);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmMode mode, const GemmArgs& g, int num_cu, hipStream_t s) {
    switch (mode) {
        case FWD_W13: return launch_mode<FWD_W13>(g, num_cu, s);
        case FWD_W2: return launch_mode<FWD_W2>(g, num_cu, s);
        case DGRAD_W2: return launch_mode<DGRAD_W2>(g, num_cu, s);
        case DGRAD_W13: return launch_mode<DGRAD_W13>(g, num_cu, s);
        case WGRAD_W2: return launch_mode<WGRAD_W2>(g, num_cu, s);
        case WGRAD_W13: return launch_mode<WGRAD_W13>(g, num_cu, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace moe
