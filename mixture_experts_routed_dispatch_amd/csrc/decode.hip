// decode.hip -- weight-streaming path of the routed expert layer for small batches.
//
// The nvfp4moe README ("MoE layer") gives batch-one and small-batch decode its
// own launch grid and fuses dispatch into it when top-k is at most 32.  With
// T*k <= 256 routed rows every active expert owns only a few rows, so the two
// expert products are matrix-vector-like and the time is the time to stream each
// active expert's W13 and W2 from HBM once.
//
// Three launches:
//   decode_w13: wave items (active expert e, block of 8 intermediate indices i0..).
//     A wave streams the 8 gate and 8 up rows of W13_e over the whole K = d and
//     writes a[t*k + j][i] = silu(g) * u in BF16 for every routed entry of e.
//   decode_w2: wave items (active expert e, block of 16 output features n0..): a wave
//     streams 16 rows of W2_e over K = I and writes o[t*k + j][n] in BF16.
//   combine: y[t] = sum_j s[t][j] * o[t*k + j], FP32, j ascending from +0.0 (the
//     prefill combine kernel, reading the rows in entry order).
// Either the four waves of a workgroup share an item, each streaming a quarter of K,
// and add their partial sums through LDS in wave order (fixed: the result does not
// depend on timing); or a wave owns its item from the first load to the last store,
// with no reduction and no barrier between waves.  The first is used when the items
// are fewer than the wave slots on the chip (one token: k experts x 96 blocks) or when
// a quarter of K still fills a wave's load batch (W13, K = d = 2048: 10,752 items at 32
// tokens are 14 per workgroup, where one wave per item leaves the last of 4 rounds half
// empty); the second for short K (W2 at 32 tokens, K = I = 768).
//
// With one token the experts are the k ids themselves (distinct by the layer's
// precondition), and the W2 products and the combine are one launch (decode_w2_one).
// With more tokens every workgroup first sorts the routed entries by expert in LDS
// (counts, their prefix over the expert ids, the active experts in ascending id, and
// each expert's entries in ascending (t, j) order).
//
// Both products use v_mfma_f32_16x16x32_bf16 with 16 weight rows as the 16 columns
// and up to 16 routed rows as the 16 rows.  The weights stream with nontemporal loads
// that each cover whole 128-byte lines of 8 rows (mma_line_pairs), kBatch K steps of 32
// per wave in flight before the MFMAs that use them.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / MOE_WAVE;
constexpr int kBatch = 16;         // K steps of 32 per wave with loads in flight at once

struct DecodeSmem {
    int ids[kMaxDecodeRows];       // expert of entry q = t*k + j (-1 when invalid)
    int cnt[256];                  // routed rows per expert
    int pfx[257];                  // entries of expert e: ent[pfx[e] .. pfx[e+1])
    int slot_expert[256];          // i-th active expert (ascending id)
    int ent[kMaxDecodeRows];       // entries grouped by expert (ascending id), ascending
    int wsum[kWaves];
    int wact[kWaves];
    int n_active;
};

// Counts, active experts, the entries sorted by expert, and routing flags, from ids;
// every workgroup of a launch runs it (block 0 reports the flags).  Threads 0 .. 255 do
// the work; a larger workgroup's other threads only take part in its barriers.
__device__ void decode_setup(DecodeSmem& sm, const int32_t* __restrict__ ids, int T, int k, int E,
                             int32_t* status, bool report) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const bool worker = tid < 256;
    const int R = T * k;
    if (worker) sm.cnt[tid] = 0;
    __syncthreads();
    int my_e = -1;
    if (worker && tid < R) {
        const int e = ids[tid];
        const bool ok = (unsigned)e < (unsigned)E;
        my_e = ok ? e : -1;
        if (ok) atomicAdd(&sm.cnt[e], 1);
        if (report) {
            int bad = ok ? 0 : kDevIdOutOfRange;
            const int t = tid / k, j = tid - t * k;
            for (int jj = 0; jj < j; ++jj)
                if (ok && ids[t * k + jj] == e) bad |= kDevIdDuplicate;
            if (bad) atomicOr(status, bad);
        }
    }
    if (worker && tid < R) sm.ids[tid] = my_e;
    __syncthreads();
    // active experts in ascending id (ballot ranks) and the exclusive prefix of the
    // counts over the expert ids (wave scans plus the wave totals)
    int c = 0, incl = 0;
    bool active = false;
    uint64_t b = 0;
    if (worker) {
        c = sm.cnt[tid];
        active = tid < E && c > 0;
        b = __ballot(active);
        incl = c;
        for (int off = 1; off < MOE_WAVE; off <<= 1) {
            const int v = __shfl_up(incl, off, MOE_WAVE);
            if (lane >= off) incl += v;
        }
        if (lane == MOE_WAVE - 1) sm.wsum[wave] = incl;
        if (lane == 0) sm.wact[wave] = __popcll(b);
    }
    __syncthreads();
    if (worker) {
        int pre = 0, pre_act = 0;
        for (int w = 0; w < wave; ++w) { pre += sm.wsum[w]; pre_act += sm.wact[w]; }
        if (active) sm.slot_expert[pre_act + __popcll(b & lanemask_lt())] = tid;
        sm.pfx[tid] = pre + incl - c;
        if (tid == 255) sm.pfx[256] = pre + incl;
        if (tid == 0) {
            int nact = 0;
            for (int w = 0; w < 4; ++w) nact += sm.wact[w];
            sm.n_active = nact;
        }
    }
    __syncthreads();
    // entry q goes after the entries q' < q of its expert
    if (my_e >= 0) {
        int rank = 0;
        for (int q = 0; q < tid; ++q) rank += sm.ids[q] == my_e;
        sm.ent[sm.pfx[my_e] + rank] = tid;
    }
    __syncthreads();
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

__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
    return *reinterpret_cast<const bf16x8_t*>(p);
}

// acc(16 rows x 16 cols) = A * B over K pairs 0 .. P - 1 (64 elements = 128 bytes of a
// row each).  The weights stream as whole 128-byte lines with nontemporal loads: per
// pair a wave issues two loads, X covering B columns 0..7 and Y columns 8..15, in which
// lane l fetches bytes 16 (l >> 3) of the pair of column row (l & 7) (X) and 8 + (l & 7)
// (Y); xo and yo are those rows' byte offsets from the bases xb and yb at the wave's
// first K element (wave-uniform bases and 32-bit lane offsets keep the addresses in few
// registers).  (Eight rows x 128 bytes per load streams about 15 % faster from HBM than
// 16 rows x 64 bytes, which is the MFMA's own operand layout.)  The 16x16x32 MFMA wants,
// in 16-lane group q, column (l & 15) at one 8-element chunk common to the group; X and
// Y hold chunk 2q in lanes 16q .. 16q + 7 and chunk 2q + 1 in lanes 16q + 8 .. 16q + 15,
// so a rotate by 8 inside each 16-lane row (DPP row_ror:8) and a select give the two
// operands: chunk 2q for the first MFMA and 2q + 1 for the second.  A row (l & 15) is
// read at the same chunks through the buffer resource ars at byte offset ao (the routed
// row at the wave's first K element); a lane whose row is absent passes kNoRow, past the
// resource's end, and reads zeros without a memory access.  (A conditional load with
// zeros on the other side compiles to a divergent branch whose zero writes wait for
// every load in flight: one round trip per K pair.)  B pairs are loaded before the MFMAs
// that use them.
__device__ __forceinline__ bf16x8_t rotate8_select(bf16x8_t keep, bf16x8_t rot, bool take_rot) {
    const int4 kv = *reinterpret_cast<const int4*>(&keep);
    const int4 rv = *reinterpret_cast<const int4*>(&rot);
    // the rotation runs in every lane (a DPP read of a lane outside the exec mask gives 0)
    const int4 r = {__builtin_amdgcn_update_dpp(0, rv.x, 0x128, 0xF, 0xF, true),
                    __builtin_amdgcn_update_dpp(0, rv.y, 0x128, 0xF, 0xF, true),
                    __builtin_amdgcn_update_dpp(0, rv.z, 0x128, 0xF, 0xF, true),
                    __builtin_amdgcn_update_dpp(0, rv.w, 0x128, 0xF, 0xF, true)};
    int4 o;
    o.x = take_rot ? r.x : kv.x;
    o.y = take_rot ? r.y : kv.y;
    o.z = take_rot ? r.z : kv.z;
    o.w = take_rot ? r.w : kv.w;
    return *reinterpret_cast<const bf16x8_t*>(&o);
}

// Raw buffer resource over `bytes` bytes at base (a uniform kernel argument).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
constexpr uint32_t kNoRow = 0x80000000u;   // beyond every resource: reads zeros

template <int B = kBatch / 2>
__device__ __forceinline__ f32x4_t mma_line_pairs(const char* xb, uint32_t xo, const char* yb, uint32_t yo,
                                                  __amdgpu_buffer_rsrc_t ars, uint32_t ao, int P) {
    const int lane = threadIdx.x & 63;
    const bool hi = (lane & 8) != 0;                   // lanes 8..15 of each 16-lane row
    xo += 16 * (lane >> 3);
    yo += 16 * (lane >> 3);
    ao += 32 * (lane >> 4);
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < P; base += B) {
        bf16x8_t xw[B], yw[B], a0[B], a1[B];
#pragma unroll
        for (int j = 0; j < B; ++j) {
            const uint32_t kb = 128u * (uint32_t)(base + j);
            if (base + j < P) {
                xw[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(xb + (xo + kb)));
                yw[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(yb + (yo + kb)));
                a0[j] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(ars, ao + kb, 0, 0));
                a1[j] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(ars, ao + kb + 16, 0, 0));
            }
        }
#pragma unroll
        for (int j = 0; j < B; ++j)
            if (base + j < P) {
                // lanes 0..7 of a row: X's own chunk 2q, or X rotated (chunk 2q + 1);
                // lanes 8..15: Y rotated (chunk 2q), or Y's own chunk 2q + 1
                const bf16x8_t b0 = rotate8_select(xw[j], yw[j], hi);
                const bf16x8_t b1 = rotate8_select(yw[j], xw[j], !hi);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0[j], b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1[j], b1, acc, 0, 0, 0);
            }
    }
    return acc;
}

// One token: the k expert ids into sm.slot_expert (the slots are the entries), so that
// an item reads its expert from LDS and not from global memory, whose wait would also
// wait for the previous item's stores.
__device__ __forceinline__ void one_token_slots(DecodeSmem& sm, const DecodeArgs& g) {
    if ((int)threadIdx.x < g.k) sm.slot_expert[threadIdx.x] = g.ids[threadIdx.x];
    __syncthreads();
}

// The expert, routed-row count and first entry of active slot `slot`; false when the
// slot's expert id is invalid (one-token path: the slot is the entry itself).  The values
// are uniform over the wave (the workgroup, with a K split), and kept in scalar registers.
__device__ __forceinline__ bool slot_info(const DecodeArgs& g, const DecodeSmem& sm, bool one, int slot,
                                          int& e, int& M, int& e0) {
    if (one) {
        e = __builtin_amdgcn_readfirstlane(sm.slot_expert[slot]);
        M = 1;
        e0 = slot;
        return (unsigned)e < (unsigned)g.E;
    }
    e = __builtin_amdgcn_readfirstlane(sm.slot_expert[slot]);
    e0 = __builtin_amdgcn_readfirstlane(sm.pfx[e]);
    M = __builtin_amdgcn_readfirstlane(sm.pfx[e + 1]) - e0;
    return true;
}

// Walks this wave's items (kSplit: this workgroup's): its global wave (workgroup) id,
// then every (number of waves (workgroups))-th item after it.  For each item,
// f(slot, block).  (A shared work counter would balance better, but one atomic per
// item on one address serialises: thousands per launch.)
template <bool kSplit, class F>
__device__ __forceinline__ void for_items(int items, int nblk, F f) {
    const int nw = kSplit ? (int)gridDim.x : (int)gridDim.x * kWaves;
    const int first = kSplit ? (int)blockIdx.x
                             : (int)blockIdx.x * kWaves + __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    items = __builtin_amdgcn_readfirstlane(items);
    for (int item = first; item < items; item += nw) {
        const int slot = item / nblk;
        f(slot, item - slot * nblk);
    }
}

// K split: wave w takes pairs [P w / 4, P (w + 1) / 4) of the P pairs of 64 elements.
template <bool kSplit>
__device__ __forceinline__ void wave_pairs(int P, int& p0, int& p1) {
    if (kSplit) {
        const int w = threadIdx.x >> 6;
        p0 = P * w / kWaves;
        p1 = P * (w + 1) / kWaves;
    } else {
        p0 = 0;
        p1 = P;
    }
}

// K split: the four waves' partial sums added in wave order; the total is valid in
// wave 0.  red is double-buffered by the caller (`par`), so one barrier per call
// suffices: a buffer is rewritten only after the next call's barrier, which wave 0
// reaches after it has read the buffer.
template <bool kSplit>
__device__ __forceinline__ f32x4_t reduce_waves(f32x4_t acc, f32x4_t (*red)[kWaves][MOE_WAVE], int& par) {
    if (!kSplit) return acc;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    red[par][wave][lane] = acc;
    __syncthreads();
    f32x4_t s = red[par][0][lane];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) s += red[par][w][lane];
    par ^= 1;
    return s;
}

template <bool kSplit, int kAct = kActSwiGLU>
__global__ __launch_bounds__(kThreads, 3) void decode_w13(DecodeArgs g) {
    __shared__ DecodeSmem sm;
    __shared__ f32x4_t red[2][kWaves][MOE_WAVE];
    int par = 0;
    const int lane = threadIdx.x & 63;
    const bool lead = !kSplit || threadIdx.x < MOE_WAVE;   // the wave that stores
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I, k = g.k;
    const int nIB = I / 8;
    const bool one = g.T == 1;
    int items;
    if (one) {
        if (blockIdx.x == 0) decode_flags_one_token(g);
        one_token_slots(sm, g);
        items = k * nIB;
    } else {
        decode_setup(sm, g.ids, g.T, k, g.E, g.status, blockIdx.x == 0);
        items = sm.n_active * nIB;
    }
    int p0, p1;
    wave_pairs<kSplit>(d / 64, p0, p1);
    for_items<kSplit>(items, nIB, [&](int slot, int ib) {
        int e, M, e0;
        if (!slot_info(g, sm, one, slot, e, M, e0)) return;
        auto entry = [&](int m) { return one ? e0 : sm.ent[e0 + m]; };
        const int i0 = ib * 8;
        // columns 0..7: gate rows i0..i0+7 (X); columns 8..15: up rows I+i0..I+i0+7 (Y)
        const char* wb = reinterpret_cast<const char*>(g.w13 + ((size_t)e * 2 * I + i0) * d);
        const uint32_t xo = (uint32_t)((lane & 7) * d + 64 * p0) * 2u;
        const uint32_t yo = xo + (uint32_t)I * (uint32_t)d * 2u;
        for (int m0 = 0; m0 < M; m0 += 16) {
            const int m = m0 + n;
            const bool mv = m < M;
            const uint32_t xoff = mv ? (uint32_t)((entry(m) / k) * d + 64 * p0) * 2u : kNoRow;
            const f32x4_t acc = reduce_waves<kSplit>(
                mma_line_pairs(wb, xo, wb, yo, rows_rsrc(g.x, (uint32_t)g.T * d * 2u), xoff, p1 - p0), red, par);
            // lane l holds rows 4 kq + z of column n; the up value of gate column c < 8
            // sits in lane l + 8 of the same 16-lane group
            float up[4];
#pragma unroll
            for (int z = 0; z < 4; ++z) up[z] = __shfl_down(acc[z], 8, 16);
            if (lead && n < 8) {
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const int mm = m0 + 4 * kq + z;
                    if (mm < M)
                        g.a[(size_t)entry(mm) * I + i0 + n] = (uint16_t)f32_to_bf16(act_f<kAct>(acc[z]) * up[z]);
                }
            }
        }
    });
}

// W13 with more items than resident workgroups (many tokens): the K split of decode_w13,
// with the next unit's weights in flight while the current unit's products, wave
// reduction and stores run, so that the reduction's barrier does not leave the memory
// pipe empty.  A unit is (item, group of 16 routed rows).  The unit's x rows sit in LDS
// (copied straight from memory, zeros past the expert's rows), so that a wave's
// registers hold only weights, two units' worth; workgroup b takes a contiguous range of
// items, mostly blocks of one expert, whose x rows are copied once.  A wave's share of K
// is at most kPipePairs pairs and d at most kPipeMaxD; the launcher checks.
constexpr int kPipePairs = kBatch / 2;
constexpr int kPipeMaxD = 2048;
constexpr int kPipeRowBytes = 2 * kPipeMaxD + 16;     // padded: 16 rows' fragment reads hit every bank once

struct PipeUnit {
    int it, m0, e, M, e0;
    bool valid;
};

template <int kAct>
__global__ __launch_bounds__(kThreads, 2) void decode_w13_pipe(DecodeArgs g) {
    __shared__ DecodeSmem sm;
    __shared__ f32x4_t red[2][kWaves][MOE_WAVE];
    __shared__ __attribute__((aligned(16))) char xs[16 * kPipeRowBytes];
    int par = 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool lead = wave == 0;                           // the wave that stores
    const bool hi = (lane & 8) != 0;
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I, k = g.k;
    const int nIB = I / 8;
    const bool one = g.T == 1;
    int items;
    if (one) {
        if (blockIdx.x == 0) decode_flags_one_token(g);
        one_token_slots(sm, g);
        items = k * nIB;
    } else {
        decode_setup(sm, g.ids, g.T, k, g.E, g.status, blockIdx.x == 0);
        items = sm.n_active * nIB;
    }
    items = __builtin_amdgcn_readfirstlane(items);
    const int G = gridDim.x, b = blockIdx.x;
    const int q = items / G, r = items - q * G;
    const int it_begin = b * q + (b < r ? b : r);
    const int it_end = it_begin + q + (b < r ? 1 : 0);
    int p0, p1;
    wave_pairs<true>(d / 64, p0, p1);
    const int P = p1 - p0;

    // the first valid unit at or after item it (row group 0)
    auto unit_at = [&](int it) {
        PipeUnit u;
        u.valid = false;
        u.m0 = 0;
        for (; it < it_end; ++it) {
            int e, M, e0;
            if (slot_info(g, sm, one, it / nIB, e, M, e0)) {
                u.it = it; u.e = e; u.M = M; u.e0 = e0; u.valid = true;
                return u;
            }
        }
        u.it = it_end; u.e = 0; u.M = 0; u.e0 = 0;
        return u;
    };
    auto next_unit = [&](const PipeUnit& u) {
        if (u.m0 + 16 < u.M) {
            PipeUnit v = u;
            v.m0 += 16;
            return v;
        }
        return unit_at(u.it + 1);
    };
    auto entry = [&](const PipeUnit& u, int m) { return one ? u.e0 : sm.ent[u.e0 + m]; };
    auto same_rows = [&](const PipeUnit& u, const PipeUnit& v) { return u.it / nIB == v.it / nIB && u.m0 == v.m0; };

    // x rows m0 .. m0 + 15 of unit u into xs (row i at i * kPipeRowBytes), 1 KiB per copy:
    // copy c of the 16 * (2d / 1024) is row c / (2d / 1024), piece c % (2d / 1024); wave w
    // issues copies w, w + 4, ...; rows past the expert's read zeros (offset past the end)
    const __amdgpu_buffer_rsrc_t xrs = rows_rsrc(g.x, (uint32_t)g.T * d * 2u);
    const uint32_t xs0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)xs;
    auto fill_x = [&](const PipeUnit& u) {
        const int pieces = (2 * d) / 1024;
        for (int c = wave; c < 16 * pieces; c += kWaves) {
            const int row = c / pieces, piece = c - row * pieces;
            const int m = u.m0 + row;
            const uint32_t src = m < u.M ? (uint32_t)(entry(u, m) / k) * (uint32_t)d * 2u + 1024u * piece + 16u * lane
                                         : kNoRow;
            const uint32_t dst = xs0 + (uint32_t)(row * kPipeRowBytes + 1024 * piece);
            asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                         :: "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(src), "s"(xrs) : "memory");
        }
    };
    const uint32_t xo = (uint32_t)((lane & 7) * d + 64 * p0) * 2u + 16u * (uint32_t)(lane >> 3);
    const uint32_t yo = xo + (uint32_t)I * (uint32_t)d * 2u;
    // weights of unit u: columns 0..7 gate rows i0..i0+7 (X), 8..15 up rows (Y)
    auto load_w = [&](const PipeUnit& u, bf16x8_t xw[kPipePairs], bf16x8_t yw[kPipePairs]) {
        const int i0 = (u.it - (u.it / nIB) * nIB) * 8;
        const char* wb = reinterpret_cast<const char*>(g.w13 + ((size_t)u.e * 2 * I + i0) * d);
#pragma unroll
        for (int j = 0; j < kPipePairs; ++j)
            if (j < P) {
                xw[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(wb + (xo + 128u * j)));
                yw[j] = __builtin_nontemporal_load(reinterpret_cast<const bf16x8_t*>(wb + (yo + 128u * j)));
            }
    };
    // A row (lane & 15) of the pair chunks from xs
    const char* xrow = xs + n * kPipeRowBytes + 128 * p0 + 32 * kq;
    // products, wave reduction and the stores of a for unit u
    auto finish = [&](const PipeUnit& u, const bf16x8_t xw[kPipePairs], const bf16x8_t yw[kPipePairs]) {
        f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kPipePairs; ++j)
            if (j < P) {
                const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(xrow + 128 * j);
                const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(xrow + 128 * j + 16);
                const bf16x8_t b0 = rotate8_select(xw[j], yw[j], hi);
                const bf16x8_t b1 = rotate8_select(yw[j], xw[j], !hi);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a0, b0, acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a1, b1, acc, 0, 0, 0);
            }
        acc = reduce_waves<true>(acc, red, par);           // ends with a barrier: xs is free again
        float up[4];
#pragma unroll
        for (int z = 0; z < 4; ++z) up[z] = __shfl_down(acc[z], 8, 16);
        if (lead && n < 8) {
            const int i0 = (u.it - (u.it / nIB) * nIB) * 8;
#pragma unroll
            for (int z = 0; z < 4; ++z) {
                const int mm = u.m0 + 4 * kq + z;
                if (mm < u.M) g.a[(size_t)entry(u, mm) * I + i0 + n] = (uint16_t)f32_to_bf16(act_f<kAct>(acc[z]) * up[z]);
            }
        }
    };
    // the x rows of a unit copied and published; with `after`, the next unit's weights
    // (2 P loads) were issued after the copies, and the wait leaves them in flight
    auto wait_x = [&](bool after) {
        if (after && P == kPipePairs) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    };
    static_assert(2 * kPipePairs == 16, "the wait above is written as vmcnt(16)");

    // Two weight buffers; the unit in buffer 0 and the next one's weights in flight into
    // buffer 1, then the roles swap.  When a unit's x rows differ from the previous
    // unit's, they are copied into xs once the previous unit's products are done (its
    // reduction ends with a barrier), the following unit's weights go out behind them,
    // and the wait covers the copies (and the older loads) only.
    bf16x8_t wx0[kPipePairs], wy0[kPipePairs], wx1[kPipePairs], wy1[kPipePairs];
    PipeUnit u = unit_at(it_begin);
    if (!u.valid) return;
    load_w(u, wx0, wy0);
    fill_x(u);
    PipeUnit v = next_unit(u);
    if (v.valid) load_w(v, wx1, wy1);
    wait_x(v.valid);
    while (true) {
        finish(u, wx0, wy0);                       // unit u (buffer 0); v's weights in buffer 1
        if (!v.valid) break;
        const bool fresh_v = !same_rows(u, v);
        if (fresh_v) fill_x(v);
        u = next_unit(v);
        if (u.valid) load_w(u, wx0, wy0);
        if (fresh_v) wait_x(u.valid);
        finish(v, wx1, wy1);                       // unit v (buffer 1); u's weights in buffer 0
        if (!u.valid) break;
        const bool fresh_u = !same_rows(v, u);
        if (fresh_u) fill_x(u);
        v = next_unit(u);
        if (v.valid) load_w(v, wx1, wy1);
        if (fresh_u) wait_x(v.valid);
    }
}

template <bool kSplit>
__global__ __launch_bounds__(kThreads, 3) void decode_w2(DecodeArgs g) {
    __shared__ DecodeSmem sm;
    __shared__ f32x4_t red[2][kWaves][MOE_WAVE];
    int par = 0;
    const int lane = threadIdx.x & 63;
    const bool lead = !kSplit || threadIdx.x < MOE_WAVE;
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I, k = g.k;
    const int nNB = d / 16;
    const bool one = g.T == 1;
    int items;
    if (one) {
        one_token_slots(sm, g);
        items = k * nNB;
    } else {
        decode_setup(sm, g.ids, g.T, k, g.E, g.status, false);
        items = sm.n_active * nNB;
    }
    int p0, p1;
    wave_pairs<kSplit>(I / 64, p0, p1);
    for_items<kSplit>(items, nNB, [&](int slot, int nb) {
        int e, M, e0;
        if (!slot_info(g, sm, one, slot, e, M, e0)) return;
        auto entry = [&](int m) { return one ? e0 : sm.ent[e0 + m]; };
        const int n0 = nb * 16;
        const char* wb = reinterpret_cast<const char*>(g.w2 + ((size_t)e * d + n0) * I);
        const uint32_t xo = (uint32_t)((lane & 7) * I + 64 * p0) * 2u;                   // columns 0..7
        const uint32_t yo = xo + (uint32_t)I * 16u;                                        // columns 8..15
        for (int m0 = 0; m0 < M; m0 += 16) {
            const int m = m0 + n;
            const bool mv = m < M;
            const uint32_t ao = mv ? (uint32_t)(entry(m) * I + 64 * p0) * 2u : kNoRow;
            const f32x4_t acc = reduce_waves<kSplit>(
                mma_line_pairs(wb, xo, wb, yo, rows_rsrc(g.a, (uint32_t)(g.T * k) * I * 2u), ao, p1 - p0), red, par);
            if (lead) {
#pragma unroll
                for (int z = 0; z < 4; ++z) {
                    const int mm = m0 + 4 * kq + z;
                    if (mm < M) g.o[(size_t)entry(mm) * d + n0 + n] = (uint16_t)f32_to_bf16(acc[z]);
                }
            }
        }
    });
}

// One token: the W2 products of all k experts and the combine, 8 output features per
// workgroup: y[n] = sum_j s_j * bf16(W2_{e_j}[n] . a_j) in FP32, j ascending from +0.0
// (the combine kernel's order and rounding, so the result equals the three-launch
// path's).  Experts 2p and 2p + 1 share one MFMA: its columns 0..7 are rows n0 .. n0 + 7
// of W2 of expert 2p, columns 8..15 the same rows of expert 2p + 1, A row 0 is a_2p and
// row 1 is a_2p+1, so D[0][c] and D[1][8 + c] are the two experts' outputs.  Wave w takes
// the pairs w, w + 4, ...; an invalid expert id contributes 0.  One workgroup per CU (d / 8
// of them), each wave loading 12 K pairs (768 elements) at once: at K = I = 768 its whole
// pair of experts in one round trip.
__global__ __launch_bounds__(kThreads, 1) void decode_w2_one(DecodeArgs g) {
    __shared__ float ov[kMaxTopK][8];
    __shared__ float sc[kMaxTopK];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15, kq = lane >> 4;
    const int d = g.d, I = g.I, k = g.k;
    const int npair = (k + 1) / 2;
    // the scores, loaded before the weights so that the combine does not wait for them
    // once the products are done (they reach LDS with the products, below)
    const float score = tid < k ? g.scores[tid] : 0.f;
    // expert id of slot j, or -1 (j >= k or an invalid id); uniform, read before the
    // weight loads that depend on it
    auto expert = [&](int j) {
        const int e = j < k ? __builtin_amdgcn_readfirstlane(g.ids[j]) : -1;
        return (unsigned)e < (unsigned)g.E ? e : -1;
    };
    for (int nb = blockIdx.x; nb < d / 8; nb += gridDim.x) {
        const int n0 = nb * 8;
        for (int p = wave; p < npair; p += kWaves) {
            // B columns 0..7 (X): expert slot 2p; columns 8..15 (Y): slot 2p + 1
            const int e_x = expert(2 * p), e_y = expert(2 * p + 1);
            const bool vx = e_x >= 0, vy = e_y >= 0;
            const int ex = vx ? e_x : 0;
            const int ey = vy ? e_y : 0;
            const char* xb = reinterpret_cast<const char*>(g.w2 + ((size_t)ex * d + n0) * I);
            const char* yb = reinterpret_cast<const char*>(g.w2 + ((size_t)ey * d + n0) * I);
            const uint32_t wo = (uint32_t)((lane & 7) * I) * 2u;
            const int jr = 2 * p + n;                       // expert slot of A row n (rows 0, 1)
            const bool rv = (n == 0 && vx) || (n == 1 && vy);
            const uint32_t ao = rv ? (uint32_t)(jr * I) * 2u : kNoRow;
            const f32x4_t acc = mma_line_pairs<12>(xb, wo, yb, wo, rows_rsrc(g.a, (uint32_t)k * I * 2u), ao, I / 64);
            // lanes with kq = 0 hold rows 0..3 of column n
            if (kq == 0) {
                if (n < 8 && 2 * p < k) ov[2 * p][n] = vx ? acc[0] : 0.f;
                if (n >= 8 && 2 * p + 1 < k) ov[2 * p + 1][n - 8] = vy ? acc[1] : 0.f;
            }
        }
        if (tid < k) sc[tid] = score;
        __syncthreads();
        if (tid < 8) {
            float y = 0.f;
            for (int j = 0; j < k; ++j) y = __builtin_fmaf(sc[j], bf16_to_f32(f32_to_bf16(ov[j][tid])), y);
            g.y[n0 + tid] = (uint16_t)f32_to_bf16(y);
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------- "Mega" decode
// The blog post's Mega mode ("What it is selling": both projections fused into a chunked
// pipeline) for small batches: one launch streams every active expert's W13 and W2 once,
// with no round trip of the SwiGLU output through memory, and a second, light launch adds
// the chunks' partial outputs and combines them.  A work item of the first launch is
// (active expert e, chunk c of 32 intermediate columns), eight waves per item; for each 16
// routed rows of e:
//   * the item's loads are issued at its start: the routed rows of x (copied straight to
//     LDS), wave w's share of W13 (8 gate and 8 up rows for intermediate columns
//     c*32 + 8 (w % 4) .., over K half w / 4) and half of its share of W2 (the chunk's 32
//     columns, 64 contiguous bytes, of every 8th block of 16 W2 rows); the other half of
//     W2 goes out as soon as the W13 products have freed their registers;
//   * part 1: g, u for the chunk (the two K halves added through LDS in a fixed order) and
//     a = silu(g) u rounded to BF16 (where the staged path rounds it) into LDS;
//   * part 2: the chunk's share of the expert output, o_c[m][n] = sum_{i in chunk}
//     W2_e[n][i] a[m][i], one MFMA per 16 rows of W2, in FP32, written to
//     part[entry][c][n].
// The combine launch then computes
//   y[t][n] = sum_j s[t][j] * bf16(sum_c part[t*k + j][c][n])   (c in a fixed order, then
// j ascending from +0.0, FP32, one rounding): the staged path's rounding points, with only
// the FP32 summation order of o differing.
constexpr int kMegaChunk = 32;     // intermediate columns per mega item
constexpr int kMegaThreads = 512;  // eight waves per item
constexpr int kMegaKC = 64;        // K steps of 32 per load round (2048 elements; two halves)
constexpr int kMegaNB = 16;        // W2 n-blocks of 16 per wave per load round (d <= 2048: all)

template <int kAct>
__global__ __launch_bounds__(kMegaThreads, 1) void mega_decode(DecodeArgs g, float* __restrict__ part) {
    constexpr int IC = kMegaChunk;
    constexpr int kHalf = kMegaKC / 2;            // K steps per wave per load round
    __shared__ DecodeSmem sm;
    __shared__ __attribute__((aligned(16))) uint16_t xs[16][kMegaKC * 32];   // x of 16 routed rows, a K chunk
    __shared__ __attribute__((aligned(16))) uint16_t as[16][IC];            // a of 16 routed rows, BF16
    __shared__ f32x4_t gu[4][MOE_WAVE];                                      // K half 1 of each block
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, kq = lane >> 4;
    const int blk = wave & 3, half = wave >> 2;
    const int d = g.d, I = g.I, k = g.k, C = I / IC;
    const int S = d / 32;
    const bool one = g.T == 1;
    int items;
    if (one) {
        if (blockIdx.x == 0 && tid < kThreads) decode_flags_one_token(g);
        one_token_slots(sm, g);
        items = k * C;
    } else {
        decode_setup(sm, g.ids, g.T, k, g.E, g.status, blockIdx.x == 0);
        items = sm.n_active * C;
    }
    // consecutive items (neighbouring chunks of one expert, which share the 128-byte lines
    // of W2) on consecutive workgroups of one XCD
    const int G = gridDim.x;
    const int vid = (G % 8 == 0) ? (int)(blockIdx.x % 8) * (G / 8) + (int)(blockIdx.x / 8) : (int)blockIdx.x;
    for (int item = vid; item < items; item += G) {
        const int slot = item / C, c = item - slot * C;
        int e, M, e0;
        if (!slot_info(g, sm, one, slot, e, M, e0)) continue;
        auto entry = [&](int m) { return one ? e0 : sm.ent[e0 + m]; };
        // W2 loads through a buffer resource over expert e's matrix: lane offset in a VGPR,
        // the n-block step in an SGPR (64-bit addresses per load would not fit the registers)
        const uint64_t w2b = (uint64_t)(uintptr_t)(g.w2 + (size_t)e * d * I);
        const __amdgpu_buffer_rsrc_t w2rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(uintptr_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(w2b >> 32)) << 32) |
                               (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)w2b)),
            (short)0, __builtin_amdgcn_readfirstlane(d * I * 2), 0x00020000);
        const int w2off = ((16 * wave + n) * I + c * IC + 8 * kq) * 2;   // bytes
        const int w2step = 8 * 16 * I * 2;                                 // bytes between this wave's n-blocks
        auto ld_w2 = [&](int q) {
            const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(w2rs, w2off, q * w2step, 0);
            return __builtin_bit_cast(bf16x8_t, v);
        };
        const int i0 = c * IC + 8 * blk;
        const int wr = (n < 8) ? (i0 + n) : (I + i0 + n - 8);
        const uint16_t* w13r = g.w13 + ((size_t)e * 2 * I + wr) * d + 8 * kq;
        const int nq_w = ((d / 16) - wave + 7) / 8;   // W2 n-blocks of this wave
        for (int m0 = 0; m0 < M; m0 += 16) {
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
            bf16x8_t wb[kMegaNB];
            for (int kc = 0; kc < S; kc += kMegaKC) {
                // the routed x rows m0 .. min(M, m0 + 16) - 1 of this K chunk go straight to
                // LDS (1 KiB per wave copy; rows past M stay as they are: they only feed
                // output rows that are never used), then this wave's W13 loads of the chunk
                // (K half `half`) and, in the first chunk, its W2 loads
                const int kw = (S - kc < kMegaKC ? S - kc : kMegaKC) * 32;    // x elements in the chunk
                const int rows = M - m0 < 16 ? M - m0 : 16;
                const int pieces = (kw + 511) / 512;                         // 512 elements per copy
                const int ncopy = rows * pieces;
                for (int q = wave; q < ncopy; q += kMegaThreads / MOE_WAVE) {
                    const int r = q / pieces, part512 = q - r * pieces;
                    const uint32_t dst = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint16_t*)&xs[r][512 * part512];
                    // lanes past the chunk (a last copy of a row shorter than 512) read the
                    // chunk's last 8 elements again; those LDS columns are never read
                    int col = 512 * part512 + 8 * lane;
                    col = col < kw - 8 ? col : kw - 8;
                    const uint32_t voff = (uint32_t)(((size_t)(entry(m0 + r) / k) * d + kc * 32 + col) * 2);
                    asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, %2"
                                 :: "s"(__builtin_amdgcn_readfirstlane(dst)), "v"(voff), "s"(g.x) : "memory");
                }
                const int s0 = kc + half * kHalf;
                bf16x8_t wv[kHalf];
#pragma unroll
                for (int s = 0; s < kHalf; ++s)
                    if (s0 + s < S) wv[s] = ld_bf16x8(w13r + 32 * (s0 + s));
                if (kc == 0) {
#pragma unroll
                    for (int q = 0; q < kMegaNB / 2; ++q)
                        if (q < nq_w) wb[q] = ld_w2(q);
                }
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");           // the x copies (and the rest)
                __syncthreads();
#pragma unroll
                for (int s = 0; s < kHalf; ++s)
                    if (s0 + s < S) {
                        const bf16x8_t xa =
                            *reinterpret_cast<const bf16x8_t*>(&xs[n][32 * (half * kHalf + s) + 8 * kq]);
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, wv[s], acc, 0, 0, 0);
                    }
                __syncthreads();                  // xs is rewritten by the next chunk
            }
            // the rest of the first W2 round, now that the W13 registers are free
#pragma unroll
            for (int q = kMegaNB / 2; q < kMegaNB; ++q)
                if (q < nq_w) wb[q] = ld_w2(q);
            // the two K halves of block blk added in order (half 0 + half 1)
            if (half == 1) gu[blk][lane] = acc;
            __syncthreads();
            if (half == 0) {
                acc += gu[blk][lane];
                // the up value of gate column n < 8 sits in lane n + 8 of the same 16-lane group
                float up[4];
#pragma unroll
                for (int z = 0; z < 4; ++z) up[z] = __shfl_down(acc[z], 8, 16);
                if (n < 8) {
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        const int mm = m0 + 4 * kq + z;
                        as[4 * kq + z][8 * blk + n] =
                            mm < M ? (uint16_t)f32_to_bf16(act_f<kAct>(acc[z]) * up[z]) : (uint16_t)0;
                    }
                }
            }
            __syncthreads();
            // part 2: o_c = W2_e[:, chunk] a for n-blocks wave, wave + 8, ...
            const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(&as[n][8 * kq]);
            for (int q0 = 0; q0 < nq_w; q0 += kMegaNB) {
                if (q0 > 0) {
#pragma unroll
                    for (int q = 0; q < kMegaNB; ++q)
                        if (q0 + q < nq_w) wb[q] = ld_w2(q0 + q);
                }
#pragma unroll
                for (int q = 0; q < kMegaNB; ++q) {
                    if (q0 + q >= nq_w) break;
                    const int nb = wave + 8 * (q0 + q);
                    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
                    const f32x4_t o = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, wb[q], zero4, 0, 0, 0);
#pragma unroll
                    for (int z = 0; z < 4; ++z) {
                        const int mm = m0 + 4 * kq + z;
                        if (mm < M) part[((size_t)entry(mm) * C + c) * d + 16 * nb + n] = o[z];
                    }
                }
            }
            __syncthreads();                      // as and gu are rewritten by the next row group
        }
    }
}

// The combine of the mega path: units (t, block of 64 features).  Thread (h, j, 8
// features) sums the chunk partials c = h, h + 4, ... of entry t*k + j in ascending c; the
// four sums are then added in h order, rounded to BF16 (o), and the k experts added in j
// order; an entry with an invalid expert id contributes 0.
__global__ __launch_bounds__(kThreads) void mega_combine(DecodeArgs g, const float* __restrict__ part) {
    __shared__ float red[4][kMaxTopK][64];
    const int tid = threadIdx.x;
    const int d = g.d, k = g.k, C = g.I / kMegaChunk;
    const int units = g.T * (d / 64);
    for (int u = blockIdx.x; u < units; u += gridDim.x) {
        const int t = u / (d / 64), n0 = (u - t * (d / 64)) * 64;
        for (int p = tid; p < 4 * k * 8; p += kThreads) {
            const int h = p & 3, f8 = ((p >> 2) & 7) * 8, j = p >> 5;
            const int q = t * k + j;
            f32x4_t o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
            if ((unsigned)g.ids[q] < (unsigned)g.E) {
                const float* src = part + (size_t)q * C * d + n0 + f8;
                constexpr int kL = 8;             // chunks per thread with loads in flight at once
                for (int cb = h; cb < C; cb += 4 * kL) {
                    f32x4_t v[kL][2];
#pragma unroll
                    for (int l = 0; l < kL; ++l) {
                        const int cc = cb + 4 * l;
                        if (cc < C) {
                            v[l][0] = *reinterpret_cast<const f32x4_t*>(src + (size_t)cc * d);
                            v[l][1] = *reinterpret_cast<const f32x4_t*>(src + (size_t)cc * d + 4);
                        }
                    }
#pragma unroll
                    for (int l = 0; l < kL; ++l)
                        if (cb + 4 * l < C) { o0 += v[l][0]; o1 += v[l][1]; }
                }
            }
#pragma unroll
            for (int z = 0; z < 4; ++z) { red[h][j][f8 + z] = o0[z]; red[h][j][f8 + 4 + z] = o1[z]; }
        }
        __syncthreads();
        if (tid < 64) {
            float y = 0.f;
            for (int j = 0; j < k; ++j) {
                const bool valid = (unsigned)g.ids[t * k + j] < (unsigned)g.E;
                const float o = ((red[0][j][tid] + red[1][j][tid]) + red[2][j][tid]) + red[3][j][tid];
                y = __builtin_fmaf(g.scores[t * k + j], valid ? bf16_to_f32(f32_to_bf16(o)) : 0.f, y);
            }
            g.y[(size_t)t * d + n0 + tid] = (uint16_t)f32_to_bf16(y);
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_decode_w2_one(const DecodeArgs& g, int num_cu, hipStream_t s) {
    if (g.T != 1 || g.k > kMaxTopK) return hipErrorInvalidValue;
    const int cap = 3 * num_cu;
    int grid = g.d / 8;
    grid = grid < cap ? grid : cap;
    hipLaunchKernelGGL(decode_w2_one, dim3(grid), dim3(kThreads), 0, s, g);
    return hipGetLastError();
}

// Items of a launch with `slots` active experts at most, `nblk` items per expert and
// `ksteps` K steps of 32 per item: one workgroup (four waves splitting K) per item when
// the items do not fill the resident wave slots, or when each wave still streams a full
// batch of loads (the items then divide evenly over workgroups instead of leaving the
// last round of waves half empty); else one wave per item.
template <class K1, class K2>
hipError_t launch_decode(K1 wave_kernel, K2 split_kernel, const DecodeArgs& g, int nblk, int ksteps,
                         int num_cu, hipStream_t s) {
    const int R = g.T * g.k;
    if (R <= 0) return hipSuccess;
    const int slots = R < g.E ? R : g.E;                  // active experts at most
    const int items = slots * nblk;
    const int cap = 3 * num_cu;                           // resident workgroups
    if (items < cap * kWaves || ksteps >= kWaves * kBatch) {
        const int grid = items < cap ? items : cap;
        hipLaunchKernelGGL(split_kernel, dim3(grid), dim3(kThreads), 0, s, g);
    } else {
        int grid = (items + kWaves - 1) / kWaves;
        grid = grid < cap ? grid : cap;
        hipLaunchKernelGGL(wave_kernel, dim3(grid), dim3(kThreads), 0, s, g);
    }
    return hipGetLastError();
}

hipError_t launch_decode_w13(const DecodeArgs& g, int num_cu, hipStream_t s) {
    // many items per workgroup (many tokens) and a wave's K share within kPipePairs pairs:
    // the pipelined kernel, two workgroups per CU
    const int R = g.T * g.k;
    const int slots = R < g.E ? R : g.E;
    const int items = slots * (g.I / 8);
    if (R > 0 && g.d <= kPipeMaxD && g.d <= 64 * kWaves * kPipePairs && g.d % 512 == 0 && items >= 8 * num_cu) {
        const int grid = 2 * num_cu;
        if (g.act == kActGeGLU) hipLaunchKernelGGL(decode_w13_pipe<kActGeGLU>, dim3(grid), dim3(kThreads), 0, s, g);
        else if (g.act == kActReGLU) hipLaunchKernelGGL(decode_w13_pipe<kActReGLU>, dim3(grid), dim3(kThreads), 0, s, g);
        else hipLaunchKernelGGL(decode_w13_pipe<kActSwiGLU>, dim3(grid), dim3(kThreads), 0, s, g);
        return hipGetLastError();
    }
    if (g.act == kActGeGLU)
        return launch_decode(decode_w13<false, kActGeGLU>, decode_w13<true, kActGeGLU>, g, g.I / 8, g.d / 32, num_cu, s);
    if (g.act == kActReGLU)
        return launch_decode(decode_w13<false, kActReGLU>, decode_w13<true, kActReGLU>, g, g.I / 8, g.d / 32, num_cu, s);
    return launch_decode(decode_w13<false>, decode_w13<true>, g, g.I / 8, g.d / 32, num_cu, s);
}

hipError_t launch_decode_w2(const DecodeArgs& g, int num_cu, hipStream_t s) {
    return launch_decode(decode_w2<false>, decode_w2<true>, g, g.d / 16, g.I / 32, num_cu, s);
}

int mega_chunk(int, int) { return kMegaChunk; }

hipError_t launch_mega_decode(const DecodeArgs& g, float* part, int num_cu, hipStream_t s) {
    const int R = g.T * g.k;
    if (R <= 0) return hipSuccess;
    if (R > kMaxDecodeRows || g.k > kMaxTopK || g.d % 64 != 0 || g.I % kMegaChunk != 0)
        return hipErrorInvalidValue;
    const int slots = R < g.E ? R : g.E;
    int grid = slots * (g.I / kMegaChunk);
    const int cap = 2 * num_cu;
    grid = grid < cap ? grid : cap;
    if (grid >= 8) grid -= grid % 8;
    const dim3 gd(grid), bd(kMegaThreads);
    if (g.act == kActGeGLU) hipLaunchKernelGGL((mega_decode<kActGeGLU>), gd, bd, 0, s, g, part);
    else if (g.act == kActReGLU) hipLaunchKernelGGL((mega_decode<kActReGLU>), gd, bd, 0, s, g, part);
    else hipLaunchKernelGGL((mega_decode<kActSwiGLU>), gd, bd, 0, s, g, part);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int cgrid = g.T * (g.d / 64);
    cgrid = cgrid < 4 * num_cu ? cgrid : 4 * num_cu;
    hipLaunchKernelGGL(mega_combine, dim3(cgrid), dim3(kThreads), 0, s, g, part);
    return hipGetLastError();
}

}  // namespace moe
