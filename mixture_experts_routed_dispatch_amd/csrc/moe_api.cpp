// moe_api.cpp -- host side of libmoe: plan, validation, workspace layout and launch
// sequencing behind the C ABI declared in include/moe.h.
//
// Nothing here reads device data or synchronises, except moe_bind_workspace
// (clears the status word) and moe_get_status (reads it); every other entry
// point only enqueues kernels on the caller's stream.
#include <hip/hip_runtime.h>

#include <cstdlib>
#include <cstring>
#include <new>
#include <cstdio>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int64_t kMaxRoutedRows = 131072;   // nvfp4moe README, "Limits"
constexpr int kMaxExperts = 256;             // nvfp4moe README, "Limits"
constexpr size_t kMaxProfileRecords = 4096;
// the status region: the sticky device flags (cleared when a workspace is bound)
constexpr int kStatusWords = 1;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

}  // namespace

struct moe_plan_s {
    moe_config_t cfg;
    int64_t R;
    bool decode;
    // workspace offsets (bytes)
    size_t off_status, off_m_indptr, off_gather, off_slots, off_probs;
    size_t off_a, off_o, off_h, off_dh, off_dxp, off_xg, off_dys, off_xq, off_xs, off_xsr, off_aq, off_as;
    // MXFP8 backward: dO and (dg, du) quantized along d and 2I (codes, block-major scales), and
    // the weight-gradient operands in the token layout (P and Q codes and scales)
    size_t off_doq, off_dos, off_dhq, off_dhs, off_tp, off_tps, off_tq, off_tqs;
    size_t tp_feat, tq_feat;           // features of the largest P / Q token-layout operand
    int64_t ntok;                      // token-layout rows: T*k + 128 E
    size_t off_part, off_split;        // split weight-gradient tiles: partial sums, descriptors
    size_t off_mega;                   // mega decode: FP32 partial expert outputs [T*k, I / chunk, d]
    size_t ws_bytes;
    char* ws;
    size_t ws_size;
    int num_cu;
    bool have_saved_forward;
    bool h_aliased;                    // recompute_h: h occupies the dxp / xg / dys region
    bool dh_aliased;                   // BF16 training: dh occupies o's region (see below)
    int32_t* status_word;              // device status word of the last call (workspace or static scratch)
    // measurement-only event pairs around kernel stages (moe_profile)
    struct ProfRec { int stage; hipEvent_t a, b; };
    bool prof_on = false;
    std::vector<hipEvent_t> ev_free;
    std::vector<ProfRec> recs;

    template <class T> T* at(size_t off) const { return reinterpret_cast<T*>(ws + off); }

    hipEvent_t take_event() {
        hipEvent_t e = nullptr;
        if (!ev_free.empty()) { e = ev_free.back(); ev_free.pop_back(); return e; }
        if (hipEventCreate(&e) != hipSuccess) return nullptr;
        return e;
    }
    // returns a record index, or -1 when not recording
    int stage_begin(int stage, hipStream_t s) {
        if (!prof_on || recs.size() >= kMaxProfileRecords) return -1;
        ProfRec r{stage, take_event(), take_event()};
        if (!r.a || !r.b || hipEventRecord(r.a, s) != hipSuccess) {
            if (r.a) ev_free.push_back(r.a);
            if (r.b) ev_free.push_back(r.b);
            return -1;
        }
        recs.push_back(r);
        return (int)recs.size() - 1;
    }
    void stage_end(int idx, hipStream_t s) {
        if (idx >= 0) (void)hipEventRecord(recs[(size_t)idx].b, s);
    }
    ~moe_plan_s() {
        for (auto& r : recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
        for (auto e : ev_free) (void)hipEventDestroy(e);
    }
};

namespace {
// launch `fn` as one profiled stage
template <class F>
hipError_t staged(moe_plan_s* p, int stage, hipStream_t s, F&& fn) {
    const int idx = p->stage_begin(stage, s);
    const hipError_t e = fn();
    p->stage_end(idx, s);
    return e;
}
}  // namespace

namespace {
// MXFP8 backward (see moe_backward in moe.h): every expert product on MXFP8 operands
// quantized along its own reduction dimension
moe_status_t mx_backward(moe_plan_s* p, const void* dy, const void* x, const moe_weights_t* w, void* dx,
                         void* dw13, void* dw2, float* dscores, hipStream_t s) {
    const moe_config_t& c = p->cfg;
    const int64_t R = p->R;
    int32_t* m_indptr = p->at<int32_t>(p->off_m_indptr);
    const int32_t* gather = p->at<int32_t>(p->off_gather);
    const int32_t* slots = p->at<int32_t>(p->off_slots);
    const float* probs = p->at<float>(p->off_probs);
    uint16_t* a = p->at<uint16_t>(p->off_a);
    uint16_t* h = p->at<uint16_t>(p->off_h);
    uint16_t* dh = p->at<uint16_t>(p->off_dh);
    uint16_t* dxp = p->at<uint16_t>(p->off_dxp);        // dA, then dxp
    uint8_t* tp = p->at<uint8_t>(p->off_tp);
    uint8_t* tps = p->at<uint8_t>(p->off_tps);
    uint8_t* tq = p->at<uint8_t>(p->off_tq);
    uint8_t* tqs = p->at<uint8_t>(p->off_tqs);
    const uint16_t* dy16 = static_cast<const uint16_t*>(dy);
    const uint16_t* x16 = static_cast<const uint16_t*>(x);
    MxGemmArgs mg{};
    mg.T = c.T; mg.d = c.d; mg.I = c.I; mg.E = c.E; mg.k = c.k;
    mg.act = c.activation;
    mg.m_indptr = m_indptr; mg.gather = gather;
    mg.accumulate = c.wgrad_accumulate;
    hipError_t e;
    if (c.T == 0) {
        // no routed rows: every expert is empty and its weight gradient +0 (or kept)
        if ((e = launch_dispatch(nullptr, nullptr, 0, c.k, c.E, m_indptr, nullptr,
                                 nullptr, nullptr, p->at<int32_t>(p->off_status), s)) != hipSuccess)
            return MOE_ERR_HIP;
    } else {
        e = staged(p, MOE_STAGE_SCORE_GRAD, s, [&] {
            return launch_score_grad(dy16, p->at<uint16_t>(p->off_o), slots, c.T, c.k, c.d, dscores, s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        if (c.recompute_h) {
            // h and a again from the forward's quantized x (still in the workspace) and
            // W13: the same kernel and inputs, so the same values
            MxGemmArgs gr = mg;
            gr.xq = p->at<uint8_t>(p->off_xq); gr.xs = p->at<uint8_t>(p->off_xsr);
            gr.w13q = static_cast<const uint8_t*>(w->w13); gr.w13s = w->w13_scale;
            gr.aq = p->at<uint8_t>(p->off_aq); gr.as = p->at<uint8_t>(p->off_as);
            gr.h_out = h; gr.a_out = a;
            e = staged(p, MOE_STAGE_RECOMPUTE_H, s, [&] { return launch_gemm_mxfp8(MX_W13, gr, p->num_cu, s); });
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        uint8_t* doq = p->at<uint8_t>(p->off_doq);
        uint8_t* dos = p->at<uint8_t>(p->off_dos);
        uint8_t* dhq = p->at<uint8_t>(p->off_dhq);
        uint8_t* dhs = p->at<uint8_t>(p->off_dhs);
        e = staged(p, MOE_STAGE_QUANT_DO, s, [&] {
            return launch_mx_scaled_rows(dy16, c.T, c.k, slots, gather, probs, R, c.d, doq, dos, s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        // dA [R, I] = dO W2_e: P = W2_e^T [I, d] blocked along d
        MxGemmArgs g1 = mg;
        g1.Kp = c.d; g1.Np = c.I;
        g1.pq = w->w2t; g1.ps = w->w2t_scale; g1.qq = doq; g1.qs = dos;
        g1.out = dxp;
        e = staged(p, MOE_STAGE_DGRAD_W2, s, [&] { return launch_gemm_mxfp8(MX_PLAIN, g1, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_ACT_BWD, s, [&] {
            return launch_mx_act_backward(dxp, h, R, c.I, c.activation, dh, dhq, dhs, s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        // dxp [R, d] = (dg, du) W13_e: P = W13_e^T [d, 2I] blocked along 2I
        MxGemmArgs g2 = mg;
        g2.Kp = 2 * c.I; g2.Np = c.d;
        g2.pq = w->w13t; g2.ps = w->w13t_scale; g2.qq = dhq; g2.qs = dhs;
        g2.out = dxp;
        e = staged(p, MOE_STAGE_DGRAD_W13, s, [&] { return launch_gemm_mxfp8(MX_PLAIN_W13, g2, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_DX_COMBINE, s, [&] {
            return launch_combine(dxp, slots, nullptr, c.T, c.k, c.d, static_cast<uint16_t*>(dx), s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    // weight gradients: operands in the token layout (blocks of 32 routed rows of one expert)
    const int32_t* gth = c.T > 0 ? gather : nullptr;
    const float* prb = c.T > 0 ? probs : nullptr;
    e = staged(p, MOE_STAGE_QUANT_T, s, [&] {
        hipError_t qe = launch_mx_transpose_quant(a, c.E, (int)R, c.I, m_indptr, nullptr, nullptr, 0, false, tp, tps, s);
        if (qe != hipSuccess) return qe;
        return launch_mx_transpose_quant(dy16, c.E, (int)R, c.d, m_indptr, gth, prb, c.T, false, tq, tqs, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
    MxGemmArgs g3 = mg;                 // dW2_e [d, I] = sum_r dO_r a_r^T
    g3.Np = c.I; g3.Nq = c.d;
    g3.pq = tp; g3.ps = tps; g3.qq = tq; g3.qs = tqs;
    g3.out = static_cast<uint16_t*>(dw2);
    e = staged(p, MOE_STAGE_WGRAD_W2, s, [&] { return launch_gemm_mxfp8(MX_WGRAD, g3, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = staged(p, MOE_STAGE_QUANT_T, s, [&] {
        hipError_t qe = launch_mx_transpose_quant(x16, c.E, (int)R, c.d, m_indptr, gth, nullptr, c.T, false, tp, tps, s);
        if (qe != hipSuccess) return qe;
        return launch_mx_transpose_quant(dh, c.E, (int)R, 2 * c.I, m_indptr, nullptr, nullptr, 0, false, tq, tqs, s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
    MxGemmArgs g4 = mg;                 // dW13_e [2I, d] = sum_r dh_r x_r^T
    g4.Np = c.d; g4.Nq = 2 * c.I;
    g4.pq = tp; g4.ps = tps; g4.qq = tq; g4.qs = tqs;
    g4.out = static_cast<uint16_t*>(dw13);
    e = staged(p, MOE_STAGE_WGRAD_W13, s, [&] { return launch_gemm_mxfp8(MX_WGRAD_W13, g4, p->num_cu, s); });
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}
}  // namespace

extern "C" {

// The BF16 backward's router gradient comes from partial sums of the W2 data-gradient
// product (one FP32 per routed row and 64 columns of I, router_grad_slots per row), held
// in the split-tile buffer, when they fit there; else from o and dy.
static int router_grad_slots(int I) { return 4 * ((I + 255) / 256); }
static bool fused_router_grad(int64_t R, int I) {
    return (size_t)R * router_grad_slots(I) * sizeof(float) <= kGemmPartBytes;
}

moe_status_t moe_plan(const moe_config_t* cfg, moe_plan_t* out) {
    if (!cfg || !out) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    const moe_config_t c = *cfg;
    if (c.T < 0 || c.d <= 0 || c.I <= 0 || c.E <= 0 || c.k <= 0) return MOE_ERR_INVALID_ARG;
    if (c.precision != MOE_BF16 && c.precision != MOE_MXFP8_E4M3) return MOE_ERR_INVALID_ARG;
    if (c.training != 0 && c.training != 1) return MOE_ERR_INVALID_ARG;
    if (c.wgrad_accumulate != 0 && c.wgrad_accumulate != 1) return MOE_ERR_INVALID_ARG;
    if (c.wgrad_accumulate && !c.training) return MOE_ERR_UNSUPPORTED;
    if (c.recompute_h != 0 && c.recompute_h != 1) return MOE_ERR_INVALID_ARG;
    if (c.recompute_h && !c.training) return MOE_ERR_UNSUPPORTED;
    if (c.activation < MOE_ACT_SWIGLU || c.activation > MOE_ACT_REGLU) return MOE_ERR_INVALID_ARG;
    if (c.path != MOE_PATH_AUTO && c.path != MOE_PATH_PREFILL && c.path != MOE_PATH_DECODE)
        return MOE_ERR_INVALID_ARG;
    if (c.d % 64 != 0 || c.I % 64 != 0) return MOE_ERR_UNSUPPORTED;
    if (c.E > kMaxExperts || c.k > c.E || c.k > kMaxTopK) return MOE_ERR_UNSUPPORTED;
    const int64_t R = (int64_t)c.T * c.k;
    if (R > kMaxRoutedRows) return MOE_ERR_UNSUPPORTED;
    // MXFP8 kernels take K in stages of 64 codes and P tiles of 256 rows
    if (c.precision == MOE_MXFP8_E4M3 && (c.d % 256 != 0 || c.I % 128 != 0)) return MOE_ERR_UNSUPPORTED;
    // MXFP8 weight gradients address a token-layout operand (features x padded rows) with
    // 32-bit offsets
    if (c.precision == MOE_MXFP8_E4M3 && c.training &&
        (int64_t)(c.d > 2 * c.I ? c.d : 2 * c.I) * (R + (int64_t)kMxWgradPad * c.E) >= (1LL << 32))
        return MOE_ERR_UNSUPPORTED;
    // 32-bit byte offsets inside x, the routed intermediates and one expert's weights
    if ((int64_t)c.T * c.d * 2 >= (1LL << 31) || R * 2 * c.I * 2 >= (1LL << 31) ||
        (int64_t)2 * c.I * c.d * 2 >= (1LL << 31))
        return MOE_ERR_UNSUPPORTED;
    // small-batch inference runs the weight-streaming kernels (nvfp4moe README,
    // "MoE layer": batch-one and small-batch decode get their own launch grid)
    const bool decode_ok = c.training == 0 && c.precision == MOE_BF16 && R > 0 &&
                           R <= kMaxDecodeRows;
    if (c.path == MOE_PATH_DECODE && !decode_ok) return MOE_ERR_UNSUPPORTED;
    if (c.mega != 0 && c.mega != 1) return MOE_ERR_INVALID_ARG;
    if (c.mega && (!decode_ok || c.path == MOE_PATH_PREFILL)) return MOE_ERR_UNSUPPORTED;

    moe_plan_s* p = new (std::nothrow) moe_plan_s();
    if (!p) return MOE_ERR_INVALID_ARG;
    p->cfg = c;
    p->R = R;
    p->decode = c.path == MOE_PATH_DECODE || (c.path == MOE_PATH_AUTO && decode_ok);
    size_t off = 0;
    auto take = [&](size_t bytes) { const size_t o = off; off = align256(off + bytes); return o; };
    p->off_status = take(sizeof(int32_t) * kStatusWords);   // the sticky status word
    p->off_m_indptr = take(sizeof(int32_t) * (size_t)(c.E + 1));
    p->off_gather = take(sizeof(int32_t) * (size_t)R);
    p->off_slots = take(sizeof(int32_t) * (size_t)R);
    p->off_probs = take(sizeof(float) * (size_t)R);
    const bool mx = c.precision == MOE_MXFP8_E4M3;
    const bool mxt = mx && c.training;
    // a in BF16: the BF16 path's W2 operand; MXFP8 training keeps it for the weight gradient
    p->off_a = (!mx || c.training) ? take(2 * (size_t)R * c.I) : 0;
    p->off_o = take(2 * (size_t)R * c.d);
    const size_t h_bytes = 2 * (size_t)R * 2 * c.I;
    p->off_h = (c.training && !c.recompute_h) ? take(h_bytes) : 0;
    // BF16 training takes the router gradient from the W2 data-gradient partials, so the
    // backward never reads o: dh, first written by that product, takes o's place when it fits
    p->dh_aliased = c.training && !mx && fused_router_grad(R, c.I) && 2 * (size_t)c.I <= (size_t)c.d;
    p->off_dh = !c.training ? 0 : p->dh_aliased ? p->off_o : take(2 * (size_t)R * 2 * c.I);
    // MXFP8: dA [R, I] first, then dxp [R, d]
    p->off_dxp = c.training ? take(2 * (size_t)R * (mx && c.I > c.d ? c.I : c.d)) : 0;
    p->off_xg = (c.training && !mx) ? take(2 * (size_t)R * c.d) : 0;
    p->off_dys = (c.training && !mx) ? take(2 * (size_t)R * c.d) : 0;
    p->h_aliased = false;
    if (c.training && c.recompute_h && !mx) {
        // the recomputed h lives from the start of the backward to DGRAD W2; dxp, xg and
        // dys (consecutive) are first written after that, so h takes their place
        if (h_bytes <= p->off_dys + 2 * (size_t)R * c.d - p->off_dxp) {
            p->off_h = p->off_dxp;
            p->h_aliased = true;
        } else {
            p->off_h = take(h_bytes);
        }
    }
    p->off_xq = mx ? take((size_t)c.T * c.d) : 0;
    p->off_xs = mx ? take((size_t)c.T * c.d / 32) : 0;
    p->off_xsr = mx ? take((size_t)R * c.d / 32) : 0;
    p->off_aq = mx ? take((size_t)R * c.I) : 0;
    p->off_as = mx ? take((size_t)R * c.I / 32) : 0;
    p->ntok = R + (int64_t)kMxWgradPad * c.E;
    p->tp_feat = (size_t)(c.I > c.d ? c.I : c.d);              // P: a^T (I), then x^T (d)
    p->tq_feat = (size_t)(c.d > 2 * c.I ? c.d : 2 * c.I);      // Q: dO^T (d), then dh^T (2I)
    p->off_doq = mxt ? take((size_t)R * c.d) : 0;
    p->off_dos = mxt ? take((size_t)R * c.d / 32) : 0;
    p->off_dhq = mxt ? take((size_t)R * 2 * c.I) : 0;
    p->off_dhs = mxt ? take((size_t)R * 2 * c.I / 32) : 0;
    p->off_tp = mxt ? take(p->tp_feat * p->ntok) : 0;
    p->off_tps = mxt ? take(p->tp_feat * p->ntok / 32) : 0;
    p->off_tq = mxt ? take(p->tq_feat * p->ntok) : 0;
    p->off_tqs = mxt ? take(p->tq_feat * p->ntok / 32) : 0;
    if (mxt && c.recompute_h) {
        // the recomputed h is read last by the activation backward; the token-layout
        // operands are first written after the input gradients, so h takes their place
        if (h_bytes <= p->off_tqs + p->tq_feat * p->ntok / 32 - p->off_tp) {
            p->off_h = p->off_tp;
            p->h_aliased = true;
        } else {
            p->off_h = take(h_bytes);
        }
    }
    const bool gemms = !mx && !p->decode;
    p->off_split = take(sizeof(int32_t) * 4 * (kMaxPieces / 2 + 1));
    p->off_part = gemms && c.training ? take(kGemmPartBytes) : 0;
    p->off_mega = c.mega ? take(sizeof(float) * (size_t)R * (c.I / mega_chunk(c.T, c.k)) * c.d) : 0;
    p->ws_bytes = off;
    p->ws = nullptr;
    p->ws_size = 0;
    p->num_cu = 0;
    p->have_saved_forward = false;
    p->status_word = nullptr;
    *out = p;
    return MOE_OK;
}

size_t moe_workspace_bytes(moe_plan_t p) { return p ? p->ws_bytes : 0; }

size_t moe_plan_explain(moe_plan_t p, char* buf, size_t len) {
    if (!p) return 0;
    const moe_config_t& c = p->cfg;
    const int64_t R = p->R;
    const bool mx = c.precision == MOE_MXFP8_E4M3;
    const bool gemms = !mx && !p->decode;
    std::string out;
    char line[512];
    auto add = [&](const char* fmt, auto... args) {
        std::snprintf(line, sizeof line, fmt, args...);
        out += line;
    };
    add("moe plan: T=%d d=%d I=%d E=%d k=%d, %lld routed rows (T*k), %s, %s, %s path\n", c.T, c.d, c.I, c.E,
        c.k, (long long)R, mx ? "MXFP8 E4M3" : "BF16", c.training ? "training" : "inference",
        p->decode ? (c.mega ? "decode (weight-streaming, mega: one fused launch)" : "decode (weight-streaming)")
                  : "grouped-GEMM");
    if (c.training)
        add("options: weight gradients %s; h %s\n", c.wgrad_accumulate ? "accumulated" : "overwritten",
            c.recompute_h ? (p->h_aliased ? "recomputed in the backward, in the dX / WGRAD-operand region"
                                          : "recomputed in the backward, in a region of its own")
                          : "saved by the forward");
    add("workspace %zu bytes (%.1f MiB):\n", p->ws_bytes, p->ws_bytes / 1048576.0);
    add("  %-10s %14s  %-8s %s\n", "region", "bytes", "kind", "holds");
    const char* keep = c.training ? "saved" : "scratch";
    auto region = [&](const char* name, size_t bytes, const char* kind, const char* what) {
        if (bytes) add("  %-10s %14zu  %-8s %s\n", name, bytes, kind, what);
    };
    size_t saved = 0;
    auto saved_region = [&](const char* name, size_t bytes, const char* what) {
        region(name, bytes, keep, what);
        if (c.training) saved += bytes;
    };
    region("status", sizeof(int32_t), "flags", "sticky device routing flags (moe_get_status)");
    saved_region("m_indptr", sizeof(int32_t) * (size_t)(c.E + 1), "expert row offsets [E+1]");
    saved_region("gather", sizeof(int32_t) * (size_t)R, "token of each routed row [R]");
    saved_region("slots", sizeof(int32_t) * (size_t)R, "routed row of each (t, j) [T, k]");
    saved_region("probs", sizeof(float) * (size_t)R, "score of each routed row [R]");
    if (!mx || c.training)
        saved_region("a", 2 * (size_t)R * c.I, mx ? "SwiGLU output [R, I] BF16 (weight-gradient operand)"
                                                  : "SwiGLU output [R, I] BF16");
    if (p->dh_aliased)
        region("o", 2 * (size_t)R * c.d, "fwd/bwd", "expert outputs [R, d] BF16; in the backward dh (g, u gradient [R, 2I])");
    else
        saved_region("o", 2 * (size_t)R * c.d, "expert outputs [R, d] BF16");
    if (c.training) {
        const size_t hb = 2 * (size_t)R * 2 * c.I;
        if (c.recompute_h)
            region("h", p->h_aliased ? 0 : hb, "backward",
                   "W13 pre-activations (g, u) [R, 2I] BF16, recomputed");
        else
            saved_region("h", hb, "W13 pre-activations (g, u) [R, 2I] BF16");
        region("dh", p->dh_aliased ? 0 : 2 * (size_t)R * 2 * c.I, "backward", "gradient w.r.t. (g, u) [R, 2I] BF16");
        if (mx) {
            region("dxp", 2 * (size_t)R * (c.I > c.d ? c.I : c.d), "backward",
                   "dA [R, I] BF16, then the per-row input gradients [R, d] BF16");
            region("dOq", (size_t)R * c.d + (size_t)R * c.d / 32, "backward",
                   "probs * dy[gather] quantized along d: codes [R, d], scales [d/128, R, 4]");
            region("dhq", (size_t)R * 2 * c.I + (size_t)R * 2 * c.I / 32, "backward",
                   "(dg, du) quantized along 2I: codes [R, 2I], scales [2I/128, R, 4]");
            region("tokP", (p->tp_feat * p->ntok) * 33 / 32, "backward",
                   p->h_aliased ? "a^T, then x[gather]^T, quantized along routed rows (first h, recomputed)"
                                : "a^T, then x[gather]^T, quantized along routed rows (token layout)");
            region("tokQ", (p->tq_feat * p->ntok) * 33 / 32, "backward",
                   "dO^T, then (dg, du)^T, quantized along routed rows (token layout)");
        } else {
            region("dxp", 2 * (size_t)R * c.d, "backward",
                   p->h_aliased ? "per-row input gradients [R, d] BF16 (first h, recomputed, with xg and dys)"
                                : "per-row input gradients [R, d] BF16");
            region("xg", 2 * (size_t)R * c.d, "backward", "x[gather] [R, d] BF16 (weight-gradient operand)");
            region("dys", 2 * (size_t)R * c.d, "backward",
                   "probs * dy[gather] [R, d] BF16 (weight-gradient operand)");
        }
    }
    if (mx) {
        region("xq", (size_t)c.T * c.d, "scratch", "E4M3 codes of x [T, d]");
        region("xs", (size_t)c.T * c.d / 32, "scratch", "E8M0 scales of x [T, d/32]");
        region("xs_routed", (size_t)R * c.d / 32, "scratch", "scales of x[gather], block-major [d/128, R, 4]");
        region("aq", (size_t)R * c.I, "scratch", "E4M3 codes of a [R, I]");
        region("as", (size_t)R * c.I / 32, "scratch", "E8M0 scales of a (block-major)");
    }
    region("split", sizeof(int32_t) * 4 * (kMaxPieces / 2 + 1), "scratch", "split weight-gradient tiles");
    if (c.mega)
        region("mega", sizeof(float) * (size_t)R * (c.I / mega_chunk(c.T, c.k)) * c.d, "scratch",
               "mega decode: FP32 partial expert outputs [T*k, I/chunk, d]");
    if (gemms && c.training)
        region("part", kGemmPartBytes, "backward", "FP32 partial sums of split weight-gradient tiles");
    add("kept from the training forward for the backward: %zu bytes (%.1f MiB)\n", saved, saved / 1048576.0);
    add("limits: T*k <= %lld routed rows, E <= %d, k <= %d, d and I multiples of 64\n",
        (long long)kMaxRoutedRows, kMaxExperts, kMaxTopK);
    if (buf && len > 0) {
        const size_t n = out.size() < len - 1 ? out.size() : len - 1;
        std::memcpy(buf, out.data(), n);
        buf[n] = '\0';
    }
    return out.size();
}

moe_status_t moe_bind_workspace(moe_plan_t p, void* dptr, size_t bytes) {
    if (!p || !dptr) return MOE_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(dptr) % 256 != 0) return MOE_ERR_INVALID_ARG;
    if (bytes < p->ws_bytes) return MOE_ERR_WORKSPACE;
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_HIP;
    if (hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return MOE_ERR_HIP;
    if (hipMemset(static_cast<char*>(dptr) + p->off_status, 0, sizeof(int32_t) * kStatusWords) != hipSuccess)
        return MOE_ERR_HIP;
    p->ws = static_cast<char*>(dptr);
    p->ws_size = bytes;
    p->num_cu = ncu > 0 ? ncu : 256;
    p->have_saved_forward = false;
    p->status_word = p->at<int32_t>(p->off_status);
    return MOE_OK;
}

moe_status_t moe_plan_destroy(moe_plan_t p) {
    delete p;
    return MOE_OK;
}

moe_status_t moe_dispatch(moe_plan_t p, const int32_t* ids, const float* scores, int32_t* m_indptr,
                          int32_t* gather, int32_t* slots, float* probs, void* stream) {
    if (!p || !m_indptr) return MOE_ERR_INVALID_ARG;
    if (p->R > 0 && (!ids || !scores || !gather || !slots || !probs)) return MOE_ERR_INVALID_ARG;
    if (!p->ws) return MOE_ERR_WORKSPACE;
    const moe_config_t& c = p->cfg;
    p->status_word = p->at<int32_t>(p->off_status);
    hipError_t e = launch_dispatch(ids, scores, c.T, c.k, c.E, m_indptr,
                                   gather, slots, probs, p->at<int32_t>(p->off_status),
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_quantize_mxfp8(const void* v, int64_t rows, int32_t K, uint8_t* codes,
                                uint8_t* scales, void* stream) {
    if (rows < 0 || K <= 0 || K % 32 != 0) return MOE_ERR_INVALID_ARG;
    if (rows > 0 && (!v || !codes || !scales)) return MOE_ERR_INVALID_ARG;
    hipError_t e = launch_quantize_mxfp8(static_cast<const uint16_t*>(v), rows, K, codes, scales, false,
                                         static_cast<hipStream_t>(stream));
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_prepare_weights(moe_plan_t p, const void* w13, const void* w2, uint8_t* w13_q,
                                 uint8_t* w13_s, uint8_t* w2_q, uint8_t* w2_s, void* stream) {
    if (!p || !w13 || !w2 || !w13_q || !w13_s || !w2_q || !w2_s) return MOE_ERR_INVALID_ARG;
    const moe_config_t& c = p->cfg;
    if (c.d % 128 != 0 || c.I % 128 != 0) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // block-major scales (the layout the MXFP8 GEMMs copy from)
    if (launch_quantize_mxfp8(static_cast<const uint16_t*>(w13), (int64_t)c.E * 2 * c.I, c.d, w13_q, w13_s,
                              true, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (launch_quantize_mxfp8(static_cast<const uint16_t*>(w2), (int64_t)c.E * c.d, c.I, w2_q, w2_s, true,
                              s) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t moe_prepare_weights_backward(moe_plan_t p, const void* w13, const void* w2, uint8_t* w13t_q,
                                          uint8_t* w13t_s, uint8_t* w2t_q, uint8_t* w2t_s, void* stream) {
    if (!p || !w13 || !w2 || !w13t_q || !w13t_s || !w2t_q || !w2t_s) return MOE_ERR_INVALID_ARG;
    const moe_config_t& c = p->cfg;
    if (c.d % 128 != 0 || c.I % 128 != 0) return MOE_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // W13_e [2I, d] -> codes [d, 2I] blocked along 2I; W2_e [d, I] -> codes [I, d] blocked along d
    if (launch_mx_transpose_quant(static_cast<const uint16_t*>(w13), c.E, 2 * c.I, c.d, nullptr, nullptr, nullptr,
                                  0, true, w13t_q, w13t_s, s) != hipSuccess)
        return MOE_ERR_HIP;
    if (launch_mx_transpose_quant(static_cast<const uint16_t*>(w2), c.E, c.d, c.I, nullptr, nullptr, nullptr, 0,
                                  true, w2t_q, w2t_s, s) != hipSuccess)
        return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t moe_forward(moe_plan_t p, const void* x, const int32_t* ids, const float* scores,
                         const moe_weights_t* w, void* y, void* stream) {
    if (!p || !w) return MOE_ERR_INVALID_ARG;
    const moe_config_t& c = p->cfg;
    if (c.T > 0 && (!x || !ids || !scores || !y || !w->w13 || !w->w2)) return MOE_ERR_INVALID_ARG;
    if (c.T > 0 && c.precision == MOE_MXFP8_E4M3 && (!w->w13_scale || !w->w2_scale))
        return MOE_ERR_INVALID_ARG;
    if (!p->ws) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    p->have_saved_forward = false;
    p->status_word = p->at<int32_t>(p->off_status);
    if (c.T == 0) {
        p->have_saved_forward = c.training != 0;
        return MOE_OK;
    }
    if (p->decode) {
        DecodeArgs dg{};
        dg.T = c.T; dg.d = c.d; dg.I = c.I; dg.E = c.E; dg.k = c.k;
        dg.act = c.activation;
        dg.ids = ids; dg.scores = scores;
        dg.x = static_cast<const uint16_t*>(x);
        dg.w13 = static_cast<const uint16_t*>(w->w13);
        dg.w2 = static_cast<const uint16_t*>(w->w2);
        dg.a = p->at<uint16_t>(p->off_a);
        dg.o = p->at<uint16_t>(p->off_o);
        dg.y = static_cast<uint16_t*>(y);
        dg.status = p->at<int32_t>(p->off_status);
        if (c.mega) {
            hipError_t e = staged(p, MOE_STAGE_MEGA, s, [&] {
                return launch_mega_decode(dg, p->at<float>(p->off_mega), p->num_cu, s);
            });
            return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
        }
        hipError_t e = staged(p, MOE_STAGE_DECODE_W13, s, [&] { return launch_decode_w13(dg, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        if (c.T == 1) {
            e = staged(p, MOE_STAGE_DECODE_W2, s, [&] { return launch_decode_w2_one(dg, p->num_cu, s); });
            return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
        }
        e = staged(p, MOE_STAGE_DECODE_W2, s, [&] { return launch_decode_w2(dg, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_COMBINE, s, [&] {
            return launch_combine(dg.o, nullptr, scores, c.T, c.k, c.d, dg.y, s);
        });
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    int32_t* m_indptr = p->at<int32_t>(p->off_m_indptr);
    int32_t* gather = p->at<int32_t>(p->off_gather);
    int32_t* slots = p->at<int32_t>(p->off_slots);
    float* probs = p->at<float>(p->off_probs);
    hipError_t e = staged(p, MOE_STAGE_DISPATCH, s, [&] {
        return launch_dispatch(ids, scores, c.T, c.k, c.E, m_indptr,
                               gather, slots, probs, p->at<int32_t>(p->off_status), s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;

    if (c.precision == MOE_MXFP8_E4M3) {
        // MXFP8 (blog post "What it is selling": activations quantized after routing,
        // prepared weights): x is quantized per token row, which equals quantizing the
        // gathered rows since every MX block lies inside one row; the scales are then
        // copied out per routed row, block-major, so that a W13 tile's scale words for one
        // K group are contiguous
        uint8_t* xq = p->at<uint8_t>(p->off_xq);
        uint8_t* xs = p->at<uint8_t>(p->off_xs);
        uint8_t* xsr = p->at<uint8_t>(p->off_xsr);
        e = staged(p, MOE_STAGE_QUANT_X, s, [&] {
            hipError_t qe = launch_quantize_mxfp8(static_cast<const uint16_t*>(x), c.T, c.d, xq, xs, false, s);
            return qe != hipSuccess ? qe : launch_route_scales(xs, c.T, gather, p->R, c.d, xsr, s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        MxGemmArgs mg{};
        mg.T = c.T; mg.d = c.d; mg.I = c.I; mg.E = c.E; mg.k = c.k;
        mg.act = c.activation;
        mg.m_indptr = m_indptr; mg.gather = gather;
        mg.xq = xq; mg.xs = xsr;
        mg.w13q = static_cast<const uint8_t*>(w->w13); mg.w13s = w->w13_scale;
        mg.w2q = static_cast<const uint8_t*>(w->w2); mg.w2s = w->w2_scale;
        mg.aq = p->at<uint8_t>(p->off_aq); mg.as = p->at<uint8_t>(p->off_as);
        mg.o = p->at<uint16_t>(p->off_o);
        if (c.training && !c.recompute_h) {
            // kept for the backward: h for the activation backward, a for dW2
            mg.h_out = p->at<uint16_t>(p->off_h);
            mg.a_out = p->at<uint16_t>(p->off_a);
        }
        e = staged(p, MOE_STAGE_W13, s, [&] { return launch_gemm_mxfp8(MX_W13, mg, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_W2, s, [&] { return launch_gemm_mxfp8(MX_W2, mg, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_COMBINE, s, [&] {
            return launch_combine(p->at<uint16_t>(p->off_o), slots, scores, c.T, c.k, c.d,
                                  static_cast<uint16_t*>(y), s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        p->have_saved_forward = c.training != 0;
        return MOE_OK;
    }
    GemmArgs g{};
    g.T = c.T; g.d = c.d; g.I = c.I; g.E = c.E; g.k = c.k;
    g.act = c.activation;
    g.part = p->at<float>(p->off_part);
    g.split = p->at<int4>(p->off_split);
    g.nsplit = p->at<int32_t>(p->off_split + sizeof(int32_t) * 4 * (kMaxPieces / 2));
    g.m_indptr = m_indptr; g.gather = gather; g.probs = probs;
    g.x = static_cast<const uint16_t*>(x);
    g.w13 = static_cast<const uint16_t*>(w->w13);
    g.w2 = static_cast<const uint16_t*>(w->w2);
    g.out = p->at<uint16_t>(p->off_a);
    g.out_h = (c.training && !c.recompute_h) ? p->at<uint16_t>(p->off_h) : nullptr;
    e = staged(p, MOE_STAGE_W13, s, [&] { return launch_gemm(FWD_W13, g, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    g.a = p->at<uint16_t>(p->off_a);
    g.out = p->at<uint16_t>(p->off_o);
    g.out_h = nullptr;
    e = staged(p, MOE_STAGE_W2, s, [&] { return launch_gemm(FWD_W2, g, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    e = staged(p, MOE_STAGE_COMBINE, s, [&] {
        return launch_combine(p->at<uint16_t>(p->off_o), slots, scores, c.T, c.k, c.d,
                              static_cast<uint16_t*>(y), s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
    p->have_saved_forward = c.training != 0;
    return MOE_OK;
}

moe_status_t moe_forward_static(moe_plan_t p, const void* x, const int32_t* ids, const float* scores,
                                const moe_weights_t* w, void* y, void* stream) {
    if (!p || !w) return MOE_ERR_INVALID_ARG;
    if (p->cfg.training) return MOE_ERR_UNSUPPORTED;
    if (p->ws_bytes > kStaticScratchBytes) return MOE_ERR_TOO_LARGE;
    void* sp = nullptr;
    int ncu = 0;
    if (static_scratch(&sp, &ncu) != hipSuccess) return MOE_ERR_HIP;
    // the forward below runs on the static scratch in place of the bound workspace (the
    // plan is not reentrant, so swapping its workspace for the call is safe); the status
    // word is cleared first, by a kernel, since the array keeps the last call's contents
    struct Swap {
        moe_plan_s* p; char* ws; size_t size; int ncu;
        ~Swap() { p->ws = ws; p->ws_size = size; p->num_cu = ncu; }
    } restore{p, p->ws, p->ws_size, p->num_cu};
    p->ws = static_cast<char*>(sp);
    p->ws_size = kStaticScratchBytes;
    p->num_cu = ncu;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (launch_fill_i32(p->at<int32_t>(p->off_status), kStatusWords, 0, s) != hipSuccess) return MOE_ERR_HIP;
    return moe_forward(p, x, ids, scores, w, y, stream);
}

moe_status_t moe_forward_routed(moe_plan_t p, const void* x_rows, const int32_t* m_indptr,
                                const moe_weights_t* w, void* out, void* stream) {
    if (!p || !w) return MOE_ERR_INVALID_ARG;
    const moe_config_t& c = p->cfg;
    const bool mx = c.precision == MOE_MXFP8_E4M3;
    if (c.training || p->decode) return MOE_ERR_UNSUPPORTED;
    if (p->R * c.d * 2 >= (1LL << 31)) return MOE_ERR_UNSUPPORTED;   // 32-bit row offsets into x_rows
    if (c.T > 0 && (!x_rows || !m_indptr || !out || !w->w13 || !w->w2)) return MOE_ERR_INVALID_ARG;
    if (c.T > 0 && mx && (!w->w13_scale || !w->w2_scale)) return MOE_ERR_INVALID_ARG;
    if (!p->ws) return MOE_ERR_WORKSPACE;
    p->have_saved_forward = false;
    p->status_word = p->at<int32_t>(p->off_status);
    if (c.T == 0) return MOE_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t* mi = p->at<int32_t>(p->off_m_indptr);
    int32_t* gather = p->at<int32_t>(p->off_gather);
    hipError_t e = staged(p, MOE_STAGE_DISPATCH, s, [&] {
        return launch_routed_prep(m_indptr, c.E, p->R, mi, gather, p->at<int32_t>(p->off_status), s);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
    if (mx) {
        // the m_indptr[E] rows are quantized as they stand, their scales written
        // block-major over the routed rows (the layout W13 copies); the codes take the
        // `o` region, which W2 does not use here since it writes the caller's rows
        uint8_t* xq = p->at<uint8_t>(p->off_o);
        uint8_t* xsr = p->at<uint8_t>(p->off_xsr);
        e = staged(p, MOE_STAGE_QUANT_X, s, [&] {
            return launch_quantize_mxfp8(static_cast<const uint16_t*>(x_rows), p->R, c.d, xq, xsr, true, s,
                                         mi + c.E);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        MxGemmArgs mg{};
        mg.T = c.T; mg.d = c.d; mg.I = c.I; mg.E = c.E; mg.k = c.k;
        mg.act = c.activation;
        mg.m_indptr = mi; mg.gather = gather;
        mg.xq = xq; mg.xs = xsr;
        mg.w13q = static_cast<const uint8_t*>(w->w13); mg.w13s = w->w13_scale;
        mg.w2q = static_cast<const uint8_t*>(w->w2); mg.w2s = w->w2_scale;
        mg.aq = p->at<uint8_t>(p->off_aq); mg.as = p->at<uint8_t>(p->off_as);
        mg.o = static_cast<uint16_t*>(out);
        e = staged(p, MOE_STAGE_W13, s, [&] { return launch_gemm_mxfp8(MX_W13, mg, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_W2, s, [&] { return launch_gemm_mxfp8(MX_W2, mg, p->num_cu, s); });
        return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
    }
    GemmArgs g{};
    g.T = c.T; g.d = c.d; g.I = c.I; g.E = c.E; g.k = c.k;
    g.act = c.activation;
    g.part = p->at<float>(p->off_part);
    g.split = p->at<int4>(p->off_split);
    g.nsplit = p->at<int32_t>(p->off_split + sizeof(int32_t) * 4 * (kMaxPieces / 2));
    g.m_indptr = mi; g.gather = gather;
    g.x = static_cast<const uint16_t*>(x_rows);
    g.w13 = static_cast<const uint16_t*>(w->w13);
    g.w2 = static_cast<const uint16_t*>(w->w2);
    g.out = p->at<uint16_t>(p->off_a);
    e = staged(p, MOE_STAGE_W13, s, [&] { return launch_gemm(FWD_W13, g, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    g.a = p->at<uint16_t>(p->off_a);
    g.out = static_cast<uint16_t*>(out);
    e = staged(p, MOE_STAGE_W2, s, [&] { return launch_gemm(FWD_W2, g, p->num_cu, s); });
    return e == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

moe_status_t moe_backward(moe_plan_t p, const void* dy, const void* x, const moe_weights_t* w,
                          void* dx, void* dw13, void* dw2, float* dscores, void* stream) {
    if (!p || !w) return MOE_ERR_INVALID_ARG;
    const moe_config_t& c = p->cfg;
    if (!c.training) return MOE_ERR_STATE;
    const bool mx = c.precision == MOE_MXFP8_E4M3;
    if (!dw13 || !dw2) return MOE_ERR_INVALID_ARG;
    if (!mx && (!w->w13 || !w->w2)) return MOE_ERR_INVALID_ARG;
    if (mx && (!w->w13t || !w->w13t_scale || !w->w2t || !w->w2t_scale)) return MOE_ERR_INVALID_ARG;
    if (mx && c.recompute_h && c.T > 0 && (!w->w13 || !w->w13_scale)) return MOE_ERR_INVALID_ARG;
    if (c.T > 0 && (!dy || !x || !dx || !dscores)) return MOE_ERR_INVALID_ARG;
    if (!p->ws) return MOE_ERR_WORKSPACE;
    if (!p->have_saved_forward) return MOE_ERR_STATE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (mx) return mx_backward(p, dy, x, w, dx, dw13, dw2, dscores, s);
    hipError_t e;
    const int32_t* slots = p->at<int32_t>(p->off_slots);
    // The router gradient: partial dot products from the W2 data-gradient product's
    // epilogue (one per routed row and 64 columns of I), held in the split-tile buffer,
    // which the weight gradients use only afterwards, and summed right after that
    // product; else (more partials than the buffer holds) from o and dy.
    const int ds_slots = router_grad_slots(c.I);
    const bool fused_ds = fused_router_grad(p->R, c.I);
    if (c.T > 0 && !fused_ds) {
        e = staged(p, MOE_STAGE_SCORE_GRAD, s, [&] {
            return launch_score_grad(static_cast<const uint16_t*>(dy), p->at<uint16_t>(p->off_o),
                                     slots, c.T, c.k, c.d, dscores, s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    GemmArgs g{};
    g.T = c.T; g.d = c.d; g.I = c.I; g.E = c.E; g.k = c.k;
    g.act = c.activation;
    g.part = p->at<float>(p->off_part);
    g.split = p->at<int4>(p->off_split);
    g.nsplit = p->at<int32_t>(p->off_split + sizeof(int32_t) * 4 * (kMaxPieces / 2));
    g.m_indptr = p->at<int32_t>(p->off_m_indptr);
    g.gather = p->at<int32_t>(p->off_gather);
    g.probs = p->at<float>(p->off_probs);
    g.x = static_cast<const uint16_t*>(x);
    g.w13 = static_cast<const uint16_t*>(w->w13);
    g.w2 = static_cast<const uint16_t*>(w->w2);
    g.a = p->at<uint16_t>(p->off_a);
    g.h = p->at<uint16_t>(p->off_h);
    g.dy = static_cast<const uint16_t*>(dy);
    g.dh = p->at<uint16_t>(p->off_dh);
    g.accumulate = c.wgrad_accumulate;
    g.xg = p->at<uint16_t>(p->off_xg);
    g.dys = p->at<uint16_t>(p->off_dys);
    if (c.T == 0) {
        // no routed rows: every expert gradient is +0 (the weight-gradient kernels write them)
        g.m_indptr = p->at<int32_t>(p->off_m_indptr);
        if ((e = launch_dispatch(nullptr, nullptr, 0, c.k, c.E,
                                 p->at<int32_t>(p->off_m_indptr), nullptr, nullptr, nullptr,
                                 p->at<int32_t>(p->off_status), s)) != hipSuccess)
            return MOE_ERR_HIP;
    } else {
        if (c.recompute_h) {
            // h again from x and W13 (the same kernel and inputs as the forward, so the
            // same values); a is rewritten with what it holds
            GemmArgs gr = g;
            gr.out = p->at<uint16_t>(p->off_a);
            gr.out_h = p->at<uint16_t>(p->off_h);
            e = staged(p, MOE_STAGE_RECOMPUTE_H, s, [&] { return launch_gemm(FWD_W13, gr, p->num_cu, s); });
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        // input gradients first, each consumer right after its producer, so that dh and
        // dxp are still in the memory-side cache when they are read back
        g.out = p->at<uint16_t>(p->off_dh);
        g.ds_part = fused_ds ? g.part : nullptr;
        g.ds_slots = ds_slots;
        e = staged(p, MOE_STAGE_DGRAD_W2, s, [&] { return launch_gemm(DGRAD_W2, g, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        g.ds_part = nullptr;
        if (fused_ds) {
            e = staged(p, MOE_STAGE_SCORE_GRAD, s, [&] {
                return launch_score_grad_sum(g.part, slots, (int)p->R, ds_slots, dscores, s);
            });
            if (e != hipSuccess) return MOE_ERR_HIP;
        }
        g.out = p->at<uint16_t>(p->off_dxp);
        e = staged(p, MOE_STAGE_DGRAD_W13, s, [&] { return launch_gemm(DGRAD_W13, g, p->num_cu, s); });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_DX_COMBINE, s, [&] {
            return launch_combine(p->at<uint16_t>(p->off_dxp), slots, nullptr, c.T, c.k, c.d,
                                  static_cast<uint16_t*>(dx), s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
        e = staged(p, MOE_STAGE_WGRAD_ROWS, s, [&] {
            return launch_wgrad_rows(g.x, g.dy, c.T, c.k, slots, g.gather, g.probs, c.d, p->at<uint16_t>(p->off_xg),
                                     p->at<uint16_t>(p->off_dys), s);
        });
        if (e != hipSuccess) return MOE_ERR_HIP;
    }
    g.out = static_cast<uint16_t*>(dw2);
    e = staged(p, MOE_STAGE_WGRAD_W2, s, [&] { return launch_gemm(WGRAD_W2, g, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    g.out = static_cast<uint16_t*>(dw13);
    e = staged(p, MOE_STAGE_WGRAD_W13, s, [&] { return launch_gemm(WGRAD_W13, g, p->num_cu, s); });
    if (e != hipSuccess) return MOE_ERR_HIP;
    return MOE_OK;
}

moe_status_t moe_get_status(moe_plan_t p, int32_t* device_flags, int32_t clear, void* stream) {
    if (!p || !device_flags) return MOE_ERR_INVALID_ARG;
    if (!p->status_word) return MOE_ERR_WORKSPACE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    int32_t v = 0;
    int32_t* dflag = p->status_word;
    if (hipMemcpyAsync(&v, dflag, sizeof(v), hipMemcpyDeviceToHost, s) != hipSuccess) return MOE_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    if (clear && v) {
        if (hipMemsetAsync(dflag, 0, sizeof(int32_t), s) != hipSuccess) return MOE_ERR_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return MOE_ERR_HIP;
    }
    *device_flags = v;
    return v ? MOE_ERR_ROUTING : MOE_OK;
}

moe_status_t moe_profile(moe_plan_t p, int32_t enable) {
    if (!p) return MOE_ERR_INVALID_ARG;
    p->prof_on = enable != 0;
    return MOE_OK;
}

moe_status_t moe_profile_read(moe_plan_t p, float* total_ms, int32_t* count, int32_t max_stages) {
    if (!p || max_stages < 0 || (max_stages > 0 && (!total_ms || !count))) return MOE_ERR_INVALID_ARG;
    for (int i = 0; i < max_stages; ++i) { total_ms[i] = 0.f; count[i] = 0; }
    moe_status_t st = MOE_OK;
    for (auto& r : p->recs) {
        float ms = 0.f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess)
            st = MOE_ERR_HIP;
        else if (r.stage < max_stages) { total_ms[r.stage] += ms; count[r.stage] += 1; }
        p->ev_free.push_back(r.a);
        p->ev_free.push_back(r.b);
    }
    p->recs.clear();
    return st;
}

const char* moe_status_string(moe_status_t st) {
    switch (st) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID_ARG: return "invalid argument";
        case MOE_ERR_UNSUPPORTED: return "unsupported shape or mode";
        case MOE_ERR_WORKSPACE: return "workspace missing or too small";
        case MOE_ERR_STATE: return "invalid call order (no saved training forward)";
        case MOE_ERR_HIP: return "HIP runtime error";
        case MOE_ERR_ROUTING: return "invalid routing detected on the device";
        case MOE_ERR_TOO_LARGE: return "the plan needs more scratch than the static array holds (MOE_STATIC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

}  // extern "C"
