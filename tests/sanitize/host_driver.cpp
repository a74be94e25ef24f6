// Host sanitizer run of the library's plan logic (tests/test_sanitize.py builds this file
// with the library's moe_api.cpp under g++ -fsanitize=address,undefined, with the kernel
// launchers replaced by stubs that fail): plan validation over valid and invalid
// configurations, workspace layout, the memory report into buffers of every size, the
// status strings and the host-side refusals of forward / backward, so that an
// out-of-bounds access, a leak or undefined behaviour in the host code stops the run.
// No device is touched: none of these calls reaches a HIP runtime function.
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "../../mixture_experts_routed_dispatch_amd/csrc/kernels.h"

namespace moe {
hipError_t launch_dispatch(const int32_t*, const float*, int, int, int, int32_t*, int32_t*, int32_t*, float*,
                           int32_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_routed_prep(const int32_t*, int, int64_t, int32_t*, int32_t*, int32_t*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_gemm(GemmMode, const GemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_gemm_mxfp8(MxMode, const MxGemmArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_combine(const uint16_t*, const int32_t*, const float*, int, int, int, uint16_t*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_score_grad_sum(const float*, const int32_t*, int, int, float*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_score_grad(const uint16_t*, const uint16_t*, const int32_t*, int, int, int, float*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_wgrad_rows(const uint16_t*, const uint16_t*, int, int, const int32_t*, const int32_t*,
                             const float*, int, uint16_t*, uint16_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_w13(const DecodeArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_w2(const DecodeArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_decode_w2_one(const DecodeArgs&, int, hipStream_t) { return hipErrorInvalidValue; }
int mega_chunk(int, int) { return 32; }
hipError_t launch_mega_decode(const DecodeArgs&, float*, int, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_quantize_mxfp8(const uint16_t*, int64_t, int, uint8_t*, uint8_t*, bool, hipStream_t,
                                 const int32_t*) { return hipErrorInvalidValue; }
hipError_t launch_route_scales(const uint8_t*, int64_t, const int32_t*, int64_t, int, uint8_t*, hipStream_t) {
    return hipErrorInvalidValue;
}
hipError_t launch_mx_scaled_rows(const uint16_t*, int, int, const int32_t*, const int32_t*, const float*, int64_t,
                                 int, uint8_t*, uint8_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mx_act_backward(const uint16_t*, const uint16_t*, int64_t, int, int, uint16_t*, uint8_t*,
                                  uint8_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_mx_transpose_quant(const uint16_t*, int, int, int, const int32_t*, const int32_t*, const float*,
                                     int, bool, uint8_t*, uint8_t*, hipStream_t) { return hipErrorInvalidValue; }
hipError_t static_scratch(void**, int*) { return hipErrorInvalidValue; }
hipError_t launch_fill_i32(int32_t*, int, int32_t, hipStream_t) { return hipErrorInvalidValue; }
}  // namespace moe

static int fails = 0;
#define CHECK(c) do { if (!(c)) { if (fails++ < 10) std::fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); } } while (0)

static moe_config_t cfg(int T, int d, int I, int E, int k) {
    moe_config_t c;
    std::memset(&c, 0, sizeof c);
    c.T = T; c.d = d; c.I = I; c.E = E; c.k = k;
    return c;
}

int main() {
    // valid plans of every kind: their workspace sizes and reports
    std::vector<moe_config_t> ok;
    ok.push_back(cfg(8192, 2048, 768, 16, 8));
    moe_config_t t = cfg(8192, 2048, 768, 128, 8); t.training = 1; ok.push_back(t);
    t.recompute_h = 1; ok.push_back(t);
    t.wgrad_accumulate = 1; t.activation = MOE_ACT_GEGLU; ok.push_back(t);
    ok.push_back(cfg(1, 2048, 768, 128, 8));
    ok.push_back(cfg(32, 2048, 768, 128, 8));
    moe_config_t m = cfg(16384, 4096, 2048, 64, 8); m.precision = MOE_MXFP8_E4M3; ok.push_back(m);
    m.training = 1; ok.push_back(m);                   // MXFP8 training, h saved
    m.recompute_h = 1; ok.push_back(m);                // h recomputed into the token-layout region
    moe_config_t m2 = cfg(300, 256, 1024, 8, 2); m2.precision = MOE_MXFP8_E4M3; m2.training = 1;
    m2.recompute_h = 1; m2.wgrad_accumulate = 1; ok.push_back(m2);   // h larger than that region
    ok.push_back(cfg(0, 256, 128, 8, 2));
    ok.push_back(cfg(4096, 256, 64, 256, 32));
    moe_config_t rc = cfg(300, 128, 256, 8, 2); rc.training = 1; rc.recompute_h = 1; ok.push_back(rc);
    moe_config_t mg = cfg(1, 2048, 768, 128, 8); mg.mega = 1; ok.push_back(mg);
    mg.T = 32; ok.push_back(mg);
    for (const moe_config_t& c : ok) {
        moe_plan_t p = nullptr;
        CHECK(moe_plan(&c, &p) == MOE_OK && p != nullptr);
        if (!p) continue;
        CHECK(moe_workspace_bytes(p) > 0 && moe_workspace_bytes(p) % 256 == 0);
        const size_t n = moe_plan_explain(p, nullptr, 0);
        CHECK(n > 0);
        for (size_t len : {size_t(1), size_t(2), size_t(17), n, n + 1, n + 100}) {
            std::string buf(len + 8, '#');
            const size_t r = moe_plan_explain(p, &buf[0], len);
            CHECK(r == n);
            const size_t w = len - 1 < n ? len - 1 : n;
            CHECK(buf[w] == '\0' && std::strlen(buf.c_str()) == w && buf[len] == '#');
        }
        CHECK(moe_profile(p, 1) == MOE_OK && moe_profile(p, 0) == MOE_OK);
        float ms[MOE_STAGE_COUNT];
        int32_t cnt[MOE_STAGE_COUNT];
        CHECK(moe_profile_read(p, ms, cnt, MOE_STAGE_COUNT) == MOE_OK);
        // no workspace bound: refused before anything is enqueued
        moe_weights_t w;
        std::memset(&w, 0, sizeof w);
        char dummy[64];
        w.w13 = dummy; w.w2 = dummy; w.w13_scale = (const uint8_t*)dummy; w.w2_scale = (const uint8_t*)dummy;
        const moe_status_t fs = moe_forward(p, dummy, (const int32_t*)dummy, (const float*)dummy, &w, dummy, nullptr);
        CHECK(fs == (c.T == 0 ? MOE_ERR_WORKSPACE : MOE_ERR_WORKSPACE));
        CHECK(moe_bind_workspace(p, nullptr, 1 << 20) == MOE_ERR_INVALID_ARG);
        CHECK(moe_bind_workspace(p, dummy + 1, 1 << 20) == MOE_ERR_INVALID_ARG);
        CHECK(moe_plan_destroy(p) == MOE_OK);
    }
    // invalid configurations are refused and allocate nothing
    struct Bad { moe_config_t c; moe_status_t want; };
    std::vector<Bad> bad;
    bad.push_back({cfg(-1, 256, 128, 8, 2), MOE_ERR_INVALID_ARG});
    bad.push_back({cfg(64, 0, 128, 8, 2), MOE_ERR_INVALID_ARG});
    bad.push_back({cfg(64, 250, 128, 8, 2), MOE_ERR_UNSUPPORTED});
    bad.push_back({cfg(64, 256, 100, 8, 2), MOE_ERR_UNSUPPORTED});
    bad.push_back({cfg(64, 256, 128, 300, 2), MOE_ERR_UNSUPPORTED});
    bad.push_back({cfg(64, 256, 128, 8, 9), MOE_ERR_UNSUPPORTED});
    bad.push_back({cfg(64, 256, 128, 64, 33), MOE_ERR_UNSUPPORTED});
    bad.push_back({cfg(131073, 256, 128, 8, 1), MOE_ERR_UNSUPPORTED});
    moe_config_t mt = cfg(64, 128, 128, 8, 2); mt.precision = MOE_MXFP8_E4M3; mt.training = 1;
    bad.push_back({mt, MOE_ERR_UNSUPPORTED});           // MXFP8 needs d % 256 == 0
    moe_config_t md = cfg(8, 256, 128, 8, 2); md.precision = MOE_MXFP8_E4M3; md.path = MOE_PATH_DECODE;
    bad.push_back({md, MOE_ERR_UNSUPPORTED});
    moe_config_t ac = cfg(64, 256, 128, 8, 2); ac.wgrad_accumulate = 1; bad.push_back({ac, MOE_ERR_UNSUPPORTED});
    moe_config_t ra = cfg(64, 256, 128, 8, 2); ra.activation = 7; bad.push_back({ra, MOE_ERR_INVALID_ARG});
    moe_config_t pa = cfg(64, 256, 128, 8, 2); pa.path = 9; bad.push_back({pa, MOE_ERR_INVALID_ARG});
    moe_config_t dp = cfg(64, 256, 128, 8, 8); dp.path = MOE_PATH_DECODE; bad.push_back({dp, MOE_ERR_UNSUPPORTED});
    moe_config_t mp = cfg(4096, 256, 128, 8, 2); mp.mega = 1; bad.push_back({mp, MOE_ERR_UNSUPPORTED});
    moe_config_t mt2 = cfg(8, 256, 128, 8, 2); mt2.mega = 1; mt2.training = 1; bad.push_back({mt2, MOE_ERR_UNSUPPORTED});
    moe_config_t mf = cfg(8, 256, 128, 8, 2); mf.mega = 1; mf.path = MOE_PATH_PREFILL; bad.push_back({mf, MOE_ERR_UNSUPPORTED});
    moe_config_t mi = cfg(8, 256, 128, 8, 2); mi.mega = 3; bad.push_back({mi, MOE_ERR_INVALID_ARG});
    for (const Bad& b : bad) {
        moe_plan_t p = reinterpret_cast<moe_plan_t>(&fails);
        CHECK(moe_plan(&b.c, &p) == b.want);
        CHECK(p == nullptr);
    }
    CHECK(moe_plan(nullptr, nullptr) == MOE_ERR_INVALID_ARG);
    CHECK(moe_workspace_bytes(nullptr) == 0 && moe_plan_explain(nullptr, nullptr, 0) == 0);
    CHECK(moe_plan_destroy(nullptr) == MOE_OK);
    for (int s = -8; s <= 1; ++s) CHECK(moe_status_string((moe_status_t)s) != nullptr);
    // the static-scratch forward refuses training plans and plans beyond its maximum
    // before it looks for the array
    {
        moe_config_t tc = cfg(64, 256, 128, 8, 2); tc.training = 1;
        moe_config_t big = cfg(65536, 2048, 768, 16, 2);
        moe_plan_t p1 = nullptr, p2 = nullptr;
        CHECK(moe_plan(&tc, &p1) == MOE_OK && moe_plan(&big, &p2) == MOE_OK);
        moe_weights_t w;
        std::memset(&w, 0, sizeof w);
        char dummy[64];
        CHECK(moe_forward_static(p1, dummy, (const int32_t*)dummy, (const float*)dummy, &w, dummy, nullptr) ==
              MOE_ERR_UNSUPPORTED);
        CHECK(moe_workspace_bytes(p2) > MOE_STATIC_SCRATCH_BYTES);
        CHECK(moe_forward_static(p2, dummy, (const int32_t*)dummy, (const float*)dummy, &w, dummy, nullptr) ==
              MOE_ERR_TOO_LARGE);
        CHECK(moe_forward_static(nullptr, dummy, nullptr, nullptr, &w, dummy, nullptr) == MOE_ERR_INVALID_ARG);
        moe_plan_destroy(p1);
        moe_plan_destroy(p2);
    }
    // the MXFP8 backward and its weight preparation refuse missing operands on the host
    {
        moe_config_t tc = cfg(64, 256, 128, 8, 2); tc.precision = MOE_MXFP8_E4M3; tc.training = 1;
        moe_config_t odd = cfg(64, 192, 128, 8, 2);
        moe_plan_t p1 = nullptr, p2 = nullptr;
        CHECK(moe_plan(&tc, &p1) == MOE_OK && moe_plan(&odd, &p2) == MOE_OK);
        moe_weights_t w;
        std::memset(&w, 0, sizeof w);
        char dummy[64];
        uint8_t* u = reinterpret_cast<uint8_t*>(dummy);
        CHECK(moe_backward(p1, dummy, dummy, &w, dummy, dummy, dummy, (float*)dummy, nullptr) == MOE_ERR_INVALID_ARG);
        w.w13t = u; w.w13t_scale = u; w.w2t = u;
        CHECK(moe_backward(p1, dummy, dummy, &w, dummy, dummy, dummy, (float*)dummy, nullptr) == MOE_ERR_INVALID_ARG);
        w.w2t_scale = u;
        CHECK(moe_backward(p1, dummy, dummy, &w, dummy, dummy, dummy, (float*)dummy, nullptr) == MOE_ERR_WORKSPACE);
        CHECK(moe_prepare_weights_backward(p1, dummy, nullptr, u, u, u, u, nullptr) == MOE_ERR_INVALID_ARG);
        CHECK(moe_prepare_weights_backward(p2, dummy, dummy, u, u, u, u, nullptr) == MOE_ERR_UNSUPPORTED);
        CHECK(moe_prepare_weights_backward(p1, dummy, dummy, u, u, u, u, nullptr) == MOE_ERR_HIP);   // stub launcher
        moe_plan_destroy(p1);
        moe_plan_destroy(p2);
    }
    if (fails) { std::fprintf(stderr, "%d checks failed\n", fails); return 1; }
    std::printf("host sanitizer run: ok\n");
    return 0;
}
