// Host-side checks of the C ABI layer, built with AddressSanitizer on its
// host code (the ABI layer's translation unit instrumented, the kernels'
// objects as the library builds them) and run without a GPU: every call here
// is rejected, or is a no-op, before anything reaches the HIP runtime, so the
// validation, the workspace arithmetic and the error-detail formatting run
// under the sanitizer's bounds checks. Exit status 0 when every expectation
// holds; a sanitizer report ends the process with a nonzero status.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "moe.h"
#include "moe_calib.h"

namespace {

int g_checks = 0, g_failed = 0;

void expect(moe_status got, moe_status want, const char* what, int line) {
    ++g_checks;
    if (got != want) {
        ++g_failed;
        std::fprintf(stderr, "line %d: %s returned %d (%s), expected %d; detail: %s\n", line, what, (int)got,
                     moe_status_string(got), (int)want, moe_last_error_detail());
    }
}

void expect_true(bool ok, const char* what, int line) {
    ++g_checks;
    if (!ok) {
        ++g_failed;
        std::fprintf(stderr, "line %d: %s is false\n", line, what);
    }
}

#define EXPECT(call, want) expect((call), (want), #call, __LINE__)
#define EXPECT_TRUE(cond) expect_true((cond), #cond, __LINE__)

// An aligned address that no call here dereferences (every call below is
// rejected on the host, or has nothing to do, before any device access).
void* const kFake = reinterpret_cast<void*>(uintptr_t(0x10000));
const float* fake_f() { return static_cast<const float*>(kFake); }
float* fake_fw() { return static_cast<float*>(kFake); }
int32_t* fake_i() { return static_cast<int32_t*>(kFake); }

moe_router_params params(int E = 8, int k = 2) {
    moe_router_params p;
    std::memset(&p, 0, sizeof(p));
    p.n_experts = E;
    p.top_k = k;
    p.mode = MOE_ROUTER_SOFTMAX_TOPK;
    p.renormalize = 1;
    p.n_group = 1;
    p.topk_group = 1;
    p.routed_scaling_factor = 1.0f;
    return p;
}

moe_experts experts(int E = 8, int d = 64, int I = 128, int fmt = MOE_W_INT8_G32) {
    moe_experts e;
    e.n_experts = E;
    e.d_model = d;
    e.d_ff = I;
    e.format = fmt;
    e.gate_q = e.up_q = e.down_q = kFake;
    e.gate_s = e.up_s = e.down_s = fake_f();
    return e;
}

moe_status fwd(int T, const moe_router_params& p, const moe_experts& r, const moe_experts* sh, int act,
               size_t ws_bytes = size_t(1) << 30, const float* x = fake_f(), void* ws = kFake) {
    return moe_layer_forward(x, T, fake_f(), &p, &r, sh, act, fake_fw(), ws, ws_bytes, nullptr);
}

void layer_validation() {
    const moe_router_params p = params();
    const moe_experts r = experts();
    EXPECT(fwd(0, p, r, nullptr, MOE_ACT_F32), MOE_OK);
    EXPECT(fwd(-1, p, r, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    EXPECT(fwd(4, p, r, nullptr, MOE_ACT_F32, size_t(1) << 30, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(fwd(4, p, r, nullptr, 5), MOE_ERR_INVALID_ARG);
    moe_router_params q = params(8, 9);
    EXPECT(fwd(4, q, r, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);   // k > E
    q = params(7, 2);
    EXPECT(fwd(4, q, r, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);   // router E != experts E
    q = params();
    q.mode = 3;
    EXPECT(fwd(4, q, r, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    q = params();
    q.top_p = std::numeric_limits<float>::quiet_NaN();
    EXPECT(fwd(4, q, r, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    EXPECT(fwd(4, p, experts(8, 65), nullptr, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);
    EXPECT(fwd(4, p, experts(8, 96), nullptr, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);
    EXPECT(fwd(4, p, experts(8, 64, 100), nullptr, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);
    EXPECT(fwd(4, p, experts(8, 64, 128, 9), nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    EXPECT(fwd(4, p, experts(8, 64, 128, MOE_W_INT2_G32), nullptr, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);
    EXPECT(fwd(0, p, experts(8, 128, 256, MOE_W_INT2_G32), nullptr, MOE_ACT_F32), MOE_OK);
    EXPECT(fwd(4, p, experts(8, 16384, 128), nullptr, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);   // GEMV K limit
    EXPECT(fwd(4, p, experts(8, 16384, 128), nullptr, MOE_ACT_Q8_0), MOE_ERR_UNSUPPORTED);  // T <= 16: GEMV
    const moe_experts sh_fmt = experts(1, 64, 128, MOE_W_INT4_G32);
    EXPECT(fwd(4, p, r, &sh_fmt, MOE_ACT_F32), MOE_ERR_UNSUPPORTED);
    const moe_experts sh2 = experts(2);
    EXPECT(fwd(4, p, r, &sh2, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    const moe_experts sh1 = experts(1);
    q = params();
    q.shared_gate = reinterpret_cast<const float*>(uintptr_t(0x10004));
    EXPECT(fwd(4, q, r, &sh1, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    moe_experts mis = experts();
    mis.gate_q = reinterpret_cast<const void*>(uintptr_t(0x10004));
    EXPECT(fwd(4, p, mis, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    moe_experts nul = experts();
    nul.up_s = nullptr;
    EXPECT(fwd(4, p, nul, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    EXPECT(fwd(4, p, r, nullptr, MOE_ACT_F32, 16), MOE_ERR_WORKSPACE);
    EXPECT(fwd(4, p, r, nullptr, MOE_ACT_F32, size_t(1) << 30, fake_f(), nullptr), MOE_ERR_WORKSPACE);
    EXPECT_TRUE(std::strstr(moe_last_error_detail(), "workspace") != nullptr);
    // noaux_tc group rules
    moe_router_params n = params(16, 3);
    n.mode = MOE_ROUTER_SIGMOID_NOAUX_TC;
    n.n_group = 4;
    n.topk_group = 2;
    n.routed_scaling_factor = 2.5f;
    const moe_experts r16 = experts(16);
    EXPECT(fwd(0, n, r16, nullptr, MOE_ACT_F32), MOE_OK);
    moe_router_params nb = n;
    nb.n_group = 5;
    EXPECT(fwd(0, nb, r16, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    nb = n;
    nb.topk_group = 5;
    EXPECT(fwd(0, nb, r16, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    nb = n;
    nb.top_k = 9;
    EXPECT(fwd(0, nb, r16, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
    nb = n;
    nb.routed_scaling_factor = std::numeric_limits<float>::infinity();
    EXPECT(fwd(0, nb, r16, nullptr, MOE_ACT_F32), MOE_ERR_INVALID_ARG);
}

void block_and_noalloc_validation() {
    const moe_router_params p = params();
    const moe_experts r = experts();
    auto blk = [&](float eps, const float* norm, const float* x) {
        return moe_block_forward(x, 4, norm, eps, fake_f(), &p, &r, nullptr, MOE_ACT_F32, fake_fw(), kFake,
                                 size_t(1) << 30, nullptr, nullptr);
    };
    EXPECT(blk(-1.0f, fake_f(), fake_f()), MOE_ERR_INVALID_ARG);
    EXPECT(blk(std::numeric_limits<float>::quiet_NaN(), fake_f(), fake_f()), MOE_ERR_INVALID_ARG);
    EXPECT(blk(1e-6f, fake_f(), nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(blk(1e-6f, reinterpret_cast<const float*>(uintptr_t(0x10004)), fake_f()), MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_forward_noalloc(fake_f(), 4, fake_f(), nullptr, &r, nullptr, 0, fake_fw(), nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_layer_forward_noalloc(fake_f(), -1, fake_f(), &p, &r, nullptr, 0, fake_fw(), nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT_TRUE(moe_workspace_size(200000, 2, 8, 64, 128, 0, 0) > MOE_NOALLOC_SCRATCH_BYTES);
    EXPECT(moe_layer_forward_noalloc(fake_f(), 200000, fake_f(), &p, &r, nullptr, 0, fake_fw(), nullptr),
           MOE_ERR_UNSUPPORTED);
    EXPECT_TRUE(std::strstr(moe_last_error_detail(), "scratch") != nullptr);
}

void piece_validation() {
    moe_router_params p = params();
    EXPECT(moe_route(fake_f(), 0, 64, fake_f(), &p, fake_i(), fake_fw(), kFake, 0, nullptr), MOE_OK);
    EXPECT(moe_route(fake_f(), 4, 64, fake_f(), nullptr, fake_i(), fake_fw(), kFake, 1 << 20, nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_route(fake_f(), 4, 64, fake_f(), &p, fake_i(), fake_fw(), kFake, 8, nullptr), MOE_ERR_WORKSPACE);
    moe_router_params big = params(2000, 2);
    EXPECT(moe_route(fake_f(), 4, 64, fake_f(), &big, fake_i(), fake_fw(), kFake, size_t(1) << 30, nullptr),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch(fake_i(), 4, 3, 2, fake_i(), fake_i(), fake_i(), fake_i(), nullptr, 0, nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_dispatch(fake_i(), 4, 2, 2000, fake_i(), fake_i(), fake_i(), fake_i(), nullptr, 0, nullptr),
           MOE_ERR_UNSUPPORTED);
    EXPECT(moe_dispatch(fake_i(), 4, 2, 8, nullptr, fake_i(), fake_i(), fake_i(), nullptr, 0, nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_combine(fake_f(), fake_f(), fake_i(), nullptr, 0, 2, 64, fake_fw(), nullptr), MOE_OK);
    EXPECT(moe_combine(fake_f(), fake_f(), fake_i(), nullptr, 4, 2, 66, fake_fw(), nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_combine(nullptr, fake_f(), fake_i(), nullptr, 4, 2, 64, fake_fw(), nullptr), MOE_ERR_INVALID_ARG);
    int8_t* q = static_cast<int8_t*>(kFake);
    EXPECT(moe_quantize_weights(fake_f(), 32, 48, 32, 0, kFake, fake_fw(), nullptr), MOE_ERR_UNSUPPORTED);
    EXPECT(moe_quantize_weights(fake_f(), 96, 64, 64, 0, kFake, fake_fw(), nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_quantize_weights(fake_f(), 32, 64, 32, 6, kFake, fake_fw(), nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_quantize_weights(fake_f(), 32, 64, 32, -1, kFake, fake_fw(), nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_quantize_weights(fake_f(), 0, 128, 32, 5, kFake, fake_fw(), nullptr), MOE_OK);
    EXPECT(moe_quantize_q8_0(fake_f(), 4, 40, q, fake_fw(), nullptr), MOE_ERR_UNSUPPORTED);
    const moe_experts e = experts();
    EXPECT(moe_expert_ffn(fake_f(), 4, 9, &e, fake_i(), fake_i(), fake_i(), 0, fake_fw(), kFake, size_t(1) << 30,
                          nullptr),
           MOE_ERR_INVALID_ARG);
    EXPECT(moe_expert_ffn(fake_f(), 4, 2, &e, fake_i(), fake_i(), fake_i(), 0, fake_fw(), kFake, 64, nullptr),
           MOE_ERR_WORKSPACE);
    EXPECT(moe_debug_q8_expert_ffn(fake_f(), 4, 2, &e, fake_i(), fake_i(), fake_i(), nullptr, fake_i(), q, fake_fw(),
                                   fake_i(), fake_fw(), kFake, size_t(1) << 30, nullptr),
           MOE_ERR_INVALID_ARG);
    uint32_t* sink = static_cast<uint32_t*>(kFake);
    EXPECT(moe_calib_stream_read(nullptr, 1 << 20, sink, 64, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_calib_stream_read(kFake, 1000, sink, 64, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_calib_prefill_mix(16, 7, fake_fw(), nullptr, nullptr), MOE_ERR_INVALID_ARG);
    EXPECT(moe_calib_prefill_mix(0, 8, fake_fw(), nullptr, nullptr), MOE_ERR_INVALID_ARG);
}

// Workspace sizes and the test hook's sections over a sweep of shapes, from
// one token to long prefills and from 1 to 1024 experts: every section is
// 256-byte aligned and ends inside the workspace.
void workspace_sweep() {
    const int Ts[] = {0, 1, 4, 16, 17, 600, 2048, 4096, 65536};
    const int Es[] = {1, 8, 64, 256, 512, 1024};
    const int ks[] = {1, 2, 8, 10, 64};
    const int ds[] = {64, 2048, 6144, 8192};
    for (int T : Ts)
        for (int E : Es)
            for (int k : ks)
                for (int d : ds)
                    for (int act = 0; act < 2; ++act)
                        for (int sh = 0; sh < 2; ++sh) {
                            const int I = d == 64 ? 128 : 1024;
                            const size_t total = moe_workspace_size(T, k, E, d, I, act, sh);
                            int64_t off[MOE_WS_SECTION_COUNT];
                            const moe_status s = moe_debug_workspace_sections(T, k, E, d, I, act, sh, off);
                            if (k > E) {
                                EXPECT_TRUE(total == 0);
                                EXPECT(s, MOE_ERR_INVALID_ARG);
                                continue;
                            }
                            EXPECT_TRUE(total > 0);
                            EXPECT(s, MOE_OK);
                            for (int i = 0; i < MOE_WS_SECTION_COUNT; ++i) {
                                if (off[i] < 0) continue;
                                EXPECT_TRUE(off[i] % 256 == 0 && (size_t)off[i] < total);
                            }
                        }
    EXPECT_TRUE(moe_workspace_size(-1, 2, 8, 64, 128, 0, 0) == 0);
    EXPECT_TRUE(moe_workspace_size(16, 2, 8, 65, 128, 0, 0) == 0);
    EXPECT_TRUE(moe_workspace_size(16, 2, 8, 64, 128, 7, 0) == 0);
}

void status_strings() {
    EXPECT_TRUE(std::strcmp(moe_status_string(MOE_OK), "MOE_OK") == 0);
    for (int st = -8; st < 0; ++st) EXPECT_TRUE(std::strlen(moe_status_string((moe_status)st)) > 0);
    EXPECT_TRUE(std::strlen(moe_status_string((moe_status)12345)) > 0);
}

}  // namespace

int main() {
    layer_validation();
    block_and_noalloc_validation();
    piece_validation();
    workspace_sweep();
    status_strings();
    std::printf("host ABI checks: %d of %d passed\n", g_checks - g_failed, g_checks);
    return g_failed == 0 ? 0 : 1;
}
