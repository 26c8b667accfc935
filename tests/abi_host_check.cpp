// Host run of the C ABI's own code (place_batchnorm_activation_amd/csrc/api.cpp:
// validation, planning, dispatch, the plan descriptions and the workspace status
// query), built with AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).
//
// The kernels' launchers are replaced by stubs that record which one a call would
// launch, and the few HIP runtime calls api.cpp makes by stand-ins: a device of
// 256 CUs, launches that always succeed, and copies and fills on host memory (the
// "device" buffers here are host buffers that no kernel ever touches).  Exit
// status 0 when every check holds.
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "fused.hpp"
#include "iabn.h"
#include "launch.hpp"
#include "plan.hpp"

static int failures = 0;
#define CHECK(cond, ...)                                                   \
    do {                                                                   \
        if (!(cond)) {                                                     \
            ++failures;                                                    \
            std::printf("FAIL %s:%d: ", __FILE__, __LINE__);               \
            std::printf(__VA_ARGS__);                                      \
            std::printf("\n");                                             \
        }                                                                  \
    } while (0)

// ---------------------------------------------------------------------------
// stand-ins for the HIP runtime calls of api.cpp

extern "C" {
hipError_t hipGetDevice(int* dev)
{
    *dev = 0;
    return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int)
{
    *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 0;
    return hipSuccess;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t n, hipMemcpyKind, hipStream_t)
{
    std::memcpy(dst, src, n);
    return hipSuccess;
}
hipError_t hipMemsetAsync(void* dst, int v, size_t n, hipStream_t)
{
    std::memset(dst, v, n);
    return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
}

// ---------------------------------------------------------------------------
// launcher stubs: the names of the launchers a call used, in order

static std::string g_launched;
static void note(const char* what, const iabn::Plan& pl)
{
    if (!g_launched.empty()) g_launched += ",";
    g_launched += what;
    // every plan a launcher gets must be self-consistent
    CHECK(pl.numel == pl.m * pl.C && pl.bytes >= iabn::kWsHeaderBytes, "%s: plan sizes", what);
}

namespace iabn {
#define STUB(name, ...)                                                    \
    void name(const Plan& pl, __VA_ARGS__) { note(#name, pl); }
STUB(launch_forward_stats, const void*, const float*, const float*, float*, float*, float*,
     float*, float, float, void*, hipStream_t)
STUB(launch_forward_apply, void*, int, float, void*, hipStream_t)
STUB(launch_forward_eval, void*, const float*, const float*, const float*, const float*, float,
     int, float, hipStream_t)
STUB(launch_backward_reduce, const void*, const void*, const float*, const float*, const float*,
     float*, float*, int, float, void*, hipStream_t)
STUB(launch_backward_eval_grads, const void*, const void*, void*, const float*, const float*,
     const float*, float, float*, float*, int, float, void*, hipStream_t)
STUB(launch_eval_consts, const float*, const float*, const float*, float, void*, hipStream_t)
STUB(launch_backward_apply, const void*, const void*, void*, int, float, void*, hipStream_t)
STUB(launch_backward_reduce_xhat, const void*, const void*, const float*, const float*,
     const float*, float*, float*, int, float, void*, hipStream_t)
STUB(launch_ckpt_forward_apply, void*, void*, const float*, const float*, const float*, int,
     float, void*, hipStream_t)
STUB(launch_ckpt_recompute, const void*, void*, const float*, const float*, int, float,
     hipStream_t)
STUB(launch_ckpt_dx, const void*, const void*, void*, const float*, const float*, int, float,
     void*, hipStream_t)
STUB(launch_forward_fused_nchw, void*, const float*, const float*, float*, float*, float*,
     float*, float, float, int, float, void*, hipStream_t)
STUB(launch_backward_fused_nchw, const void*, const void*, void*, const float*, const float*,
     const float*, float*, float*, int, float, void*, hipStream_t)
STUB(launch_forward_fused_scalar, void*, const float*, const float*, float*, float*, float*,
     float*, float, float, int, float, hipStream_t)
STUB(launch_backward_fused_scalar, const void*, const void*, void*, const float*, const float*,
     const float*, float*, float*, int, float, hipStream_t)
STUB(launch_forward_fused_nhwc, void*, const float*, const float*, float*, float*, float*,
     float*, float, float, int, float, void*, hipStream_t)
STUB(launch_backward_fused_nhwc, const void*, const void*, void*, const float*, const float*,
     const float*, float*, float*, int, float, void*, hipStream_t)
STUB(launch_forward_stream_nhwc, void*, const float*, const float*, float*, float*, float*,
     float*, float, float, int, float, void*, hipStream_t)
STUB(launch_backward_stream_nhwc, const void*, const void*, void*, const float*, const float*,
     const float*, float*, float*, int, float, void*, hipStream_t)
#undef STUB
}  // namespace iabn

// ---------------------------------------------------------------------------

struct Shape {
    int64_t N, C, H, W;
    iabn_layout layout;
    iabn_dtype dtype;
};

// Fake device addresses: 256-aligned, far apart; never dereferenced (the stubs
// launch nothing).
static char* fake(int k) { return reinterpret_cast<char*>(uintptr_t(1) << 40) + (uintptr_t(k) << 36); }

static void run_shape(const Shape& s)
{
    const size_t ws = iabn_workspace_size(s.N, s.C, s.H, s.W, s.layout, s.dtype);
    const int64_t numel = s.N * s.C * s.H * s.W;
    CHECK(numel == 0 ? ws == 0 : ws >= iabn::kWsHeaderBytes, "workspace size %zu", ws);
    float* v = reinterpret_cast<float*>(fake(1));
    for (int act = 0; act < 3; ++act) {
        const float a = act == 0 ? 0.f : 0.5f;
        for (int shift = 0; shift < 2; ++shift) {
            // shift: tensors one element off 16-byte alignment (the scalar plans)
            const size_t es = s.dtype == IABN_F32 ? 4 : 2;
            char* x = fake(2) + shift * es;
            char* dy = fake(3) + shift * es;
            char* dx = fake(4) + shift * es;
            char* y = fake(5) + shift * es;
            char buf[256];
            const int n = iabn_describe_plan(s.N, s.C, s.H, s.W, s.layout, s.dtype, iabn_act(act),
                                             !shift, buf, sizeof buf);
            CHECK(n > 0 && size_t(n) < sizeof buf, "describe_plan length %d", n);
            // truncation: snprintf semantics on small buffers
            char small[8];
            std::memset(small, 'x', sizeof small);
            const int n2 = iabn_describe_plan(s.N, s.C, s.H, s.W, s.layout, s.dtype,
                                              iabn_act(act), !shift, small, 5);
            CHECK(n2 == n && small[4] == '\0' && small[5] == 'x', "describe_plan truncation");
            CHECK(iabn_describe_plan(s.N, s.C, s.H, s.W, s.layout, s.dtype, iabn_act(act), !shift,
                                     nullptr, 0) == n, "describe_plan length query");

            g_launched.clear();
            iabn_status st = iabn_forward_train(x, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v,
                                                v, v, v, iabn_act(act), a, 1e-5f, 0.1f, fake(6),
                                                ws, nullptr);
            const bool m_ok = s.N * s.H * s.W >= 2 || s.C == 0;
            CHECK(st == (m_ok ? IABN_OK : IABN_ERR_INVALID_ARG), "forward_train status %d", st);
            if (m_ok && s.C > 0) {
                CHECK(!g_launched.empty(), "forward_train launched nothing");
                // the description names the family the call launched
                const std::string d(buf);
                const bool split = d.find("forward=split") == 0;
                CHECK(split == (g_launched.find("launch_forward_stats") == 0),
                      "forward: plan '%s' but launched '%s'", buf, g_launched.c_str());
            }
            g_launched.clear();
            st = iabn_backward(y, dy, dx, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v, v,
                               iabn_act(act), a, fake(6), ws, nullptr);
            CHECK(st == (m_ok ? IABN_OK : IABN_ERR_INVALID_ARG), "backward status %d", st);
            st = iabn_backward(y, dy, dy, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v, v,
                               iabn_act(act), a, fake(6), ws, nullptr);
            CHECK(st == (m_ok ? IABN_OK : IABN_ERR_INVALID_ARG), "backward dx=dy status %d", st);
            if (ws > 0) {
                st = iabn_forward_train(x, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v, v,
                                        v, iabn_act(act), a, 1e-5f, 0.1f, fake(6), ws - 1,
                                        nullptr);
                // the size covers every plan of the shape; one byte short fails at
                // least the plan that needs it all, and never passes an invalid call
                CHECK(m_ok ? (st == IABN_OK || st == IABN_ERR_WORKSPACE)
                           : st == IABN_ERR_INVALID_ARG, "short workspace %d", st);
            }
            st = iabn_forward_eval(x, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v,
                                   iabn_act(act), a, 1e-5f, nullptr);
            CHECK(st == IABN_OK, "forward_eval status %d", st);
            st = iabn_backward_eval(y, dy, dx, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v,
                                    1e-5f, v, v, iabn_act(act), a, fake(6), ws, nullptr);
            CHECK(st == (s.N * s.H * s.W >= 1 || s.C == 0 ? IABN_OK : IABN_ERR_INVALID_ARG),
                  "backward_eval status %d", st);
            st = iabn_forward_train_ckpt(x, y, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v,
                                         v, v, iabn_act(act), a, 1e-5f, 0.1f, fake(6), ws,
                                         nullptr);
            CHECK(st == (m_ok ? IABN_OK : IABN_ERR_INVALID_ARG), "forward_train_ckpt %d", st);
            st = iabn_recompute_from_xhat(x, y, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v,
                                          iabn_act(act), a, nullptr);
            CHECK(st == IABN_OK, "recompute_from_xhat %d", st);
            st = iabn_backward_ckpt(x, dy, dx, s.N, s.C, s.H, s.W, s.layout, s.dtype, v, v, v, v,
                                    v, iabn_act(act), a, fake(6), ws, nullptr);
            CHECK(st == (m_ok ? IABN_OK : IABN_ERR_INVALID_ARG), "backward_ckpt %d", st);
        }
    }
}

static void status_word()
{
    // the query on a host buffer standing in for the workspace
    std::vector<uint64_t> w(32, 0x0123456789abcdefull);
    int flag = 7;
    CHECK(iabn_workspace_status(w.data(), 256, 1, &flag, nullptr) == IABN_OK && flag == 0,
          "garbage word read as a timeout");
    CHECK(w[0] == 0x0123456789abcdefull, "a clear query must not write");
    w[0] = iabn::kExchangeTimeout;
    CHECK(iabn_workspace_status(w.data(), 256, 0, &flag, nullptr) == IABN_OK && flag == 1,
          "timeout not reported");
    CHECK(w[0] == iabn::kExchangeTimeout, "clear=0 must keep the word");
    CHECK(iabn_workspace_status(w.data(), 256, 1, &flag, nullptr) == IABN_OK && flag == 1,
          "timeout not reported (clear)");
    CHECK(w[0] == 0, "clear=1 must reset the word");
    CHECK(iabn_workspace_status(w.data(), 255, 0, &flag, nullptr) == IABN_ERR_WORKSPACE,
          "short workspace");
    CHECK(iabn_workspace_status(w.data(), 256, 0, nullptr, nullptr) == IABN_ERR_INVALID_ARG,
          "null flag");
}

int main()
{
    std::vector<Shape> shapes = {
        {2, 4, 8, 8, IABN_NCHW, IABN_F32},        {32, 256, 56, 56, IABN_NCHW, IABN_F32},
        {2, 256, 512, 512, IABN_NHWC, IABN_BF16}, {16, 512, 28, 28, IABN_NCHW, IABN_F32},
        {64, 2048, 7, 7, IABN_NHWC, IABN_BF16},   {32, 64, 112, 112, IABN_NCHW, IABN_F32},
        {32, 64, 112, 112, IABN_NHWC, IABN_BF16}, {3, 5, 17, 19, IABN_NCHW, IABN_F16},
        {2, 13, 10, 7, IABN_NHWC, IABN_F32},      {1, 1, 1, 2, IABN_NCHW, IABN_F32},
        {1, 3, 1, 1, IABN_NHWC, IABN_BF16},       {0, 5, 4, 4, IABN_NCHW, IABN_F32},
        {2, 0, 4, 4, IABN_NHWC, IABN_F32},        {8, 16, 2048, 4100, IABN_NCHW, IABN_F32},
        {1, 1 << 20, 16, 16, IABN_NHWC, IABN_BF16}, {32, 1024, 14, 14, IABN_NHWC, IABN_F16},
        {4, 2048, 56, 56, IABN_NHWC, IABN_BF16},  {1, 128, 400, 400, IABN_NHWC, IABN_F32}};
    for (int grouped = 1; grouped >= 0; --grouped) {
        iabn_set_grouped_kernels(grouped);
        for (const Shape& s : shapes) run_shape(s);
    }
    iabn_set_grouped_kernels(1);
    status_word();
    // invalid enums and sizes never plan
    char buf[64];
    CHECK(iabn_describe_plan(2, 4, 4, 4, iabn_layout(7), IABN_F32, IABN_ACT_IDENTITY, 1, buf,
                             sizeof buf) == -1, "bad layout");
    CHECK(iabn_workspace_size(-1, 4, 4, 4, IABN_NCHW, IABN_F32) == 0, "negative extent");
    CHECK(iabn_workspace_size(1 << 30, 1 << 30, 1 << 30, 1 << 30, IABN_NCHW, IABN_F32) == 0,
          "overflowing shape");
    if (failures) {
        std::printf("FAILED %d checks\n", failures);
        return 1;
    }
    std::printf("OK\n");
    return 0;
}
