// A caller of the library from C++ alone: no Python and no PyTorch in the
// process.  It reads one problem from a file, sizes and allocates the workspace
// itself, runs iabn_forward_train and iabn_backward on a HIP stream of its own,
// checks the workspace's exchange status, and writes every output to a file.
// The GPU test tests/test_c_caller.py writes the problem and checks the outputs.
//
// Problem file (little-endian):
//   8 bytes "IABNCALL"; int64 N, C, H, W; int32 layout, dtype, act;
//   float act_param, eps, momentum;
//   x, then dy: N*C*H*W elements of the storage dtype, in the layout's order;
//   gamma, beta, running_mean, running_var: C floats each.
// Output file: y, dx (storage dtype, same order); save_mean, save_invstd,
//   running_mean, running_var, dgamma, dbeta (C floats each); int32 timed_out.
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "iabn.h"

namespace {

bool hip_ok(hipError_t e, const char* what)
{
    if (e == hipSuccess) return true;
    fprintf(stderr, "c_caller: %s: %s\n", what, hipGetErrorString(e));
    return false;
}

bool iabn_ok(iabn_status s, const char* what)
{
    if (s == IABN_OK) return true;
    fprintf(stderr, "c_caller: %s: %s\n", what, iabn_status_string(s));
    return false;
}

template <typename T>
bool read_all(FILE* f, T* p, size_t n)
{
    return fread(p, sizeof(T), n, f) == n;
}

template <typename T>
bool write_all(FILE* f, const T* p, size_t n)
{
    return fwrite(p, sizeof(T), n, f) == n;
}

struct DeviceBuffer {
    void* p = nullptr;
    ~DeviceBuffer() { if (p) (void)hipFree(p); }
};

}  // namespace

int main(int argc, char** argv)
{
    if (argc != 3) {
        fprintf(stderr, "usage: c_caller problem.bin outputs.bin\n");
        return 2;
    }
    FILE* in = fopen(argv[1], "rb");
    if (!in) {
        fprintf(stderr, "c_caller: cannot open %s\n", argv[1]);
        return 2;
    }
    char magic[8];
    int64_t shape[4];
    int32_t codes[3];
    float params[3];
    if (!read_all(in, magic, 8) || memcmp(magic, "IABNCALL", 8) != 0 || !read_all(in, shape, 4) ||
        !read_all(in, codes, 3) || !read_all(in, params, 3)) {
        fprintf(stderr, "c_caller: bad problem header\n");
        fclose(in);
        return 2;
    }
    const int64_t N = shape[0], C = shape[1], H = shape[2], W = shape[3];
    const iabn_layout layout = static_cast<iabn_layout>(codes[0]);
    const iabn_dtype dtype = static_cast<iabn_dtype>(codes[1]);
    const iabn_act act = static_cast<iabn_act>(codes[2]);
    const float act_param = params[0], eps = params[1], momentum = params[2];
    if (N <= 0 || C <= 0 || H <= 0 || W <= 0 || N * C * H * W > (int64_t(1) << 28)) {
        fprintf(stderr, "c_caller: shape out of this program's range\n");
        fclose(in);
        return 2;
    }
    const size_t esize = dtype == IABN_F32 ? 4 : 2;
    const size_t tensor_bytes = size_t(N * C * H * W) * esize;
    const size_t vec_bytes = size_t(C) * sizeof(float);
    std::vector<unsigned char> x(tensor_bytes), dy(tensor_bytes);
    std::vector<float> vecs(4 * size_t(C));
    const bool read_ok = read_all(in, x.data(), tensor_bytes) &&
                         read_all(in, dy.data(), tensor_bytes) &&
                         read_all(in, vecs.data(), vecs.size());
    fclose(in);
    if (!read_ok) {
        fprintf(stderr, "c_caller: short problem file\n");
        return 2;
    }

    const size_t ws_bytes = iabn_workspace_size(N, C, H, W, layout, dtype);
    if (ws_bytes == 0) {
        fprintf(stderr, "c_caller: iabn_workspace_size rejected the shape\n");
        return 1;
    }
    // device buffers: x (y after the forward), dy, dx, the workspace, and the
    // per-channel vectors gamma, beta, running_mean, running_var, save_mean,
    // save_invstd, dgamma, dbeta
    DeviceBuffer dx_, dy_, ddx, dws, dvec;
    if (!hip_ok(hipMalloc(&dx_.p, tensor_bytes), "hipMalloc x") ||
        !hip_ok(hipMalloc(&dy_.p, tensor_bytes), "hipMalloc dy") ||
        !hip_ok(hipMalloc(&ddx.p, tensor_bytes), "hipMalloc dx") ||
        !hip_ok(hipMalloc(&dws.p, ws_bytes), "hipMalloc workspace") ||
        !hip_ok(hipMalloc(&dvec.p, 8 * vec_bytes), "hipMalloc vectors"))
        return 1;
    float* v = static_cast<float*>(dvec.p);
    float *gamma = v, *beta = v + C, *rm = v + 2 * C, *rv = v + 3 * C;
    float *save_mean = v + 4 * C, *save_invstd = v + 5 * C, *dgamma = v + 6 * C,
          *dbeta = v + 7 * C;
    hipStream_t s = nullptr;
    if (!hip_ok(hipStreamCreate(&s), "hipStreamCreate")) return 1;
    bool ok = hip_ok(hipMemcpyAsync(dx_.p, x.data(), tensor_bytes, hipMemcpyHostToDevice, s),
                     "copy x") &&
              hip_ok(hipMemcpyAsync(dy_.p, dy.data(), tensor_bytes, hipMemcpyHostToDevice, s),
                     "copy dy") &&
              hip_ok(hipMemcpyAsync(v, vecs.data(), 4 * vec_bytes, hipMemcpyHostToDevice, s),
                     "copy vectors") &&
              hip_ok(hipStreamSynchronize(s), "sync after copies");
    ok = ok && iabn_ok(iabn_forward_train(dx_.p, N, C, H, W, layout, dtype, gamma, beta, rm, rv,
                                          save_mean, save_invstd, act, act_param, eps, momentum,
                                          dws.p, ws_bytes, s),
                       "iabn_forward_train");
    ok = ok && iabn_ok(iabn_backward(dx_.p, dy_.p, ddx.p, N, C, H, W, layout, dtype, gamma, beta,
                                     save_invstd, dgamma, dbeta, act, act_param, dws.p, ws_bytes,
                                     s),
                       "iabn_backward");
    ok = ok && hip_ok(hipStreamSynchronize(s), "sync after the library calls");
    int timed_out = 0;
    ok = ok && iabn_ok(iabn_workspace_status(dws.p, ws_bytes, 1, &timed_out, s),
                       "iabn_workspace_status");
    std::vector<unsigned char> y(tensor_bytes), dx(tensor_bytes);
    std::vector<float> outv(6 * size_t(C));
    ok = ok && hip_ok(hipMemcpy(y.data(), dx_.p, tensor_bytes, hipMemcpyDeviceToHost), "copy y") &&
         hip_ok(hipMemcpy(dx.data(), ddx.p, tensor_bytes, hipMemcpyDeviceToHost), "copy dx") &&
         hip_ok(hipMemcpy(outv.data(), v + 4 * C, 4 * vec_bytes, hipMemcpyDeviceToHost),
                "copy statistics and gradients") &&
         hip_ok(hipMemcpy(outv.data() + 4 * C, rm, 2 * vec_bytes, hipMemcpyDeviceToHost),
                "copy running statistics");
    (void)hipStreamDestroy(s);
    if (!ok) return 1;
    // outputs in file order: save_mean, save_invstd, running_mean, running_var,
    // dgamma, dbeta
    const float* sm_h = outv.data();
    const float* si_h = outv.data() + C;
    const float* dg_h = outv.data() + 2 * C;
    const float* db_h = outv.data() + 3 * C;
    const float* rm_h = outv.data() + 4 * C;
    const float* rv_h = outv.data() + 5 * C;
    FILE* out = fopen(argv[2], "wb");
    if (!out) {
        fprintf(stderr, "c_caller: cannot open %s\n", argv[2]);
        return 2;
    }
    const int32_t t32 = timed_out;
    const bool wrote = write_all(out, y.data(), tensor_bytes) &&
                       write_all(out, dx.data(), tensor_bytes) && write_all(out, sm_h, size_t(C)) &&
                       write_all(out, si_h, size_t(C)) && write_all(out, rm_h, size_t(C)) &&
                       write_all(out, rv_h, size_t(C)) && write_all(out, dg_h, size_t(C)) &&
                       write_all(out, db_h, size_t(C)) && write_all(out, &t32, 1);
    fclose(out);
    if (!wrote) {
        fprintf(stderr, "c_caller: short write\n");
        return 1;
    }
    char plan[256];
    if (iabn_describe_plan(N, C, H, W, layout, dtype, act, 1, plan, sizeof plan) < 0)
        strcpy(plan, "?");
    printf("c_caller: ok, workspace %zu bytes, %s\n", ws_bytes, plan);
    return 0;
}
