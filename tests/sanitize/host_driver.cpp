// Drives the library's host side — list validation, chunking, the workspace
// tables and every entry point's argument checks — without a GPU, so that a
// build of that code with AddressSanitizer and UndefinedBehaviorSanitizer
// reports any access past a buffer or any undefined operation.  Calls that
// would reach the device are made to fail their checks first.  Test
// infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../include/mps_adamw.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what)
{
    if (!ok) {
        std::printf("FAILED: %s (%s)\n", what, adamw_last_error());
        ++failures;
    }
}

uintptr_t fake(int64_t k) { return 0x7f0000000000ull + static_cast<uintptr_t>(k) * (1ull << 24); }

std::vector<mps_tensor> list(const std::vector<int64_t>& sizes, int misalign)
{
    std::vector<mps_tensor> t(sizes.size());
    for (size_t i = 0; i < sizes.size(); ++i) {
        const uintptr_t b = fake(static_cast<int64_t>(4 * i)) + 4 * misalign;
        t[i] = {reinterpret_cast<float*>(b), reinterpret_cast<float*>(b + (1ull << 22)),
                reinterpret_cast<float*>(b + (2ull << 22)), reinterpret_cast<const void*>(b + (3ull << 22)),
                nullptr, sizes[i]};
    }
    return t;
}

std::vector<mps_tensor8> list8(const std::vector<int64_t>& sizes)
{
    std::vector<mps_tensor8> t(sizes.size());
    for (size_t i = 0; i < sizes.size(); ++i) {
        const uintptr_t b = fake(static_cast<int64_t>(8 * i));
        t[i] = {reinterpret_cast<float*>(b), reinterpret_cast<uint8_t*>(b + (1ull << 22)),
                reinterpret_cast<uint8_t*>(b + (2ull << 22)), reinterpret_cast<uint8_t*>(b + (3ull << 22)),
                reinterpret_cast<uint8_t*>(b + (4ull << 22)), reinterpret_cast<const void*>(b + (5ull << 22)),
                nullptr, sizes[i]};
    }
    return t;
}

}  // namespace

int main()
{
    const std::vector<std::vector<int64_t>> lists = {
        {1}, {0}, {0, 0, 0}, {0, 1, 3, 4, 5, 7, 8, 9, 63, 64, 65, 2047, 2048, 2049, 4097, 100003},
        {(1ll << 31) + 1003}, {1 << 20}, std::vector<int64_t>(600, 3), {62736416}};
    size_t total = 0;
    for (const auto& sizes : lists) {
        for (int misalign = 0; misalign < 2; ++misalign) {
            auto t = list(sizes, misalign);
            const size_t b = adamw_workspace_bytes(t.data(), static_cast<int>(t.size()));
            expect(b > 0, "workspace size of a valid list");
            total += b;
        }
        auto t8 = list8(sizes);
        const size_t b8 = adamw8_workspace_bytes(t8.data(), static_cast<int>(t8.size()));
        expect(b8 > 0, "workspace size of a valid 8-bit list");
        total += b8;
    }
    auto t = list({4096, 5}, 0);
    const int n = 2;
    expect(adamw_workspace_bytes(nullptr, 1) == 0, "NULL list");
    expect(adamw_workspace_bytes(t.data(), 0) == 0, "empty list");
    auto bad = t;
    bad[1].numel = -1;
    expect(adamw_workspace_bytes(bad.data(), n) == 0, "negative numel");

    void* ws = reinterpret_cast<void*>(0x7e0000000000ull);
    double* s = reinterpret_cast<double*>(0x7d0000000000ull);
    float* c = reinterpret_cast<float*>(0x7d0000001000ull);
    int32_t* step = reinterpret_cast<int32_t*>(0x7d0000002000ull);
    const size_t big = 1u << 30;
    expect(grad_norm_sq(t.data(), n, MPS_DTYPE_F32, nullptr, 1, 1, c, ws, big, nullptr) ==
               MPS_ERR_INVALID_ARGUMENT, "norm without d_sumsq");
    expect(grad_norm_sq(t.data(), n, static_cast<mps_dtype>(7), s, 1, 1, c, ws, big, nullptr) ==
               MPS_ERR_INVALID_ARGUMENT, "unknown dtype");
    expect(grad_norm_sq(t.data(), n, MPS_DTYPE_F32, s, 0.0, 1, c, ws, big, nullptr) ==
               MPS_ERR_INVALID_ARGUMENT, "max_norm 0");
    expect(grad_norm_sq(t.data(), n, MPS_DTYPE_F32, s, 1, 1, c, nullptr, big, nullptr) ==
               MPS_ERR_WORKSPACE, "norm without workspace");
    expect(grad_norm_sq(t.data(), n, MPS_DTYPE_F32, s, 1, 1, c, ws, 16, nullptr) ==
               MPS_ERR_WORKSPACE, "norm with a small workspace");
    expect(clip_coef(nullptr, 1, 1, c, nullptr) == MPS_ERR_INVALID_ARGUMENT, "clip without S");
    expect(adamw_multi_tensor_step(t.data(), n, MPS_DTYPE_F32, c, nullptr, nullptr, 3e-4, 0.9,
                                   0.95, 1e-8, 0.1, ws, big, nullptr) == MPS_ERR_INVALID_ARGUMENT,
           "step without counter");
    expect(adamw_multi_tensor_step(t.data(), n, MPS_DTYPE_F32, c, nullptr, step, 3e-4, 1.0, 0.95,
                                   1e-8, 0.1, ws, big, nullptr) == MPS_ERR_INVALID_ARGUMENT,
           "beta1 = 1");
    auto nomaster = t;
    nomaster[0].master = nullptr;
    expect(adamw_multi_tensor_step(nomaster.data(), n, MPS_DTYPE_F32, c, nullptr, step, 3e-4, 0.9,
                                   0.95, 1e-8, 0.1, ws, big, nullptr) == MPS_ERR_INVALID_ARGUMENT,
           "step without master");
    auto odd = t;
    odd[0].grad = reinterpret_cast<const void*>(fake(1) + 2);
    expect(adamw_multi_tensor_step(odd.data(), n, MPS_DTYPE_F32, c, nullptr, step, 3e-4, 0.9,
                                   0.95, 1e-8, 0.1, ws, big, nullptr) == MPS_ERR_INVALID_ARGUMENT,
           "fp32 gradient not 4-byte aligned");
    expect(adamw_fused_step(t.data(), n, MPS_DTYPE_BF16, 1, 1, 0, s, c, step, 3e-4, 0.9, 0.95,
                            1e-8, 0.1, nullptr, big, nullptr) == MPS_ERR_WORKSPACE,
           "fused step without workspace");
    expect(adamw_clipped_step(t.data(), n, MPS_DTYPE_BF16, 1, 1, 0, s, c, step, 3e-4, 0.9, 0.95,
                              1e-8, 0.1, ws, 64, nullptr, nullptr) == MPS_ERR_WORKSPACE,
           "clipped step with a small workspace");
    expect(adamw_clipped_step(t.data(), n, MPS_DTYPE_BF16, 1, -1, 0, s, c, step, 3e-4, 0.9, 0.95,
                              1e-8, 0.1, ws, big, nullptr, nullptr) == MPS_ERR_INVALID_ARGUMENT,
           "negative gradient scale");
    auto t8 = list8({100, 33});
    expect(adamw8_clipped_step(t8.data(), 2, MPS_DTYPE_BF16, 1, 1, 0, s, c, step, 3e-4, 0.9, 0.95,
                               1e-8, 0.1, nullptr, big, nullptr, nullptr) == MPS_ERR_WORKSPACE,
           "8-bit clipped step without workspace");
    expect(adamw8_grad_norm_sq(t8.data(), 2, MPS_DTYPE_BF16, s, 1, 1, c, ws, 8, nullptr) ==
               MPS_ERR_WORKSPACE, "8-bit norm with a small workspace");
    expect(adamw8_quantize(nullptr, 10, MPS_Q8_E4M3, nullptr, nullptr, nullptr) ==
               MPS_ERR_INVALID_ARGUMENT, "quantize without buffers");
    expect(adamw_workspace_release(ws) == 0, "release of an unknown workspace");
    std::printf("host driver %s: %zu workspace bytes planned\n", failures ? "FAILED" : "ok", total);
    return failures ? 1 : 0;
}
