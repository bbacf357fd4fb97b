// Drives the library's table uploads against the fake device: list changes
// on one workspace while the device runs nothing (no call may wait for it),
// the device then running everything in order (every launch must find its
// own list's tables), staging buffers reused only after their copies ran,
// the same list again (no copy, no allocation), and the release (the one
// call allowed to wait), after which every pinned buffer is freed.  Test
// infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/mps_adamw.h"
#include "fake_device.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what)
{
    if (!ok) {
        std::printf("FAILED: %s (%s)\n", what, adamw_last_error());
        ++failures;
    }
}

uintptr_t fake_ptr(int64_t k) { return 0x7f0000000000ull + static_cast<uintptr_t>(k) * (1ull << 26); }

std::vector<mps_tensor> list(const std::vector<int64_t>& sizes, int salt)
{
    std::vector<mps_tensor> t(sizes.size());
    for (size_t i = 0; i < sizes.size(); ++i) {
        const uintptr_t b = fake_ptr(static_cast<int64_t>(8 * i + 64 * salt));
        t[i] = {reinterpret_cast<float*>(b), reinterpret_cast<float*>(b + (1ull << 24)),
                reinterpret_cast<float*>(b + (2ull << 24)), reinterpret_cast<const void*>(b + (3ull << 24)),
                nullptr, sizes[i]};
    }
    return t;
}

int step(const std::vector<mps_tensor>& t, void* ws, size_t bytes)
{
    return adamw_clipped_step(t.data(), static_cast<int>(t.size()), MPS_DTYPE_F32, 1.0, 1.0, 0,
                              nullptr, nullptr, reinterpret_cast<int32_t*>(0x1000), 3e-4, 0.9, 0.95,
                              1e-8, 0.1, ws, bytes, nullptr, nullptr);
}

}  // namespace

int main()
{
    const auto a = list({5000, 3, 1 << 20}, 1);
    const auto b = list({100003}, 2);
    const auto c = list(std::vector<int64_t>(50, 4097), 3);
    size_t bytes = 0;
    for (const auto* t : {&a, &b, &c}) {
        const size_t n = adamw_workspace_bytes(t->data(), static_cast<int>(t->size()));
        expect(n > 0, "workspace size");
        bytes = n > bytes ? n : bytes;
    }
    void* ws = std::aligned_alloc(256, (bytes + 255) / 256 * 256);

    // Alternate lists while the device runs nothing: every call uploads, none
    // waits, and every upload holds its own staging buffer.
    const std::vector<mps_tensor>* order[] = {&a, &b, &c};
    for (int i = 0; i < 30; ++i) expect(step(*order[i % 3], ws, bytes) == MPS_OK, "step (device idle)");
    expect(fake::counts().copies == 30, "one upload per list change");
    expect(fake::counts().host_mallocs == 30, "no staging buffer reused before its copy ran");

    // Half the queue runs: the finished uploads' buffers become reusable.
    fake::run(fake::queued() / 2);
    for (int i = 0; i < 6; ++i) expect(step(*order[i % 3], ws, bytes) == MPS_OK, "step (half run)");
    expect(fake::counts().host_mallocs == 30, "finished buffers are reused");
    fake::run_all();
    expect(fake::counts().launches_checked == fake::counts().launches,
           "every launch found its own list's tables");

    // Another list, then the same list again and again: one copy, and no
    // allocation (the finished buffers serve it).
    const uint64_t copies = fake::counts().copies;
    for (int i = 0; i < 100; ++i) expect(step(b, ws, bytes) == MPS_OK, "step (same list)");
    expect(fake::counts().copies == copies + 1, "one upload for a repeated list");
    expect(fake::counts().host_mallocs == 30, "no new staging buffer");
    fake::run_all();
    expect(fake::counts().launches_checked == fake::counts().launches, "launches after reuse");

    // A norm-only call plans without the state; the step that follows with
    // the same list checks the state pointers but uploads nothing new.
    expect(grad_norm_sq(c.data(), static_cast<int>(c.size()), MPS_DTYPE_F32,
                        reinterpret_cast<double*>(0x2000), 0.0, 1.0, nullptr, ws, bytes, nullptr) ==
               MPS_OK,
           "norm");
    const uint64_t before_norm_step = fake::counts().copies;
    expect(step(c, ws, bytes) == MPS_OK, "step after norm");
    expect(fake::counts().copies == before_norm_step, "the step reuses the norm's tables");
    fake::run_all();
    expect(fake::counts().launches_checked == fake::counts().launches, "norm then step");

    // Release: waits for the running copies, frees every pinned buffer.
    for (int i = 0; i < 4; ++i) expect(step(*order[i % 3], ws, bytes) == MPS_OK, "step before release");
    fake::allow_wait(true);
    expect(adamw_workspace_release(ws) == MPS_OK, "release");
    fake::allow_wait(false);
    expect(fake::pinned_live() == 0, "release frees the staging buffers");
    fake::run_all();
    std::free(ws);

    if (failures) return 1;
    std::printf("upload driver ok: %llu copies, %llu staging buffers, %llu launches\n",
                static_cast<unsigned long long>(fake::counts().copies),
                static_cast<unsigned long long>(fake::counts().host_mallocs),
                static_cast<unsigned long long>(fake::counts().launches));
    return 0;
}
