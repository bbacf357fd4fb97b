// Drives the library's list planning against the fake device with seeded
// random lists: tensor counts from 1 to 1500, sizes from empty to past the
// whole-model threshold (2^30 elements), every stream of a tensor either
// sharing one element misalignment or misaligned on its own, fp32 or bf16
// gradients, with or without the bf16 copy, fp32 or 8-bit moment state, and
// each list through every entry point (the norm, the three-call update, the
// clipped step, the single-launch step, the 8-bit step).  The fake device
// runs each launch's check_tables on the tables it finds; any violation
// aborts.  Pointers are fake addresses: nothing here touches tensor memory.
// Test infrastructure only.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "../../include/mps_adamw.h"
#include "fake_device.h"

namespace {

int failures = 0;

void expect(bool ok, const char* what, int list)
{
    if (!ok) {
        std::printf("FAILED: %s, list %d (%s)\n", what, list, adamw_last_error());
        ++failures;
    }
}

uint64_t rng = 0x706c616eull;

uint64_t next_u64()
{
    uint64_t z = (rng += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

int64_t below(int64_t n) { return static_cast<int64_t>(next_u64() % static_cast<uint64_t>(n)); }

int64_t random_size()
{
    const int64_t r = below(100);
    if (r < 10) return 0;
    if (r < 40) return 1 + below(100);
    if (r < 80) return 1 + below(70000);
    if (r < 97) return 1 + below(5000000);
    return (int64_t{1} << 30) + below(int64_t{1} << 24);  // alone past the whole-model threshold
}

// Stream s of tensor i: its own region of the fake address space, plus an
// element offset.
uintptr_t address(int s, int i, int64_t offset_elems, int elem_bytes)
{
    return (uintptr_t{1} << 40) + static_cast<uintptr_t>(s) * (uintptr_t{1} << 45) +
           static_cast<uintptr_t>(i) * (uintptr_t{1} << 34) +
           static_cast<uintptr_t>(offset_elems * elem_bytes);
}

}  // namespace

int main()
{
    int32_t* d_step = reinterpret_cast<int32_t*>(0x1000);
    double* d_sumsq = reinterpret_cast<double*>(0x2000);
    float* d_coef = reinterpret_cast<float*>(0x3000);
    int lists = 0;
    for (int l = 0; l < 400; ++l) {
        const int r = static_cast<int>(below(100));
        const int n = r < 15 ? 1 : r < 90 ? 1 + static_cast<int>(below(40)) : 200 + static_cast<int>(below(1300));
        const bool bf16 = below(2) == 1;
        const bool copy = below(2) == 1;
        const bool shared = below(3) != 0;  // one misalignment for every stream of a tensor
        const mps_dtype dtype = bf16 ? MPS_DTYPE_BF16 : MPS_DTYPE_F32;
        const int gbytes = bf16 ? 2 : 4;
        std::vector<mps_tensor> t(n);
        std::vector<mps_tensor8> t8(n);
        for (int i = 0; i < n; ++i) {
            const int64_t numel = n > 100 ? below(50000) : random_size();
            int64_t off[5];
            const int64_t one = below(4);
            for (int s = 0; s < 5; ++s) off[s] = shared ? one : below(4);
            t[i] = {reinterpret_cast<float*>(address(0, i, off[0], 4)),
                    reinterpret_cast<float*>(address(1, i, off[1], 4)),
                    reinterpret_cast<float*>(address(2, i, off[2], 4)),
                    reinterpret_cast<const void*>(address(3, i, off[3], gbytes)),
                    copy ? reinterpret_cast<uint16_t*>(address(4, i, off[4], 2)) : nullptr, numel};
            t8[i] = {t[i].master,
                     reinterpret_cast<uint8_t*>(address(1, i, off[1], 1)),
                     reinterpret_cast<uint8_t*>(address(2, i, 0, 1)),
                     reinterpret_cast<uint8_t*>(address(1, i, off[2], 1) + (uintptr_t{1} << 44)),
                     reinterpret_cast<uint8_t*>(address(2, i, 0, 1) + (uintptr_t{1} << 44)),
                     t[i].grad, t[i].param_bf16, numel};
        }

        const size_t bytes = adamw_workspace_bytes(t.data(), n);
        expect(bytes > 0, "workspace size", l);
        void* ws = std::aligned_alloc(256, (bytes + 255) / 256 * 256);
        expect(grad_norm_sq(t.data(), n, dtype, d_sumsq, 1.0, 1.0, d_coef, ws, bytes, nullptr) == MPS_OK,
               "grad_norm_sq", l);
        expect(adamw_multi_tensor_step(t.data(), n, dtype, d_coef, nullptr, d_step, 3e-4, 0.9, 0.95,
                                       1e-8, 0.1, ws, bytes, nullptr) == MPS_OK,
               "adamw_multi_tensor_step", l);
        expect(adamw_clipped_step(t.data(), n, dtype, 1.0, 1.0, 0, d_sumsq, d_coef, d_step, 3e-4, 0.9,
                                  0.95, 1e-8, 0.1, ws, bytes, nullptr, nullptr) == MPS_OK,
               "adamw_clipped_step", l);
        if (l % 4 == 0) {
            expect(adamw_fused_step(t.data(), n, dtype, 1.0, 1.0, 0, d_sumsq, d_coef, d_step, 3e-4,
                                    0.9, 0.95, 1e-8, 0.1, ws, bytes, nullptr) == MPS_OK,
                   "adamw_fused_step", l);
        }
        fake::run_all();
        fake::allow_wait(true);
        expect(adamw_workspace_release(ws) == MPS_OK, "release", l);
        fake::allow_wait(false);
        std::free(ws);

        const size_t bytes8 = adamw8_workspace_bytes(t8.data(), n);
        expect(bytes8 > 0, "8-bit workspace size", l);
        void* ws8 = std::aligned_alloc(256, (bytes8 + 255) / 256 * 256);
        expect(adamw8_clipped_step(t8.data(), n, dtype, 1.0, 1.0, 0, d_sumsq, d_coef, d_step, 3e-4,
                                   0.9, 0.95, 1e-8, 0.1, ws8, bytes8, nullptr, nullptr) == MPS_OK,
               "adamw8_clipped_step", l);
        expect(adamw8_multi_tensor_step(t8.data(), n, dtype, d_coef, nullptr, d_step, 3e-4, 0.9, 0.95,
                                        1e-8, 0.1, ws8, bytes8, nullptr) == MPS_OK,
               "adamw8_multi_tensor_step", l);
        fake::run_all();
        fake::allow_wait(true);
        expect(adamw_workspace_release(ws8) == MPS_OK, "release (8-bit)", l);
        fake::allow_wait(false);
        std::free(ws8);
        ++lists;
    }
    if (failures) return 1;
    if (fake::counts().tables_checked != fake::counts().launches) {
        std::printf("FAILED: %llu of %llu launches had their tables checked\n",
                    static_cast<unsigned long long>(fake::counts().tables_checked),
                    static_cast<unsigned long long>(fake::counts().launches));
        return 1;
    }
    std::printf("plan driver ok: %d lists, %llu launches, every table checked\n", lists,
                static_cast<unsigned long long>(fake::counts().launches));
    return 0;
}
