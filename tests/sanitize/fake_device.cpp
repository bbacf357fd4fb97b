// A stand-in for the HIP runtime and the kernel launchers, for the host-side
// sanitizer build of the library: one in-order "device" queue that runs only
// when the driver says so.  Table copies are queued and performed when the
// queue runs (reading the pinned source then, as the hardware would), each
// launch checks that the workspace header holds the tables it was planned
// with, and every call that would make the host wait for the device aborts.
// Copies from memory that did not come from hipHostMalloc abort too: the
// runtime performs those synchronously.  Test infrastructure only.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <set>

#include "../../mixed_precision_sharded_amd/csrc/kernels.h"
#include "fake_device.h"

struct ihipEvent_t {
    uint64_t after = 0;  // completes once this many queued operations have run
};

namespace {

struct Op {
    bool copy = false;
    void* dst = nullptr;
    const void* src = nullptr;
    size_t bytes = 0;
    mps::WorkspaceHeader* header = nullptr;  // a launch: the header it reads
    uint64_t tag = 0;                        // and the tag it expects there
};

std::deque<Op> g_queue;     // not yet run
uint64_t g_enqueued = 0;    // operations ever enqueued
uint64_t g_ran = 0;         // operations ever run
std::set<void*> g_pinned;
bool g_allow_wait = false;
fake::Counters g_counts;

[[noreturn]] void die(const char* what)
{
    std::fprintf(stderr, "fake device: %s\n", what);
    std::abort();
}

void run_one()
{
    Op op = g_queue.front();
    g_queue.pop_front();
    if (op.copy) {
        std::memcpy(op.dst, op.src, op.bytes);
    } else if (op.header->tag != op.tag) {
        die("a launch found another list's tables in its workspace");
    } else {
        ++g_counts.launches_checked;
    }
    ++g_ran;
}

void enqueue_launch(const mps::WorkspaceView& ws)
{
    Op op;
    op.header = ws.header;
    op.tag = ws.tag;
    g_queue.push_back(op);
    ++g_enqueued;
    ++g_counts.launches;
}

}  // namespace

namespace fake {
void run(size_t n)
{
    for (size_t i = 0; i < n && !g_queue.empty(); ++i) run_one();
}
void run_all() { run(g_queue.size()); }
size_t queued() { return g_queue.size(); }
void allow_wait(bool allow) { g_allow_wait = allow; }
const Counters& counts() { return g_counts; }
size_t pinned_live() { return g_pinned.size(); }
}  // namespace fake

extern "C" {

hipError_t hipHostMalloc(void** ptr, size_t size, unsigned int)
{
    *ptr = std::malloc(size);
    if (!*ptr) return hipErrorOutOfMemory;
    g_pinned.insert(*ptr);
    ++g_counts.host_mallocs;
    return hipSuccess;
}

hipError_t hipHostFree(void* ptr)
{
    if (!g_pinned.erase(ptr)) die("hipHostFree of memory that hipHostMalloc did not return");
    for (const Op& op : g_queue) {
        if (op.copy && op.src == ptr) die("a pinned buffer was freed while a copy from it was queued");
    }
    std::free(ptr);
    return hipSuccess;
}

hipError_t hipEventCreateWithFlags(hipEvent_t* event, unsigned)
{
    *event = new ihipEvent_t;
    return hipSuccess;
}

hipError_t hipEventDestroy(hipEvent_t event)
{
    delete event;
    return hipSuccess;
}

hipError_t hipEventRecord(hipEvent_t event, hipStream_t)
{
    event->after = g_enqueued;
    return hipSuccess;
}

hipError_t hipEventQuery(hipEvent_t event)
{
    ++g_counts.queries;
    return g_ran >= event->after ? hipSuccess : hipErrorNotReady;
}

hipError_t hipEventSynchronize(hipEvent_t event)
{
    if (!g_allow_wait) die("hipEventSynchronize: a call made the host wait for the device");
    while (g_ran < event->after) run_one();
    return hipSuccess;
}

hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t)
{
    if (kind != hipMemcpyHostToDevice) die("unexpected copy kind");
    bool pinned = false;
    for (void* p : g_pinned) {
        // the source must lie inside one pinned allocation (its start, here)
        if (p == src) pinned = true;
    }
    if (!pinned) die("hipMemcpyAsync from pageable memory (the runtime copies it synchronously)");
    Op op;
    op.copy = true;
    op.dst = dst;
    op.src = src;
    op.bytes = bytes;
    g_queue.push_back(op);
    ++g_enqueued;
    ++g_counts.copies;
    return hipSuccess;
}

const char* hipGetErrorString(hipError_t) { return "fake device error"; }

hipError_t hipGetDevice(int* device)
{
    *device = 0;
    return hipSuccess;
}

}  // extern "C"

namespace mps {
hipError_t launch_grad_norm(const WorkspaceView& ws, bool, int, int, double*, double, double,
                            float*, hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_grad_norm_partials(const WorkspaceView& ws, bool, int, int, const int32_t*,
                                     hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_clip_coef(const double*, double, double, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_adamw_step(const WorkspaceView& ws, bool, bool, int, const float*, const double*,
                             int32_t*, const HyperParams&, hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_clipped_step(const WorkspaceView& ws, bool, bool, int, int, double, double, int,
                               double*, float*, int32_t*, const HyperParams&, hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t fused_grid_limit(bool, int* max_blocks)
{
    *max_blocks = 256;
    return hipSuccess;
}
hipError_t launch_fused_step(const WorkspaceView& ws, bool, int, int, double, double, int, double*,
                             float*, int32_t*, const HyperParams&, uint32_t, hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_fused_status(WorkspaceHeader*, uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t scratch_address(int, void**) { return hipErrorInvalidDevice; }
hipError_t launch_adamw8_step(const WorkspaceView& ws, const QuantEntry*, bool, int, const float*,
                              const double*, int32_t*, const HyperParams&, hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_adamw8_clipped(const WorkspaceView& ws, const QuantEntry*, bool, int, int, double,
                                 double, int, double*, float*, int32_t*, const HyperParams&,
                                 hipStream_t)
{
    enqueue_launch(ws);
    return hipSuccess;
}
hipError_t launch_quantize(const float*, int64_t, bool, uint8_t*, uint8_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_dequantize(const uint8_t*, const uint8_t*, int64_t, bool, float*, hipStream_t) { return hipSuccess; }
}  // namespace mps
