// A stand-in for the HIP runtime and the kernel launchers, for the host-side
// sanitizer build of the library: one in-order "device" queue that runs only
// when the driver says so.  Table copies are queued and performed when the
// queue runs (reading the pinned source then, as the hardware would), each
// launch checks that the workspace header holds the tables it was planned
// with, and every call that would make the host wait for the device aborts.
// Copies from memory that did not come from hipHostMalloc abort too: the
// runtime performs those synchronously.  When a launch runs, the tables it
// finds are also checked against what the kernels rely on (check_tables):
// every chunk of every tensor mapped to that tensor in order, the alignment
// head of each tensor from its stream addresses, the one-tensor entry, the
// whole-model flag and the partial-sum bound of the grids.  Test
// infrastructure only.
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

// What a launch knows about its list, for check_tables.
enum class ListKind { kState32, kState8, kNormOnly };

struct Op {
    bool copy = false;
    void* dst = nullptr;
    const void* src = nullptr;
    size_t bytes = 0;
    mps::WorkspaceHeader* header = nullptr;  // a launch: the header it reads
    uint64_t tag = 0;                        // and the tag it expects there
    mps::WorkspaceView view{};
    ListKind kind = ListKind::kNormOnly;
    bool grad_bf16 = false;
    int large = -1;                          // the launch's whole-model flag, -1: none
    const mps::QuantEntry* quant = nullptr;  // an 8-bit list's state table
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

// The element offset h in [0, 4) at which a stream of `elem` bytes per
// element reaches a group of four aligned to 4 * elem bytes, or -1 when the
// address is not even element-aligned.
int stream_head(const void* p, uintptr_t elem)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a % elem) return -1;
    return static_cast<int>((4 - (a / elem) % 4) % 4);
}

// The head the fp32-state kernels need: the offset every present stream
// agrees on, else -1.
int expected_head(const mps::TensorEntry& e, bool grad_bf16)
{
    int head = -2;  // no stream seen yet
    auto meet = [&](const void* p, uintptr_t elem) {
        if (!p) return;
        const int h = stream_head(p, elem);
        head = (head == -2 || head == h) ? h : -1;
    };
    meet(e.master, 4);
    meet(e.exp_avg, 4);
    meet(e.exp_avg_sq, 4);
    meet(e.grad, grad_bf16 ? 2 : 4);
    meet(e.param_bf16, 2);
    return head == -2 ? 0 : head;
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

void check_tables(const Op& op)
{
    const mps::WorkspaceView& v = op.view;
    const mps::WorkspaceHeader* h = v.header;
    if (h->n_tensors != v.n_tensors || h->n_chunks != v.n_chunks || h->chunk_elems != v.chunk_elems) {
        die("table check: the header disagrees with the launch's view");
    }
    if (v.n_tensors < 1) die("table check: a list without tensor entries");
    const int64_t c = v.chunk_elems;
    if (c < mps::kChunkMin || c % mps::kChunkQuantum) die("table check: chunk size");
    int64_t next = 0, total = 0;
    int with_elements = 0, last = -1;
    for (int i = 0; i < v.n_tensors; ++i) {
        const mps::TensorEntry& e = v.tensors[i];
        if (e.numel < 0) die("table check: negative numel");
        if (e.first_chunk != next) die("table check: a tensor's first chunk");
        const int64_t k = (e.numel + c - 1) / c;
        for (int64_t j = 0; j < k; ++j) {
            if (v.chunk_map[next + j] != static_cast<uint32_t>(i)) die("table check: chunk map");
        }
        next += k;
        total += e.numel;
        if (e.numel == 0) {
            if (e.master || e.exp_avg || e.exp_avg_sq || e.grad || e.param_bf16) {
                die("table check: an empty tensor's entry holds pointers");
            }
            continue;
        }
        ++with_elements;
        last = i;
        if (e.head < -1 || e.head > 3) die("table check: head out of range");
        if (e.head >= 0) {  // the gradient stream, which every kernel reads, is aligned there
            const uintptr_t ge = op.grad_bf16 ? 2 : 4;
            if ((reinterpret_cast<uintptr_t>(e.grad) + ge * e.head) % (4 * ge)) {
                die("table check: head leaves the gradient misaligned");
            }
        }
        if (op.kind == ListKind::kState32 && e.head != expected_head(e, op.grad_bf16)) {
            die("table check: head of a tensor");
        }
        if (op.kind == ListKind::kState8) {
            const mps::QuantEntry& q = op.quant[i];
            const bool vector = aligned(e.master, 16) && aligned(e.grad, 16) &&
                                aligned(e.param_bf16, 16) && aligned(q.m_codes, 8) &&
                                aligned(q.v_codes, 8);
            if (e.head != (vector ? 0 : -1)) die("table check: head of an 8-bit tensor");
        }
    }
    if (next != v.n_chunks) die("table check: chunk count");
    const int solo = with_elements == 1 ? last : -1;
    if (v.solo_tensor != solo) die("table check: the one-tensor index");
    if (solo >= 0) {
        const mps::TensorEntry& e = v.tensors[solo];
        const mps::SoloEntry& s = v.solo;
        if (s.master != e.master || s.exp_avg != e.exp_avg || s.exp_avg_sq != e.exp_avg_sq ||
            s.grad != e.grad || s.param_bf16 != e.param_bf16 || s.numel != e.numel ||
            s.first_chunk != e.first_chunk || s.head != e.head) {
            die("table check: the one-tensor entry");
        }
    }
    if (op.large >= 0 && op.large != (total >= mps::kLargeListElems ? 1 : 0)) {
        die("table check: the whole-model flag");
    }
    const int64_t cap = op.kind == ListKind::kState8         ? mps::kQ8ChunkMax
                        : total >= mps::kLargeListElems ? mps::kLargeChunkMax
                                                        : mps::kChunkMax;
    if (op.kind != ListKind::kNormOnly && c > cap) die("table check: chunk size above its cap");
    for (int g = 0; g <= mps::kTicketGroups; ++g) {
        if (v.tickets[mps::kTicketStride * g] != 0) die("table check: tickets not at zero");
    }
    ++g_counts.tables_checked;
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
        check_tables(op);
    }
    ++g_ran;
}

void enqueue_launch(const mps::WorkspaceView& ws, ListKind kind, bool grad_bf16, int large = -1,
                    const mps::QuantEntry* quant = nullptr)
{
    Op op;
    op.header = ws.header;
    op.tag = ws.tag;
    op.view = ws;
    op.kind = kind;
    op.grad_bf16 = grad_bf16;
    op.large = large;
    op.quant = quant;
    g_queue.push_back(op);
    ++g_enqueued;
    ++g_counts.launches;
}

// Grids whose blocks write or read one partial sum each must fit the
// workspace's partials.
void check_partials_grid(int grid)
{
    if (grid < 1 || grid > mps::kPartials) die("a norm grid beyond the workspace's partial sums");
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
hipError_t launch_grad_norm(const WorkspaceView& ws, bool bf16, int grid, int, double*, double,
                            double, float*, hipStream_t)
{
    check_partials_grid(grid);
    enqueue_launch(ws, ListKind::kNormOnly, bf16);
    return hipSuccess;
}
hipError_t launch_grad_norm_partials(const WorkspaceView& ws, bool bf16, int grid, int,
                                     const int32_t*, hipStream_t)
{
    check_partials_grid(grid);
    enqueue_launch(ws, ListKind::kNormOnly, bf16);
    return hipSuccess;
}
hipError_t launch_clip_coef(const double*, double, double, float*, hipStream_t) { return hipSuccess; }
hipError_t launch_adamw_step(const WorkspaceView& ws, bool bf16, bool large, int, const float*,
                             const double*, int32_t*, const HyperParams&, hipStream_t)
{
    enqueue_launch(ws, ListKind::kState32, bf16, large ? 1 : 0);
    return hipSuccess;
}
hipError_t launch_clipped_step(const WorkspaceView& ws, bool bf16, bool large, int, int n_partials,
                               double, double, int, double*, float*, int32_t*, const HyperParams&,
                               hipStream_t)
{
    check_partials_grid(n_partials);
    enqueue_launch(ws, ListKind::kState32, bf16, large ? 1 : 0);
    return hipSuccess;
}
hipError_t fused_grid_limit(bool, int* max_blocks)
{
    *max_blocks = 256;
    return hipSuccess;
}
hipError_t launch_fused_step(const WorkspaceView& ws, bool bf16, int grid, int, double, double, int,
                             double*, float*, int32_t*, const HyperParams&, uint32_t, hipStream_t)
{
    check_partials_grid(grid);
    enqueue_launch(ws, ListKind::kState32, bf16);
    return hipSuccess;
}
hipError_t launch_fused_status(WorkspaceHeader*, uint32_t*, hipStream_t) { return hipSuccess; }
hipError_t scratch_address(int, void**) { return hipErrorInvalidDevice; }
hipError_t launch_adamw8_step(const WorkspaceView& ws, const QuantEntry* quant, bool bf16, int,
                              const float*, const double*, int32_t*, const HyperParams&, hipStream_t)
{
    enqueue_launch(ws, ListKind::kState8, bf16, -1, quant);
    return hipSuccess;
}
hipError_t launch_adamw8_clipped(const WorkspaceView& ws, const QuantEntry* quant, bool bf16, int,
                                 int n_partials, double, double, int, double*, float*, int32_t*,
                                 const HyperParams&, hipStream_t)
{
    check_partials_grid(n_partials);
    enqueue_launch(ws, ListKind::kState8, bf16, -1, quant);
    return hipSuccess;
}
hipError_t launch_quantize(const float*, int64_t, bool, uint8_t*, uint8_t*, hipStream_t) { return hipSuccess; }
hipError_t launch_dequantize(const uint8_t*, const uint8_t*, int64_t, bool, float*, hipStream_t) { return hipSuccess; }
}  // namespace mps
