// C ABI of the clipped mixed-precision AdamW step: argument validation, the
// multi-tensor chunk table, its upload into the caller's workspace, and the
// kernel launches.  Declared in include/mps_adamw.h.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <deque>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/mps_adamw.h"
#include "kernels.h"
#include "layout.h"

namespace {

using mps::TensorEntry;
using mps::WorkspaceHeader;

static_assert(mps::kScratchBytes == MPS_NOALLOC_WORKSPACE_BYTES,
              "the header states the library-held workspace's size");

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int ok()
{
    g_last_error.clear();
    return MPS_OK;
}

// ------------------------------------------------------------ the plan ---

// Host image of everything the kernels read from the workspace, plus where
// each part sits.
struct Plan {
    std::vector<unsigned char> image;  // header, tensor entries, chunk map, ticket lines
    size_t tensors_off = 0;
    size_t quant_off = 0;   // 8-bit lists: QuantEntry table (else == chunks_off)
    size_t chunks_off = 0;
    size_t tickets_off = 0;
    size_t constants_off = 0;
    size_t partials_off = 0;
    size_t total_bytes = 0;
    int n_tensors = 0;
    int n_chunks = 0;
    int solo_tensor = -1;   // the one tensor with elements, else -1
    mps::SoloEntry solo{};  // its entry, passed with every launch
    mps::QuantEntry solo_quant{};  // an 8-bit list: its 8-bit state
    int64_t chunk_elems = 0;
    bool large = false;     // an fp32-state list of at least kLargeListElems elements
    uint64_t tag = 0;
};

int64_t pick_chunk_elems(int64_t total, int64_t max_elems)
{
    int64_t c = total / mps::kChunkTarget;
    c = (c / mps::kChunkQuantum) * mps::kChunkQuantum;
    if (c < mps::kChunkMin) c = mps::kChunkMin;
    if (c > max_elems) c = max_elems;
    return c;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Smallest h in [0, 4) such that every present stream is 16-byte aligned
// (fp32) or 8-byte aligned (bf16) at element h; -1 if there is none.
int common_head(const mps::TensorEntry& e, bool grad_bf16)
{
    for (int h = 0; h < 4; ++h) {
        bool good = true;
        auto need = [&](const void* p, int elem_bytes) {
            if (!p) return;
            const uintptr_t a = reinterpret_cast<uintptr_t>(p) + static_cast<uintptr_t>(h) * elem_bytes;
            if (a % (4 * elem_bytes) != 0) good = false;
        };
        need(e.master, 4);
        need(e.exp_avg, 4);
        need(e.exp_avg_sq, 4);
        need(e.grad, grad_bf16 ? 2 : 4);
        need(e.param_bf16, 2);
        if (good) return h;
    }
    return -1;
}

// A 64-bit digest of the tables, eight bytes per step (a byte-at-a-time hash
// cost the host ~1 ns per byte: 2 ms per call for the 8B model's 2 MB chunk
// map).  Each word is folded in with a multiply by an odd constant and a
// shift-xor; it only has to tell one set of tables from another.
uint64_t digest(const unsigned char* p, size_t n, uint64_t h)
{
    constexpr uint64_t kOdd = 0x9E3779B97F4A7C15ull;
    size_t i = 0;
    for (; i + 8 <= n; i += 8) {
        uint64_t w;
        std::memcpy(&w, p + i, 8);
        h = (h ^ w) * kOdd;
        h ^= h >> 29;
    }
    for (; i < n; ++i) {
        h = (h ^ p[i]) * kOdd;
        h ^= h >> 29;
    }
    return h;
}

// Chunk the list and build the workspace image: header, tensor entries,
// the QuantEntry table of an 8-bit list (`quant` non-NULL), chunk map.
// `entries` carry numel, pointers and head; first_chunk is filled in here.
int layout_plan(std::vector<TensorEntry>& entries, const std::vector<mps::QuantEntry>* quant,
                int64_t total, Plan& plan)
{
    const int n = static_cast<int>(entries.size());
    plan.large = !quant && total >= mps::kLargeListElems;
    plan.chunk_elems = pick_chunk_elems(
        total, quant ? mps::kQ8ChunkMax : (plan.large ? mps::kLargeChunkMax : mps::kChunkMax));
    int64_t n_chunks = 0;
    for (TensorEntry& e : entries) {
        e.first_chunk = static_cast<int32_t>(n_chunks);
        n_chunks += (e.numel + plan.chunk_elems - 1) / plan.chunk_elems;
        if (n_chunks > INT32_MAX) return fail(MPS_ERR_INVALID_ARGUMENT, "too many chunks");
    }
    plan.n_tensors = n;
    plan.n_chunks = static_cast<int>(n_chunks);
    plan.solo_tensor = -1;
    for (int i = 0; i < n; ++i) {
        if (entries[i].numel == 0) continue;
        if (plan.solo_tensor >= 0) {
            plan.solo_tensor = -1;
            break;
        }
        plan.solo_tensor = i;
    }
    if (plan.solo_tensor >= 0) {
        const TensorEntry& e = entries[plan.solo_tensor];
        plan.solo = mps::SoloEntry{e.master, e.exp_avg,    e.exp_avg_sq, e.grad,
                                   e.param_bf16, e.numel, e.first_chunk, e.head};
        if (quant) plan.solo_quant = (*quant)[plan.solo_tensor];
    }

    plan.tensors_off = sizeof(WorkspaceHeader);
    plan.quant_off = plan.tensors_off + sizeof(TensorEntry) * static_cast<size_t>(n);
    plan.chunks_off = plan.quant_off + (quant ? sizeof(mps::QuantEntry) * static_cast<size_t>(n) : 0);
    // At least one chunk-map slot (zero for a list without elements), so
    // that the kernels' first lookup is always in the table.
    const int64_t map_slots = n_chunks > 0 ? n_chunks : 1;
    plan.tickets_off = round_up(plan.chunks_off + sizeof(uint32_t) * map_slots, 128);
    plan.constants_off = plan.tickets_off +
                         sizeof(uint32_t) * mps::kTicketStride * (mps::kTicketGroups + 1);
    plan.partials_off = round_up(plan.constants_off + sizeof(mps::WorkspaceConstants), 256);
    plan.total_bytes = plan.partials_off + sizeof(double) * mps::kPartials;

    plan.image.assign(plan.partials_off, 0);
    unsigned char* base = plan.image.data();
    std::memcpy(base + plan.tensors_off, entries.data(), sizeof(TensorEntry) * n);
    if (quant) std::memcpy(base + plan.quant_off, quant->data(), sizeof(mps::QuantEntry) * n);
    auto* constants = reinterpret_cast<mps::WorkspaceConstants*>(base + plan.constants_off);
    constants->zero = 0.0;
    constants->one = 1.0f;
    uint32_t* map = reinterpret_cast<uint32_t*>(base + plan.chunks_off);
    for (int i = 0; i < n; ++i) {
        const int64_t k = (entries[i].numel + plan.chunk_elems - 1) / plan.chunk_elems;
        for (int64_t j = 0; j < k; ++j) map[entries[i].first_chunk + j] = static_cast<uint32_t>(i);
    }

    // The tag identifies the tables; it never equals zero, so freshly
    // zeroed memory is never mistaken for an upload.
    uint64_t tag = digest(base + plan.tensors_off, plan.partials_off - plan.tensors_off,
                          0x6D70735F74616273ull);
    tag = digest(reinterpret_cast<const unsigned char*>(&plan.chunk_elems), sizeof plan.chunk_elems,
                 tag);
    plan.tag = tag ? tag : 1;

    WorkspaceHeader* hdr = reinterpret_cast<WorkspaceHeader*>(base);
    hdr->tag = plan.tag;
    hdr->n_tensors = n;
    hdr->n_chunks = plan.n_chunks;
    hdr->chunk_elems = plan.chunk_elems;
    return MPS_OK;
}

// Validate the list and lay out the workspace.  `need_state` asks for the
// master / moment pointers (the step); the norm reads gradients only.
int build_plan(const mps_tensor* tensors, int n, int grad_dtype, bool need_state, Plan& plan)
{
    if (!tensors) return fail(MPS_ERR_INVALID_ARGUMENT, "tensors is NULL");
    if (n <= 0) return fail(MPS_ERR_INVALID_ARGUMENT, "n_tensors must be >= 1 (got %d)", n);
    if (grad_dtype != MPS_DTYPE_F32 && grad_dtype != MPS_DTYPE_BF16) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "unknown gradient dtype %d", grad_dtype);
    }
    const bool bf16 = grad_dtype == MPS_DTYPE_BF16;
    const int gbytes = bf16 ? 2 : 4;

    int64_t total = 0;
    for (int i = 0; i < n; ++i) {
        const mps_tensor& t = tensors[i];
        if (t.numel < 0) return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: numel < 0", i);
        if (t.numel == 0) continue;
        if (!t.grad) return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: grad is NULL", i);
        if (reinterpret_cast<uintptr_t>(t.grad) % gbytes) {
            return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: grad not %d-byte aligned", i, gbytes);
        }
        if (need_state) {
            if (!t.master || !t.exp_avg || !t.exp_avg_sq) {
                return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: master/exp_avg/exp_avg_sq NULL", i);
            }
            if ((reinterpret_cast<uintptr_t>(t.master) | reinterpret_cast<uintptr_t>(t.exp_avg) |
                 reinterpret_cast<uintptr_t>(t.exp_avg_sq)) % 4) {
                return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: fp32 state not 4-byte aligned", i);
            }
            if (reinterpret_cast<uintptr_t>(t.param_bf16) % 2) {
                return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: param_bf16 not 2-byte aligned", i);
            }
        }
        if (total > INT64_MAX - t.numel) return fail(MPS_ERR_INVALID_ARGUMENT, "total numel overflows");
        total += t.numel;
    }

    std::vector<TensorEntry> entries(n);
    for (int i = 0; i < n; ++i) {
        const mps_tensor& t = tensors[i];
        TensorEntry& e = entries[i];
        std::memset(&e, 0, sizeof e);
        e.numel = t.numel;
        if (t.numel == 0) continue;  // no chunks; pointers stay NULL
        e.master = t.master;
        e.exp_avg = t.exp_avg;
        e.exp_avg_sq = t.exp_avg_sq;
        e.grad = t.grad;
        e.param_bf16 = t.param_bf16;  // the same list gives the same tables for both calls
        e.head = common_head(e, bf16);
    }
    return layout_plan(entries, nullptr, total, plan);
}

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// The same for a list with 8-bit moments.  head is 0 when every stream is
// aligned for the vector path at the tensor's start, -1 otherwise.
int build_plan8(const mps_tensor8* tensors, int n, int grad_dtype, bool need_state, Plan& plan)
{
    if (!tensors) return fail(MPS_ERR_INVALID_ARGUMENT, "tensors is NULL");
    if (n <= 0) return fail(MPS_ERR_INVALID_ARGUMENT, "n_tensors must be >= 1 (got %d)", n);
    if (grad_dtype != MPS_DTYPE_F32 && grad_dtype != MPS_DTYPE_BF16) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "unknown gradient dtype %d", grad_dtype);
    }
    const bool bf16 = grad_dtype == MPS_DTYPE_BF16;
    const int gbytes = bf16 ? 2 : 4;

    int64_t total = 0;
    std::vector<TensorEntry> entries(n);
    std::vector<mps::QuantEntry> quant(n);
    for (int i = 0; i < n; ++i) {
        const mps_tensor8& t = tensors[i];
        if (t.numel < 0) return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: numel < 0", i);
        TensorEntry& e = entries[i];
        mps::QuantEntry& q = quant[i];
        std::memset(&e, 0, sizeof e);
        std::memset(&q, 0, sizeof q);
        e.numel = t.numel;
        if (t.numel == 0) continue;
        if (!t.grad) return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: grad is NULL", i);
        if (!aligned(t.grad, gbytes)) {
            return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: grad not %d-byte aligned", i, gbytes);
        }
        if (need_state) {
            if (!t.master || !t.exp_avg_codes || !t.exp_avg_scales || !t.exp_avg_sq_codes ||
                !t.exp_avg_sq_scales) {
                return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: master or 8-bit state is NULL", i);
            }
            if (!aligned(t.master, 4)) return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: master not 4-byte aligned", i);
            if (!aligned(t.param_bf16, 2)) {
                return fail(MPS_ERR_INVALID_ARGUMENT, "tensor %d: param_bf16 not 2-byte aligned", i);
            }
        }
        if (total > INT64_MAX - t.numel) return fail(MPS_ERR_INVALID_ARGUMENT, "total numel overflows");
        total += t.numel;
        e.master = t.master;
        e.grad = t.grad;
        e.param_bf16 = t.param_bf16;
        q.m_codes = t.exp_avg_codes;
        q.m_scales = t.exp_avg_scales;
        q.v_codes = t.exp_avg_sq_codes;
        q.v_scales = t.exp_avg_sq_scales;
        const bool vector = aligned(t.master, 16) && aligned(t.grad, 16) && aligned(t.param_bf16, 16) &&
                            aligned(t.exp_avg_codes, 8) && aligned(t.exp_avg_sq_codes, 8);
        e.head = vector ? 0 : -1;
    }
    return layout_plan(entries, &quant, total, plan);
}

// -------------------------------------------------- workspace upload cache ---

// A pinned host buffer that carries one table upload.  Copies from pageable
// memory are performed synchronously by the HIP runtime (they would make a
// list change wait for the stream); from pinned memory the copy is only
// enqueued, and the buffer must then stay untouched until the copy is done,
// which its event tells.
struct Staging {
    void* host = nullptr;
    size_t capacity = 0;
    hipEvent_t done = nullptr;
};

struct Uploaded {
    uint64_t tag = 0;             // tables the workspace holds (enqueued), 0 = none
    std::deque<Staging> in_flight;  // uploads whose copies may still run, oldest first
    std::vector<Staging> idle;      // buffers whose copies have finished
    // The call that last planned this workspace: list kind, gradient dtype
    // and the caller's tensor array, byte for byte; whether its state
    // pointers were checked (a norm-only call leaves them unchecked); and its
    // plan without the image.
    std::vector<unsigned char> key;
    bool state_checked = false;
    Plan meta;
};

std::mutex g_cache_mutex;
std::unordered_map<void*, Uploaded> g_cache;

int check_workspace(void* ws, size_t bytes, const Plan& plan)
{
    if (!ws) return fail(MPS_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MPS_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (bytes < plan.total_bytes) {
        return fail(MPS_ERR_WORKSPACE, "workspace too small: %zu bytes, need %zu", bytes, plan.total_bytes);
    }
    return MPS_OK;
}

// Move the uploads whose copies have finished to the idle buffers, oldest
// first, without waiting: the first one still running stops the scan.
int reap_uploads(Uploaded& u)
{
    while (!u.in_flight.empty()) {
        const hipError_t e = hipEventQuery(u.in_flight.front().done);
        if (e == hipErrorNotReady) break;
        if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "hipEventQuery: %s", hipGetErrorString(e));
        u.idle.push_back(u.in_flight.front());
        u.in_flight.pop_front();
    }
    return MPS_OK;
}

// An idle buffer of at least `bytes` (the smallest that fits), or a new one.
int staging_buffer(Uploaded& u, size_t bytes, Staging& out)
{
    size_t best = u.idle.size();
    for (size_t i = 0; i < u.idle.size(); ++i) {
        if (u.idle[i].capacity >= bytes &&
            (best == u.idle.size() || u.idle[i].capacity < u.idle[best].capacity)) {
            best = i;
        }
    }
    if (best < u.idle.size()) {
        out = u.idle[best];
        u.idle.erase(u.idle.begin() + static_cast<std::ptrdiff_t>(best));
        return MPS_OK;
    }
    Staging s;
    s.capacity = std::max<size_t>(4096, round_up(bytes, 4096));
    hipError_t e = hipHostMalloc(&s.host, s.capacity, hipHostMallocDefault);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "hipHostMalloc (table staging): %s", hipGetErrorString(e));
    e = hipEventCreateWithFlags(&s.done, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipHostFree(s.host);
        return fail(MPS_ERR_DEVICE, "hipEventCreate: %s", hipGetErrorString(e));
    }
    out = s;
    return MPS_OK;
}

// Make the workspace hold `plan`'s tables (stream-ordered), uploading them
// only when the workspace last received different ones.  Never waits for
// the device: the image goes through a pinned buffer, which is reused only
// after its copy's event has completed.  `allocate` false: no staging buffer
// is allocated; the copy then comes from the plan's own (pageable) image,
// which the runtime copies synchronously, so the image may go right after.
int ensure_uploaded(void* ws, Plan& plan, hipStream_t stream, bool allocate)
{
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    Uploaded& u = g_cache[ws];
    if (u.tag == plan.tag) return MPS_OK;
    if (!allocate) {
        u.tag = 0;
        u.key.clear();
        const hipError_t e =
            hipMemcpyAsync(ws, plan.image.data(), plan.image.size(), hipMemcpyHostToDevice, stream);
        if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "table upload: %s", hipGetErrorString(e));
        u.tag = plan.tag;
        return MPS_OK;
    }
    int rc = reap_uploads(u);
    if (rc) return rc;
    Staging buf;
    if ((rc = staging_buffer(u, plan.image.size(), buf))) return rc;
    u.tag = 0;
    u.key.clear();  // until this upload is enqueued, no plan matches the workspace
    std::memcpy(buf.host, plan.image.data(), plan.image.size());
    hipError_t e = hipMemcpyAsync(ws, buf.host, plan.image.size(), hipMemcpyHostToDevice, stream);
    if (e == hipSuccess) e = hipEventRecord(buf.done, stream);
    if (e != hipSuccess) {
        // The copy may have been enqueued: keep the buffer until its event
        // (recorded or not) reports completion.
        u.in_flight.push_back(buf);
        return fail(MPS_ERR_DEVICE, "table upload: %s", hipGetErrorString(e));
    }
    u.in_flight.push_back(buf);
    u.tag = plan.tag;
    return MPS_OK;
}

// Release every buffer of a workspace's uploads (waits for running copies).
void release_uploads(Uploaded& u)
{
    for (Staging& s : u.in_flight) {
        (void)hipEventSynchronize(s.done);
        u.idle.push_back(s);
    }
    u.in_flight.clear();
    for (Staging& s : u.idle) {
        (void)hipEventDestroy(s.done);
        (void)hipHostFree(s.host);
    }
    u.idle.clear();
}

int plan_list(const mps_tensor* t, int n, int grad_dtype, bool need_state, Plan& plan)
{
    return build_plan(t, n, grad_dtype, need_state, plan);
}

int plan_list(const mps_tensor8* t, int n, int grad_dtype, bool need_state, Plan& plan)
{
    return build_plan8(t, n, grad_dtype, need_state, plan);
}

// The key of a call: record size and gradient dtype, then the caller's
// tensor array byte for byte.
template <class Tensor>
bool same_key(const std::vector<unsigned char>& key, const Tensor* tensors, int n, int grad_dtype)
{
    const size_t bytes = sizeof(Tensor) * static_cast<size_t>(n);
    return key.size() == bytes + 2 && key[0] == static_cast<unsigned char>(sizeof(Tensor)) &&
           key[1] == static_cast<unsigned char>(grad_dtype) &&
           std::memcmp(key.data() + 2, tensors, bytes) == 0;
}

template <class Tensor>
void set_key(std::vector<unsigned char>& key, const Tensor* tensors, int n, int grad_dtype)
{
    const auto* raw = reinterpret_cast<const unsigned char*>(tensors);
    key.assign(2 + sizeof(Tensor) * static_cast<size_t>(n), 0);
    key[0] = static_cast<unsigned char>(sizeof(Tensor));
    key[1] = static_cast<unsigned char>(grad_dtype);
    std::memcpy(key.data() + 2, raw, sizeof(Tensor) * static_cast<size_t>(n));
}

// The plan of a call, with its tables in the workspace.  When the workspace
// was last planned for this very list (same kind, gradient dtype and tensor
// array, byte for byte, and the state pointers checked if this call needs
// them), that plan is reused: validating, chunking and hashing a list costs
// the host 7 us for one tensor and 0.4 ms for 1137 (3 ms for the 8B-parameter
// list of 291 tensors, 490K chunks), on every call.  The reuse compares in
// place and allocates nothing.  Otherwise the list is validated, planned
// and, if its tables differ from the workspace's, uploaded.  The device
// still compares the table tag, so a workspace written behind the library's
// back is never trusted.
template <class Tensor>
int prepare(const Tensor* tensors, int n, int grad_dtype, bool need_state, void* ws,
            size_t ws_bytes, hipStream_t stream, Plan& plan, bool allocate = true)
{
    if (tensors && n > 0) {
        std::lock_guard<std::mutex> lock(g_cache_mutex);
        auto it = g_cache.find(ws);
        if (it != g_cache.end() && it->second.tag != 0 &&
            same_key(it->second.key, tensors, n, grad_dtype) &&
            (!need_state || it->second.state_checked)) {
            plan = it->second.meta;
            return check_workspace(ws, ws_bytes, plan);
        }
    }
    int rc = plan_list(tensors, n, grad_dtype, need_state, plan);
    if (rc) return rc;
    if ((rc = check_workspace(ws, ws_bytes, plan))) return rc;
    if ((rc = ensure_uploaded(ws, plan, stream, allocate))) return rc;
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    Uploaded& u = g_cache[ws];
    set_key(u.key, tensors, n, grad_dtype);
    u.state_checked = need_state;
    u.meta = plan;
    u.meta.image.clear();
    u.meta.image.shrink_to_fit();
    return MPS_OK;
}

mps::WorkspaceView view_of(void* ws, const Plan& plan)
{
    unsigned char* base = static_cast<unsigned char*>(ws);
    mps::WorkspaceView v;
    v.header = reinterpret_cast<WorkspaceHeader*>(base);
    v.tensors = reinterpret_cast<const TensorEntry*>(base + plan.tensors_off);
    v.chunk_map = reinterpret_cast<const uint32_t*>(base + plan.chunks_off);
    v.tickets = reinterpret_cast<uint32_t*>(base + plan.tickets_off);
    v.partials = reinterpret_cast<double*>(base + plan.partials_off);
    v.n_tensors = plan.n_tensors;
    v.n_chunks = plan.n_chunks;
    v.solo_tensor = plan.solo_tensor;
    v.solo = plan.solo;
    v.solo_quant = plan.solo_quant;
    v.chunk_elems = plan.chunk_elems;
    v.tag = plan.tag;
    return v;
}

// The optional inputs of the update: the caller's pointer, or the
// workspace constant that stands for "absent" (coefficient 1, never skip).
const float* coef_or_one(const float* d_coef, void* ws, const Plan& plan)
{
    return d_coef ? d_coef
                  : &reinterpret_cast<const mps::WorkspaceConstants*>(
                         static_cast<unsigned char*>(ws) + plan.constants_off)->one;
}

const double* skip_or_zero(const double* d_skip, void* ws, const Plan& plan)
{
    return d_skip ? d_skip
                  : &reinterpret_cast<const mps::WorkspaceConstants*>(
                         static_cast<unsigned char*>(ws) + plan.constants_off)->zero;
}

// At most `cap` blocks, every block taking the same number of chunks (the
// last one possibly fewer): ceil(n / ceil(n / cap)).
int grid_for(int n_chunks, int cap)
{
    if (n_chunks < 1) return 1;
    const int per_block = (n_chunks + cap - 1) / cap;
    return (n_chunks + per_block - 1) / per_block;
}

// The fp32-state update's grid: for a whole-model list at most
// kLargeMaxBlocks; for a shard one block per chunk up to kStepSpreadChunks
// chunks (its step is bound by latency: the fewer chunks one block walks in
// turn, the shorter), else at most one block per CU.  Every block walks the
// same number of chunks but the last.
int step_grid(const Plan& plan)
{
    const int n_chunks = plan.n_chunks;
    if (plan.large) return grid_for(n_chunks, mps::kLargeMaxBlocks);
    return n_chunks <= mps::kStepSpreadChunks ? std::max(n_chunks, 1)
                                              : grid_for(n_chunks, mps::kStepMaxBlocks);
}

bool finite_in(double x, double lo, double hi_exclusive)
{
    return std::isfinite(x) && x >= lo && x < hi_exclusive;
}

int check_hyperparameters(double lr, double beta1, double beta2, double eps, double weight_decay)
{
    if (!(std::isfinite(lr) && lr >= 0.0)) return fail(MPS_ERR_INVALID_ARGUMENT, "lr must be finite and >= 0");
    if (!finite_in(beta1, 0.0, 1.0)) return fail(MPS_ERR_INVALID_ARGUMENT, "beta1 must be in [0, 1)");
    if (!finite_in(beta2, 0.0, 1.0)) return fail(MPS_ERR_INVALID_ARGUMENT, "beta2 must be in [0, 1)");
    if (!(std::isfinite(eps) && eps >= 0.0)) return fail(MPS_ERR_INVALID_ARGUMENT, "eps must be finite and >= 0");
    if (!(std::isfinite(weight_decay) && weight_decay >= 0.0)) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "weight_decay must be finite and >= 0");
    }
    return MPS_OK;
}

int check_clip_arguments(double max_norm, double grad_scale)
{
    if (!(std::isfinite(max_norm) && max_norm > 0.0)) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "max_norm must be finite and > 0");
    }
    if (!(std::isfinite(grad_scale) && grad_scale > 0.0)) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "grad_scale must be finite and > 0");
    }
    return MPS_OK;
}

// How many leading blocks of a norm grid read their gradients with the
// default cache policy: as many whole block runs (the longest run, for a
// bound) as fit the cache budget.  Those gradients are still in the
// Infinity Cache when the update reads them again; the other blocks stream
// theirs nontemporally, which is faster and leaves the cache to the first.
// A list within the budget is read the default way throughout.
int norm_cached_blocks(const Plan& plan, bool bf16, int grid)
{
    const int64_t run_chunks = (static_cast<int64_t>(plan.n_chunks) + grid - 1) / grid;
    const int64_t run_bytes = run_chunks * plan.chunk_elems * (bf16 ? 2 : 4);
    if (run_bytes <= 0) return grid;
    return static_cast<int>(std::min<int64_t>(grid, mps::kNormCacheBudget / run_bytes));
}

// Rounds of the single-launch step's bounded barrier wait: 0 (the kernel's
// default, about 1 s) unless MPS_FUSED_SPIN_LIMIT holds a positive number.
// That variable is a test hook: a tiny limit makes waiters give the launch
// up, so the failure path runs while every block still ends normally.
uint32_t fused_spin_limit()
{
    const char* v = std::getenv("MPS_FUSED_SPIN_LIMIT");
    if (!v || !*v) return 0;
    const unsigned long x = std::strtoul(v, nullptr, 10);
    return x > 0 && x < 0xFFFFFFFFul ? static_cast<uint32_t>(x) : 0;
}

// Launch the norm (and optionally the clip coefficient) over a planned list.
int run_grad_norm(const Plan& plan, bool bf16, double* d_sumsq, double max_norm,
                  double grad_scale, float* d_coef, void* d_workspace, hipStream_t st)
{
    const int grid = grid_for(plan.n_chunks, mps::kNormMaxBlocks);
    hipError_t e = mps::launch_grad_norm(view_of(d_workspace, plan), bf16, grid,
                                         norm_cached_blocks(plan, bf16, grid), d_sumsq, max_norm,
                                         grad_scale, d_coef, st);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "grad_norm launch: %s", hipGetErrorString(e));
    return ok();
}

int check_clipped_arguments(const int32_t* d_step, double max_norm, double grad_scale, double lr,
                            double beta1, double beta2, double eps, double weight_decay)
{
    if (!d_step) return fail(MPS_ERR_INVALID_ARGUMENT, "d_step is NULL");
    int rc = check_clip_arguments(max_norm, grad_scale);
    if (!rc) rc = check_hyperparameters(lr, beta1, beta2, eps, weight_decay);
    return rc;
}

// The clipped step's two launches over a planned list: the norm's partial
// sums (and the step number) into the workspace, the optional event, then
// `update(view, norm grid, stream)`, which finishes the sum.
template <class Update>
int run_clipped(const Plan& plan, bool bf16, const int32_t* d_step, void* d_workspace,
                hipStream_t st, void* mid_event, Update update)
{
    const mps::WorkspaceView ws = view_of(d_workspace, plan);
    // The same norm grid as grad_norm_sq, so the partials and S match it.
    const int norm_grid = grid_for(plan.n_chunks, mps::kNormMaxBlocks);
    hipError_t e = mps::launch_grad_norm_partials(ws, bf16, norm_grid,
                                                  norm_cached_blocks(plan, bf16, norm_grid), d_step,
                                                  st);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "grad_norm launch: %s", hipGetErrorString(e));
    if (mid_event && (e = hipEventRecord(static_cast<hipEvent_t>(mid_event), st)) != hipSuccess) {
        return fail(MPS_ERR_DEVICE, "hipEventRecord (mid_event): %s", hipGetErrorString(e));
    }
    if ((e = update(ws, norm_grid, st)) != hipSuccess) {
        return fail(MPS_ERR_DEVICE, "clipped update launch: %s", hipGetErrorString(e));
    }
    return ok();
}

// The clipped step on a prepared workspace (the caller's or the library's).
int clipped_step_on(const Plan& plan, mps_dtype grad_dtype, double max_norm, double grad_scale,
                    int skip_if_nonfinite, double* d_sumsq, float* d_coef, int32_t* d_step,
                    double lr, double beta1, double beta2, double eps, double weight_decay,
                    void* d_workspace, hipStream_t stream_, void* mid_event)
{
    const bool bf16 = grad_dtype == MPS_DTYPE_BF16;
    const mps::HyperParams hp{lr, beta1, beta2, eps, weight_decay};
    const int grid = step_grid(plan);
    return run_clipped(plan, bf16, d_step, d_workspace, stream_, mid_event,
                       [&](const mps::WorkspaceView& ws, int norm_grid, hipStream_t st) {
                           return mps::launch_clipped_step(ws, bf16, plan.large, grid, norm_grid,
                                                           max_norm, grad_scale,
                                                           skip_if_nonfinite ? 1 : 0, d_sumsq,
                                                           d_coef, d_step, hp, st);
                       });
}

}  // namespace

extern "C" {

size_t adamw_workspace_bytes(const mps_tensor* tensors, int n_tensors)
{
    Plan plan;
    // The table size does not depend on the gradient dtype; validate with the
    // weaker (bf16, 2-byte) alignment so that either dtype is accepted here.
    if (build_plan(tensors, n_tensors, MPS_DTYPE_BF16, false, plan) != MPS_OK) return 0;
    ok();
    return plan.total_bytes;
}

int adamw_workspace_release(void* d_workspace)
{
    std::lock_guard<std::mutex> lock(g_cache_mutex);
    auto it = g_cache.find(d_workspace);
    if (it != g_cache.end()) {
        release_uploads(it->second);
        g_cache.erase(it);
    }
    return ok();
}

int grad_norm_sq(const mps_tensor* tensors, int n_tensors, mps_dtype grad_dtype, double* d_sumsq,
                 double max_norm, double grad_scale, float* d_coef, void* d_workspace,
                 size_t workspace_bytes, void* stream)
{
    if (!d_sumsq) return fail(MPS_ERR_INVALID_ARGUMENT, "d_sumsq is NULL");
    int rc = d_coef ? check_clip_arguments(max_norm, grad_scale) : MPS_OK;
    if (rc) return rc;
    Plan plan;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, false, d_workspace, workspace_bytes, st,
                      plan))) {
        return rc;
    }
    return run_grad_norm(plan, grad_dtype == MPS_DTYPE_BF16, d_sumsq, max_norm, grad_scale, d_coef,
                         d_workspace, st);
}

int clip_coef(const double* d_sumsq, double max_norm, double grad_scale, float* d_coef,
              void* stream)
{
    if (!d_sumsq || !d_coef) return fail(MPS_ERR_INVALID_ARGUMENT, "d_sumsq / d_coef is NULL");
    if (int rc = check_clip_arguments(max_norm, grad_scale)) return rc;
    hipError_t e = mps::launch_clip_coef(d_sumsq, max_norm, grad_scale, d_coef,
                                         static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "clip_coef launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw_multi_tensor_step(const mps_tensor* tensors, int n_tensors, mps_dtype grad_dtype,
                            const float* d_coef, const double* d_skip_if_nonfinite,
                            int32_t* d_step, double lr, double beta1, double beta2, double eps,
                            double weight_decay, void* d_workspace, size_t workspace_bytes,
                            void* stream)
{
    if (!d_step) return fail(MPS_ERR_INVALID_ARGUMENT, "d_step is NULL");
    int rc = check_hyperparameters(lr, beta1, beta2, eps, weight_decay);
    if (rc) return rc;
    Plan plan;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, true, d_workspace, workspace_bytes, st,
                      plan))) {
        return rc;
    }
    mps::HyperParams hp{lr, beta1, beta2, eps, weight_decay};
    const int grid = step_grid(plan);
    hipError_t e = mps::launch_adamw_step(
        view_of(d_workspace, plan), grad_dtype == MPS_DTYPE_BF16, plan.large, grid,
        coef_or_one(d_coef, d_workspace, plan),
        skip_or_zero(d_skip_if_nonfinite, d_workspace, plan), d_step, hp, st);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "adamw_step launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw_fused_step(const mps_tensor* tensors, int n_tensors, mps_dtype grad_dtype,
                     double max_norm, double grad_scale, int skip_if_nonfinite, double* d_sumsq,
                     float* d_coef, int32_t* d_step, double lr, double beta1, double beta2,
                     double eps, double weight_decay, void* d_workspace, size_t workspace_bytes,
                     void* stream)
{
    int rc = check_clipped_arguments(d_step, max_norm, grad_scale, lr, beta1, beta2, eps,
                                     weight_decay);
    if (rc) return rc;
    Plan plan;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, true, d_workspace, workspace_bytes, st,
                      plan))) {
        return rc;
    }
    const bool bf16 = grad_dtype == MPS_DTYPE_BF16;
    int resident = 0;
    hipError_t e = mps::fused_grid_limit(bf16, &resident);
    if (e != hipSuccess || resident < 1) {
        return fail(MPS_ERR_DEVICE, "fused step occupancy query: %s", hipGetErrorString(e));
    }
    const int cap = resident < mps::kFusedMaxBlocks ? resident : mps::kFusedMaxBlocks;
    const int grid = grid_for(plan.n_chunks, cap);
    mps::HyperParams hp{lr, beta1, beta2, eps, weight_decay};
    e = mps::launch_fused_step(view_of(d_workspace, plan), bf16, grid,
                               norm_cached_blocks(plan, bf16, grid), max_norm, grad_scale,
                               skip_if_nonfinite ? 1 : 0, d_sumsq, d_coef, d_step, hp,
                               fused_spin_limit(), st);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "fused step launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw_fused_status(void* d_workspace, size_t workspace_bytes, uint32_t* d_error, void* stream)
{
    if (!d_error) return fail(MPS_ERR_INVALID_ARGUMENT, "d_error is NULL");
    if (!d_workspace) return fail(MPS_ERR_WORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(d_workspace) % 256) {
        return fail(MPS_ERR_WORKSPACE, "workspace not 256-byte aligned");
    }
    if (workspace_bytes < sizeof(WorkspaceHeader)) {
        return fail(MPS_ERR_WORKSPACE, "workspace too small: %zu bytes", workspace_bytes);
    }
    hipError_t e = mps::launch_fused_status(static_cast<WorkspaceHeader*>(d_workspace), d_error,
                                            static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "fused status launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw_clipped_step(const mps_tensor* tensors, int n_tensors, mps_dtype grad_dtype,
                       double max_norm, double grad_scale, int skip_if_nonfinite, double* d_sumsq,
                       float* d_coef, int32_t* d_step, double lr, double beta1, double beta2,
                       double eps, double weight_decay, void* d_workspace, size_t workspace_bytes,
                       void* stream, void* mid_event)
{
    int rc = check_clipped_arguments(d_step, max_norm, grad_scale, lr, beta1, beta2, eps,
                                     weight_decay);
    if (rc) return rc;
    Plan plan;
    hipStream_t stream_ = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, true, d_workspace, workspace_bytes, stream_,
                      plan))) {
        return rc;
    }
    return clipped_step_on(plan, grad_dtype, max_norm, grad_scale, skip_if_nonfinite, d_sumsq,
                           d_coef, d_step, lr, beta1, beta2, eps, weight_decay, d_workspace,
                           stream_, mid_event);
}

int adamw_clipped_step_noalloc(const mps_tensor* tensors, int n_tensors, mps_dtype grad_dtype,
                               double max_norm, double grad_scale, int skip_if_nonfinite,
                               double* d_sumsq, float* d_coef, int32_t* d_step, double lr,
                               double beta1, double beta2, double eps, double weight_decay,
                               void* stream, void* mid_event)
{
    int rc = check_clipped_arguments(d_step, max_norm, grad_scale, lr, beta1, beta2, eps,
                                     weight_decay);
    if (rc) return rc;
    int device = -1;
    hipError_t e = hipGetDevice(&device);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    void* scratch = nullptr;
    if ((e = mps::scratch_address(device, &scratch)) != hipSuccess) {
        return fail(MPS_ERR_DEVICE, "library workspace of device %d: %s", device,
                    hipGetErrorString(e));
    }
    Plan plan;
    hipStream_t stream_ = static_cast<hipStream_t>(stream);
    rc = prepare(tensors, n_tensors, grad_dtype, true, scratch, mps::kScratchBytes, stream_, plan,
                 /*allocate=*/false);
    if (rc == MPS_ERR_WORKSPACE) {
        return fail(MPS_ERR_WORKSPACE,
                    "the list needs %zu bytes of workspace, more than the library's %zu "
                    "(use adamw_clipped_step with a workspace of your own)",
                    plan.total_bytes, mps::kScratchBytes);
    }
    if (rc) return rc;
    return clipped_step_on(plan, grad_dtype, max_norm, grad_scale, skip_if_nonfinite, d_sumsq,
                           d_coef, d_step, lr, beta1, beta2, eps, weight_decay, scratch, stream_,
                           mid_event);
}

size_t adamw8_workspace_bytes(const mps_tensor8* tensors, int n_tensors)
{
    Plan plan;
    if (build_plan8(tensors, n_tensors, MPS_DTYPE_BF16, false, plan) != MPS_OK) return 0;
    ok();
    return plan.total_bytes;
}

int adamw8_grad_norm_sq(const mps_tensor8* tensors, int n_tensors, mps_dtype grad_dtype,
                        double* d_sumsq, double max_norm, double grad_scale, float* d_coef,
                        void* d_workspace, size_t workspace_bytes, void* stream)
{
    if (!d_sumsq) return fail(MPS_ERR_INVALID_ARGUMENT, "d_sumsq is NULL");
    int rc = d_coef ? check_clip_arguments(max_norm, grad_scale) : MPS_OK;
    if (rc) return rc;
    Plan plan;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, false, d_workspace, workspace_bytes, st,
                      plan))) {
        return rc;
    }
    return run_grad_norm(plan, grad_dtype == MPS_DTYPE_BF16, d_sumsq, max_norm, grad_scale, d_coef,
                         d_workspace, st);
}

int adamw8_multi_tensor_step(const mps_tensor8* tensors, int n_tensors, mps_dtype grad_dtype,
                             const float* d_coef, const double* d_skip_if_nonfinite,
                             int32_t* d_step, double lr, double beta1, double beta2, double eps,
                             double weight_decay, void* d_workspace, size_t workspace_bytes,
                             void* stream)
{
    if (!d_step) return fail(MPS_ERR_INVALID_ARGUMENT, "d_step is NULL");
    int rc = check_hyperparameters(lr, beta1, beta2, eps, weight_decay);
    if (rc) return rc;
    Plan plan;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, true, d_workspace, workspace_bytes, st,
                      plan))) {
        return rc;
    }
    mps::HyperParams hp{lr, beta1, beta2, eps, weight_decay};
    const int grid = grid_for(plan.n_chunks, mps::kQ8MaxBlocks);
    const auto* quant = reinterpret_cast<const mps::QuantEntry*>(static_cast<unsigned char*>(d_workspace) +
                                                                 plan.quant_off);
    hipError_t e = mps::launch_adamw8_step(
        view_of(d_workspace, plan), quant, grad_dtype == MPS_DTYPE_BF16, grid,
        coef_or_one(d_coef, d_workspace, plan),
        skip_or_zero(d_skip_if_nonfinite, d_workspace, plan), d_step, hp, st);
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "adamw8_step launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw8_clipped_step(const mps_tensor8* tensors, int n_tensors, mps_dtype grad_dtype,
                        double max_norm, double grad_scale, int skip_if_nonfinite, double* d_sumsq,
                        float* d_coef, int32_t* d_step, double lr, double beta1, double beta2,
                        double eps, double weight_decay, void* d_workspace,
                        size_t workspace_bytes, void* stream, void* mid_event)
{
    int rc = check_clipped_arguments(d_step, max_norm, grad_scale, lr, beta1, beta2, eps,
                                     weight_decay);
    if (rc) return rc;
    Plan plan;
    hipStream_t stream_ = static_cast<hipStream_t>(stream);
    if ((rc = prepare(tensors, n_tensors, grad_dtype, true, d_workspace, workspace_bytes, stream_,
                      plan))) {
        return rc;
    }
    const bool bf16 = grad_dtype == MPS_DTYPE_BF16;
    const mps::HyperParams hp{lr, beta1, beta2, eps, weight_decay};
    const int grid = grid_for(plan.n_chunks, mps::kQ8MaxBlocks);
    const auto* quant = reinterpret_cast<const mps::QuantEntry*>(static_cast<unsigned char*>(d_workspace) +
                                                                 plan.quant_off);
    return run_clipped(plan, bf16, d_step, d_workspace, stream_, mid_event,
                       [&](const mps::WorkspaceView& ws, int norm_grid, hipStream_t st) {
                           return mps::launch_adamw8_clipped(ws, quant, bf16, grid, norm_grid,
                                                             max_norm, grad_scale,
                                                             skip_if_nonfinite ? 1 : 0, d_sumsq,
                                                             d_coef, d_step, hp, st);
                       });
}

int adamw8_quantize(const float* d_x, int64_t n, mps_q8_format format, uint8_t* d_codes,
                    uint8_t* d_scales, void* stream)
{
    if (n < 0) return fail(MPS_ERR_INVALID_ARGUMENT, "n < 0");
    if (format != MPS_Q8_E4M3 && format != MPS_Q8_E5M2) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "unknown 8-bit format %d", static_cast<int>(format));
    }
    if (n == 0) return ok();
    if (!d_x || !d_codes || !d_scales) return fail(MPS_ERR_INVALID_ARGUMENT, "NULL pointer");
    hipError_t e = mps::launch_quantize(d_x, n, format == MPS_Q8_E4M3, d_codes, d_scales,
                                        static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "quantize launch: %s", hipGetErrorString(e));
    return ok();
}

int adamw8_dequantize(const uint8_t* d_codes, const uint8_t* d_scales, int64_t n,
                      mps_q8_format format, float* d_x, void* stream)
{
    if (n < 0) return fail(MPS_ERR_INVALID_ARGUMENT, "n < 0");
    if (format != MPS_Q8_E4M3 && format != MPS_Q8_E5M2) {
        return fail(MPS_ERR_INVALID_ARGUMENT, "unknown 8-bit format %d", static_cast<int>(format));
    }
    if (n == 0) return ok();
    if (!d_x || !d_codes || !d_scales) return fail(MPS_ERR_INVALID_ARGUMENT, "NULL pointer");
    hipError_t e = mps::launch_dequantize(d_codes, d_scales, n, format == MPS_Q8_E4M3, d_x,
                                          static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(MPS_ERR_DEVICE, "dequantize launch: %s", hipGetErrorString(e));
    return ok();
}

const char* adamw_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
