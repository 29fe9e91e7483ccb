// Host side of the C ABI declared in include/pw.h: argument validation, the
// weight page table (device array of BlockDesc, host mirror), the device slab
// pool for planes and LUTs, pinned host masters, committed-width changes with
// asynchronous host->device plane movement, and kernel launches.
//
// PagedWeight pages, "Technical summary: PagedWeight", Core components 1
// (weight page table tracking each linear block's committed width; pages
// resident on the GPU, on the CPU or in transfer) and 3 (asynchronous page
// movement, widths committed only at safe boundaries).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <condition_variable>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <thread>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "../../include/pw.h"
#include "pw_internal.h"

using namespace pw;

namespace {

thread_local std::string g_err;

pw_status fail(pw_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pw_status fail(pw_status st, const char* fmt, ...)
{
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return st;
}

pw_status hip_fail(hipError_t e, const char* what)
{
    return fail(PW_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}


// Entry points return statuses, never exceptions: a C++ exception (host
// memory exhausted in a container, a thread that cannot start) becomes OOM or
// INVALID with a message instead of unwinding into a C caller.
template <class F>
pw_status guarded(const char* fn, F&& body)
{
    try {
        return body();
    } catch (const std::bad_alloc&) {
        return fail(PW_ERR_OOM, "%s: host memory exhausted", fn);
    } catch (const std::exception& e) {
        return fail(PW_ERR_INVALID, "%s: %s", fn, e.what());
    } catch (...) {
        return fail(PW_ERR_INVALID, "%s: unexpected exception", fn);
    }
}

pw_status ok()
{
    g_err.clear();
    return PW_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }

// Events recorded behind library work (copies of a width change, page-table
// updates), recycled once no one needs them any more: each holder takes a
// reference, and an event whose last reference is dropped goes back to the
// free list (a later hipEventRecord re-arms it; waits already enqueued on its
// earlier record are not affected).
class EventPool {
public:
    ~EventPool() { clear(); }

    hipError_t acquire(hipEvent_t* ev)
    {
        if (!free_.empty()) {
            *ev = free_.back();
            free_.pop_back();
        } else {
            hipError_t e = hipEventCreateWithFlags(ev, hipEventDisableTiming);
            if (e != hipSuccess) return e;
            ++created_;
        }
        refs_[*ev] = 0;
        return hipSuccess;
    }

    void hold(hipEvent_t ev) { ++refs_[ev]; }

    // drops one reference; an event with none left is free again
    void drop(hipEvent_t ev)
    {
        auto it = refs_.find(ev);
        if (it == refs_.end()) return;
        if (--it->second <= 0) {
            refs_.erase(it);
            free_.push_back(ev);
        }
    }

    size_t created() const { return created_; }
    size_t in_use() const { return refs_.size(); }

    void clear()
    {
        for (auto ev : free_) (void)hipEventDestroy(ev);
        for (auto& kv : refs_) (void)hipEventDestroy(kv.first);
        free_.clear();
        refs_.clear();
        created_ = 0;
    }

private:
    std::vector<hipEvent_t> free_;
    std::unordered_map<hipEvent_t, int> refs_;
    size_t created_ = 0;
};

// Device slabs for planes and LUTs.  Slabs are carved from chunks of about
// kChunkBytes, one chunk per class (slab size, plane index or LUT): a device
// allocation (hipMalloc) stalls the kernels running on the device for tens
// of microseconds, so a width change of hundreds of blocks must not make one
// per slab.  A released slab goes back to its class's free list, but only
// after an event recorded behind the last work that may read it (the pool
// holds a reference on that event until then).  trim() returns the chunks
// whose slabs are all free to the device (dropping plane p of many blocks
// frees whole plane-p chunks).
class SlabPool {
public:
    static constexpr size_t kChunkBytes = (size_t)32 << 20;
    static constexpr int kLutTag = 8;  // class tag of LUT slabs (planes use their index 0..7)

    explicit SlabPool(EventPool* evs) : evs_(evs) {}
    ~SlabPool() { clear(); }

    hipError_t alloc(size_t bytes, int tag, void** out)
    {
        bytes = round(bytes);
        reclaim();
        const uint64_t key = cls(bytes, tag);
        auto it = free_.find(key);
        if (it != free_.end() && !it->second.empty()) {
            *out = it->second.back();
            it->second.pop_back();
            chunk_of(*out).live++;
            free_bytes_ -= bytes;
            resident_ += bytes;
            return hipSuccess;
        }
        auto op = open_.find(key);
        if (op == open_.end()) {
            int n = (int)std::max<size_t>(1, std::min<size_t>(64, kChunkBytes / bytes));
            void* base = nullptr;
            hipError_t e = hipMalloc(&base, (size_t)n * bytes);
            if (e != hipSuccess && n > 1) {
                (void)hipGetLastError();
                n = 1;
                e = hipMalloc(&base, bytes);
            }
            if (e != hipSuccess) {
                (void)hipGetLastError();
                return e;
            }
            ++device_allocs_;
            held_ += (size_t)n * bytes;
            chunks_[(char*)base] = Chunk{key, bytes, n, 0, 0};
            op = open_.emplace(key, (char*)base).first;
        }
        Chunk& ch = chunks_[op->second];
        *out = op->second + (size_t)ch.carved * bytes;
        ch.carved++;
        ch.live++;
        if (ch.carved == ch.n) open_.erase(op);
        resident_ += bytes;
        return hipSuccess;
    }

    void release_now(void* p, size_t bytes, int tag)
    {
        if (!p) return;
        bytes = round(bytes);
        free_[cls(bytes, tag)].push_back(p);
        chunk_of(p).live--;
        free_bytes_ += bytes;
        resident_ -= bytes;
    }

    void release_after(void* p, size_t bytes, int tag, hipEvent_t ev)
    {
        if (!p) return;
        bytes = round(bytes);
        evs_->hold(ev);
        pending_.push_back({p, bytes, cls(bytes, tag), ev});
        resident_ -= bytes;
    }

    void reclaim()
    {
        size_t w = 0;
        for (size_t i = 0; i < pending_.size(); ++i) {
            if (hipEventQuery(pending_[i].ev) == hipSuccess) {
                free_[pending_[i].key].push_back(pending_[i].p);
                chunk_of(pending_[i].p).live--;
                free_bytes_ += pending_[i].bytes;
                evs_->drop(pending_[i].ev);
            } else {
                pending_[w++] = pending_[i];
            }
        }
        pending_.resize(w);
    }

    // hipFree every chunk none of whose slabs is in use or waiting; returns
    // the bytes given back to the device
    size_t trim()
    {
        reclaim();
        size_t freed = 0;
        for (auto it = chunks_.begin(); it != chunks_.end();) {
            Chunk& ch = it->second;
            if (ch.live != 0) {
                ++it;
                continue;
            }
            char* base = it->first;
            char* end = base + (size_t)ch.n * ch.slab;
            auto& fl = free_[ch.key];
            const size_t before = fl.size();
            fl.erase(std::remove_if(fl.begin(), fl.end(), [&](void* q) { return (char*)q >= base && (char*)q < end; }),
                     fl.end());
            free_bytes_ -= (before - fl.size()) * ch.slab;
            auto op = open_.find(ch.key);
            if (op != open_.end() && op->second == base) open_.erase(op);
            (void)hipFree(base);
            held_ -= (size_t)ch.n * ch.slab;
            freed += (size_t)ch.n * ch.slab;
            it = chunks_.erase(it);
        }
        return freed;
    }

    int64_t resident() const { return (int64_t)resident_; }
    int64_t free_bytes() const { return (int64_t)free_bytes_; }
    int64_t held() const { return (int64_t)held_; }
    int64_t device_allocs() const { return (int64_t)device_allocs_; }
    int64_t waiting_bytes() const
    {
        size_t b = 0;
        for (const auto& p : pending_) b += p.bytes;
        return (int64_t)b;
    }

    void clear()
    {
        for (auto& kv : chunks_) (void)hipFree(kv.first);
        chunks_.clear();
        open_.clear();
        free_.clear();
        pending_.clear();
        resident_ = 0;
        free_bytes_ = 0;
        held_ = 0;
    }

private:
    static size_t round(size_t b) { return (b + 255) & ~size_t(255); }
    static uint64_t cls(size_t bytes, int tag) { return ((uint64_t)bytes << 4) | (uint64_t)tag; }
    struct Chunk {
        uint64_t key;
        size_t slab;
        int n, carved, live;  // slabs in the chunk, carved so far, in use or waiting
    };
    struct Pending {
        void* p;
        size_t bytes;
        uint64_t key;
        hipEvent_t ev;
    };
    Chunk& chunk_of(void* p)
    {
        auto it = chunks_.upper_bound((char*)p);
        --it;  // every slab lies in a chunk
        return it->second;
    }
    EventPool* evs_;
    std::map<char*, Chunk> chunks_;                           // by base address
    std::unordered_map<uint64_t, char*> open_;                // class -> chunk with uncarved slabs
    std::unordered_map<uint64_t, std::vector<void*>> free_;   // class -> free slabs
    std::vector<Pending> pending_;
    size_t resident_ = 0, free_bytes_ = 0, held_ = 0, device_allocs_ = 0;
};

struct HostBlock {
    bool registered = false;
    int R = 0, K = 0, q = 0;
    int S = 0;       // LUT slots
    int64_t pw = 0;  // words per plane
    void* dplanes[8] = {};
    void* dlut = nullptr;
    uint32_t* hplanes = nullptr;  // pinned master: 8 planes
    uint32_t* hluts = nullptr;    // pinned master: LUT_3..LUT_8, each in the device slot layout
    // the masters' device-side addresses (read by the blocking path's copy kernel), or null
    const uint32_t* dv_hplanes = nullptr;
    const uint32_t* dv_hluts = nullptr;
};

// A small persistent gang of host threads for the gather copies of width
// changes: run(fn) calls fn(m, n) on every member m < n (the caller is member
// 0) and returns once all have finished.  Members that cannot be started
// leave a smaller gang.
class Gang {
public:
    explicit Gang(int n)
    {
        for (int i = 1; i < n; ++i) {
            try {
                th_.emplace_back([this, i] { loop(i); });
            } catch (...) {
                break;
            }
        }
        n_ = 1 + (int)th_.size();
    }
    ~Gang()
    {
        {
            std::lock_guard<std::mutex> g(mu_);
            stop_ = true;
        }
        cv_.notify_all();
        for (auto& t : th_) t.join();
    }
    void run(const std::function<void(int, int)>& fn)
    {
        std::lock_guard<std::mutex> one(run_mu_);  // one run at a time (callers on several threads)
        {
            std::lock_guard<std::mutex> g(mu_);
            fn_ = &fn;
            left_ = n_ - 1;
            ++gen_;
        }
        cv_.notify_all();
        fn(0, n_);
        std::unique_lock<std::mutex> g(mu_);
        done_.wait(g, [this] { return left_ == 0; });
        fn_ = nullptr;
    }

private:
    void loop(int i)
    {
        uint64_t seen = 0;
        for (;;) {
            const std::function<void(int, int)>* fn;
            {
                std::unique_lock<std::mutex> g(mu_);
                cv_.wait(g, [&] { return stop_ || gen_ != seen; });
                if (stop_) return;
                seen = gen_;
                fn = fn_;
            }
            (*fn)(i, n_);
            std::lock_guard<std::mutex> g(mu_);
            if (--left_ == 0) done_.notify_one();
        }
    }
    int n_ = 1;
    std::vector<std::thread> th_;
    std::mutex run_mu_, mu_;
    std::condition_variable cv_, done_;
    const std::function<void(int, int)>* fn_ = nullptr;
    uint64_t gen_ = 0;
    int left_ = 0;
    bool stop_ = false;
};

// Width-change copies go through staging chunks: host threads gather the
// copies' source ranges (plane and LUT masters) into a pinned chunk, one DMA
// moves the chunk to its device twin, and the copy kernel scatters it into the
// new slabs.  Measured beside a 24-layer decode stack: DMA copies of >= 1 MB
// cost the running kernels nothing, while copies of 64-256 KB (one per plane
// or LUT) and the copy kernel reading pinned host memory directly slowed them
// by as much as the copies took.
constexpr size_t kStageChunkBytes = (size_t)32 << 20;
constexpr size_t kStageChunksMax = 16;
constexpr int kStageListMax = 4096;   // copies per chunk
constexpr int kGatherThreads = 8;     // pinned-to-pinned memcpy: 33 GB/s on one thread, 92 on four, 116 on eight

struct StageChunk {
    char* h = nullptr;              // pinned host
    char* d = nullptr;              // device
    CopyDesc* list = nullptr;       // pinned copy list ...
    const CopyDesc* dlist = nullptr;  // ... and its device-side address
    hipEvent_t ev = nullptr;        // behind the chunk's last scatter
    hipEvent_t gev = nullptr;       // behind the chunk's gather (gather stream)
    uint64_t used = 0;              // use order
};

// One host-to-device copy of a width change.
struct CopyItem {
    const char* src;
    void* dst;
    size_t bytes;
};

// A width change of one block: its new slabs (planes q_old..q_new-1 and
// LUT_{q_new}) and the event behind their copies.
struct WidthChange {
    int id;
    int qo, qn;
    void* planes[8];
    void* lut;
    hipEvent_t copied;
};

// device LUT_q in the slot layout, and its offset in the host master (words)
size_t lut_bytes(int S, int q) { return (size_t)S * ((size_t)1 << q) * 4; }
size_t lut_offset_words(int S, int q) { return (size_t)S * (((size_t)1 << q) - 8); }

struct ProfRec {
    hipEvent_t a, b;
};

}  // namespace

namespace pw {
// error path of the host planner (pw_planner.cpp): the thread-local message
pw_status plan_fail(const char* msg) { return fail(PW_ERR_INVALID, "%s", msg); }
pw_status plan_exception(const char* fn, bool oom)
{
    return oom ? fail(PW_ERR_OOM, "%s: host memory exhausted", fn) : fail(PW_ERR_INVALID, "%s: unexpected exception", fn);
}
}  // namespace pw

struct pw_ctx {
    int device = 0;
    pw_model_desc d{};
    int nblocks = 0;
    BlockDesc* d_table = nullptr;
    std::vector<BlockDesc> h_table;
    std::vector<HostBlock> blocks;
    EventPool evs;  // declared before the slab pool, which holds references on its events
    SlabPool pool{&evs};
    // pinned staging (copy lists, page-table entries) read by kernels through
    // its device-side address, reused once the event behind its last reader
    // has completed
    struct Staging {
        void* p;
        void* dp;
        size_t bytes;
        hipEvent_t ev;
    };
    std::vector<Staging> staging;
    std::vector<StageChunk> chunks;  // gather staging of width-change copies (reserved to kStageChunksMax)
    uint64_t chunk_uses = 0;
    std::unique_ptr<Gang> gang;      // gather threads, started with the first width change
    hipStream_t gather_stream = nullptr;  // runs the gathers of staged copies (host functions)
    int num_cus = 256;  // compute units of the device (decode tile schedule)
    int tok_pass = 0;   // decode tokens per pass set by pw_set_tokens_per_pass (0: chosen per call)
    void* scratch = nullptr;  // this device's library-held workspace (pw_moe_layer_noalloc)
    std::map<int, WidthChange> pending;  // width requests whose commit has not happened
    double* d_mass = nullptr;  // routing-mass accumulator [L][E] fp64 (pw_routing_mass_enable)
    bool mass_on = false;
    bool profiling = false;
    std::map<std::string, std::vector<ProfRec>> prof;
    std::vector<hipEvent_t> prof_pool;
    size_t prof_next = 0;
};

namespace {

// An event from the context's pool with one reference held by the caller.
hipError_t new_event(pw_ctx* c, hipEvent_t* ev)
{
    hipError_t e = c->evs.acquire(ev);
    if (e == hipSuccess) c->evs.hold(*ev);
    return e;
}

// A free pinned staging buffer of at least `bytes` (one whose event has
// completed), or a new one.  The caller records st.ev behind the work that
// reads it and hands it back with put_staging.
pw_status take_staging(pw_ctx* c, size_t bytes, pw_ctx::Staging& st)
{
    for (size_t i = 0; i < c->staging.size(); ++i) {
        if (c->staging[i].bytes >= bytes && hipEventQuery(c->staging[i].ev) == hipSuccess) {
            st = c->staging[i];
            c->staging.erase(c->staging.begin() + i);
            return PW_OK;
        }
    }
    st = pw_ctx::Staging{nullptr, nullptr, (bytes + 4095) & ~size_t(4095), nullptr};
    if (hipHostMalloc(&st.p, st.bytes, hipHostMallocDefault) != hipSuccess) {
        (void)hipGetLastError();
        return fail(PW_ERR_OOM, "pinned staging of %zu B", st.bytes);
    }
    hipError_t e = hipHostGetDevicePointer(&st.dp, st.p, 0);
    if (e == hipSuccess) e = new_event(c, &st.ev);
    if (e != hipSuccess) {
        (void)hipHostFree(st.p);
        return hip_fail(e, "pinned staging");
    }
    return PW_OK;
}

void put_staging(pw_ctx* c, const pw_ctx::Staging& st) { c->staging.push_back(st); }

int block_id(const pw_ctx* c, int layer, int expert, int module)
{
    const int E = c->d.num_experts;
    if (layer < 0 || layer >= c->d.num_layers) return -1;
    if (module != PW_MODULE_GATE_UP && module != PW_MODULE_DOWN) return -1;
    int slot;
    if (expert == PW_EXPERT_SHARED) {
        if (c->d.inter_shared <= 0) return -1;
        slot = E;
    } else if (expert >= 0 && expert < E) {
        slot = expert;
    } else {
        return -1;
    }
    return (layer * (E + 1) + slot) * 2 + module;
}

void block_shape(const pw_ctx* c, int id, int* R, int* K)
{
    const int E = c->d.num_experts;
    const int module = id & 1;
    const int slot = (id >> 1) % (E + 1);
    const int I = slot == E ? c->d.inter_shared : c->d.inter;
    if (module == PW_MODULE_GATE_UP) {
        *R = 2 * I;
        *K = c->d.hidden;
    } else {
        *R = c->d.hidden;
        *K = I;
    }
}

BlockDesc make_desc(const HostBlock& b)
{
    BlockDesc d;
    std::memset(&d, 0, sizeof d);
    for (int p = 0; p < 8; ++p) d.planes[p] = p < b.q ? (const uint32_t*)b.dplanes[p] : nullptr;
    d.lut = (const uint32_t*)b.dlut;
    d.slots = b.S;
    d.q = b.q;
    d.R = b.R;
    d.K = b.K;
    d.nchunks = (b.K + kChunkCols - 1) / kChunkCols;
    d.kwords = b.K / 32;
    return d;
}

void free_block_now(pw_ctx* c, HostBlock& b)
{
    for (int p = 0; p < 8; ++p) {
        c->pool.release_now(b.dplanes[p], (size_t)b.pw * 4, p);
        b.dplanes[p] = nullptr;
    }
    c->pool.release_now(b.dlut, lut_bytes(b.S, b.q), SlabPool::kLutTag);
    b.dlut = nullptr;
    if (b.hplanes) (void)hipHostFree(b.hplanes);
    if (b.hluts) (void)hipHostFree(b.hluts);
    b.hplanes = nullptr;
    b.hluts = nullptr;
    b.dv_hplanes = nullptr;
    b.dv_hluts = nullptr;
    b.registered = false;
}

// Per-kernel HIP-event timing: events come from a pool created when profiling
// is enabled, so recording adds no allocation to the launch path.
constexpr size_t kProfEvents = 1 << 14;

// The first kernel launched inside the scope records a pair of pool events
// from its own dispatch (start and end of the kernel itself).
struct ProfScope {
    pw_ctx* c;
    const char* name;
    LaunchEvents ev;
    ProfScope(pw_ctx* c_, const char* n, hipStream_t) : c(c_), name(n)
    {
        if (c->profiling && c->prof_next + 2 <= c->prof_pool.size()) {
            ev.start = c->prof_pool[c->prof_next++];
            ev.stop = c->prof_pool[c->prof_next++];
            launch_events = &ev;
        }
    }
    ~ProfScope()
    {
        if (!ev.start) return;
        launch_events = nullptr;
        if (ev.used) c->prof[name].push_back({ev.start, ev.stop});
    }
};

void prof_reset(pw_ctx* c)
{
    c->prof.clear();
    c->prof_next = 0;
}

void prof_release(pw_ctx* c)
{
    prof_reset(c);
    for (auto ev : c->prof_pool) (void)hipEventDestroy(ev);
    c->prof_pool.clear();
}

}  // namespace

extern "C" {

const char* pw_last_error(void) { return g_err.c_str(); }

int64_t pw_plane_words(int64_t R, int64_t K) { return (R > 0 && K > 0) ? plane_words(R, K) : 0; }

pw_status pw_pack_bitplanes(const uint8_t* codes, int64_t R, int64_t K, uint32_t* planes)
{
    return guarded("pw_pack_bitplanes", [&]() -> pw_status {
        if (!codes || !planes) return fail(PW_ERR_INVALID, "pw_pack_bitplanes: null pointer");
        if (R <= 0 || K <= 0 || K % 32 != 0 || R > (1 << 24) || K > (1 << 24))
            return fail(PW_ERR_INVALID, "pw_pack_bitplanes: need R > 0 and K a positive multiple of 32 (R=%lld K=%lld)",
                        (long long)R, (long long)K);
        pack_bitplanes(codes, R, K, planes);
        return ok();
    });
}

pw_status pw_create(pw_ctx** out, int hip_device, const pw_model_desc* d)
{
    return guarded("pw_create", [&]() -> pw_status {
        if (!out || !d) return fail(PW_ERR_INVALID, "pw_create: null pointer");
        *out = nullptr;
        const bool shape_ok = d->num_layers >= 1 && d->num_layers <= 4096 && d->num_experts >= 1 &&
                              d->num_experts <= 256 && d->hidden >= 32 && d->hidden <= 32768 &&
                              d->hidden % 32 == 0 && d->inter >= 32 && d->inter <= 131072 && d->inter % 32 == 0 &&
                              d->inter_shared >= 0 && d->inter_shared <= 131072 && d->inter_shared % 32 == 0 &&
                              d->top_k >= 1 && d->top_k <= 8 && d->top_k <= d->num_experts;
        if (!shape_ok) return fail(PW_ERR_INVALID, "pw_create: model description out of range");
        int ndev = 0;
        hipError_t e = hipGetDeviceCount(&ndev);
        if (e != hipSuccess) return hip_fail(e, "hipGetDeviceCount");
        if (hip_device < 0 || hip_device >= ndev) return fail(PW_ERR_INVALID, "pw_create: no HIP device %d", hip_device);
        e = hipSetDevice(hip_device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        pw_ctx* c = new (std::nothrow) pw_ctx();
        if (!c) return fail(PW_ERR_OOM, "pw_create: host allocation");
        c->device = hip_device;
        c->d = *d;
        c->nblocks = d->num_layers * (d->num_experts + 1) * 2;
        c->h_table.assign(c->nblocks, BlockDesc{});
        c->blocks.assign(c->nblocks, HostBlock{});
        e = hipMalloc(&c->d_table, sizeof(BlockDesc) * c->nblocks);
        if (e != hipSuccess) {
            delete c;
            return fail(PW_ERR_OOM, "pw_create: page table: %s", hipGetErrorString(e));
        }
        e = hipMemset(c->d_table, 0, sizeof(BlockDesc) * c->nblocks);
        if (e != hipSuccess) {
            (void)hipFree(c->d_table);
            delete c;
            return hip_fail(e, "hipMemset(page table)");
        }
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, hip_device) == hipSuccess && cus > 0)
            c->num_cus = cus;
        // device address of the library-held workspace, with this device current
        e = static_scratch(hip_device, &c->scratch);
        if (e != hipSuccess) {
            (void)hipFree(c->d_table);
            delete c;
            return hip_fail(e, "pw_create: static scratch address");
        }
        *out = c;
        return ok();
    });
}

static void free_chunk(StageChunk& ch);

pw_status pw_destroy(pw_ctx* c)
{
    return guarded("pw_destroy", [&]() -> pw_status {
        if (!c) return ok();
        (void)hipSetDevice(c->device);
        (void)hipDeviceSynchronize();
        if (c->gather_stream) (void)hipStreamSynchronize(c->gather_stream);  // gathers use the gang and chunks
        prof_release(c);
        for (auto& b : c->blocks)
            if (b.registered) free_block_now(c, b);
        for (auto& s : c->staging) (void)hipHostFree(s.p);
        c->gang.reset();
        for (auto& ch : c->chunks) free_chunk(ch);
        if (c->gather_stream) (void)hipStreamDestroy(c->gather_stream);
        c->pool.clear();
        c->evs.clear();
        (void)hipFree(c->d_table);
        if (c->d_mass) (void)hipFree(c->d_mass);
        delete c;
        return ok();
    });
}

int32_t pw_block_id(const pw_ctx* c, int layer, int expert, int module)
{
    return c ? block_id(c, layer, expert, module) : -1;
}

pw_status pw_register_block(pw_ctx* c, int layer, int expert, int module, const uint32_t* host_planes,
                            const uint16_t* host_luts, int q_init)
{
    return guarded("pw_register_block", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_register_block: null context");
        const int id = block_id(c, layer, expert, module);
        if (id < 0) return fail(PW_ERR_INVALID, "pw_register_block: (layer %d, expert %d, module %d) out of range",
                                layer, expert, module);
        if (!host_planes || !host_luts) return fail(PW_ERR_INVALID, "pw_register_block: null pointer");
        if (c->pending.count(id)) return fail(PW_ERR_STATE, "pw_register_block: block has a width request in flight");
        if (q_init < PW_QMIN || q_init > PW_QMAX) return fail(PW_ERR_INVALID, "pw_register_block: q_init %d not in 3..8", q_init);
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        int R, K;
        block_shape(c, id, &R, &K);
        HostBlock nb;
        nb.R = R;
        nb.K = K;
        nb.q = q_init;
        nb.S = lut_slots(R, module);
        nb.pw = plane_words(R, K);
        const size_t plane_b = (size_t)nb.pw * 4;
        const size_t luts_b = lut_offset_words(nb.S, PW_QMAX + 1) * 4;  // LUT_3..LUT_8, slot layout
        auto undo = [&]() {
            for (int p = 0; p < 8; ++p) c->pool.release_now(nb.dplanes[p], plane_b, p);
            c->pool.release_now(nb.dlut, lut_bytes(nb.S, q_init), SlabPool::kLutTag);
            if (nb.hplanes) (void)hipHostFree(nb.hplanes);
            if (nb.hluts) (void)hipHostFree(nb.hluts);
        };
        for (int p = 0; p < q_init; ++p) {
            if ((e = c->pool.alloc(plane_b, p, &nb.dplanes[p])) != hipSuccess) {
                undo();
                return fail(PW_ERR_OOM, "pw_register_block: device plane: %s", hipGetErrorString(e));
            }
        }
        if ((e = c->pool.alloc(lut_bytes(nb.S, q_init), SlabPool::kLutTag, &nb.dlut)) != hipSuccess) {
            undo();
            return fail(PW_ERR_OOM, "pw_register_block: device LUT: %s", hipGetErrorString(e));
        }
        if (c->d.keep_host_masters) {
            if (hipHostMalloc((void**)&nb.hplanes, plane_b * 8, hipHostMallocDefault) != hipSuccess ||
                hipHostMalloc((void**)&nb.hluts, luts_b, hipHostMallocDefault) != hipSuccess) {
                (void)hipGetLastError();
                undo();
                return fail(PW_ERR_OOM, "pw_register_block: pinned host master");
            }
            void *dvp = nullptr, *dvl = nullptr;
            if (hipHostGetDevicePointer(&dvp, nb.hplanes, 0) == hipSuccess &&
                hipHostGetDevicePointer(&dvl, nb.hluts, 0) == hipSuccess) {
                nb.dv_hplanes = (const uint32_t*)dvp;
                nb.dv_hluts = (const uint32_t*)dvl;
            }
            (void)hipGetLastError();
            std::memcpy(nb.hplanes, host_planes, plane_b * 8);
            for (int q = PW_QMIN; q <= PW_QMAX; ++q)
                convert_lut(host_luts, R, module, q, nb.hluts + lut_offset_words(nb.S, q));
        }
        for (int p = 0; p < q_init && e == hipSuccess; ++p)
            e = hipMemcpy(nb.dplanes[p], host_planes + (size_t)p * nb.pw, plane_b, hipMemcpyHostToDevice);
        if (e == hipSuccess) {
            std::vector<uint32_t> lq(lut_bytes(nb.S, q_init) / 4);
            convert_lut(host_luts, R, module, q_init, lq.data());
            e = hipMemcpy(nb.dlut, lq.data(), lut_bytes(nb.S, q_init), hipMemcpyHostToDevice);
        }
        if (e != hipSuccess) {
            undo();
            return hip_fail(e, "pw_register_block: copy to device");
        }
        nb.registered = true;
        BlockDesc desc = make_desc(nb);
        e = hipMemcpy(c->d_table + id, &desc, sizeof desc, hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            undo();
            return hip_fail(e, "pw_register_block: page-table entry");
        }
        if (c->blocks[id].registered) {
            (void)hipDeviceSynchronize();
            free_block_now(c, c->blocks[id]);
        }
        c->blocks[id] = nb;
        c->h_table[id] = desc;
        return ok();
    });
}

size_t pw_workspace_size(const pw_ctx* c, int T)
{
    if (!c || T <= 0) return 0;
    return ws_layout(T, c->d.top_k, c->d.hidden, c->d.inter, c->d.inter_shared).total;
}

pw_status pw_set_tokens_per_pass(pw_ctx* c, int tokens)
{
    return guarded("pw_set_tokens_per_pass", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_set_tokens_per_pass: null context");
        if (tokens != 0 && tokens != 8 && tokens != 16 && tokens != 32)
            return fail(PW_ERR_INVALID, "pw_set_tokens_per_pass: %d is not 0, 8, 16 or 32", tokens);
        c->tok_pass = tokens;
        return ok();
    });
}

int32_t pw_decode_tokens_per_pass(int T, int top_k, int E, int I_shared)
{
    if (T <= 0 || T >= kPrefillMinT || top_k <= 0 || E <= 0) return 0;
    return decode_tok_pass(T, top_k, E, I_shared);
}

pw_status pw_route_topk(pw_ctx* c, const float* logits, int T, int32_t* idx, float* w, pw_stream stream)
{
    return guarded("pw_route_topk", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_route_topk: null context");
        if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "pw_route_topk: T=%d out of range", T);
        if (T == 0) return ok();
        if (!logits || !idx || !w) return fail(PW_ERR_INVALID, "pw_route_topk: null pointer");
        if (!aligned4(logits) || !aligned4(idx) || !aligned4(w))
            return fail(PW_ERR_INVALID, "pw_route_topk: device pointers must be 4-byte aligned");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        ProfScope ps(c, "route", (hipStream_t)stream);
        e = launch_route_topk(logits, T, c->d.num_experts, c->d.top_k, idx, w, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "route_topk launch");
    });
}

pw_status pw_route_permute(pw_ctx* c, const float* logits, int T, int32_t* idx, float* w, int32_t* offsets,
                           int32_t* sorted, pw_stream stream)
{
    return guarded("pw_route_permute", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_route_permute: null context");
        if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "pw_route_permute: T=%d out of range", T);
        if (!offsets) return fail(PW_ERR_INVALID, "pw_route_permute: null offsets");
        if (T > 0 && (!logits || !idx || !w || !sorted)) return fail(PW_ERR_INVALID, "pw_route_permute: null pointer");
        if (!aligned4(offsets) || (T > 0 && (!aligned4(logits) || !aligned4(idx) || !aligned4(w) || !aligned4(sorted))))
            return fail(PW_ERR_INVALID, "pw_route_permute: device pointers must be 4-byte aligned");
        const int k = c->d.top_k, E = c->d.num_experts;
        if ((long long)T * k > kFusedMaxAssign) {
            pw_status st = pw_route_topk(c, logits, T, idx, w, stream);
            return st != PW_OK ? st : pw_permute_by_expert(c, idx, T, offsets, sorted, stream);
        }
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        ProfScope ps(c, "route", (hipStream_t)stream);
        e = launch_route_permute(logits, T, E, k, idx, w, offsets, sorted, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "route_permute launch");
    });
}

pw_status pw_permute_by_expert(pw_ctx* c, const int32_t* idx, int T, int32_t* offsets, int32_t* sorted,
                               pw_stream stream)
{
    return guarded("pw_permute_by_expert", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_permute_by_expert: null context");
        if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "pw_permute_by_expert: T=%d out of range", T);
        if (!offsets) return fail(PW_ERR_INVALID, "pw_permute_by_expert: null offsets");
        if (T > 0 && (!idx || !sorted)) return fail(PW_ERR_INVALID, "pw_permute_by_expert: null pointer");
        if (!aligned4(offsets) || (T > 0 && (!aligned4(idx) || !aligned4(sorted))))
            return fail(PW_ERR_INVALID, "pw_permute_by_expert: device pointers must be 4-byte aligned");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        ProfScope ps(c, "permute", (hipStream_t)stream);
        e = launch_permute(idx, T, c->d.top_k, c->d.num_experts, offsets, sorted, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "permute launch");
    });
}

// Argument checks of the FFN (fn names the entry point in messages).
static pw_status ffn_check(const pw_ctx* c, const char* fn, int layer, const uint16_t* x, int T, const int32_t* idx,
                           const float* w, const int32_t* offsets, const int32_t* sorted, const uint16_t* y,
                           const void* workspace, size_t ws_bytes)
{
    if (!c) return fail(PW_ERR_INVALID, "%s: null context", fn);
    if (layer < 0 || layer >= c->d.num_layers) return fail(PW_ERR_INVALID, "%s: layer %d out of range", fn, layer);
    if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "%s: T=%d out of range", fn, T);
    if (T == 0) return ok();
    if (!x || !idx || !w || !offsets || !sorted || !y || !workspace) return fail(PW_ERR_INVALID, "%s: null pointer", fn);
    if (!aligned16(x) || !aligned4(idx) || !aligned4(w) || !aligned4(offsets) || !aligned4(sorted) ||
        !aligned16(y) || ((uintptr_t)workspace & 255u))
        return fail(PW_ERR_INVALID, "%s: misaligned pointer (x, y 16 B; index arrays 4 B; workspace 256 B)", fn);
    const pw_model_desc& d = c->d;
    const WsLayout L = ws_layout(T, d.top_k, d.hidden, d.inter, d.inter_shared);
    if (ws_bytes < L.total) return fail(PW_ERR_INVALID, "%s: workspace %zu B < %zu B needed", fn, ws_bytes, L.total);
    if (T >= kPrefillMinT) {
        // the prefill kernels address x and h by 32-bit byte offsets
        const uint64_t xb = (uint64_t)T * d.hidden * 2;
        const uint64_t hb = (uint64_t)T * (d.top_k + 1) * std::max(d.inter, d.inter_shared) * 2;
        if (std::max(xb, hb) > 0xffffffffull)
            return fail(PW_ERR_INVALID, "%s: T=%d: x or h of the prefill path exceeds 4 GiB; split the batch", fn, T);
    }
    const int E = d.num_experts;
    for (int s = 0; s <= E; ++s) {
        if (s == E && d.inter_shared == 0) break;
        for (int m = 0; m < 2; ++m) {
            const int id = (layer * (E + 1) + s) * 2 + m;
            if (!c->blocks[id].registered)
                return fail(PW_ERR_STATE, "%s: block (layer %d, slot %d, module %d) not registered", fn, layer, s, m);
        }
    }
    return ok();
}

// Routing results computed by the decode gate_up launch itself.
struct LayerRoute {
    const float* logits;
    int32_t* idx;
    float* w;
    int32_t* offsets;
    int32_t* sorted;
    double* mass;  // this layer's routing-mass row, or null
};

// Enqueues the FFN of checked arguments (T > 0).
static pw_status ffn_launch(pw_ctx* c, int layer, const uint16_t* x, int T, const float* w, const int32_t* offsets,
                            const int32_t* sorted, uint16_t* y, void* workspace, pw_stream stream,
                            const LayerRoute* route)
{
    const pw_model_desc& d = c->d;
    const WsLayout L = ws_layout(T, d.top_k, d.hidden, d.inter, d.inter_shared);
    const int E = d.num_experts;
    hipError_t e = hipSetDevice(c->device);
    if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
    char* ws = (char*)workspace;
    FfnArgs a;
    std::memset(&a, 0, sizeof a);
    a.table = c->d_table + (size_t)layer * (E + 1) * 2;
    a.x = x;
    a.offsets = offsets;
    a.sorted = sorted;
    a.topk_w = w;
    a.h = (uint16_t*)(ws + L.h);
    a.dout = (float*)(ws + L.dout);
    a.y = y;
    a.T = T;
    a.H = d.hidden;
    a.I = d.inter;
    a.Is = d.inter_shared;
    a.E = E;
    a.k = d.top_k;
    a.n_slots = std::min(E, T * d.top_k);
    a.tok_pass = c->tok_pass ? c->tok_pass : decode_tok_pass(T, d.top_k, E, d.inter_shared);
    a.keep_planes = keep_planes(T, d.top_k, E, d.inter_shared, a.tok_pass) ? 1 : 0;
    a.hstride = std::max(d.inter, d.inter_shared);
    a.drows = T * d.top_k + (d.inter_shared ? T : 0);
    hipStream_t s = (hipStream_t)stream;
    if (T >= kPrefillMinT) {
        // prefill: GEMM tiles of 128 weight rows x 512 tokens, full K; an
        // expert's tail of fewer than kPrefillTail tokens past its last whole
        // tile goes to the decode kernels instead (32-token passes that stream
        // the expert's weights once per pass, where a GEMM tile decodes them in
        // full for a few dozen tokens; the shared expert keeps its tiles)
        const int tt = (T + 511) / 512;
        a.tok_tiles_shared = d.inter_shared ? tt : 0;
        a.tok_tiles_routed = (T * d.top_k + 511) / 512 + std::min(E, T * d.top_k);
        a.pf_tail = kPrefillTail;
        // the decode launches on the tails: routed experts only, whole
        // 128-row gate_up tiles, 32-token passes with planes kept in the MALL
        // for a tail's later passes
        FfnArgs tl = a;
        tl.tiles_shared = 0;
        tl.splits_shared = 1;
        tl.n_slots = E;
        tl.tok_pass = 32;
        tl.keep_planes = 1;
        tl.big_wgs = 0;
        {
            ProfScope ps(c, "gate_up", s);
            a.tiles_routed = (d.inter + 63) / 64;
            a.tiles_shared = d.inter_shared ? (d.inter_shared + 63) / 64 : 0;
            if ((e = launch_prefill(a, 0, s)) != hipSuccess) return hip_fail(e, "prefill gate_up launch");
        }
        {
            ProfScope ps(c, "gate_up_tail", s);
            tl.rg = kGateUpRowGroups;
            tl.tiles_routed = (d.inter + 16 * tl.rg - 1) / (16 * tl.rg);
            tl.splits_routed = 1;
            if ((e = launch_gate_up(tl, s)) != hipSuccess) return hip_fail(e, "prefill tail gate_up launch");
        }
        // K in two halves where the workspace holds two partial planes (the
        // combine sums the planes of every row, tails included)
        const int ws_splits = std::max(down_splits(d.inter), d.inter_shared ? down_splits(d.inter_shared) : 1);
        const int pf_splits = std::min(2, ws_splits);
        {
            ProfScope ps(c, "down", s);
            a.tiles_routed = (d.hidden + 127) / 128;
            a.tiles_shared = d.inter_shared ? (d.hidden + 127) / 128 : 0;
            a.splits_routed = a.splits_shared = pf_splits;
            if ((e = launch_prefill(a, 1, s)) != hipSuccess) return hip_fail(e, "prefill down launch");
        }
        {
            ProfScope ps(c, "down_tail", s);
            tl.rg = kDownRowGroups;
            tl.tiles_routed = (d.hidden + 32 * tl.rg - 1) / (32 * tl.rg);
            tl.splits_routed = pf_splits;
            if ((e = launch_down(tl, s)) != hipSuccess) return hip_fail(e, "prefill tail down launch");
        }
        {
            ProfScope ps(c, "combine", s);
            if ((e = launch_combine(a, s)) != hipSuccess) return hip_fail(e, "combine launch");
        }
        return ok();
    }
    {
        ProfScope ps(c, "gate_up", s);
        // Expected 128-row units: the shared tiles plus the tiles of the experts
        // a batch is expected to activate (each with probability 1 - (1 - k/E)^T).
        // More than three per CU means several rounds of workgroups whatever the
        // tile split; such launches take whole 128-row tiles (see big_wgs below),
        // and 32-token passes where 16 would do: a 128-row tile needs 32-token
        // passes (the 16-token form is for 64-row tiles only), and halving the
        // workgroups paid more than the wider passes cost (Qwen-shaped gate_up
        // batch 16 34.5 -> 29.5 us, batch 12 31.0 -> 29.0, Mixtral-shaped batch
        // 32 186 -> 176; at batch 9 and 10, below the threshold, 64-row tiles of
        // 16-token passes stay faster: 29.4 vs 31.1 us).
        const double active = E * (1.0 - std::pow(1.0 - (double)d.top_k / E, (double)T));
        const bool rounds = (d.inter_shared + 63) / 64 + active * ((d.inter + 63) / 64) > 3.0 * c->num_cus;
        const int tok_pass_call = a.tok_pass;
        if (a.tok_pass == 16 && !c->tok_pass && rounds) a.tok_pass = 32;
        a.rg = a.tok_pass == 16 ? 2 : kGateUpRowGroups;
        a.tiles_routed = (d.inter + 16 * a.rg - 1) / (16 * a.rg);
        a.tiles_shared = (d.inter_shared + 16 * a.rg - 1) / (16 * a.rg);
        a.splits_routed = 1;
        a.splits_shared = 1;
        // 128-row tiles: one whole unit per CU first, later units in 64-row
        // halves, so a CU's second slot carries half a unit.  That pays while
        // the halves fit in the second slots; a single token activates exactly
        // k experts, and when those units' halves would overflow the second
        // slots into another round, whole units are faster (Mixtral-shaped
        // batch 1: 448 units, gate_up 47.6 -> 44.7 us).  A launch that runs
        // several rounds anyway (`rounds`) only gains workgroup start-ups from
        // halves: whole units took Mixtral-shaped gate_up batch 4 111 -> 109 us,
        // batch 16 165 -> 155, batch 64 208 -> 181 (at two to three units per
        // CU, Qwen-shaped batch 6 and 8, halves stay faster).
        a.big_wgs = a.rg == 4 ? c->num_cus : 0;
        if (a.rg == 4 && T == 1) {
            const long long units = a.tiles_shared + (long long)d.top_k * a.tiles_routed;
            if (2 * (units - c->num_cus) > c->num_cus) a.big_wgs = 0;
        }
        if (a.rg == 4 && rounds) a.big_wgs = 0;
        if (route) {
            a.logits = route->logits;
            a.idx_out = route->idx;
            a.w_out = route->w;
            a.offsets_out = route->offsets;
            a.sorted_out = route->sorted;
            a.mass = route->mass;
        }
        if ((e = launch_gate_up(a, s)) != hipSuccess) return hip_fail(e, "gate_up launch");
        a.tok_pass = tok_pass_call;
        a.logits = nullptr;
        a.mass = nullptr;
    }
    {
        ProfScope ps(c, "down", s);
        a.rg = kDownRowGroups;
        a.big_wgs = a.rg == 4 ? c->num_cus : 0;
        a.tiles_routed = (d.hidden + 32 * a.rg - 1) / (32 * a.rg);
        a.tiles_shared = d.inter_shared ? (d.hidden + 32 * a.rg - 1) / (32 * a.rg) : 0;
        a.splits_routed = down_splits_routed(d.inter, T, d.top_k, E, a.tiles_routed, c->num_cus);
        a.splits_shared = d.inter_shared ? down_splits(d.inter_shared) : 1;
        if ((e = launch_down(a, s)) != hipSuccess) return hip_fail(e, "down launch");
    }
    {
        ProfScope ps(c, "combine", s);
        if ((e = launch_combine(a, s)) != hipSuccess) return hip_fail(e, "combine launch");
    }
    return ok();
}

pw_status pw_moe_ffn_bitplane(pw_ctx* c, int layer, const uint16_t* x, int T, const int32_t* idx,
                              const float* w, const int32_t* offsets, const int32_t* sorted, uint16_t* y,
                              void* workspace, size_t ws_bytes, pw_stream stream)
{
    return guarded("pw_moe_ffn_bitplane", [&]() -> pw_status {
        const pw_status st =
            ffn_check(c, "pw_moe_ffn_bitplane", layer, x, T, idx, w, offsets, sorted, y, workspace, ws_bytes);
        if (st != PW_OK || T == 0) return st;
        return ffn_launch(c, layer, x, T, w, offsets, sorted, y, workspace, stream, nullptr);
    });
}

pw_status pw_moe_layer(pw_ctx* c, int layer, const float* logits, const uint16_t* x, int T, int32_t* idx, float* w,
                       int32_t* offsets, int32_t* sorted, uint16_t* y, void* workspace, size_t ws_bytes,
                       pw_stream stream)
{
    return guarded("pw_moe_layer", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_moe_layer: null context");
        if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "pw_moe_layer: T=%d out of range", T);
        if (!offsets) return fail(PW_ERR_INVALID, "pw_moe_layer: null offsets");
        if (!aligned4(offsets) || (T > 0 && (!logits || !aligned4(logits))))
            return fail(PW_ERR_INVALID, "pw_moe_layer: null or misaligned logits / offsets (4 B)");
        pw_status st = ffn_check(c, "pw_moe_layer", layer, x, T, idx, w, offsets, sorted, y, workspace, ws_bytes);
        if (st != PW_OK) return st;
        // In-launch routing pays off only when every gate_up work unit gets a
        // workgroup slot at once (two per CU): each routed workgroup routes the
        // batch itself, so a launch with several rounds of workgroups would repeat
        // it per round.
        const pw_model_desc& d = c->d;
        const long long n = (long long)T * d.top_k;
        const long long gu_rows = 16LL * kGateUpRowGroups;
        // units of the shared tiles and of the experts a batch is expected to
        // activate (the slots past the active ones exit right after routing;
        // Qwen-shaped batch 5: 0.0445 -> 0.0432 ms with the routing inside)
        const double act_e = d.num_experts * (1.0 - std::pow(1.0 - (double)d.top_k / d.num_experts, (double)T));
        const long long gu_units = (d.inter_shared + gu_rows - 1) / gu_rows +
                                   (long long)(act_e * ((d.inter + gu_rows - 1) / gu_rows));
        double* mass = c->mass_on ? c->d_mass + (size_t)layer * d.num_experts : nullptr;
        if (T == 0 || T >= kPrefillMinT || n > kLayerRouteMaxAssign || gu_units > 2LL * c->num_cus ||
            (c->tok_pass ? c->tok_pass : decode_tok_pass(T, d.top_k, d.num_experts, d.inter_shared)) != 8) {
            // the separate routing launch, then the FFN (identical results)
            st = pw_route_permute(c, logits, T, idx, w, offsets, sorted, stream);
            if (st != PW_OK || T == 0) return st;
            if (mass) {
                const hipError_t e = launch_routing_mass(offsets, sorted, w, d.num_experts, mass, (hipStream_t)stream);
                if (e != hipSuccess) return hip_fail(e, "routing mass launch");
            }
            return ffn_launch(c, layer, x, T, w, offsets, sorted, y, workspace, stream, nullptr);
        }
        const LayerRoute r{logits, idx, w, offsets, sorted, mass};
        return ffn_launch(c, layer, x, T, w, offsets, sorted, y, workspace, stream, &r);
    });
}

pw_status pw_moe_layer_noalloc(pw_ctx* c, int layer, const float* logits, const uint16_t* x, int T, int32_t* idx,
                               float* w, int32_t* offsets, int32_t* sorted, uint16_t* y, pw_stream stream)
{
    return guarded("pw_moe_layer_noalloc", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_moe_layer_noalloc: null context");
        if (T < 0 || T > PW_MAX_TOKENS) return fail(PW_ERR_INVALID, "pw_moe_layer_noalloc: T=%d out of range", T);
        const size_t need = pw_workspace_size(c, T);
        if (need > kStaticScratchBytes)
            return fail(PW_ERR_INVALID, "pw_moe_layer_noalloc: T=%d needs %zu B of workspace, above the %zu B the library "
                        "holds; use pw_moe_layer with a caller workspace", T, need, kStaticScratchBytes);
        return pw_moe_layer(c, layer, logits, x, T, idx, w, offsets, sorted, y, c->scratch, kStaticScratchBytes, stream);
    });
}

pw_status pw_routing_mass_enable(pw_ctx* c, int on)
{
    return guarded("pw_routing_mass_enable", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_routing_mass_enable: null context");
        if (on && !c->d_mass) {
            hipError_t e = hipSetDevice(c->device);
            if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
            const size_t bytes = sizeof(double) * (size_t)c->d.num_layers * c->d.num_experts;
            double* p = nullptr;
            if ((e = hipMalloc((void**)&p, bytes)) != hipSuccess) return fail(PW_ERR_OOM, "pw_routing_mass_enable: %s", hipGetErrorString(e));
            if ((e = hipMemset(p, 0, bytes)) != hipSuccess || (e = hipDeviceSynchronize()) != hipSuccess) {
                (void)hipFree(p);
                return hip_fail(e, "pw_routing_mass_enable: zero");
            }
            c->d_mass = p;
        }
        c->mass_on = on != 0;
        return ok();
    });
}

pw_status pw_routing_mass_reset(pw_ctx* c, pw_stream stream)
{
    return guarded("pw_routing_mass_reset", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_routing_mass_reset: null context");
        if (!c->d_mass) return fail(PW_ERR_STATE, "pw_routing_mass_reset: routing mass was never enabled");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        e = launch_fill_f64(c->d_mass, (int64_t)c->d.num_layers * c->d.num_experts, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "routing mass reset launch");
    });
}

pw_status pw_routing_mass_read(pw_ctx* c, double* host_out, pw_stream stream)
{
    return guarded("pw_routing_mass_read", [&]() -> pw_status {
        if (!c || !host_out) return fail(PW_ERR_INVALID, "pw_routing_mass_read: null pointer");
        if (!c->d_mass) return fail(PW_ERR_STATE, "pw_routing_mass_read: routing mass was never enabled");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        const size_t bytes = sizeof(double) * (size_t)c->d.num_layers * c->d.num_experts;
        e = hipMemcpyAsync(host_out, c->d_mass, bytes, hipMemcpyDeviceToHost, (hipStream_t)stream);
        if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "pw_routing_mass_read: copy");
    });
}

pw_status pw_get_committed_bits(const pw_ctx* c, int32_t id, int32_t* q_out)
{
    return guarded("pw_get_committed_bits", [&]() -> pw_status {
        if (!c || !q_out) return fail(PW_ERR_INVALID, "pw_get_committed_bits: null pointer");
        if (id < 0 || id >= c->nblocks) return fail(PW_ERR_INVALID, "pw_get_committed_bits: block id %d out of range", id);
        *q_out = c->blocks[id].registered ? c->blocks[id].q : 0;
        return ok();
    });
}

int64_t pw_resident_bytes(const pw_ctx* c) { return c ? c->pool.resident() : 0; }

// Width changes in two phases.  prepare: new slabs for planes q_old..q_new-1
// and LUT_{q_new}, their copies from the pinned masters on the copy stream,
// an event behind them.  apply: the page-table entries on the compute stream
// (stream-ordered, so work enqueued earlier keeps the old widths), old slabs
// recycled after that update.

static void free_chunk(StageChunk& ch)
{
    if (ch.ev) {
        (void)hipEventSynchronize(ch.ev);
        (void)hipEventDestroy(ch.ev);
    }
    if (ch.gev) (void)hipEventDestroy(ch.gev);
    if (ch.h) (void)hipHostFree(ch.h);
    if (ch.list) (void)hipHostFree(ch.list);
    if (ch.d) (void)hipFree(ch.d);
    ch = StageChunk{};
}

static hipError_t alloc_chunk(StageChunk& ch)
{
    hipError_t e = hipHostMalloc((void**)&ch.h, kStageChunkBytes, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc((void**)&ch.list, kStageListMax * sizeof(CopyDesc), hipHostMallocDefault);
    void* dl = nullptr;
    if (e == hipSuccess) e = hipHostGetDevicePointer(&dl, ch.list, 0);
    if (e == hipSuccess) e = hipMalloc((void**)&ch.d, kStageChunkBytes);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ch.ev, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ch.gev, hipEventDisableTiming);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        free_chunk(ch);
        return e;
    }
    ch.dlist = (const CopyDesc*)dl;
    return hipSuccess;
}

// A staging chunk whose last copies have completed: an idle one, else a new
// one (up to kStageChunksMax), else the least recently used after waiting.
// Null with hipSuccess when none can be had (no chunk and no memory).
static hipError_t take_chunk(pw_ctx* c, StageChunk** out)
{
    *out = nullptr;
    if (c->chunks.capacity() < kStageChunksMax) c->chunks.reserve(kStageChunksMax);  // chunks never move
    StageChunk* oldest = nullptr;
    for (auto& ch : c->chunks) {
        const hipError_t q = hipEventQuery(ch.ev);
        if (q == hipSuccess) {
            oldest = &ch;
            break;
        }
        if (q != hipErrorNotReady) return q;
        if (!oldest || ch.used < oldest->used) oldest = &ch;
    }
    if (oldest && hipEventQuery(oldest->ev) == hipSuccess) {
        *out = oldest;
    } else {
        if (c->chunks.size() < kStageChunksMax) {
            StageChunk ch;
            if (alloc_chunk(ch) == hipSuccess) {
                c->chunks.push_back(ch);
                *out = &c->chunks.back();
            }
        }
        if (!*out && oldest) {
            const hipError_t e = hipEventSynchronize(oldest->ev);
            if (e != hipSuccess) return e;
            *out = oldest;
        }
    }
    if (*out) (*out)->used = ++c->chunk_uses;
    return hipSuccess;
}

// The gather of one staging chunk, run as a host function on the context's
// gather stream: the gang copies the items' source ranges into the pinned
// chunk, and the chunk's DMA on the copy stream waits for it (an event).  The
// caller of a width request is not held for the gathers (~3 ms per 300 MB),
// and one chunk's gather runs while the previous chunk is in flight.  The
// function makes no HIP calls.
struct GatherJob {
    Gang* gang;
    char* dst;
    size_t total;
    std::vector<std::pair<const char*, size_t>> src;  // source, bytes
    std::vector<size_t> at;                            // offsets in the chunk
};

static void gather_in_stream(void* user)
{
    GatherJob* j = (GatherJob*)user;
    try {
        j->gang->run([j](int m, int M) {
            const size_t lo = j->total * m / M, hi = j->total * (m + 1) / M;
            for (size_t k = 0; k < j->src.size(); ++k) {
                const size_t a = j->at[k], b = a + j->src[k].second;
                const size_t s0 = std::max(a, lo), s1 = std::min(b, hi);
                if (s0 < s1) std::memcpy(j->dst + s0, j->src[k].first + (s0 - a), s1 - s0);
            }
        });
    } catch (...) {
        // a gang that cannot run leaves the whole copy to this thread
        for (size_t k = 0; k < j->src.size(); ++k) std::memcpy(j->dst + j->at[k], j->src[k].first, j->src[k].second);
    }
    delete j;
}

// Enqueue `items` on stream xs through the staging chunks (see StageChunk):
// per chunk the gather (host threads, a host function on the gather stream),
// one DMA after it, one scatter launch.  Items larger than a chunk, and every
// item when no chunk can be allocated, are one DMA each.  Returns once
// everything is enqueued.
static hipError_t stage_copies(pw_ctx* c, const std::vector<CopyItem>& items, hipStream_t xs)
{
    if (!c->gang) {
        const unsigned hw = std::thread::hardware_concurrency();
        c->gang.reset(new Gang(std::max(1, std::min(kGatherThreads, (int)(hw / 2)))));
    }
    if (!c->gather_stream) {
        const hipError_t e = hipStreamCreateWithFlags(&c->gather_stream, hipStreamNonBlocking);
        if (e != hipSuccess) return e;
    }
    std::vector<size_t> at;
    size_t i = 0;
    while (i < items.size()) {
        StageChunk* ch = nullptr;
        if (items[i].bytes <= kStageChunkBytes) {
            const hipError_t e = take_chunk(c, &ch);
            if (e != hipSuccess) return e;
        }
        if (!ch) {
            const hipError_t e = hipMemcpyAsync(items[i].dst, items[i].src, items[i].bytes, hipMemcpyHostToDevice, xs);
            if (e != hipSuccess) return e;
            ++i;
            continue;
        }
        // the items that fit, at 256-byte aligned offsets
        const size_t i0 = i;
        size_t off = 0, total = 0;
        at.clear();
        while (i < items.size() && (int)(i - i0) < kStageListMax && off + items[i].bytes <= kStageChunkBytes) {
            ch->list[i - i0] = CopyDesc{ch->d + off, items[i].dst, (uint64_t)items[i].bytes};
            at.push_back(off);
            total = off + items[i].bytes;
            off = (total + 255) & ~(size_t)255;
            ++i;
        }
        // the gather (gang member m copies bytes [total m / M, total (m + 1) / M)
        // of the packed chunk) runs on the stream ahead of the chunk's DMA
        const size_t i1 = i;
        std::unique_ptr<GatherJob> job(new GatherJob);
        job->gang = c->gang.get();
        job->dst = ch->h;
        job->total = total;
        job->at = at;
        job->src.reserve(i1 - i0);
        for (size_t j = i0; j < i1; ++j) job->src.emplace_back(items[j].src, items[j].bytes);
        hipError_t e = hipLaunchHostFunc(c->gather_stream, gather_in_stream, job.get());
        if (e != hipSuccess) return e;
        job.release();  // gather_in_stream frees it
        e = hipEventRecord(ch->gev, c->gather_stream);
        if (e == hipSuccess) e = hipStreamWaitEvent(xs, ch->gev, 0);
        if (e == hipSuccess) e = hipMemcpyAsync(ch->d, ch->h, total, hipMemcpyHostToDevice, xs);
        if (e == hipSuccess) e = launch_scatter_copy(ch->dlist, (int)(i1 - i0), xs);
        if (e == hipSuccess) e = hipEventRecord(ch->ev, xs);
        if (e != hipSuccess) {
            // the chunk's event is stale: let the queued gather and copies end
            // before the chunk (or a slab they write) can be reused
            (void)hipStreamSynchronize(c->gather_stream);
            (void)hipStreamSynchronize(xs);
            return e;
        }
    }
    return hipSuccess;
}

// Undo prepared changes that will not be committed: their new slabs go back
// to the pool and each plan's reference on the copy event is dropped.
static void release_prepared(pw_ctx* c, const std::vector<WidthChange>& plans)
{
    for (const auto& p : plans) {
        const HostBlock& b = c->blocks[p.id];
        for (int j = p.qo; j < p.qn; ++j) c->pool.release_now(p.planes[j], (size_t)b.pw * 4, j);
        c->pool.release_now(p.lut, lut_bytes(b.S, p.qn), SlabPool::kLutTag);
        c->evs.drop(p.copied);
    }
}

// After a commit: the plans' references on their copy event.
static void drop_copy_events(pw_ctx* c, const std::vector<WidthChange>& plans)
{
    for (const auto& p : plans) c->evs.drop(p.copied);
}

// staged: the copies go through the staging chunks (DMA, no interference with
// the kernels running meanwhile: pw_request_widths); else one copy kernel
// reads the pinned masters directly (faster end to end, for the blocking
// pw_set_committed_bits, whose compute stream waits for the copies anyway).
static pw_status prepare_changes(pw_ctx* c, const char* fn, const std::vector<std::pair<int, int>>& todo,
                                 hipStream_t xs, bool staged, std::vector<WidthChange>& plans)
{
    hipError_t e = hipSuccess;
    plans.clear();
    plans.reserve(todo.size());
    for (const auto& t : todo) {
        WidthChange p;
        std::memset(&p, 0, sizeof p);
        p.id = t.first;
        const HostBlock& b = c->blocks[p.id];
        p.qo = b.q;
        p.qn = t.second;
        plans.push_back(p);
        WidthChange& pr = plans.back();
        for (int j = pr.qo; j < pr.qn; ++j) {
            if ((e = c->pool.alloc((size_t)b.pw * 4, j, &pr.planes[j])) != hipSuccess) {
                release_prepared(c, plans);
                return fail(PW_ERR_OOM, "%s: device plane: %s", fn, hipGetErrorString(e));
            }
        }
        if ((e = c->pool.alloc(lut_bytes(b.S, pr.qn), SlabPool::kLutTag, &pr.lut)) != hipSuccess) {
            release_prepared(c, plans);
            return fail(PW_ERR_OOM, "%s: device LUT: %s", fn, hipGetErrorString(e));
        }
    }
    // the copies: planes q_old..q_new-1 and LUT_{q_new} of every block
    std::vector<CopyItem> items;
    for (const auto& p : plans) {
        const HostBlock& b = c->blocks[p.id];
        for (int j = p.qo; j < p.qn; ++j)
            items.push_back(CopyItem{(const char*)(b.hplanes + (size_t)j * b.pw), p.planes[j], (size_t)b.pw * 4});
        items.push_back(CopyItem{(const char*)(b.hluts + lut_offset_words(b.S, p.qn)), p.lut, lut_bytes(b.S, p.qn)});
    }
    bool direct = !staged;
    for (const auto& p : plans) direct = direct && c->blocks[p.id].dv_hplanes && c->blocks[p.id].dv_hluts;
    if (direct) {
        pw_ctx::Staging st{};
        const pw_status sst = take_staging(c, items.size() * sizeof(CopyDesc), st);
        if (sst != PW_OK) {
            release_prepared(c, plans);
            return sst;
        }
        CopyDesc* list = (CopyDesc*)st.p;
        size_t n = 0;
        for (const auto& p : plans) {
            const HostBlock& b = c->blocks[p.id];
            for (int j = p.qo; j < p.qn; ++j)
                list[n++] = CopyDesc{b.dv_hplanes + (size_t)j * b.pw, p.planes[j], (uint64_t)b.pw * 4};
            list[n++] = CopyDesc{b.dv_hluts + lut_offset_words(b.S, p.qn), p.lut, (uint64_t)lut_bytes(b.S, p.qn)};
        }
        e = launch_pull_copy((const CopyDesc*)st.dp, (int)n, xs);
        if (e == hipSuccess) e = hipEventRecord(st.ev, xs);
        put_staging(c, st);
    } else {
        e = stage_copies(c, items, xs);
    }
    hipEvent_t copied = nullptr;
    if (e == hipSuccess) e = new_event(c, &copied);
    if (e == hipSuccess) e = hipEventRecord(copied, xs);
    if (e != hipSuccess) {
        // copies may be in flight into the new slabs: wait before recycling them
        (void)hipStreamSynchronize(xs);
        release_prepared(c, plans);
        if (copied) c->evs.drop(copied);
        return hip_fail(e, "enqueue plane / LUT copies");
    }
    // every plan holds a reference on the copy event until it is committed
    for (auto& p : plans) {
        p.copied = copied;
        c->evs.hold(copied);
    }
    c->evs.drop(copied);
    return ok();
}

static pw_status apply_changes(pw_ctx* c, std::vector<WidthChange>& plans, hipStream_t cs)
{
    hipError_t e = hipSuccess;
    // the new entries and their ids in pinned staging, scattered into the
    // device table by one kernel on the compute stream
    const size_t n = plans.size();
    pw_ctx::Staging st{};
    {
        const pw_status sst = take_staging(c, n * (sizeof(BlockDesc) + sizeof(int32_t)), st);
        if (sst != PW_OK) return sst;
    }
    BlockDesc* descs = (BlockDesc*)st.p;
    int32_t* sids = (int32_t*)(descs + n);
    std::vector<BlockDesc> newdesc(n);
    for (size_t i = 0; i < n; ++i) {
        HostBlock nb = c->blocks[plans[i].id];
        for (int j = 0; j < 8; ++j)
            if (j >= plans[i].qo && j < plans[i].qn) nb.dplanes[j] = plans[i].planes[j];
        for (int j = plans[i].qn; j < 8; ++j) nb.dplanes[j] = nullptr;
        nb.q = plans[i].qn;
        nb.dlut = plans[i].lut;
        newdesc[i] = make_desc(nb);
        descs[i] = newdesc[i];
        sids[i] = plans[i].id;
    }
    e = launch_scatter_desc(c->d_table, (const int32_t*)((BlockDesc*)st.dp + n), (const BlockDesc*)st.dp, (int)n, cs);
    hipEvent_t updated = nullptr;
    if (e == hipSuccess) e = new_event(c, &updated);
    if (e == hipSuccess) e = hipEventRecord(updated, cs);
    if (e == hipSuccess) e = hipEventRecord(st.ev, cs);
    if (e != hipSuccess) {
        (void)hipStreamSynchronize(cs);
        // the device table may hold some new entries: restore the old ones
        for (auto& p : plans) (void)hipMemcpy(c->d_table + p.id, &c->h_table[p.id], sizeof(BlockDesc), hipMemcpyHostToDevice);
        put_staging(c, st);
        if (updated) c->evs.drop(updated);
        return hip_fail(e, "page-table update");
    }
    put_staging(c, st);
    // commit on the host; old slabs are recycled after `updated`
    for (size_t i = 0; i < plans.size(); ++i) {
        HostBlock& b = c->blocks[plans[i].id];
        for (int j = plans[i].qn; j < plans[i].qo; ++j) {
            c->pool.release_after(b.dplanes[j], (size_t)b.pw * 4, j, updated);
            b.dplanes[j] = nullptr;
        }
        for (int j = plans[i].qo; j < plans[i].qn; ++j) b.dplanes[j] = plans[i].planes[j];
        c->pool.release_after(b.dlut, lut_bytes(b.S, b.q), SlabPool::kLutTag, updated);
        b.dlut = plans[i].lut;
        b.q = plans[i].qn;
        c->h_table[plans[i].id] = newdesc[i];
    }
    c->evs.drop(updated);  // the released slabs hold it until they are reclaimed
    return ok();
}

// Shared argument checks: registered ids, widths in range, no duplicates, no
// block with a request in flight.  Collects the blocks whose width changes.
static pw_status check_changes(pw_ctx* c, const char* fn, int n, const int32_t* ids, const uint8_t* q_new,
                               std::vector<std::pair<int, int>>& todo)
{
    if (n < 0) return fail(PW_ERR_INVALID, "%s: n < 0", fn);
    if (n > 0 && (!ids || !q_new)) return fail(PW_ERR_INVALID, "%s: null pointer", fn);
    std::unordered_set<int32_t> seen;
    for (int i = 0; i < n; ++i) {
        const int32_t id = ids[i];
        if (id < 0 || id >= c->nblocks || !c->blocks[id].registered)
            return fail(PW_ERR_INVALID, "%s: block id %d not registered", fn, id);
        if (q_new[i] < PW_QMIN || q_new[i] > PW_QMAX) return fail(PW_ERR_INVALID, "%s: q %d not in 3..8", fn, (int)q_new[i]);
        if (!seen.insert(id).second) return fail(PW_ERR_INVALID, "%s: duplicate block id %d", fn, id);
        if (c->pending.count(id)) return fail(PW_ERR_STATE, "%s: block id %d has a width request in flight", fn, id);
    }
    todo.clear();
    for (int i = 0; i < n; ++i)
        if (q_new[i] != c->blocks[ids[i]].q) todo.push_back({ids[i], (int)q_new[i]});
    if (!todo.empty() && !c->d.keep_host_masters)
        return fail(PW_ERR_STATE, "%s: the context keeps no host masters (keep_host_masters = 0)", fn);
    return ok();
}

pw_status pw_set_committed_bits(pw_ctx* c, int n, const int32_t* ids, const uint8_t* q_new, pw_stream compute,
                                pw_stream copy)
{
    return guarded("pw_set_committed_bits", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_set_committed_bits: null context");
        std::vector<std::pair<int, int>> todo;
        pw_status st = check_changes(c, "pw_set_committed_bits", n, ids, q_new, todo);
        if (st != PW_OK || todo.empty()) return st;
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        hipStream_t cs = (hipStream_t)compute, xs = (hipStream_t)copy;
        std::vector<WidthChange> plans;
        if ((st = prepare_changes(c, "pw_set_committed_bits", todo, xs, false, plans)) != PW_OK) return st;
        if ((e = hipStreamWaitEvent(cs, plans[0].copied, 0)) != hipSuccess) {
            (void)hipStreamSynchronize(xs);
            release_prepared(c, plans);
            return hip_fail(e, "pw_set_committed_bits: compute waits for the copies");
        }
        if ((st = apply_changes(c, plans, cs)) != PW_OK) {
            (void)hipStreamSynchronize(xs);
            release_prepared(c, plans);
            return st;
        }
        drop_copy_events(c, plans);
        return st;
    });
}

pw_status pw_request_widths(pw_ctx* c, int n, const int32_t* ids, const uint8_t* q_desired, pw_stream copy)
{
    return guarded("pw_request_widths", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_request_widths: null context");
        std::vector<std::pair<int, int>> todo;
        pw_status st = check_changes(c, "pw_request_widths", n, ids, q_desired, todo);
        if (st != PW_OK || todo.empty()) return st;
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        std::vector<WidthChange> plans;
        if ((st = prepare_changes(c, "pw_request_widths", todo, (hipStream_t)copy, true, plans)) != PW_OK) return st;
        for (const auto& p : plans) c->pending[p.id] = p;
        return ok();
    });
}

pw_status pw_commit_ready(pw_ctx* c, pw_stream compute, int* n_committed)
{
    return guarded("pw_commit_ready", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_commit_ready: null context");
        if (n_committed) *n_committed = 0;
        if (c->pending.empty()) return ok();
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        std::vector<WidthChange> ready;
        for (const auto& kv : c->pending) {
            const hipError_t q = hipEventQuery(kv.second.copied);
            if (q == hipSuccess) ready.push_back(kv.second);
            else if (q != hipErrorNotReady) return hip_fail(q, "pw_commit_ready: copy event");
        }
        if (ready.empty()) return ok();
        std::sort(ready.begin(), ready.end(), [](const WidthChange& a, const WidthChange& b) { return a.id < b.id; });
        const pw_status st = apply_changes(c, ready, (hipStream_t)compute);
        if (st != PW_OK) return st;
        drop_copy_events(c, ready);
        for (const auto& p : ready) c->pending.erase(p.id);
        if (n_committed) *n_committed = (int)ready.size();
        return ok();
    });
}

pw_status pw_block_state(const pw_ctx* c, int32_t id, int32_t* q_committed, int32_t* q_desired, int32_t* state)
{
    return guarded("pw_block_state", [&]() -> pw_status {
        if (!c || !q_committed || !q_desired || !state) return fail(PW_ERR_INVALID, "pw_block_state: null pointer");
        if (id < 0 || id >= c->nblocks || !c->blocks[id].registered)
            return fail(PW_ERR_INVALID, "pw_block_state: block id %d not registered", id);
        *q_committed = c->blocks[id].q;
        const auto it = c->pending.find(id);
        if (it == c->pending.end()) {
            *q_desired = c->blocks[id].q;
            *state = PW_PAGE_RESIDENT;
            return ok();
        }
        *q_desired = it->second.qn;
        const hipError_t q = hipEventQuery(it->second.copied);
        if (q != hipSuccess && q != hipErrorNotReady) return hip_fail(q, "pw_block_state: copy event");
        *state = q == hipSuccess ? PW_PAGE_READY : PW_PAGE_IN_TRANSFER;
        return ok();
    });
}

pw_status pw_committed_widths(const pw_ctx* c, uint8_t* q_out)
{
    return guarded("pw_committed_widths", [&]() -> pw_status {
        if (!c || !q_out) return fail(PW_ERR_INVALID, "pw_committed_widths: null pointer");
        for (int id = 0; id < c->nblocks; ++id) q_out[id] = c->blocks[id].registered ? (uint8_t)c->blocks[id].q : 0;
        return ok();
    });
}

pw_status pw_routing_mass_copy(pw_ctx* c, double* dst, pw_stream stream)
{
    return guarded("pw_routing_mass_copy", [&]() -> pw_status {
        if (!c || !dst) return fail(PW_ERR_INVALID, "pw_routing_mass_copy: null pointer");
        if (!c->d_mass) return fail(PW_ERR_STATE, "pw_routing_mass_copy: routing mass was never enabled");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        const size_t bytes = sizeof(double) * (size_t)c->d.num_layers * c->d.num_experts;
        e = hipMemcpyAsync(dst, c->d_mass, bytes, hipMemcpyDefault, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "pw_routing_mass_copy");
    });
}

pw_status pw_plane_states(const pw_ctx* c, int32_t id, int32_t* states)
{
    return guarded("pw_plane_states", [&]() -> pw_status {
        if (!c || !states) return fail(PW_ERR_INVALID, "pw_plane_states: null pointer");
        if (id < 0 || id >= c->nblocks || !c->blocks[id].registered)
            return fail(PW_ERR_INVALID, "pw_plane_states: block id %d not registered", id);
        const HostBlock& b = c->blocks[id];
        const int off_gpu = c->d.keep_host_masters ? PW_PLANE_CPU : PW_PLANE_ABSENT;
        const auto it = c->pending.find(id);
        if (it == c->pending.end()) {
            for (int p = 0; p < 8; ++p) states[p] = p < b.q ? PW_PLANE_GPU : off_gpu;
            states[8] = PW_PLANE_GPU;
            return ok();
        }
        const hipError_t q = hipEventQuery(it->second.copied);
        if (q != hipSuccess && q != hipErrorNotReady) return hip_fail(q, "pw_plane_states: copy event");
        const int moving = q == hipSuccess ? PW_PLANE_READY : PW_PLANE_IN_TRANSFER;
        const int qo = it->second.qo, qn = it->second.qn;
        for (int p = 0; p < 8; ++p) {
            if (p < qo) states[p] = PW_PLANE_GPU;  // lowering: planes qn..qo-1 stay in use until the commit
            else if (p < qn) states[p] = moving;
            else states[p] = off_gpu;
        }
        states[8] = moving;  // LUT_{d_i}
        return ok();
    });
}

pw_status pw_trim(pw_ctx* c, int64_t* freed_bytes)
{
    return guarded("pw_trim", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_trim: null context");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        const size_t freed = c->pool.trim();
        if (freed_bytes) *freed_bytes = (int64_t)freed;
        return ok();
    });
}

pw_status pw_pool_stats(const pw_ctx* c, int64_t* resident, int64_t* cached, int64_t* waiting, int64_t* held,
                        int64_t* device_allocs, int64_t* events)
{
    return guarded("pw_pool_stats", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_pool_stats: null context");
        if (resident) *resident = c->pool.resident();
        if (cached) *cached = c->pool.free_bytes();
        if (waiting) *waiting = c->pool.waiting_bytes();
        if (held) *held = c->pool.held();
        if (device_allocs) *device_allocs = c->pool.device_allocs();
        if (events) *events = (int64_t)c->evs.created();
        return ok();
    });
}

pw_status pw_retarget(pw_ctx* c, int64_t byte_target, const double* mass, const float* sens,
                      const pw_plan_params* params, pw_stream copy, int* n_requested, int64_t* planned_bytes)
{
    return guarded("pw_retarget", [&]() -> pw_status {
        if (!c || !mass || !sens || !params) return fail(PW_ERR_INVALID, "pw_retarget: null pointer");
        if (n_requested) *n_requested = 0;
        const int L = c->d.num_layers, E = c->d.num_experts;
        std::vector<uint8_t> q_cur((size_t)L * E * 2), q_plan(q_cur.size());
        for (int l = 0; l < L; ++l)
            for (int e = 0; e < E; ++e)
                for (int m = 0; m < 2; ++m) {
                    const int id = (l * (E + 1) + e) * 2 + m;
                    if (!c->blocks[id].registered)
                        return fail(PW_ERR_STATE, "pw_retarget: block (layer %d, expert %d, module %d) not registered", l, e, m);
                    const auto it = c->pending.find(id);
                    q_cur[((size_t)l * E + e) * 2 + m] = (uint8_t)(it == c->pending.end() ? c->blocks[id].q : it->second.qn);
                }
        int64_t total = 0;
        pw_status st = pw_plan_widths(L, E, c->d.hidden, c->d.inter, q_cur.data(), mass, sens, params, byte_target,
                                      q_plan.data(), &total);
        if (st != PW_OK) return st;
        std::vector<int32_t> ids;
        std::vector<uint8_t> qs;
        for (int l = 0; l < L; ++l)
            for (int e = 0; e < E; ++e)
                for (int m = 0; m < 2; ++m) {
                    const size_t b = ((size_t)l * E + e) * 2 + m;
                    const int id = (l * (E + 1) + e) * 2 + m;
                    if (q_plan[b] != q_cur[b] && !c->pending.count(id)) {
                        ids.push_back(id);
                        qs.push_back(q_plan[b]);
                    }
                }
        if (!ids.empty()) {
            st = pw_request_widths(c, (int)ids.size(), ids.data(), qs.data(), copy);
            if (st != PW_OK) return st;
        }
        if (n_requested) *n_requested = (int)ids.size();
        if (planned_bytes) *planned_bytes = total;
        return ok();
    });
}

pw_status pw_debug_decode(pw_ctx* c, int32_t id, int path, uint8_t* codes_out, uint16_t* w_out, pw_stream stream)
{
    return guarded("pw_debug_decode", [&]() -> pw_status {
        if (!c || (!codes_out && !w_out)) return fail(PW_ERR_INVALID, "pw_debug_decode: null pointer");
        if (id < 0 || id >= c->nblocks || !c->blocks[id].registered)
            return fail(PW_ERR_INVALID, "pw_debug_decode: block id %d not registered", id);
        if (path < PW_DECODE_PATH_TILE128 || path > PW_DECODE_PATH_TILE64_WIDE)
            return fail(PW_ERR_INVALID, "pw_debug_decode: path %d not in 0..3", path);
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        e = launch_debug_decode(c->d_table + id, id & 1, c->blocks[id].R, path, codes_out, w_out, (hipStream_t)stream);
        return e == hipSuccess ? ok() : hip_fail(e, "debug decode launch");
    });
}

// The decode contraction's tile of each module: gate_up 128-row tiles, down
// 64-row tiles.
static int default_decode_path(int32_t id) { return (id & 1) ? PW_DECODE_PATH_TILE64 : PW_DECODE_PATH_TILE128; }

pw_status pw_debug_decode_codes(pw_ctx* c, int32_t id, uint8_t* out, pw_stream stream)
{
    return guarded("pw_debug_decode_codes", [&]() -> pw_status {
        if (!out) return fail(PW_ERR_INVALID, "pw_debug_decode_codes: null pointer");
        return pw_debug_decode(c, id, default_decode_path(id), out, nullptr, stream);
    });
}

pw_status pw_debug_dequant(pw_ctx* c, int32_t id, uint16_t* out, pw_stream stream)
{
    return guarded("pw_debug_dequant", [&]() -> pw_status {
        if (!out) return fail(PW_ERR_INVALID, "pw_debug_dequant: null pointer");
        return pw_debug_decode(c, id, default_decode_path(id), nullptr, out, stream);
    });
}

pw_status pw_profile_enable(pw_ctx* c, int on)
{
    return guarded("pw_profile_enable", [&]() -> pw_status {
        if (!c) return fail(PW_ERR_INVALID, "pw_profile_enable: null context");
        hipError_t e = hipSetDevice(c->device);
        if (e != hipSuccess) return hip_fail(e, "hipSetDevice");
        (void)hipDeviceSynchronize();
        prof_reset(c);
        if (on && c->prof_pool.empty()) {
            c->prof_pool.reserve(kProfEvents);
            for (size_t i = 0; i < kProfEvents; ++i) {
                hipEvent_t ev;
                if ((e = hipEventCreate(&ev)) != hipSuccess) {
                    prof_release(c);
                    return hip_fail(e, "pw_profile_enable: hipEventCreate");
                }
                c->prof_pool.push_back(ev);
            }
        }
        c->profiling = on != 0;
        return ok();
    });
}

pw_status pw_profile_read(pw_ctx* c, const char* kernel, double* total_ms, int64_t* launches)
{
    return guarded("pw_profile_read", [&]() -> pw_status {
        if (!c || !kernel || !total_ms || !launches) return fail(PW_ERR_INVALID, "pw_profile_read: null pointer");
        *total_ms = 0.0;
        *launches = 0;
        auto it = c->prof.find(kernel);
        if (it == c->prof.end()) return ok();
        for (auto& r : it->second) {
            float ms = 0.0f;
            hipError_t e = hipEventElapsedTime(&ms, r.a, r.b);
            if (e != hipSuccess) return hip_fail(e, "pw_profile_read: hipEventElapsedTime (stream not synchronised?)");
            *total_ms += ms;
            *launches += 1;
        }
        return ok();
    });
}

}  // extern "C"

namespace pw {

WsLayout ws_layout(int T, int k, int H, int I, int Is)
{
    auto up = [](size_t b) { return (b + 255) & ~size_t(255); };
    const size_t rows = (size_t)T * k + (Is ? (size_t)T : 0);
    const size_t hs = (size_t)std::max(I, Is);
    const size_t splits = (size_t)std::max(down_splits(I), Is ? down_splits(Is) : 1);
    WsLayout L;
    L.h = 0;
    L.dout = up(L.h + rows * hs * 2);
    L.total = up(L.dout + splits * rows * (size_t)H * 4);
    return L;
}

}  // namespace pw
