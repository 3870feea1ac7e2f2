// kev_api.hip -- the C ABI: argument checks, stream-ordered workspace, per-stream error words,
// launches.
//
// Everything host-checkable is checked before the first HIP call.  The
// boundary follows the pages' statement of the problem: the packed stream plus
// question intervals in cu_seqlens form, never a dense mask (Kev article,
// icman.com.cn, sections 2.2, 5.2, 6.4); one fixed-capacity slot per question
// in a caller-owned pool that is passed in explicitly rather than held as
// hidden state (Kev part 2, gsyq.cn, section 2.2; KV-cache isolation article,
// hnwysp.cn, section 3.3); and a slot that would overflow is an error, never a
// re-layout (Kev part 2, section 4.2).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdio>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/kev.h"
#include "kev_host.h"
#include "kev_internal.h"

namespace {

using namespace kev;

struct Buffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};

struct DevPool {
    bool tried = false;
    hipMemPool_t pool = nullptr;   // null: the device has no stream-ordered allocator
};

struct State {
    std::mutex mu;
    std::map<std::pair<int, void *>, int32_t *> err_word;    // (device, stream) -> error word
    std::map<int, DevPool> pools;                            // device -> workspace pool
    std::map<std::pair<int, void *>, Buffer> cached_ws;      // fallback workspace per (device, stream)
    std::map<int, int32_t *> scratch_ptr;                    // device -> address of `scratch`
};

State &state() {
    static State *s = new State();   // never destroyed: outlives static teardown order
    return *s;
}

// Scratch of the no-allocation prefill (kev_packed_attn_prefill_noalloc): a file-scope device
// array, one copy per GPU, held until the process ends.  Word 0 is that entry point's error
// word; its work-list tables start 256 bytes in.  In host code `scratch` only names the
// symbol: its device address on each GPU comes from hipGetSymbolAddress (scratch_on).
constexpr size_t kScratchBytes = (size_t)4 << 20;
constexpr size_t kScratchTables = 256;   // bytes before the tables (the error word lives there)
static __device__ __align__(256) int32_t scratch[kScratchBytes / sizeof(int32_t)];

// Device address of `scratch` on device `dev` (looked up once per device, with it current).
int scratch_on(int dev, int32_t **out) {
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    auto it = st.scratch_ptr.find(dev);
    if (it != st.scratch_ptr.end()) {
        *out = it->second;
        return KEV_OK;
    }
    int32_t *ptr = nullptr;
    if (hipGetSymbolAddress((void **)&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KEV_ERR_DEVICE;
    st.scratch_ptr[dev] = ptr;
    *out = ptr;
    return KEV_OK;
}

// Events the calls of this host thread record around their main kernel (kev_set_kernel_events).
thread_local hipEvent_t t_ev_start = nullptr, t_ev_end = nullptr;

// Launch `f` (returning hipError_t) between the optional timing events.
template <typename F>
int timed_launch(hipStream_t stream, F f) {
    if (t_ev_start && hipEventRecord(t_ev_start, stream) != hipSuccess) return KEV_ERR_DEVICE;
    const hipError_t e = f();
    if (e != hipSuccess) return KEV_ERR_DEVICE;
    if (t_ev_end && hipEventRecord(t_ev_end, stream) != hipSuccess) return KEV_ERR_DEVICE;
    return KEV_OK;
}

bool env_flag(const char *name) {
    const char *e = std::getenv(name);
    return e && e[0] == '1';
}
bool check_enabled() { return env_flag("KEV_CHECK"); }
bool log_enabled() { return env_flag("KEV_LOG"); }

int to_status(hipError_t e) { return e == hipSuccess ? KEV_OK : KEV_ERR_DEVICE; }

// Error word of (device, stream): the kernels a call enqueues on `stream` set bits in it, and
// kev_get_device_errors(stream) reads and clears it, so streams never see each other's flags.
// Allocated and zeroed on the first call on that stream (kept until the process ends).
int error_word(int dev, hipStream_t stream, int32_t **out) {
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    const auto key = std::make_pair(dev, (void *)stream);
    auto it = st.err_word.find(key);
    if (it != st.err_word.end()) {
        *out = it->second;
        return KEV_OK;
    }
    int32_t *p = nullptr;
    if (hipMalloc(&p, 256) != hipSuccess) return KEV_ERR_NO_MEMORY;
    if (hipMemset(p, 0, 256) != hipSuccess) return KEV_ERR_DEVICE;
    st.err_word[key] = p;
    *out = p;
    return KEV_OK;
}

// Workspace of one call.  Taken stream-ordered from a library-owned pool of the device
// (hipMallocFromPoolAsync on the caller's stream, returned with hipFreeAsync on the same
// stream after the call's last kernel): nothing synchronises, concurrent streams never share
// memory, and the pool keeps its memory between calls (release threshold at the maximum).
// Devices without a stream-ordered allocator fall back to one cached buffer per (device,
// stream) that grows on demand; growing it synchronises that stream.
struct Workspace {
    void *ptr = nullptr;
    bool pooled = false;
};

hipMemPool_t device_pool(int dev) {
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    DevPool &dp = st.pools[dev];
    if (!dp.tried) {
        dp.tried = true;
        int ok = 0;
        if (!std::getenv("KEV_NO_MEMPOOL") &&
            hipDeviceGetAttribute(&ok, hipDeviceAttributeMemoryPoolsSupported, dev) == hipSuccess && ok) {
            hipMemPoolProps props;
            std::memset(&props, 0, sizeof props);
            props.allocType = hipMemAllocationTypePinned;
            props.handleTypes = hipMemHandleTypeNone;
            props.location.type = hipMemLocationTypeDevice;
            props.location.id = dev;
            hipMemPool_t pool = nullptr;
            if (hipMemPoolCreate(&pool, &props) == hipSuccess) {
                uint64_t keep = UINT64_MAX;
                if (hipMemPoolSetAttribute(pool, hipMemPoolAttrReleaseThreshold, &keep) == hipSuccess) dp.pool = pool;
                else hipMemPoolDestroy(pool);
            }
        }
        (void)hipGetLastError();   // a refused attribute or pool is not an error of this call
    }
    return dp.pool;
}

int workspace_acquire(int dev, hipStream_t stream, size_t bytes, Workspace *ws) {
    bytes = std::max(bytes, (size_t)256);
    if (hipMemPool_t pool = device_pool(dev)) {
        if (hipMallocFromPoolAsync(&ws->ptr, bytes, pool, stream) != hipSuccess) {
            ws->ptr = nullptr;
            return KEV_ERR_NO_MEMORY;
        }
        ws->pooled = true;
        return KEV_OK;
    }
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    Buffer &b = st.cached_ws[{dev, (void *)stream}];
    if (b.bytes < bytes) {
        if (b.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return KEV_ERR_DEVICE;
            if (hipFree(b.ptr) != hipSuccess) return KEV_ERR_DEVICE;
            b.ptr = nullptr;
            b.bytes = 0;
        }
        const size_t want = std::max(bytes, (size_t)1 << 16);
        if (hipMalloc(&b.ptr, want) != hipSuccess) {
            b.ptr = nullptr;
            return KEV_ERR_NO_MEMORY;
        }
        b.bytes = want;
    }
    ws->ptr = b.ptr;
    ws->pooled = false;
    return KEV_OK;
}

// Returns the workspace once every kernel of the call that uses it has been enqueued.
int workspace_release(Workspace &ws, hipStream_t stream) {
    if (!ws.pooled || !ws.ptr) return KEV_OK;
    const hipError_t e = hipFreeAsync(ws.ptr, stream);
    ws.ptr = nullptr;
    return to_status(e);
}

bool prefill_supported(int32_t head_dim, int32_t dtype) {
    if (dtype == KEV_BF16) return head_dim == 64 || head_dim == 128;
    if (dtype == KEV_F32) return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
    return false;
}

int32_t block_rows_for(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype) {
    if (dtype == KEV_F32) return kF32BlockRows;
    return prefill_shape_bf16(heads, kv_heads, head_dim).block_rows;
}

// Item order of a prefill call: question-major, so concurrently running workgroups share one
// question's K/V rows in their XCD's L2.  Level-major (longest items first overall) is kept
// for the schedule entry points; on the Qwen-shaped workloads it timed the same within noise
// while reading about 40% more bytes from HBM, so calls do not use it.
int32_t prefill_order(int32_t total_tokens, int32_t head_dim, int32_t dtype) {
    (void)total_tokens;
    (void)head_dim;
    (void)dtype;
    return kOrderQuestion;
}

// Copies `n` int32 of device memory to the host and waits (KEV_CHECK / KEV_LOG only).
bool fetch(std::vector<int32_t> &dst, const int32_t *src, size_t n, hipStream_t stream) {
    dst.resize(n);
    return n == 0 || (hipMemcpyAsync(dst.data(), src, sizeof(int32_t) * n, hipMemcpyDeviceToHost, stream) ==
                          hipSuccess &&
                      hipStreamSynchronize(stream) == hipSuccess);
}

// XCDs of a device (workgroups of a launch are dealt to them round-robin), 1 if unknown.
int xcd_count(int dev) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        return 1;
    }
    return n;
}

// Item streams of a bf16 prefill (1 = one question-major work list).  When an XCD would
// otherwise share a (question, KV head) pair with another XCD (fewer KV heads than XCDs), the
// questions are split into n_xcd / kv_heads streams and every XCD serves one (stream, KV head)
// pair, so a question's K/V rows are fetched into one L2 only.  Used for two streams with at
// least 4 questions each way, at most 64 questions (the one-wavefront work-list pass deals
// them); KEV_XCD_STREAMS=0 turns it off.
int32_t prefill_streams(int32_t kv_heads, int32_t n_seg, int n_xcd, int32_t dtype) {
    if (dtype != KEV_BF16 || n_xcd <= kv_heads || n_xcd % kv_heads != 0) return 1;
    if (const char *e = std::getenv("KEV_XCD_STREAMS"))
        if (e[0] == '0') return 1;
    const int32_t n = n_xcd / kv_heads;
    if (n > 2 || n > kStreamsMax || n_seg > 64 || n_seg < 4 * n) return 1;
    return n;
}

// Schedule-table geometry of a prefill call.
struct PrefillPlan {
    int32_t block_rows, hist_len, n_streams, n_xcd;
    int64_t n_max;   // item capacity per stream
    ScheduleLayout lay;
};

int plan_prefill(int32_t n_seg, int32_t total_tokens, int32_t heads, int32_t kv_heads, int32_t head_dim,
                 int32_t dtype, int dev, PrefillPlan *pl) {
    pl->block_rows = block_rows_for(heads, kv_heads, head_dim, dtype);
    pl->n_max = max_items(total_tokens, n_seg, pl->block_rows);
    pl->n_xcd = xcd_count(dev);
    pl->n_streams = prefill_streams(kv_heads, n_seg, pl->n_xcd, dtype);
    const int64_t hist_len = qblocks(total_tokens, pl->block_rows) + 2;
    if (hist_len > INT32_MAX || pl->n_max * pl->n_streams > INT32_MAX / 4) return KEV_ERR_INVALID_ARG;
    pl->hist_len = (int32_t)hist_len;
    pl->lay = schedule_layout(n_seg, pl->hist_len, pl->n_max * pl->n_streams);
    return KEV_OK;
}

// Slot side of a chunked prefill: question s continues prefix_lens[s] rows of slot slot_ids[s].
struct SlotPrefix {
    const kev_kv_pool *pool;
    const int32_t *slot_ids, *prefix_lens;
};

// Host checks of a prefill call (everything that needs no device memory).
int check_prefill_args(const void *q, const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg,
                       int32_t heads, int32_t kv_heads, int32_t head_dim, const void *out, int32_t total_tokens,
                       int32_t dtype, const SlotPrefix *pre) {
    if (n_seg < 0 || total_tokens < 0 || heads <= 0 || kv_heads <= 0 || head_dim <= 0)
        return KEV_ERR_INVALID_ARG;
    if (heads % kv_heads != 0) return KEV_ERR_INVALID_ARG;
    if (dtype != KEV_BF16 && dtype != KEV_F32) return KEV_ERR_UNSUPPORTED;
    if (!prefill_supported(head_dim, dtype)) return KEV_ERR_UNSUPPORTED;
    if (pre && dtype != KEV_BF16) return KEV_ERR_UNSUPPORTED;   // slot prefixes: bf16 pools only
    if (n_seg == 0) return total_tokens == 0 ? KEV_OK : KEV_ERR_BAD_SEQLENS;
    if (!cu_seqlens) return KEV_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !out)) return KEV_ERR_INVALID_ARG;
    return KEV_OK;
}

// Enqueues the work-list pass and the attention kernel of a checked prefill call, with its
// schedule tables at `ws` (plan.lay.total int32) and its error word at `err`.
int enqueue_prefill(const void *q, const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg,
                    int32_t heads, int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                    int32_t dtype, const SlotPrefix *pre, const PrefillPlan &pl, int32_t *ws, int32_t *err,
                    hipStream_t stream, bool may_log = true) {
    ScheduleArgs sa{cu_seqlens, n_seg, total_tokens, pl.block_rows, pl.hist_len,
                    prefill_order(total_tokens, head_dim, dtype), pl.n_max, ws, err,
                    pre ? pre->prefix_lens : nullptr, pl.n_streams};
    int rc = to_status(launch_schedule(sa, stream));
    if (rc) return rc;
    if (may_log && log_enabled()) {
        std::vector<int32_t> n;
        if (!fetch(n, ws, 1, stream)) return KEV_ERR_DEVICE;
        std::fprintf(stderr, "[kev] prefill: %d questions, %d tokens, %d/%d heads, d=%d; %d items of %d rows "
                             "(capacity %lld), %d stream(s) over %d XCDs, workspace %lld B%s\n",
                     n_seg, total_tokens, heads, kv_heads, head_dim, n[0], pl.block_rows, (long long)pl.n_max,
                     pl.n_streams, pl.n_xcd, (long long)(pl.lay.total * 4), pre ? ", slot prefixes" : "");
    }
    if (total_tokens == 0) return KEV_OK;   // only empty questions; cu_seqlens still checked

    PrefillArgs pa{};
    pa.q = q;
    pa.k = k;
    pa.v = v;
    pa.out = out;
    pa.cu = cu_seqlens;
    pa.sched = ws;
    pa.items_off = pl.lay.items;
    pa.rec = ws + pl.lay.rec;
    pa.heads = heads;
    pa.kv_heads = kv_heads;
    pa.group = heads / kv_heads;
    pa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    pa.err = err;
    if (dtype == KEV_BF16) {
        const PrefillShape sh = prefill_shape_bf16(heads, kv_heads, head_dim);
        pa.row_blocks = sh.row_blocks;
        pa.block_rows = sh.block_rows;
        pa.wg_per_kvh = sh.wg_per_kvh;
        pa.n_streams = pl.n_streams;
        pa.n_xcd = pl.n_xcd;
        pa.stream_cap = (int32_t)pl.n_max;
        const int64_t grid = pl.n_max * pl.n_streams * kv_heads * sh.wg_per_kvh;
        if (grid > INT32_MAX) return KEV_ERR_INVALID_ARG;
        if (pre) {
            pa.slot_ids = pre->slot_ids;
            pa.prefix_lens = pre->prefix_lens;
            pa.pool = pre->pool->data;
            pa.n_slots = pre->pool->n_slots;
            pa.capacity = pre->pool->capacity;
        }
        return timed_launch(stream, [&] { return launch_prefill_bf16(pa, head_dim, grid, pre != nullptr, stream); });
    }
    pa.heads_per_wg = 1;
    pa.row_blocks = 1;
    pa.block_rows = kF32BlockRows;
    pa.n_hgroups = heads;
    const int64_t grid = pl.n_max * heads;
    if (grid > INT32_MAX) return KEV_ERR_INVALID_ARG;
    return timed_launch(stream, [&] { return launch_prefill_f32(pa, head_dim, grid, stream); });
}

// KEV_CHECK of cu_seqlens (synchronous).
int check_seqlens_on_host(const int32_t *cu_seqlens, int32_t n_seg, int32_t total_tokens, hipStream_t stream) {
    std::vector<int32_t> h;
    if (!fetch(h, cu_seqlens, (size_t)n_seg + 1, stream)) return KEV_ERR_DEVICE;
    return host::check_seqlens(h.data(), n_seg, total_tokens);
}

// Packed prefill; with `pre`, every question is a chunk continuing its slot's cached rows.
// The schedule tables come from the call's stream-ordered workspace.
int prefill_impl(const void *q, const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg,
                 int32_t heads, int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                 int32_t dtype, void *stream_, const SlotPrefix *pre) {
    int rc = check_prefill_args(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype,
                                pre);
    if (rc || n_seg == 0) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (check_enabled()) {
        rc = check_seqlens_on_host(cu_seqlens, n_seg, total_tokens, stream);
        if (rc) return rc;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    PrefillPlan pl;
    rc = plan_prefill(n_seg, total_tokens, heads, kv_heads, head_dim, dtype, dev, &pl);
    if (rc) return rc;
    int32_t *err = nullptr;
    rc = error_word(dev, stream, &err);
    if (rc) return rc;
    Workspace ws;
    rc = workspace_acquire(dev, stream, (size_t)pl.lay.total * sizeof(int32_t), &ws);
    if (rc) return rc;
    rc = enqueue_prefill(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype, pre, pl,
                         static_cast<int32_t *>(ws.ptr), err, stream);
    const int rc2 = workspace_release(ws, stream);
    return rc ? rc : rc2;
}

// Arguments shared by the two slot-writing prefills: a bf16 pool that matches the K/V heads.
int check_pool(const kev_kv_pool *pool, int32_t n_seg, int32_t total_tokens, int32_t kv_heads,
               int32_t head_dim, const int32_t *slot_ids) {
    if (!pool || n_seg < 0 || total_tokens < 0 || kv_heads <= 0) return KEV_ERR_INVALID_ARG;
    if (pool->dtype != KEV_BF16) return KEV_ERR_UNSUPPORTED;
    if (pool->kv_heads != kv_heads || pool->head_dim != head_dim || pool->n_slots <= 0 ||
        pool->capacity <= 0)
        return KEV_ERR_INVALID_ARG;
    if (n_seg > 0 && (!slot_ids || !pool->data)) return KEV_ERR_INVALID_ARG;
    if (n_seg > pool->n_slots) return KEV_ERR_BAD_SLOT;
    return KEV_OK;
}

// KEV_CHECK: slot ids in range and distinct, and every question's rows (after its prefix,
// if any) fit the slot.
int check_slots_on_host(const kev_kv_pool *pool, const int32_t *slot_ids, const int32_t *prefix_lens,
                        const int32_t *cu_seqlens, int32_t n_seg, hipStream_t stream) {
    std::vector<int32_t> ids, cu, pre;
    if (!fetch(ids, slot_ids, (size_t)n_seg, stream) || !fetch(cu, cu_seqlens, (size_t)n_seg + 1, stream) ||
        (prefix_lens && !fetch(pre, prefix_lens, (size_t)n_seg, stream)))
        return KEV_ERR_DEVICE;
    return host::check_slot_list(ids.data(), prefix_lens ? pre.data() : nullptr, cu.data(), n_seg, pool->n_slots,
                                 pool->capacity);
}

// Write every question's K/V rows into its slot, after its prefix rows if any.
int store_rows(const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg, int32_t kv_heads,
               int32_t head_dim, int32_t total_tokens, const kev_kv_pool *pool, const int32_t *slot_ids,
               const int32_t *prefix_lens, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t *err = nullptr;
    int rc = error_word(dev, stream, &err);
    if (rc) return rc;
    StoreKvArgs sa{k, v, cu_seqlens, slot_ids, prefix_lens, pool->data, n_seg, total_tokens, kv_heads,
                   pool->n_slots, pool->capacity, err};
    return to_status(launch_store_kv(sa, head_dim, stream));
}

// Decode shapes the kernel covers: bf16, head_dim 64 or 128, up to 32 query heads per KV head
// (they are the columns of one MFMA tile).
int check_decode_shape(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype) {
    if (heads % kv_heads != 0) return KEV_ERR_INVALID_ARG;
    if (dtype != KEV_BF16) return KEV_ERR_UNSUPPORTED;
    if (head_dim != 64 && head_dim != 128) return KEV_ERR_UNSUPPORTED;
    if (heads / kv_heads > 32) return KEV_ERR_UNSUPPORTED;
    return KEV_OK;
}

int forced_splits() {
    const char *e = std::getenv("KEV_DECODE_SPLITS");
    return e ? std::atoi(e) : 0;
}

// Launch a decode (slot or paged pool) once the pool-specific fields of `da` are set.
int run_decode(DecodeArgs &da, const void *q, void *data, int32_t kv_heads, int32_t head_dim,
               const int32_t *cache_lens, void *out, const void *k_new, const void *v_new, int32_t n_req,
               int32_t heads, bool paged, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int rc = error_word(dev, stream, &da.err);
    if (rc) return rc;
    da.q = q;
    da.pool = data;
    da.cache_lens = cache_lens;
    da.out = out;
    da.k_new = k_new;
    da.v_new = v_new;
    da.n_req = n_req;
    da.heads = heads;
    da.kv_heads = kv_heads;
    da.group = heads / kv_heads;
    da.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    const int64_t units = (int64_t)n_req * kv_heads;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1)
        return KEV_ERR_DEVICE;
    da.n_split = host::decode_splits(units, cus, forced_splits());
    if (units * da.n_split > INT32_MAX) return KEV_ERR_INVALID_ARG;
    // Unit order (requests ranked by length inside the kernel, at most 64 requests): longest
    // first when the grid does not fit the CUs at once (two workgroups each); when it fits but
    // some CUs hold two workgroups, a long and a short unit share each such CU (measured on the
    // 64-request decode workload: 61.4 us against 67.7 us in request order).
    da.ranked = 0;
    da.cus = cus;
    if (da.n_split == 1 && n_req <= 64) {
        if (units > 2 * (int64_t)cus) da.ranked = 1;
        else if (units > cus) da.ranked = 2;
    }
    const size_t part_bytes =
        da.n_split > 1 ? (size_t)units * da.n_split * da.group * (head_dim + 2) * sizeof(float) : 0;
    if (log_enabled())
        std::fprintf(stderr, "[kev] %s decode: %d requests, %d/%d heads, d=%d; %lld units x %d splits, "
                             "order %d, workspace %zu B\n",
                     paged ? "paged" : "slot", n_req, heads, kv_heads, head_dim, (long long)units, da.n_split,
                     da.ranked, part_bytes);
    Workspace ws;
    if (da.n_split > 1) {
        rc = workspace_acquire(dev, stream, part_bytes, &ws);
        if (rc) return rc;
        da.part = static_cast<float *>(ws.ptr);
    }
    rc = timed_launch(stream, [&] { return launch_decode_bf16(da, head_dim, paged, stream); });
    const int rc2 = workspace_release(ws, stream);
    return rc ? rc : rc2;
}

}  // namespace

extern "C" {

const char *kev_status_string(int status) {
    switch (status) {
    case KEV_OK: return "ok";
    case KEV_ERR_INVALID_ARG: return "invalid argument";
    case KEV_ERR_UNSUPPORTED: return "unsupported dtype/head_dim combination";
    case KEV_ERR_BAD_SEQLENS: return "cu_seqlens must start at 0, be non-decreasing and end at total_tokens";
    case KEV_ERR_SLOT_OVERFLOW: return "cache length (or prefix plus chunk rows) outside the slot or block-table capacity";
    case KEV_ERR_BAD_SLOT: return "slot or block id out of range, or repeated";
    case KEV_ERR_DEVICE: return "HIP runtime error";
    case KEV_ERR_NO_MEMORY: return "workspace allocation failed";
    case KEV_ERR_SCRATCH_LIMIT: return "work list larger than the no-allocation prefill's 4 MiB device scratch";
    default: return "unknown status";
    }
}

int kev_prefill_block_rows(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype) {
    if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) return 0;
    if (!prefill_supported(head_dim, dtype)) return 0;
    return block_rows_for(heads, kv_heads, head_dim, dtype);
}

int kev_packed_attn_prefill(const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int32_t n_seg,
                            int32_t heads, int32_t kv_heads, int32_t head_dim,
                            void *out, int32_t total_tokens, int32_t dtype, void *stream) {
    return prefill_impl(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype,
                        stream, nullptr);
}

int kev_packed_attn_prefill_noalloc(const void *q, const void *k, const void *v,
                                    const int32_t *cu_seqlens, int32_t n_seg,
                                    int32_t heads, int32_t kv_heads, int32_t head_dim,
                                    void *out, int32_t total_tokens, int32_t dtype, void *stream_) {
    int rc = check_prefill_args(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype,
                                nullptr);
    if (rc || n_seg == 0) return rc;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    PrefillPlan pl;
    rc = plan_prefill(n_seg, total_tokens, heads, kv_heads, head_dim, dtype, dev, &pl);
    if (rc) return rc;
    if ((size_t)pl.lay.total * sizeof(int32_t) > kScratchBytes - kScratchTables) return KEV_ERR_SCRATCH_LIMIT;
    int32_t *sp = nullptr;
    rc = scratch_on(dev, &sp);
    if (rc) return rc;
    return enqueue_prefill(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype, nullptr,
                           pl, sp + kScratchTables / sizeof(int32_t), sp, static_cast<hipStream_t>(stream_),
                           /*may_log=*/false);
}

int kev_packed_attn_prefill_slots(const void *q, const void *k, const void *v,
                                  const int32_t *cu_seqlens, int32_t n_seg, int32_t heads,
                                  int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                                  const kev_kv_pool *pool, const int32_t *slot_ids, void *stream_) {
    int rc = check_pool(pool, n_seg, total_tokens, kv_heads, head_dim, slot_ids);
    if (rc) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (check_enabled() && n_seg > 0) {
        rc = check_slots_on_host(pool, slot_ids, nullptr, cu_seqlens, n_seg, stream);
        if (rc) return rc;
    }
    rc = prefill_impl(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, KEV_BF16,
                      stream_, nullptr);
    if (rc || total_tokens == 0) return rc;
    return store_rows(k, v, cu_seqlens, n_seg, kv_heads, head_dim, total_tokens, pool, slot_ids, nullptr,
                      stream);
}

int kev_chunked_prefill_slots(const void *q, const void *k, const void *v, const int32_t *cu_seqlens,
                              int32_t n_seg, int32_t heads, int32_t kv_heads, int32_t head_dim, void *out,
                              int32_t total_tokens, const kev_kv_pool *pool, const int32_t *slot_ids,
                              const int32_t *prefix_lens, void *stream_) {
    int rc = check_pool(pool, n_seg, total_tokens, kv_heads, head_dim, slot_ids);
    if (rc) return rc;
    if (n_seg > 0 && !prefix_lens) return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (check_enabled() && n_seg > 0) {
        rc = check_slots_on_host(pool, slot_ids, prefix_lens, cu_seqlens, n_seg, stream);
        if (rc) return rc;
    }
    const SlotPrefix pre{pool, slot_ids, prefix_lens};
    rc = prefill_impl(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, KEV_BF16,
                      stream_, &pre);
    if (rc || total_tokens == 0) return rc;
    return store_rows(k, v, cu_seqlens, n_seg, kv_heads, head_dim, total_tokens, pool, slot_ids, prefix_lens,
                      stream);
}

int kev_slot_attn_decode(const void *q, const kev_kv_pool *pool, const int32_t *slot_ids,
                         const int32_t *cache_lens, void *out, const void *k_new,
                         const void *v_new, int32_t n_req, int32_t heads, void *stream_) {
    if (!pool || n_req < 0 || heads <= 0) return KEV_ERR_INVALID_ARG;
    if (pool->n_slots <= 0 || pool->capacity <= 0 || pool->kv_heads <= 0 || pool->head_dim <= 0)
        return KEV_ERR_INVALID_ARG;
    int rc = check_decode_shape(heads, pool->kv_heads, pool->head_dim, pool->dtype);
    if (rc) return rc;
    if (n_req == 0) return KEV_OK;
    if (n_req > pool->n_slots) return KEV_ERR_BAD_SLOT;
    if (!q || !pool->data || !slot_ids || !cache_lens || !out || !k_new || !v_new)
        return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);

    if (check_enabled()) {
        std::vector<int32_t> ids, lens;
        if (!fetch(ids, slot_ids, (size_t)n_req, stream) || !fetch(lens, cache_lens, (size_t)n_req, stream))
            return KEV_ERR_DEVICE;
        rc = host::check_decode(ids.data(), lens.data(), n_req, pool->n_slots, pool->capacity);
        if (rc) return rc;
    }
    DecodeArgs da{};
    da.slot_ids = slot_ids;
    da.n_slots = pool->n_slots;
    da.capacity = pool->capacity;
    return run_decode(da, q, pool->data, pool->kv_heads, pool->head_dim, cache_lens, out, k_new, v_new, n_req,
                      heads, false, stream);
}

int kev_paged_attn_decode(const void *q, const kev_paged_pool *pool, const int32_t *block_tables,
                          int32_t max_blocks, const int32_t *cache_lens, void *out, const void *k_new,
                          const void *v_new, int32_t n_req, int32_t heads, void *stream_) {
    if (!pool || n_req < 0 || heads <= 0 || max_blocks <= 0) return KEV_ERR_INVALID_ARG;
    if (pool->n_blocks <= 0 || pool->kv_heads <= 0 || pool->head_dim <= 0) return KEV_ERR_INVALID_ARG;
    const int32_t bs = pool->block_size;
    if (bs <= 0 || (bs & (bs - 1)) != 0) return KEV_ERR_INVALID_ARG;   // a power of two
    int rc = check_decode_shape(heads, pool->kv_heads, pool->head_dim, pool->dtype);
    if (rc) return rc;
    if (n_req == 0) return KEV_OK;
    if (!q || !pool->data || !block_tables || !cache_lens || !out || !k_new || !v_new)
        return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);

    if (check_enabled()) {
        std::vector<int32_t> tables, lens;
        if (!fetch(tables, block_tables, (size_t)n_req * max_blocks, stream) ||
            !fetch(lens, cache_lens, (size_t)n_req, stream))
            return KEV_ERR_DEVICE;
        rc = host::check_paged(tables.data(), lens.data(), n_req, max_blocks, pool->n_blocks, bs);
        if (rc) return rc;
    }
    DecodeArgs da{};
    da.n_slots = pool->n_blocks;
    da.capacity = bs;
    da.block_tables = block_tables;
    da.max_blocks = max_blocks;
    da.block_shift = __builtin_ctz((unsigned)bs);
    return run_decode(da, q, pool->data, pool->kv_heads, pool->head_dim, cache_lens, out, k_new, v_new, n_req,
                      heads, true, stream);
}

int kev_set_kernel_events(void *start, void *end) {
    if ((start == nullptr) != (end == nullptr)) return KEV_ERR_INVALID_ARG;
    t_ev_start = static_cast<hipEvent_t>(start);
    t_ev_end = static_cast<hipEvent_t>(end);
    return KEV_OK;
}

int kev_get_device_errors(void *stream_, int32_t *flags_out) {
    if (!flags_out) return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t *err = nullptr;
    int rc = error_word(dev, stream, &err);
    if (rc) return rc;
    int32_t v = 0, w = 0;
    // Stream order: the read follows every kernel enqueued on this stream before the call, and
    // the clear follows the read.
    if (hipMemcpyAsync(&v, err, sizeof v, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemsetAsync(err, 0, sizeof v, stream) != hipSuccess)
        return KEV_ERR_DEVICE;
    // The no-allocation prefill's error word (one per device, shared by every stream).
    int32_t *sp = nullptr;
    {
        State &st = state();
        std::lock_guard<std::mutex> lock(st.mu);
        auto it = st.scratch_ptr.find(dev);
        if (it != st.scratch_ptr.end()) sp = it->second;
    }
    if (sp && (hipMemcpyAsync(&w, sp, sizeof w, hipMemcpyDeviceToHost, stream) != hipSuccess ||
               hipMemsetAsync(sp, 0, sizeof w, stream) != hipSuccess))
        return KEV_ERR_DEVICE;
    if (hipStreamSynchronize(stream) != hipSuccess) return KEV_ERR_DEVICE;
    *flags_out = v | w;
    return KEV_OK;
}

int kev_prefill_order(int32_t total_tokens, int32_t head_dim, int32_t dtype) {
    return prefill_order(total_tokens, head_dim, dtype);
}

int kev_schedule_host(const int32_t *cu, int32_t n_seg, int32_t block_rows, int32_t order,
                      int32_t *items_out, int32_t max_items_, int32_t *n_items_out) {
    return host::schedule(cu, n_seg, block_rows, order, items_out, max_items_, n_items_out);
}

int kev_schedule_device(const int32_t *cu_seqlens, int32_t n_seg, int32_t total_tokens,
                        int32_t block_rows, int32_t order, int32_t *items_out, int32_t max_items_,
                        int32_t *n_items_out, void *stream_) {
    if (!cu_seqlens || n_seg <= 0 || total_tokens < 0 || block_rows <= 0 || !n_items_out)
        return KEV_ERR_INVALID_ARG;
    if (order != kOrderQuestion && order != kOrderLevel) return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    const int64_t n_max = max_items(total_tokens, n_seg, block_rows);
    const int64_t hist_len = qblocks(total_tokens, block_rows) + 2;
    if (hist_len > INT32_MAX || n_max > INT32_MAX / 2) return KEV_ERR_INVALID_ARG;
    const ScheduleLayout lay = schedule_layout(n_seg, (int32_t)hist_len, n_max);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t *err = nullptr;
    int rc = error_word(dev, stream, &err);
    if (rc) return rc;
    Workspace ws;
    rc = workspace_acquire(dev, stream, (size_t)lay.total * sizeof(int32_t), &ws);
    if (rc) return rc;
    int32_t *w = static_cast<int32_t *>(ws.ptr);
    ScheduleArgs sa{cu_seqlens, n_seg, total_tokens, block_rows, (int32_t)hist_len, order, n_max, w, err, nullptr, 1};
    rc = to_status(launch_schedule(sa, stream));
    std::vector<int32_t> n, items;
    if (!rc && !fetch(n, w, 1, stream)) rc = KEV_ERR_DEVICE;
    if (!rc && (n[0] > max_items_ || (n[0] > 0 && !items_out))) rc = KEV_ERR_INVALID_ARG;
    if (!rc && !fetch(items, w + lay.items, 2 * (size_t)n[0], stream)) rc = KEV_ERR_DEVICE;
    const int rc2 = workspace_release(ws, stream);
    if (rc) return rc;
    if (rc2) return rc2;
    std::copy(items.begin(), items.end(), items_out);
    *n_items_out = n[0];
    return KEV_OK;
}

}  // extern "C"
