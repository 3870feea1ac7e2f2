// kev_api.hip -- the C ABI: argument checks, per-stream workspace, launches.
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
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/kev.h"
#include "kev_internal.h"

namespace {

using namespace kev;

struct Buffer {
    void *ptr = nullptr;
    size_t bytes = 0;
};

struct State {
    std::mutex mu;
    std::map<int, int32_t *> err_word;                        // device -> error word
    std::map<std::pair<int, void *>, Buffer> sched_ws;        // (device, stream)
    std::map<std::pair<int, void *>, Buffer> decode_ws;       // (device, stream): split states
};

State &state() {
    static State *s = new State();   // never destroyed: outlives static teardown order
    return *s;
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

bool check_enabled() {
    const char *e = std::getenv("KEV_CHECK");
    return e && e[0] == '1';
}

int to_status(hipError_t e) { return e == hipSuccess ? KEV_OK : KEV_ERR_DEVICE; }

// Device error word of the current device (allocated and zeroed on first use).
int error_word(int dev, int32_t **out) {
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    auto it = st.err_word.find(dev);
    if (it != st.err_word.end()) {
        *out = it->second;
        return KEV_OK;
    }
    int32_t *p = nullptr;
    if (hipMalloc(&p, 256) != hipSuccess) return KEV_ERR_NO_MEMORY;
    if (hipMemset(p, 0, 256) != hipSuccess) return KEV_ERR_DEVICE;
    st.err_word[dev] = p;
    *out = p;
    return KEV_OK;
}

// Workspace of at least `bytes` for (device, stream), grown on demand.
int workspace(std::map<std::pair<int, void *>, Buffer> &m, int dev, hipStream_t stream,
              size_t bytes, void **out) {
    State &st = state();
    std::lock_guard<std::mutex> lock(st.mu);
    Buffer &b = m[{dev, (void *)stream}];
    if (b.bytes < bytes) {
        if (b.ptr) {
            if (hipStreamSynchronize(stream) != hipSuccess) return KEV_ERR_DEVICE;
            if (hipFree(b.ptr) != hipSuccess) return KEV_ERR_DEVICE;
            b.ptr = nullptr;
            b.bytes = 0;
        }
        size_t want = std::max(bytes, (size_t)1 << 16);
        if (hipMalloc(&b.ptr, want) != hipSuccess) {
            b.ptr = nullptr;
            return KEV_ERR_NO_MEMORY;
        }
        b.bytes = want;
    }
    *out = b.ptr;
    return KEV_OK;
}

bool prefill_supported(int32_t head_dim, int32_t dtype) {
    if (dtype == KEV_BF16) return head_dim == 64 || head_dim == 128;
    if (dtype == KEV_F32) return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128;
    return false;
}

int32_t block_rows_for(int32_t heads, int32_t kv_heads, int32_t dtype) {
    if (dtype == KEV_F32) return kF32BlockRows;
    return prefill_shape_bf16(heads, kv_heads).block_rows;
}

int host_check_seqlens(const int32_t *cu, int32_t n_seg, int32_t total_tokens) {
    if (cu[0] != 0 || cu[n_seg] != total_tokens) return KEV_ERR_BAD_SEQLENS;
    for (int32_t s = 0; s < n_seg; ++s)
        if (cu[s + 1] < cu[s]) return KEV_ERR_BAD_SEQLENS;
    return KEV_OK;
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

// Schedule on the device into the (device, stream) workspace.
int run_schedule(const int32_t *cu, int32_t n_seg, int32_t total_tokens, int32_t block_rows,
                 int32_t order, hipStream_t stream, int32_t **ws_out, ScheduleLayout *lay_out,
                 const int32_t *prefix_lens = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t *err = nullptr;
    int rc = error_word(dev, &err);
    if (rc) return rc;
    const int64_t n_max = max_items(total_tokens, n_seg, block_rows);
    const int64_t hist_len = qblocks(total_tokens, block_rows) + 2;
    if (hist_len > INT32_MAX || n_max > INT32_MAX / 2) return KEV_ERR_INVALID_ARG;
    const ScheduleLayout lay = schedule_layout(n_seg, (int32_t)hist_len, n_max);
    void *ws = nullptr;
    rc = workspace(state().sched_ws, dev, stream, (size_t)lay.total * sizeof(int32_t), &ws);
    if (rc) return rc;
    ScheduleArgs sa{cu, n_seg, total_tokens, block_rows, (int32_t)hist_len, order, n_max,
                    static_cast<int32_t *>(ws), err, prefix_lens};
    rc = to_status(launch_schedule(sa, stream));
    if (rc) return rc;
    *ws_out = static_cast<int32_t *>(ws);
    *lay_out = lay;
    return KEV_OK;
}

// Slot side of a chunked prefill: question s continues prefix_lens[s] rows of slot slot_ids[s].
struct SlotPrefix {
    const kev_kv_pool *pool;
    const int32_t *slot_ids, *prefix_lens;
};

// Packed prefill; with `pre`, every question is a chunk continuing its slot's cached rows.
int prefill_impl(const void *q, const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg,
                 int32_t heads, int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                 int32_t dtype, void *stream_, const SlotPrefix *pre) {
    if (n_seg < 0 || total_tokens < 0 || heads <= 0 || kv_heads <= 0 || head_dim <= 0)
        return KEV_ERR_INVALID_ARG;
    if (heads % kv_heads != 0) return KEV_ERR_INVALID_ARG;
    if (dtype != KEV_BF16 && dtype != KEV_F32) return KEV_ERR_UNSUPPORTED;
    if (!prefill_supported(head_dim, dtype)) return KEV_ERR_UNSUPPORTED;
    if (pre && dtype != KEV_BF16) return KEV_ERR_UNSUPPORTED;   // slot prefixes: bf16 pools only
    if (n_seg == 0) return total_tokens == 0 ? KEV_OK : KEV_ERR_BAD_SEQLENS;
    if (!cu_seqlens) return KEV_ERR_INVALID_ARG;
    if (total_tokens > 0 && (!q || !k || !v || !out)) return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);

    if (check_enabled()) {
        std::vector<int32_t> h(n_seg + 1);
        if (hipMemcpyAsync(h.data(), cu_seqlens, sizeof(int32_t) * (n_seg + 1),
                           hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return KEV_ERR_DEVICE;
        int rc = host_check_seqlens(h.data(), n_seg, total_tokens);
        if (rc) return rc;
    }
    const int32_t br = block_rows_for(heads, kv_heads, dtype);
    int32_t *ws = nullptr;
    ScheduleLayout lay;
    int rc = run_schedule(cu_seqlens, n_seg, total_tokens, br, prefill_order(total_tokens, head_dim, dtype),
                          stream, &ws, &lay, pre ? pre->prefix_lens : nullptr);
    if (rc) return rc;
    if (total_tokens == 0) return KEV_OK;   // only empty questions; cu_seqlens still checked

    const int64_t n_max = max_items(total_tokens, n_seg, br);
    PrefillArgs pa{};
    pa.q = q;
    pa.k = k;
    pa.v = v;
    pa.out = out;
    pa.cu = cu_seqlens;
    pa.sched = ws;
    pa.items_off = lay.items;
    pa.rec = ws + lay.rec;
    pa.heads = heads;
    pa.kv_heads = kv_heads;
    pa.group = heads / kv_heads;
    pa.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
    if (dtype == KEV_BF16) {
        const PrefillShape sh = prefill_shape_bf16(heads, kv_heads);
        pa.row_blocks = sh.row_blocks;
        pa.block_rows = sh.block_rows;
        pa.wg_per_kvh = sh.wg_per_kvh;
        const int64_t grid = n_max * kv_heads * sh.wg_per_kvh;
        if (grid > INT32_MAX) return KEV_ERR_INVALID_ARG;
        if (pre) {
            int dev = 0;
            if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
            rc = error_word(dev, &pa.err);
            if (rc) return rc;
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
    const int64_t grid = n_max * heads;
    if (grid > INT32_MAX) return KEV_ERR_INVALID_ARG;
    return timed_launch(stream, [&] { return launch_prefill_f32(pa, head_dim, grid, stream); });
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
int host_check_slots(const kev_kv_pool *pool, const int32_t *slot_ids, const int32_t *prefix_lens,
                     const int32_t *cu_seqlens, int32_t n_seg, hipStream_t stream) {
    std::vector<int32_t> ids(n_seg), cu(n_seg + 1), pre(n_seg, 0);
    if (hipMemcpyAsync(ids.data(), slot_ids, sizeof(int32_t) * n_seg, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipMemcpyAsync(cu.data(), cu_seqlens, sizeof(int32_t) * (n_seg + 1), hipMemcpyDeviceToHost, stream) != hipSuccess ||
        (prefix_lens && hipMemcpyAsync(pre.data(), prefix_lens, sizeof(int32_t) * n_seg, hipMemcpyDeviceToHost,
                                       stream) != hipSuccess) ||
        hipStreamSynchronize(stream) != hipSuccess)
        return KEV_ERR_DEVICE;
    std::vector<char> seen(pool->n_slots, 0);
    for (int32_t s = 0; s < n_seg; ++s) {
        if (ids[s] < 0 || ids[s] >= pool->n_slots || seen[ids[s]]) return KEV_ERR_BAD_SLOT;
        seen[ids[s]] = 1;
        if (pre[s] < 0 || (int64_t)pre[s] + cu[s + 1] - cu[s] > pool->capacity) return KEV_ERR_SLOT_OVERFLOW;
    }
    return KEV_OK;
}

// Write every question's K/V rows into its slot, after its prefix rows if any.
int store_rows(const void *k, const void *v, const int32_t *cu_seqlens, int32_t n_seg, int32_t kv_heads,
               int32_t head_dim, int32_t total_tokens, const kev_kv_pool *pool, const int32_t *slot_ids,
               const int32_t *prefix_lens, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t *err = nullptr;
    int rc = error_word(dev, &err);
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

// KEV_CHECK for a paged decode: cache lengths in range, the block ids a request reads inside
// the pool, and every append target (block, row) touched by no other request of the call.
int host_check_paged(const std::vector<int32_t> &tables, const std::vector<int32_t> &lens, int32_t max_blocks,
                     int32_t n_blocks, int32_t bs) {
    const int32_t n_req = (int32_t)lens.size();
    const int64_t limit = std::min<int64_t>(max_blocks, KEV_PAGED_MAX_BLOCKS) * (int64_t)bs;
    std::vector<char> appended((size_t)n_blocks * bs, 0);
    for (int32_t r = 0; r < n_req; ++r) {
        if (lens[r] < 1 || lens[r] > limit) return KEV_ERR_SLOT_OVERFLOW;
        for (int32_t j = 0; j <= (lens[r] - 1) / bs; ++j) {
            const int32_t b = tables[(size_t)r * max_blocks + j];
            if (b < 0 || b >= n_blocks) return KEV_ERR_BAD_SLOT;
        }
        const int32_t p = lens[r] - 1;
        char &a = appended[(size_t)tables[(size_t)r * max_blocks + p / bs] * bs + p % bs];
        if (a) return KEV_ERR_BAD_SLOT;
        a = 1;
    }
    for (int32_t r = 0; r < n_req; ++r)
        for (int32_t p = 0; p + 1 < lens[r]; ++p)
            if (appended[(size_t)tables[(size_t)r * max_blocks + p / bs] * bs + p % bs]) return KEV_ERR_BAD_SLOT;
    return KEV_OK;
}

// Workgroups per decode unit (request, KV head).  With fewer units than the CUs hold at once
// (two workgroups each), one workgroup per unit leaves CUs idle and each unit's time is the
// latency of a few sequential tile loads, so its tiles are split: about two workgroups per CU
// in total, at most 8 per unit (more splits cost more in the merge than they save; measured
// on the 64-request decode workload cut to 1..32 requests).  KEV_DECODE_SPLITS=N forces N.
int decode_splits(int64_t units, int cus) {
    if (const char *e = std::getenv("KEV_DECODE_SPLITS")) {
        const int n = std::atoi(e);
        if (n >= 1) return std::min(n, kMaxDecodeSplits);
    }
    if (units >= (int64_t)cus) return 1;
    return (int)std::min<int64_t>(8, (2 * (int64_t)cus + units - 1) / units);
}

// Launch a decode (slot or paged pool) once the pool-specific fields of `da` are set.
int run_decode(DecodeArgs &da, const void *q, void *data, int32_t kv_heads, int32_t head_dim,
               const int32_t *cache_lens, void *out, const void *k_new, const void *v_new, int32_t n_req,
               int32_t heads, bool paged, hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KEV_ERR_DEVICE;
    int rc = error_word(dev, &da.err);
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
    da.n_split = decode_splits(units, cus);
    if (units * da.n_split > INT32_MAX) return KEV_ERR_INVALID_ARG;
    if (da.n_split > 1) {
        void *ws = nullptr;
        const size_t bytes = (size_t)units * da.n_split * da.group * (head_dim + 2) * sizeof(float);
        rc = workspace(state().decode_ws, dev, stream, bytes, &ws);
        if (rc) return rc;
        da.part = static_cast<float *>(ws);
    }
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
    return timed_launch(stream, [&] { return launch_decode_bf16(da, head_dim, paged, stream); });
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
    default: return "unknown status";
    }
}

int kev_prefill_block_rows(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype) {
    if (heads <= 0 || kv_heads <= 0 || heads % kv_heads != 0) return 0;
    if (!prefill_supported(head_dim, dtype)) return 0;
    return block_rows_for(heads, kv_heads, dtype);
}

int kev_packed_attn_prefill(const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int32_t n_seg,
                            int32_t heads, int32_t kv_heads, int32_t head_dim,
                            void *out, int32_t total_tokens, int32_t dtype, void *stream) {
    return prefill_impl(q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens, dtype,
                        stream, nullptr);
}

int kev_packed_attn_prefill_slots(const void *q, const void *k, const void *v,
                                  const int32_t *cu_seqlens, int32_t n_seg, int32_t heads,
                                  int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                                  const kev_kv_pool *pool, const int32_t *slot_ids, void *stream_) {
    int rc = check_pool(pool, n_seg, total_tokens, kv_heads, head_dim, slot_ids);
    if (rc) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    if (check_enabled() && n_seg > 0) {
        rc = host_check_slots(pool, slot_ids, nullptr, cu_seqlens, n_seg, stream);
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
        rc = host_check_slots(pool, slot_ids, prefix_lens, cu_seqlens, n_seg, stream);
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
        std::vector<int32_t> ids(n_req), lens(n_req);
        if (hipMemcpyAsync(ids.data(), slot_ids, sizeof(int32_t) * n_req, hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipMemcpyAsync(lens.data(), cache_lens, sizeof(int32_t) * n_req, hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return KEV_ERR_DEVICE;
        std::vector<char> seen(pool->n_slots, 0);
        for (int32_t r = 0; r < n_req; ++r) {
            if (ids[r] < 0 || ids[r] >= pool->n_slots || seen[ids[r]]) return KEV_ERR_BAD_SLOT;
            seen[ids[r]] = 1;
            if (lens[r] < 1 || lens[r] > pool->capacity) return KEV_ERR_SLOT_OVERFLOW;
        }
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
        std::vector<int32_t> tables((size_t)n_req * max_blocks), lens(n_req);
        if (hipMemcpyAsync(tables.data(), block_tables, sizeof(int32_t) * tables.size(), hipMemcpyDeviceToHost,
                           stream) != hipSuccess ||
            hipMemcpyAsync(lens.data(), cache_lens, sizeof(int32_t) * n_req, hipMemcpyDeviceToHost, stream) != hipSuccess ||
            hipStreamSynchronize(stream) != hipSuccess)
            return KEV_ERR_DEVICE;
        rc = host_check_paged(tables, lens, max_blocks, pool->n_blocks, bs);
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
    int rc = error_word(dev, &err);
    if (rc) return rc;
    if (hipStreamSynchronize(stream) != hipSuccess) return KEV_ERR_DEVICE;
    int32_t v = 0;
    if (hipMemcpy(&v, err, sizeof v, hipMemcpyDeviceToHost) != hipSuccess) return KEV_ERR_DEVICE;
    if (hipMemset(err, 0, sizeof v) != hipSuccess) return KEV_ERR_DEVICE;
    if (hipDeviceSynchronize() != hipSuccess) return KEV_ERR_DEVICE;
    *flags_out = v;
    return KEV_OK;
}

int kev_prefill_order(int32_t total_tokens, int32_t head_dim, int32_t dtype) {
    return prefill_order(total_tokens, head_dim, dtype);
}

int kev_schedule_host(const int32_t *cu, int32_t n_seg, int32_t block_rows, int32_t order,
                      int32_t *items_out, int32_t max_items_, int32_t *n_items_out) {
    if (!cu || n_seg < 0 || block_rows <= 0 || !n_items_out) return KEV_ERR_INVALID_ARG;
    if (order != kOrderQuestion && order != kOrderLevel) return KEV_ERR_INVALID_ARG;
    if (n_seg == 0) {
        *n_items_out = 0;
        return KEV_OK;
    }
    int rc = host_check_seqlens(cu, n_seg, cu[n_seg]);
    if (rc) return rc;
    std::vector<int32_t> nb(n_seg), qs(n_seg);   // qs: questions by descending block count
    int64_t total = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        nb[s] = qblocks(cu[s + 1] - cu[s], block_rows);
        total += nb[s];
        qs[s] = s;
    }
    if (total > max_items_ || (total > 0 && !items_out)) return KEV_ERR_INVALID_ARG;
    std::stable_sort(qs.begin(), qs.end(), [&](int32_t x, int32_t y) { return nb[x] > nb[y]; });
    int64_t p = 0;
    if (order == kOrderLevel) {
        int32_t maxnb = 0;
        for (int32_t s = 0; s < n_seg; ++s) maxnb = std::max(maxnb, nb[s]);
        for (int32_t t = maxnb - 1; t >= 0; --t)
            for (int32_t i = 0; i < n_seg && nb[qs[i]] > t; ++i) {
                items_out[2 * p] = qs[i];
                items_out[2 * p + 1] = t;
                ++p;
            }
    } else {
        for (int32_t i = 0; i < n_seg; ++i)
            for (int32_t t = nb[qs[i]] - 1; t >= 0; --t) {
                items_out[2 * p] = qs[i];
                items_out[2 * p + 1] = t;
                ++p;
            }
    }
    *n_items_out = (int32_t)p;
    return KEV_OK;
}

int kev_schedule_device(const int32_t *cu_seqlens, int32_t n_seg, int32_t total_tokens,
                        int32_t block_rows, int32_t order, int32_t *items_out, int32_t max_items_,
                        int32_t *n_items_out, void *stream_) {
    if (!cu_seqlens || n_seg <= 0 || total_tokens < 0 || block_rows <= 0 || !n_items_out)
        return KEV_ERR_INVALID_ARG;
    if (order != kOrderQuestion && order != kOrderLevel) return KEV_ERR_INVALID_ARG;
    hipStream_t stream = static_cast<hipStream_t>(stream_);
    int32_t *ws = nullptr;
    ScheduleLayout lay;
    int rc = run_schedule(cu_seqlens, n_seg, total_tokens, block_rows, order, stream, &ws, &lay);
    if (rc) return rc;
    int32_t n = 0;
    if (hipMemcpyAsync(&n, ws, sizeof n, hipMemcpyDeviceToHost, stream) != hipSuccess ||
        hipStreamSynchronize(stream) != hipSuccess)
        return KEV_ERR_DEVICE;
    if (n > max_items_ || (n > 0 && !items_out)) return KEV_ERR_INVALID_ARG;
    if (n > 0 && (hipMemcpyAsync(items_out, ws + lay.items, sizeof(int32_t) * 2 * n,
                                 hipMemcpyDeviceToHost, stream) != hipSuccess ||
                  hipStreamSynchronize(stream) != hipSuccess))
        return KEV_ERR_DEVICE;
    *n_items_out = n;
    return KEV_OK;
}

}  // extern "C"
