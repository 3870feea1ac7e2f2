// kev_internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kev {

// ---------------------------------------------------------------------------
// Work decomposition of the packed prefill (host and device use the same math).
//
// A question s of length L is cut into query blocks of `block_rows` rows; block
// t covers rows [t*block_rows, min((t+1)*block_rows, L)) of the question and
// needs keys [0, min((t+1)*block_rows, L)) of the same question: everything at
// or left of its diagonal and nothing of any other question.  Work items are
// (question, query block) pairs; item t costs t+1 blocks of keys.  They are
// listed question by question (longest question first), t descending inside a
// question.
// ---------------------------------------------------------------------------
__host__ __device__ inline int32_t qblocks(int32_t len, int32_t block_rows) {
    return len <= 0 ? 0 : (len + block_rows - 1) / block_rows;
}

// Upper bound on the number of items for total_tokens tokens in n_seg questions.
__host__ __device__ inline int64_t max_items(int64_t total_tokens, int64_t n_seg,
                                             int32_t block_rows) {
    return (total_tokens + block_rows - 1) / block_rows + n_seg;
}

// bf16 path: an item of 32*R rows holds G*R (head, 32-row block) units per KV head, one
// wavefront each, in workgroups of 4 wavefronts; R is the smallest power of two that makes
// G*R a multiple of 4.
struct PrefillShape {
    int32_t row_blocks;     // R
    int32_t block_rows;     // 32 * R
    int32_t wg_per_kvh;     // G * R / 4 workgroups per item and KV head
};

constexpr int32_t kPrefillUnitsPerWg = 4;   // wavefronts per workgroup

inline PrefillShape prefill_shape_bf16(int32_t heads, int32_t kv_heads) {
    const int32_t G = heads / kv_heads;
    int32_t r = 1;
    while ((G * r) % kPrefillUnitsPerWg != 0) r *= 2;
    return PrefillShape{r, 32 * r, G * r / kPrefillUnitsPerWg};
}

constexpr int32_t kF32BlockRows = 64;   // fp32 path: one wavefront of 64 rows per item and head

// ---------------------------------------------------------------------------
// Launch arguments
// ---------------------------------------------------------------------------
struct ScheduleArgs {
    const int32_t *cu;        // [n_seg + 1]
    int32_t n_seg;
    int32_t total_tokens;
    int32_t block_rows;
    int32_t hist_len;         // >= max query blocks per question + 2
    int32_t order;            // kOrderQuestion or kOrderLevel
    int64_t n_max_items;      // item capacity the workspace was laid out for
    int32_t *ws;              // workspace, see schedule_layout()
    int32_t *err;             // device error word
    // chunked prefill: rows already cached per question; with at most 64 questions the
    // question order then follows the blocks of prefix + chunk (the work of the last block)
    const int32_t *prefix_lens;
};

// Item orders.  Question-major: questions in descending length, query block t descending
// inside a question (workgroups running together share one question's K/V rows).
// Level-major: t descending over all questions, then descending length (longest items
// first overall: the best balance when all K/V rows fit in the caches anyway).
constexpr int32_t kOrderQuestion = 0;
constexpr int32_t kOrderLevel = 1;

// Workspace layout of the scheduler (int32 units):
//   [0] n_items  [1..3] unused  [4..] hist[hist_len] | fill[hist_len] | cnt[hist_len] |
//   start[hist_len] | sigma[n_seg] | qoff[n_seg] | items[2 * max_items] (question, t) |
//   rec[4 * max_items] ({question start, question length, t, question index}, 16-byte aligned)
struct ScheduleLayout {
    int64_t hist, fill, cnt, start, sigma, qoff, items, rec, total;
};
__host__ __device__ inline ScheduleLayout schedule_layout(int32_t n_seg, int32_t hist_len, int64_t n_max_items) {
    ScheduleLayout L;
    L.hist = 4;
    L.fill = L.hist + hist_len;
    L.cnt = L.fill + hist_len;
    L.start = L.cnt + hist_len;
    L.sigma = L.start + hist_len;
    L.qoff = L.sigma + n_seg;
    L.items = (L.qoff + n_seg + 3) & ~int64_t(3);
    L.rec = (L.items + 2 * n_max_items + 3) & ~int64_t(3);
    L.total = L.rec + 4 * n_max_items;
    return L;
}

struct PrefillArgs {
    const void *q, *k, *v;
    void *out;
    const int32_t *cu;
    const int32_t *sched;     // scheduler workspace (n_items at [0], items at items_off)
    int64_t items_off;
    const int32_t *rec;       // item records {question start, length, t, question index}
    int32_t heads, kv_heads, group;     // group = heads / kv_heads
    int32_t heads_per_wg, row_blocks, block_rows, n_hgroups;   // fp32 path
    int32_t wg_per_kvh;                 // bf16 path: workgroups per item and KV head
    float scale_log2;                   // log2(e) / sqrt(head_dim)
    // Chunked prefill only: question s continues the prefix_lens[s] rows cached in slot
    // slot_ids[s] of the pool [n_slots][2][kv_heads][capacity][head_dim].
    const int32_t *slot_ids, *prefix_lens;
    const void *pool;
    int32_t n_slots, capacity;
    int32_t *err;
};

// Block ids a paged decode workgroup keeps in LDS: at most this many blocks per request
// (KEV_PAGED_MAX_BLOCKS of the public header).
constexpr int kDecodeMaxBlocks = 2048;
// Most workgroups one decode unit (request, KV head) is split over.
constexpr int kMaxDecodeSplits = 32;

struct DecodeArgs {
    const void *q;
    void *pool;
    const int32_t *slot_ids, *cache_lens;
    void *out;
    const void *k_new, *v_new;
    int32_t n_req, heads, kv_heads, group;
    int32_t n_slots, capacity;   // paged: number of blocks, block size
    int32_t ranked;           // 1: units longest first; 2: long and short units paired per CU (n_req <= 64)
    int32_t cus;              // compute units of the device (paired order)
    float scale_log2;
    int32_t *err;
    // paged pool only: block_tables[n_req][max_blocks], block size 1 << block_shift
    const int32_t *block_tables;
    int32_t max_blocks, block_shift;
    // n_split > 1: each unit's tiles are cut into n_split ranges whose unnormalised states go
    // to part (o: [units * n_split][group][head_dim] fp32, then {max, sum} per head)
    int32_t n_split;
    float *part;
};

struct StoreKvArgs {
    const void *k, *v;        // [total_tokens, kv_heads, head_dim]
    const int32_t *cu;        // [n_seg + 1]
    const int32_t *slot_ids;  // [n_seg]
    const int32_t *prefix_lens;   // [n_seg] rows already in each slot, or null (all 0)
    void *pool;               // [n_slots][2][kv_heads][capacity][head_dim]
    int32_t n_seg, total_tokens, kv_heads, n_slots, capacity;
    int32_t *err;
};

// Launchers (each lives in the translation unit of its kernel).
hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, int32_t head_dim, int64_t grid,
                               bool prefix, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, int32_t head_dim, int64_t grid,
                              hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs &a, int32_t head_dim, bool paged, hipStream_t s);
hipError_t launch_store_kv(const StoreKvArgs &a, int32_t head_dim, hipStream_t s);

}  // namespace kev
