// kev_internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define KEV_HD __host__ __device__
#include "kev_tiles.h"

namespace kev {

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
    int64_t n_max_items;      // item capacity (per stream) the workspace was laid out for
    int32_t *ws;              // workspace, see schedule_layout()
    int32_t *err;             // device error word
    // chunked prefill: rows already cached per question; with at most 64 questions the
    // question order then follows the blocks of prefix + chunk (the work of the last block)
    const int32_t *prefix_lens;
    // n_streams > 1 (at most 64 questions, question-major order): questions are dealt to
    // n_streams streams, longest first, each to the stream with the least work so far; stream s
    // lists its questions' items question-major at records [s * n_max_items, ...), and the
    // records after its last item carry length -1
    int32_t n_streams;
};


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
    // bf16 path, n_streams > 1: workgroup b runs on XCD x = b % n_xcd (workgroups are dealt to
    // the XCDs round-robin) and serves KV head x % kv_heads of stream x / kv_heads, as that
    // pair's (b / n_xcd)-th workgroup; stream s's records start at s * stream_cap
    int32_t n_streams, n_xcd, stream_cap;
    float scale_log2;                   // log2(e) / sqrt(head_dim)
    // Chunked prefill only: question s continues the prefix_lens[s] rows cached in slot
    // slot_ids[s] of the pool [n_slots][2][kv_heads][capacity][head_dim].
    const int32_t *slot_ids, *prefix_lens;
    const void *pool;
    int32_t n_slots, capacity;
    int32_t *err;
};


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
