// kev_tiles.h -- work decomposition of the packed prefill, shared by the host code and the
// kernels (no HIP types here, so the host-only sources build with a plain C++ compiler too).
//
// A question s of length L is cut into query blocks of `block_rows` rows; block t covers rows
// [t*block_rows, min((t+1)*block_rows, L)) of the question and needs keys
// [0, min((t+1)*block_rows, L)) of the same question: everything at or left of its diagonal
// and nothing of any other question.  Work items are (question, query block) pairs; item t
// costs t+1 blocks of keys.
#pragma once

#include <stdint.h>

// Functions used on both sides carry KEV_HD: the HIP sources define it as __host__ __device__
// before including this header; host-only sources leave it empty.
#ifndef KEV_HD
#define KEV_HD
#endif

namespace kev {

KEV_HD inline int32_t qblocks(int32_t len, int32_t block_rows) {
    return len <= 0 ? 0 : (len + block_rows - 1) / block_rows;
}

// Upper bound on the number of items for total_tokens tokens in n_seg questions.
KEV_HD inline int64_t max_items(int64_t total_tokens, int64_t n_seg, int32_t block_rows) {
    return (total_tokens + block_rows - 1) / block_rows + n_seg;
}

// bf16 path: an item of W*R rows holds G*R (head, W-row block) units per KV head, one
// wavefront each, in workgroups of 4 wavefronts; R is the smallest power of two that makes
// G*R a multiple of 4.  W, the query rows of one wavefront, is 48 for head_dim 128 (three
// 16-row MFMA blocks) and 32 for head_dim 64.
struct PrefillShape {
    int32_t row_blocks;     // R
    int32_t block_rows;     // W * R
    int32_t wg_per_kvh;     // G * R / 4 workgroups per item and KV head
};

constexpr int32_t kPrefillUnitsPerWg = 4;   // wavefronts per workgroup

inline int32_t prefill_wave_rows(int32_t head_dim) { return head_dim == 128 ? 48 : 32; }

inline PrefillShape prefill_shape_bf16(int32_t heads, int32_t kv_heads, int32_t head_dim) {
    const int32_t G = heads / kv_heads;
    int32_t r = 1;
    while ((G * r) % kPrefillUnitsPerWg != 0) r *= 2;
    return PrefillShape{r, prefill_wave_rows(head_dim) * r, G * r / kPrefillUnitsPerWg};
}

constexpr int32_t kF32BlockRows = 64;   // fp32 path: one wavefront of 64 rows per item and head

// Item orders.  Question-major: questions in descending length, query block t descending
// inside a question (workgroups running together share one question's K/V rows).
// Level-major: t descending over all questions, then descending length (longest items
// first overall: the best balance when all K/V rows fit in the caches anyway).
constexpr int32_t kOrderQuestion = 0;
constexpr int32_t kOrderLevel = 1;

// Most item streams of an XCD-aware prefill launch (the work-list pass keeps one count per stream).
constexpr int32_t kStreamsMax = 8;

// Workspace layout of the scheduler (int32 units; max_items counts every stream's records):
//   [0] n_items  [1..3] unused  [4..] hist[hist_len] | fill[hist_len] | cnt[hist_len] |
//   start[hist_len] | sigma[n_seg] | qoff[n_seg] | items[2 * max_items] (question, t) |
//   rec[4 * max_items] ({question start, question length, t, question index}, 16-byte aligned)
struct ScheduleLayout {
    int64_t hist, fill, cnt, start, sigma, qoff, items, rec, total;
};
KEV_HD inline ScheduleLayout schedule_layout(int32_t n_seg, int32_t hist_len, int64_t n_max_items) {
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

// Block ids a paged decode workgroup keeps in LDS: at most this many blocks per request
// (KEV_PAGED_MAX_BLOCKS of the public header).
constexpr int kDecodeMaxBlocks = 2048;
// Most workgroups one decode unit (request, KV head) is split over.
constexpr int kMaxDecodeSplits = 32;

}  // namespace kev
