// kev_host.cpp -- host-only checks and the host-side work list (see kev_host.h).
#include "kev_host.h"

#include <algorithm>
#include <vector>

#include "../../include/kev.h"
#include "kev_tiles.h"

namespace kev {
namespace host {

int check_seqlens(const int32_t *cu, int32_t n_seg, int32_t total_tokens) {
    if (n_seg < 0 || !cu) return KEV_ERR_INVALID_ARG;
    if (cu[0] != 0 || cu[n_seg] != total_tokens) return KEV_ERR_BAD_SEQLENS;
    for (int32_t s = 0; s < n_seg; ++s)
        if (cu[s + 1] < cu[s]) return KEV_ERR_BAD_SEQLENS;
    return KEV_OK;
}

int check_slot_list(const int32_t *ids, const int32_t *prefix, const int32_t *cu, int32_t n_seg,
                    int32_t n_slots, int32_t capacity) {
    if (n_seg < 0 || n_slots <= 0) return KEV_ERR_INVALID_ARG;
    std::vector<char> seen((size_t)n_slots, 0);
    for (int32_t s = 0; s < n_seg; ++s) {
        if (ids[s] < 0 || ids[s] >= n_slots || seen[(size_t)ids[s]]) return KEV_ERR_BAD_SLOT;
        seen[(size_t)ids[s]] = 1;
        const int64_t pre = prefix ? prefix[s] : 0;
        if (pre < 0 || pre + (int64_t)cu[s + 1] - cu[s] > capacity) return KEV_ERR_SLOT_OVERFLOW;
    }
    return KEV_OK;
}

int check_decode(const int32_t *ids, const int32_t *lens, int32_t n_req, int32_t n_slots, int32_t capacity) {
    if (n_req < 0 || n_slots <= 0) return KEV_ERR_INVALID_ARG;
    std::vector<char> seen((size_t)n_slots, 0);
    for (int32_t r = 0; r < n_req; ++r) {
        if (ids[r] < 0 || ids[r] >= n_slots || seen[(size_t)ids[r]]) return KEV_ERR_BAD_SLOT;
        seen[(size_t)ids[r]] = 1;
        if (lens[r] < 1 || lens[r] > capacity) return KEV_ERR_SLOT_OVERFLOW;
    }
    return KEV_OK;
}

int check_paged(const int32_t *tables, const int32_t *lens, int32_t n_req, int32_t max_blocks,
                int32_t n_blocks, int32_t bs) {
    if (n_req < 0 || max_blocks <= 0 || n_blocks <= 0 || bs <= 0) return KEV_ERR_INVALID_ARG;
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

int schedule(const int32_t *cu, int32_t n_seg, int32_t block_rows, int32_t order, int32_t *items,
             int32_t max_items_, int32_t *n_items) {
    if (!cu || n_seg < 0 || block_rows <= 0 || !n_items) return KEV_ERR_INVALID_ARG;
    if (order != kOrderQuestion && order != kOrderLevel) return KEV_ERR_INVALID_ARG;
    if (n_seg == 0) {
        *n_items = 0;
        return KEV_OK;
    }
    int rc = check_seqlens(cu, n_seg, cu[n_seg]);
    if (rc) return rc;
    std::vector<int32_t> nb((size_t)n_seg), qs((size_t)n_seg);   // qs: questions by descending block count
    int64_t total = 0;
    for (int32_t s = 0; s < n_seg; ++s) {
        nb[s] = qblocks(cu[s + 1] - cu[s], block_rows);
        total += nb[s];
        qs[s] = s;
    }
    if (total > max_items_ || (total > 0 && !items)) return KEV_ERR_INVALID_ARG;
    std::stable_sort(qs.begin(), qs.end(), [&](int32_t x, int32_t y) { return nb[x] > nb[y]; });
    int64_t p = 0;
    if (order == kOrderLevel) {
        int32_t maxnb = 0;
        for (int32_t s = 0; s < n_seg; ++s) maxnb = std::max(maxnb, nb[s]);
        for (int32_t t = maxnb - 1; t >= 0; --t)
            for (int32_t i = 0; i < n_seg && nb[qs[i]] > t; ++i) {
                items[2 * p] = qs[i];
                items[2 * p + 1] = t;
                ++p;
            }
    } else {
        for (int32_t i = 0; i < n_seg; ++i)
            for (int32_t t = nb[qs[i]] - 1; t >= 0; --t) {
                items[2 * p] = qs[i];
                items[2 * p + 1] = t;
                ++p;
            }
    }
    *n_items = (int32_t)p;
    return KEV_OK;
}

// With fewer units than the CUs hold at once (two workgroups each), one workgroup per unit
// leaves CUs idle and each unit's time is the latency of a few sequential tile loads, so its
// tiles are split: about two workgroups per CU in total, at most 8 per unit (more splits cost
// more in the merge than they save; measured on the 64-request decode workload cut to 1..32
// requests).
int decode_splits(int64_t units, int cus, int forced) {
    if (forced >= 1) return std::min(forced, kMaxDecodeSplits);
    if (units <= 0 || units >= (int64_t)cus) return 1;
    return (int)std::min<int64_t>(8, (2 * (int64_t)cus + units - 1) / units);
}

}  // namespace host
}  // namespace kev
