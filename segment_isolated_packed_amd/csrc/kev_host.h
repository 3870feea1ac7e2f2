// kev_host.h -- host-only parts of the library: checks of device-array contents copied to the
// host (KEV_CHECK=1), the host-side work list, and the decode split count.  Plain C++ (no HIP),
// so the same sources also build with a host compiler and its sanitizers.
#pragma once

#include <stdint.h>

namespace kev {
namespace host {

// cu_seqlens: cu[0] = 0, non-decreasing, cu[n_seg] = total_tokens.
int check_seqlens(const int32_t *cu, int32_t n_seg, int32_t total_tokens);

// Slot ids of a slot-writing prefill in [0, n_slots) and distinct; every question's rows
// (after its prefix, if prefix is non-null) fit the slot.
int check_slot_list(const int32_t *ids, const int32_t *prefix, const int32_t *cu, int32_t n_seg,
                    int32_t n_slots, int32_t capacity);

// Slot decode: slot ids in range and distinct, cache lengths in [1, capacity].
int check_decode(const int32_t *ids, const int32_t *lens, int32_t n_req, int32_t n_slots, int32_t capacity);

// Paged decode: cache lengths in range, the block ids a request reads inside the pool, and
// every append target (block, row) touched by no other request of the call.
int check_paged(const int32_t *tables, const int32_t *lens, int32_t n_req, int32_t max_blocks,
                int32_t n_blocks, int32_t block_size);

// Work list from a host copy of cu_seqlens (items[2i] = question, items[2i+1] = query block).
int schedule(const int32_t *cu, int32_t n_seg, int32_t block_rows, int32_t order, int32_t *items,
             int32_t max_items, int32_t *n_items);

// Workgroups per decode unit (request, KV head); forced > 0 overrides (capped).
int decode_splits(int64_t units, int cus, int forced);

}  // namespace host
}  // namespace kev
