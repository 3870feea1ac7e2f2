/*
 * kev.h -- C ABI of the segment-isolated packed attention library (gfx950).
 *
 * Entry points:
 *
 *   kev_packed_attn_prefill  packed prefill.  Several independent questions
 *       are concatenated into one token stream and each token attends only to
 *       earlier-or-equal positions of its own question:
 *           Z = softmax(Q K^T / sqrt(d_h) + M) V
 *       with M_ij = 0 when j <= i and i, j lie in the same question interval,
 *       and -inf otherwise.  The formula and the causal mask are those of the
 *       inference-engine primer (sakurs2.com, section 2.1); the mask is the
 *       AND of the causal lower triangle and the block-diagonal isolation mask
 *       of the Kev article (icman.com.cn, sections 2.1 and 2.3), and the
 *       question intervals are handed over in flash-attn's varlen cu_seqlens
 *       form rather than as a dense matrix (same article, sections 5.2, 6.4).
 *
 *   kev_slot_attn_decode  single-token decode against a pre-allocated KV pool
 *       cut into fixed-capacity slots, one slot per question (Kev part 2,
 *       gsyq.cn, section 2.2).  The new token's K/V are written into the slot
 *       in place, not concatenated (primer, section 2.2), and the new query
 *       attends over all cached positions with no mask (same section).
 *
 *   kev_packed_attn_prefill_slots  the prefill, and each question's K/V rows
 *       stored into its slot of that pool (the handoff to decode).
 *
 *   kev_chunked_prefill_slots  chunked prefill: each question of the packed
 *       stream is the next chunk of a prompt whose earlier rows are already
 *       cached in its slot; the chunk attends to them and to itself causally,
 *       and its K/V rows are appended to the slot.
 *
 *   kev_paged_attn_decode  the decode step against a paged pool: fixed-size
 *       blocks placed anywhere, found through per-request block tables.
 *
 * Conventions shared by every call
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous in
 *     the layouts stated below, never freed or retained by the library.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL means the default stream): they validate, enqueue and return.
 *   - Arguments that can be checked without reading device memory are checked
 *     before any HIP call; a failing check returns a negative kev_status and
 *     enqueues nothing.  n_seg == 0 or n_req == 0 is a successful no-op.
 *   - Device-array contents (cu_seqlens, slot_ids, cache_lens, prefix_lens) are guarded in
 *     the kernels: an invalid unit is skipped (its outputs are left untouched,
 *     nothing out of range is read or written) and a bit is set in the error
 *     word of the call's (device, stream), read by kev_get_device_errors on that
 *     stream.  With the environment variable KEV_CHECK=1 they are also copied to
 *     the host and checked synchronously before launch, returning the matching
 *     status.
 *   - Workspace (the prefill's work list, the split decode's partial states)
 *     is stream-ordered: taken from a library-owned memory pool of the device
 *     with hipMallocFromPoolAsync on the call's stream and returned with
 *     hipFreeAsync on the same stream after the call's last kernel, so no call
 *     synchronises and calls in flight on different streams never share it.
 *     The pool keeps its memory for later calls.  On a device without the
 *     stream-ordered allocator (or with KEV_NO_MEMPOOL=1) one cached buffer per
 *     (device, stream) is used instead; growing it synchronises that stream,
 *     and calls on one stream must then come from one host thread at a time.
 *   - The first call on a (device, stream) allocates that stream's error word
 *     (256 bytes, kept until the process ends).
 *   - KEV_LOG=1 prints each call's work decomposition (items, splits, workspace
 *     bytes) to stderr; it synchronises the stream to read the item count.
 *   - Head grouping: query head h reads KV head h / (heads / kv_heads).
 */
#ifndef KEV_H
#define KEV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { KEV_BF16 = 0, KEV_F32 = 1 } kev_dtype;

typedef enum {
    KEV_OK = 0,
    KEV_ERR_INVALID_ARG = -1,   /* null pointer, non-positive size, heads % kv_heads != 0 */
    KEV_ERR_UNSUPPORTED = -2,   /* dtype / head_dim combination not built */
    KEV_ERR_BAD_SEQLENS = -3,   /* cu_seqlens not 0-based, decreasing, or != total_tokens at the end */
    KEV_ERR_SLOT_OVERFLOW = -4, /* a cache length outside [1, capacity] */
    KEV_ERR_BAD_SLOT = -5,      /* a slot id outside [0, n_slots), or repeated within one call */
    KEV_ERR_DEVICE = -6,        /* a HIP call failed */
    KEV_ERR_NO_MEMORY = -7,     /* workspace allocation failed */
    KEV_ERR_SCRATCH_LIMIT = -8  /* kev_packed_attn_prefill_noalloc: work list exceeds its scratch */
} kev_status;

/* Bits of the per-stream error word (kev_get_device_errors). */
#define KEV_DEVERR_SEQLENS 1u   /* cu_seqlens invalid; the prefill call computed nothing */
#define KEV_DEVERR_SLOT 2u      /* a request's slot id was out of range; request skipped */
#define KEV_DEVERR_CACHE_LEN 4u /* a request's cache length was outside [1, capacity]; skipped */
#define KEV_DEVERR_BLOCK 8u     /* a paged request's block id was outside the pool; skipped */

/*
 * Packed, segment-isolated causal prefill.
 *
 *   q            [total_tokens, heads, head_dim]      dtype
 *   k, v         [total_tokens, kv_heads, head_dim]   dtype (already position-encoded)
 *   cu_seqlens   int32 [n_seg + 1], device; cu[0] = 0, non-decreasing,
 *                cu[n_seg] = total_tokens; question s owns tokens
 *                [cu[s], cu[s+1]) (half-open; empty questions are allowed)
 *   out          [total_tokens, heads, head_dim]      dtype, written for every token
 *   total_tokens the host's copy of cu[n_seg] (bounds the launch and the workspace)
 *   dtype        KEV_BF16 (head_dim 64 or 128; bf16 MFMA, fp32 accumulation and
 *                softmax, output rounded to nearest even) or KEV_F32
 *                (head_dim 16, 32, 64 or 128; fp32 arithmetic throughout)
 *
 * The scale is fixed at 1/sqrt(head_dim); there is no bias, dropout or softcap.
 * No dense mask is built: a scheduler kernel lists the (question, query block)
 * work items from cu_seqlens and the attention kernel visits only key blocks
 * at or left of each block's diagonal inside its own question.
 * Returns KEV_OK or a negative kev_status.
 */
int kev_packed_attn_prefill(const void *q, const void *k, const void *v,
                            const int32_t *cu_seqlens, int32_t n_seg,
                            int32_t heads, int32_t kv_heads, int32_t head_dim,
                            void *out, int32_t total_tokens, int32_t dtype, void *stream);

/*
 * kev_packed_attn_prefill without any allocation, for callers that cannot
 * allocate device memory during the call: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  Same arguments, checks,
 * kernels and results as kev_packed_attn_prefill (bitwise); it calls no
 * hipMalloc, hipFree or allocating library routine.
 *
 * Its work list and its error word live in a device array of 4 MiB that the
 * library holds on every GPU it runs on until the process ends.  A call whose
 * work list needs more (about 5 M tokens at the 48-row blocks of the 32/8-head,
 * head_dim-128 shape, fewer with more questions) returns KEV_ERR_SCRATCH_LIMIT
 * and enqueues nothing.  Every call on one GPU shares that array, and a call
 * overwrites what the previous one left there: calls that overlap on one GPU
 * (on different streams, or from different host threads without ordering) race
 * and are not allowed.  Device-array errors set bits in the array's own error word, which
 * the next kev_get_device_errors on that GPU (any stream) reports and clears.
 * KEV_CHECK and KEV_LOG are ignored (both would copy to the host and wait).
 */
int kev_packed_attn_prefill_noalloc(const void *q, const void *k, const void *v,
                                    const int32_t *cu_seqlens, int32_t n_seg,
                                    int32_t heads, int32_t kv_heads, int32_t head_dim,
                                    void *out, int32_t total_tokens, int32_t dtype, void *stream);

/*
 * KV slot pool geometry.  `data` is a caller-owned device buffer laid out as
 *   [n_slots][2][kv_heads][capacity][head_dim]      (index 0 = K, 1 = V)
 * i.e. each slot is one contiguous block holding a per-head cache
 * [kv_heads][capacity][head_dim] for K followed by the same for V.
 */
typedef struct {
    void *data;
    int32_t n_slots;
    int32_t capacity;
    int32_t kv_heads;
    int32_t head_dim;
    int32_t dtype; /* kev_dtype; KEV_BF16 only */
} kev_kv_pool;

/*
 * Single-token decode over the slot pool, with in-kernel append.
 *
 *   q            [n_req, heads, head_dim]          bf16
 *   kv_pool      host pointer to the pool descriptor (read during the call only)
 *   slot_ids     int32 [n_req], device; distinct slots in [0, n_slots)
 *   cache_lens   int32 [n_req], device; tokens in the slot AFTER the append,
 *                in [1, capacity] (1 = empty cache before this step)
 *   out          [n_req, heads, head_dim]          bf16
 *   k_new, v_new [n_req, kv_heads, head_dim]       bf16
 *
 * For request r with slot s = slot_ids[r] and L = cache_lens[r]: row L-1 of
 * slot s (K and V, every KV head) is overwritten with k_new[r] / v_new[r];
 * then query r attends over rows 0..L-1 of slot s.  No other pool byte is
 * written.  Repeated slot ids in one call are undefined behaviour (rejected
 * with KEV_ERR_BAD_SLOT under KEV_CHECK=1).  A slot is never truncated or
 * re-laid out: a length past capacity is an error, not a reallocation.
 * head_dim must be 64 or 128 and equal to the pool's.
 *
 * Small batches (fewer (request, KV head) units than CUs -- e.g. a batch that
 * has shrunk as requests finished and left, Kev part 2, gsyq.cn, section 2.3)
 * split every unit's positions over up to 8 workgroups and merge their
 * partial softmax states in a second kernel, using the stream's workspace.
 * The environment variable KEV_DECODE_SPLITS=N (1..32) forces N splits per
 * unit (1: never split); results agree within rounding either way.
 */
int kev_slot_attn_decode(const void *q, const kev_kv_pool *kv_pool,
                         const int32_t *slot_ids, const int32_t *cache_lens, void *out,
                         const void *k_new, const void *v_new, int32_t n_req, int32_t heads,
                         void *stream);

/*
 * Paged KV pool: n_blocks blocks of block_size positions each, stored as
 * [n_blocks][2][kv_heads][block_size][head_dim] (per block and KV head, the
 * block's K rows then, kv_heads*block_size*head_dim elements later, its V
 * rows).  A block is a slot of capacity block_size; blocks are handed out on
 * demand and may sit anywhere (primer, sakurs2.com, section 2.5).
 */
typedef struct kev_paged_pool {
    void *data;         /* device pointer */
    int32_t n_blocks;
    int32_t block_size; /* a power of two */
    int32_t kv_heads;
    int32_t head_dim;
    int32_t dtype;      /* kev_dtype; KEV_BF16 only */
} kev_paged_pool;

/* Most blocks one paged decode request may span (block ids are staged on chip). */
#define KEV_PAGED_MAX_BLOCKS 2048

/*
 * Single-token decode over a paged pool, with in-kernel append: the step of
 * kev_slot_attn_decode, with position p of request r found in block
 * block_tables[r * max_blocks + p / block_size], row p % block_size, rather
 * than in a contiguous slot (primer, sakurs2.com, section 2.5: the attention
 * reads K/V through the block table, without first gathering them into one
 * contiguous span).  Row L-1 (L = cache_lens[r]) of that mapping is
 * overwritten with k_new[r] / v_new[r] in place (same page, section 2.2), and
 * query r attends over positions 0..L-1 with no mask.
 *
 *   q            [n_req, heads, head_dim]          bf16
 *   kv_pool      host pointer to the paged pool descriptor
 *   block_tables int32 [n_req, max_blocks], device; entries 0..(L-1)/block_size
 *                of row r are block ids in [0, n_blocks), the rest are not read
 *   cache_lens   int32 [n_req], device; positions AFTER the append, in
 *                [1, min(max_blocks, KEV_PAGED_MAX_BLOCKS) * block_size]
 *   out          [n_req, heads, head_dim]          bf16
 *   k_new, v_new [n_req, kv_heads, head_dim]       bf16
 *
 * Blocks may be shared between requests for reading (a common prefix), but
 * the row a request appends must be read or written by no other request of
 * the call (rejected with KEV_ERR_BAD_SLOT under KEV_CHECK=1; undefined
 * otherwise).  A request with a block id outside the pool, or a length out
 * of range, is skipped (KEV_DEVERR_BLOCK / KEV_DEVERR_CACHE_LEN).  head_dim
 * must be 64 or 128 and at most 32 query heads may share a KV head.  Small
 * batches are split as for kev_slot_attn_decode.
 */
int kev_paged_attn_decode(const void *q, const kev_paged_pool *kv_pool, const int32_t *block_tables,
                          int32_t max_blocks, const int32_t *cache_lens, void *out,
                          const void *k_new, const void *v_new, int32_t n_req, int32_t heads,
                          void *stream);

/*
 * Packed prefill that also hands each question its slot: the prefill above,
 * then question s's K and V rows become rows 0..len_s-1 of slot slot_ids[s]
 * (every KV head, K and V planes), written in place -- each question gets a
 * slot on entry and decode continues it there (Kev part 2, gsyq.cn, section
 * 2.2; primer, sakurs2.com, section 2.2).  A following kev_slot_attn_decode
 * with cache_lens[r] = len_s + 1 appends the question's next token.
 *
 *   q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens:
 *                as for kev_packed_attn_prefill (bf16 only)
 *   kv_pool      host pointer to the pool descriptor; kv_heads and head_dim
 *                must equal the call's, dtype KEV_BF16
 *   slot_ids     int32 [n_seg], device; distinct slots in [0, n_slots)
 *
 * Rows len_s .. capacity-1 of a slot and all other slots are not written.
 * A question longer than the capacity, or with an out-of-range slot id, is
 * not stored (KEV_DEVERR_CACHE_LEN / KEV_DEVERR_SLOT in the device error
 * word; KEV_ERR_SLOT_OVERFLOW / KEV_ERR_BAD_SLOT under KEV_CHECK=1, which also
 * rejects repeated slot ids); its attention output is still computed.
 */
int kev_packed_attn_prefill_slots(const void *q, const void *k, const void *v,
                                  const int32_t *cu_seqlens, int32_t n_seg, int32_t heads,
                                  int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                                  const kev_kv_pool *kv_pool, const int32_t *slot_ids, void *stream);

/*
 * Chunked prefill against a slot prefix.  Question s of the packed stream is
 * a chunk of len_s = cu_seqlens[s+1] - cu_seqlens[s] tokens that continues the
 * P_s = prefix_lens[s] rows already held in slot slot_ids[s].  Chunk row i is
 * position P_s + i of its question and attends, under the causal mask of the
 * primer (sakurs2.com, sections 2.1 and 2.6), to slot rows 0..P_s-1 and chunk
 * rows 0..i of its own question only; other questions stay invisible (Kev
 * article, icman.com.cn, sections 2.1 and 2.3).  The slot is the question's
 * own (Kev part 2, gsyq.cn, section 2.2).  After the call the chunk's K and V
 * rows are rows P_s..P_s+len_s-1 of the slot (every KV head), written in place.
 *
 *   q, k, v, cu_seqlens, n_seg, heads, kv_heads, head_dim, out, total_tokens:
 *                as for kev_packed_attn_prefill (bf16 only), describing the
 *                chunks' own tokens
 *   kv_pool      host pointer to the pool descriptor; kv_heads and head_dim
 *                must equal the call's, dtype KEV_BF16
 *   slot_ids     int32 [n_seg], device; distinct slots in [0, n_slots)
 *   prefix_lens  int32 [n_seg], device; cached rows per question, with
 *                0 <= P_s and P_s + len_s <= capacity (P_s = 0 is a fresh
 *                question: the call then equals kev_packed_attn_prefill_slots)
 *
 * The prefix rows are read, never written; rows past P_s + len_s and other
 * slots are untouched.  A question whose slot id is out of range, or whose
 * rows overflow the slot, gets neither output rows nor stored rows
 * (KEV_DEVERR_SLOT / KEV_DEVERR_CACHE_LEN in the device error word;
 * KEV_ERR_BAD_SLOT / KEV_ERR_SLOT_OVERFLOW under KEV_CHECK=1, which also
 * rejects repeated slot ids).
 */
int kev_chunked_prefill_slots(const void *q, const void *k, const void *v,
                              const int32_t *cu_seqlens, int32_t n_seg, int32_t heads,
                              int32_t kv_heads, int32_t head_dim, void *out, int32_t total_tokens,
                              const kev_kv_pool *kv_pool, const int32_t *slot_ids,
                              const int32_t *prefix_lens, void *stream);

/*
 * Profiling hook.  Until called again with NULL, every call on this host
 * thread records `start` (a hipEvent_t passed as void*) on its stream right
 * before launching its main kernel -- the attention kernel of a prefill (not
 * the work-list pass or the K/V store), the decode kernel (and, for split
 * units, its merge kernel) -- and `end` right after it, so the events time
 * that kernel alone.  Both NULL clears; exactly one NULL is KEV_ERR_INVALID_ARG.
 * The events are the caller's and must stay valid while set.
 */
int kev_set_kernel_events(void *start, void *end);

/* Human-readable text for a kev_status value (static storage). */
const char *kev_status_string(int status);

/*
 * Reads and clears the error word of (current device, `stream`) into
 * *flags_out (a KEV_DEVERR_* bitmask, 0 if every unit of every call enqueued
 * on `stream` since the last read was valid), after all work enqueued on
 * `stream` before this call; returns once the read is done (synchronises
 * `stream`).  Flags raised by calls on other streams are not seen here, except
 * those of kev_packed_attn_prefill_noalloc, whose one error word per device is
 * read and cleared too.
 */
int kev_get_device_errors(void *stream, int32_t *flags_out);

/*
 * Schedule inspection (tests and tuning).
 *
 * kev_prefill_block_rows: query rows per work item that a prefill call with
 * these arguments uses (0 if the combination is unsupported).
 *
 * kev_prefill_order: the work-list order a prefill call with these arguments
 * uses.  Currently always KEV_ORDER_QUESTION (question by question, longest
 * question first, query block descending inside a question, so concurrently
 * running workgroups share one question's rows in the L2 of their XCD).
 * KEV_ORDER_LEVEL (query block descending over all questions, longest items
 * first overall) is available to the schedule entry points below.
 *
 * kev_schedule_host: the work list computed on the host from a HOST copy of
 * cu_seqlens in the given order: items_out[2*i] = question, items_out[2*i+1] =
 * query block.  Questions of equal block count come by index here and in an
 * unspecified order on the device.  Returns KEV_OK and *n_items_out, or
 * KEV_ERR_INVALID_ARG if max_items is too small or the order is unknown.
 *
 * kev_schedule_device: runs the device scheduler kernel on device cu_seqlens
 * and copies its work list to the host buffer items_out (synchronises).
 */
#define KEV_ORDER_QUESTION 0
#define KEV_ORDER_LEVEL 1
int kev_prefill_block_rows(int32_t heads, int32_t kv_heads, int32_t head_dim, int32_t dtype);
int kev_prefill_order(int32_t total_tokens, int32_t head_dim, int32_t dtype);
int kev_schedule_host(const int32_t *cu_seqlens_host, int32_t n_seg, int32_t block_rows,
                      int32_t order, int32_t *items_out, int32_t max_items, int32_t *n_items_out);
int kev_schedule_device(const int32_t *cu_seqlens, int32_t n_seg, int32_t total_tokens,
                        int32_t block_rows, int32_t order, int32_t *items_out, int32_t max_items,
                        int32_t *n_items_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KEV_H */
