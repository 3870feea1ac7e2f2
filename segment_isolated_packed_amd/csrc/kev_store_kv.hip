// kev_store_kv.hip -- prefill-to-slot handoff: question K/V rows into the slot pool.
//
// Every question of a packed prefill gets a slot of the pre-allocated pool on
// entry (Kev part 2, gsyq.cn, section 2.2), and its K and V rows become rows
// 0..len-1 of that slot, written in place (primer, sakurs2.com, section 2.2),
// so that decode can continue each question from its slot.  For a chunk that
// continues P rows already in its slot (chunked prefill), the rows go to
// P..P+len-1 instead.
//
// The copy is pure data movement, bound by HBM: each workgroup moves 32 token
// rows of one KV head for K and for V, 16 bytes per lane, whole rows per
// instruction on both sides (the source rows are strided by kv_heads*d, the
// slot rows are contiguous), with the nontemporal hint on both sides since no
// byte is touched twice (10% less time than plain loads and stores on the
// chunked-prefill store of 67 MB).  A row's question comes from a binary search in
// cu_seqlens.  Rows of a question whose slot id or length is invalid are not
// written, and the device error word records why.
#include "kev_internal.h"
#include "../../include/kev.h"

namespace kev {

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 32;        // token rows per workgroup
constexpr int kThreads = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void store_kv_kernel(StoreKvArgs a) {
    constexpr int CPR = D / 8;                  // 16-byte chunks per row
    constexpr int RPP = kThreads / CPR;         // rows per pass
    const int g = blockIdx.x % a.kv_heads;
    const int row0 = (blockIdx.x / a.kv_heads) * kRows;
    const int chunk = threadIdx.x % CPR;
#pragma unroll
    for (int pass = 0; pass < kRows / RPP; ++pass) {
        const int t = row0 + pass * RPP + threadIdx.x / CPR;
        if (t >= a.total_tokens) return;
        // question s with cu[s] <= t < cu[s+1] (the last such s if empty questions repeat cu)
        int lo = 0, hi = a.n_seg - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (a.cu[mid] <= t) lo = mid;
            else hi = mid - 1;
        }
        const int s = lo;
        const int start = a.cu[s], len = a.cu[s + 1] - start;
        const int i = t - start;
        const int slot = a.slot_ids[s];
        const int P = a.prefix_lens ? a.prefix_lens[s] : 0;
        if (slot < 0 || slot >= a.n_slots) {
            if (i == 0 && chunk == 0 && g == 0) atomicOr(a.err, (int32_t)KEV_DEVERR_SLOT);
            continue;
        }
        if (P < 0 || len > a.capacity - P) {
            if (i == 0 && chunk == 0 && g == 0) atomicOr(a.err, (int32_t)KEV_DEVERR_CACHE_LEN);
            continue;
        }
        if (i < 0 || i >= len) continue;   // cu_seqlens not a valid partition (flagged by the prefill)
        const int pos = P + i;
        const int64_t plane = (int64_t)a.capacity * D;
        uint16_t *kdst = static_cast<uint16_t *>(a.pool) + ((int64_t)slot * 2 * a.kv_heads + g) * plane +
                         (int64_t)pos * D + chunk * 8;
        uint16_t *vdst = kdst + (int64_t)a.kv_heads * plane;
        const int64_t src = ((int64_t)t * a.kv_heads + g) * D + chunk * 8;
        const u32x4 kx = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.k) + src));
        const u32x4 vx = __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.v) + src));
        __builtin_nontemporal_store(kx, reinterpret_cast<u32x4 *>(kdst));
        __builtin_nontemporal_store(vx, reinterpret_cast<u32x4 *>(vdst));
    }
}

}  // namespace

hipError_t launch_store_kv(const StoreKvArgs &a, int32_t head_dim, hipStream_t s) {
    if (a.total_tokens == 0) return hipSuccess;
    const int64_t grid = (int64_t)((a.total_tokens + kRows - 1) / kRows) * a.kv_heads;
    switch (head_dim) {
    case 64: hipLaunchKernelGGL((store_kv_kernel<64>), dim3((unsigned)grid), dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL((store_kv_kernel<128>), dim3((unsigned)grid), dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kev
