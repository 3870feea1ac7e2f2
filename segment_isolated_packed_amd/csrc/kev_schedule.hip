// kev_schedule.hip -- device work-list builder for the packed prefill.
//
// Replaces the dense mask: the pages build a T x T causal x block-diagonal
// matrix (Kev article, icman.com.cn, sections 2.3 and 5.3) whose construction
// they measure at 15-20% of inference time (section 5.4) and whose size grows
// as T^2 (section 6.4).  Here one workgroup reads cu_seqlens and lists the
// (question, query block) items; the attention kernel then visits only key
// blocks inside the item's own question at or left of its diagonal, so
// cross-question and future tiles are never loaded.
//
// Orders (item t costs t+1 key blocks; questions of equal block count come in an
// unspecified order: an atomic counting sort):
//  - question-major: questions in descending number of query blocks, the items of
//    one question with t descending.  Workgroups that run at the same time then
//    mostly share one question's K/V rows, which stay in the L2 of their XCD.
//  - level-major: t descending over all questions, ties by descending length.  The
//    longest items are issued first overall, the best balance of the two.
// The order only decides which workgroup computes what: every item is computed the
// same way wherever it runs, so outputs do not depend on it.
#include "kev_internal.h"
#include "../../include/kev.h"

namespace kev {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;

// Inclusive prefix sum over the workgroup; *total receives the sum of all v.
__device__ int32_t block_scan(int32_t v, int32_t *lds, int32_t *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        int32_t t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    if (lane == 63) lds[wave] = v;
    __syncthreads();
    if (wave == 0) {
        int32_t w = lane < kWaves ? lds[lane] : 0;
#pragma unroll
        for (int o = 1; o < kWaves; o <<= 1) {
            int32_t t = __shfl_up(w, o);
            if (lane >= o) w += t;
        }
        if (lane < kWaves) lds[lane] = w;
    }
    __syncthreads();
    int32_t add = wave > 0 ? lds[wave - 1] : 0;
    *total = lds[kWaves - 1];
    __syncthreads();
    return v + add;
}

// Tables live in LDS when they fit (the common case: a few hundred questions
// and query blocks), else in the global workspace; the code is the same through
// generic pointers.
constexpr int kLds = 2048;

__global__ __launch_bounds__(kThreads) void schedule_kernel(ScheduleArgs a) {
    __shared__ int32_t lds[kWaves];
    __shared__ int32_t s_bad, s_maxnb;
    __shared__ int32_t t_cu[kLds + 1], t_hist[kLds], t_fill[kLds], t_cnt[kLds], t_start[kLds],
        t_sigma[kLds], t_qoff[kLds];
    const int tid = threadIdx.x;
    const ScheduleLayout lay = schedule_layout(a.n_seg, a.hist_len, a.n_max_items);   // one stream
    int32_t *ws = a.ws;
    int32_t *items = ws + lay.items;
    int4 *rec = reinterpret_cast<int4 *>(ws + lay.rec);
    const int32_t br = a.block_rows;
    const bool cu_small = a.n_seg + 1 <= kLds + 1;

    const int32_t *cu = a.cu;
    if (cu_small) {
        for (int i = tid; i <= a.n_seg; i += kThreads) t_cu[i] = a.cu[i];
        cu = t_cu;
    }
    if (tid == 0) {
        s_bad = (a.cu[0] != 0 || a.cu[a.n_seg] != a.total_tokens) ? 1 : 0;
        s_maxnb = 0;
    }
    __syncthreads();

    // Query blocks per question: validity and the largest count.
    int32_t my_max = 0, bad = 0;
    for (int s = tid; s < a.n_seg; s += kThreads) {
        int32_t len = cu[s + 1] - cu[s];
        int32_t nb = qblocks(len, br);
        if (len < 0 || nb + 1 >= a.hist_len) bad = 1;
        else my_max = max(my_max, nb);
    }
    if (bad) atomicOr(&s_bad, 1);
    atomicMax(&s_maxnb, my_max);
    __syncthreads();
    if (s_bad) {
        if (tid == 0) {
            ws[0] = 0;
            atomicOr(a.err, (int32_t)KEV_DEVERR_SEQLENS);
        }
        return;
    }
    const int32_t maxnb = s_maxnb;
    const bool small = maxnb + 2 <= kLds && a.n_seg <= kLds;
    int32_t *hist = small ? t_hist : ws + lay.hist;
    int32_t *fill = small ? t_fill : ws + lay.fill;
    int32_t *cnt = small ? t_cnt : ws + lay.cnt;
    int32_t *start = small ? t_start : ws + lay.start;
    int32_t *sigma = small ? t_sigma : ws + lay.sigma;
    int32_t *qoff = small ? t_qoff : ws + lay.qoff;

    for (int i = tid; i < maxnb + 2; i += kThreads) {
        hist[i] = 0;
        fill[i] = 0;
    }
    __syncthreads();
    for (int s = tid; s < a.n_seg; s += kThreads) atomicAdd(&hist[qblocks(cu[s + 1] - cu[s], br)], 1);
    __syncthreads();

    // cnt[c] = #questions with more than c query blocks = sum of hist[c+1 .. maxnb].
    int32_t carry = 0, tot;
    for (int base = 0; base < maxnb; base += kThreads) {
        int j = base + tid;
        int32_t x = j < maxnb ? hist[maxnb - j] : 0;
        int32_t incl = block_scan(x, lds, &tot) + carry;
        if (j < maxnb) cnt[maxnb - 1 - j] = incl;
        carry += tot;
    }
    if (tid == 0) cnt[maxnb] = 0;
    __syncthreads();
    const int32_t n_q = maxnb > 0 ? cnt[0] : 0;   // questions with at least one block

    // sigma: questions in descending block count.
    for (int s = tid; s < a.n_seg; s += kThreads) {
        int32_t nb = qblocks(cu[s + 1] - cu[s], br);
        if (nb > 0) sigma[cnt[nb] + atomicAdd(&fill[nb], 1)] = s;
    }
    __syncthreads();

    int32_t n_items;
    if (a.order == kOrderLevel) {
        // start[e] = first item of level e (query block t = maxnb-1-e), which holds the
        // cnt[t] questions with more than t blocks: sigma[0 .. cnt[t]).
        carry = 0;
        for (int base = 0; base < maxnb; base += kThreads) {
            const int e = base + tid;
            const int32_t y = e < maxnb ? cnt[maxnb - 1 - e] : 0;
            const int32_t incl = block_scan(y, lds, &tot) + carry;
            if (e < maxnb) start[e] = incl - y;
            carry += tot;
        }
        n_items = carry;
        __syncthreads();
        for (int p = tid; p < n_items; p += kThreads) {
            int lo = 0, hi = maxnb - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (start[mid] <= p) lo = mid;
                else hi = mid - 1;
            }
            const int32_t s = sigma[p - start[lo]], t = maxnb - 1 - lo;
            items[2 * p] = s;
            items[2 * p + 1] = t;
            rec[p] = make_int4(cu[s], cu[s + 1] - cu[s], t, s);
        }
    } else {
        // qoff[r] = first item of the r-th question in that order.
        carry = 0;
        for (int base = 0; base < n_q; base += kThreads) {
            const int r = base + tid;
            int32_t nb = 0;
            if (r < n_q) {
                const int32_t s = sigma[r];
                nb = qblocks(cu[s + 1] - cu[s], br);
            }
            const int32_t incl = block_scan(nb, lds, &tot) + carry;
            if (r < n_q) qoff[r] = incl - nb;
            carry += tot;
        }
        n_items = carry;
        __syncthreads();
        // Item p belongs to the last question r with qoff[r] <= p; its t counts down from nb-1.
        for (int p = tid; p < n_items; p += kThreads) {
            int lo = 0, hi = n_q - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (qoff[mid] <= p) lo = mid;
                else hi = mid - 1;
            }
            const int32_t s = sigma[lo];
            const int32_t nb = qblocks(cu[s + 1] - cu[s], br);
            const int32_t t = nb - 1 - (p - qoff[lo]);
            items[2 * p] = s;
            items[2 * p + 1] = t;
            rec[p] = make_int4(cu[s], cu[s + 1] - cu[s], t, s);
        }
    }
    if (tid == 0) ws[0] = n_items;
}

// The same work list for at most 64 questions, built by one wavefront with every question
// in a lane: no LDS tables and no workgroup barriers, so the pass costs little more than one
// read of cu_seqlens and the stores of the list.  Ties in block count go by question index.
__global__ __launch_bounds__(64) void schedule_small_kernel(ScheduleArgs a) {
    const ScheduleLayout lay = schedule_layout(a.n_seg, a.hist_len, a.n_max_items * max(a.n_streams, 1));
    int32_t *ws = a.ws;
    int32_t *items = ws + lay.items;
    int4 *rec = reinterpret_cast<int4 *>(ws + lay.rec);
    const int lane = threadIdx.x;
    int q0 = 0, len = 0;
    if (lane < a.n_seg) {
        q0 = a.cu[lane];
        len = a.cu[lane + 1] - q0;
    }
    const int nb = lane < a.n_seg ? qblocks(len, a.block_rows) : 0;
    const bool bad = __any(len < 0 || nb + 1 >= a.hist_len) || a.cu[0] != 0 || a.cu[a.n_seg] != a.total_tokens;
    if (bad) {
        if (lane == 0) {
            ws[0] = 0;
            atomicOr(a.err, (int32_t)KEV_DEVERR_SEQLENS);
        }
        return;
    }
    // rank: position in descending order key (ties by index); before: items of the questions
    // ranked ahead (question-major offset of this question's first item).  The key is the
    // block count, or for chunks continuing a cached prefix the blocks of prefix + chunk, so
    // that the questions whose items read the most keys come first.
    int key = nb;
    if (a.prefix_lens && a.order != kOrderLevel && lane < a.n_seg && nb > 0)   // level-major needs nb order
        key = qblocks(max(a.prefix_lens[lane], 0) + len, a.block_rows);
    int rank = 0, before = 0, maxnb = 0;
    for (int j = 0; j < a.n_seg; ++j) {
        const int nj = __builtin_amdgcn_readlane(nb, j);
        const int kj = __builtin_amdgcn_readlane(key, j);
        const bool ahead = kj > key || (kj == key && j < lane);
        rank += ahead ? 1 : 0;
        before += ahead ? nj : 0;
        maxnb = max(maxnb, nj);
    }
    int n_items = 0;
    for (int j = 0; j < a.n_seg; ++j) n_items += __builtin_amdgcn_readlane(nb, j);
    if (a.order == kOrderLevel) {
        // level t holds the questions with more than t blocks, in rank order; levels go
        // from t = maxnb-1 down, so item (q, t) sits after every item of the levels above
        int above = 0;   // items in levels t' > t
        for (int t = maxnb - 1; t >= 0; --t) {
            if (nb > t) {
                const int p = above + rank;
                items[2 * p] = lane;
                items[2 * p + 1] = t;
                rec[p] = make_int4(q0, len, t, lane);
            }
            int c = 0;
            for (int j = 0; j < a.n_seg; ++j) c += __builtin_amdgcn_readlane(nb, j) > t ? 1 : 0;
            above += c;
        }
    } else if (a.n_streams > 1) {
        // Streams of whole questions: in rank order, each question joins the stream with the
        // least work so far (work of a question: the key blocks its items read, prefix included),
        // and takes the next items of that stream.  Stream s owns records [s * cap, (s+1) * cap);
        // the records after its last item get length -1.
        const int pre = (a.prefix_lens && lane < a.n_seg && nb > 0) ? max(a.prefix_lens[lane], 0) : 0;
        const float work = (float)nb * (float)qblocks(pre, a.block_rows) + 0.5f * (float)nb * (float)(nb + 1);
        const int64_t cap = a.n_max_items;
        float load[kStreamsMax];
        int fill[kStreamsMax];
#pragma unroll
        for (int st = 0; st < kStreamsMax; ++st) {
            load[st] = 0.f;
            fill[st] = 0;
        }
        int my_stream = 0, my_pos = 0;
        for (int k = 0; k < a.n_seg; ++k) {
            const uint64_t who = __ballot(lane < a.n_seg && rank == k);
            const int ql = (int)__builtin_ctzll(who);   // ranks are a permutation: always hit
            const int qnb = __builtin_amdgcn_readlane(nb, ql);
            if (qnb == 0) continue;
            const float qw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(work), ql));
            int best = 0;
            float bl = load[0];
#pragma unroll
            for (int st = 1; st < kStreamsMax; ++st)
                if (st < a.n_streams && load[st] < bl) {
                    best = st;
                    bl = load[st];
                }
            int at = 0;
#pragma unroll
            for (int st = 0; st < kStreamsMax; ++st)
                if (st == best) {
                    at = fill[st];
                    fill[st] += qnb;
                    load[st] += qw;
                }
            if (lane == ql) {
                my_stream = best;
                my_pos = at;
            }
        }
        // A chunk that continues a cached prefix lists its query blocks in ascending order:
        // a prefix's K/V (up to an L2's worth) is then swept by the blocks of the chunk in the
        // order they start, so later blocks find more of it still resident.  Fresh questions
        // rank last in their stream and keep the descending order (longest item first).
        for (int k = 0; k < nb; ++k) {
            const int64_t p = my_stream * cap + my_pos + k;
            const int t = pre > 0 ? k : nb - 1 - k;
            items[2 * p] = lane;
            items[2 * p + 1] = t;
            rec[p] = make_int4(q0, len, t, lane);
        }
#pragma unroll
        for (int st = 0; st < kStreamsMax; ++st)
            if (st < a.n_streams)
                for (int64_t p = fill[st] + lane; p < cap; p += 64) rec[st * cap + p] = make_int4(0, -1, 0, 0);
    } else {
        for (int k = 0; k < nb; ++k) {
            const int p = before + k, t = nb - 1 - k;
            items[2 * p] = lane;
            items[2 * p + 1] = t;
            rec[p] = make_int4(q0, len, t, lane);
        }
    }
    if (lane == 0) ws[0] = n_items;
}

}  // namespace

hipError_t launch_schedule(const ScheduleArgs &a, hipStream_t s) {
    if (a.n_seg <= 64) hipLaunchKernelGGL(schedule_small_kernel, dim3(1), dim3(64), 0, s, a);
    else hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace kev
