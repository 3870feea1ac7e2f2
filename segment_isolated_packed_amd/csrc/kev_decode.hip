// kev_decode.hip -- single-token decode over a slot-partitioned KV pool (gfx950).
//
// Request r owns slot s = slot_ids[r] of a pre-allocated pool cut into
// fixed-capacity slots (Kev part 2, gsyq.cn, section 2.2).  Its new K/V row is
// written in place at position L-1 = cache_lens[r]-1 (primer, sakurs2.com,
// section 2.2: engines write the new position into pre-allocated space rather
// than concatenating), and its query attends over positions 0..L-1 of its own
// slot with no mask (same section: the new query is last, so every cached
// position is visible).  Nothing outside rows 0..L-1 of slot s is read.
//
// Decode reads every cached K/V byte once and does little arithmetic per byte,
// so the kernel is shaped for HBM bandwidth, which on this part needs many
// bytes in flight per CU and neighbouring addresses in flight together:
//   - one workgroup of four wavefronts per unit (request, KV head); wavefront
//     w takes the unit's 32-position tiles w, w+4, w+8, ..., so the four read
//     adjacent 8 KB blocks of the K and V planes at the same time.  Two
//     workgroups share a CU (eight wavefronts, one K and one V tile in flight
//     each);
//   - a tile is loaded row-wise (16 bytes per lane, whole 256-byte rows, with
//     the nontemporal hint: each row is read once) into registers, written to the wavefront's own LDS buffers in the swizzled
//     layout of kev_mfma_core.h, and read back as MFMA fragments; the next
//     tile's loads are issued as soon as the registers are free, so they fly
//     while the current tile is computed.  LDS holds 16 KB per wavefront, not
//     a multi-stage pipeline, which is what allows eight wavefronts per CU;
//   - the `group` query heads of the KV head are the columns of MFMA tiles
//     (v_mfma_f32_32x32x16_bf16: S^T = K Q^T, O^T += V^T P^T), so the dot
//     products and the weighted sum of V cost matrix-core cycles, not VALU;
//   - the softmax is online (running max / sum / rescaled accumulator, primer
//     section 2.4) within each wavefront; the four partial states are merged
//     in LDS with the same rescaling identity, so a call is one kernel with
//     no global partials;
//   - when there are more units than the CUs hold at once (and at most 64
//     requests), workgroups are issued longest unit first, so the short units
//     fill in at the end; when every unit is resident at once but CUs hold two,
//     long and short units are paired on a CU, so no CU is left with two long ones.
//
// Paged variant (the PAGED instantiation).  The cache may instead be cut into
// fixed-size blocks of B positions placed anywhere in the pool, request r
// finding position p in block block_tables[r][p / B], row p % B (primer,
// section 2.5: blocks allocated on demand and read through a block table, not
// copied into one contiguous span first).  A block holds, per KV head, B K
// rows then B V rows, i.e. it is a slot of capacity B.  The workgroup first
// copies the request's block ids into LDS (checking them), then every row
// address of a tile is looked up there; the rest of the kernel is unchanged.
//
// Split units (the SPLIT instantiation).  With few requests -- a batch that
// shrinks as requests finish and leave (Kev part 2, gsyq.cn, section 2.3) --
// one workgroup per unit leaves most CUs idle and each unit's time is bound
// by the latency of one workgroup's loads.  The unit's tiles are then cut
// into n_split contiguous ranges, one workgroup each; a workgroup writes its
// unnormalised state (O^T, running max, row sum per query head) to a
// workspace, and decode_merge_kernel combines the ranges with the same
// rescaling identity and writes the output.
#include "kev_internal.h"
#include "kev_mfma_core.h"
#include "../../include/kev.h"

namespace kev {

namespace {

using namespace core;

constexpr int DKT = 32;        // positions per tile
constexpr int kWaves = 4;      // wavefronts per workgroup (one unit)

template <bool PAGED>
__device__ inline bool req_valid(int slot, int L, const DecodeArgs &p) {
    if constexpr (PAGED) return L >= 1 && ((L - 1) >> p.block_shift) < min(p.max_blocks, kDecodeMaxBlocks);
    return slot >= 0 && slot < p.n_slots && L >= 1 && L <= p.capacity;
}

// Request, slot and length for the workgroups of rank b_req: requests ordered by tile count,
// descending (ties by index).  Used when there are at most 64 requests and more units than
// the CUs hold at once, so that short units fill in at the end.
struct Req {
    int r, slot, L;
};
template <bool PAGED>
__device__ inline Req ranked_request(int b_req, const DecodeArgs &p, __attribute__((address_space(3))) int *keys) {
    const int lane = threadIdx.x & 63;
    int t = -1, sl = 0, ln = 0;
    if (lane < p.n_req) {
        sl = PAGED ? 0 : p.slot_ids[lane];
        ln = p.cache_lens[lane];
        t = req_valid<PAGED>(sl, ln, p) ? (ln + DKT - 1) / DKT : 0;
    }
    // Every lane's tile count goes to 64 words of this wavefront's own LDS, and each lane counts
    // the requests ranked ahead of it from broadcast reads of four counts at a time (lanes past
    // n_req hold -1 and rank last).  A loop of 64 lane reads into scalar registers, each
    // feeding a vector compare, took about twice as long on this path, which every workgroup
    // runs before its first load.
    keys[lane] = t;
    __builtin_amdgcn_wave_barrier();
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const __attribute__((address_space(3))) i32x4 *k4 = reinterpret_cast<const __attribute__((address_space(3))) i32x4 *>(keys);
    int rank = 0;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
        const i32x4 v = k4[q];
        const int j = 4 * q;
        rank += (v.x > t || (v.x == t && j < lane)) ? 1 : 0;
        rank += (v.y > t || (v.y == t && j + 1 < lane)) ? 1 : 0;
        rank += (v.z > t || (v.z == t && j + 2 < lane)) ? 1 : 0;
        rank += (v.w > t || (v.w == t && j + 3 < lane)) ? 1 : 0;
    }
    const uint64_t hit = __ballot(lane < p.n_req && rank == b_req);
    const int f = hit ? (int)__builtin_ctzll(hit) : 0;   // ranks are a permutation: always hit
    return Req{f, __builtin_amdgcn_readlane(sl, f), __builtin_amdgcn_readlane(ln, f)};
}

// 16 bytes of cached K/V, loaded with the nontemporal hint: every cached row is read once per
// call, and streaming loads keep the caches from allocating lines that are never read again
// (streaming reads of per-workgroup contiguous ranges ran at 7.1 TB/s with the hint on this
// part, 6.2 TB/s without).
__device__ __forceinline__ u32x4 stream_load(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// A unit with T tiles uses min(T, n_split) splits, so every split it uses has at least one
// tile; split s < that count takes tiles [split_begin(s), split_begin(s + 1)).
__device__ inline int splits_used(int T, int S) { return min(T, S); }
__device__ inline int split_begin(int s, int T, int Se) { return (int)((int64_t)s * T / Se); }

// Paged: the request's block ids 0..(L-1)/B, checked against the pool (all threads agree).
__device__ inline bool blocks_valid(const DecodeArgs &p, int r, int L) {
    const int n_bl = ((L - 1) >> p.block_shift) + 1;
    const int32_t *bt = p.block_tables + (int64_t)r * p.max_blocks;
    int bad = 0;
    for (int j = threadIdx.x; j < n_bl; j += blockDim.x) bad |= (bt[j] < 0 || bt[j] >= p.n_slots) ? 1 : 0;
    return !__syncthreads_or(bad);
}

template <int D, bool PAGED, bool SPLIT>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_bf16_kernel(DecodeArgs p) {
    using GM = Geom<D>;
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int TB = DKT * D * 2;                  // bytes of one K (or V) tile
    constexpr int RPI = GM::RPI, IPT = DKT / RPI;    // rows per 1 KB load, loads per tile
    constexpr int NO = DB * 16;                      // accumulator values per lane
    static_assert(kWaves * 2 * TB >= 2 * (NO + 2) * 64 * 4, "merge area must fit");
    // Tile buffers, then (paged) the request's block ids.
    __shared__ __attribute__((aligned(1024))) char smem[kWaves * 2 * TB + (PAGED ? kDecodeMaxBlocks * 4 : 0)];

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int col = lane & 31, half = lane >> 5;
    const int G = p.group, KVH = p.kv_heads;
    // Split grids are split-major: the first range of every unit, then the second, ...
    const int n_units = p.n_req * KVH;
    const int split = SPLIT ? blockIdx.x / n_units : 0;
    int ublk = SPLIT ? blockIdx.x - split * n_units : blockIdx.x;   // unit = request * KVH + head
    if (!SPLIT && p.ranked == 2) {
        // Paired order: the dispatcher gives every CU one workgroup of the first `cus` and then
        // a second one, so workgroups b and b + cus share a CU.  Units are ranked longest first
        // and workgroup b + cus takes the unit ranked as far from the end as b is from the
        // start: each CU holding two units gets a long one and a short one.
        ublk = blockIdx.x < p.cus ? blockIdx.x : n_units - 1 - (blockIdx.x - p.cus);
    }
    const int g = ublk % KVH;
    int r, slot, L;
    if (!SPLIT && p.ranked) {
        // ranking scratch: the first 256 bytes of this wavefront's own tile buffer, which it
        // fills only after the ranking
        const Req q = ranked_request<PAGED>(
            ublk / KVH, p, reinterpret_cast<__attribute__((address_space(3))) int *>((lds_t *)smem + wave * 2 * TB));
        r = q.r;
        slot = q.slot;
        L = q.L;
    } else {
        r = ublk / KVH;
        slot = PAGED ? 0 : p.slot_ids[r];
        L = p.cache_lens[r];
    }
    if (!req_valid<PAGED>(slot, L, p)) {
        if (g == 0 && split == 0 && threadIdx.x == 0)
            atomicOr(p.err, (int32_t)((!PAGED && (slot < 0 || slot >= p.n_slots)) ? KEV_DEVERR_SLOT
                                                                                   : KEV_DEVERR_CACHE_LEN));
        return;
    }
    const int T = (L + DKT - 1) / DKT;
    const int n_used = SPLIT ? splits_used(T, p.n_split) : 1;
    if (split >= n_used) return;                                      // a split the unit does not use
    const int t0 = SPLIT ? split_begin(split, T, n_used) : 0;         // this workgroup's tiles [t0, t1)
    const int t1 = SPLIT ? split_begin(split + 1, T, n_used) : T;
    const int n_mine = wave < t1 - t0 ? (t1 - t0 - 1 - wave) / kWaves + 1 : 0;   // t0+wave, +4, ...

    uint16_t *pool = static_cast<uint16_t *>(p.pool);
    const int64_t plane = (int64_t)p.capacity * D;   // paged: capacity is the block size
    uint16_t *kbase = pool + ((int64_t)slot * 2 * KVH + g) * plane;
    uint16_t *vbase = kbase + (int64_t)KVH * plane;
    int *tbl = reinterpret_cast<int *>(smem + kWaves * 2 * TB);
    if constexpr (PAGED) {
        // The request's block ids 0..(L-1)/B into LDS; an id outside the pool skips the request.
        const int n_bl = ((L - 1) >> p.block_shift) + 1;
        const int32_t *bt = p.block_tables + (int64_t)r * p.max_blocks;
        int bad = 0;
        for (int j = threadIdx.x; j < n_bl; j += kWaves * 64) {
            const int b = bt[j];
            bad |= (b < 0 || b >= p.n_slots) ? 1 : 0;
            tbl[j] = b;
        }
        if (__syncthreads_or(bad)) {
            if (g == 0 && split == 0 && threadIdx.x == 0) atomicOr(p.err, (int32_t)KEV_DEVERR_BLOCK);
            return;
        }
    }
    // Element offset of K row `key` of this unit in the pool (its V row is KVH*plane later).
    auto row_off = [&](int key) -> int64_t {
        if constexpr (PAGED)
            return ((int64_t)tbl[key >> p.block_shift] * 2 * KVH + g) * plane +
                   (int64_t)(key & (p.capacity - 1)) * D;
        else
            return ((int64_t)slot * 2 * KVH + g) * plane + (int64_t)key * D;
    };
    const uint16_t *knew = static_cast<const uint16_t *>(p.k_new) + ((int64_t)r * KVH + g) * D;
    const uint16_t *vnew = static_cast<const uint16_t *>(p.v_new) + ((int64_t)r * KVH + g) * D;
    lds_t *kbuf = (lds_t *)smem + wave * 2 * TB;
    lds_t *vbuf = kbuf + TB;

    // In-place append of the new token (by the wavefront that owns the unit's last tile).
    // That tile reads row L-1 from k_new / v_new and no other tile reads it, so the store
    // needs no ordering against any load.
    if (t1 == T && (T - 1 - t0) % kWaves == wave && lane < 2 * (D / 8)) {
        const int part = lane % (D / 8);
        uint16_t *dst = pool + row_off(L - 1) + (lane < D / 8 ? 0 : (int64_t)KVH * plane) + part * 8;
        const uint16_t *src = (lane < D / 8 ? knew : vnew) + part * 8;
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }

    // Query rows: lane holds head g*G + min(col, G-1), d = dc*16 + half*8 .. +8.
    bf16x8 qf[DC];
    {
        const uint16_t *qp = static_cast<const uint16_t *>(p.q) +
                             ((int64_t)r * p.heads + g * G + min(col, G - 1)) * D + half * 8;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) qf[dc] = *reinterpret_cast<const bf16x8 *>(qp + dc * 16);
    }

    // Row-wise tile loads: load i covers tile rows i*RPI .. +RPI, lane -> row i*RPI + lane/CPR,
    // chunk lane % CPR.  Rows at or past L-1 read row L-1 from k_new / v_new.
    const int lrow = lane / GM::CPR, lchunk = lane % GM::CPR;
    u32x4 kr[IPT], vr[IPT];
    auto load_tile = [&](int j) {
        const int k0 = j * DKT;
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int key = min(k0 + i * RPI + lrow, L - 1);
            const bool nw = key == L - 1;
            if constexpr (PAGED) {
                const int64_t off = row_off(key) + lchunk * 8;
                kr[i] = stream_load(nw ? knew + lchunk * 8 : pool + off);
                vr[i] = stream_load(nw ? vnew + lchunk * 8 : pool + off + (int64_t)KVH * plane);
            } else {
                const int64_t off = (int64_t)key * D + lchunk * 8;
                kr[i] = stream_load(nw ? knew + lchunk * 8 : kbase + off);
                vr[i] = stream_load(nw ? vnew + lchunk * 8 : vbase + off);
            }
        }
    };

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float cs = p.scale_log2;

    if (n_mine > 0) load_tile(t0 + wave);
    for (int it = 0; it < n_mine; ++it) {
        const int j = t0 + wave + it * kWaves;
        // Registers -> this wavefront's LDS tiles.  LDS operations of one wavefront run in
        // order, so these writes land after the previous tile's fragment reads and before
        // this tile's.
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int row = i * RPI + lrow;
            *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(kbuf + GM::off(row, lchunk)) = kr[i];
            *reinterpret_cast<__attribute__((address_space(3))) u32x4 *>(vbuf + GM::off(row, lchunk)) = vr[i];
        }
        if (it + 1 < n_mine) load_tile(j + kWaves);   // flies while this tile is computed

        const int k0 = j * DKT;
        f32x16 sc = scores1<D>(kbuf, 0, qf);
        if (k0 + DKT > L) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
                if (key >= L) sc[i] = -INFINITY;
            }
        }
        float mx = fmaxf(sc[0], sc[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, sc[i]), sc[i + 1]);
        mx = max_halves_valu(mx) * cs;
        if (__any(mx > m_run + kLazy)) {
            const float m_new = fmaxf(m_run, mx);
            const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
            m_run = m_new;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) o[db][i] *= alpha;
        }
        const float mneg = -m_run;
        bf16x8 pb[2];
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            f32x8 e;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = __builtin_amdgcn_exp2f(fmaf(sc[h8 * 8 + i], cs, mneg));
                l_run += e[i];
            }
            pb[h8] = __builtin_convertvector(e, bf16x8);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_frag<D>(vbuf, cc, db), pb[cc], o[db], 0, 0, 0);
    }

    // ---- merge the four wavefronts' states: 2 and 3 into 0 and 1, then 1 into 0 ----
    // Per lane: NO accumulator values, the running max (uniform over the lane pair) and the
    // lane's partial row sum, stored value-major ([k][lane]) in the freed tile buffers.
    float *mg = reinterpret_cast<float *>(smem);
    auto put = [&](int region) {
        float *b = mg + region * (NO + 2) * 64;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) b[(db * 16 + i) * 64 + lane] = o[db][i];
        b[NO * 64 + lane] = m_run;
        b[(NO + 1) * 64 + lane] = l_run;
    };
    auto take = [&](int region) {
        const float *b = mg + region * (NO + 2) * 64;
        const float m2 = b[NO * 64 + lane], l2 = b[(NO + 1) * 64 + lane];
        const float mn = fmaxf(m_run, m2);
        if (mn == -INFINITY) return;   // neither side saw a key
        const float f1 = __builtin_amdgcn_exp2f(m_run - mn), f2 = __builtin_amdgcn_exp2f(m2 - mn);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] = o[db][i] * f1 + b[(db * 16 + i) * 64 + lane] * f2;
        l_run = l_run * f1 + l2 * f2;
        m_run = mn;
    };
    __syncthreads();                        // every wavefront is done with its tile buffers
    if (wave >= 2) put(wave - 2);
    __syncthreads();
    if (wave < 2) take(wave);
    __syncthreads();
    if (wave == 1) put(0);
    __syncthreads();
    if (wave != 0) return;
    take(0);

    // Lanes l and l+32 hold the same head; rows d = db*32 + 8*(i/4) + 4*half + i%4.
    const float l_tot = sum_halves(l_run);
    if (col >= G) return;
    if constexpr (SPLIT) {
        // Unnormalised state of query head col over this tile range: O^T rows, max, row sum.
        const int64_t pidx = (int64_t)ublk * p.n_split + split;   // unit-major in the workspace
        float *po = p.part + (pidx * G + col) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4)
                *reinterpret_cast<f32x4 *>(po + db * 32 + g4 * 8 + half * 4) =
                    f32x4{o[db][g4 * 4], o[db][g4 * 4 + 1], o[db][g4 * 4 + 2], o[db][g4 * 4 + 3]};
        if (half == 0) {
            float *pml = p.part + (int64_t)gridDim.x * G * D + (pidx * G + col) * 2;
            *reinterpret_cast<float2 *>(pml) = float2{m_run, l_tot};
        }
        return;
    }
    const float inv = 1.f / l_tot;
    uint16_t *op = static_cast<uint16_t *>(p.out) + ((int64_t)r * p.heads + g * G + col) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) f[jj] = o[db][g4 * 4 + jj] * inv;
            *reinterpret_cast<bf16x4 *>(op + db * 32 + g4 * 8 + half * 4) = __builtin_convertvector(f, bf16x4);
        }
}

// Combines the partial states of every unit (one workgroup per unit): with M the largest
// running max over the unit's splits, out = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
// Latency decides this kernel's time, so every read is issued at once: the request's length,
// the {max, sum} pairs and the O rows of all n_split splits (those past the splits the unit
// used hold stale values that are never combined).  The weights are then formed once per
// head in LDS.  Units of invalid requests are skipped (the split kernel flagged them), so
// their outputs stay untouched.
template <int D, bool PAGED>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecodeArgs p) {
    __shared__ float wts[kMaxDecodeSplits * 32];   // [split][head]: m, then the weight
    __shared__ float sums[kMaxDecodeSplits * 32];  // [split][head]: l
    const int u = blockIdx.x, KVH = p.kv_heads, G = p.group, S = p.n_split;
    const int r = u / KVH, g = u % KVH;
    const int slot = PAGED ? 0 : p.slot_ids[r];
    const int L = p.cache_lens[r];
    const int64_t n_part = (int64_t)gridDim.x * S;   // workgroups of the split kernel
    const float *po = p.part + (int64_t)u * S * G * D;
    const float2 *pml = reinterpret_cast<const float2 *>(p.part + n_part * G * D) + (int64_t)u * S * G;
    for (int e = threadIdx.x; e < S * G; e += blockDim.x) {
        const float2 ml = pml[e];
        wts[e] = ml.x;
        sums[e] = ml.y;
    }
    constexpr int E4 = D / 4;                  // float4 columns per head
    const int n_el = G * E4;
    const bool mine = threadIdx.x < n_el;      // first output element of this thread
    const int h0 = mine ? threadIdx.x / E4 : 0, d40 = threadIdx.x % E4;
    f32x4 v[kMaxDecodeSplits];
#pragma unroll
    for (int s = 0; s < kMaxDecodeSplits; ++s)
        if (s < S && mine) v[s] = *reinterpret_cast<const f32x4 *>(po + ((int64_t)s * G + h0) * D + d40 * 4);
    if (!req_valid<PAGED>(slot, L, p)) return;
    if constexpr (PAGED) {
        if (!blocks_valid(p, r, L)) return;
    }
    const int Se = splits_used((L + DKT - 1) / DKT, S);
    __syncthreads();
    if (threadIdx.x < G) {
        const int h = threadIdx.x;
        float mx = -INFINITY;
        for (int s = 0; s < Se; ++s) mx = fmaxf(mx, wts[s * G + h]);
        float l = 0.f;
        for (int s = 0; s < Se; ++s) {
            const float w = __builtin_amdgcn_exp2f(wts[s * G + h] - mx);
            wts[s * G + h] = w;
            l += w * sums[s * G + h];
        }
        const float inv = 1.f / l;
        for (int s = 0; s < Se; ++s) wts[s * G + h] *= inv;
    }
    __syncthreads();
    uint16_t *out = static_cast<uint16_t *>(p.out) + ((int64_t)r * p.heads + g * G) * D;
    if (mine) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kMaxDecodeSplits; ++s)
            if (s < Se) acc += wts[s * G + h0] * v[s];
        *reinterpret_cast<bf16x4 *>(out + h0 * D + d40 * 4) = __builtin_convertvector(acc, bf16x4);
    }
    // more than 256 output elements (G * D / 4 > 256): the rest, one split after another
    for (int e = threadIdx.x + blockDim.x; e < n_el; e += blockDim.x) {
        const int h = e / E4, d4 = e % E4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int s = 0; s < Se; ++s)
            acc += wts[s * G + h] * *reinterpret_cast<const f32x4 *>(po + ((int64_t)s * G + h) * D + d4 * 4);
        *reinterpret_cast<bf16x4 *>(out + h * D + d4 * 4) = __builtin_convertvector(acc, bf16x4);
    }
}

}  // namespace

template <int D, bool PAGED>
hipError_t launch_decode_d(const DecodeArgs &a, hipStream_t s) {
    const int64_t units = (int64_t)a.n_req * a.kv_heads;
    const dim3 b(kWaves * 64);
    if (a.n_split <= 1) {
        hipLaunchKernelGGL((decode_bf16_kernel<D, PAGED, false>), dim3((unsigned)units), b, 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((decode_bf16_kernel<D, PAGED, true>), dim3((unsigned)(units * a.n_split)), b, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_merge_kernel<D, PAGED>), dim3((unsigned)units), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode_bf16(const DecodeArgs &a, int32_t head_dim, bool paged, hipStream_t s) {
    switch (head_dim * 2 + (paged ? 1 : 0)) {
    case 128: return launch_decode_d<64, false>(a, s);
    case 129: return launch_decode_d<64, true>(a, s);
    case 256: return launch_decode_d<128, false>(a, s);
    case 257: return launch_decode_d<128, true>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kev
