// kev_prefill_bf16.hip -- packed, segment-isolated causal prefill on bf16 MFMA (gfx950).
//
// Computes, for every question interval [a, b) of the packed stream, query
// head h and row i in [a, b):
//     out[i,h,:] = sum_{j=a..i} softmax_j(q[i,h,:] . k[j,g,:] / sqrt(d)) v[j,g,:]
// with g = h / (heads / kv_heads): the primer's Z = softmax(QK^T/sqrt(d_h) + M)V
// (sakurs2.com, section 2.1) under the causal AND block-diagonal mask of the
// Kev article (icman.com.cn, sections 2.1, 2.3), evaluated FlashAttention-style:
// K/V tiles staged on chip, the score matrix never written to HBM, and the
// softmax kept as a running max, running sum and rescaled accumulator that are
// corrected whenever a later block raises the max (primer, section 2.4).
//
// Decomposition.  A work item from the scheduler is (question, block of W*R
// query rows); per KV head it holds G*R units of (query head of the group,
// W-row block), one wavefront each.  R is the smallest power of two with G*R
// a multiple of 4, so the units fill workgroups of exactly 4 wavefronts (one
// per SIMD).  Unit u of workgroup w is u = 4w + wave, with row block u / G and
// head u % G: a workgroup spans at most two adjacent row blocks, so its waves
// need nearly the same keys.  All four read the same K/V tiles from LDS.
// W = 48 for head_dim 128 (prefill_r48_kernel, three 16-row blocks on
// v_mfma_f32_16x16x32_bf16) and W = 32 for head_dim 64 (prefill_bf16_kernel,
// one 32-row block on v_mfma_f32_32x32x16_bf16).  Every wavefront issues the
// same loads, LDS reads and barriers per key tile whatever its row count, so
// more rows per wavefront spread that fixed cost over more MFMA work; 48 rows
// is what the register file holds at head_dim 128 (O^T 96 and Q 48 registers
// per lane).
//
// Placement.  Workgroups are dealt to the 8 XCDs round-robin by index, and
// each XCD has its own L2.  The KV head is the fastest-varying part of the
// workgroup index, so when kv_heads divides 8 every XCD serves a single KV
// head; with the scheduler's question-major order, the workgroups resident on
// one XCD then read the K/V rows of one (question, KV head) from its L2.  With
// fewer KV heads than XCDs (kv_heads = 4) the scheduler deals the questions to
// two item streams instead and each XCD serves one (stream, KV head) pair
// (PrefillArgs::n_streams), so no two XCDs fetch the same question's K/V.
//
// Occupancy.  A workgroup uses at most 80 KB of LDS and 256 registers per lane,
// so two workgroups share each CU and every SIMD runs two wavefronts that belong
// to different workgroups.  Their barriers are independent, so one wavefront's
// MFMA work can overlap the other's softmax work.
//
// MFMA orientation (fp32 accumulation):
//   S^T[key][q] = K_tile[key][:] . Q^T[:][q]     A = K from LDS, B = Q in VGPRs
//   O^T[d][q]  += V^T[d][key]   . P^T[key][q]    A = V^T from LDS, B = P^T in VGPRs
// With the query index on the lane (n = lane % 32 on the 32x32 MFMA, lane % 16
// on the 16x16 one), each lane owns one query row per row block: a row max
// needs an exchange between the two half-waves (four lanes on the 16x16
// MFMA), the rescale of O^T is lane-uniform, and P^T feeds the second MFMA
// straight from the first one's accumulators (converted to bf16).  Staging and
// operand reads are described in kev_mfma_core.h and at prefill_r48_kernel.
//
// Softmax.  The weights of a tile are taken against the running max as it
// stands and the max only moves when a lane's sum of its weights of the tile
// leaves a fixed bound (tile_pv, and the per-row move in prefill_r48_kernel),
// so the common tile spends one FMA and one exp per score, a bf16 conversion
// per pair and a dot product per pair for the row sum.
//
// Pipeline.  Tiles are 32 keys.  K and V each have NS LDS stages and direct
// loads run NS-1 tiles ahead: five stages (80 KB per workgroup) in the 32-row
// kernel, four (64 KB) in the 48-row kernel; either way two workgroups share a
// CU.  Iteration j starts with the scores of tile j already issued on MFMA.
// The wavefront waits for its own loads of K(j+1) and V(j), meets the others
// at one barrier (which also retires all reads of K(j) and V(j-1), so their
// stages take K(j+NS) and V(j+NS-1)), reads every fragment of V(j) and then
// K(j+1) into registers at once, takes the softmax of tile j while those reads
// land, runs P.V of tile j and issues the scores of tile j+1, which execute
// while it waits at the next barrier.  (The 48-row kernel has no room to hold
// both fragment sets through the softmax: it reads V(j) after the softmax and
// K(j+1) after P.V.)  The loop is unrolled by the stage count, so all LDS
// addresses carry the stage as an immediate offset.  In the 32-row kernel the
// wavefront holds a raised issue priority while it issues its 16 MFMAs of a
// tile, so that when both wavefronts of a SIMD have work ready the one feeding
// the matrix unit goes first and the other's softmax fills the gaps; the
// 48-row kernel ran faster without it (measured on every shape).  The softmax
// scale is waited for before the loop: a scalar load still in flight there
// would turn the first use of the scale in every tile into a wait for all
// outstanding LDS reads (scalar loads return out of order), and the softmax
// would then wait for the fragment reads it does not use.
// Only tiles inside the item's own question and at or left of its diagonal are
// loaded; the causal select (-inf, not a multiply) is applied only to tiles
// that cross a wavefront's diagonal or the end of the question.
//
// Chunked prefill (the PREFIX instantiation).  A question of the packed stream
// may be a chunk that continues P rows already cached in its slot of the KV
// pool: chunk row i is position P + i of the question and attends to the
// slot's rows 0..P-1 and the chunk's rows 0..i (primer, sakurs2.com, sections
// 2.1 and 2.6; the slot is the question's own, Kev part 2, gsyq.cn, section
// 2.2).  The kernel then walks the concatenated key sequence [slot rows ;
// chunk rows]: key tiles wholly inside the prefix are loaded from the slot
// (contiguous rows), tiles wholly inside the chunk from the packed K/V, and the
// one tile that straddles the boundary per lane from either.  The diagonal and
// the question end move right by P.  A question's K/V here can fill an XCD's L2,
// so the chunk's query rows and outputs go through with the non-temporal hint
// (read and written once, they should not displace K/V lines).
#include <type_traits>

#include "../../include/kev.h"
#include "kev_internal.h"
#include "kev_mfma_core.h"

namespace kev {

namespace {

using namespace core;

constexpr int KT = 32;      // keys per tile
constexpr int NWAVE = 4;    // wavefronts per workgroup
// LDS stages per tensor (loads run NS-1 tiles ahead): five for the 32-row kernel, four for
// the 48-row kernel (each measured against the other count on the same box).
constexpr int NS32 = 5;
constexpr int NS48 = 4;

template <int D, int NS>
struct Cfg {
    static constexpr int DC = D / 16;                    // k steps of the S MFMA
    static constexpr int DB = D / 32;                    // 32-row d blocks of O^T
    static constexpr int RPI = Geom<D>::RPI;             // tile rows per direct load
    static constexpr int IPT = KT / RPI;                 // direct loads per K (or V) tile
    static constexpr int NIT = IPT / NWAVE;              // per wavefront per tensor (4 waves)
    static constexpr int TB = KT * D * 2;                // bytes per tile
    static constexpr int LDS = 2 * NS * TB;
    static_assert(IPT % NWAVE == 0 && NIT >= 1, "loads must split evenly");
    static_assert(NS >= 4 && NS <= 5, "the loop is unrolled for four or five stages; the epilogue takes"
                                      " three K stages and one V stage that no wavefront still reads");
};

// Direct loads of K or V tiles by NW wavefronts.  Wavefront w fills tile rows
// ((w + NW*i) mod IPT) * RPI .. +RPI for i < NIT; when NW exceeds the number of loads per
// tile, several wavefronts issue the same load (same data to the same place), so every
// wavefront issues exactly NIT loads per tile and one vmcnt value fits all.  The global
// address is a wave-uniform tile base plus a per-lane offset that is the same for every
// full tile.  In the tile that holds key_end, rows at or past key_end are clamped to
// key_end - 1: a row of the same question, so nothing outside it is read.
//
// With PREFIX, key index kk < prefix is row kk of the slot's plane (rows D elements apart)
// and kk >= prefix is row kk - prefix of the packed K/V.
template <int D, int NW, bool PREFIX, int SW = 0>
struct TileLoader {
    static constexpr int RPI = Geom<D, SW>::RPI;
    static constexpr int IPT = KT / RPI;
    static constexpr int NIT = (IPT + NW - 1) / NW;
    static constexpr int PROW = D * 2;   // bytes per slot row
    unsigned voff[NIT];     // byte offset of this lane's chunk inside a full tile
    unsigned lds_row[NIT];  // LDS byte offset of the load's first row inside a stage
    const char *kbase, *vbase;  // packed K/V row of key `prefix`
    const char *pkbase, *pvbase;  // slot K/V planes (PREFIX only)
    int row_bytes;
    int key_end;
    int prefix;

    __device__ static int first_row(int wave, int i) { return ((wave + NW * i) % IPT) * RPI; }

    __device__ void init(const uint16_t *k, const uint16_t *v, int64_t row_stride, int kend, int wave,
                         const uint16_t *pk = nullptr, const uint16_t *pv = nullptr, int p = 0) {
        kbase = reinterpret_cast<const char *>(k);
        vbase = reinterpret_cast<const char *>(v);
        pkbase = reinterpret_cast<const char *>(pk);
        pvbase = reinterpret_cast<const char *>(pv);
        prefix = PREFIX ? p : 0;
        row_bytes = (int)(row_stride * 2);
        key_end = kend;
#pragma unroll
        for (int i = 0; i < NIT; ++i) {
            DmaLane<D, SW> ln;
            const int r0 = first_row(wave, i);
            ln.init(r0);
            voff[i] = (unsigned)(ln.row * row_bytes + ln.coff * 2);
            lds_row[i] = (unsigned)(r0 * Geom<D, SW>::ROWB);
        }
    }

    // A tile of the packed stream that ends before key_end (no clamped rows, no slot rows).
    __device__ __forceinline__ void issue_inner(const char *base, int tile, unsigned stage_addr) const {
        const char *tb = base + (int64_t)(tile * KT - prefix) * row_bytes;
#pragma unroll
        for (int i = 0; i < NIT; ++i) dma16s(tb, voff[i], stage_addr + lds_row[i]);
    }

    __device__ __forceinline__ void issue(const char *base, const char *pbase, int tile, unsigned stage_addr,
                                          int wave) const {
        const int k0 = tile * KT;
        if constexpr (PREFIX) {
            if (k0 + KT <= prefix) {   // whole tile in the slot
                const char *tb = pbase + (int64_t)k0 * PROW;
#pragma unroll
                for (int i = 0; i < NIT; ++i) {
                    DmaLane<D, SW> ln;
                    ln.init(first_row(wave, i));
                    dma16s(tb, (unsigned)(ln.row * PROW + ln.coff * 2), stage_addr + lds_row[i]);
                }
                return;
            }
            if (k0 < prefix) {         // straddles the slot / chunk boundary: per-lane source
#pragma unroll
                for (int i = 0; i < NIT; ++i) {
                    DmaLane<D, SW> ln;
                    ln.init(first_row(wave, i));
                    const int kk = min(k0 + ln.row, key_end - 1);
                    const char *g = kk < prefix ? pbase + (int64_t)kk * PROW + ln.coff * 2
                                                : base + (int64_t)(kk - prefix) * row_bytes + ln.coff * 2;
                    dma16(g, stage_addr + lds_row[i]);
                }
                return;
            }
        }
        const char *tb = base + (int64_t)(k0 - prefix) * row_bytes;
        if (k0 + KT <= key_end) {
#pragma unroll
            for (int i = 0; i < NIT; ++i) dma16s(tb, voff[i], stage_addr + lds_row[i]);
        } else {
#pragma unroll
            for (int i = 0; i < NIT; ++i) {
                DmaLane<D, SW> ln;
                ln.init(first_row(wave, i));
                const int r = min(k0 + ln.row, key_end - 1) - k0;
                dma16s(tb, (unsigned)(r * row_bytes + ln.coff * 2), stage_addr + lds_row[i]);
            }
        }
    }
};

// Online-softmax state of one lane (one query row; the lane pair l, l^32 shares it).
template <int D>
struct RowState {
    f32x16 o[D / 32];
    float m, l;
};

// Weights of a tile are taken against the running max m as it stands.  A lane's sum of its 16
// weights bounds each of them; only when that sum exceeds 2^15, or is not finite (the first
// tile, where m is still -inf), is m moved to the tile's max and O^T, l rescaled (rare after
// the first tile: the max has to grow by about 11 in log2 units).  Either way out = O / l is
// the same softmax average; the per-tile row max and its half-wave exchange leave the common
// path.
constexpr float kGuardSum = 32768.f;

// P = exp2(S*c - m) in bf16 (two 16-key chunks, the B operand of P.V) and this lane's sum of
// the 16 weights, taken from the bf16 values with v_dot2_f32_bf16 against (1, 1), so the row
// sum holds exactly the weights P.V uses.  (Inline asm: the compiler's builtin for this
// instruction, fed from a bit-cast vector, was seen to read the first pair for all four.)
__device__ __forceinline__ float tile_p(const f32x16 &s, float c, float mneg, bf16x8 *pb) {
    const unsigned one2 = 0x3F803F80u;   // bf16 (1, 1)
    float acc = 0.f;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
        f32x8 e;
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_exp2f(fmaf(s[cc * 8 + i], c, mneg));
        pb[cc] = __builtin_convertvector(e, bf16x8);
        const u32x4 w = __builtin_bit_cast(u32x4, pb[cc]);
#pragma unroll
        for (int i = 0; i < 4; ++i) asm("v_dot2_f32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(w[i]), "v"(one2));
    }
    return acc;
}

// Moves the running max of the rows that need it (`need`: the row's tile sum left the bound in
// either half-wave) to the max of the scored tile, and rescales their O^T and l.  Other rows
// keep their max (alpha = 1, exact), so their weights come out bit for bit as without the
// move: what a row computes never depends on another row's scores, and in particular not on
// keys past its diagonal that a later row of the same wavefront sees.
template <int D>
__device__ __forceinline__ void move_max(const f32x16 &s, float c, bool need, RowState<D> &st) {
    float mx = fmaxf(s[0], s[1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
    mx = max_halves_valu(mx) * c;
    const bool row_need = max_halves_valu(need ? 1.f : 0.f) > 0.f;
    const float m_new = row_need ? fmaxf(st.m, mx) : st.m;
    const float alpha = row_need ? __builtin_amdgcn_exp2f(st.m - m_new) : 1.f;
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[db][i] *= alpha;
}

// O^T += V^T P^T with the V^T fragments of the tile in registers (vf[cc * DB + db]:
// 16-key chunk cc, d block db).
template <int D>
__device__ __forceinline__ void tile_o(const bf16x8 *pb, const bf16x8 *vf, RowState<D> &st) {
    constexpr int DB = D / 32;
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[cc * DB + db], pb[cc], st.o[db], 0, 0, 0);
}

// Softmax of a scored (and, where needed, masked) tile and its P.V product.
template <int D>
__device__ __forceinline__ void tile_pv(const f32x16 &s, const bf16x8 *vf, float c, RowState<D> &st) {
    bf16x8 pb[2];
    float lt = tile_p(s, c, -st.m, pb);
    const bool need = !(lt <= kGuardSum);
    if (__any(need)) {   // wave-uniform branch; the move itself is per row
        move_max<D>(s, c, need, st);
        lt = tile_p(s, c, -st.m, pb);
    }
    st.l += lt;
    __builtin_amdgcn_s_setprio(3);   // dropped again once the scores of the next tile are issued
    tile_o<D>(pb, vf, st);
}

// Causal / question-end select on a 32-key tile that crosses the diagonal or the end.
template <int D>
__device__ __forceinline__ void mask_tile(f32x16 &s, int k0, int qrow, int L) {
    const int half = (threadIdx.x & 63) >> 5;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int key = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
        if (key > qrow || key >= L) s[i] = -INFINITY;
    }
}

// The work item of this workgroup: record {question start a, length L, query block t,
// question index sq}, its KV head and its place w among the item's workgroups of that head.
// The record and the item count are read together (one round trip); records past the count
// exist (the record array covers the whole grid) and are not used (valid = false).
struct ItemRef {
    int a, L, t, sq, kvh, w;
    bool valid;
};

__device__ __forceinline__ ItemRef prefill_item(const PrefillArgs &p) {
    int item, kvh, w;
    if (p.n_streams > 1) {
        // XCD-aware: this workgroup runs on XCD x and serves one (stream, KV head) pair there,
        // so the XCD's L2 holds that pair's K/V rows only (see PrefillArgs)
        const int x = blockIdx.x % p.n_xcd, kk = blockIdx.x / p.n_xcd;
        kvh = x % p.kv_heads;
        const int idx = kk / p.wg_per_kvh;
        w = kk - idx * p.wg_per_kvh;
        item = (x / p.kv_heads) * p.stream_cap + idx;
    } else {
        const int per_item = p.kv_heads * p.wg_per_kvh;
        item = blockIdx.x / per_item;
        const int rem = blockIdx.x - item * per_item;
        kvh = rem % p.kv_heads;   // KV head fastest: see Placement
        w = rem / p.kv_heads;
    }
    const __attribute__((address_space(4))) int *recs = (const __attribute__((address_space(4))) int *)p.rec;
    ItemRef r;
    r.a = recs[4 * item];
    r.L = recs[4 * item + 1];
    r.t = recs[4 * item + 2];
    r.sq = recs[4 * item + 3];
    r.kvh = kvh;
    r.w = w;
    const int32_t n_items = ((const __attribute__((address_space(4))) int *)p.sched)[0];
    r.valid = p.n_streams > 1 ? (n_items != 0 && r.L >= 0) : item < n_items;
    return r;
}

// Chunked prefill: the question continues P rows cached in its slot; pk / pv are that slot's
// K and V planes of KV head it.kvh.  Returns false, and the first workgroup of the question
// flags the error, when the slot id or P is out of range (the question's rows are then not
// written).
template <int D>
__device__ __forceinline__ bool slot_prefix(const PrefillArgs &p, const ItemRef &it, int &P, const uint16_t *&pk,
                                            const uint16_t *&pv) {
    const int slot = p.slot_ids[it.sq];
    P = p.prefix_lens[it.sq];
    const bool bad_slot = slot < 0 || slot >= p.n_slots;
    if (bad_slot || P < 0 || P > p.capacity - it.L) {
        if (threadIdx.x == 0 && it.t == 0 && it.w == 0 && it.kvh == 0)
            atomicOr(p.err, (int32_t)(bad_slot ? KEV_DEVERR_SLOT : KEV_DEVERR_CACHE_LEN));
        return false;
    }
    const int64_t plane = (int64_t)p.capacity * D;
    pk = static_cast<const uint16_t *>(p.pool) + ((int64_t)slot * 2 * p.kv_heads + it.kvh) * plane;
    pv = pk + (int64_t)p.kv_heads * plane;
    return true;
}

// Runs iteration(j, std::integral_constant<int, j % NS>) for j = 0 .. n_tiles-1, unrolled by
// the stage count so that every stage index is a compile-time constant.
template <int NS, typename F>
__device__ __forceinline__ void tile_loop(int n_tiles, F &&iteration) {
    for (int j0 = 0; j0 < n_tiles; j0 += NS) {
        iteration(j0, std::integral_constant<int, 0>{});
        if (j0 + 1 >= n_tiles) break;
        iteration(j0 + 1, std::integral_constant<int, 1 % NS>{});
        if (j0 + 2 >= n_tiles) break;
        iteration(j0 + 2, std::integral_constant<int, 2 % NS>{});
        if (j0 + 3 >= n_tiles) break;
        iteration(j0 + 3, std::integral_constant<int, 3 % NS>{});
        if (NS > 4) {
            if (j0 + 4 >= n_tiles) break;
            iteration(j0 + 4, std::integral_constant<int, 4 % NS>{});
        }
    }
}

template <int D, bool PREFIX>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_bf16_kernel(PrefillArgs p) {
    constexpr int NS = NS32;
    using C = Cfg<D, NS>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_t *)smem;
    // K stages at [0, NS*TB), V stages after them.
    auto kst = [&](int s) { return (lds_t *)smem + s * C::TB; };
    auto vst = [&](int s) { return (lds_t *)smem + (NS + s) * C::TB; };

    const ItemRef it = prefill_item(p);
    if (!it.valid) return;   // past the work list
    const int a = it.a, L = it.L, t = it.t, kvh = it.kvh, w = it.w;
    const int G = p.group;

    const int item_row0 = t * p.block_rows;
    const int wg_row_lo = item_row0 + ((NWAVE * w) / G) * 32;
    if (wg_row_lo >= L) return;   // every wavefront of this workgroup is past the question

    // Keys are indexed in the question: P cached rows (chunked prefill), then the L rows here.
    int P = 0;
    const uint16_t *pk = nullptr, *pv = nullptr;
    if constexpr (PREFIX)
        if (!slot_prefix<D>(p, it, P, pk, pv)) return;
    const int wg_key_end = P + min(item_row0 + ((NWAVE * w + NWAVE - 1) / G + 1) * 32, L);
    const int n_tiles = (wg_key_end + KT - 1) / KT;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
    const int lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int u = NWAVE * w + wave;
    const int rb = u / G;
    const int head = kvh * G + (u - rb * G);
    const int row0 = item_row0 + rb * 32;                       // question-relative
    const int wave_key_end = row0 < L ? P + min(row0 + 32, L) : 0;
    const int my_tiles = (wave_key_end + KT - 1) / KT;
    const int n_full = (P + min(row0 + 1, L)) / KT;             // tiles needing no mask

    const int64_t kv_stride = (int64_t)p.kv_heads * D;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)a * p.kv_heads + kvh) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + ((int64_t)a * p.kv_heads + kvh) * D;

    const int qrow = row0 + col;

    RowState<D> st;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) st.o[db][i] = 0.f;
    st.m = -INFINITY;
    st.l = 0.f;
    float c = p.scale_log2;   // in a register before the loop (see Pipeline)
    asm volatile("" : "+s"(c));

    TileLoader<D, NWAVE, PREFIX> ld;
    ld.init(kg, vg, kv_stride, wg_key_end, wave, pk, pv, P);
    auto kaddr = [&](int s) { return lds0 + (unsigned)(s * C::TB); };
    auto vaddr = [&](int s) { return lds0 + (unsigned)((NS + s) * C::TB); };

    // Q^T operand: lane holds q row (row0 + col), d = dc*16 + half*8 .. +8; rows past the
    // question read its last row (finite values in columns that are never stored).  Loaded
    // with inline asm before the K/V prologue, so the one counted wait for K(0) below also
    // covers these loads and no compiler wait drains the prologue.
    bf16x8 qf[C::DC];
    {
        const uint16_t *qp = static_cast<const uint16_t *>(p.q) +
                             ((int64_t)(a + min(qrow, L - 1)) * p.heads + head) * D + half * 8;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
        {
            if (PREFIX)   // non-temporal: the rows are read once and should not displace K/V in L2
                asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(qf[dc]) : "v"(qp + dc * 16) : "memory");
            else
                asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(qf[dc]) : "v"(qp + dc * 16) : "memory");
        }
    }

    // Issue order: K(0); then, per (virtual) iteration i, K(i+NS) and V(i+NS-1).  At the
    // barrier of iteration j the wave needs K(j+1) and V(j), both issued at iteration
    // j-NS+1 with V last; the loads of at most NS-2 later iterations may stay in flight.
    ld.issue(ld.kbase, ld.pkbase, 0, kaddr(0), wave);
    for (int i = 1 - NS; i < 0; ++i) {
        if (i + NS < n_tiles) ld.issue(ld.kbase, ld.pkbase, i + NS, kaddr(i + NS), wave);
        if (i + NS - 1 < n_tiles) ld.issue(ld.vbase, ld.pvbase, i + NS - 1, vaddr(i + NS - 1), wave);
    }
    if (n_tiles >= NS) wait_vmcnt<2 * C::NIT * (NS - 1)>();   // q and K(0) have landed
    else wait_vmcnt<0>();
    asm volatile("" : "+v"(qf[0]), "+v"(qf[1]), "+v"(qf[2]), "+v"(qf[3]));
    if (C::DC > 4) asm volatile("" : "+v"(qf[4 % C::DC]), "+v"(qf[5 % C::DC]), "+v"(qf[6 % C::DC]), "+v"(qf[7 % C::DC]));
    barrier();

    bf16x8 kf[C::DC];             // K fragments of the next tile to score
    bf16x8 vf[2 * C::DB];         // V^T fragments of the current tile
    f32x16 s;                     // scores of the current tile
    auto score = [&]() {
        f32x16 acc;
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc)
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[dc], qf[dc], acc, 0, 0, 0);
        return acc;
    };
    if (my_tiles > 0) {
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) kf[dc] = k_frag<D>(kst(0), dc);
        s = score();
    }

    // Iteration j: the scores of tile j are in flight on MFMA.  After the barrier the wave
    // reads all fragments of V(j) and K(j+1) at once, takes the softmax of tile j while
    // those reads land, runs P.V of tile j and issues the scores of tile j+1, which then
    // execute while the wave waits at the next barrier.
    // The loop is unrolled by NS so every stage address is a compile-time offset.
    auto iteration = [&](const int j, auto U) {
        constexpr int u = decltype(U)::value;   // j % NS
        if (j + NS - 1 < n_tiles) wait_vmcnt<2 * C::NIT * (NS - 2)>();
        else wait_vmcnt<0>();
        barrier();
        if (j + NS < n_tiles) ld.issue(ld.kbase, ld.pkbase, j + NS, kaddr(u), wave);
        if (j + NS - 1 < n_tiles) ld.issue(ld.vbase, ld.pvbase, j + NS - 1, vaddr((u + NS - 1) % NS), wave);
        if (j < my_tiles) {
            const lds_t *kn = kst((u + 1) % NS);   // past the last tile: an unused read
            const lds_t *vc = vst(u);
            // V(j) first: LDS reads return in order, and P.V of tile j needs them before the
            // scores of tile j+1 need K(j+1).
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
                for (int db = 0; db < C::DB; ++db) vf[cc * C::DB + db] = vt_frag<D>(vc, cc, db);
#pragma unroll
            for (int dc = 0; dc < C::DC; ++dc) kf[dc] = k_frag<D>(kn, dc);
            if (j >= n_full) mask_tile<D>(s, j * KT, P + qrow, P + L);
            tile_pv<D>(s, vf, c, st);
            if (j + 1 < my_tiles) s = score();
            __builtin_amdgcn_s_setprio(0);
        }
    };
    tile_loop<NS>(n_tiles, iteration);

    wait_vmcnt<0>();   // no direct load may outlive the workgroup's LDS

    // ---- epilogue: divide by the row sum, round to bf16, store rows inside the question ----
    // A lane holds 4-element pieces of one row, so direct stores would touch 32 rows per
    // instruction.  Each wavefront instead writes its 32 x D block to a free LDS stage (in
    // the swizzled row layout) and stores whole rows from there: D/8 lanes per row, 16 B
    // each.  Free stages: after the last barrier the other wavefronts read only K stage
    // n_tiles % NS and V stage (n_tiles - 1) % NS, and no direct load is in flight, so
    // wavefronts 0..2 take the next three K stages after it and wavefront 3 takes V stage
    // n_tiles % NS.  LDS operations of one wavefront complete in order, so the reads see
    // the writes without a barrier.
    const float l_tot = sum_halves(st.l);
    if (row0 >= L) return;
    const float inv = 1.f / l_tot;
    using GM = Geom<D>;
    lds_t *ob = wave < 3 ? kst((n_tiles + 1 + wave) % NS) : vst(n_tiles % NS);
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) f[jj] = st.o[db][g4 * 4 + jj] * inv;
            // row col, d = db*32 + g4*8 + half*4 .. +4: the half-chunk `half` of chunk db*4+g4
            *reinterpret_cast<__attribute__((address_space(3))) bf16x4 *>(ob + GM::off(col, db * 4 + g4) + half * 8) =
                __builtin_convertvector(f, bf16x4);
        }
    const int rr = lane / GM::CPR, cc = lane % GM::CPR;
    uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)(a + row0) * p.heads + head) * D + cc * 8;
    const int64_t rstride = (int64_t)p.heads * D;
#pragma unroll
    for (int k = 0; k < 32 / GM::RPI; ++k) {
        const int r = k * GM::RPI + rr;
        const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(ob + GM::off(r, cc));
        if (row0 + r < L) {
            if (PREFIX) __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(orow + r * rstride));
            else *reinterpret_cast<u32x4 *>(orow + r * rstride) = x;
        }
    }
}


// ---- head_dim 128: 48 query rows per wavefront on v_mfma_f32_16x16x32_bf16 ----
//
// Lane (m = lane % 16, g = lane / 16).  The wavefront's rows form three 16-row blocks rb; the
// lane owns query row rb*16 + m of each.  Key block kb (16 keys) of a 32-key tile.
//   S^T block (kb, rb):  acc[i] = S^T[kb*16 + 4g + i][rb*16 + m]     A = K from LDS, B = Q^T
//   O^T block (db, rb):  acc[i] = O^T[db*16 + 4g + i][rb*16 + m]     A = V^T from LDS, B = P^T
// The P^T operand of row block rb takes the lane's 8 weights in the order (kb, i), so its
// k-slot 8g + 4kb + i is key kb*16 + 4g + i; the V^T operand lists the keys in that same
// order.  A row's 32 weights of a tile sit in the four lanes m, m+16, m+32, m+48.

// Tiles of this kernel use their own swizzle (Geom<128, 1>), under which the K reads and
// the transposed V^T reads below are free of bank conflicts.
//
// K fragment (kb, s): row kb*16 + m, 16-byte chunk 4s + g (d = 32s + 8g .. +8).  Its byte
// offset in a stage is (m*256 + ((g ^ swz(m)) << 4)) ^ (s << 6), plus kb*4096 (the swizzle
// depends on the row only through its low four bits), so one lane base serves all eight.
__device__ __forceinline__ unsigned k16_lane() {
    using G = Geom<128, 1>;
    const int lane = threadIdx.x & 63, m = lane & 15, g = lane >> 4;
    return (unsigned)(m * 256 + ((g ^ G::swz(m)) << 4));
}
__device__ __forceinline__ bf16x8 k16_frag(const lds_t *stage, unsigned kl, int kb, int s) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(
                                          stage + kb * 4096 + (kl ^ (unsigned)(s << 6))));
}

// V^T fragment of d block db: two transposed reads (keys 4g + (n>>2) and 16 + 4g + (n>>2)
// of 16-lane group g, four d values from chunk 2db + ((n>>1)&1), half n&1), which leave
// V[key][db*16 + n] for the lane's eight keys in the P^T order.  Byte offset
// (r0*256 + ((((n>>1)&1) ^ swz(r0)) << 4) + (n&1)*8) ^ (db << 5), plus 4096 for the
// second read (rows 16 apart share the swizzle).
__device__ __forceinline__ unsigned vt16_lane() {
    using G = Geom<128, 1>;
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    const int r0 = 4 * g + (n >> 2);
    return (unsigned)(r0 * 256 + ((((n >> 1) & 1) ^ G::swz(r0)) << 4) + (n & 1) * 8);
}
__device__ __forceinline__ bf16x8 vt16_frag(const lds_t *stage, unsigned vl, int db) {
    const lds_t *a = stage + (vl ^ (unsigned)(db << 5));
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a);
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a + 4096));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// max / sum over the four lanes of a row
__device__ __forceinline__ float row_max4(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    return fmaxf(x, __shfl_xor(x, 32));
}
__device__ __forceinline__ float row_sum4(float x) {
    x += __shfl_xor(x, 16);
    return x + __shfl_xor(x, 32);
}

// P = exp2(S*c - m) in bf16 for row block rb and the lane's sum of those 8 weights (from the
// bf16 values, as in tile_p).
__device__ __forceinline__ float tile_p16(const f32x4 &s0, const f32x4 &s1, float c, float mneg, bf16x8 &pb) {
    const unsigned one2 = 0x3F803F80u;
    f32x8 e;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        e[i] = __builtin_amdgcn_exp2f(fmaf(s0[i], c, mneg));
        e[4 + i] = __builtin_amdgcn_exp2f(fmaf(s1[i], c, mneg));
    }
    pb = __builtin_convertvector(e, bf16x8);
    const u32x4 w = __builtin_bit_cast(u32x4, pb);
    float acc = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) asm("v_dot2_f32_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(w[i]), "v"(one2));
    return acc;
}

template <bool PREFIX>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_r48_kernel(PrefillArgs p) {
    constexpr int D = 128, WR = 48;
    constexpr int NS = NS48;
    using C = Cfg<D, NS>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS];
    const unsigned lds0 = (unsigned)(uintptr_t)(lds_t *)smem;
    auto kst = [&](int s) { return (lds_t *)smem + s * C::TB; };
    auto vst = [&](int s) { return (lds_t *)smem + (NS + s) * C::TB; };

    const ItemRef it = prefill_item(p);
    if (!it.valid) return;
    const int a = it.a, L = it.L, t = it.t, kvh = it.kvh, w = it.w;
    const int G = p.group;

    const int item_row0 = t * p.block_rows;
    const int wg_row_lo = item_row0 + ((NWAVE * w) / G) * WR;
    if (wg_row_lo >= L) return;

    int P = 0;
    const uint16_t *pk = nullptr, *pv = nullptr;
    if constexpr (PREFIX)
        if (!slot_prefix<D>(p, it, P, pk, pv)) return;
    const int wg_key_end = P + min(item_row0 + ((NWAVE * w + NWAVE - 1) / G + 1) * WR, L);
    const int n_tiles = (wg_key_end + KT - 1) / KT;

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, m16 = lane & 15, g4 = lane >> 4;
    const int u = NWAVE * w + wave;
    const int rbu = u / G;
    const int head = kvh * G + (u - rbu * G);
    const int row0 = item_row0 + rbu * WR;
    const int wave_key_end = row0 < L ? P + min(row0 + WR, L) : 0;
    const int my_tiles = (wave_key_end + KT - 1) / KT;
    const int n_full = (P + min(row0 + 1, L)) / KT;

    const int64_t kv_stride = (int64_t)p.kv_heads * D;
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)a * p.kv_heads + kvh) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + ((int64_t)a * p.kv_heads + kvh) * D;

    f32x4 o[8][3];
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int rb = 0; rb < 3; ++rb) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
    float mrow[3], lrow[3];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) {
        mrow[rb] = -INFINITY;
        lrow[rb] = 0.f;
    }
    float c = p.scale_log2;
    asm volatile("" : "+s"(c));

    TileLoader<D, NWAVE, PREFIX, 1> ld;
    ld.init(kg, vg, kv_stride, wg_key_end, wave, pk, pv, P);
    auto kaddr = [&](int s) { return lds0 + (unsigned)(s * C::TB); };
    auto vaddr = [&](int s) { return lds0 + (unsigned)((NS + s) * C::TB); };

    // Q^T operands: qf[rb][s] holds q row row0 + rb*16 + m, d = 32s + 8g .. +8 (rows past the
    // question read its last row)
    bf16x8 qf[3][4];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) {
        const int qr = min(row0 + rb * 16 + m16, L - 1);
        const uint16_t *qp = static_cast<const uint16_t *>(p.q) + ((int64_t)(a + qr) * p.heads + head) * D + g4 * 8;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (PREFIX)
                asm volatile("global_load_dwordx4 %0, %1, off nt" : "=v"(qf[rb][s]) : "v"(qp + s * 32) : "memory");
            else
                asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(qf[rb][s]) : "v"(qp + s * 32) : "memory");
        }
    }
    ld.issue(ld.kbase, ld.pkbase, 0, kaddr(0), wave);
    for (int i = 1 - NS; i < 0; ++i) {
        if (i + NS < n_tiles) ld.issue(ld.kbase, ld.pkbase, i + NS, kaddr(i + NS), wave);
        if (i + NS - 1 < n_tiles) ld.issue(ld.vbase, ld.pvbase, i + NS - 1, vaddr(i + NS - 1), wave);
    }
    if (n_tiles >= NS) wait_vmcnt<2 * C::NIT * (NS - 1)>();
    else wait_vmcnt<0>();
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) asm volatile("" : "+v"(qf[rb][0]), "+v"(qf[rb][1]), "+v"(qf[rb][2]), "+v"(qf[rb][3]));
    barrier();

    bf16x8 kf[2][4];
    bf16x8 vf[8];
    f32x4 sacc[2][3];
    auto score = [&]() {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int rb = 0; rb < 3; ++rb) sacc[kb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int rb = 0; rb < 3; ++rb)
                    sacc[kb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kb][s], qf[rb][s], sacc[kb][rb], 0, 0, 0);
    };
    if (my_tiles > 0) {
        const unsigned kl = k16_lane();
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int s = 0; s < 4; ++s) kf[kb][s] = k16_frag(kst(0), kl, kb, s);
        score();
    }

    auto iteration = [&](const int j, auto U) {
        constexpr int uu = decltype(U)::value;   // j % NS
        // both loads of this tile go to tiles before the last one of the workgroup's range (and,
        // with a slot prefix, past the prefix): no bound checks
        if (j + NS + 1 < n_tiles && (!PREFIX || (j + NS - 1) * KT >= P)) {
            wait_vmcnt<2 * C::NIT * (NS - 2)>();
            barrier();
            ld.issue_inner(ld.kbase, j + NS, kaddr(uu));
            ld.issue_inner(ld.vbase, j + NS - 1, vaddr((uu + NS - 1) % NS));
        } else {
            if (j + NS - 1 < n_tiles) wait_vmcnt<2 * C::NIT * (NS - 2)>();
            else wait_vmcnt<0>();
            barrier();
            if (j + NS < n_tiles) ld.issue(ld.kbase, ld.pkbase, j + NS, kaddr(uu), wave);
            if (j + NS - 1 < n_tiles) ld.issue(ld.vbase, ld.pvbase, j + NS - 1, vaddr((uu + NS - 1) % NS), wave);
        }
        if (j < my_tiles) {
            // lane bases and the mask's lane terms are rebuilt in every tile (one instruction
            // each) rather than kept live across the loop
            unsigned kl = k16_lane(), vl = vt16_lane();
            int ldiff = P + row0 + m16 - 4 * g4, g4x4 = 4 * g4;
            asm volatile("" : "+v"(kl), "+v"(vl), "+v"(ldiff), "+v"(g4x4));
            if (j >= n_full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int rb = 0; rb < 3; ++rb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            // key j*32 + kb*16 + 4g + i against position P + row0 + rb*16 + m
                            const int kk = j * KT + kb * 16 + i;
                            if (kk - rb * 16 > ldiff || kk + g4x4 >= P + L) sacc[kb][rb][i] = -INFINITY;
                        }
            }
            bf16x8 pb[3];
            float lt[3];
            bool need = false;
#pragma unroll
            for (int rb = 0; rb < 3; ++rb) {
                lt[rb] = tile_p16(sacc[0][rb], sacc[1][rb], c, -mrow[rb], pb[rb]);
                need |= !(lt[rb] <= kGuardSum);
            }
            if (__any(need)) {
                // move the max of every row where one of its four lanes left the bound
#pragma unroll
                for (int rb = 0; rb < 3; ++rb) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[kb][rb][i]);
                    mx = row_max4(mx) * c;
                    if (row_max4(!(lt[rb] <= kGuardSum) ? 1.f : 0.f) > 0.f) {
                        const float m_new = fmaxf(mrow[rb], mx);
                        const float alpha = __builtin_amdgcn_exp2f(mrow[rb] - m_new);
                        mrow[rb] = m_new;
                        lrow[rb] *= alpha;
#pragma unroll
                        for (int db = 0; db < 8; ++db) o[db][rb] *= alpha;
                        lt[rb] = tile_p16(sacc[0][rb], sacc[1][rb], c, -mrow[rb], pb[rb]);
                    }
                }
            }
#pragma unroll
            for (int rb = 0; rb < 3; ++rb) lrow[rb] += lt[rb];
            const lds_t *vc = vst(uu);
#pragma unroll
            for (int db = 0; db < 8; ++db) vf[db] = vt16_frag(vc, vl, db);
#pragma unroll
            for (int db = 0; db < 8; ++db)
#pragma unroll
                for (int rb = 0; rb < 3; ++rb)
                    o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[db], pb[rb], o[db][rb], 0, 0, 0);
            if (j + 1 < my_tiles) {
                const lds_t *kn = kst((uu + 1) % NS);
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int s = 0; s < 4; ++s) kf[kb][s] = k16_frag(kn, kl, kb, s);
                score();
            }
        }
    };
    tile_loop<NS>(n_tiles, iteration);
    wait_vmcnt<0>();

    // Epilogue: each 16-row block goes through a free stage (the same stages as the 32-row
    // kernel takes: no wavefront reads K stages after the last barrier, nor V stage n_tiles % NS).
    float inv[3];
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) inv[rb] = 1.f / row_sum4(lrow[rb]);
    if (row0 >= L) return;
    using GM = Geom<D, 1>;
    lds_t *ob = wave < 3 ? kst((n_tiles + 1 + wave) % NS) : vst(n_tiles % NS);
    const int rr = lane / GM::CPR, cc = lane % GM::CPR;
    const int64_t rstride = (int64_t)p.heads * D;
#pragma unroll
    for (int rb = 0; rb < 3; ++rb) {
        if (row0 + rb * 16 >= L) break;
#pragma unroll
        for (int db = 0; db < 8; ++db) {
            // row m, d = db*16 + 4g .. +4: half g & 1 of chunk 2db + (g >> 1)
            const int dofs = db * 16 + 4 * g4;
            *reinterpret_cast<__attribute__((address_space(3))) bf16x4 *>(ob + GM::off(m16, dofs >> 3) + (dofs & 7) * 2) =
                __builtin_convertvector(o[db][rb] * inv[rb], bf16x4);
        }
        uint16_t *orow = static_cast<uint16_t *>(p.out) + ((int64_t)(a + row0 + rb * 16) * p.heads + head) * D + cc * 8;
#pragma unroll
        for (int k = 0; k < 16 / GM::RPI; ++k) {
            const int r = k * GM::RPI + rr;
            const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4 *>(ob + GM::off(r, cc));
            if (row0 + rb * 16 + r < L) {
                if (PREFIX) __builtin_nontemporal_store(x, reinterpret_cast<u32x4 *>(orow + r * rstride));
                else *reinterpret_cast<u32x4 *>(orow + r * rstride) = x;
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int32_t head_dim, int64_t grid, bool prefix,
                               hipStream_t s) {
    const dim3 g((unsigned)grid), b(NWAVE * 64);
    switch (head_dim * 2 + (prefix ? 1 : 0)) {
    case 128: hipLaunchKernelGGL((prefill_bf16_kernel<64, false>), g, b, 0, s, a); break;
    case 129: hipLaunchKernelGGL((prefill_bf16_kernel<64, true>), g, b, 0, s, a); break;
    case 256: hipLaunchKernelGGL(prefill_r48_kernel<false>, g, b, 0, s, a); break;
    case 257: hipLaunchKernelGGL(prefill_r48_kernel<true>, g, b, 0, s, a); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace kev
