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
// Work item = (question, block of 32*R query rows) from the scheduler, times a
// group of `heads_per_wg` query heads that share one KV head.  One wavefront
// owns 32 query rows of one head.  All wavefronts of a workgroup read the same
// K/V tiles (64 keys) from LDS, so each tile load serves heads_per_wg * R
// wavefronts.  Only key tiles inside the item's own question and at or left of
// its diagonal are loaded; inside a tile, 32-key sub-blocks that lie entirely
// above a wavefront's rows are skipped and the causal select (-inf, not a
// multiply) is applied only to sub-blocks that cross the diagonal or the end
// of the question.
//
// MFMA orientation (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T[key][q] = K_tile[key][:] . Q^T[:][q]     A = K from LDS, B = Q in VGPRs
//   O^T[d][q]  += V^T[d][key]   . P^T[key][q]    A = V^T from LDS, B = P^T in VGPRs
// With the query index on the lane (n = lane % 32), each lane owns one query
// row: row max and row sum need one exchange between the two half-waves, the
// rescale of O^T is lane-uniform, and P^T feeds the second MFMA straight from
// the first one's accumulators (converted to bf16).  Staging and operand reads
// are described in kev_mfma_core.h.
//
// Pipeline: three LDS stages per tensor.  At tile t every wavefront waits for
// its own direct loads of tile t, meets the others at one barrier (which also
// retires all reads of tile t-1), issues the loads of tile t+2 into the stage
// tile t-1 used, and computes tile t.  The stages are separate __shared__
// arrays so the compiler can see that reads of one stage never alias loads
// in flight to another.
#include "kev_internal.h"
#include "kev_mfma_core.h"

namespace kev {

namespace {

using namespace core;

constexpr int KT = 64;   // keys per tile

template <int D, int NW>
struct Cfg {
    static constexpr int DC = D / 16;                    // k steps of the S MFMA
    static constexpr int DB = D / 32;                    // 32-row d blocks of O^T
    static constexpr int IPT = KT / Geom<D>::RPI;        // direct loads per K (or V) tile
    static constexpr int NIT = (IPT + NW - 1) / NW;      // per wavefront per tensor (uniform)
    static constexpr int NI = 2 * NIT;                   // per wavefront per tile
    static constexpr int TB = KT * D * 2;                // bytes per tile
};

// Direct loads of one K and V tile into one stage.  Every wavefront issues exactly NIT
// loads per tensor (a few re-issue another wavefront's load when NW does not divide the
// count; same data, same place), so one vmcnt value fits all.  Rows past key_end are
// clamped to key_end-1: a valid row of the same question, so nothing outside the question
// is read and staged values stay finite wherever the question's own values are.
template <int D, int NW>
struct TileLoader {
    using C = Cfg<D, NW>;
    DmaLane<D> ln[C::NIT];
    int r0[C::NIT];
    int64_t stride;
    const uint16_t *kg, *vg;

    __device__ void init(const uint16_t *k, const uint16_t *v, int64_t row_stride) {
        const int wave = threadIdx.x >> 6;
        kg = k;
        vg = v;
        stride = row_stride;
#pragma unroll
        for (int i = 0; i < C::NIT; ++i) {
            r0[i] = ((wave + NW * i) % C::IPT) * Geom<D>::RPI;
            ln[i].init(r0[i]);
        }
    }

    __device__ __forceinline__ void issue(int tile, int key_end, lds_t *ks, lds_t *vs) const {
        const int k0 = tile * KT;
        const bool full = k0 + KT <= key_end;
#pragma unroll
        for (int i = 0; i < C::NIT; ++i) {
            const int key = full ? k0 + ln[i].row : min(k0 + ln[i].row, key_end - 1);
            const int64_t off = (int64_t)key * stride + ln[i].coff;
            dma16(kg + off, ks + r0[i] * Geom<D>::ROWB);
            dma16(vg + off, vs + r0[i] * Geom<D>::ROWB);
        }
    }
};

// One wavefront's work on a staged tile: 32 query rows (row0 ..) against keys k0 .. k0+63.
// `edge` marks the tile that crosses this wavefront's diagonal or the question's end; only
// there are scores masked (a select to -inf).
template <int D>
__device__ __forceinline__ void compute_tile(const lds_t *ks, const lds_t *vs, int k0, bool edge,
                                             int qrow, int L, float c, const bf16x8 *qf,
                                             f32x16 *o, float &m_run, float &l_run) {
    constexpr int DB = D / 32;
    const int half = (threadIdx.x & 63) >> 5;
    f32x16 s[2];
    scores2<D>(ks, qf, s[0], s[1]);
    if (edge) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + kb * 32 + (i >> 2) * 8 + half * 4 + (i & 3);
                if (key > qrow || key >= L) s[kb][i] = -INFINITY;
            }
    }
    float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
    for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[0][i]), s[0][i + 1]);
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[1][i]), s[1][i + 1]);
    mx = max_halves(mx) * c;

    // lazy rescale: move the running max only when some row grew by more than kLazy
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
    bf16x8 pb[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h8 = 0; h8 < 2; ++h8) {
            f32x8 e;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                e[i] = __builtin_amdgcn_exp2f(fmaf(s[kb][h8 * 8 + i], c, mneg));
                l_run += e[i];
            }
            pb[kb * 2 + h8] = __builtin_convertvector(e, bf16x8);
        }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
        for (int db = 0; db < DB; ++db)
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_frag<D>(vs, cc, db), pb[cc], o[db], 0, 0, 0);
}

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs p) {
    using C = Cfg<D, NW>;
    __shared__ __attribute__((aligned(1024))) char sk0[C::TB], sk1[C::TB], sk2[C::TB];
    __shared__ __attribute__((aligned(1024))) char sv0[C::TB], sv1[C::TB], sv2[C::TB];
    lds_t *K0 = (lds_t *)sk0, *K1 = (lds_t *)sk1, *K2 = (lds_t *)sk2;
    lds_t *V0 = (lds_t *)sv0, *V1 = (lds_t *)sv1, *V2 = (lds_t *)sv2;

    const int32_t n_items = p.sched[0];
    const int item = blockIdx.x / p.n_hgroups;
    if (item >= n_items) return;
    const int hg = blockIdx.x % p.n_hgroups;
    const int32_t *it = p.sched + p.items_off + 2 * item;
    const int seg = it[0], t = it[1];
    const int a = p.cu[seg], L = p.cu[seg + 1] - a;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;
    const int hw = wave % p.heads_per_wg, rb = wave / p.heads_per_wg;
    const int head = hg * p.heads_per_wg + hw;
    const int kvh = (hg * p.heads_per_wg) / p.group;

    const int row0 = t * p.block_rows + rb * 32;                 // question-relative
    const int item_key_end = min((t + 1) * p.block_rows, L);
    const int wave_key_end = row0 < L ? min(row0 + 32, L) : 0;  // keys this wavefront needs
    const int n_tiles = (item_key_end + KT - 1) / KT;

    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)a * p.kv_heads + kvh) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + ((int64_t)a * p.kv_heads + kvh) * D;
    const int64_t kv_stride = (int64_t)p.kv_heads * D;

    // Q^T operand: lane holds q row (row0 + col), d = dc*16 + half*8 .. +8.
    const int qrow = row0 + col;
    bf16x8 qf[C::DC];
    {
        const uint16_t *qp = static_cast<const uint16_t *>(p.q) +
                             ((int64_t)(a + qrow) * p.heads + head) * D + half * 8;
#pragma unroll
        for (int dc = 0; dc < C::DC; ++dc) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qrow < L) u = *reinterpret_cast<const uint4 *>(qp + dc * 16);
            qf[dc] = __builtin_bit_cast(bf16x8, u);
        }
    }

    wait_vmcnt<0>();   // q is in registers before any direct load is in flight

    f32x16 o[C::DB];
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float c = p.scale_log2;

    TileLoader<D, NW> ld;
    ld.init(kg, vg, kv_stride);
    ld.issue(0, item_key_end, K0, V0);
    if (n_tiles > 1) ld.issue(1, item_key_end, K1, V1);

#define KEV_STEP(T, KC, VC, KN, VN)                                                           \
    {                                                                                          \
        if ((T) + 1 < n_tiles) wait_vmcnt<C::NI>();                                            \
        else wait_vmcnt<0>();                                                                  \
        barrier();                                                                             \
        if ((T) + 2 < n_tiles) ld.issue((T) + 2, item_key_end, KN, VN);                       \
        if ((T) * KT < wave_key_end)                                                           \
            compute_tile<D>(KC, VC, (T) * KT, (T) * KT + KT - 1 > row0 || (T) * KT + KT > L,     \
                            qrow, L, c, qf, o, m_run, l_run);                                  \
    }
    for (int kt = 0; kt < n_tiles; kt += 3) {
        KEV_STEP(kt, K0, V0, K2, V2)
        if (kt + 1 >= n_tiles) break;
        KEV_STEP(kt + 1, K1, V1, K0, V0)
        if (kt + 2 >= n_tiles) break;
        KEV_STEP(kt + 2, K2, V2, K1, V1)
    }
#undef KEV_STEP

    wait_vmcnt<0>();   // no direct load may outlive the workgroup's LDS

    // ---- epilogue: divide by the row sum, round to bf16, store rows inside the question ----
    const float l_tot = sum_halves(l_run);
    if (qrow >= L || row0 >= L) return;
    const float inv = 1.f / l_tot;
    uint16_t *op = static_cast<uint16_t *>(p.out) + ((int64_t)(a + qrow) * p.heads + head) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            f32x4 f;
#pragma unroll
            for (int j = 0; j < 4; ++j) f[j] = o[db][g4 * 4 + j] * inv;
            *reinterpret_cast<bf16x4 *>(op + db * 32 + g4 * 8 + half * 4) = __builtin_convertvector(f, bf16x4);
        }
}

template <int D, int NW>
hipError_t launch_nw(const PrefillArgs &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, NW>), dim3((unsigned)grid), dim3(NW * 64), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs &a, int32_t waves, int64_t grid, hipStream_t s) {
    switch (waves) {
    case 1: return launch_nw<D, 1>(a, grid, s);
    case 2: return launch_nw<D, 2>(a, grid, s);
    case 3: return launch_nw<D, 3>(a, grid, s);
    case 4: return launch_nw<D, 4>(a, grid, s);
    case 5: return launch_nw<D, 5>(a, grid, s);
    case 6: return launch_nw<D, 6>(a, grid, s);
    case 7: return launch_nw<D, 7>(a, grid, s);
    case 8: return launch_nw<D, 8>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs &a, int32_t head_dim, int32_t waves,
                               int64_t grid, hipStream_t s) {
    switch (head_dim) {
    case 64: return launch_d<64>(a, waves, grid, s);
    case 128: return launch_d<128>(a, waves, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kev
