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
// Decode reads every cached K/V byte once; the arithmetic per byte is tiny, so
// the kernel is shaped for HBM bandwidth and keeps the vector ALUs nearly idle:
//   - a unit is (request, KV head); its positions are cut into chunks of
//     kDecodeChunk positions, one single-wavefront workgroup per chunk, so long
//     and short slots spread evenly over the CUs and several workgroups share
//     a CU;
//   - the `group` query heads of the KV head are the columns of MFMA tiles
//     (v_mfma_f32_32x32x16_bf16: S^T = K Q^T, O^T += V^T P^T), so the dot
//     products and the weighted sum of V cost matrix-core cycles, not VALU;
//   - K and V rows of the slot plane go straight from HBM into LDS with direct
//     loads, three 32-position stages deep, 1 KB per load instruction; the row
//     holding the new token is read from k_new / v_new instead;
//   - the softmax is online (running max / sum / rescaled accumulator, primer
//     section 2.4); a unit with one chunk writes its output directly, otherwise
//     each chunk writes (max, sum, accumulator) and a second small kernel merges
//     the chunks with the same rescaling identity.  (A last-arriving-workgroup
//     merge inside one kernel would need device-scope fences, which write back
//     and invalidate the XCD's L2 on every workgroup.)
#include "kev_internal.h"
#include "kev_mfma_core.h"
#include "../../include/kev.h"

namespace kev {

namespace {

__device__ inline uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

using namespace core;

constexpr int DKT = 32;   // positions per staged tile

// Direct loads of one 32-position K and V tile of a slot plane into one stage.  Rows past
// the chunk end are clamped to its last row; the row of the new token comes from
// k_new / v_new.
template <int D>
struct DecodeLoader {
    static constexpr int IPT = DKT / Geom<D>::RPI;   // 1 KB loads per tensor per tile
    DmaLane<D> ln[IPT];
    const uint16_t *kbase, *vbase, *knew, *vnew;
    int newpos, last;

    __device__ __forceinline__ void issue(int k0, lds_t *ks, lds_t *vs) const {
#pragma unroll
        for (int i = 0; i < IPT; ++i) {
            const int key = min(k0 + ln[i].row, last);
            const bool nw = key == newpos;
            const int64_t off = (int64_t)key * D + ln[i].coff;
            dma16(nw ? knew + ln[i].coff : kbase + off, ks + i * Geom<D>::RPI * Geom<D>::ROWB);
            dma16(nw ? vnew + ln[i].coff : vbase + off, vs + i * Geom<D>::RPI * Geom<D>::ROWB);
        }
    }
};

template <int D>
__global__ __launch_bounds__(64) void decode_bf16_kernel(DecodeArgs p) {
    constexpr int DC = D / 16, DB = D / 32;
    constexpr int TB = DKT * D * 2;
    constexpr int NI = 2 * DecodeLoader<D>::IPT;      // direct loads per tile
    __shared__ __attribute__((aligned(1024))) char sk0[TB], sk1[TB], sk2[TB];
    __shared__ __attribute__((aligned(1024))) char sv0[TB], sv1[TB], sv2[TB];
    lds_t *K0 = (lds_t *)sk0, *K1 = (lds_t *)sk1, *K2 = (lds_t *)sk2;
    lds_t *V0 = (lds_t *)sv0, *V1 = (lds_t *)sv1, *V2 = (lds_t *)sv2;

    const int G = p.group;
    const int unit = blockIdx.x / p.max_chunks;
    const int c = blockIdx.x % p.max_chunks;
    const int r = unit / p.kv_heads, g = unit % p.kv_heads;
    const int slot = p.slot_ids[r];
    const int L = p.cache_lens[r];
    const int lane = threadIdx.x;
    if (slot < 0 || slot >= p.n_slots) {
        if (c == 0 && lane == 0) atomicOr(p.err, (int32_t)KEV_DEVERR_SLOT);
        return;
    }
    if (L < 1 || L > p.capacity) {
        if (c == 0 && lane == 0) atomicOr(p.err, (int32_t)KEV_DEVERR_CACHE_LEN);
        return;
    }
    const int nchunks = (L + p.chunk - 1) / p.chunk;
    if (c >= nchunks) return;

    uint16_t *pool = static_cast<uint16_t *>(p.pool);
    const int64_t plane = (int64_t)p.capacity * D;
    uint16_t *kbase = pool + ((int64_t)slot * 2 * p.kv_heads + g) * plane;
    uint16_t *vbase = kbase + (int64_t)p.kv_heads * plane;
    const uint16_t *knew = static_cast<const uint16_t *>(p.k_new) + ((int64_t)r * p.kv_heads + g) * D;
    const uint16_t *vnew = static_cast<const uint16_t *>(p.v_new) + ((int64_t)r * p.kv_heads + g) * D;

    // In-place append of the new token (by the chunk that holds position L-1).  This chunk
    // reads that row from k_new / v_new, and no other chunk reads it, so the store needs
    // no ordering against the loads below.
    if (c == (L - 1) / p.chunk && lane < 2 * (D / 8)) {
        const int part = lane % (D / 8);
        uint16_t *dst = (lane < D / 8 ? kbase : vbase) + (int64_t)(L - 1) * D + part * 8;
        const uint16_t *src = (lane < D / 8 ? knew : vnew) + part * 8;
        *reinterpret_cast<uint4 *>(dst) = *reinterpret_cast<const uint4 *>(src);
    }

    const int p0 = c * p.chunk;
    const int p1 = min(p0 + p.chunk, L);
    const int n_tiles = (p1 - p0 + DKT - 1) / DKT;
    DecodeLoader<D> ld;
#pragma unroll
    for (int i = 0; i < DecodeLoader<D>::IPT; ++i) ld.ln[i].init(i * Geom<D>::RPI);
    ld.kbase = kbase;
    ld.vbase = vbase;
    ld.knew = knew;
    ld.vnew = vnew;
    ld.newpos = L - 1;
    ld.last = p1 - 1;

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;
    const float cs = p.scale_log2;

    ld.issue(p0, K0, V0);
    if (n_tiles > 1) ld.issue(p0 + DKT, K1, V1);

    // Query heads of this KV head are the MFMA columns: lane holds head (lane % 32).
    const int col = lane & 31, half = lane >> 5;
    bf16x8 qf[DC];
    {
        const uint16_t *qp = static_cast<const uint16_t *>(p.q) +
                             ((int64_t)r * p.heads + g * G + col) * D + half * 8;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (col < G) u = *reinterpret_cast<const uint4 *>(qp + dc * 16);
            qf[dc] = __builtin_bit_cast(bf16x8, u);
        }
    }
    wait_vmcnt<0>();   // q, and the first two tiles issued before it, have landed

    auto compute = [&](const lds_t *ks, const lds_t *vs, int k0) {
        f32x16 s = scores1<D>(ks, 0, qf);
        if (k0 + DKT > p1) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = k0 + (i >> 2) * 8 + half * 4 + (i & 3);
                if (key >= p1) s[i] = -INFINITY;
            }
        }
        float mx = fmaxf(s[0], s[1]);
#pragma unroll
        for (int i = 2; i < 16; i += 2) mx = fmaxf(fmaxf(mx, s[i]), s[i + 1]);
        mx = max_halves(mx) * cs;
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
                e[i] = __builtin_amdgcn_exp2f(fmaf(s[h8 * 8 + i], cs, mneg));
                l_run += e[i];
            }
            pb[h8] = __builtin_convertvector(e, bf16x8);
        }
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int db = 0; db < DB; ++db)
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vt_frag<D>(vs, cc, db), pb[cc], o[db], 0, 0, 0);
    };

#define KEV_DSTEP(T, KC, VC, KN, VN)                                   \
    {                                                                  \
        if ((T) + 1 < n_tiles) wait_vmcnt<NI>();                       \
        else wait_vmcnt<0>();                                          \
        asm volatile("" ::: "memory");                                 \
        if ((T) + 2 < n_tiles) ld.issue(p0 + ((T) + 2) * DKT, KN, VN); \
        compute(KC, VC, p0 + (T) * DKT);                               \
    }
    for (int t = 0; t < n_tiles; t += 3) {
        KEV_DSTEP(t, K0, V0, K2, V2)
        if (t + 1 >= n_tiles) break;
        KEV_DSTEP(t + 1, K1, V1, K0, V0)
        if (t + 2 >= n_tiles) break;
        KEV_DSTEP(t + 2, K2, V2, K1, V1)
    }
#undef KEV_DSTEP
    wait_vmcnt<0>();

    // Lanes l and l+32 hold the same head; rows d = db*32 + 8*(i/4) + 4*half + i%4.
    const float l_tot = sum_halves(l_run);
    if (col >= G) return;
    if (nchunks == 1) {
        const float inv = 1.f / l_tot;
        uint16_t *op = static_cast<uint16_t *>(p.out) + ((int64_t)r * p.heads + g * G + col) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 f;
#pragma unroll
                for (int j = 0; j < 4; ++j) f[j] = o[db][g4 * 4 + j] * inv;
                *reinterpret_cast<bf16x4 *>(op + db * 32 + g4 * 8 + half * 4) = __builtin_convertvector(f, bf16x4);
            }
    } else {
        float *pp = p.partials + (((int64_t)unit * p.max_chunks + c) * G + col) * (D + 2);
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                f32x4 f;
#pragma unroll
                for (int j = 0; j < 4; ++j) f[j] = o[db][g4 * 4 + j];
                *reinterpret_cast<f32x4 *>(pp + db * 32 + g4 * 8 + half * 4) = f;
            }
        if (half == 0) {
            pp[D] = m_run;
            pp[D + 1] = l_tot;
        }
    }
}

// Merge the chunk partials of every unit that spans more than one chunk.  One thread per
// (head, d); all chunk loads are issued before any is used (one memory latency).
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs p) {
    const int G = p.group;
    const int e = blockIdx.x * 256 + threadIdx.x;          // over units x G x D
    const int unit = e / (G * D);
    if (unit >= p.n_req * p.kv_heads) return;
    const int h = (e / D) % G, d = e % D;
    const int r = unit / p.kv_heads, g = unit % p.kv_heads;
    const int slot = p.slot_ids[r];
    const int L = p.cache_lens[r];
    if (slot < 0 || slot >= p.n_slots || L < 1 || L > p.capacity) return;
    const int nchunks = (L + p.chunk - 1) / p.chunk;
    if (nchunks == 1) return;
    const float *part = p.partials + ((int64_t)unit * p.max_chunks * G + h) * (D + 2);
    const int64_t cstride = (int64_t)G * (D + 2);
    float mv[kDecodeMaxChunks], av[kDecodeMaxChunks], lv[kDecodeMaxChunks];
#pragma unroll
    for (int cc = 0; cc < kDecodeMaxChunks; ++cc) {
        const bool ok = cc < nchunks;
        const float *pp = part + cc * cstride;
        mv[cc] = ok ? pp[D] : -INFINITY;
        av[cc] = ok ? pp[d] : 0.f;
        lv[cc] = ok ? pp[D + 1] : 0.f;
    }
    float M = -INFINITY;
#pragma unroll
    for (int cc = 0; cc < kDecodeMaxChunks; ++cc) M = fmaxf(M, mv[cc]);
    float A = 0.f, S = 0.f;
#pragma unroll
    for (int cc = 0; cc < kDecodeMaxChunks; ++cc) {
        const float f = __builtin_amdgcn_exp2f(mv[cc] - M);
        A = fmaf(f, av[cc], A);
        S = fmaf(f, lv[cc], S);
    }
    static_cast<uint16_t *>(p.out)[((int64_t)r * p.heads + g * G + h) * D + d] = to_bf16(A / S);
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    const int64_t units = (int64_t)a.n_req * a.kv_heads;
    hipLaunchKernelGGL((decode_bf16_kernel<D>), dim3((unsigned)(units * a.max_chunks)), dim3(64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_chunks == 1) return e;
    const int64_t threads = units * a.group * D;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, int32_t head_dim, hipStream_t s) {
    switch (head_dim) {
    case 64: return launch_d<64>(a, s);
    case 128: return launch_d<128>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kev
