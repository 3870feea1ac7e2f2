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
// rescale of O^T by exp2(m_old - m_new) is lane-uniform, and P^T feeds the
// second MFMA straight from the first one's accumulators (converted to bf16).
// V is stored transposed in LDS with each 16-key group reordered (4-key groups
// 0,2,1,3) so that a lane's 8 B-operand keys match the accumulator rows it holds.
#include "kev_internal.h"

namespace kev {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int KT = 64;             // keys per LDS tile
constexpr int KROW = 8;            // bf16 padding per K row in LDS (bank spread)
constexpr int VROW = 8;            // bf16 padding per V^T row in LDS

template <int D>
struct Smem {
    uint16_t k[2][KT][D + KROW];   // K tile, row-major [key][d]
    uint16_t vt[2][D][KT + VROW];  // V tile transposed [d][key], 4-key groups reordered
};

__device__ inline bf16x8 as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8, u); }

// Position of 4-key group `kg` (keys 4kg..4kg+3 of a tile) inside its V^T row.
__device__ inline int vt_pos(int kg) {
    const int q = kg & 3;
    return (kg & ~3) * 4 + ((q == 1) ? 2 : (q == 2) ? 1 : q) * 4;
}

// Byte-select helpers: low / high bf16 halves of two dwords into one dword.
__device__ inline uint32_t pack_lo(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x05040100u); }
__device__ inline uint32_t pack_hi(uint32_t a, uint32_t b) { return __builtin_amdgcn_perm(b, a, 0x07060302u); }

template <int D, int NW>
struct Loader {
    static constexpr int NT = NW * 64;
    static constexpr int KCH = KT * D / 8;              // 16-byte chunks of a K tile
    static constexpr int NK = (KCH + NT - 1) / NT;
    static constexpr int VU = (KT / 4) * (D / 8);       // (4 keys x 8 d) units of a V tile
    static constexpr int NV = (VU + NT - 1) / NT;
    uint4 kr[NK];
    uint4 vr[NV][4];

    // Global -> registers for key tile starting at question-relative key k0.
    // Keys at or past key_end (end of what this item needs) read as zero.
    __device__ void load(const uint16_t *kbase, const uint16_t *vbase, int64_t row_stride,
                         int k0, int key_end) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            int c = tid + i * NT;
            kr[i] = make_uint4(0, 0, 0, 0);
            if (c < KCH) {
                int key = k0 + c / (D / 8), ch = c % (D / 8);
                if (key < key_end)
                    kr[i] = *reinterpret_cast<const uint4 *>(kbase + key * row_stride + ch * 8);
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int u = tid + i * NT;
#pragma unroll
            for (int r = 0; r < 4; ++r) vr[i][r] = make_uint4(0, 0, 0, 0);
            if (u < VU) {
                int dg = u / (KT / 4), kg = u % (KT / 4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    int key = k0 + kg * 4 + r;
                    if (key < key_end)
                        vr[i][r] = *reinterpret_cast<const uint4 *>(vbase + key * row_stride + dg * 8);
                }
            }
        }
    }

    // Registers -> LDS buffer.  V is transposed: 4 keys x 8 d become 8 rows of 4 keys.
    __device__ void store(Smem<D> &sm, int buf) {
        const int tid = threadIdx.x;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            int c = tid + i * NT;
            if (c < KCH) {
                int row = c / (D / 8), ch = c % (D / 8);
                *reinterpret_cast<uint4 *>(&sm.k[buf][row][ch * 8]) = kr[i];
            }
        }
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            int u = tid + i * NT;
            if (u < VU) {
                int dg = u / (KT / 4), kg = u % (KT / 4);
                int pos = vt_pos(kg);
                const uint32_t *a0 = reinterpret_cast<const uint32_t *>(&vr[i][0]);
                const uint32_t *a1 = reinterpret_cast<const uint32_t *>(&vr[i][1]);
                const uint32_t *a2 = reinterpret_cast<const uint32_t *>(&vr[i][2]);
                const uint32_t *a3 = reinterpret_cast<const uint32_t *>(&vr[i][3]);
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    // dword w of each key holds d = 2w (low half) and 2w+1 (high half)
                    uint2 lo = make_uint2(pack_lo(a0[w], a1[w]), pack_lo(a2[w], a3[w]));
                    uint2 hi = make_uint2(pack_hi(a0[w], a1[w]), pack_hi(a2[w], a3[w]));
                    *reinterpret_cast<uint2 *>(&sm.vt[buf][dg * 8 + 2 * w][pos]) = lo;
                    *reinterpret_cast<uint2 *>(&sm.vt[buf][dg * 8 + 2 * w + 1][pos]) = hi;
                }
            }
        }
    }
};

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void prefill_bf16_kernel(PrefillArgs p) {
    constexpr int DC = D / 16;   // 16-wide d chunks (k steps of the S MFMA)
    constexpr int DB = D / 32;   // 32-row d blocks of O^T
    __shared__ Smem<D> sm;

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

    const int row0 = t * p.block_rows + rb * 32;          // question-relative first row
    const int item_key_end = min((t + 1) * p.block_rows, L);
    const int wave_key_end = row0 < L ? min(row0 + 32, L) : 0;   // keys this wavefront needs
    const int n_tiles = (item_key_end + KT - 1) / KT;

    const uint16_t *qg = static_cast<const uint16_t *>(p.q);
    const uint16_t *kg = static_cast<const uint16_t *>(p.k) + ((int64_t)a * p.kv_heads + kvh) * D;
    const uint16_t *vg = static_cast<const uint16_t *>(p.v) + ((int64_t)a * p.kv_heads + kvh) * D;
    const int64_t kv_stride = (int64_t)p.kv_heads * D;

    // Q^T operand: lane holds q row (row0 + col), d = dc*16 + half*8 .. +8.
    const int qrow = row0 + col;
    bf16x8 qf[DC];
    {
        const uint16_t *qp = qg + ((int64_t)(a + qrow) * p.heads + head) * D + half * 8;
#pragma unroll
        for (int dc = 0; dc < DC; ++dc) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qrow < L) u = *reinterpret_cast<const uint4 *>(qp + dc * 16);
            qf[dc] = as_bf16x8(u);
        }
    }

    f32x16 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[db][i] = 0.f;
    float m_run = -INFINITY;   // running max of scaled scores (log2 units)
    float l_run = 0.f;         // running sum of this lane's half of the keys

    Loader<D, NW> ld;
    ld.load(kg, vg, kv_stride, 0, item_key_end);

    for (int kt = 0; kt < n_tiles; ++kt) {
        const int buf = kt & 1;
        ld.store(sm, buf);
        __syncthreads();
        if (kt + 1 < n_tiles) ld.load(kg, vg, kv_stride, (kt + 1) * KT, item_key_end);

        const int k0 = kt * KT;
        if (k0 >= wave_key_end) continue;   // tile entirely above this wavefront's rows

        // ---- S^T = K Q^T for two 32-key sub-blocks ----
        f32x16 s[2];
        bool active[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            active[kb] = (k0 + kb * 32) < wave_key_end;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kb][i] = 0.f;
            if (active[kb]) {
                const uint16_t *kr = &sm.k[buf][kb * 32 + col][half * 8];
#pragma unroll
                for (int dc = 0; dc < DC; ++dc) {
                    bf16x8 kf = as_bf16x8(*reinterpret_cast<const uint4 *>(kr + dc * 16));
                    s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[dc], s[kb], 0, 0, 0);
                }
            }
        }

        // ---- mask (diagonal / tail sub-blocks only), row max ----
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int ks = k0 + kb * 32;
            if (!active[kb]) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kb][i] = -INFINITY;
            } else if (ks + 31 > row0 || ks + 32 > L) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = ks + (i >> 2) * 8 + half * 4 + (i & 3);
                    if (key > qrow || key >= L) s[kb][i] = -INFINITY;
                }
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 32));

        // ---- online softmax update ----
        const float m_new = fmaxf(m_run, mx * p.scale_log2);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        m_run = m_new;
        float rs = 0.f;
        bf16x8 pb[4];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            f32x8 lo8, hi8;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float e = __builtin_amdgcn_exp2f(s[kb][i] * p.scale_log2 - m_new);
                rs += e;
                if (i < 8) lo8[i] = e;
                else hi8[i - 8] = e;
            }
            pb[kb * 2] = __builtin_convertvector(lo8, bf16x8);
            pb[kb * 2 + 1] = __builtin_convertvector(hi8, bf16x8);
        }
        l_run = l_run * alpha + rs;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) o[db][i] *= alpha;

        // ---- O^T += V^T P^T ----
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            if (!active[c >> 1]) continue;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const uint16_t *vr = &sm.vt[buf][db * 32 + col][c * 16 + half * 8];
                bf16x8 vf = as_bf16x8(*reinterpret_cast<const uint4 *>(vr));
                o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pb[c], o[db], 0, 0, 0);
            }
        }
    }

    // ---- epilogue: divide by the row sum, round to bf16, store rows inside the question ----
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (qrow >= L || row0 >= L) return;
    const float inv = 1.f / l_tot;
    uint16_t *op = static_cast<uint16_t *>(p.out) + ((int64_t)(a + qrow) * p.heads + head) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
            f32x4 f;
#pragma unroll
            for (int j = 0; j < 4; ++j) f[j] = o[db][g4 * 4 + j] * inv;
            bf16x4 b = __builtin_convertvector(f, bf16x4);
            *reinterpret_cast<bf16x4 *>(op + db * 32 + g4 * 8 + half * 4) = b;
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
