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
// Decode reads every cached K/V byte once and does ~4 FLOP per byte, far
// below the MI355X ridge point, so the kernel is shaped for HBM bandwidth:
//   - a unit is (request, KV head); its positions are cut into chunks of
//     kDecodeChunk positions, one workgroup per chunk, so long and short
//     slots spread evenly over the CUs;
//   - each wavefront streams a contiguous quarter of the chunk; 16 lanes read
//     one 256-byte K (or V) row with 16-byte loads, 4 rows per instruction,
//     fully coalesced along the slot's contiguous [position][d] plane;
//   - all `group` query heads of the KV head are served from the same loaded
//     rows (scores via v_dot2_f32_bf16, cross-lane sums via DPP);
//   - the softmax is blockwise online (running max / sum / rescaled
//     accumulator, primer section 2.4) over 32-position sub-blocks, then
//     wavefronts are merged in LDS; a unit with one chunk writes its output
//     directly, otherwise each chunk writes (max, sum, accumulator) and a
//     second small kernel merges the chunks with the same rescaling identity.
//     (A last-arriving-workgroup merge inside one kernel would need
//     device-scope fences, which write back and invalidate the XCD's L2 on
//     every workgroup; the kernel boundary gives the same ordering once.)
#include "kev_internal.h"
#include "../../include/kev.h"

namespace kev {

namespace {

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int CTRL>
__device__ inline float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                                 CTRL, 0xF, 0xF, false));
}

// Sum over groups of LANES (8 or 16) consecutive lanes; every lane gets the group sum.
template <int LANES>
__device__ inline float group_sum(float x) {
    x += dpp<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);   // row_half_mirror: 8-lane groups
    if (LANES == 16) x += dpp<0x140>(x);   // row_mirror: 16-lane rows
    return x;
}

__device__ inline float dot8(uint4 a, uint4 b, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.x), __builtin_bit_cast(bf16x2, b.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.y), __builtin_bit_cast(bf16x2, b.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.z), __builtin_bit_cast(bf16x2, b.z), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a.w), __builtin_bit_cast(bf16x2, b.w), acc, false);
    return acc;
}

__device__ inline void unpack8(uint4 u, float f[8]) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
}

__device__ inline uint16_t to_bf16(float x) {
    return __builtin_bit_cast(uint16_t, (__bf16)x);
}

template <int D, int GMAX>
__global__ __launch_bounds__(kDecodeWaves * 64) void decode_bf16_kernel(DecodeArgs p) {
    constexpr int NW = kDecodeWaves;
    constexpr int DG = D / 8;          // lanes per row (8 bf16 each)
    constexpr int RPI = 64 / DG;       // rows per wavefront instruction
    constexpr int SB = 32;             // positions per online-softmax sub-block
    constexpr int NI = SB / RPI;       // instructions per sub-block
    __shared__ float w_m[NW][GMAX], w_l[NW][GMAX];
    __shared__ float w_acc[NW][GMAX][D];

    const int G = (GMAX == 1 || GMAX == 2 || GMAX == 4) ? GMAX : p.group;
    const int unit = blockIdx.x / p.max_chunks;
    const int c = blockIdx.x % p.max_chunks;
    const int r = unit / p.kv_heads, g = unit % p.kv_heads;
    const int slot = p.slot_ids[r];
    const int L = p.cache_lens[r];
    const int tid = threadIdx.x;
    if (slot < 0 || slot >= p.n_slots) {
        if (c == 0 && tid == 0) atomicOr(p.err, (int32_t)KEV_DEVERR_SLOT);
        return;
    }
    if (L < 1 || L > p.capacity) {
        if (c == 0 && tid == 0) atomicOr(p.err, (int32_t)KEV_DEVERR_CACHE_LEN);
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

    // In-place append of the new token (by the chunk that holds position L-1).
    if (c == (L - 1) / p.chunk) {
        if (tid < DG)
            *reinterpret_cast<uint4 *>(kbase + (int64_t)(L - 1) * D + tid * 8) =
                *reinterpret_cast<const uint4 *>(knew + tid * 8);
        else if (tid < 2 * DG)
            *reinterpret_cast<uint4 *>(vbase + (int64_t)(L - 1) * D + (tid - DG) * 8) =
                *reinterpret_cast<const uint4 *>(vnew + (tid - DG) * 8);
    }

    const int wave = tid >> 6, lane = tid & 63;
    const int rg = lane / DG, dg = lane % DG;

    uint4 qv[GMAX];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        qv[h] = make_uint4(0, 0, 0, 0);
        if (h < G)
            qv[h] = *reinterpret_cast<const uint4 *>(
                static_cast<const uint16_t *>(p.q) + ((int64_t)r * p.heads + g * G + h) * D + dg * 8);
    }

    float m[GMAX], l[GMAX], acc[GMAX][8];
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        m[h] = -INFINITY;
        l[h] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[h][j] = 0.f;
    }

    const int per_wave = p.chunk / NW;
    const int p0 = c * p.chunk + wave * per_wave;
    const int p1 = min(p0 + per_wave, L);

    for (int sb = p0; sb < p1; sb += SB) {
        uint4 kr[NI], vr[NI];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int pos = sb + i * RPI + rg;
            kr[i] = make_uint4(0, 0, 0, 0);
            vr[i] = make_uint4(0, 0, 0, 0);
            if (pos < p1) {
                const bool is_new = pos == L - 1;
                kr[i] = *reinterpret_cast<const uint4 *>(is_new ? knew + dg * 8 : kbase + (int64_t)pos * D + dg * 8);
                vr[i] = *reinterpret_cast<const uint4 *>(is_new ? vnew + dg * 8 : vbase + (int64_t)pos * D + dg * 8);
            }
        }
        float s[NI][GMAX];
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const bool live = sb + i * RPI + rg < p1;
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h >= G) continue;
                float x = group_sum<DG>(dot8(kr[i], qv[h], 0.f)) * p.scale_log2;
                s[i][h] = live ? x : -INFINITY;
            }
        }
#pragma unroll
        for (int h = 0; h < GMAX; ++h) {
            if (h >= G) continue;
            float mb = -INFINITY;
#pragma unroll
            for (int i = 0; i < NI; ++i) mb = fmaxf(mb, s[i][h]);
#pragma unroll
            for (int o = DG; o < 64; o <<= 1) mb = fmaxf(mb, __shfl_xor(mb, o));
            const float m_new = fmaxf(m[h], mb);
            const float alpha = __builtin_amdgcn_exp2f(m[h] - m_new);
            m[h] = m_new;
            float rs = 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                s[i][h] = __builtin_amdgcn_exp2f(s[i][h] - m_new);
                rs += s[i][h];
            }
            l[h] = l[h] * alpha + rs;
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] *= alpha;
        }
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            float vf[8];
            unpack8(vr[i], vf);
#pragma unroll
            for (int h = 0; h < GMAX; ++h) {
                if (h >= G) continue;
#pragma unroll
                for (int j = 0; j < 8; ++j) acc[h][j] = fmaf(s[i][h], vf[j], acc[h][j]);
            }
        }
    }

    // Merge the row groups of the wavefront (they share m), then the wavefronts in LDS.
#pragma unroll
    for (int h = 0; h < GMAX; ++h) {
        if (h >= G) continue;
#pragma unroll
        for (int o = DG; o < 64; o <<= 1) {
            l[h] += __shfl_xor(l[h], o);
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[h][j] += __shfl_xor(acc[h][j], o);
        }
        if (lane < DG) {
#pragma unroll
            for (int j = 0; j < 8; ++j) w_acc[wave][h][dg * 8 + j] = acc[h][j];
        }
        if (lane == 0) {
            w_m[wave][h] = m[h];
            w_l[wave][h] = l[h];
        }
    }
    __syncthreads();

    float *part = p.partials + ((int64_t)unit * p.max_chunks) * G * (D + 2);
    uint16_t *out = static_cast<uint16_t *>(p.out) + ((int64_t)r * p.heads + g * G) * D;
    for (int e = tid; e < G * D; e += NW * 64) {
        const int h = e / D, d = e % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, w_m[w][h]);
        float A = 0.f, S = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
            const float f = __builtin_amdgcn_exp2f(w_m[w][h] - M);
            A = fmaf(f, w_acc[w][h][d], A);
            S = fmaf(f, w_l[w][h], S);
        }
        if (nchunks == 1) {
            out[h * D + d] = to_bf16(A / S);
        } else {
            float *pp = part + ((int64_t)c * G + h) * (D + 2);
            pp[d] = A;
            if (d == 0) {
                pp[D] = M;
                pp[D + 1] = S;
            }
        }
    }
}

// Merge the chunk partials of every unit that spans more than one chunk.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(DecodeArgs p) {
    const int unit = blockIdx.x;
    const int r = unit / p.kv_heads, g = unit % p.kv_heads;
    const int slot = p.slot_ids[r];
    const int L = p.cache_lens[r];
    if (slot < 0 || slot >= p.n_slots || L < 1 || L > p.capacity) return;
    const int nchunks = (L + p.chunk - 1) / p.chunk;
    if (nchunks == 1) return;
    const int G = p.group;
    const float *part = p.partials + ((int64_t)unit * p.max_chunks) * G * (D + 2);
    uint16_t *out = static_cast<uint16_t *>(p.out) + ((int64_t)r * p.heads + g * G) * D;
    for (int e = threadIdx.x; e < G * D; e += 256) {
        const int h = e / D, d = e % D;
        float M = -INFINITY;
        for (int cc = 0; cc < nchunks; ++cc) M = fmaxf(M, part[((int64_t)cc * G + h) * (D + 2) + D]);
        float A = 0.f, S = 0.f;
        for (int cc = 0; cc < nchunks; ++cc) {
            const float *pp = part + ((int64_t)cc * G + h) * (D + 2);
            const float f = __builtin_amdgcn_exp2f(pp[D] - M);
            A = fmaf(f, pp[d], A);
            S = fmaf(f, pp[D + 1], S);
        }
        out[h * D + d] = to_bf16(A / S);
    }
}

template <int D, int GMAX>
hipError_t launch(const DecodeArgs &a, hipStream_t s) {
    const int64_t units = (int64_t)a.n_req * a.kv_heads;
    hipLaunchKernelGGL((decode_bf16_kernel<D, GMAX>), dim3((unsigned)(units * a.max_chunks)),
                       dim3(kDecodeWaves * 64), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_chunks == 1) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D>), dim3((unsigned)units), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs &a, hipStream_t s) {
    switch (a.group) {
    case 1: return launch<D, 1>(a, s);
    case 2: return launch<D, 2>(a, s);
    case 4: return launch<D, 4>(a, s);
    case 8: return launch<D, 8>(a, s);
    default: return launch<D, 8>(a, s);   // other group sizes up to 8, guarded by p.group
    }
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
