// kev_prefill_f32.hip -- packed, segment-isolated causal prefill in fp32 (small head dims).
//
// Same definition as the bf16 kernel (primer sakurs2.com section 2.1 formula,
// causal AND block-diagonal mask of the Kev article icman.com.cn sections 2.1
// and 2.3), with every product, exponential and sum in fp32 so that results
// stay within fp32 rounding of the exact value.  One wavefront per (work item,
// query head); each lane owns one query row and keeps a running max, running
// sum and rescaled accumulator updated key by key (the online softmax of the
// primer's section 2.4 with blocks of one key).  K/V tiles of 64 keys of the
// item's own question are staged in LDS; keys past the row are never visited.
#include "kev_internal.h"

namespace kev {

namespace {

constexpr int KT = 64;

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(PrefillArgs p) {
    __shared__ float ks[KT][D];
    __shared__ float vs[KT][D];

    const int32_t n_items = p.sched[0];
    const int item = blockIdx.x / p.heads;
    if (item >= n_items) return;
    const int head = blockIdx.x % p.heads;
    const int kvh = head / p.group;
    const int32_t *it = p.sched + p.items_off + 2 * item;
    const int seg = it[0], t = it[1];
    const int a = p.cu[seg], L = p.cu[seg + 1] - a;
    const int lane = threadIdx.x;
    const int row = t * kF32BlockRows + lane;
    const bool valid = row < L;
    const int key_end = min((t + 1) * kF32BlockRows, L);

    const float *qg = static_cast<const float *>(p.q);
    const float *kg = static_cast<const float *>(p.k) + ((int64_t)a * p.kv_heads + kvh) * D;
    const float *vg = static_cast<const float *>(p.v) + ((int64_t)a * p.kv_heads + kvh) * D;
    const int64_t kv_stride = (int64_t)p.kv_heads * D;

    float q[D], acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        q[c] = valid ? qg[((int64_t)(a + row) * p.heads + head) * D + c] * p.scale_log2 : 0.f;
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    for (int k0 = 0; k0 < key_end; k0 += KT) {
        __syncthreads();
        for (int e = lane; e < KT * D / 4; e += 64) {
            int kr = e / (D / 4), c4 = e % (D / 4);
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f), vv4 = kv4;
            if (k0 + kr < key_end) {
                kv4 = *reinterpret_cast<const float4 *>(kg + (k0 + kr) * kv_stride + c4 * 4);
                vv4 = *reinterpret_cast<const float4 *>(vg + (k0 + kr) * kv_stride + c4 * 4);
            }
            *reinterpret_cast<float4 *>(&ks[kr][c4 * 4]) = kv4;
            *reinterpret_cast<float4 *>(&vs[kr][c4 * 4]) = vv4;
        }
        __syncthreads();
        if (!valid) continue;
        const int jn = min(KT, row + 1 - k0);   // keys k0 .. row of this tile
        for (int j = 0; j < jn; ++j) {
            float s = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) s = fmaf(q[c], ks[j][c], s);
            const float m_new = fmaxf(m, s);
            const float corr = exp2f(m - m_new);
            const float e = exp2f(s - m_new);
            l = l * corr + e;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(e, vs[j][c], acc[c] * corr);
            m = m_new;
        }
    }
    if (!valid) return;
    float *op = static_cast<float *>(p.out) + ((int64_t)(a + row) * p.heads + head) * D;
    const float inv = 1.f / l;
#pragma unroll
    for (int c = 0; c < D; ++c) op[c] = acc[c] * inv;
}

template <int D>
hipError_t launch(const PrefillArgs &a, int64_t grid, hipStream_t s) {
    hipLaunchKernelGGL((prefill_f32_kernel<D>), dim3((unsigned)grid), dim3(64), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs &a, int32_t head_dim, int64_t grid,
                              hipStream_t s) {
    switch (head_dim) {
    case 16: return launch<16>(a, grid, s);
    case 32: return launch<32>(a, grid, s);
    case 64: return launch<64>(a, grid, s);
    case 128: return launch<128>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace kev
