// fp32 attention forward (VALU FMA, no reduced precision anywhere).
//
// Tiled exact attention with an online softmax [Attention variants deep-dive,
// §6.2 forward pseudocode]: one wavefront owns 64 query rows of one query
// head, K/V tiles of the head's K/V group are staged in LDS, scores never leave
// registers.  Each lane owns one query row: its running max, running sum and
// output accumulator.  K/V head of query head h is h / g [Attention variants
// deep-dive, §5 GQA code: each K/V head repeated g times along the head axis].
//
// This path serves fp32 inputs (small problems: latency-bound); the MFMA path
// in prefill_bf16.hip is the throughput kernel.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kRows = 64;      // query rows per workgroup (one per lane)
constexpr int kKeys = 16;      // keys per LDS tile

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, int Hq, int Hkv, int Sq, int Sk, float scale_log2, int causal) {
    __shared__ float ks[kKeys][D + 1];
    __shared__ float vs[kKeys][D];

    const int lane = threadIdx.x;
    const int row0 = blockIdx.x * kRows;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = Hq / Hkv;
    const int hk = h / g;
    const int row = row0 + lane;
    const bool live = row < Sq;

    const size_t qoff = ((size_t)(b * Hq + h) * Sq) * D;
    const size_t kvoff = ((size_t)(b * Hkv + hk) * Sk) * D;

    float qr[D];
    float acc[D];
#pragma unroll
    for (int c = 0; c < D; ++c) {
        qr[c] = live ? q[qoff + (size_t)row * D + c] : 0.f;
        acc[c] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    // Keys this workgroup can see: causal rows see j <= row + (Sk - Sq).
    int kend = Sk;
    if (causal) {
        const int last_row = min(row0 + kRows, Sq) - 1;
        kend = min(Sk, last_row + (Sk - Sq) + 1);
    }
    const int my_last = causal ? row + (Sk - Sq) : Sk - 1;

    for (int j0 = 0; j0 < kend; j0 += kKeys) {
        __syncthreads();
        for (int e = lane; e < kKeys * D; e += 64) {
            const int r = e / D, c = e % D;
            const bool in = (j0 + r) < Sk;
            ks[r][c] = in ? k[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
            vs[r][c] = in ? v[kvoff + (size_t)(j0 + r) * D + c] : 0.f;
        }
        __syncthreads();

        float s[kKeys];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            float dot = 0.f;
#pragma unroll
            for (int c = 0; c < D; ++c) dot = fmaf(qr[c], ks[r][c], dot);
            const int j = j0 + r;
            const bool vis = (j < Sk) && (j <= my_last);
            s[r] = vis ? dot * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;           // nothing visible yet for this row
        const float alpha = exp2f(m - m_new);       // 0 when m == -inf
        l *= alpha;
#pragma unroll
        for (int c = 0; c < D; ++c) acc[c] *= alpha;
#pragma unroll
        for (int r = 0; r < kKeys; ++r) {
            const float p = exp2f(s[r] - m_new);
            l += p;
#pragma unroll
            for (int c = 0; c < D; ++c) acc[c] = fmaf(p, vs[r][c], acc[c]);
        }
        m = m_new;
    }

    if (live) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) o[qoff + (size_t)row * D + c] = acc[c] * inv;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    dim3 grid((a.Sq + kRows - 1) / kRows, a.Hq, a.B);
    const float sl = a.scale * kLog2e;
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    if (a.d == 64)
        hipLaunchKernelGGL(prefill_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, o, a.Hq, a.Hkv,
                           a.Sq, a.Sk, sl, a.causal);
    else
        hipLaunchKernelGGL(prefill_f32_kernel<128>, grid, dim3(64), 0, stream, q, k, v, o, a.Hq, a.Hkv,
                           a.Sq, a.Sk, sl, a.causal);
    return hipGetLastError();
}

}  // namespace gqa
