// fp32 attention forward (VALU FMA, no reduced precision anywhere).
//
// Tiled exact attention with an online softmax [Attention variants deep-dive,
// §6.2 forward pseudocode]: a workgroup owns 16 query rows of one query head,
// K/V tiles of the head's K/V group are staged in LDS, scores never leave
// registers.  K/V head of query head h is h / g [Attention variants
// deep-dive, §5 GQA code: each K/V head repeated g times along the head axis].
//
// Sixteen lanes share a query row, each holding D/16 of its dimensions (its
// slice of q and of the output accumulator): a score is a 16-lane sum of
// partial dot products, after which every lane of the group holds it and
// keeps the row's running max and sum.  Per 32-key tile the scores are
// computed first, then one rescale and the P.V update.
//
// This path serves fp32 inputs (small problems: latency-bound); the MFMA path
// in prefill_bf16.hip is the throughput kernel.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kLanesPerRow = 16;
constexpr int kThreadsF32 = 256;
constexpr int kRowsF32 = kThreadsF32 / kLanesPerRow;   // query rows per workgroup
constexpr int kKeysF32 = 32;                           // keys per LDS tile

template <int D, bool kWindow>
__global__ __launch_bounds__(kThreadsF32) void prefill_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, int Hq, int Hkv, int Sq, int Sk, float scale_log2, int causal, int window,
    float* __restrict__ lse) {
    constexpr int DL = D / kLanesPerRow;               // dimensions per lane
    __shared__ float ks[kKeysF32][D + 4];
    __shared__ float vs[kKeysF32][D + 4];

    const int tid = threadIdx.x;
    const int sub = tid & (kLanesPerRow - 1);          // dimension slice of this lane
    const int row0 = blockIdx.x * kRowsF32;
    const int row = row0 + tid / kLanesPerRow;
    const int h = blockIdx.y;
    const int b = blockIdx.z;
    const int g = Hq / Hkv;
    const int hk = h / g;
    const bool live = row < Sq;

    const size_t qoff = ((size_t)(b * Hq + h) * Sq) * D;
    const size_t kvoff = ((size_t)(b * Hkv + hk) * Sk) * D;

    float qr[DL], acc[DL];
#pragma unroll
    for (int i = 0; i < DL; ++i) {
        qr[i] = live ? q[qoff + (size_t)row * D + sub * DL + i] : 0.f;
        acc[i] = 0.f;
    }
    float m = -INFINITY, l = 0.f;

    // Keys this workgroup can see: causal rows see j <= row + (Sk - Sq); with
    // a sliding window (window > 0, causal) also j > row + (Sk - Sq) - window,
    // so the first tile is the one holding the first row's first key.
    int kend = Sk;
    if (causal) {
        const int last_row = min(row0 + kRowsF32, Sq) - 1;
        kend = min(Sk, last_row + (Sk - Sq) + 1);
    }
    const int my_last = causal ? row + (Sk - Sq) : Sk - 1;
    const int kbeg = kWindow ? max(0, row0 + (Sk - Sq) - window + 1) / kKeysF32 * kKeysF32 : 0;

    // The next tile's K and V rows are loaded into registers while the
    // current tile is computed (its LDS copy is written at the top of the
    // next iteration), so a tile's load latency is paid once per row block,
    // not once per tile.
    constexpr int kPer = kKeysF32 * D / 4 / kThreadsF32;   // float4 of K (and of V) per thread
    float4 nk[kPer], nv[kPer];
    auto fetch = [&](int j0) {
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const int e = x * kThreadsF32 + tid;
            const int r = e / (D / 4), c = 4 * (e % (D / 4));
            const bool in = (j0 + r) < Sk;
            nk[x] = in ? *reinterpret_cast<const float4*>(k + kvoff + (size_t)(j0 + r) * D + c)
                       : float4{0.f, 0.f, 0.f, 0.f};
            nv[x] = in ? *reinterpret_cast<const float4*>(v + kvoff + (size_t)(j0 + r) * D + c)
                       : float4{0.f, 0.f, 0.f, 0.f};
        }
    };
    if (kbeg < kend) fetch(kbeg);
    for (int j0 = kbeg; j0 < kend; j0 += kKeysF32) {
        __syncthreads();
#pragma unroll
        for (int x = 0; x < kPer; ++x) {
            const int e = x * kThreadsF32 + tid;
            const int r = e / (D / 4), c = 4 * (e % (D / 4));
            *reinterpret_cast<float4*>(&ks[r][c]) = nk[x];
            *reinterpret_cast<float4*>(&vs[r][c]) = nv[x];
        }
        __syncthreads();
        if (j0 + kKeysF32 < kend) fetch(j0 + kKeysF32);

        float s[kKeysF32];
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < kKeysF32; ++r) {
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < DL; ++i) dot = fmaf(qr[i], ks[r][sub * DL + i], dot);
#pragma unroll
            for (int x = 1; x < kLanesPerRow; x <<= 1) dot += __shfl_xor(dot, x, 64);
            const int j = j0 + r;
            const bool vis = (j < Sk) && (j <= my_last) && (!kWindow || j > my_last - window);
            s[r] = vis ? dot * scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, s[r]);
        }
        const float m_new = fmaxf(m, tmax);
        if (m_new == -INFINITY) continue;              // nothing visible yet for this row
        const float alpha = exp2f(m - m_new);          // 0 when m == -inf
        l *= alpha;
#pragma unroll
        for (int i = 0; i < DL; ++i) acc[i] *= alpha;
#pragma unroll
        for (int r = 0; r < kKeysF32; ++r) {
            const float p = exp2f(s[r] - m_new);
            l += p;
#pragma unroll
            for (int i = 0; i < DL; ++i) acc[i] = fmaf(p, vs[r][sub * DL + i], acc[i]);
        }
        m = m_new;
    }

    if (live) {
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int i = 0; i < DL; ++i) o[qoff + (size_t)row * D + sub * DL + i] = acc[i] * inv;
        // optional natural-log log-sum-exp of the row: ln 2 * (m + log2 l)
        if (lse && sub == 0) lse[((size_t)b * Hq + h) * Sq + row] = (m + __builtin_amdgcn_logf(l)) * kLn2;
    }
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream) {
    const int window = a.window > 0 ? a.window : 0;
    dim3 grid((a.Sq + kRowsF32 - 1) / kRowsF32, a.Hq, a.B);
    const float sl = a.scale * kLog2e;
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    float* o = static_cast<float*>(a.o);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kThreadsF32), 0, stream, q, k, v, o, a.Hq, a.Hkv, a.Sq, a.Sk, sl,
                           a.causal, window, a.lse);
    };
    if (a.d == 64)
        window > 0 ? launch(prefill_f32_kernel<64, true>) : launch(prefill_f32_kernel<64, false>);
    else
        window > 0 ? launch(prefill_f32_kernel<128, true>) : launch(prefill_f32_kernel<128, false>);
    return hipGetLastError();
}

}  // namespace gqa
