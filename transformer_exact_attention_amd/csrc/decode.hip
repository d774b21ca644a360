// Decode attention over a KV cache: split-KV partials + log-sum-exp combine.
//
// The method: during autoregressive generation the new token's query attends
// to every cached key and value; the cost is streaming the cache from device
// memory, and fewer K/V heads stream fewer bytes [Attention variants
// deep-dive, §1 and §7 KV Cache; Different attention mechanisms, §2 MQA and §3
// GQA advantages].  Each K/V head is therefore read exactly once per group of
// g = Hq / Hkv query heads (head h reads K/V head h / g, [Attention variants
// deep-dive, §5 GQA code]).  The cache is contiguous, or paged: fixed-size
// 16-token blocks placed anywhere, found through a per-sequence block table
// [Different attention mechanisms, §5 Page Attention, steps 1-2].
//
// Kernel 1 (split): workgroup = (split of kSplit tokens, K/V head, sequence),
// four wavefronts of 64 tokens each.  Per 16-token block a wavefront computes
//   S^T (16 keys x 16 heads) = K (16 x d) . Q^T (d x 16)    v_mfma_f32_16x16x32_bf16
//   O^T (d x 16 heads)      += V^T (d x 16 keys) . P^T      v_mfma_f32_16x16x16_bf16
// Lane i (c = i%16, q4 = i/16) loads K row c of the block (contraction over d)
// and V rows 4*q4..4*q4+3 at d-chunk c.  For the PV product the 16 "rows" of
// MFMA j are d = 8*m + j, m = 0..15, so each lane's own V rows supply its A
// operand with one byte permute per dword and the S^T accumulator already is
// the P^T operand: no LDS transpose, no cross-lane traffic.  The four
// wavefronts' (max, sum, accumulator) are merged in LDS in a fixed order and
// written as one normalised partial + base-2 log-sum-exp per (head, split).
//
// Kernel 2 (combine): per (sequence, query head) merges the partials with
// weights 2^(lse_s - max lse), the rescale step of the tiled online softmax
// [Attention variants deep-dive, §6.2 forward pseudocode] applied across
// splits, and writes bf16.  Fixed reduction order everywhere: results are
// bitwise reproducible, and paged == contiguous bitwise for equal contents.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kWaveKeys = 64;
constexpr int kWaves = kDecodeSplit / kWaveKeys;     // 4
constexpr int kThreads = kWaves * 64;

struct ContiguousRows {
    const uint16_t* base;     // cache base
    int Hkv, S_max;
    // Pointer to the first of 16 consecutive tokens t0..t0+15 (t0 % 16 == 0).
    __device__ __forceinline__ const uint16_t* block(int b, int hk, int t0) const {
        return base + (((size_t)b * Hkv + hk) * S_max + t0) * kD;
    }
};

struct PagedRows {
    const uint16_t* base;     // pages [num_blocks, Hkv, 16, d]
    const int32_t* table;     // [B, max_blocks]
    int Hkv, max_blocks;
    __device__ __forceinline__ const uint16_t* block(int b, int hk, int t0) const {
        const int phys = table[(size_t)b * max_blocks + (t0 >> 4)];
        return base + (((size_t)phys * Hkv + hk) * 16) * kD;
    }
};

template <int NHB, class Rows>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(
    const uint16_t* __restrict__ q, Rows krows, Rows vrows, const int32_t* __restrict__ seq_lens,
    float* __restrict__ opart, float* __restrict__ lsepart, int Hq, int Hkv, int g, int nsplit_max,
    float scale_log2) {
    constexpr int NH = 16 * NHB;                     // head columns computed
    __shared__ float sm[kWaves][NH];
    __shared__ float sl[kWaves][NH];
    __shared__ __attribute__((aligned(16))) float so[kWaves][NH][kD];

    const int split = blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
    const int L = seq_lens[b];
    const int t_begin = split * kDecodeSplit;
    if (t_begin >= L) return;                        // uniform for the workgroup

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15;
    const int q4 = lane >> 4;
    const int tw = t_begin + wave * kWaveKeys;
    const bool wlive = tw < L;                       // uniform for the wavefront

    float m_w[NHB], l_w[NHB];
    f32x4 oacc[NHB][8];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        m_w[hb] = -INFINITY;
        l_w[hb] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[hb][j] = f32x4{};
    }

    if (wlive) {
        // Q^T operand: lane holds Q[head hb*16 + c][32*ds + 8*q4 .. +8] (zero for heads >= g).
        bf16x8 qf[NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const int hl = hb * 16 + c;
            const bool hv = hl < g;
            const uint16_t* qp = q + ((size_t)b * Hq + hk * g + (hv ? hl : 0)) * kD;
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) {
                u32x4 w = {0u, 0u, 0u, 0u};
                if (hv) w = *reinterpret_cast<const u32x4*>(qp + 32 * ds + 8 * q4);
                qf[hb][ds] = __builtin_bit_cast(bf16x8, w);
            }
        }

        // Issue every load of the wavefront's 64 tokens up front.
        u32x4 kr[4][4], vr[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int t0 = tw + 16 * kb;
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                kr[kb][x] = u32x4{0u, 0u, 0u, 0u};
                vr[kb][x] = u32x4{0u, 0u, 0u, 0u};
            }
            if (t0 < L) {
                const uint16_t* kp = krows.block(b, hk, t0);
                const uint16_t* vp = vrows.block(b, hk, t0);
                if (t0 + c < L) {
#pragma unroll
                    for (int ds = 0; ds < 4; ++ds)
                        kr[kb][ds] = *reinterpret_cast<const u32x4*>(kp + c * kD + 32 * ds + 8 * q4);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    if (t0 + 4 * q4 + rr < L)
                        vr[kb][rr] = *reinterpret_cast<const u32x4*>(vp + (4 * q4 + rr) * kD + 8 * c);
                }
            }
        }

        // Scores, masked past the sequence end.
        float s[NHB][4][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int ds = 0; ds < 4; ++ds)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[kb][ds]),
                                                                   qf[hb][ds], acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = tw + 16 * kb + 4 * q4 + r;
                    s[hb][kb][r] = key < L ? acc[r] * scale_log2 : -INFINITY;
                }
            }
        }

        // Per head: max and sum over the wavefront's keys (lanes c, c+16, c+32, c+48).
        bf16x4 pf[NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float mx = -INFINITY;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[hb][kb][r]);
            mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
            mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
            float sum = 0.f;
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                float p[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    p[r] = exp2_fast(s[hb][kb][r] - mx);
                    sum += p[r];
                }
                u32x2 w;
                w.x = pack_bf16x2(p[0], p[1]);
                w.y = pack_bf16x2(p[2], p[3]);
                pf[hb][kb] = __builtin_bit_cast(bf16x4, w);
            }
            sum += __shfl_xor(sum, 16, 64);
            sum += __shfl_xor(sum, 32, 64);
            m_w[hb] = mx;
            l_w[hb] = sum;
        }

        // O^T += V^T . P^T; MFMA j covers d = 8*m + j.
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int dw = j >> 1;
                u32x2 a;
                if (j & 1) {
                    a.x = pack_hi16(vr[kb][0][dw], vr[kb][1][dw]);
                    a.y = pack_hi16(vr[kb][2][dw], vr[kb][3][dw]);
                } else {
                    a.x = pack_lo16(vr[kb][0][dw], vr[kb][1][dw]);
                    a.y = pack_lo16(vr[kb][2][dw], vr[kb][3][dw]);
                }
                const bf16x4 av = __builtin_bit_cast(bf16x4, a);
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb)
                    oacc[hb][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pf[hb][kb], oacc[hb][j], 0, 0, 0);
            }
        }
    }

    // Publish this wavefront's state.  Lane holds head hb*16 + c, d = 32*q4 + 8*r + j.
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        if (q4 == 0) {
            sm[wave][hb * 16 + c] = m_w[hb];
            sl[wave][hb * 16 + c] = l_w[hb];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            f32x4 lo = {oacc[hb][0][r], oacc[hb][1][r], oacc[hb][2][r], oacc[hb][3][r]};
            f32x4 hi = {oacc[hb][4][r], oacc[hb][5][r], oacc[hb][6][r], oacc[hb][7][r]};
            float* dst = &so[wave][hb * 16 + c][32 * q4 + 8 * r];
            *reinterpret_cast<f32x4*>(dst) = lo;
            *reinterpret_cast<f32x4*>(dst + 4) = hi;
        }
    }
    __syncthreads();

    // Merge the wavefronts (fixed order) and write the split's partial.
    for (int idx = tid; idx < g * kD; idx += kThreads) {
        const int hl = idx / kD, dd = idx % kD;
        float M = sm[0][hl];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sm[w][hl]);
        float num = 0.f, den = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = exp2_fast(sm[w][hl] - M);    // 0 for wavefronts past the end
            num += f * so[w][hl][dd];
            den += f * sl[w][hl];
        }
        const size_t row = ((size_t)b * Hq + hk * g + hl) * nsplit_max + split;
        opart[row * kD + dd] = num / den;
        if (dd == 0) lsepart[row] = M + __builtin_amdgcn_logf(den);   // v_log_f32: log2
    }
}

__global__ __launch_bounds__(kD) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o, int Hq, int nsplit_max) {
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int dd = threadIdx.x;
    const int L = seq_lens[b];
    const int ns = (L + kDecodeSplit - 1) / kDecodeSplit;
    const size_t row0 = ((size_t)b * Hq + hq) * nsplit_max;
    float out = 0.f;
    if (ns > 0) {
        float M = -INFINITY;
        for (int s = 0; s < ns; ++s) M = fmaxf(M, lsepart[row0 + s]);
        float num = 0.f, den = 0.f;
        for (int s = 0; s < ns; ++s) {
            const float w = exp2_fast(lsepart[row0 + s] - M);
            num += w * opart[(row0 + s) * kD + dd];
            den += w;
        }
        out = num / den;
    }
    const uint32_t packed = pack_bf16x2(out, 0.f);
    o[((size_t)b * Hq + hq) * kD + dd] = (uint16_t)(packed & 0xffffu);
}

template <int NHB>
hipError_t launch_split(const DecodeArgs& a, hipStream_t stream, float* opart, float* lsepart, int ns_max) {
    dim3 grid(ns_max, a.Hkv, a.B);
    const int g = a.Hq / a.Hkv;
    const float sl = a.scale * kLog2e;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
    if (a.block_table) {
        PagedRows kr{kc, a.block_table, a.Hkv, a.max_blocks_per_seq};
        PagedRows vr{vc, a.block_table, a.Hkv, a.max_blocks_per_seq};
        hipLaunchKernelGGL((decode_split_kernel<NHB, PagedRows>), grid, dim3(kThreads), 0, stream, q, kr, vr,
                           a.seq_lens, opart, lsepart, a.Hq, a.Hkv, g, ns_max, sl);
    } else {
        ContiguousRows kr{kc, a.Hkv, a.max_seq_len};
        ContiguousRows vr{vc, a.Hkv, a.max_seq_len};
        hipLaunchKernelGGL((decode_split_kernel<NHB, ContiguousRows>), grid, dim3(kThreads), 0, stream, q, kr,
                           vr, a.seq_lens, opart, lsepart, a.Hq, a.Hkv, g, ns_max, sl);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const int ns_max = decode_nsplit_max(a.max_seq_len);
    float* opart = static_cast<float*>(a.workspace);
    float* lsepart = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                              align256((size_t)a.B * a.Hq * ns_max * kD * 4));
    const int g = a.Hq / a.Hkv;
    hipError_t e = g <= 16 ? launch_split<1>(a, stream, opart, lsepart, ns_max)
                           : launch_split<2>(a, stream, opart, lsepart, ns_max);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(kD), 0, stream, opart, lsepart, a.seq_lens,
                       static_cast<uint16_t*>(a.o), a.Hq, ns_max);
    return hipGetLastError();
}

}  // namespace gqa
