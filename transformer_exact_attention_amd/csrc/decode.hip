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
// Kernel 1 (split): workgroup = (split of T tokens, K/V head, sequence), four
// wavefronts, each streaming a contiguous quarter of the split in 32-token
// chunks: the loads of chunk i+1 are in flight while chunk i is computed, and
// an online softmax runs across chunks.  Per 16-token block a wavefront computes
//   S^T (16 keys x 16 heads) = K (16 x d) . Q^T (d x 16)    v_mfma_f32_16x16x32_bf16
//   O^T (d x 16 heads)      += V^T (d x 16 keys) . P^T      v_mfma_f32_16x16x16_bf16
// Lane i (c = i%16, q4 = i/16) loads K row c of the block (contraction over d)
// and V rows 4*q4..4*q4+3 at d-chunk c.  For the PV product the 16 "rows" of
// MFMA j are d = 8*m + j, m = 0..15, so each lane's own V rows supply its A
// operand with one byte permute per dword and the S^T accumulator already is
// the P^T operand: no LDS transpose, no cross-lane traffic.  The four
// wavefronts' (reference max, sum, accumulator) are merged in LDS in a fixed
// order and written as one normalised partial + base-2 log-sum-exp per
// (head, split).
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
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 32;               // tokens per pipeline stage (two 16-token blocks)
constexpr float kRescaleSlack = 8.0f;    // base-2 units, as in the prefill kernel

// Row addressing.  offset() gives the element offset of token t0 (a multiple
// of 16) of K/V head hk of sequence b; the 16 tokens t0..t0+15 follow it
// contiguously in both layouts.
struct ContiguousRows {
    const uint16_t* kbase;
    const uint16_t* vbase;
    int Hkv, S_max;
    __device__ __forceinline__ int prefetch(int, int, int, int) const { return 0; }
    __device__ __forceinline__ size_t offset(int, int b, int hk, int t0, int) const {
        return (((size_t)b * Hkv + hk) * S_max + t0) * kD;
    }
};

struct PagedRows {
    const uint16_t* kbase;       // pages [num_blocks, Hkv, 16, d]
    const uint16_t* vbase;
    const int32_t* table;        // [B, max_blocks]
    int Hkv, max_blocks;
    // Lane i fetches the table entry of the wavefront's i-th block (once).
    __device__ __forceinline__ int prefetch(int b, int blk0, int nblk, int lane) const {
        return lane < nblk ? table[(size_t)b * max_blocks + blk0 + lane] : 0;
    }
    // Block idx (wavefront-uniform) of this wavefront's range: read its entry from lane idx.
    __device__ __forceinline__ size_t offset(int pref, int, int hk, int, int idx) const {
        const int phys = __builtin_amdgcn_readlane(pref, idx);
        return ((size_t)phys * Hkv + hk) * 16 * kD;
    }
};

template <int NHB, class Rows>
__global__ __launch_bounds__(kThreads, NHB == 1 ? 2 : 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, Rows rows, const int32_t* __restrict__ seq_lens,
    float* __restrict__ opart, float* __restrict__ lsepart, int Hq, int g, int ns, int T, float scale_log2) {
    constexpr int NH = 16 * NHB;                     // head columns computed
    __shared__ float sm[kWaves][NH];
    __shared__ float sl[kWaves][NH];
    __shared__ __attribute__((aligned(16))) float so[kWaves][NH][kD];

    const int split = blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
    const int L = seq_lens[b];
    const int t_begin = split * T;
    if (t_begin >= L) return;                        // uniform for the workgroup

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15;
    const int q4 = lane >> 4;
    const int per_wave = T / kWaves;                 // multiple of kChunk
    const int tw0 = t_begin + wave * per_wave;
    const int tw1 = min(tw0 + per_wave, L);
    const int nchunks = tw1 > tw0 ? (tw1 - tw0 + kChunk - 1) / kChunk : 0;   // wavefront-uniform

    float ref[NHB], lsum[NHB];
    f32x4 oacc[NHB][8];
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        ref[hb] = -INFINITY;
        lsum[hb] = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) oacc[hb][j] = f32x4{};
    }

    if (nchunks > 0) {
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
        const int pref = rows.prefetch(b, tw0 >> 4, (tw1 - tw0 + 15) >> 4, lane);

        typedef u32x4 Buf[2][4];
        // Every load is issued unconditionally through a buffer resource that
        // covers only the block's valid tokens (none past the wavefront's
        // range): the hardware returns zeros beyond it.  With a fixed number of
        // loads per chunk the wait counts stay exact, so chunk i+1 streams in
        // while chunk i is computed.
        auto load = [&](Buf& kr, Buf& vr, int ci) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int t0 = tw0 + ci * kChunk + 16 * blk;
                const int nvalid = min(max(tw1 - t0, 0), 16);                 // wavefront-uniform
                const size_t off = nvalid > 0 ? rows.offset(pref, b, hk, t0, 2 * ci + blk) : 0;
                const __amdgpu_buffer_rsrc_t kr_rs = make_rsrc(rows.kbase + off, (uint32_t)nvalid * kD * 2);
                const __amdgpu_buffer_rsrc_t vr_rs = make_rsrc(rows.vbase + off, (uint32_t)nvalid * kD * 2);
#pragma unroll
                for (int ds = 0; ds < 4; ++ds)
                    kr[blk][ds] = buffer_load16(kr_rs, (uint32_t)(c * kD + 32 * ds + 8 * q4) * 2);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vr[blk][rr] = buffer_load16(vr_rs, (uint32_t)((4 * q4 + rr) * kD + 8 * c) * 2);
            }
        };

        auto process = [&](const Buf& kr, const Buf& vr, int ci) {
            bf16x4 pf[NHB][2];
#pragma unroll
            for (int hb = 0; hb < NHB; ++hb) {
                float s[2][4];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    f32x4 acc = f32x4{};
#pragma unroll
                    for (int ds = 0; ds < 4; ++ds)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kr[blk][ds]),
                                                                       qf[hb][ds], acc, 0, 0, 0);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = tw0 + ci * kChunk + 16 * blk + 4 * q4 + r;
                        s[blk][r] = key < tw1 ? acc[r] : -INFINITY;
                    }
                }
                float tmax = s[0][0];
#pragma unroll
                for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, s[blk][r]);
                tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * scale_log2;
                const bool raise = tmax > ref[hb] + kRescaleSlack;
                if (__builtin_amdgcn_ballot_w64(raise)) {      // wavefront-uniform branch
                    const float ref_new = raise ? tmax : ref[hb];
                    const float alpha = exp2_fast(ref[hb] - ref_new);
                    ref[hb] = ref_new;
                    lsum[hb] *= alpha;
#pragma unroll
                    for (int j = 0; j < 8; ++j) oacc[hb][j] *= alpha;
                }
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        p[r] = exp2_fast(fmaf(s[blk][r], scale_log2, -ref[hb]));
                        lsum[hb] += p[r];
                    }
                    u32x2 w;
                    w.x = pack_bf16x2(p[0], p[1]);
                    w.y = pack_bf16x2(p[2], p[3]);
                    pf[hb][blk] = __builtin_bit_cast(bf16x4, w);
                }
            }
            // O^T += V^T . P^T; MFMA j covers d = 8*m + j.
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int dw = j >> 1;
                    u32x2 a;
                    if (j & 1) {
                        a.x = pack_hi16(vr[blk][0][dw], vr[blk][1][dw]);
                        a.y = pack_hi16(vr[blk][2][dw], vr[blk][3][dw]);
                    } else {
                        a.x = pack_lo16(vr[blk][0][dw], vr[blk][1][dw]);
                        a.y = pack_lo16(vr[blk][2][dw], vr[blk][3][dw]);
                    }
                    const bf16x4 av = __builtin_bit_cast(bf16x4, a);
#pragma unroll
                    for (int hb = 0; hb < NHB; ++hb)
                        oacc[hb][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pf[hb][blk], oacc[hb][j], 0, 0, 0);
                }
            }
        };

        Buf ka, va, kb, vb;
        wait_all_memory();             // q fragments and table entries are in registers
        load(ka, va, 0);
        // Loads are issued even for chunks past the end (zero-length buffer
        // resources: no memory traffic) so that no branch changes the count of
        // loads in flight and the waits before each process() stay exact.
        for (int ci = 0; ci < nchunks; ci += 2) {
            load(kb, vb, ci + 1);
            process(ka, va, ci);
            load(ka, va, ci + 2);
            if (ci + 1 < nchunks) process(kb, vb, ci + 1);
        }
        // Each lane summed its own keys; the four lanes of a head share its reference.
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            lsum[hb] += __shfl_xor(lsum[hb], 16, 64);
            lsum[hb] += __shfl_xor(lsum[hb], 32, 64);
        }
    }

    // Publish this wavefront's state.  Lane holds head hb*16 + c, d = 32*q4 + 8*r + j.
#pragma unroll
    for (int hb = 0; hb < NHB; ++hb) {
        if (q4 == 0) {
            sm[wave][hb * 16 + c] = ref[hb];
            sl[wave][hb * 16 + c] = lsum[hb];
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
        const size_t row = ((size_t)b * Hq + hk * g + hl) * ns + split;
        opart[row * kD + dd] = num / den;
        if (dd == 0) lsepart[row] = M + __builtin_amdgcn_logf(den);   // v_log_f32: log2
    }
}

// One wavefront per (query head, sequence); lane owns d = 2*lane, 2*lane+1.
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart,
    const int32_t* __restrict__ seq_lens, uint16_t* __restrict__ o, int Hq, int ns_max, int T) {
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int L = seq_lens[b];
    const int ns = (L + T - 1) / T;
    const size_t row0 = ((size_t)b * Hq + hq) * ns_max;
    float o0 = 0.f, o1 = 0.f;
    if (ns > 0) {
        float M = -INFINITY;
        for (int s = lane; s < ns; s += 64) M = fmaxf(M, lsepart[row0 + s]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
        float den = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll 8
        for (int s = 0; s < ns; ++s) {
            const float w = exp2_fast(lsepart[row0 + s] - M);
            const float2 x = *reinterpret_cast<const float2*>(opart + (row0 + s) * kD + 2 * lane);
            den += w;
            a0 += w * x.x;
            a1 += w * x.y;
        }
        o0 = a0 / den;
        o1 = a1 / den;
    }
    reinterpret_cast<uint32_t*>(o + ((size_t)b * Hq + hq) * kD)[lane] = pack_bf16x2(o0, o1);
}

// Split size: the largest power of two in [kDecodeSplitMin, kDecodeSplitMax]
// that still gives about kTargetWorkgroups workgroups for the longest
// sequences; large query groups (whose partials cost more) use at least 512.
constexpr long kTargetWorkgroups = 4096;

int choose_split(int B, int Hkv, int g, int max_seq_len) {
    int T = g >= 16 ? 2 * kDecodeSplitMin : kDecodeSplitMin;
    while (T < kDecodeSplitMax &&
           (long)B * Hkv * decode_nsplit(max_seq_len, 2 * T) >= kTargetWorkgroups)
        T *= 2;
    return T;
}

template <int NHB, class Rows>
void launch_split(const DecodeArgs& a, const Rows& rows, hipStream_t stream, float* opart, float* lsepart, int ns,
                  int T) {
    dim3 grid(ns, a.Hkv, a.B);
    hipLaunchKernelGGL((decode_split_kernel<NHB, Rows>), grid, dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), rows, a.seq_lens, opart, lsepart, a.Hq, a.Hq / a.Hkv, ns,
                       T, a.scale * kLog2e);
}

template <class Rows>
void launch_split_any(const DecodeArgs& a, const Rows& rows, hipStream_t stream, float* opart, float* lsepart,
                      int ns, int T) {
    if (a.Hq / a.Hkv <= 16)
        launch_split<1>(a, rows, stream, opart, lsepart, ns, T);
    else
        launch_split<2>(a, rows, stream, opart, lsepart, ns, T);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const int g = a.Hq / a.Hkv;
    const int T = choose_split(a.B, a.Hkv, g, a.max_seq_len);
    const int ns = decode_nsplit(a.max_seq_len, T);
    float* opart = static_cast<float*>(a.workspace);
    float* lsepart = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                              align256((size_t)a.B * a.Hq * ns * kD * 4));
    const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
    if (a.block_table)
        launch_split_any(a, PagedRows{kc, vc, a.block_table, a.Hkv, a.max_blocks_per_seq}, stream, opart, lsepart,
                         ns, T);
    else
        launch_split_any(a, ContiguousRows{kc, vc, a.Hkv, a.max_seq_len}, stream, opart, lsepart, ns, T);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(64), 0, stream, opart, lsepart, a.seq_lens,
                       static_cast<uint16_t*>(a.o), a.Hq, ns, T);
    return hipGetLastError();
}

}  // namespace gqa
