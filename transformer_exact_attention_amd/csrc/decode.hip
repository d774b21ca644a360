// Decode attention over a KV cache: balanced split-KV partials + log-sum-exp combine.
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
// Kernel 1 (split).  The flattened space of W = Hkv * sum_b L_b (sequence,
// K/V head, token) triples is cut into equal consecutive shares of Q tokens,
// one per wavefront, and exactly as many wavefronts are launched as the GPU
// holds at once: every wavefront streams the same number of bytes, whatever
// the length mix.  A share crossing segment boundaries (a segment = one K/V
// head of one sequence) is processed piece by piece; each piece ends in one
// partial result (normalised output + base-2 log-sum-exp for the g query
// heads of the group).  Within a piece the wavefront streams 32-token chunks,
// double-buffered: chunk i+1 is loaded (non-temporal, range-checked buffer
// loads, no branches) while chunk i is computed; an online softmax runs across
// chunks.  Per 16-token block:
//   S^T (16 keys x 16 heads) = K (16 x d) . Q^T (d x 16)    v_mfma_f32_16x16x32_bf16
//   O^T (d x 16 heads)      += V^T (d x 16 keys) . P^T      v_mfma_f32_16x16x16_bf16
// Lane i (c = i%16, q4 = i/16) loads K row c of the block (contraction over d)
// and V rows 4*q4..4*q4+3 at d-chunk c.  For the PV product the 16 "rows" of
// MFMA j are d = 8*m + j, m = 0..15, so each lane's own V rows supply its A
// operand with one byte permute per dword and the S^T accumulator already is
// the P^T operand: no LDS traffic, no cross-lane traffic.
//
// Kernel 2 (combine): per (sequence, query head) finds the partials of its
// segment from the same share arithmetic and merges them with weights
// 2^(lse_s - max lse), the rescale step of the tiled online softmax
// [Attention variants deep-dive, §6.2 forward pseudocode] applied across
// pieces, and writes bf16.  Fixed work assignment and reduction order: results
// are bitwise reproducible, and paged == contiguous bitwise for equal contents.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kD = 128;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int kChunk = 32;               // tokens per pipeline stage (two 16-token blocks)
constexpr float kRescaleSlack = 8.0f;    // base-2 units, as in the prefill kernel
constexpr int kStreamAux = 2;            // non-temporal loads: every K/V byte is read once

// Q tokens per wavefront share: W / NW rounded up to 16, at least kDecodeMinShare.
__device__ __forceinline__ long long share_tokens(long long W, long long NW) {
    long long q = (W + NW - 1) / NW;
    q = (q + 15) & ~15ll;
    return q < kDecodeMinShare ? kDecodeMinShare : q;
}

// Row addressing: element offset of the 16 tokens t0..t0+15 (t0 % 16 == 0) of
// K/V head hk of sequence b; the 16 rows follow each other in both layouts.
struct ContiguousRows {
    const uint16_t* kbase;
    const uint16_t* vbase;
    int Hkv, S_max;
    __device__ __forceinline__ int lookup(const int32_t*, int, int) const { return 0; }
    __device__ __forceinline__ size_t offset(int, int b, int hk, int t0) const {
        return (((size_t)b * Hkv + hk) * S_max + t0) * kD;
    }
};

struct PagedRows {
    const uint16_t* kbase;       // pages [num_blocks, Hkv, 16, d]
    const uint16_t* vbase;
    int Hkv, max_blocks;
    // Physical block of logical block blk of sequence b, from the block table
    // [B, max_blocks] (a separate restrict kernel argument, so this uniform
    // read is a scalar load whose wait does not drain the vector loads).
    __device__ __forceinline__ int lookup(const int32_t* __restrict__ table, int b, int blk) const {
        return table[(size_t)b * max_blocks + blk];
    }
    __device__ __forceinline__ size_t offset(int phys, int, int hk, int) const {
        return ((size_t)phys * Hkv + hk) * 16 * kD;
    }
};

template <int NHB, class Rows>
__global__ __launch_bounds__(kThreads, NHB == 1 ? 2 : 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, Rows rows, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ opart, float* __restrict__ lsepart, long long* __restrict__ prefix_out,
    int B, int Hq, int g, int P, float scale_log2) {
    __shared__ long long pre[kDecodeMaxBatch + 1];
    __shared__ long long part[kThreads];

    const int tid = threadIdx.x;
    const int Hkv = Hq / g;

    // Token prefix sums over sequences: pre[b] = sum of L_b' for b' < b.
    {
        const int per = (B + kThreads - 1) / kThreads;
        const int lo = min(B, tid * per), hi = min(B, lo + per);
        long long acc = 0;
        for (int i = lo; i < hi; ++i) {
            acc += seq_lens[i];
            pre[i + 1] = acc;
        }
        part[tid] = acc;
        __syncthreads();
        for (int step = 1; step < kThreads; step <<= 1) {          // inclusive scan of the thread sums
            const long long x = tid >= step ? part[tid - step] : 0;
            __syncthreads();
            part[tid] += x;
            __syncthreads();
        }
        const long long base = tid > 0 ? part[tid - 1] : 0;
        for (int i = lo; i < hi; ++i) pre[i + 1] += base;
        if (tid == 0) pre[0] = 0;
        __syncthreads();
        if (blockIdx.x == 0)
            for (int i = tid; i <= B; i += kThreads) prefix_out[i] = pre[i];
    }

    const long long W = pre[B] * Hkv;
    const long long NW = (long long)gridDim.x * kWaves;
    const long long Q = share_tokens(W, NW);
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int c = lane & 15;
    const int q4 = lane >> 4;
    const long long w = (long long)blockIdx.x * kWaves + wave;
    const long long start = w * Q;
    const long long end = min(start + Q, W);

    typedef u32x4 Buf[2][4];

    for (long long pos = start; pos < end;) {
        // Segment (b, hk) holding flattened position pos: largest b with pre[b]*Hkv <= pos.
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] * Hkv <= pos) lo = mid; else hi = mid - 1;
        }
        // Everything describing the piece is wavefront-uniform; readfirstlane
        // makes that explicit, so table lookups become scalar loads.
        const int b = __builtin_amdgcn_readfirstlane(lo);
        const int L = __builtin_amdgcn_readfirstlane((int)(pre[b + 1] - pre[b]));
        const long long seg0 = pre[b] * Hkv;
        const int hk = __builtin_amdgcn_readfirstlane((int)((pos - seg0) / L));
        const long long S = seg0 + (long long)hk * L;                 // segment start
        const int p0 = __builtin_amdgcn_readfirstlane((int)(pos - S));
        const int p1 = __builtin_amdgcn_readfirstlane((int)(min(end, S + L) - S));   // piece: tokens [p0, p1)
        const int slot = __builtin_amdgcn_readfirstlane((int)(w - S / Q));          // partial index in the segment
        pos = S + p1;

        // Q^T operand: lane holds Q[head hb*16 + c][32*ds + 8*q4 .. +8] (zero for heads >= g).
        bf16x8 qf[NHB][4];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const int hl = hb * 16 + c;
            const bool hv = hl < g;
            const uint16_t* qp = q + ((size_t)b * Hq + hk * g + (hv ? hl : 0)) * kD;
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) {
                u32x4 x = {0u, 0u, 0u, 0u};
                if (hv) x = *reinterpret_cast<const u32x4*>(qp + 32 * ds + 8 * q4);
                qf[hb][ds] = __builtin_bit_cast(bf16x8, x);
            }
        }

        float ref[NHB], lsum[NHB];
        f32x4 oacc[NHB][8];
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            ref[hb] = -INFINITY;
            lsum[hb] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) oacc[hb][j] = f32x4{};
        }

        const int c0 = p0 & ~15;                                   // first 16-aligned block
        const int nchunks = (p1 - c0 + kChunk - 1) / kChunk;       // >= 1

        // Table entries of a chunk's two blocks (wavefront-uniform scalar loads),
        // fetched one chunk ahead of the loads that use them.
        auto lookup = [&](int (&ph)[2], int ci) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int t0 = c0 + ci * kChunk + 16 * blk;
                ph[blk] = t0 < p1 ? rows.lookup(table, b, t0 >> 4) : 0;
            }
        };
        // Every load is issued unconditionally through a buffer resource that
        // covers only the block's tokens below p1: the hardware returns zeros
        // beyond it (chunks past the end cost no memory traffic).  With a fixed
        // number of loads per chunk the wait counts stay exact, so chunk i+1
        // streams in while chunk i is computed.
        auto load = [&](Buf& kr, Buf& vr, const int (&ph)[2], int ci) {
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                const int t0 = c0 + ci * kChunk + 16 * blk;
                // (uniform; kept in scalar registers so the descriptors are too)
                const int nvalid = __builtin_amdgcn_readfirstlane(min(max(p1 - t0, 0), 16));
                const size_t off = nvalid > 0 ? rows.offset(ph[blk], b, hk, t0) : 0;
                const __amdgpu_buffer_rsrc_t krs = make_rsrc(rows.kbase + off, (uint32_t)nvalid * kD * 2);
                const __amdgpu_buffer_rsrc_t vrs = make_rsrc(rows.vbase + off, (uint32_t)nvalid * kD * 2);
#pragma unroll
                for (int ds = 0; ds < 4; ++ds)
                    kr[blk][ds] = __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (uint32_t)(c * kD + 32 * ds + 8 * q4) * 2, 0, kStreamAux);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vr[blk][rr] = __builtin_amdgcn_raw_buffer_load_b128(
                        vrs, (uint32_t)((4 * q4 + rr) * kD + 8 * c) * 2, 0, kStreamAux);
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
                        const int key = c0 + ci * kChunk + 16 * blk + 4 * q4 + r;
                        s[blk][r] = (key >= p0 && key < p1) ? acc[r] : -INFINITY;
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
                    u32x2 x;
                    x.x = pack_bf16x2(p[0], p[1]);
                    x.y = pack_bf16x2(p[2], p[3]);
                    pf[hb][blk] = __builtin_bit_cast(bf16x4, x);
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
        int pha[2], phb[2];
        lookup(pha, 0);
        lookup(phb, 1);
        wait_all_memory();             // q fragments and table entries are in registers
        load(ka, va, pha, 0);
        for (int ci = 0; ci < nchunks; ci += 2) {
            lookup(pha, ci + 2);
            load(kb, vb, phb, ci + 1);
            process(ka, va, ci);
            lookup(phb, ci + 3);
            load(ka, va, pha, ci + 2);
            if (ci + 1 < nchunks) process(kb, vb, ci + 1);
        }

        // Finish the piece: each lane summed its own keys; the four lanes of a
        // head share its reference.  Lane holds head hb*16 + c, d = 32*q4 + 8*r + j.
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float lt = lsum[hb] + __shfl_xor(lsum[hb], 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            const int hl = hb * 16 + c;
            if (hl < g) {
                const size_t row = ((size_t)b * Hq + hk * g + hl) * P + slot;
                const float inv = 1.f / lt;
                float* dst = opart + row * kD + 32 * q4;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    f32x4 lo = {oacc[hb][0][r] * inv, oacc[hb][1][r] * inv, oacc[hb][2][r] * inv, oacc[hb][3][r] * inv};
                    f32x4 hi = {oacc[hb][4][r] * inv, oacc[hb][5][r] * inv, oacc[hb][6][r] * inv, oacc[hb][7][r] * inv};
                    *reinterpret_cast<f32x4*>(dst + 8 * r) = lo;
                    *reinterpret_cast<f32x4*>(dst + 8 * r + 4) = hi;
                }
                if (q4 == 0) lsepart[row] = ref[hb] + __builtin_amdgcn_logf(lt);   // v_log_f32: log2
            }
        }
    }
}

// One wavefront per (query head, sequence); lane owns d = 2*lane, 2*lane+1.
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart, const long long* __restrict__ prefix,
    uint16_t* __restrict__ o, int B, int Hq, int g, int P, long long NW) {
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int Hkv = Hq / g;
    const long long L = prefix[b + 1] - prefix[b];
    float o0 = 0.f, o1 = 0.f;
    if (L > 0) {
        const long long W = prefix[B] * Hkv;
        const long long Q = share_tokens(W, NW);
        const long long S = prefix[b] * Hkv + (long long)(hq / g) * L;
        const int np = (int)((S + L - 1) / Q - S / Q) + 1;
        const size_t row0 = ((size_t)b * Hq + hq) * P;
        float M = -INFINITY;
        for (int s = lane; s < np; s += 64) M = fmaxf(M, lsepart[row0 + s]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
        float den = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll 8
        for (int s = 0; s < np; ++s) {
            const float wgt = exp2_fast(lsepart[row0 + s] - M);
            const float2 x = *reinterpret_cast<const float2*>(opart + (row0 + s) * kD + 2 * lane);
            den += wgt;
            a0 += wgt * x.x;
            a1 += wgt * x.y;
        }
        o0 = a0 / den;
        o1 = a1 / den;
    }
    reinterpret_cast<uint32_t*>(o + ((size_t)b * Hq + hq) * kD)[lane] = pack_bf16x2(o0, o1);
}

template <int NHB, class Rows>
hipError_t launch_both(const DecodeArgs& a, const Rows& rows, hipStream_t stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    const int nwg = cus * (NHB == 1 ? 2 : 1);                      // every workgroup resident at once
    const DecodeWorkspace ws = decode_workspace_layout(a.B, a.Hq, kD, a.max_seq_len);
    char* base = static_cast<char*>(a.workspace);
    float* opart = reinterpret_cast<float*>(base + ws.part_o);
    float* lsepart = reinterpret_cast<float*>(base + ws.part_lse);
    long long* prefix = reinterpret_cast<long long*>(base + ws.prefix);
    const int P = decode_max_partials(a.max_seq_len);
    const int g = a.Hq / a.Hkv;
    hipLaunchKernelGGL((decode_split_kernel<NHB, Rows>), dim3(nwg), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), rows, a.block_table, a.seq_lens, opart, lsepart, prefix, a.B,
                       a.Hq, g, P,
                       a.scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_combine_kernel, dim3(a.Hq, a.B), dim3(64), 0, stream, opart, lsepart, prefix,
                       static_cast<uint16_t*>(a.o), a.B, a.Hq, g, P, (long long)nwg * kWaves);
    return hipGetLastError();
}

template <class Rows>
hipError_t launch_rows(const DecodeArgs& a, const Rows& rows, hipStream_t stream) {
    return a.Hq / a.Hkv <= 16 ? launch_both<1>(a, rows, stream) : launch_both<2>(a, rows, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    const uint16_t* kc = static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vc = static_cast<const uint16_t*>(a.v_cache);
    if (a.block_table)
        return launch_rows(a, PagedRows{kc, vc, a.Hkv, a.max_blocks_per_seq}, stream);
    return launch_rows(a, ContiguousRows{kc, vc, a.Hkv, a.max_seq_len}, stream);
}

}  // namespace gqa
