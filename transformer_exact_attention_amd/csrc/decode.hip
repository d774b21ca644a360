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
// heads of the group).  The wavefront streams 32-token chunks, double-buffered
// across its whole share: chunk i+1 is loaded (non-temporal, range-checked
// buffer loads, no branches) while chunk i is computed, and the next piece's
// first chunk and Q fragments are fetched while the current piece finishes;
// an online softmax runs across the chunks of a piece.  Per 16-token block:
//   S^T (16 keys x 16 heads) = K (16 x d) . Q^T (d x 16)    v_mfma_f32_16x16x32_bf16
//   O^T (d x 16 heads)      += V^T (d x 16 keys) . P^T      v_mfma_f32_16x16x16_bf16
// Lane i (c = i%16, q4 = i/16) loads K row c of the block (contraction over d)
// and V rows 4*q4..4*q4+3 at d-chunk c.  For the PV product the 16 "rows" of
// MFMA j are d = 8*m + j, m = 0..15, so each lane's own V rows supply its A
// operand with one byte permute per dword and the S^T accumulator already is
// the P^T operand: no LDS traffic, no cross-lane traffic.
//
// Kernel 2 (combine): per (sequence, query head) finds the partials of its
// segment from the same share arithmetic and merges them in one pass with a
// running maximum, weights 2^(lse_s - max), the rescale step of the tiled
// online softmax [Attention variants deep-dive, §6.2 forward pseudocode]
// applied across pieces, and writes bf16.  Fixed work assignment and reduction order: results
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

// A 64-bit value the compiler cannot prove wavefront-uniform (it came from
// LDS) made uniform explicitly, so what derives from it stays scalar.
__device__ __forceinline__ long long uniform64(long long x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((unsigned long long)x >> 32));
    return (long long)(((unsigned long long)hi << 32) | lo);
}

// Q tokens per wavefront share: W / NW rounded up to 16, at least kDecodeMinShare.
__device__ __forceinline__ long long share_tokens(long long W, long long NW) {
    long long q = (W + NW - 1) / NW;
    q = (q + 15) & ~15ll;
    return q < kDecodeMinShare ? kDecodeMinShare : q;
}

// Row addressing: index of the row holding token t0 (t0 % 16 == 0) of K/V
// head hk of sequence b; the 16 rows of a block follow each other in both
// layouts, and the per-row scales of an fp8 cache are indexed by the same
// row number.
struct ContiguousRows {
    const char* kbase;           // [B, Hkv, S_max, d] elements
    const char* vbase;
    const float* kscale;         // fp8 caches: [B, Hkv, S_max]
    const float* vscale;
    int Hkv, S_max;
    __device__ __forceinline__ int lookup(const int32_t*, int, int) const { return 0; }
    __device__ __forceinline__ size_t row(int, int b, int hk, int t0) const {
        return ((size_t)b * Hkv + hk) * S_max + t0;
    }
};

struct PagedRows {
    const char* kbase;           // pages [num_blocks, Hkv, 16, d]
    const char* vbase;
    const float* kscale;         // fp8 caches: [num_blocks, Hkv, 16]
    const float* vscale;
    int Hkv, max_blocks;
    // Physical block of logical block blk of sequence b, from the block table
    // [B, max_blocks] (a separate restrict kernel argument, so this uniform
    // read is a scalar load whose wait does not drain the vector loads).
    __device__ __forceinline__ int lookup(const int32_t* __restrict__ table, int b, int blk) const {
        return table[(size_t)b * max_blocks + blk];
    }
    __device__ __forceinline__ size_t row(int phys, int, int hk, int) const {
        return ((size_t)phys * Hkv + hk) * 16;
    }
};

// Cache element formats.  bf16: rows of d bf16 values.  fp8: rows of d E4M3
// codes (OCP: sign, 4 exponent bits with bias 7, 3 mantissa bits) with one
// fp32 scale per row, standing for code * scale [Attention variants
// deep-dive, §7 KV Cache: fp16 -> fp8 halves the cache].  Every E4M3 value is
// exactly a bf16, so the fp8 rows are widened to bf16 operands of the same
// MFMAs; a key's scale multiplies its score, a value row's scale multiplies
// its probability in the P.V product (not in the row sum).
struct Bf16Kv {
    static constexpr bool kFp8 = false;
    static constexpr int kRowBytes = kD * 2;
    struct KBuf { u32x4 r[2][4]; };                  // [block][d-step]
    struct VBuf { u32x4 r[2][4]; };                  // [block][row]
};
struct Fp8Kv {
    static constexpr bool kFp8 = true;
    static constexpr int kRowBytes = kD;
    struct KBuf { u32x4 r[2][2]; f32x4 s[2]; };      // 32 codes of row c at d = 32 q4 .., scales of keys 4 q4 ..
    struct VBuf { u32x2 r[2][4]; f32x4 s[2]; };      // 8 codes of rows 4 q4 + rr at d = 8 c .., scales
};

// Eight E4M3 codes (two dwords, element e in byte e) -> eight bf16, exactly
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1: two codes per instruction).
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    return u32x4{__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false)),
                 __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true))};
}

template <int NHB, class Rows, class Fmt>
__global__ __launch_bounds__(kThreads, NHB == 1 ? 2 : 1) void decode_split_kernel(
    const uint16_t* __restrict__ q, Rows rows, const int32_t* __restrict__ table,
    const int32_t* __restrict__ seq_lens, float* __restrict__ opart, float* __restrict__ lsepart, long long* __restrict__ prefix_out,
    int B, int Hq, int g, int P, float scale_log2, int window) {
    __shared__ long long pre[kDecodeMaxBatch + 1];
    __shared__ long long part[kThreads];

    const int tid = threadIdx.x;
    const int Hkv = Hq / g;

    // Token prefix sums over sequences: pre[b] = sum of L_b' for b' < b,
    // where a sliding window (window > 0) keeps only a sequence's last
    // `window` tokens: its segment is tokens [L - min(L, window), L).
    {
        const int per = (B + kThreads - 1) / kThreads;
        const int lo = min(B, tid * per), hi = min(B, lo + per);
        long long acc = 0;
        for (int i = lo; i < hi; ++i) {
            acc += window > 0 ? min(seq_lens[i], window) : seq_lens[i];
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

    const long long W = uniform64(pre[B] * Hkv);
    const long long NW = (long long)gridDim.x * kWaves;
    const long long Q = share_tokens(W, NW);
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int c = lane & 15;
    const int q4 = lane >> 4;
    const long long w = (long long)blockIdx.x * kWaves + wave;
    const long long start = w * Q;
    const long long end = min(start + Q, W);

    typedef typename Fmt::KBuf KBuf;
    typedef typename Fmt::VBuf VBuf;
    if (start >= end) return;

    // A piece: the part of one segment (b, hk) inside this wavefront's share,
    // tokens [p0, p1) of the segment, streamed as 32-token chunks from the
    // 16-aligned token c0.  Everything in it is wavefront-uniform
    // (readfirstlane makes that explicit, so table lookups are scalar loads).
    struct Piece {
        int b, hk, p0, p1, slot, c0, nchunks;
        long long next;                     // flattened position after the piece
    };
    auto describe = [&](long long pos) {
        // segment holding pos: largest b with pre[b]*Hkv <= pos
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] * Hkv <= pos) lo = mid; else hi = mid - 1;
        }
        Piece p;
        p.b = __builtin_amdgcn_readfirstlane(lo);
        const int L = __builtin_amdgcn_readfirstlane((int)(pre[p.b + 1] - pre[p.b]));
        const long long seg0 = uniform64(pre[p.b] * Hkv);
        p.hk = __builtin_amdgcn_readfirstlane((int)((pos - seg0) / L));
        const long long S = seg0 + (long long)p.hk * L;               // segment start
        // first cached token of the segment (window: the sequence's last L tokens)
        const int t_first = window > 0 ? __builtin_amdgcn_readfirstlane(seq_lens[p.b]) - L : 0;
        const int p1 = __builtin_amdgcn_readfirstlane((int)(min(end, S + L) - S));
        p.p0 = t_first + __builtin_amdgcn_readfirstlane((int)(pos - S));
        p.p1 = t_first + p1;
        p.slot = __builtin_amdgcn_readfirstlane((int)(w - S / Q));  // partial index in the segment
        p.c0 = p.p0 & ~15;
        p.nchunks = (p.p1 - p.c0 + kChunk - 1) / kChunk;            // >= 1
        p.next = S + p1;
        return p;
    };
    const Piece none = {0, 0, 0, 0, 0, 0, 0, end};                  // loads nothing

    // Q^T operand: lane holds Q[head hb*16 + c][32*ds + 8*q4 .. +8] (fp8
    // caches: Q[..][32*q4 + 8*ds .. +8], the order a lane's 32 contiguous K
    // codes come in; any order of the contraction gives the same dot
    // product, Q and K only have to agree).  Columns
    // of heads >= g repeat the group's first head (their results are never
    // written; every column of the MFMAs is independent), so the loads need
    // no branch.
    auto load_q = [&](bf16x8 (&qf)[NHB][4], const Piece& p) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const int hl = hb * 16 + c;
            const uint16_t* qp = q + ((size_t)p.b * Hq + p.hk * g + (hl < g ? hl : 0)) * kD;
#pragma unroll
            for (int ds = 0; ds < 4; ++ds)
                qf[hb][ds] = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4*>(qp + (Fmt::kFp8 ? 32 * q4 + 8 * ds : 32 * ds + 8 * q4)));
        }
    };

    // Chunk x of the stream seen from piece cur, whose chunks are processed in
    // pairs: with ne = nchunks rounded up to even, x < nchunks is cur's own
    // chunk, nchunks <= x < ne an empty slot, x == ne the next piece's chunk 0
    // (prefetched while cur finishes) and x == ne + 1 the next piece's chunk 1
    // (table entries only).  A piece therefore always starts with its chunk 0
    // in buffer A.
    struct Src {
        int b, hk, c0, p1, ci;
    };
    auto src_of = [&](const Piece& cur, const Piece& nxt, int x) {
        const int ne = (cur.nchunks + 1) & ~1;
        const bool own = x < cur.nchunks;
        Src r;
        r.b = own ? cur.b : nxt.b;
        r.hk = own ? cur.hk : nxt.hk;
        r.c0 = own ? cur.c0 : nxt.c0;
        r.p1 = own ? cur.p1 : (x >= ne ? nxt.p1 : 0);
        r.ci = own ? x : (x >= ne ? x - ne : 0);      // empty slot: token 0, nothing valid
        return r;
    };
    // Table entries of a chunk's two blocks, fetched one chunk ahead of the
    // loads that use them.
    auto lookup = [&](int (&ph)[2], const Src& sr) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int t0 = sr.c0 + sr.ci * kChunk + 16 * blk;
            ph[blk] = t0 < sr.p1 ? rows.lookup(table, sr.b, t0 >> 4) : 0;
        }
    };
    // Every load is issued unconditionally through a buffer resource that
    // covers only the block's tokens below p1: the hardware returns zeros
    // beyond it (chunks past the end cost no memory traffic).  With a fixed
    // number of loads per chunk the wait counts stay exact, so the next
    // chunk streams in while the current one is computed.
    auto load = [&](KBuf& kr, VBuf& vr, const int (&ph)[2], const Src& sr) {
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int t0 = sr.c0 + sr.ci * kChunk + 16 * blk;
            // (uniform; kept in scalar registers so the descriptors are too)
            const int nvalid = __builtin_amdgcn_readfirstlane(min(max(sr.p1 - t0, 0), 16));
            const size_t row = nvalid > 0 ? rows.row(ph[blk], sr.b, sr.hk, t0) : 0;
            const __amdgpu_buffer_rsrc_t krs =
                make_rsrc(rows.kbase + row * Fmt::kRowBytes, (uint32_t)nvalid * Fmt::kRowBytes);
            const __amdgpu_buffer_rsrc_t vrs =
                make_rsrc(rows.vbase + row * Fmt::kRowBytes, (uint32_t)nvalid * Fmt::kRowBytes);
            if constexpr (!Fmt::kFp8) {
#pragma unroll
                for (int ds = 0; ds < 4; ++ds)
                    kr.r[blk][ds] = __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (uint32_t)(c * kD + 32 * ds + 8 * q4) * 2, 0, kStreamAux);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vr.r[blk][rr] = __builtin_amdgcn_raw_buffer_load_b128(
                        vrs, (uint32_t)((4 * q4 + rr) * kD + 8 * c) * 2, 0, kStreamAux);
            } else {
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    kr.r[blk][h] = __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (uint32_t)(c * kD + 32 * q4 + 16 * h), 0, kStreamAux);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    vr.r[blk][rr] = __builtin_amdgcn_raw_buffer_load_b64(
                        vrs, (uint32_t)((4 * q4 + rr) * kD + 8 * c), 0, kStreamAux);
                // The scales of all 16 rows of a block with any valid row are
                // read (a block's rows all exist in memory); those of rows past
                // the valid ones are never used: their scores are masked and
                // their probabilities are zero.  An empty block reads nothing.
                const uint32_t sbytes = nvalid > 0 ? 64u : 0u;
                const __amdgpu_buffer_rsrc_t kss = make_rsrc(rows.kscale + row, sbytes);
                const __amdgpu_buffer_rsrc_t vss = make_rsrc(rows.vscale + row, sbytes);
                kr.s[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kss, 16u * q4, 0, 0));
                vr.s[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vss, 16u * q4, 0, 0));
            }
        }
    };

    bf16x8 qf[NHB][4], qn[NHB][4];
    float ref[NHB], lsum[NHB];
    f32x4 oacc[NHB][8];

    auto process = [&](const KBuf& kr, const VBuf& vr, const Piece& cur, int ci) {
        bf16x4 pf[NHB][2];
        // bf16 operands of the chunk: K for each block and d-step, V rows
        // (fp8 codes widened once, for all head blocks).
        u32x4 kop[2][4], vrow[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                if constexpr (!Fmt::kFp8) {
                    kop[blk][x] = kr.r[blk][x];
                    vrow[blk][x] = vr.r[blk][x];
                } else {
                    const u32x4 w = kr.r[blk][x >> 1];
                    kop[blk][x] = (x & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
                    vrow[blk][x] = fp8x8_to_bf16x8(vr.r[blk][x][0], vr.r[blk][x][1]);
                }
            }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float s[2][4];
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int ds = 0; ds < 4; ++ds)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kop[blk][ds]),
                                                                   qf[hb][ds], acc, 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int key = cur.c0 + ci * kChunk + 16 * blk + 4 * q4 + r;
                    float sc = acc[r];
                    if constexpr (Fmt::kFp8) sc *= kr.s[blk][r];
                    s[blk][r] = (key >= cur.p0 && key < cur.p1) ? sc : -INFINITY;
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
                    // fp8: the value row's scale (a masked row's p is 0 and its
                    // scale is never read as a number)
                    if constexpr (Fmt::kFp8) p[r] = p[r] > 0.f ? p[r] * vr.s[blk][r] : 0.f;
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
                    a.x = pack_hi16(vrow[blk][0][dw], vrow[blk][1][dw]);
                    a.y = pack_hi16(vrow[blk][2][dw], vrow[blk][3][dw]);
                } else {
                    a.x = pack_lo16(vrow[blk][0][dw], vrow[blk][1][dw]);
                    a.y = pack_lo16(vrow[blk][2][dw], vrow[blk][3][dw]);
                }
                const bf16x4 av = __builtin_bit_cast(bf16x4, a);
#pragma unroll
                for (int hb = 0; hb < NHB; ++hb)
                    oacc[hb][j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pf[hb][blk], oacc[hb][j], 0, 0, 0);
            }
        }
    };

    // Finish a piece: each lane summed its own keys; the four lanes of a head
    // share its reference.  Lane holds head hb*16 + c, d = 32*q4 + 8*r + j.
    auto finish = [&](const Piece& cur) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float lt = lsum[hb] + __shfl_xor(lsum[hb], 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            const int hl = hb * 16 + c;
            if (hl < g) {
                const size_t row = ((size_t)cur.b * Hq + cur.hk * g + hl) * P + cur.slot;
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
    };

    // Two chunk buffers (chunk x of a piece in buffer x % 2) with their table
    // entries.
    KBuf ka, kb;
    VBuf va, vb;
    int pha[2], phb[2];
    auto pair = [&](const Piece& cur, const Piece& nxt, int ci, bool last) {
        lookup(pha, src_of(cur, nxt, ci + 2));
        load(kb, vb, phb, src_of(cur, nxt, ci + 1));
        process(ka, va, cur, ci);
        lookup(phb, src_of(cur, nxt, ci + 3));
        // The last pair also fetches the next piece's Q fragments (into qn)
        // with its chunk 0, in straight-line code after the loop, so the wait
        // before qf takes them over counts only what follows.
        if (last) load_q(qn, nxt);
        load(ka, va, pha, src_of(cur, nxt, ci + 2));
        if (ci + 1 < cur.nchunks) process(kb, vb, cur, ci + 1);
    };

    Piece cur = describe(start);
    load_q(qf, cur);
    lookup(pha, src_of(cur, none, 0));
    lookup(phb, src_of(cur, none, 1));
    load(ka, va, pha, src_of(cur, none, 0));
    for (;;) {
        const bool more = cur.next < end;
        const Piece nxt = more ? describe(cur.next) : none;   // none: q of head 0, no K/V
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            ref[hb] = -INFINITY;
            lsum[hb] = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) oacc[hb][j] = f32x4{};
        }
        const int last = ((cur.nchunks + 1) & ~1) - 2;
        for (int ci = 0; ci < last; ci += 2) pair(cur, nxt, ci, false);
        pair(cur, nxt, last, true);
        finish(cur);
        if (!more) break;
        cur = nxt;
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb)
#pragma unroll
            for (int ds = 0; ds < 4; ++ds) qf[hb][ds] = qn[hb][ds];
    }
}

// One workgroup of kCombineWaves wavefronts per (query head, sequence); lane
// owns d = 2*lane, 2*lane+1.  Wavefront w merges partials w, w + kCombineWaves,
// ... in one pass with a running maximum (the rescale step of the tiled
// online softmax), issuing the loads of several partials at once; the
// wavefronts' results are then merged in LDS in a fixed order.  With few
// partials per row (short caches) one wavefront per row does it all.
constexpr int kCombineBatch = 4;         // partials in flight per wavefront
constexpr int kCombineFewPartials = 32;  // at most this many per row: one wavefront

template <int kCombineWaves>
__global__ __launch_bounds__(64 * kCombineWaves) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart, const long long* __restrict__ prefix,
    uint16_t* __restrict__ o, int B, int Hq, int g, int P, long long NW) {
    __shared__ float red[kCombineWaves][2][64 + 1];
    __shared__ float red_m[kCombineWaves], red_den[kCombineWaves];
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int Hkv = Hq / g;
    const long long L = prefix[b + 1] - prefix[b];
    float m = -INFINITY, den = 0.f, a0 = 0.f, a1 = 0.f;
    if (L > 0) {
        const long long W = prefix[B] * Hkv;
        const long long Q = share_tokens(W, NW);
        const long long S = prefix[b] * Hkv + (long long)(hq / g) * L;
        const int np = (int)((S + L - 1) / Q - S / Q) + 1;
        const size_t row0 = ((size_t)b * Hq + hq) * P;
        for (int s0 = wave; s0 < np; s0 += kCombineWaves * kCombineBatch) {
            float x[kCombineBatch];
            float2 v[kCombineBatch];
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const int s = s0 + u * kCombineWaves;
                const int sc = s < np ? s : np - 1;
                x[u] = s < np ? lsepart[row0 + sc] : -INFINITY;
                v[u] = *reinterpret_cast<const float2*>(opart + (row0 + sc) * kD + 2 * lane);
            }
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const float mn = fmaxf(m, x[u]);
                const float sc = mn == m ? 1.f : exp2_fast(m - mn);
                const float wgt = x[u] == -INFINITY ? 0.f : exp2_fast(x[u] - mn);
                den = den * sc + wgt;
                a0 = a0 * sc + wgt * v[u].x;
                a1 = a1 * sc + wgt * v[u].y;
                m = mn;
            }
        }
    }
    red[wave][0][lane] = a0;
    red[wave][1][lane] = a1;
    if (lane == 0) {
        red_m[wave] = m;
        red_den[wave] = den;
    }
    __syncthreads();
    if (wave == 0) {
        float M = red_m[0];
#pragma unroll
        for (int w = 1; w < kCombineWaves; ++w) M = fmaxf(M, red_m[w]);
        float dt = 0.f, o0 = 0.f, o1 = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kCombineWaves; ++w) {
                const float f = red_m[w] == -INFINITY ? 0.f : exp2_fast(red_m[w] - M);
                dt += f * red_den[w];
                o0 += f * red[w][0][lane];
                o1 += f * red[w][1][lane];
            }
            o0 /= dt;
            o1 /= dt;
        }
        reinterpret_cast<uint32_t*>(o + ((size_t)b * Hq + hq) * kD)[lane] = pack_bf16x2(o0, o1);
    }
}

template <int NHB, class Fmt, class Rows>
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
    hipLaunchKernelGGL((decode_split_kernel<NHB, Rows, Fmt>), dim3(nwg), dim3(kThreads), 0, stream,
                       static_cast<const uint16_t*>(a.q), rows, a.block_table, a.seq_lens, opart, lsepart, prefix, a.B,
                       a.Hq, g, P,
                       a.scale * kLog2e, a.window > 0 ? a.window : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (P <= kCombineFewPartials)
        hipLaunchKernelGGL(decode_combine_kernel<1>, dim3(a.Hq, a.B), dim3(64), 0, stream, opart, lsepart, prefix,
                           static_cast<uint16_t*>(a.o), a.B, a.Hq, g, P, (long long)nwg * kWaves);
    else
        hipLaunchKernelGGL(decode_combine_kernel<4>, dim3(a.Hq, a.B), dim3(256), 0, stream, opart, lsepart, prefix,
                           static_cast<uint16_t*>(a.o), a.B, a.Hq, g, P, (long long)nwg * kWaves);
    return hipGetLastError();
}

template <class Fmt, class Rows>
hipError_t launch_rows(const DecodeArgs& a, const Rows& rows, hipStream_t stream) {
    return a.Hq / a.Hkv <= 16 ? launch_both<1, Fmt>(a, rows, stream) : launch_both<2, Fmt>(a, rows, stream);
}

template <class Fmt>
hipError_t launch_fmt(const DecodeArgs& a, hipStream_t stream) {
    const char* kc = static_cast<const char*>(a.k_cache);
    const char* vc = static_cast<const char*>(a.v_cache);
    if (a.block_table)
        return launch_rows<Fmt>(a, PagedRows{kc, vc, a.k_scale, a.v_scale, a.Hkv, a.max_blocks_per_seq}, stream);
    return launch_rows<Fmt>(a, ContiguousRows{kc, vc, a.k_scale, a.v_scale, a.Hkv, a.max_seq_len}, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) { return launch_fmt<Bf16Kv>(a, stream); }

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) { return launch_fmt<Fp8Kv>(a, stream); }

}  // namespace gqa
