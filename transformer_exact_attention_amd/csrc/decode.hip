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
// head of one sequence) is processed piece by piece; each piece ends in a
// partial result (normalised output + base-2 log-sum-exp for the g query
// heads of the group), and the pieces a segment has in the four shares of
// one workgroup are merged in LDS, so a segment gets one partial per
// workgroup it meets.  The wavefront streams 32-token chunks, double-buffered
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

#include <mutex>

namespace gqa {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
// Tokens per pipeline stage: 16-token blocks per chunk (two chunks in flight
// per wavefront).  Longer chunks measured no faster: four blocks at g = 32
// (one wavefront per SIMD), three for fp8 caches.
constexpr int kChunkBlocks = 2;
constexpr float kRescaleSlack = 8.0f;    // base-2 units, as in the prefill kernel
constexpr int kStreamAux = 2;            // non-temporal loads: every K/V byte is read once
constexpr int kMergeSlots = 2 * (kWaves - 1);   // merge area slots of a workgroup (see the split kernel)

// Bytes of a workgroup's merge area for g query heads of dimension d.
inline size_t decode_merge_bytes(int g, int d) {
    return (size_t)kMergeSlots * g * (d + 4) * 4 + (size_t)kMergeSlots * g * 4;
}

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
// A lane's K piece per d-step is 8 elements at d = 32 ds + 8 q4 (the
// 16x16x32 contraction); its V piece is D/16 elements of each of its four
// rows at d = (D/16) c ..
template <int D>
struct Bf16Kv {
    static constexpr bool kFp8 = false;
    static constexpr int kD = D;
    static constexpr int kRowBytes = D * 2;
    static constexpr int kDSteps = D / 32;           // 16x16x32 contraction steps over d
    static constexpr int kVDwords = D / 32;          // dwords of a lane's V piece per row
    template <int NB> struct KBuf { u32x4 r[NB][kDSteps]; };              // [block][d-step]
    template <int NB> struct VBuf { uint32_t r[NB][4][kVDwords]; };       // [block][row][dword]
};
struct Fp8Kv {                                       // d = 128 only
    static constexpr bool kFp8 = true;
    static constexpr int kD = 128;
    static constexpr int kRowBytes = 128;
    static constexpr int kDSteps = 4;
    static constexpr int kVDwords = 4;
    template <int NB> struct KBuf { u32x4 r[NB][2]; f32x4 s[NB]; };   // 32 codes of row c at d = 32 q4 .., scales of keys 4 q4 ..
    template <int NB> struct VBuf { u32x2 r[NB][4]; f32x4 s[NB]; };   // 8 codes of rows 4 q4 + rr at d = 8 c .., scales
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
    int B, int Hq, int g, int P, float scale_log2, int window, int merge) {
    __shared__ long long pre[kDecodeMaxBatch + 1];
    // Merge area (merge != 0; dynamic LDS, see decode_merge_bytes): the
    // pieces that share a segment with a neighbouring wavefront of the
    // workgroup, kMergeSlots slots of g rows of kD + 4 floats (normalised
    // output; the pad spreads a store's 16 rows over the banks), then
    // kMergeSlots x g base-2 log-sum-exps.  Slot w (w < kWaves - 1) holds
    // the last piece of wavefront w when its segment continues into
    // wavefront w + 1; slot kWaves - 2 + w (w >= 1) the first piece of
    // wavefront w when its segment began in wavefront w - 1 (and does not
    // continue past it).
    extern __shared__ __attribute__((aligned(16))) float xm[];
    __shared__ int xflag[kWaves];       // bit 0: slot w used; bit 1: that piece began in w - 1; bit 2: slot of the first piece used
    __shared__ int xdst[kWaves][3];     // (b, hk, partial index) of the segment whose merge group starts at w

    constexpr int kD = Fmt::kD;
    constexpr int kDSteps = Fmt::kDSteps;
    constexpr int kNB = kChunkBlocks;                 // 16-token blocks per chunk
    constexpr int kChunk = 16 * kNB;
    constexpr int kPV = kD / 16;                      // P.V MFMAs per block (d = kPV * m + j)
    const int tid = threadIdx.x;
    const int Hkv = Hq / g;

    // Token prefix sums over sequences: pre[b] = sum of L_b' for b' < b,
    // where a sliding window (window > 0) keeps only a sequence's last
    // `window` tokens: its segment is tokens [L - min(L, window), L).
    // The first wavefront alone: lane l sums the lengths of sequences
    // [l*per, (l+1)*per), the 64 lane sums are scanned across the wavefront,
    // and each lane writes the running sums of its sequences.
    if (tid < 64) {
        const int per = (B + 63) / 64;
        const int lo = min(B, tid * per), hi = min(B, lo + per);
        long long acc = 0;
        for (int i = lo; i < hi; ++i) acc += window > 0 ? min(seq_lens[i], window) : seq_lens[i];
        long long x = acc;                                      // inclusive scan of the lane sums
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const long long y = __shfl_up(x, off, 64);
            if (tid >= off) x += y;
        }
        long long run = x - acc;
        for (int i = lo; i < hi; ++i) {
            run += window > 0 ? min(seq_lens[i], window) : seq_lens[i];
            pre[i + 1] = run;
        }
        if (tid == 0) pre[0] = 0;
    }
    if (tid < kWaves) xflag[tid] = 0;
    __syncthreads();
    if (blockIdx.x == 0)
        for (int i = tid; i <= B; i += kThreads) prefix_out[i] = pre[i];

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
    // Tokens per partial result: a workgroup's four shares (merge) or one.
    const long long Qp = merge ? Q * kWaves : Q;
    const long long pid = merge ? (long long)blockIdx.x : w;

    typedef typename Fmt::template KBuf<kNB> KBuf;
    typedef typename Fmt::template VBuf<kNB> VBuf;

    // A piece: the part of one segment (b, hk) inside this wavefront's share,
    // tokens [p0, p1) of the segment, streamed as 32-token chunks from the
    // 16-aligned token c0.  Everything in it is wavefront-uniform
    // (readfirstlane makes that explicit, so table lookups are scalar loads).
    struct Piece {
        int b, hk, p0, p1, slot, c0, nchunks;
        long long next;                     // flattened position after the piece
        long long seg, seg_end;             // flattened range of its segment
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
        p.slot = __builtin_amdgcn_readfirstlane((int)(pid - S / Qp));  // partial index in the segment
        p.c0 = p.p0 & ~15;
        p.nchunks = (p.p1 - p.c0 + kChunk - 1) / kChunk;            // >= 1
        p.next = S + p1;
        p.seg = S;
        p.seg_end = S + L;
        return p;
    };
    const Piece none = {0, 0, 0, 0, 0, 0, 0, end, 0, 0};            // loads nothing

    // Q^T operand: lane holds Q[head hb*16 + c][32*ds + 8*q4 .. +8] (fp8
    // caches: Q[..][32*q4 + 8*ds .. +8], the order a lane's 32 contiguous K
    // codes come in; any order of the contraction gives the same dot
    // product, Q and K only have to agree).  Columns
    // of heads >= g repeat the group's first head (their results are never
    // written; every column of the MFMAs is independent), so the loads need
    // no branch.
    auto load_q = [&](bf16x8 (&qf)[NHB][kDSteps], const Piece& p) {
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            const int hl = hb * 16 + c;
            const uint16_t* qp = q + ((size_t)p.b * Hq + p.hk * g + (hl < g ? hl : 0)) * kD;
#pragma unroll
            for (int ds = 0; ds < kDSteps; ++ds)
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
    auto lookup = [&](int (&ph)[kNB], const Src& sr) {
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
            const int t0 = sr.c0 + sr.ci * kChunk + 16 * blk;
            ph[blk] = t0 < sr.p1 ? rows.lookup(table, sr.b, t0 >> 4) : 0;
        }
    };
    // Every load is issued unconditionally through a buffer resource that
    // covers only the block's tokens below p1: the hardware returns zeros
    // beyond it (chunks past the end cost no memory traffic).  With a fixed
    // number of loads per chunk the wait counts stay exact, so the next
    // chunk streams in while the current one is computed.
    auto load = [&](KBuf& kr, VBuf& vr, const int (&ph)[kNB], const Src& sr) {
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
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
                for (int ds = 0; ds < kDSteps; ++ds)
                    kr.r[blk][ds] = __builtin_amdgcn_raw_buffer_load_b128(
                        krs, (uint32_t)(c * kD + 32 * ds + 8 * q4) * 2, 0, kStreamAux);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const uint32_t off = (uint32_t)((4 * q4 + rr) * kD + (kD / 16) * c) * 2;
                    if constexpr (kD == 128) {
                        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(vrs, off, 0, kStreamAux);
#pragma unroll
                        for (int e = 0; e < 4; ++e) vr.r[blk][rr][e] = x[e];
                    } else {
                        const u32x2 x = __builtin_bit_cast(
                            u32x2, __builtin_amdgcn_raw_buffer_load_b64(vrs, off, 0, kStreamAux));
                        vr.r[blk][rr][0] = x[0];
                        vr.r[blk][rr][1] = x[1];
                    }
                }
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
                // Non-temporal like the codes: the scales are read once too,
                // and cached loads of them cost the fp8 call 20-27 %.
                const uint32_t sbytes = nvalid > 0 ? 64u : 0u;
                const __amdgpu_buffer_rsrc_t kss = make_rsrc(rows.kscale + row, sbytes);
                const __amdgpu_buffer_rsrc_t vss = make_rsrc(rows.vscale + row, sbytes);
                kr.s[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(kss, 16u * q4, 0, kStreamAux));
                vr.s[blk] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(vss, 16u * q4, 0, kStreamAux));
            }
        }
    };

    bf16x8 qf[NHB][kDSteps], qn[NHB][kDSteps];
    float ref[NHB], lsum[NHB];
    f32x4 oacc[NHB][kPV];

    auto process = [&](const KBuf& kr, const VBuf& vr, const Piece& cur, int ci) {
        bf16x4 pf[NHB][kNB];
        // bf16 operands of the chunk: K for each block and d-step, V row
        // pieces (fp8 codes widened once, for all head blocks).
        u32x4 kop[kNB][kDSteps];
        uint32_t vrow[kNB][4][Fmt::kVDwords];
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
            for (int x = 0; x < kDSteps; ++x) {
                if constexpr (!Fmt::kFp8) {
                    kop[blk][x] = kr.r[blk][x];
                } else {
                    const u32x4 w = kr.r[blk][x >> 1];
                    kop[blk][x] = (x & 1) ? fp8x8_to_bf16x8(w[2], w[3]) : fp8x8_to_bf16x8(w[0], w[1]);
                }
            }
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                if constexpr (!Fmt::kFp8) {
#pragma unroll
                    for (int e = 0; e < Fmt::kVDwords; ++e) vrow[blk][rr][e] = vr.r[blk][rr][e];
                } else {
                    const u32x4 w = fp8x8_to_bf16x8(vr.r[blk][rr][0], vr.r[blk][rr][1]);
#pragma unroll
                    for (int e = 0; e < 4; ++e) vrow[blk][rr][e] = w[e];
                }
            }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float s[kNB][4];
#pragma unroll
            for (int blk = 0; blk < kNB; ++blk) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int ds = 0; ds < kDSteps; ++ds)
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
            // The reference of a head (shared by its four lanes) is raised
            // only when its chunk maximum exceeds it by the slack.  A lane
            // first tests its own scores; only when some lane of the
            // wavefront is over does the wavefront form the heads' maxima
            // across lanes (a head whose lanes are all under would not be
            // raised either way, so the result is the same).
            float lmax = s[0][0];
#pragma unroll
            for (int blk = 0; blk < kNB; ++blk)
#pragma unroll
                for (int r = 0; r < 4; ++r) lmax = fmaxf(lmax, s[blk][r]);
            if (__builtin_amdgcn_ballot_w64(lmax * scale_log2 > ref[hb] + kRescaleSlack)) {   // uniform branch
                float tmax = fmaxf(lmax, __shfl_xor(lmax, 16, 64));
                tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * scale_log2;
                const bool raise = tmax > ref[hb] + kRescaleSlack;
                const float ref_new = raise ? tmax : ref[hb];
                const float alpha = exp2_fast(ref[hb] - ref_new);
                ref[hb] = ref_new;
                lsum[hb] *= alpha;
#pragma unroll
                for (int j = 0; j < kPV; ++j) oacc[hb][j] *= alpha;
            }
#pragma unroll
            for (int blk = 0; blk < kNB; ++blk) {
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
        // O^T += V^T . P^T; MFMA j covers d = kPV*m + j (m = 0..15, the lane
        // group c holding d-piece m).
#pragma unroll
        for (int blk = 0; blk < kNB; ++blk) {
#pragma unroll
            for (int j = 0; j < kPV; ++j) {
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
    // share its reference.  Lane holds head hb*16 + c, d = kPV*(4*q4 + r) + j.
    // With merge, a piece whose segment continues into the next wavefront of
    // the workgroup (or began in the previous one) goes to the merge area;
    // the workgroup merges each such group after its loop and writes one
    // partial.  A segment inside one wavefront's share of the workgroup
    // writes its partial directly.
    auto finish = [&](const Piece& cur) {
        const bool cross_l = merge && wave > 0 && cur.seg < start;
        const bool cross_r = merge && wave < kWaves - 1 && cur.seg_end > end;
        const int xs = cross_r ? wave : kWaves - 2 + wave;        // merge slot
        if (cross_l || cross_r) {
            if (lane == 0) {
                xflag[wave] |= cross_r ? (1 | (cross_l ? 2 : 0)) : 4;
                if (cross_r && !cross_l) {
                    xdst[wave][0] = cur.b;
                    xdst[wave][1] = cur.hk;
                    xdst[wave][2] = cur.slot;
                }
            }
        }
#pragma unroll
        for (int hb = 0; hb < NHB; ++hb) {
            float lt = lsum[hb] + __shfl_xor(lsum[hb], 16, 64);
            lt += __shfl_xor(lt, 32, 64);
            const int hl = hb * 16 + c;
            if (hl < g) {
                const size_t row = ((size_t)cur.b * Hq + cur.hk * g + hl) * P + cur.slot;
                const float inv = 1.f / lt;
                const float lse2 = ref[hb] + __builtin_amdgcn_logf(lt);   // v_log_f32: log2
                float* dst = (cross_l || cross_r) ? xm + ((size_t)xs * g + hl) * (kD + 4) + 4 * kPV * q4
                                                  : opart + row * kD + 4 * kPV * q4;
#pragma unroll
                for (int r = 0; r < 4; ++r)
#pragma unroll
                    for (int j4 = 0; j4 < kPV; j4 += 4) {
                        const f32x4 x = {oacc[hb][j4][r] * inv, oacc[hb][j4 + 1][r] * inv, oacc[hb][j4 + 2][r] * inv,
                                         oacc[hb][j4 + 3][r] * inv};
                        *reinterpret_cast<f32x4*>(dst + kPV * r + j4) = x;
                    }
                if (q4 == 0) {
                    if (cross_l || cross_r) xm[(size_t)kMergeSlots * g * (kD + 4) + xs * g + hl] = lse2;
                    else lsepart[row] = lse2;
                }
            }
        }
    };

    // Two chunk buffers (chunk x of a piece in buffer x % 2) with their table
    // entries.
    KBuf ka, kb;
    VBuf va, vb;
    int pha[kNB], phb[kNB];
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

    if (start < end) {
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
                for (int j = 0; j < kPV; ++j) oacc[hb][j] = f32x4{};
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
                for (int ds = 0; ds < kDSteps; ++ds) qf[hb][ds] = qn[hb][ds];
        }
    }
    if (!merge) return;

    // Merge groups: a group starts at a wavefront whose last piece continues
    // into the next wavefront and did not begin in the previous one; it holds
    // that piece, the whole-share pieces of the wavefronts inside the segment
    // and the first piece of the wavefront where the segment ends.  The
    // pieces are merged in wavefront order with weights 2^(lse - max), the
    // same rescale the combine applies across workgroups.
    __syncthreads();
    const float* const xlse = xm + (size_t)kMergeSlots * g * (kD + 4);
    // The groups (at most kWaves - 1): first wavefront and piece count.
    int gw0[kWaves - 1], gnm[kWaves - 1], ng = 0;
#pragma unroll
    for (int w0 = 0; w0 < kWaves - 1; ++w0) {
        if ((xflag[w0] & 3) != 1) continue;
        int wl = w0 + 1;
        while (wl < kWaves - 1 && (xflag[wl] & 3) == 3) ++wl;
        gw0[ng] = w0;
        gnm[ng] = wl - w0 + 1;          // pieces: slots w0 .. wl-1, then kWaves - 2 + wl
        ++ng;
    }
    // One unit = 16 consecutive elements of one head's row: its weights are
    // formed once, the rows are read and written 16 bytes at a time.
    constexpr int kUnitsPerRow = kD / 16;
    const int units = g * kUnitsPerRow;
    for (int u = tid; u < ng * units; u += kThreads) {
        const int gi = u / units, r = u - gi * units;
        const int hl = r / kUnitsPerRow, d0 = 16 * (r % kUnitsPerRow);
        const int w0 = gw0[gi], nm = gnm[gi];
        int si[kWaves];
        float lv[kWaves], mx = -INFINITY;
#pragma unroll
        for (int m = 0; m < kWaves; ++m) {
            si[m] = m < nm - 1 ? w0 + m : kWaves - 2 + w0 + nm - 1;
            lv[m] = m < nm ? xlse[si[m] * g + hl] : -INFINITY;
            mx = fmaxf(mx, lv[m]);
        }
        float wt[kWaves], den = 0.f;
#pragma unroll
        for (int m = 0; m < kWaves; ++m) {
            wt[m] = m < nm ? exp2_fast(lv[m] - mx) : 0.f;
            den += wt[m];
        }
        const float inv = 1.f / den;
        const size_t row = ((size_t)xdst[w0][0] * Hq + (size_t)xdst[w0][1] * g + hl) * P + xdst[w0][2];
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int m = 0; m < kWaves; ++m)
                if (m < nm)
                    acc += wt[m] * *reinterpret_cast<const f32x4*>(xm + ((size_t)si[m] * g + hl) * (kD + 4) + d0 + 4 * c4);
            *reinterpret_cast<f32x4*>(opart + row * kD + d0 + 4 * c4) = acc * inv;
        }
        if (d0 == 0) lsepart[row] = mx + __builtin_amdgcn_logf(den);
    }
}

// Combine: the partial results of a (sequence, query head) row are merged
// with a running maximum, weights 2^(lse_s - max), the rescale step of the
// tiled online softmax applied across pieces.  Every kernel finds a row's
// partials from the same share arithmetic as the split kernel.
//
// Few partials per row (caches up to 7,936 tokens): one wavefront per row,
// lane owning d = kE*lane .., merging the partials in order.
constexpr int kCombineBatch = 4;         // partials in flight per lane
constexpr int kCombineFewPartials = 32;  // at most this many per row: one wavefront

template <int kD>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart, const long long* __restrict__ prefix,
    uint16_t* __restrict__ o, int B, int Hq, int g, int P, long long NW, int per) {
    constexpr int kE = kD / 64;          // output elements per lane: d = kE * lane ..
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int lane = threadIdx.x;
    const int Hkv = Hq / g;
    const long long L = prefix[b + 1] - prefix[b];
    float m = -INFINITY, den = 0.f, a0 = 0.f, a1 = 0.f;
    if (L > 0) {
        const long long W = prefix[B] * Hkv;
        const long long Q = share_tokens(W, NW) * per;      // tokens per partial
        const long long S = prefix[b] * Hkv + (long long)(hq / g) * L;
        const int np = (int)((S + L - 1) / Q - S / Q) + 1;
        const size_t row0 = ((size_t)b * Hq + hq) * P;
        for (int s0 = 0; s0 < np; s0 += kCombineBatch) {
            float x[kCombineBatch];
            float2 v[kCombineBatch];
#pragma unroll
            for (int u = 0; u < kCombineBatch; ++u) {
                const int s = s0 + u;
                const int sc = s < np ? s : np - 1;
                x[u] = s < np ? lsepart[row0 + sc] : -INFINITY;
                if constexpr (kE == 2)
                    v[u] = *reinterpret_cast<const float2*>(opart + (row0 + sc) * kD + 2 * lane);
                else
                    v[u] = float2{opart[(row0 + sc) * kD + lane], 0.f};
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
    float o0 = 0.f, o1 = 0.f;
    if (m != -INFINITY) {
        o0 = a0 / den;
        o1 = a1 / den;
    }
    if constexpr (kE == 2)
        reinterpret_cast<uint32_t*>(o + ((size_t)b * Hq + hq) * kD)[lane] = pack_bf16x2(o0, o1);
    else
        o[((size_t)b * Hq + hq) * kD + lane] = (uint16_t)(pack_bf16x2(o0, 0.f) & 0xffffu);
}

// Many partials per row: a workgroup of 256 threads per row.  Thread t owns
// the 4-float column c = t % kCols of the row and reads partials
// t / kCols, t / kCols + kGroups, ..., up to kWideBatch of them per round,
// all loads issued together; the kGroups running results of a column are
// then merged in LDS in a fixed order, so the output is reproducible bit for
// bit.
constexpr int kWideBatch = 8;

template <int kD>
__global__ __launch_bounds__(256) void decode_combine_wide_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart, const long long* __restrict__ prefix,
    uint16_t* __restrict__ o, int B, int Hq, int g, int P, long long NW, int per) {
    constexpr int kCols = kD / 4;
    constexpr int kGroups = 256 / kCols;
    __shared__ f32x4 red_acc[kGroups][kCols];
    __shared__ float red_m[kGroups], red_den[kGroups];
    const int hq = blockIdx.x;
    const int b = blockIdx.y;
    const int t = threadIdx.x;
    const int col = t % kCols, grp = t / kCols;
    const int Hkv = Hq / g;
    const long long L = prefix[b + 1] - prefix[b];
    float m = -INFINITY, den = 0.f;
    f32x4 acc = f32x4{};
    if (L > 0) {
        const long long W = prefix[B] * Hkv;
        const long long Q = share_tokens(W, NW) * per;      // tokens per partial
        const long long S = prefix[b] * Hkv + (long long)(hq / g) * L;
        const int np = (int)((S + L - 1) / Q - S / Q) + 1;
        const size_t row0 = ((size_t)b * Hq + hq) * P;
        for (int s0 = grp; s0 < np; s0 += kGroups * kWideBatch) {
            float x[kWideBatch];
            f32x4 v[kWideBatch];
#pragma unroll
            for (int u = 0; u < kWideBatch; ++u) {
                const int s = s0 + u * kGroups;
                const int sc = s < np ? s : np - 1;
                x[u] = s < np ? lsepart[row0 + sc] : -INFINITY;
                v[u] = *reinterpret_cast<const f32x4*>(opart + (row0 + sc) * kD + 4 * col);
            }
#pragma unroll
            for (int u = 0; u < kWideBatch; ++u) {
                const float mn = fmaxf(m, x[u]);
                const float sc = mn == m ? 1.f : exp2_fast(m - mn);
                const float wgt = x[u] == -INFINITY ? 0.f : exp2_fast(x[u] - mn);
                den = den * sc + wgt;
                acc = acc * sc + wgt * v[u];
                m = mn;
            }
        }
    }
    red_acc[grp][col] = acc;
    if (col == 0) {
        red_m[grp] = m;
        red_den[grp] = den;
    }
    __syncthreads();
    if (grp == 0) {
        float M = red_m[0];
#pragma unroll
        for (int k = 1; k < kGroups; ++k) M = fmaxf(M, red_m[k]);
        float dt = 0.f;
        f32x4 r = f32x4{};
        if (M != -INFINITY) {
#pragma unroll
            for (int k = 0; k < kGroups; ++k) {
                const float f = red_m[k] == -INFINITY ? 0.f : exp2_fast(red_m[k] - M);
                dt += f * red_den[k];
                r += f * red_acc[k][col];
            }
            r /= dt;
        }
        const u32x2 w = {pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
        *reinterpret_cast<u32x2*>(o + ((size_t)b * Hq + hq) * kD + 4 * col) = w;
    }
}

template <int NHB, class Fmt, class Rows>
hipError_t launch_both(const DecodeArgs& a, const Rows& rows, hipStream_t stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return hipErrorInvalidDevice;
    const int nwg = cus * (NHB == 1 ? 2 : 1);                      // every workgroup resident at once
    constexpr int kD = Fmt::kD;
    const DecodeWorkspace ws = decode_workspace_layout(a.B, a.Hq, kD, a.max_seq_len);
    char* base = static_cast<char*>(a.workspace);
    float* opart = reinterpret_cast<float*>(base + ws.part_o);
    float* lsepart = reinterpret_cast<float*>(base + ws.part_lse);
    long long* prefix = reinterpret_cast<long long*>(base + ws.prefix);
    const int P = decode_max_partials(a.max_seq_len);
    const int g = a.Hq / a.Hkv;
    // Merge within workgroups when the merge area fits beside the prefix
    // sums without lowering the number of resident workgroups (the CU's LDS,
    // 160 KB on gfx950, shared by the resident workgroups).
    const size_t xbytes = decode_merge_bytes(g, kD);
    int lds_cu = 0;
    if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) != hipSuccess)
        lds_cu = 0;                                                   // unknown: no merge
    const size_t lds_budget = (size_t)lds_cu / (NHB == 1 ? 2 : 1);
    const size_t static_lds = (size_t)(kDecodeMaxBatch + 1) * 8 + 1024;
    const int merge = lds_budget > static_lds && xbytes <= lds_budget - static_lds ? 1 : 0;
    auto kernel = decode_split_kernel<NHB, Rows, Fmt>;
    if (merge && xbytes > 64 * 1024) {       // above the default dynamic LDS limit
        const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                    hipFuncAttributeMaxDynamicSharedMemorySize,
                                                    (int)(lds_budget - static_lds));
        if (attr != hipSuccess) return attr;
    }
    hipLaunchKernelGGL(kernel, dim3(nwg), dim3(kThreads), merge ? xbytes : 0, stream,
                       static_cast<const uint16_t*>(a.q), rows, a.block_table, a.seq_lens, opart, lsepart, prefix, a.B,
                       a.Hq, g, P, a.scale * kLog2e, a.window > 0 ? a.window : 0, merge);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int per = merge ? kWaves : 1;
    if (P <= kCombineFewPartials)
        hipLaunchKernelGGL((decode_combine_kernel<kD>), dim3(a.Hq, a.B), dim3(64), 0, stream, opart, lsepart,
                           prefix, static_cast<uint16_t*>(a.o), a.B, a.Hq, g, P, (long long)nwg * kWaves, per);
    else
        hipLaunchKernelGGL((decode_combine_wide_kernel<kD>), dim3(a.Hq, a.B), dim3(256), 0, stream, opart, lsepart,
                           prefix, static_cast<uint16_t*>(a.o), a.B, a.Hq, g, P, (long long)nwg * kWaves, per);
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

// Workspace of the allocation-free entry point: one static array per GPU.
// Host code never passes this name to a kernel or a copy (on the host it is
// only a stand-in for the device symbol); it uses the device address that
// hipGetSymbolAddress returns, taken once per device with that device
// current and kept in scratch_addr.  Every call on a GPU shares its array,
// so calls that overlap on one GPU (two streams, two threads) race on it.
static __device__ __align__(256) unsigned char scratch[kDecodeStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_addr[kMaxDevices] = {};

hipError_t static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(scratch_mutex);
    if (!scratch_addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        scratch_addr[dev] = p;
    }
    *out = scratch_addr[dev];
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
    return a.d == 64 ? launch_fmt<Bf16Kv<64>>(a, stream) : launch_fmt<Bf16Kv<128>>(a, stream);
}

hipError_t launch_decode_bf16_static(const DecodeArgs& a, hipStream_t stream) {
    DecodeArgs s = a;
    const hipError_t e = static_scratch(&s.workspace);
    if (e != hipSuccess) return e;
    return launch_decode_bf16(s, stream);
}

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) { return launch_fmt<Fp8Kv>(a, stream); }

}  // namespace gqa
