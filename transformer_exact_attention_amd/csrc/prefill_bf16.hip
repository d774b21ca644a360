// bf16 attention forward on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The method: exact attention computed tile by tile with an online softmax, so
// the Sq x Sk score matrix never reaches device memory [Attention variants
// deep-dive, §6.2: tiling, forward pseudocode; Different attention
// mechanisms, §4 Flash Attention: tiling, kernel fusion, online softmax].
// Query head h reads K/V head h / g [Attention variants deep-dive, §5 GQA
// code], without copying K/V per query head (§5, the note after the code).
//
// Work decomposition (one workgroup = 4 wavefronts, one workgroup per CU):
//   * a workgroup owns one K/V head of one batch entry and 256 "query rows":
//     256/g consecutive query positions x all g query heads of the group,
//     ordered position-major (row r -> position p0 + r/g, head hk*g + r%g);
//   * wavefront w owns rows 64w..64w+63 as two 32-row blocks nb = 0, 1; lane i
//     owns query column i%32 of each block and lane half hh = i/32 (the MFMA
//     operand split along the contraction);
//   * the workgroup's Q rows are staged once through LDS (whole-row loads);
//     each wavefront then keeps its Q fragments in AGPRs, where the score
//     MFMAs take them as B operand, and the Q area is reused at the end to
//     transpose the output for row-contiguous stores; K/V tiles
//     of 64 keys are staged in LDS by direct-to-LDS buffer loads, three
//     buffers each, and serve all 256 rows: the g query heads of a group
//     share them.  The step that computes the scores of tile j+1
//     loads K tile j+2 and V tile j+1, spread over its first half so that the
//     four wavefronts do not queue 32 KB of requests at once.
//
// Per KV tile every wavefront computes the transposed score tile
//   S^T (64 keys x 64 queries) = K (64 x d) . Q^T (d x 64)
// so the 32x32 accumulator layout puts one query column in each lane and a
// query's softmax state lives in that lane (and its partner i^32).  The
// probabilities are then already in the B-operand layout of
//   O^T (d x 64 queries) += V^T (d x 64 keys) . P^T (64 keys x 64 queries).
// The V^T operand (8 keys of one d per lane) is read from the row-major V tile
// with two transposing LDS reads (ds_read_b64_tr_b16): in each 16-lane group,
// lane l receives element l%4 of the 8-byte pieces addressed by lanes l/4,
// l/4+4, l/4+8, l/4+12, so pointing lane r of the group at key row r/4,
// columns 4*(r%4).. gives lane l four keys of column l.  Holding 64 query
// columns per wavefront makes every LDS operand read feed two MFMAs.
//
// Software pipeline.  While the softmax of tile j runs on the vector ALU, the
// matrix cores compute the scores of tile j+1 and the P.V product of tile
// j-1, so the exponentials overlap matrix work instead of alternating with it.
//
// Softmax runs in base 2: scores are multiplied by scale*log2(e) in fp32 and
// exponentiated with v_exp_f32; exp(x) = 2^(x log2 e) changes only rounding.
// The reference point of the exponent is raised lazily: p = 2^(s*c - ref)
// with ref a past running max; a tile is redone against its true max (and the
// accumulator and sum rescaled) only when some lane's tile sum of p exceeds
// 2^8, which bounds every p by 2^8.  Softmax does not depend on the reference
// point, so the result is exact up to rounding.  P is rounded to bf16 for the
// PV product; the row sums add the fp32 values of p (the recomputing path adds
// the rounded ones); accumulation is fp32 throughout.
#include "common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace gqa {

namespace {

constexpr int kBc = 64;                  // keys per KV tile
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsWG = 64 * kWaves;     // query rows per workgroup
constexpr float kSumLimit = 256.0f;      // 2^8: per-lane tile sum of p that forces a rescale

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tiles are row-major [rows][D] bf16 with 16-byte chunks XOR-swizzled
// against bank conflicts for their read patterns:
//   Q, K: chunk c of row r at chunk c ^ (r % chunks)   (reads: 32 rows, one chunk)
//   V:    chunk c of row r at chunk c ^ ((4 * (r & 3)) % chunks)
//         (transposing reads: 4 consecutive rows x 32 bytes per 16 lanes)
template <int D>
__device__ __forceinline__ int k_swz(int r) { return r & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int v_swz(int r) { return (4 * (r & 3)) & (D / 8 - 1); }
template <int D>
__device__ __forceinline__ int k_byte(int r, int chunk) { return r * D * 2 + ((chunk ^ k_swz<D>(r)) << 4); }
template <int D>
__device__ __forceinline__ int v_byte(int r, int chunk) { return r * D * 2 + ((chunk ^ v_swz<D>(r)) << 4); }

// O^T accumulation in AGPRs.  The compiler would otherwise give every MFMA
// the same register file, and the score accumulators, which the softmax reads
// with vector instructions, must stay in VGPRs.  The compiler does not see
// into the asm, so it cannot supply the two wait states an MFMA needs after a
// vector instruction wrote its A/B operands: the build checks the generated
// code for that (asm_check.py).  Back to back on the same accumulator the
// MFMA needs none.  Code that reads the accumulator afterwards first passes
// through agpr_settle().
__device__ __forceinline__ void mfma_agpr(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Score MFMAs: the Q^T operand comes from AGPRs (it is read from global
// memory once and never changes), the accumulator stays in VGPRs for the
// softmax.  The same wait-state caveat as mfma_agpr applies.
__device__ __forceinline__ void mfma_qk_first(f32x16& acc, const bf16x8& k, const bf16x8& q) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(k), "a"(q));
}
__device__ __forceinline__ void mfma_qk(f32x16& acc, const bf16x8& k, const bf16x8& q) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(k), "a"(q));
}

// Workgroup barrier without a memory fence.  Every wavefront first waits for
// its own direct-to-LDS loads whose data the others are about to read; a
// fenced barrier would also wait for the loads still meant to be in flight.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}
// Wait until at most N vector-memory operations of this wavefront are in
// flight (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most N LDS operations of this wavefront are in flight.
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt range");
    __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (N << 8) | (3 << 14));
}

// Wait states between the last MFMA that wrote an accumulator and a vector
// instruction reading it (more than the 8-pass MFMA's result latency).
template <int N>
__device__ __forceinline__ void agpr_settle(f32x16 (&acc)[2][N]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < N; ++t) asm volatile("" : "+a"(acc[nb][t]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < N; ++t) asm volatile("" : "+a"(acc[nb][t]));
}

__device__ __forceinline__ float dot2_sum(uint32_t packed, float acc) {
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

template <int D, bool kWindow>
__global__ __launch_bounds__(kThreads, 1) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, int Hq, int Hkv, int Sq, int Sk, int lg, int nqb, int by_cost,
    float scale_log2, int causal, int window, float* __restrict__ lse) {
    constexpr int kChunks = D / 8;                          // 16-byte chunks per row
    constexpr int kDSteps = D / 16;                         // MFMA contraction steps over d
    constexpr int kDTiles = D / 32;                         // 32-row output tiles of O^T
    constexpr int kTileLoads = kBc * kChunks / 64 / kWaves; // 1 KB direct loads per wavefront per tile
    constexpr int kStepsPerWindow = kDSteps / 4;            // score steps per pipeline window

    // Separate arrays, so that the compiler can tell the buffers being filled
    // by direct loads from the ones being read.
    __shared__ __attribute__((aligned(1024))) uint16_t k_s0[kBc * D];
    __shared__ __attribute__((aligned(1024))) uint16_t k_s1[kBc * D];
    __shared__ __attribute__((aligned(1024))) uint16_t k_s2[kBc * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s0[kBc * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s1[kBc * D];
    __shared__ __attribute__((aligned(1024))) uint16_t v_s2[kBc * D];
    // Q rows of the workgroup (read into registers once), then the output
    // transpose of the epilogue.
    __shared__ __attribute__((aligned(1024))) uint16_t q_s[kRowsWG * D];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int g = 1 << lg;
    const int npos = kRowsWG >> lg;         // query positions per workgroup

    // Work item of this workgroup.  Items are ordered plane by plane (plane =
    // (batch, K/V head)), heaviest query block first within a plane.  The
    // hardware hands consecutive workgroup ids to the 8 XCDs in turn, so
    // workgroup id L runs on XCD L % 8; when the item count divides by 8, XCD x
    // is given the contiguous item range [x * N/8, (x+1) * N/8): whole planes,
    // whose K/V then stay in that XCD's L2 instead of being fetched by all 8.
    // With by_cost (planes too short to fill an XCD), the XCD's items are
    // handed out heaviest query block first across a group of its planes
    // (four, when the XCD's plane count divides by four; whose K/V, 1 MB
    // each at S = 2048, stay in the XCD's 4 MB L2), group after group, so
    // the CUs that start with light items do not meet heavy ones at the end.
    const int nitems = (int)gridDim.x;
    const int L = (int)blockIdx.x;
    int plane, qb;
    if (by_cost) {
        const int ppx = nitems / (8 * nqb);               // planes per XCD
        const int j = L >> 3;
        const int G = (ppx % 4) == 0 ? 4 : ppx;           // planes dealt together
        const int grp = j / (G * nqb), jj = j - grp * (G * nqb);
        plane = (L & 7) * ppx + grp * G + jj % G;
        qb = nqb - 1 - jj / G;
    } else {
        const int item = (nitems & 7) == 0 ? (L & 7) * (nitems >> 3) + (L >> 3) : L;
        plane = item / nqb;
        qb = nqb - 1 - (item - plane * nqb);
    }
    const int hk = plane % Hkv;
    const int b = plane / Hkv;
    const int p0 = qb * npos;
    const int off = Sk - Sq;                // causal: key j visible iff j <= pos + off

    // Sliding window (window > 0, causal): position pos sees keys
    // (pos + off - window, pos + off].  Keys are counted from kb0, the first
    // tile holding a key of the workgroup's first row, so the tiles before
    // it are neither loaded nor computed.
    const int kb0 = kWindow ? max(0, p0 + off - window + 1) & ~(kBc - 1) : 0;

    // Last visible key of this lane's two query columns (counted from kb0).
    int my_last[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int r = 64 * wave + 32 * nb + n;
        my_last[nb] = (causal ? p0 + (r >> lg) + off : Sk - 1) - kb0;
    }

    // Keys this workgroup needs; tiles past the wavefront's first diagonal
    // key, or (window) before its last row's first key, need the mask.
    const int p_last = min(p0 + npos, Sq) - 1;
    const int kend = causal ? min(Sk, p_last + off + 1) : Sk;
    const int ntiles = (kend - kb0 + kBc - 1) / kBc;
    const int wave_first_last = (causal ? min(p0 + ((64 * wave) >> lg) + off, Sk - 1) : Sk - 1) - kb0;

    // ---- staging -------------------------------------------------------
    // A direct load moves 16 bytes per lane into consecutive LDS slots
    // (lane i -> slot base + i), so each lane fetches the global chunk whose
    // swizzled place is its slot.  The buffer resources end at key kend:
    // keys past it (the rest of the last tile, and the tiles past the last
    // that the final steps address) are not fetched.  The K/V tiles are
    // zero-filled once, so such rows hold zeros or an older tile's finite
    // values, and the mask removes them.
    const size_t kvbase = ((size_t)b * Hkv + hk) * (size_t)Sk * D + (size_t)kb0 * D;
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(k + kvbase, (uint32_t)(kend - kb0) * D * 2);
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(v + kvbase, (uint32_t)(kend - kb0) * D * 2);
    // Load x of wavefront w fills the 1 KB slot group t = 4x + w, i.e. rows
    // (64 t + lane) / chunks.  Every row of load x is 16x (d = 128) or 32x
    // (d = 64) rows past that of load 0, a multiple of the swizzle period, so
    // a lane fetches the same chunk column in all its loads and its byte
    // offset is one base plus 4096 x.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // wave-uniform LDS bases
    uint32_t st_kbase, st_vbase;
    {
        const int s = 64 * wave + lane;
        const int row = s / kChunks, pp = s % kChunks;
        st_kbase = (uint32_t)(row * D * 2 + 16 * (pp ^ k_swz<D>(row)));
        st_vbase = (uint32_t)(row * D * 2 + 16 * (pp ^ v_swz<D>(row)));
    }
    // wave_lds = 1024 * wave; passing it through an empty asm once per step
    // keeps the compiler from precomputing every load's LDS address in its
    // own scalar register (they would not fit and get spilled).
    auto issue_load = [&](__amdgpu_buffer_rsrc_t r, uint32_t vbase, uint16_t* dst, int tile, int x, int wave_lds) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (lds_void*)((lds_char*)(dst) + 4096 * x + wave_lds), 16,
            vbase + (uint32_t)(tile * (kBc * D * 2) + 4096 * x), 0, 0, 0);
    };
    auto issue_tile = [&](__amdgpu_buffer_rsrc_t r, uint32_t vbase, uint16_t* dst, int tile) {
#pragma unroll
        for (int x = 0; x < kTileLoads; ++x) issue_load(r, vbase, dst, tile, x, 1024 * wave_u);
    };

    bf16x8 qa[2][kDSteps];   // filled from q_s once the loads have landed
    // Zero what no load may write before it is read: V buffer 2 (the first
    // step multiplies a zero P by it) and, when the last tile is partial
    // (its rows past kend are not fetched), every K/V buffer.  Rows past the
    // last tile that later steps read keep earlier, finite contents.
    const bool partial = (kend & (kBc - 1)) != 0;
    for (int i = tid; i < kBc * D / 8; i += kThreads) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        ((lds_u32x4*)(lds_char*)v_s2)[i] = z;
        if (partial) {
            ((lds_u32x4*)(lds_char*)k_s0)[i] = z;
            ((lds_u32x4*)(lds_char*)k_s1)[i] = z;
            ((lds_u32x4*)(lds_char*)k_s2)[i] = z;
            ((lds_u32x4*)(lds_char*)v_s0)[i] = z;
            ((lds_u32x4*)(lds_char*)v_s1)[i] = z;
        }
    }
    __syncthreads();
    // Q rows of the workgroup -> LDS by direct loads (16 lanes per row, so
    // whole rows are fetched), swizzled like K; rows past Sq read the last
    // row and are never stored.
    {
        constexpr int kQLoads = kRowsWG * kChunks / 64 / kWaves;
        const uint16_t* qgroup = q + ((size_t)b * Hq + (size_t)hk * g) * (size_t)Sq * D;
#pragma unroll
        for (int x = 0; x < kQLoads; ++x) {
            const int t = wave * kQLoads + x;
            const int s = 64 * t + lane;
            const int row = s / kChunks, pp = s % kChunks;
            const int c = pp ^ k_swz<D>(row);
            const int prow = min(p0 + (row >> lg), Sq - 1);
            const uint16_t* src = qgroup + ((size_t)(row & (g - 1)) * Sq + prow) * D + 8 * c;
            __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                             (lds_void*)((lds_char*)q_s + 1024 * t), 16, 0, 0);
        }
    }
    issue_tile(krsrc, st_kbase, k_s0, 0);
    issue_tile(krsrc, st_kbase, k_s1, 1);
    issue_tile(vrsrc, st_vbase, v_s0, 0);

    // ---- operand reads -------------------------------------------------
    auto qk_mfma = [&](f32x16& acc, const u32x4& kfrag, const bf16x8& qf, bool first) {
        if (first) mfma_qk_first(acc, __builtin_bit_cast(bf16x8, kfrag), qf);
        else mfma_qk(acc, __builtin_bit_cast(bf16x8, kfrag), qf);
    };
    auto qk_step = [&](const uint16_t* ks, f32x16 (&sacc)[2][2], int t, bool first) {
        const u32x4 a0 = *(lds_u32x4*)((lds_char*)ks + k_byte<D>(n, 2 * t + hh));
        const u32x4 a1 = *(lds_u32x4*)((lds_char*)ks + k_byte<D>(32 + n, 2 * t + hh));
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            qk_mfma(sacc[nb][0], a0, qa[nb][t], first);
            qk_mfma(sacc[nb][1], a1, qa[nb][t], first);
        }
    };
    // Transposed V reads: in 16-lane group G = lane/16, lane rr = lane%16 points
    // at key row 16s + 4*(G/2) + 8*piece + rr/4 and column 32t + 16*(G%2) + 4*(rr%4).
    const int G = lane >> 4, rr = lane & 15;
    const int vrow0 = 4 * (G >> 1) + (rr >> 2);
    const int vcol0 = 16 * (G & 1) + 4 * (rr & 3);
    auto pv_step = [&](const uint16_t* vs, f32x16 (&oacc)[2][kDTiles], const bf16x8 (&pf)[2][4], int s) {
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
            const int col = 32 * t + vcol0;
            const int row_a = 16 * s + vrow0;
            const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)((lds_char*)vs + v_byte<D>(row_a, col >> 3) + (col & 7) * 2));
            const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)((lds_char*)vs + v_byte<D>(row_a + 8, col >> 3) + (col & 7) * 2));
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
                mfma_agpr(oacc[nb][t], a, pf[nb][s]);
        }
    };
    // P block (nb, kb) = 2^(s*c - ref) as bf16 B-operand fragments for the
    // 16-key steps 2kb, 2kb+1 (step s holds keys 16s + {4hh..4hh+3,
    // 8+4hh..8+4hh+3}), plus their sum.
    auto softmax_block = [&](const f32x16& sblk, float ref, bf16x8& pf0, bf16x8& pf1, float& sum) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) p[e] = exp2_fast(fmaf(sblk[8 * half + e], scale_log2, -ref));
            u32x4 w;
            w.x = pack_bf16x2(p[0], p[1]);
            w.y = pack_bf16x2(p[2], p[3]);
            w.z = pack_bf16x2(p[4], p[5]);
            w.w = pack_bf16x2(p[6], p[7]);
            sum = dot2_sum(w.w, dot2_sum(w.z, dot2_sum(w.y, dot2_sum(w.x, sum))));
            (half ? pf1 : pf0) = __builtin_bit_cast(bf16x8, w);
        }
    };

    f32x16 oacc[2][kDTiles];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) oacc[nb][t] = f32x16{};
    bf16x8 pprev[2][4];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int s = 0; s < 4; ++s) pprev[nb][s] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    float ref[2] = {-INFINITY, -INFINITY};   // reference max, scaled base-2 units
    float l[2] = {0.f, 0.f};                 // running sum over this lane's keys

    // Q and K tile 0 have landed (loads complete in issue order); K tile 1
    // and V tile 0 may still be in flight: the first step waits for them.
    wait_vmcnt<2 * kTileLoads>();
    lds_barrier();
    // Q^T operand fragments of this lane's two query columns: Q[row][16t +
    // 8hh .. +8] for d-step t, kept in AGPRs.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int t = 0; t < kDSteps; ++t)
            qa[nb][t] = __builtin_bit_cast(
                bf16x8, *(lds_u32x4*)((lds_char*)q_s + k_byte<D>(64 * wave + 32 * nb + n, 2 * t + hh)));
    f32x16 scur[2][2];
#pragma unroll
    for (int t = 0; t < kDSteps; ++t) qk_step(k_s0, scur, t, t == 0);

    // Reference of the first tile: its largest visible score (the largest of
    // the lane pair's 32 keys per query column), so that the first step
    // needs no rescaling pass; a column with no visible key in the tile keeps
    // -inf and takes that pass, as any later tile whose sum exceeds the bound.
    // The score MFMAs must have finished before their results are read.
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(scur[nb][kb]));
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) asm volatile("" : "+v"(scur[nb][kb]));
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        float tm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int key = 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
                const bool hidden = kWindow ? (uint32_t)(my_last[nb] - key) >= (uint32_t)window : key > my_last[nb];
                tm = hidden ? tm : fmaxf(tm, scur[nb][kb][e]);
            }
        tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
        ref[nb] = tm * scale_log2;
    }

    // Operands of one 4-MFMA group of the pipelined step.  A score group
    // (QK, d-step t) reads K rows n and 32+n of d-chunk 2t+hh (two LDS
    // reads); a P.V group reads the transposed V fragments of two d-tiles
    // (four LDS reads).
    struct Ops {
        u32x4 r[2];     // QK: K rows n, 32+n
        s16x4 t[4];     // PV: lo/hi of d-tile 0, lo/hi of d-tile 1
    };
    auto group_reads = [](int gi) { return (gi & 1) == 0 ? 4 : 2; };
    auto issue_read = [&](const uint16_t* ks, const uint16_t* vs, int x, int gi, int r, Ops& op) {
        if ((gi & 1) != 0) {
            const int t = kStepsPerWindow * x + (gi >> 1);
            op.r[r] = *(lds_u32x4*)((lds_char*)ks + k_byte<D>(n + 32 * r, 2 * t + hh));
        } else {
            const int dt = 2 * (gi >> 1) + (r >> 1);
            const int col = 32 * dt + vcol0;
            const int row = 16 * x + vrow0 + ((r & 1) ? 8 : 0);
            op.t[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4*)((lds_char*)vs + v_byte<D>(row, col >> 3) + (col & 7) * 2));
        }
    };
    auto group_mfma = [&](int x, int gi, int m, const Ops& op, f32x16 (&sacc)[2][2]) {
        if ((gi & 1) != 0) {
            const int t = kStepsPerWindow * x + (gi >> 1);
            const int nb = m >> 1, kb = m & 1;
            qk_mfma(sacc[nb][kb], op.r[kb], qa[nb][t], t == 0);
        } else {
            const int dt = 2 * (gi >> 1) + (m >> 1), nb = m & 1;
            const s16x4 lo = op.t[(m >> 1) * 2], hi = op.t[(m >> 1) * 2 + 1];
            const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            mfma_agpr(oacc[nb][dt], a, pprev[nb][x]);
        }
    };

    // One pipeline step for tile j (PAR = j % 3); tile t lives in k_s[t % 3]
    // and v_s[t % 3].
    auto step = [&](auto par_c, int j) {
        constexpr int PAR = decltype(par_c)::value;
        uint16_t* const ks[3] = {k_s0, k_s1, k_s2};
        uint16_t* const vs[3] = {v_s0, v_s1, v_s2};
        uint16_t* const k_fill = ks[(PAR + 2) % 3];        // <- tile j+2
        uint16_t* const v_fill = vs[(PAR + 1) % 3];        // <- tile j+1
        const uint16_t* const k_read = ks[(PAR + 1) % 3];  // tile j+1
        const uint16_t* const v_read = vs[(PAR + 2) % 3];  // tile j-1

        // The main block below is scheduled by hand, one slot at a time: an
        // MFMA, the vector work of one or two softmax elements, and one LDS
        // read of the next 4-MFMA group, fenced so the compiler keeps the
        // order.  Groups alternate between two d-tiles of the P.V product of
        // tile j-1 (PV) and a score step of tile j+1 (QK); the operands of a
        // group are read during the group before it.
        constexpr int kGroups = 2 * kStepsPerWindow;        // 4-MFMA groups per window
        constexpr int kElems = 16 / (4 * kGroups);          // softmax elements per slot
        // Operands are read kAhead groups ahead of their MFMAs.
        constexpr int kAhead = 2;
        Ops ops[kAhead + 1];
        // The first group, P.V of tile j-1, reads a V tile that is resident
        // since the previous barrier and is not refilled in this step: its
        // operands are read before the barrier, so the matrix cores start as
        // soon as it opens.
#pragma unroll
        for (int r = 0; r < group_reads(0); ++r) issue_read(k_read, v_read, 0, 0, r, ops[0]);
        // After the barrier the previous step's loads have landed, and every
        // wavefront is done with the buffers refilled during this step.  The
        // loads are issued from the main block below, also past the last tile
        // (keys are clamped), which keeps that block free of branches.
        wait_vmcnt<0>();
        lds_barrier();
        int wave_lds = 1024 * wave_u;
        asm volatile("" : "+s"(wave_lds));
#pragma unroll
        for (int ga = 1; ga < kAhead; ++ga)
#pragma unroll
            for (int r = 0; r < group_reads(ga % kGroups); ++r)
                issue_read(k_read, v_read, ga / kGroups, ga % kGroups, r, ops[ga]);

        const int j0 = j * kBc;
        // (window) the wavefront's last row sees no key before this one
        const int wave_last_first = kWindow ? p0 + ((64 * wave_u + 63) >> lg) + off - window + 1 - kb0 : 0;
        if (j0 + kBc - 1 > wave_first_last || (kWindow && j0 < wave_last_first)) {
            int lim[2] = {my_last[0], my_last[1]};
            // (window) taken as new values here, so that nothing derived from
            // them is computed ahead of the loop and kept in registers
            if constexpr (kWindow) asm volatile("" : "+v"(lim[0]), "+v"(lim[1]));
#pragma unroll
            for (int nb = 0; nb < 2; ++nb)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int key = j0 + 32 * kb + 8 * (e >> 2) + 4 * hh + (e & 3);
                        // visible: my_last - window < key <= my_last, one unsigned compare
                        const bool hidden = kWindow ? (uint32_t)(lim[nb] - key) >= (uint32_t)window
                                                    : key > lim[nb];
                        if (hidden) scur[nb][kb][e] = -INFINITY;
                    }
        }
        __builtin_amdgcn_sched_barrier(0);

        // Softmax element G (0..63) is element G%16 of block x = G/16, (nb, kb)
        // = (x/2, x%2).  Its vector work runs as a pipeline over the slots so
        // that no instruction waits on one issued in the same slot: slot i
        // computes s*c - ref for the elements of slot i+2, their exponentials
        // for slot i+1, packs slot i's values to bf16 and adds the packs of
        // slot i-1 to the row sums.
        f32x16 snext[2][2];
        float psum[2] = {0.f, 0.f};
        float xs[64], pe[64];
        uint32_t pw[32];
        constexpr int kSlots = 64 / kElems;
        auto stage_a = [&](int sl) {
#pragma unroll
            for (int u = 0; u < kElems; ++u) {
                const int G = sl * kElems + u;
                if (sl < kSlots)
                    xs[G] = fmaf(scur[G >> 5][(G >> 4) & 1][G & 15], scale_log2, -ref[G >> 5]);
            }
        };
        auto stage_b = [&](int sl) {
#pragma unroll
            for (int u = 0; u < kElems; ++u) {
                const int G = sl * kElems + u;
                if (sl < kSlots) pe[G] = exp2_fast(xs[G]);
            }
        };
        auto stage_c = [&](int sl) {
#pragma unroll
            for (int u = 0; u < kElems; ++u) {
                const int G = sl * kElems + u;
                if (sl >= 0 && sl < kSlots && (G & 1)) {
                    pw[G >> 1] = pack_bf16x2(pe[G - 1], pe[G]);
                    asm volatile("" ::"v"(pw[G >> 1]));   // keep the pack in its slot
                }
            }
        };
        float psum2[2] = {0.f, 0.f};
        auto stage_d = [&](int sl) {
#pragma unroll
            for (int u = 0; u < kElems; ++u) {
                const int G = sl * kElems + u;
                if (sl >= 0 && sl < kSlots) {
                    if (G & 1) psum2[G >> 5] += pe[G];
                    else psum[G >> 5] += pe[G];
                }
            }
        };
        stage_a(0);
        stage_a(1);
        stage_b(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
#pragma unroll
            for (int gi = 0; gi < kGroups; ++gi) {
                const int gg = x * kGroups + gi;
                const Ops& cur = ops[gg % (kAhead + 1)];
                Ops& nxt = ops[(gg + kAhead) % (kAhead + 1)];
                const int nx = (gg + kAhead) / kGroups, ngi = (gg + kAhead) % kGroups;
                // One wait per group: its reads have landed (the next
                // group's may still be in flight).
                if (gg + 1 >= 4 * kGroups) wait_lgkmcnt<0>();
                else if (group_reads((gg + 1) % kGroups) == 4) wait_lgkmcnt<4>();
                else wait_lgkmcnt<2>();
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    const int sl = gg * 4 + m;
                    group_mfma(x, gi, m, cur, snext);
                    stage_a(sl + 2);
                    stage_b(sl + 1);
                    stage_c(sl);
                    stage_d(sl - 1);
                    if (gg + kAhead < 4 * kGroups && m < group_reads(ngi))
                        issue_read(k_read, v_read, nx, ngi, m, nxt);
                    if ((sl & 3) == 1 && (sl >> 2) < 2 * kTileLoads) {
                        const int li = sl >> 2;
                        if (li < kTileLoads) issue_load(krsrc, st_kbase, k_fill, j + 2, li, wave_lds);
                        else issue_load(vrsrc, st_vbase, v_fill, j + 1, li - kTileLoads, wave_lds);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
        }
        stage_d(kSlots - 1);
        psum[0] += psum2[0];
        psum[1] += psum2[1];
        bf16x8 pcur[2][4];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
#pragma unroll
            for (int s4 = 0; s4 < 4; ++s4) {
                const int w0 = 16 * nb + 4 * s4;
                pcur[nb][s4] = __builtin_bit_cast(bf16x8, u32x4{pw[w0], pw[w0 + 1], pw[w0 + 2], pw[w0 + 3]});
            }

        // Rare: some p exceeded the bound (or a column has seen no visible key
        // yet, so its reference is still -inf).  Redo
        // the tile against its true max and rescale what came before.
        const bool over = !(psum[0] <= kSumLimit) || !(psum[1] <= kSumLimit);
        if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
            for (int nb = 0; nb < 2; ++nb) {
                float tm = -INFINITY;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int e = 0; e < 16; ++e) tm = fmaxf(tm, scur[nb][kb][e]);
                tm = fmaxf(tm, __shfl_xor(tm, 32, 64));
                const float rnew = fmaxf(ref[nb], tm * scale_log2);
                const float alpha = rnew == ref[nb] ? 1.f : exp2_fast(ref[nb] - rnew);
                const float ruse = rnew == -INFINITY ? 0.f : rnew;
                ref[nb] = rnew;
                l[nb] *= alpha;
                if (nb == 0) agpr_settle(oacc);
#pragma unroll
                for (int t = 0; t < kDTiles; ++t) oacc[nb][t] *= alpha;
                psum[nb] = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
                    softmax_block(scur[nb][kb], ruse, pcur[nb][2 * kb], pcur[nb][2 * kb + 1], psum[nb]);
            }
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
            l[nb] += psum[nb];
#pragma unroll
            for (int s = 0; s < 4; ++s) pprev[nb][s] = pcur[nb][s];
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) scur[nb][kb] = snext[nb][kb];
        }
    };

    for (int j = 0;;) {
        step(std::integral_constant<int, 0>{}, j);
        if (++j >= ntiles) break;
        step(std::integral_constant<int, 1>{}, j);
        if (++j >= ntiles) break;
        step(std::integral_constant<int, 2>{}, j);
        if (++j >= ntiles) break;
    }

    // P.V of the last tile.
    wait_all_memory();
    __syncthreads();
    {
        const int last = (ntiles - 1) % 3;
        const uint16_t* const v_last = last == 0 ? v_s0 : (last == 1 ? v_s1 : v_s2);
#pragma unroll
        for (int s = 0; s < 4; ++s) pv_step(v_last, oacc, pprev, s);
    }

    // Epilogue: combine the lane pair's partial sums, normalise, round to
    // bf16, and write whole output rows.  Each lane holds 8-byte pieces of
    // many rows, so the rows are first transposed through LDS: wavefront w
    // stores its 64 rows x D in its quarter of the Q area (free since the
    // prologue) as 8-byte units XOR-swizzled by row (unit u of row q at
    // u ^ (q % units)), and reads them back as 16-byte row chunks, which it
    // stores 4 rows per instruction.
    agpr_settle(oacc);
    float inv[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const float lt = l[nb] + __shfl_xor(l[nb], 32, 64);
        inv[nb] = lt > 0.f ? 1.f / lt : 0.f;
        // Optional log-sum-exp of the row (natural log): ln(sum_j e^{s_j})
        // = ln 2 * (ref + log2(l)), the value a backward pass needs to
        // recompute the probabilities.
        if (lse && hh == 0) {
            const int r = 64 * wave + 32 * nb + n;
            const int pos = p0 + (r >> lg);
            if (pos < Sq)
                lse[((size_t)b * Hq + hk * g + (r & (g - 1))) * Sq + pos] =
                    (ref[nb] + __builtin_amdgcn_logf(lt)) * kLn2;
        }
    }
    constexpr int kUnits = D / 4;                           // 8-byte units per row
    lds_char* const obuf = (lds_char*)q_s + wave_u * (64 * D * 2);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        const int q = 32 * nb + n;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int u = (32 * t + 8 * grp + 4 * hh) / 4;
                u32x2 w;
                w.x = pack_bf16x2(oacc[nb][t][4 * grp + 0] * inv[nb], oacc[nb][t][4 * grp + 1] * inv[nb]);
                w.y = pack_bf16x2(oacc[nb][t][4 * grp + 2] * inv[nb], oacc[nb][t][4 * grp + 3] * inv[nb]);
                *(__attribute__((address_space(3))) u32x2*)(obuf + q * D * 2 + 8 * (u ^ (q & (kUnits - 1)))) = w;
            }
        }
    }
#pragma unroll
    for (int x = 0; x < kChunks; ++x) {
        const int sidx = 64 * x + lane;
        const int q = sidx / kChunks, m = sidx % kChunks;
        const int sw = q & (kUnits - 1);
        u32x4 w = *(lds_u32x4*)(obuf + q * D * 2 + 16 * (m ^ (sw >> 1)));
        if (sw & 1) w = u32x4{w.z, w.w, w.x, w.y};
        const int r = 64 * wave + q;
        const int pos = p0 + (r >> lg);
        if (pos < Sq) {
            const int head = hk * g + (r & (g - 1));
            uint16_t* const dst = o + (((size_t)b * Hq + head) * Sq + pos) * D + 8 * m;
            __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(dst));   // written once, never re-read here
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int window = a.window > 0 ? a.window : 0;
    const int g = a.Hq / a.Hkv;
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const int npos = kRowsWG >> lg;
    const int nqb = (a.Sq + npos - 1) / npos;
    dim3 grid(nqb * a.Hkv * a.B);
    const float sl = a.scale * kLog2e;
    // Order items by cost across planes when a plane has fewer query blocks
    // than an XCD has CUs (8 XCDs; needs a plane count divisible by 8).
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return hipErrorInvalidDevice;
    const int nplanes = a.Hkv * a.B;
    const int by_cost = (nplanes % 8 == 0) && (nqb * 8 < cus) ? 1 : 0;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* o = static_cast<uint16_t*>(a.o);
    auto launch = [&](auto kernel) {
        hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, stream, q, k, v, o, a.Hq, a.Hkv, a.Sq, a.Sk, lg, nqb,
                           by_cost, sl, a.causal, window, a.lse);
    };
    if (a.d == 64)
        window > 0 ? launch(prefill_bf16_kernel<64, true>) : launch(prefill_bf16_kernel<64, false>);
    else
        window > 0 ? launch(prefill_bf16_kernel<128, true>) : launch(prefill_bf16_kernel<128, false>);
    return hipGetLastError();
}

}  // namespace gqa
