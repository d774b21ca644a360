// Attention backward pass (bf16 inputs, fp32 accumulation) by recomputation.
//
// The backward keeps no attention matrix from the forward: it recomputes the
// probabilities from the saved Q, K, V and the forward's per-row
// log-sum-exp, tile by tile, so memory stays O(n) [Attention variants
// deep-dive, §6.2 technique 2 (recomputation); §8 follow-ups 2-3].  With
// S = scale Q K^T (masked entries -inf), P = exp(S - LSE), and the output
// gradient dO:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D),  D_i = sum_d dO_id O_id,
//   dQ = scale dS K,  dK = scale dS^T Q,
// with a K/V head's gradients summed over the g query heads that read it
// [Attention variants deep-dive, §5 GQA code].
//
// Three kernels, no atomics:
//   * rowdot: D for every query row;
//   * dkdv: a workgroup of 8 wavefronts owns 256 keys of one K/V head (a
//     wavefront 32 of them, their K rows in registers, the V rows of all 256
//     in LDS) and walks every 64-row query tile of the group's g heads,
//     keeping dK and dV in registers;
//   * dq: a workgroup of 8 wavefronts owns 256 query rows of one head (a
//     wavefront 32) and walks the 64-key tiles, keeping dQ^T in registers.
// Eight wavefronts share every staged tile (half the tile bytes per FLOP of
// four) and two share each SIMD; keeping V in LDS is what fits a dK/dV
// wavefront in 256 registers.
// Products are v_mfma_f32_32x32x16_bf16.  Each product computed in the
// accumulator layout is already an operand of the product that consumes it:
// P and dS (rows q, columns keys) are the A operands of dV = P^T dO and
// dK = dS^T Q, and dS^T (rows keys, columns q) is the B operand of
// dQ^T = K^T dS^T.  Tiles are staged in LDS with XOR-swizzled 16-byte units
// (D = 128), so row reads and transposing column reads (ds_read_b64_tr_b16)
// are both conflict-free.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;

constexpr int kBwdThreads = 256;
constexpr int kTileRows = 64;            // rows of a staged tile (4 wavefronts x 16)

// LDS tile of 64 rows x D bf16.  Operands are read two ways: 16-byte row
// pieces of 16 consecutive rows at one column (ds_read_b128), and 8-byte
// pieces of 4 consecutive rows x 32 columns (transposing reads, two 16-lane
// groups at a time).  D = 128: rows of 256 bytes with their 16-byte units
// XOR-swizzled by f(row) = 4 (row % 4) + (row / 4) % 4, a bijection on 16
// rows (row reads hit 16 distinct 4-bank groups) that moves the 4 rows of a
// transposing read to disjoint unit groups (all 64 banks once).  D = 64: rows
// padded to 144 bytes.
template <int D>
struct Tile {
    static constexpr int kRowBytes = D == 128 ? 256 : D * 2 + 16;
    static constexpr int kBytes = kTileRows * kRowBytes;
    // byte offset of element `col` (a multiple of 4) of `row`
    static __device__ __forceinline__ int off(int row, int col) {
        if constexpr (D == 128) {
            const int f = ((row & 3) << 2) | ((row >> 2) & 3);
            return row * kRowBytes + ((((col >> 3) ^ f)) << 4) + ((col & 7) << 1);
        } else {
            return row * kRowBytes + 2 * col;
        }
    }
};

// 64 x D bf16 rows [row0, row0 + 64) of a [rows_total, D] matrix -> LDS tile.
// The loads go through a buffer resource that starts at row0 and ends at the
// matrix's last row (row0 is wavefront-uniform, so the resource is scalar
// and each lane's offset is the same for every tile): rows past rows_total
// read as zeros, finite values whose products the callers multiply by a
// zero probability, and the loads stay unconditional, so no branch keeps
// the compiler from overlapping them with the tile's work.
template <int D, int NT = kBwdThreads>
__device__ __forceinline__ void load_rows(u32x4 (&reg)[kTileRows * D / 8 / NT], const uint16_t* base,
                                          int row0, int rows_total) {
    constexpr int kChunks = D / 8;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base + (size_t)row0 * D, (uint32_t)(rows_total - row0) * D * 2);
#pragma unroll
    for (int x = 0; x < kTileRows * kChunks / NT; ++x) {
        const int i = x * NT + (int)threadIdx.x;
        const int rr = i / kChunks, c = i % kChunks;
        reg[x] = buffer_load16(r, (uint32_t)((rr * D + 8 * c) * 2));
    }
}
template <int D, int NT = kBwdThreads>
__device__ __forceinline__ void store_rows(lds_char* tile, const u32x4 (&reg)[kTileRows * D / 8 / NT]) {
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int x = 0; x < kTileRows * kChunks / NT; ++x) {
        const int i = x * NT + (int)threadIdx.x;
        const int r = i / kChunks, c = i % kChunks;
        *(lds_u32x4*)(tile + Tile<D>::off(r, 8 * c)) = reg[x];
    }
}

// D[row] = sum_d dO[row][d] * O[row][d]; 16 lanes per row (D = 128: 8
// elements each; D = 64: 4).
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_rowdot_kernel(const uint16_t* __restrict__ o,
                                                                 const uint16_t* __restrict__ dout,
                                                                 float* __restrict__ dsum, long long rows) {
    constexpr int E = D / 16;
    const long long i = (long long)blockIdx.x * kBwdThreads + threadIdx.x;
    const long long row = i >> 4;
    const int sub = (int)(i & 15);
    float acc = 0.f;
    if (row < rows) {
        const uint16_t* po = o + row * D + sub * E;
        const uint16_t* pd = dout + row * D + sub * E;
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc = fmaf(__uint_as_float((uint32_t)po[e] << 16), __uint_as_float((uint32_t)pd[e] << 16), acc);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows && sub == 0) dsum[row] = acc;
}

// 32-row operand fragments for v_mfma_f32_32x32x16_bf16 (A: lane l holds
// row l % 32, k = 8 (l / 32) .. +7; B: k = 8 (l / 32) .. +7 of column l % 32;
// D: register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4 of column
// l % 32).  A D-layout result used as the contraction operand of the next
// product is taken in the order its registers hold it: in 16-row step s,
// position e of lane half h stands for row
//   m(s, h, e) = 16 s + 8 (e / 4) + 4 h + e % 4,
// and the other operand supplies the same rows with two transposing reads
// (rows 16 s + 4 h + 0..3 and 16 s + 8 + 4 h + 0..3).
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// A/B fragment of a row: 8 bf16 at (row, col .. col + 7).
template <int D>
__device__ __forceinline__ bf16x8 row_frag8(const lds_char* tile, int row, int col) {
    return __builtin_bit_cast(bf16x8, *(const lds_u32x4*)(tile + Tile<D>::off(row, col)));
}
// Column fragment in the m(s, h, e) order: column col0 + (lane % 32) of rows
// r0 + 16 s + {4 h .. 4 h + 3, 8 + 4 h .. 8 + 4 h + 3}.
template <int D>
__device__ __forceinline__ bf16x8 col_frag8(const lds_char* tile, int r0, int col0, int lane) {
    const int grp = lane >> 4, r = lane & 15;
    const int h = grp >> 1;
    const int row = r0 + 4 * h + (r >> 2);
    const int col = col0 + 16 * (grp & 1) + 4 * (r & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + Tile<D>::off(row, col)));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + Tile<D>::off(row + 8, col)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
__device__ __forceinline__ bf16x8 pack8(const f32x16& x, int s) {
    const u32x4 w = {pack_bf16x2(x[8 * s + 0], x[8 * s + 1]), pack_bf16x2(x[8 * s + 2], x[8 * s + 3]),
                     pack_bf16x2(x[8 * s + 4], x[8 * s + 5]), pack_bf16x2(x[8 * s + 6], x[8 * s + 7])};
    return __builtin_bit_cast(bf16x8, w);
}

constexpr int kWaveRows = 32;                      // keys (dK/dV) or query rows (dQ) per wavefront

// dK, dV for 256 keys of K/V head hk of batch b (32 per wavefront).  Query
// tiles of 64 rows of every head of the group stream through LDS.
constexpr int kDkWaves = 8;
constexpr int kDkThreads = 64 * kDkWaves;
constexpr int kDkBlockRows = kDkWaves * kWaveRows;

template <int D>
__global__ __launch_bounds__(kDkThreads) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int Sq, int Sk, float scale,
    int causal, int window) {
    constexpr int kT = D / 16;                             // 16-wide d steps
    constexpr int kNT = D / 32;                            // 32-wide d tiles of dK, dV
    constexpr int kRegs = kTileRows * D / 8 / kDkThreads;
    __shared__ __attribute__((aligned(16))) char q_raw[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char d_raw[2][Tile<D>::kBytes];
    __shared__ float2 row_s[2][kTileRows];                 // (lse * log2 e, D) per row
    __shared__ __attribute__((aligned(16))) char v_all[kDkBlockRows * Tile<D>::kRowBytes];   // V rows of the block's keys

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    // 1-D grid, key block slowest: under a causal mask the first key blocks
    // see the most query rows, so the heaviest workgroups start first
    const int planes = (int)gridDim.x / ((Sk + kDkBlockRows - 1) / kDkBlockRows);     // Hkv * B
    const int kb = (int)blockIdx.x / planes, hk = (int)blockIdx.x % Hkv, b = ((int)blockIdx.x % planes) / Hkv;
    const int g = Hq / Hkv;
    const int off = Sk - Sq;
    const int kw0 = kb * kDkBlockRows + kWaveRows * wave;    // this wavefront's keys kw0 .. kw0 + 31
    const int key = kw0 + n;                               // this lane's key column
    const float sl2 = scale * kLog2e;
    const uint32_t wlim = window > 0 ? (uint32_t)window : 0x80000000u;   // causal only: d >= 0

    // K rows of the wavefront's keys as B operands (k = d, column = key) in
    // registers; the V rows of all the workgroup's keys in LDS (read as the
    // same B operand each sub-step), which keeps a wavefront within 256
    // registers so two share each SIMD.
    bf16x8 kf[kT];
    {
        const size_t kvrow = ((size_t)b * Hkv + hk) * Sk;
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            u32x4 kw = {0u, 0u, 0u, 0u};
            if (key < Sk) kw = *reinterpret_cast<const u32x4*>(k + (kvrow + key) * D + 16 * t + 8 * h);
            kf[t] = __builtin_bit_cast(bf16x8, kw);
        }
        constexpr int kVChunks = kDkBlockRows * D / 8 / kDkThreads;
#pragma unroll
        for (int x = 0; x < kVChunks; ++x) {
            const int i = x * kDkThreads + (int)threadIdx.x;
            const int r = i / (D / 8), c = i % (D / 8);
            const int row = min(kb * kDkBlockRows + r, Sk - 1);
            *(lds_u32x4*)((lds_char*)v_all + Tile<D>::off(r, 8 * c)) =
                *reinterpret_cast<const u32x4*>(v + (kvrow + row) * D + 8 * c);
        }
        // Redefine the fragments past their loads: the loop below then sees
        // registers with no load pending and never waits on the tile
        // prefetches it has in flight (the wait counter is in order).
#pragma unroll
        for (int t = 0; t < kT; ++t) asm volatile("" : "+v"(kf[t]));
    }
    const lds_char* const vrow = (const lds_char*)v_all;
    const int vr = kWaveRows * wave + n;                   // this lane's key row in v_all
    f32x16 dka[kNT], dva[kNT];
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dka[t][r] = dva[t][r] = 0.f;

    // Query tiles: for each head of the group, the tiles holding a row that
    // sees one of the workgroup's keys (causal: rows i >= key - off; window W:
    // also i < key - off + W).  They are walked tile-major over the group's
    // heads, from the last tile down: every workgroup of a K/V head starts on
    // the same tile at the same time (causal: the key blocks differ only in
    // where they stop), so the Q and dO tiles are fetched once into the L2
    // they share (the key blocks of a head run on one XCD) instead of once
    // per workgroup.
    const int first_tile = causal ? max(0, kb * kDkBlockRows - off) / kTileRows : 0;
    int end_tile = (Sq + kTileRows - 1) / kTileRows;
    if (window > 0)
        end_tile = min(end_tile, max(0, kb * kDkBlockRows + kDkBlockRows - 1 - off + window - 1) / kTileRows + 1);
    const int n_per_head = max(0, end_tile - first_tile);
    const int total = g * n_per_head;
    u32x4 qr[kRegs], dr[kRegs];
    auto tile_row0 = [&](int it) { return (first_tile + n_per_head - 1 - it / g) * kTileRows; };
    auto fetch = [&](int it) {
        const int hq = hk * g + it % g;
        const int row0 = tile_row0(it);
        const size_t base = ((size_t)b * Hq + hq) * Sq;
        load_rows<D, kDkThreads>(qr, q + base * D, row0, Sq);
        load_rows<D, kDkThreads>(dr, dout + base * D, row0, Sq);
    };
    auto stash = [&](int it, int buf) {
        const int hq = hk * g + it % g;
        const int row0 = tile_row0(it);
        const size_t base = ((size_t)b * Hq + hq) * Sq;
        store_rows<D, kDkThreads>((lds_char*)q_raw[buf], qr);
        store_rows<D, kDkThreads>((lds_char*)d_raw[buf], dr);
        if (threadIdx.x < kTileRows) {
            const int row = row0 + threadIdx.x;
            // rows past Sq: lse = +inf makes their probabilities 0
            row_s[buf][threadIdx.x] = row < Sq ? float2{lse[base + row] * kLog2e, dsum[base + row]}
                                               : float2{INFINITY, 0.f};
        }
    };
    if (total > 0) {
        fetch(0);
        stash(0, 0);
    }
    __syncthreads();
    for (int it = 0; it < total; ++it) {
        const int buf = it & 1;
        if (it + 1 < total) fetch(it + 1);                 // in flight while this tile is computed
        const int row0 = tile_row0(it);
        const lds_char* qt = (const lds_char*)q_raw[buf];
        const lds_char* dt = (const lds_char*)d_raw[buf];
#pragma unroll
        for (int sub = 0; sub < kTileRows / kWaveRows; ++sub) {
            const int r0 = kWaveRows * sub;                 // tile rows r0 .. r0 + 31
            const int pos0 = row0 + r0;
            // rows that see none of the wavefront's keys contribute nothing
            if (causal && pos0 + kWaveRows - 1 + off < kw0) continue;
            if (window > 0 && pos0 + off - window >= kw0 + kWaveRows - 1) continue;
            // S (32 rows x 32 keys) = Q K^T; dP = dO V^T
            f32x16 sc, dp;
#pragma unroll
            for (int r = 0; r < 16; ++r) sc[r] = dp[r] = 0.f;
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                sc = mfma32(row_frag8<D>(qt, r0 + n, 16 * t + 8 * h), kf[t], sc);
                dp = mfma32(row_frag8<D>(dt, r0 + n, 16 * t + 8 * h), row_frag8<D>(vrow, vr, 16 * t + 8 * h), dp);
            }
            // every (row, key) of the block visible?
            const bool full = (!causal || pos0 + off >= kw0 + kWaveRows - 1) &&
                              (window <= 0 || pos0 + kWaveRows - 1 + off - window < kw0);
            const int dbase = row0 + r0 + 4 * h + off - key;
            f32x16 p, ds;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qi = r0 + 8 * (r >> 2) + 4 * h + (r & 3);
                const float2 ld = row_s[buf][qi];
                // branch-free (a branch here doubles the register spills):
                // with d = row + off - key, visible iff 0 <= d < window, one
                // unsigned compare (no window: limit 2^31, i.e. d >= 0)
                const bool vis = full | ((uint32_t)(dbase + 8 * (r >> 2) + (r & 3)) < wlim);
                const float e = exp2_fast(fmaf(sc[r], sl2, -ld.x));
                p[r] = vis ? e : 0.f;
                ds[r] = p[r] * (dp[r] - ld.y);
            }
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 pa = pack8(p, s2), dsa = pack8(ds, s2);   // P^T, dS^T as A (rows = keys)
#pragma unroll
                for (int t = 0; t < kNT; ++t) {
                    dva[t] = mfma32(pa, col_frag8<D>(dt, r0 + 16 * s2, 32 * t, lane), dva[t]);
                    dka[t] = mfma32(dsa, col_frag8<D>(qt, r0 + 16 * s2, 32 * t, lane), dka[t]);
                }
            }
        }
        // The other buffer was last read while computing the previous tile,
        // which every wavefront finished before the barrier that published
        // this tile: it can be refilled at once.  One barrier per tile then
        // makes the new tile visible (and keeps any wavefront from running
        // more than one tile ahead).
        if (it + 1 < total) {
            stash(it + 1, buf ^ 1);
            __syncthreads();
        }
    }
    // register r: key kw0 + 8 (r / 4) + 4 h + r % 4, column 32 t + n
    const size_t kvrow = ((size_t)b * Hkv + hk) * Sk;
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kr = kw0 + 8 * (r >> 2) + 4 * h + (r & 3);
            if (kr < Sk) {
                const size_t at = (kvrow + kr) * D + 32 * t + n;
                const uint32_t pk = pack_bf16x2(dka[t][r] * scale, dva[t][r]);
                dk[at] = (uint16_t)(pk & 0xffffu);
                dv[at] = (uint16_t)(pk >> 16);
            }
        }
}

// dQ for 256 query rows of head hq of batch b (32 per wavefront).  Key tiles
// of 64 keys stream through LDS.
constexpr int kDqWaves = 8;
constexpr int kDqThreads = 64 * kDqWaves;
constexpr int kDqBlockRows = kDqWaves * kWaveRows;

template <int D>
__global__ __launch_bounds__(kDqThreads) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    uint16_t* __restrict__ dq, int Hq, int Hkv, int Sq, int Sk, float scale, int causal, int window) {
    constexpr int kT = D / 16;
    constexpr int kNT = D / 32;
    constexpr int kRegs = kTileRows * D / 8 / kDqThreads;
    __shared__ __attribute__((aligned(16))) char k_raw[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char v_raw[2][Tile<D>::kBytes];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n = lane & 31, h = lane >> 5;
    // 1-D grid, query block slowest; causal: the last query blocks see the
    // most keys, so they start first.  Workgroup id L runs on XCD L % 8; when
    // the K/V groups (b, hk) divide among the 8 XCDs, XCD x takes whole
    // groups (all g heads, every query block), so a group's K/V tiles, which
    // all its workgroups walk from key 0 up, are fetched into one L2; each
    // XCD still gets an equal share of every query block.
    const int nqb = (Sq + kDqBlockRows - 1) / kDqBlockRows;
    const int g = Hq / Hkv;
    const int L = (int)blockIdx.x;
    const int ngroups = Hkv * ((int)gridDim.x / nqb / Hq);                      // Hkv * B
    int rank, hq, b;
    if ((ngroups & 7) == 0) {
        const int per_rank = ngroups / 8 * g;                                   // items of one rank per XCD
        const int j = L >> 3;
        rank = j / per_rank;
        const int rem = j % per_rank;
        const int grp = (L & 7) * (ngroups / 8) + rem / g;
        b = grp / Hkv;
        hq = (grp % Hkv) * g + rem % g;
    } else {
        const int planes = (int)gridDim.x / nqb;                                // Hq * B
        rank = L / planes;
        hq = L % Hq;
        b = (L % planes) / Hq;
    }
    const int qb = causal ? nqb - 1 - rank : rank;
    const int hk = hq / g;
    const int off = Sk - Sq;
    const int qw0 = qb * kDqBlockRows + kWaveRows * wave;    // this wavefront's rows qw0 .. qw0 + 31
    const int qrow = qw0 + n;                              // this lane's query column
    const float sl2 = scale * kLog2e;
    const size_t qbase = ((size_t)b * Hq + hq) * Sq;

    // Q and dO of the lane's query as B operands (k = d, column = query).
    bf16x8 qf[kT], of[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        u32x4 qw = {0u, 0u, 0u, 0u}, ow = {0u, 0u, 0u, 0u};
        if (qrow < Sq) {
            qw = *reinterpret_cast<const u32x4*>(q + (qbase + qrow) * D + 16 * t + 8 * h);
            ow = *reinterpret_cast<const u32x4*>(dout + (qbase + qrow) * D + 16 * t + 8 * h);
        }
        qf[t] = __builtin_bit_cast(bf16x8, qw);
        of[t] = __builtin_bit_cast(bf16x8, ow);
    }
    float lse2 = qrow < Sq ? lse[qbase + qrow] * kLog2e : INFINITY;
    float dsq = qrow < Sq ? dsum[qbase + qrow] : 0.f;
    // as in the dK/dV kernel: no load left pending into the tile loop
#pragma unroll
    for (int t = 0; t < kT; ++t) asm volatile("" : "+v"(qf[t]), "+v"(of[t]));
    asm volatile("" : "+v"(lse2), "+v"(dsq));
    f32x16 dqa[kNT];                                       // dQ^T: register r = d 32 t + 8 (r/4) + 4 h + r % 4
#pragma unroll
    for (int t = 0; t < kNT; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) dqa[t][r] = 0.f;

    // Key tiles seen by the block's rows (causal: keys <= row + off; window W:
    // also keys > row + off - W).
    const int q_last = min(qb * kDqBlockRows + kDqBlockRows, Sq) - 1;
    const int kend = causal ? min(Sk, q_last + off + 1) : Sk;
    const int kfirst = window > 0 ? max(0, qb * kDqBlockRows + off - window + 1) / kTileRows : 0;
    const int ntiles = max(0, (kend + kTileRows - 1) / kTileRows - kfirst);
    const size_t kvbase = ((size_t)b * Hkv + hk) * Sk;
    u32x4 kr[kRegs], vr[kRegs];
    auto fetch = [&](int i) {
        load_rows<D, kDqThreads>(kr, k + kvbase * D, (kfirst + i) * kTileRows, Sk);
        load_rows<D, kDqThreads>(vr, v + kvbase * D, (kfirst + i) * kTileRows, Sk);
    };
    auto stash = [&](int buf) {
        store_rows<D, kDqThreads>((lds_char*)k_raw[buf], kr);
        store_rows<D, kDqThreads>((lds_char*)v_raw[buf], vr);
    };
    if (ntiles > 0) {
        fetch(0);
        stash(0);
    }
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
        const int buf = it & 1;
        const int tile = kfirst + it;
        if (it + 1 < ntiles) fetch(it + 1);
        const lds_char* kt = (const lds_char*)k_raw[buf];
        const lds_char* vt = (const lds_char*)v_raw[buf];
#pragma unroll
        for (int sub = 0; sub < kTileRows / kWaveRows; ++sub) {
            const int r0 = kWaveRows * sub;                 // keys tile * 64 + r0 .. + 31
            const int key0 = tile * kTileRows + r0;
            // keys no row of the wavefront sees contribute nothing
            if (causal && key0 > qw0 + kWaveRows - 1 + off) continue;
            if (window > 0 && key0 + kWaveRows - 1 <= qw0 + off - window) continue;
            // S^T (32 keys x 32 rows) = K Q^T; dP^T = V dO^T
            f32x16 st, dpt;
#pragma unroll
            for (int r = 0; r < 16; ++r) st[r] = dpt[r] = 0.f;
            bf16x8 ka[kT], va[kT];                          // all operand reads first, one wait
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                ka[t] = row_frag8<D>(kt, r0 + n, 16 * t + 8 * h);
                va[t] = row_frag8<D>(vt, r0 + n, 16 * t + 8 * h);
            }
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                st = mfma32(ka[t], qf[t], st);
                dpt = mfma32(va[t], of[t], dpt);
            }
            const bool full = key0 + kWaveRows - 1 < Sk && (!causal || key0 + kWaveRows - 1 <= qw0 + off) &&
                              (window <= 0 || key0 > qw0 + kWaveRows - 1 + off - window);
            f32x16 ds;
            if (full) {
#pragma unroll
                for (int r = 0; r < 16; ++r) ds[r] = exp2_fast(fmaf(st[r], sl2, -lse2)) * (dpt[r] - dsq);
            } else {
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int kk = key0 + 8 * (r >> 2) + 4 * h + (r & 3);
                    const bool vis = (kk < Sk) & (!causal | (kk <= qrow + off)) & ((window <= 0) | (kk > qrow + off - window));
                    const float e = exp2_fast(fmaf(st[r], sl2, -lse2));
                    ds[r] = (vis ? e : 0.f) * (dpt[r] - dsq);
                }
            }
            bf16x8 kc[2][kNT];
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
                for (int t = 0; t < kNT; ++t) kc[s2][t] = col_frag8<D>(kt, r0 + 16 * s2, 32 * t, lane);
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                const bf16x8 dsb = pack8(ds, s2);           // dS^T as B operand (k = keys, column = query)
#pragma unroll
                for (int t = 0; t < kNT; ++t) dqa[t] = mfma32(kc[s2][t], dsb, dqa[t]);
            }
        }
        // (one barrier per tile, as in the dK/dV kernel: the other buffer
        // was last read in the previous tile, before the last barrier)
        if (it + 1 < ntiles) {
            stash(buf ^ 1);
            __syncthreads();
        }
    }
    if (qrow < Sq) {
#pragma unroll
        for (int t = 0; t < kNT; ++t)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u32x2 w = {pack_bf16x2(dqa[t][4 * j + 0] * scale, dqa[t][4 * j + 1] * scale),
                                 pack_bf16x2(dqa[t][4 * j + 2] * scale, dqa[t][4 * j + 3] * scale)};
                *reinterpret_cast<u32x2*>(dq + (qbase + qrow) * D + 32 * t + 8 * j + 4 * h) = w;
            }
    }
}

template <int D>
hipError_t launch_bwd(const BackwardArgs& a, hipStream_t stream) {
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    const uint16_t* o = static_cast<const uint16_t*>(a.o);
    const uint16_t* dout = static_cast<const uint16_t*>(a.dout);
    const long long rows = (long long)a.B * a.Hq * a.Sq;
    const int causal = a.causal != 0 || a.window > 0 ? 1 : 0;
    if (rows > 0)
        hipLaunchKernelGGL(bwd_rowdot_kernel<D>, dim3((unsigned)((rows * 16 + kBwdThreads - 1) / kBwdThreads)),
                           dim3(kBwdThreads), 0, stream, o, dout, a.dsum, rows);
    // 1-D grids of (blocks x heads x B) workgroups
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((a.Sk + kDkBlockRows - 1) / kDkBlockRows * a.Hkv * a.B),
                       dim3(kDkThreads), 0, stream, q, k, v, dout, a.lse, a.dsum, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), a.Hq, a.Hkv, a.Sq, a.Sk, a.scale, causal, a.window);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((a.Sq + kDqBlockRows - 1) / kDqBlockRows * a.Hq * a.B), dim3(kDqThreads),
                       0, stream, q, k, v, dout, a.lse, a.dsum, static_cast<uint16_t*>(a.dq), a.Hq, a.Hkv, a.Sq,
                       a.Sk, a.scale, causal, a.window);
    return hipGetLastError();
}

// fp32 backward on the vector ALU (the fp32 forward's counterpart, for
// small problems): one wavefront per row, lane l holding elements
// l, l + 64, ... of it; dot products reduce across the wavefront.
constexpr int kF32Waves = 4;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m, 64);
    return x;
}

// D = rowsum(dO * O) per query row.
template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void bwd_f32_rowdot_kernel(const float* __restrict__ o,
                                                                        const float* __restrict__ dout,
                                                                        float* __restrict__ dsum, long long rows) {
    constexpr int E = D / 64;
    const long long row = (long long)blockIdx.x * kF32Waves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;                               // whole wavefronts leave together
    float acc = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) acc = fmaf(o[row * D + lane + 64 * e], dout[row * D + lane + 64 * e], acc);
    acc = wave_sum(acc);
    if (lane == 0) dsum[row] = acc;
}

// dQ of one query row: sum over its visible keys j of dS_ij k_j.
template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void bwd_f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    float* __restrict__ dq, int Hq, int Hkv, int Sq, int Sk, float scale, int causal, int window, long long rows) {
    constexpr int E = D / 64;
    const long long row = (long long)blockIdx.x * kF32Waves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int i = (int)(row % Sq);
    const long long bh = row / Sq;                         // b * Hq + h
    const int h = (int)(bh % Hq), b = (int)(bh / Hq);
    const int hk = h / (Hq / Hkv);
    const int off = Sk - Sq;
    const float sl2 = scale * kLog2e, l2 = lse[row] * kLog2e, dd = dsum[row];
    float qv[E], ov[E], acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        qv[e] = q[row * D + lane + 64 * e];
        ov[e] = dout[row * D + lane + 64 * e];
        acc[e] = 0.f;
    }
    const int jend = causal ? min(Sk, i + off + 1) : Sk;
    const int jbeg = window > 0 ? max(0, i + off - window + 1) : 0;
    const float* kb = k + ((size_t)b * Hkv + hk) * Sk * D;
    const float* vb = v + ((size_t)b * Hkv + hk) * Sk * D;
    for (int j = jbeg; j < jend; ++j) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            s = fmaf(qv[e], kb[(size_t)j * D + lane + 64 * e], s);
            dp = fmaf(ov[e], vb[(size_t)j * D + lane + 64 * e], dp);
        }
        s = wave_sum(s);
        dp = wave_sum(dp);
        const float ds = exp2_fast(fmaf(s, sl2, -l2)) * (dp - dd);
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = fmaf(ds, kb[(size_t)j * D + lane + 64 * e], acc[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e) dq[row * D + lane + 64 * e] = acc[e] * scale;
}

// dK, dV of one key row: sums over the visible rows i of the g query heads
// reading it of dS_ij q_i and P_ij dO_i.
template <int D>
__global__ __launch_bounds__(64 * kF32Waves) void bwd_f32_dkdv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    float* __restrict__ dk, float* __restrict__ dv, int Hq, int Hkv, int Sq, int Sk, float scale, int causal,
    int window, long long rows) {
    constexpr int E = D / 64;
    const long long row = (long long)blockIdx.x * kF32Waves + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const int j = (int)(row % Sk);
    const long long bh = row / Sk;                         // b * Hkv + hk
    const int hk = (int)(bh % Hkv), b = (int)(bh / Hkv);
    const int g = Hq / Hkv;
    const int off = Sk - Sq;
    const float sl2 = scale * kLog2e;
    float kv[E], vv[E], ak[E], av[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        kv[e] = k[row * D + lane + 64 * e];
        vv[e] = v[row * D + lane + 64 * e];
        ak[e] = av[e] = 0.f;
    }
    // rows i that see key j: i >= j - off (causal), i < j - off + W (window)
    const int ibeg = causal ? max(0, j - off) : 0;
    const int iend = window > 0 ? min(Sq, j - off + window) : Sq;
    for (int hh = 0; hh < g; ++hh) {
        const size_t base = ((size_t)b * Hq + (size_t)hk * g + hh) * Sq;
        for (int i = ibeg; i < iend; ++i) {
            const float* qi = q + (base + i) * D;
            const float* oi = dout + (base + i) * D;
            float s = 0.f, dp = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                s = fmaf(qi[lane + 64 * e], kv[e], s);
                dp = fmaf(oi[lane + 64 * e], vv[e], dp);
            }
            s = wave_sum(s);
            dp = wave_sum(dp);
            const float p = exp2_fast(fmaf(s, sl2, -lse[base + i] * kLog2e));
            const float ds = p * (dp - dsum[base + i]);
#pragma unroll
            for (int e = 0; e < E; ++e) {
                av[e] = fmaf(p, oi[lane + 64 * e], av[e]);
                ak[e] = fmaf(ds, qi[lane + 64 * e], ak[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) {
        dk[row * D + lane + 64 * e] = ak[e] * scale;
        dv[row * D + lane + 64 * e] = av[e];
    }
}

template <int D>
hipError_t launch_bwd_f32(const BackwardArgs& a, hipStream_t stream) {
    const float* q = static_cast<const float*>(a.q);
    const float* k = static_cast<const float*>(a.k);
    const float* v = static_cast<const float*>(a.v);
    const float* dout = static_cast<const float*>(a.dout);
    const long long qrows = (long long)a.B * a.Hq * a.Sq, krows = (long long)a.B * a.Hkv * a.Sk;
    const int causal = a.causal != 0 || a.window > 0 ? 1 : 0;
    const dim3 blk(64 * kF32Waves);
    hipLaunchKernelGGL(bwd_f32_rowdot_kernel<D>, dim3((unsigned)((qrows + kF32Waves - 1) / kF32Waves)), blk, 0,
                       stream, static_cast<const float*>(a.o), dout, a.dsum, qrows);
    hipLaunchKernelGGL(bwd_f32_dq_kernel<D>, dim3((unsigned)((qrows + kF32Waves - 1) / kF32Waves)), blk, 0, stream,
                       q, k, v, dout, a.lse, a.dsum, static_cast<float*>(a.dq), a.Hq, a.Hkv, a.Sq, a.Sk, a.scale,
                       causal, a.window, qrows);
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<D>, dim3((unsigned)((krows + kF32Waves - 1) / kF32Waves)), blk, 0,
                       stream, q, k, v, dout, a.lse, a.dsum, static_cast<float*>(a.dk), static_cast<float*>(a.dv),
                       a.Hq, a.Hkv, a.Sq, a.Sk, a.scale, causal, a.window, krows);
    return hipGetLastError();
}

}  // namespace

// Sizes are validated by the caller: B, Hq, Hkv, Sq, Sk > 0, d in {64, 128}.
hipError_t launch_prefill_bwd_bf16(const BackwardArgs& a, hipStream_t stream) {
    return a.d == 64 ? launch_bwd<64>(a, stream) : launch_bwd<128>(a, stream);
}

hipError_t launch_prefill_bwd_f32(const BackwardArgs& a, hipStream_t stream) {
    return a.d == 64 ? launch_bwd_f32<64>(a, stream) : launch_bwd_f32<128>(a, stream);
}

}  // namespace gqa
