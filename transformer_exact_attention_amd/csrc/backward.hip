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
//   * dkdv: a workgroup owns 64 keys of one K/V head (a wavefront 16 of
//     them) and walks every query tile of the group's g heads, keeping dK and
//     dV in registers;
//   * dq: a workgroup owns 64 query rows of one head (a wavefront 16) and
//     walks the key tiles, keeping dQ^T in registers.
// Products are v_mfma_f32_16x16x16_bf16 (A: lane (c, q4) holds row c,
// k = 4 q4..4 q4+3; B: k = 4 q4..+3 of column c; D: rows 4 q4..+3 of column c,
// with c = lane % 16, q4 = lane / 16).  Tiles of 64 rows are staged in LDS
// with rows padded to D*2 + 16 bytes (row reads of 16 lanes hit distinct
// banks); column operands come from transposing LDS reads
// (ds_read_b64_tr_b16: lane r of a 16-lane group addressing row r/4,
// columns 4 (r%4).. delivers to lane l the four rows of column l).
// Each product computed in D layout is already the A or B layout of the
// product that consumes it: P (rows q, columns keys) is P^T's A layout, and
// dS^T (rows keys, columns q) is dQ^T's B layout.
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

__device__ __forceinline__ f32x4 mfma16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

template <int D>
struct Tile {
    static constexpr int kRowBytes = D * 2 + 16;
    static constexpr int kBytes = kTileRows * kRowBytes;
};

// 64 x D bf16 rows [row0, row0 + 64) of a [rows_total, D] matrix -> LDS tile
// (rows past rows_total are zero).  256 threads, 16-byte chunks.
template <int D>
__device__ __forceinline__ void load_rows(u32x4 (&reg)[kTileRows * D / 8 / kBwdThreads], const uint16_t* base,
                                          int row0, int rows_total) {
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int x = 0; x < kTileRows * kChunks / kBwdThreads; ++x) {
        const int i = x * kBwdThreads + (int)threadIdx.x;
        const int r = i / kChunks, c = i % kChunks;
        const int row = row0 + r;
        reg[x] = row < rows_total ? *reinterpret_cast<const u32x4*>(base + (size_t)row * D + 8 * c)
                                  : u32x4{0u, 0u, 0u, 0u};
    }
}
template <int D>
__device__ __forceinline__ void store_rows(lds_char* tile, const u32x4 (&reg)[kTileRows * D / 8 / kBwdThreads]) {
    constexpr int kChunks = D / 8;
#pragma unroll
    for (int x = 0; x < kTileRows * kChunks / kBwdThreads; ++x) {
        const int i = x * kBwdThreads + (int)threadIdx.x;
        const int r = i / kChunks, c = i % kChunks;
        *(lds_u32x4*)(tile + r * Tile<D>::kRowBytes + 16 * c) = reg[x];
    }
}
// A/B fragment from a row: 4 bf16 at (row, col..col+3).
template <int D>
__device__ __forceinline__ bf16x4 row_frag(const lds_char* tile, int row, int col) {
    return __builtin_bit_cast(bf16x4, *(const lds_u32x2*)(tile + row * Tile<D>::kRowBytes + 2 * col));
}
// Column fragment: rows r0 + 4 q4 .. +3 of column col0 + (lane % 16).
template <int D>
__device__ __forceinline__ bf16x4 col_frag(const lds_char* tile, int r0, int col0, int lane) {
    const int g = lane >> 4, r = lane & 15;
    const int row = r0 + 4 * g + (r >> 2);
    const int col = col0 + 4 * (r & 3);
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_s16x4*)(tile + row * Tile<D>::kRowBytes + 2 * col));
    return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x4 pack4(const f32x4& x) {
    const u32x2 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3])};
    return __builtin_bit_cast(bf16x4, w);
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

// dK, dV for 64 keys of K/V head hk of batch b.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int Hq, int Hkv, int Sq, int Sk, float scale,
    int causal, int window) {
    constexpr int kT = D / 16;                             // 16-wide d steps
    constexpr int kRegs = kTileRows * D / 8 / kBwdThreads;
    __shared__ __attribute__((aligned(16))) char q_raw[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char d_raw[2][Tile<D>::kBytes];
    __shared__ float lse_s[2][kTileRows], dsum_s[2][kTileRows];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, q4 = lane >> 4;
    const int kb = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int g = Hq / Hkv;
    const int off = Sk - Sq;
    const int key0 = kb * kTileRows + 16 * wave;           // this wavefront's keys key0 .. key0 + 15
    const float sl2 = scale * kLog2e;

    // K and V rows of the wavefront's keys as B operands (k = d, column = key c).
    bf16x4 kf[kT], vf[kT];
    {
        const size_t kvrow = ((size_t)b * Hkv + hk) * Sk;
        const int key = key0 + c;
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            u32x2 kw = {0u, 0u}, vw = {0u, 0u};
            if (key < Sk) {
                kw = *reinterpret_cast<const u32x2*>(k + (kvrow + key) * D + 16 * t + 4 * q4);
                vw = *reinterpret_cast<const u32x2*>(v + (kvrow + key) * D + 16 * t + 4 * q4);
            }
            kf[t] = __builtin_bit_cast(bf16x4, kw);
            vf[t] = __builtin_bit_cast(bf16x4, vw);
        }
    }
    f32x4 dka[kT], dva[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) dka[t] = dva[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Query tiles: for each head of the group, the tiles holding a row that
    // sees one of the workgroup's keys (causal: rows i >= key - off; window W:
    // also i < key - off + W).
    const int first_tile = causal ? max(0, kb * kTileRows - off) / kTileRows : 0;
    int end_tile = (Sq + kTileRows - 1) / kTileRows;
    if (window > 0) end_tile = min(end_tile, max(0, kb * kTileRows + kTileRows - 1 - off + window - 1) / kTileRows + 1);
    const int n_per_head = max(0, end_tile - first_tile);
    const int total = g * n_per_head;
    u32x4 qr[kRegs], dr[kRegs];
    auto fetch = [&](int it) {
        const int h = hk * g + it / n_per_head;
        const int row0 = (first_tile + it % n_per_head) * kTileRows;
        const size_t base = ((size_t)b * Hq + h) * Sq;
        load_rows<D>(qr, q + base * D, row0, Sq);
        load_rows<D>(dr, dout + base * D, row0, Sq);
    };
    auto stash = [&](int it, int buf) {
        const int h = hk * g + it / n_per_head;
        const int row0 = (first_tile + it % n_per_head) * kTileRows;
        const size_t base = ((size_t)b * Hq + h) * Sq;
        store_rows<D>((lds_char*)q_raw[buf], qr);
        store_rows<D>((lds_char*)d_raw[buf], dr);
        if (threadIdx.x < kTileRows) {
            const int row = row0 + threadIdx.x;
            // rows past Sq: lse = +inf makes their probabilities 0
            lse_s[buf][threadIdx.x] = row < Sq ? lse[base + row] * kLog2e : INFINITY;
            dsum_s[buf][threadIdx.x] = row < Sq ? dsum[base + row] : 0.f;
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
        const int row0 = (first_tile + it % n_per_head) * kTileRows;
        const lds_char* qt = (const lds_char*)q_raw[buf];
        const lds_char* dt = (const lds_char*)d_raw[buf];
#pragma unroll
        for (int sub = 0; sub < kTileRows / 16; ++sub) {
            const int r0 = 16 * sub;                        // query rows row0 + r0 .. +15
            // S (16 q x 16 keys) = Q K^T; dP = dO V^T
            f32x4 s = {0.f, 0.f, 0.f, 0.f}, dp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                s = mfma16(row_frag<D>(qt, r0 + c, 16 * t + 4 * q4), kf[t], s);
                dp = mfma16(row_frag<D>(dt, r0 + c, 16 * t + 4 * q4), vf[t], dp);
            }
            // lane holds rows q = r0 + 4 q4 + r of column key0 + c
            f32x4 p, ds;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int qi = r0 + 4 * q4 + r;
                const int pos = row0 + qi;
                const bool vis = (!causal || key0 + c <= pos + off) && (window <= 0 || key0 + c > pos + off - window);
                p[r] = vis ? exp2_fast(fmaf(s[r], sl2, -lse_s[buf][qi])) : 0.f;
                ds[r] = p[r] * (dp[r] - dsum_s[buf][qi]);
            }
            const bf16x4 pa = pack4(p), dsa = pack4(ds);   // P^T, dS^T as A operands (rows = keys)
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                dva[t] = mfma16(pa, col_frag<D>(dt, r0, 16 * t, lane), dva[t]);
                dka[t] = mfma16(dsa, col_frag<D>(qt, r0, 16 * t, lane), dka[t]);
            }
        }
        if (it + 1 < total) {
            __syncthreads();                                // everyone is done with the other buffer
            stash(it + 1, buf ^ 1);
            __syncthreads();
        }
    }
    // rows key0 + 4 q4 + r, columns 16 t + c
    const size_t kvrow = ((size_t)b * Hkv + hk) * Sk;
#pragma unroll
    for (int t = 0; t < kT; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int key = key0 + 4 * q4 + r;
            if (key < Sk) {
                const size_t at = (kvrow + key) * D + 16 * t + c;
                const uint32_t pk = pack_bf16x2(dka[t][r] * scale, dva[t][r]);
                dk[at] = (uint16_t)(pk & 0xffffu);
                dv[at] = (uint16_t)(pk >> 16);
            }
        }
}

// dQ for 64 query rows of head h of batch b.
template <int D>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ dsum,
    uint16_t* __restrict__ dq, int Hq, int Hkv, int Sq, int Sk, float scale, int causal, int window) {
    constexpr int kT = D / 16;
    constexpr int kRegs = kTileRows * D / 8 / kBwdThreads;
    __shared__ __attribute__((aligned(16))) char k_raw[2][Tile<D>::kBytes];
    __shared__ __attribute__((aligned(16))) char v_raw[2][Tile<D>::kBytes];

    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c = lane & 15, q4 = lane >> 4;
    const int qb = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int g = Hq / Hkv, hk = h / g;
    const int off = Sk - Sq;
    const int qrow = qb * kTileRows + 16 * wave + c;       // this lane's query column
    const float sl2 = scale * kLog2e;
    const size_t qbase = ((size_t)b * Hq + h) * Sq;

    // Q and dO of the lane's query as B operands (k = d, column = query c).
    bf16x4 qf[kT], of[kT];
#pragma unroll
    for (int t = 0; t < kT; ++t) {
        u32x2 qw = {0u, 0u}, ow = {0u, 0u};
        if (qrow < Sq) {
            qw = *reinterpret_cast<const u32x2*>(q + (qbase + qrow) * D + 16 * t + 4 * q4);
            ow = *reinterpret_cast<const u32x2*>(dout + (qbase + qrow) * D + 16 * t + 4 * q4);
        }
        qf[t] = __builtin_bit_cast(bf16x4, qw);
        of[t] = __builtin_bit_cast(bf16x4, ow);
    }
    const float lse2 = qrow < Sq ? lse[qbase + qrow] * kLog2e : INFINITY;
    const float dsq = qrow < Sq ? dsum[qbase + qrow] : 0.f;
    f32x4 dqa[kT];                                         // dQ^T: rows d = 16 t + 4 q4 + r, column = query c
#pragma unroll
    for (int t = 0; t < kT; ++t) dqa[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Key tiles seen by the block's rows (causal: keys <= row + off; window W:
    // also keys > row + off - W).
    const int q_last = min(qb * kTileRows + kTileRows, Sq) - 1;
    const int kend = causal ? min(Sk, q_last + off + 1) : Sk;
    const int kfirst = window > 0 ? max(0, qb * kTileRows + off - window + 1) / kTileRows : 0;
    const int ntiles = max(0, (kend + kTileRows - 1) / kTileRows - kfirst);
    const size_t kvbase = ((size_t)b * Hkv + hk) * Sk;
    u32x4 kr[kRegs], vr[kRegs];
    auto fetch = [&](int i) {
        load_rows<D>(kr, k + kvbase * D, (kfirst + i) * kTileRows, Sk);
        load_rows<D>(vr, v + kvbase * D, (kfirst + i) * kTileRows, Sk);
    };
    auto stash = [&](int buf) {
        store_rows<D>((lds_char*)k_raw[buf], kr);
        store_rows<D>((lds_char*)v_raw[buf], vr);
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
        for (int sub = 0; sub < kTileRows / 16; ++sub) {
            const int r0 = 16 * sub;                        // keys tile*64 + r0 .. +15
            // S^T (16 keys x 16 q) = K Q^T; dP^T = V dO^T
            f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int t = 0; t < kT; ++t) {
                st = mfma16(row_frag<D>(kt, r0 + c, 16 * t + 4 * q4), qf[t], st);
                dpt = mfma16(row_frag<D>(vt, r0 + c, 16 * t + 4 * q4), of[t], dpt);
            }
            // lane holds keys tile*64 + r0 + 4 q4 + r of column qrow
            f32x4 ds;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int key = tile * kTileRows + r0 + 4 * q4 + r;
                const bool vis = key < Sk && (!causal || key <= qrow + off) && (window <= 0 || key > qrow + off - window);
                const float p = vis ? exp2_fast(fmaf(st[r], sl2, -lse2)) : 0.f;
                ds[r] = p * (dpt[r] - dsq);
            }
            const bf16x4 dsb = pack4(ds);                   // dS^T as B operand (k = keys, column = query)
#pragma unroll
            for (int t = 0; t < kT; ++t) dqa[t] = mfma16(col_frag<D>(kt, r0, 16 * t, lane), dsb, dqa[t]);
        }
        if (it + 1 < ntiles) {
            __syncthreads();
            stash(buf ^ 1);
            __syncthreads();
        }
    }
    if (qrow < Sq) {
#pragma unroll
        for (int t = 0; t < kT; ++t) {
            const u32x2 w = {pack_bf16x2(dqa[t][0] * scale, dqa[t][1] * scale),
                             pack_bf16x2(dqa[t][2] * scale, dqa[t][3] * scale)};
            *reinterpret_cast<u32x2*>(dq + (qbase + qrow) * D + 16 * t + 4 * q4) = w;
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
    hipLaunchKernelGGL(bwd_dkdv_kernel<D>, dim3((a.Sk + kTileRows - 1) / kTileRows, a.Hkv, a.B),
                       dim3(kBwdThreads), 0, stream, q, k, v, dout, a.lse, a.dsum, static_cast<uint16_t*>(a.dk),
                       static_cast<uint16_t*>(a.dv), a.Hq, a.Hkv, a.Sq, a.Sk, a.scale, causal, a.window);
    hipLaunchKernelGGL(bwd_dq_kernel<D>, dim3((a.Sq + kTileRows - 1) / kTileRows, a.Hq, a.B), dim3(kBwdThreads),
                       0, stream, q, k, v, dout, a.lse, a.dsum, static_cast<uint16_t*>(a.dq), a.Hq, a.Hkv, a.Sq,
                       a.Sk, a.scale, causal, a.window);
    return hipGetLastError();
}

}  // namespace

// Sizes are validated by the caller: B, Hq, Hkv, Sq, Sk > 0, d in {64, 128}.
hipError_t launch_prefill_bwd_bf16(const BackwardArgs& a, hipStream_t stream) {
    return a.d == 64 ? launch_bwd<64>(a, stream) : launch_bwd<128>(a, stream);
}

}  // namespace gqa
