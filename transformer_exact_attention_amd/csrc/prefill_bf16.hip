// bf16 attention forward on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// The method: exact attention computed tile by tile with an online softmax, so
// the Sq x Sk score matrix never reaches device memory [Attention variants
// deep-dive, §6.2: tiling, forward pseudocode; Different attention
// mechanisms, §4 Flash Attention: tiling, kernel fusion, online softmax].
// Query head h reads K/V head h / g [Attention variants deep-dive, §5 GQA
// code], without copying K/V per query head (§5, the note after the code).
//
// Work decomposition (one workgroup = 4 wavefronts = 256 lanes):
//   * a workgroup owns one K/V head of one batch entry and 128 "query rows":
//     P = 128/g consecutive query positions x all g query heads of the group,
//     ordered position-major (row r -> position p0 + r/g, head hk*g + r%g);
//   * wavefront w owns rows 32w..32w+31; lane i owns query column n = i%32 and
//     lane half hh = i/32 (the MFMA operand split along the contraction);
//   * K/V tiles of 64 keys are staged row-major in LDS once per workgroup
//     (double-buffered, one barrier per tile) and serve all 128 rows: the g
//     query heads of a group share them.
//
// Per KV tile every wavefront computes the transposed score tile
//   S^T (64 keys x 32 queries) = K (64 x d) . Q^T (d x 32)
// so the 32x32 accumulator layout puts one query column in each lane: the
// running max / sum of a query live in that lane (and its partner i^32), and
// only one cross-lane exchange per tile is needed.  The probabilities are then
// already in the B-operand layout of
//   O^T (d x 32 queries) += V^T (d x 64 keys) . P^T (64 keys x 32 queries).
// The V^T operand (8 keys of one d per lane) is read from the row-major V tile
// with two transposing LDS reads (ds_read_b64_tr_b16): in each 16-lane group,
// lane l receives element l%4 of the 8-byte pieces addressed by lanes l/4,
// l/4+4, l/4+8, l/4+12, so pointing lane r of the group at key row r/4,
// columns 4*(r%4).. gives lane l four keys of column l.
//
// Softmax runs in base 2: scores are multiplied by scale*log2(e) in fp32 and
// exponentiated with v_exp_f32; exp(x) = 2^(x log2 e) changes only rounding.
// P is rounded to bf16 for the PV product; accumulation is fp32 throughout.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kBc = 64;        // keys per KV tile
constexpr int kRowsWG = 128;   // query rows per workgroup
constexpr int kThreads = 256;
constexpr float kRescaleSlack = 8.0f;   // base-2 units: p <= 256 between rescales

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// LDS tiles: K and V row-major [64 keys][D] bf16, 16-byte chunks XOR-swizzled
// against bank conflicts for their read patterns:
//   K: chunk c of key row r at chunk c ^ (r % chunks)    (reads: 32 rows, one chunk)
//   V: chunk c of key row r at chunk c ^ ((4 * (r & 3)) % chunks)
//      (transposing reads: 4 consecutive rows x 32 bytes per 16 lanes)
template <int D>
struct Lds {
    uint16_t ks[kBc * D];
    uint16_t vs[kBc * D];
};

template <int D>
__device__ __forceinline__ int k_byte(int r, int chunk) {
    return r * D * 2 + ((chunk ^ (r & (D / 8 - 1))) << 4);
}
template <int D>
__device__ __forceinline__ int v_byte(int r, int chunk) {
    return r * D * 2 + ((chunk ^ ((4 * (r & 3)) & (D / 8 - 1))) << 4);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, int Hq, int Hkv, int Sq, int Sk, int lg, int nqb,
    float scale_log2, int causal) {
    constexpr int kChunks = D / 8;          // 16-byte chunks per key row
    constexpr int kDSteps = D / 16;         // MFMA contraction steps over d
    constexpr int kDTiles = D / 32;         // 32-row output tiles of O^T
    constexpr int kLoads = kBc * kChunks / kThreads;   // 16-byte chunks per thread per tile (K and V each)
    constexpr int kTileBytes = kBc * D * 2;

    __shared__ __attribute__((aligned(16))) Lds<D> ldsbuf[2];
    lds_char* const lds0 = (lds_char*)&ldsbuf[0];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int g = 1 << lg;
    const int P = kRowsWG >> lg;            // query positions per workgroup

    // Work item of this workgroup.  Items are ordered plane by plane (plane =
    // (batch, K/V head)), heaviest query block first within a plane.  The
    // hardware hands consecutive workgroup ids to the 8 XCDs in turn, so
    // workgroup id L runs on XCD L % 8; when the item count divides by 8, XCD x
    // is given the contiguous item range [x * N/8, (x+1) * N/8): whole planes,
    // whose K/V then stay in that XCD's L2 instead of being fetched by all 8.
    const int nitems = (int)gridDim.x;
    const int L = (int)blockIdx.x;
    const int item = (nitems & 7) == 0 ? (L & 7) * (nitems >> 3) + (L >> 3) : L;
    const int plane = item / nqb;
    const int qb = nqb - 1 - (item - plane * nqb);
    const int hk = plane % Hkv;
    const int b = plane / Hkv;
    const int p0 = qb * P;

    // This lane's query column.
    const int r = wave * 32 + n;
    const int pos = p0 + (r >> lg);
    const int head = hk * g + (r & (g - 1));
    const bool qlive = pos < Sq;
    const int off = Sk - Sq;                // causal: key j visible iff j <= pos + off

    const size_t qrow = (((size_t)b * Hq + head) * Sq + (qlive ? pos : 0)) * D;
    const size_t kvbase = ((size_t)b * Hkv + hk) * (size_t)Sk * D;

    // Q^T operand fragments: lane holds Q[query n][16t + 8hh .. +8].
    bf16x8 qf[kDSteps];
#pragma unroll
    for (int t = 0; t < kDSteps; ++t) {
        u32x4 w = {0u, 0u, 0u, 0u};
        if (qlive) w = *reinterpret_cast<const u32x4*>(q + qrow + 16 * t + 8 * hh);
        qf[t] = __builtin_bit_cast(bf16x8, w);
    }

    // Keys this workgroup needs.
    const int p_last = min(p0 + P, Sq) - 1;
    const int kend = causal ? min(Sk, p_last + off + 1) : Sk;
    const int ntiles = (kend + kBc - 1) / kBc;
    const int my_last = causal ? pos + off : Sk - 1;          // last visible key of this column
    const int wg_first_last = causal ? min(p0 + off, Sk - 1) : Sk - 1;  // min over the workgroup

    // K/V plane of this (batch, K/V head); keys past Sk read as zeros.
    const __amdgpu_buffer_rsrc_t krsrc = make_rsrc(k + kvbase, (uint32_t)Sk * D * 2);
    const __amdgpu_buffer_rsrc_t vrsrc = make_rsrc(v + kvbase, (uint32_t)Sk * D * 2);

    // Staging: thread covers chunk sc of rows srow + x * kRowStep, for K and V alike.
    const int sc = tid % kChunks;
    const int srow = tid / kChunks;
    constexpr int kRowStep = kThreads / kChunks;
    u32x4 kreg[kLoads], vreg[kLoads];
    auto load_tile = [&](int j0) {
#pragma unroll
        for (int x = 0; x < kLoads; ++x) {
            const uint32_t eoff = (uint32_t)((j0 + srow + x * kRowStep) * D + 8 * sc) * 2;
            kreg[x] = buffer_load16(krsrc, eoff);
            vreg[x] = buffer_load16(vrsrc, eoff);
        }
    };
    auto store_tile = [&](int buf) {
        lds_char* const base = lds0 + buf * (int)sizeof(Lds<D>);
#pragma unroll
        for (int x = 0; x < kLoads; ++x) {
            const int row = srow + x * kRowStep;
            *(lds_u32x4*)(base + k_byte<D>(row, sc)) = kreg[x];
            *(lds_u32x4*)(base + kTileBytes + v_byte<D>(row, sc)) = vreg[x];
        }
    };

    // Transposed V reads: in 16-lane group G = lane/16, lane rr = lane%16 points
    // at key row 16s + 4*(G/2) + 8*piece + rr/4 and column 32t + 16*(G%2) + 4*(rr%4).
    const int G = lane >> 4, rr = lane & 15;
    const int vrow0 = 4 * (G >> 1) + (rr >> 2);
    const int vcol0 = 16 * (G & 1) + 4 * (rr & 3);

    f32x16 oacc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) oacc[t] = f32x16{};
    // Running reference max in scaled base-2 units.  It is raised only when a
    // tile's max exceeds it by more than kRescaleSlack (then the accumulator
    // and sum are rescaled); otherwise p = 2^(s*c - ref) <= 2^kRescaleSlack.
    // Softmax does not depend on the reference, so this is exact up to
    // rounding, and most tiles skip the O-accumulator rescale entirely.
    float ref = -INFINITY;
    float l = 0.f;           // running sum over this lane's keys

    if (ntiles > 0) {
        load_tile(0);
        store_tile(0);
    }
    // Nothing may stay in flight into the loop: the loop's first MFMA reads the
    // Q fragments, and a load still pending there would make every iteration
    // wait for the next tile's prefetch as well.
    wait_all_memory();
    __syncthreads();
    for (int kt = 0; kt < ntiles; ++kt) {
        const int j0 = kt * kBc;
        lds_char* const kb = lds0 + (kt & 1) * (int)sizeof(Lds<D>);
        lds_char* const vb = kb + kTileBytes;
        if (kt + 1 < ntiles) load_tile(j0 + kBc);        // in flight during this tile

        // S^T = K . Q^T for keys j0 .. j0+63 (two independent 32-key chains).
        f32x16 sacc[2] = {f32x16{}, f32x16{}};
#pragma unroll
        for (int t = 0; t < kDSteps; ++t) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const u32x4 w = *(lds_u32x4*)(kb + k_byte<D>(32 * u + n, 2 * t + hh));
                sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[t],
                                                                   sacc[u], 0, 0, 0);
            }
        }

        // Mask (only tiles crossing the causal diagonal or the key end), tile max.
        if ((j0 + kBc - 1) > wg_first_last) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int j = 0; j < 16; ++j) {
                    const int key = j0 + 32 * u + 8 * (j >> 2) + 4 * hh + (j & 3);
                    if (key > my_last) sacc[u][j] = -INFINITY;
                }
        }
        float tmax = sacc[0][0];
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int j = 0; j < 16; ++j) tmax = fmaxf(tmax, sacc[u][j]);
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64)) * scale_log2;
        const bool raise = tmax > ref + kRescaleSlack;
        if (__builtin_amdgcn_ballot_w64(raise)) {        // wave-uniform branch
            const float ref_new = raise ? tmax : ref;
            const float alpha = exp2_fast(ref - ref_new);  // 1 if kept, 0 on the first tile
            ref = ref_new;
            l *= alpha;
#pragma unroll
            for (int t = 0; t < kDTiles; ++t) oacc[t] *= alpha;
        }

        // P = 2^(s*c - ref), bf16 B-operand fragments for the four 16-key steps:
        // step s = 2u + half holds keys 16s + {4hh..4hh+3, 8+4hh..8+4hh+3}.
        bf16x8 pf[4];
        float psum4[4];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) p[e] = exp2_fast(fmaf(sacc[u][8 * half + e], scale_log2, -ref));
                psum4[2 * u + half] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
                u32x4 w;
                w.x = pack_bf16x2(p[0], p[1]);
                w.y = pack_bf16x2(p[2], p[3]);
                w.z = pack_bf16x2(p[4], p[5]);
                w.w = pack_bf16x2(p[6], p[7]);
                pf[2 * u + half] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l += (psum4[0] + psum4[1]) + (psum4[2] + psum4[3]);

        // O^T += V^T . P^T; the A operand of (t, s) is two transposed reads:
        // keys 16s + 4hh + 0..3 and 16s + 8 + 4hh + 0..3 of column 32t + n.
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int t = 0; t < kDTiles; ++t) {
                const int col = 32 * t + vcol0;
                const int row_a = 16 * s + vrow0;
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vb + v_byte<D>(row_a, col >> 3) + (col & 7) * 2));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4*)(vb + v_byte<D>(row_a + 8, col >> 3) + (col & 7) * 2));
                const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[s], oacc[t], 0, 0, 0);
            }
        }

        if (kt + 1 < ntiles) store_tile((kt + 1) & 1);
        __syncthreads();
    }

    // Epilogue: combine the lane pair's partial sums, normalise, store bf16.
    const float lt = l + __shfl_xor(l, 32, 64);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    if (qlive) {
        uint16_t* orow = o + qrow;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
#pragma unroll
            for (int grp = 0; grp < 4; ++grp) {
                const int d0 = 32 * t + 8 * grp + 4 * hh;
                u32x2 w;
                w.x = pack_bf16x2(oacc[t][4 * grp + 0] * inv, oacc[t][4 * grp + 1] * inv);
                w.y = pack_bf16x2(oacc[t][4 * grp + 2] * inv, oacc[t][4 * grp + 3] * inv);
                *reinterpret_cast<u32x2*>(orow + d0) = w;
            }
        }
    }
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream) {
    const int g = a.Hq / a.Hkv;
    int lg = 0;
    while ((1 << lg) < g) ++lg;
    const int P = kRowsWG >> lg;
    const int nqb = (a.Sq + P - 1) / P;
    dim3 grid(nqb * a.Hkv * a.B);
    const float sl = a.scale * kLog2e;
    const uint16_t* q = static_cast<const uint16_t*>(a.q);
    const uint16_t* k = static_cast<const uint16_t*>(a.k);
    const uint16_t* v = static_cast<const uint16_t*>(a.v);
    uint16_t* o = static_cast<uint16_t*>(a.o);
    if (a.d == 64)
        hipLaunchKernelGGL(prefill_bf16_kernel<64>, grid, dim3(kThreads), 0, stream, q, k, v, o, a.Hq,
                           a.Hkv, a.Sq, a.Sk, lg, nqb, sl, a.causal);
    else
        hipLaunchKernelGGL(prefill_bf16_kernel<128>, grid, dim3(kThreads), 0, stream, q, k, v, o, a.Hq,
                           a.Hkv, a.Sq, a.Sk, lg, nqb, sl, a.causal);
    return hipGetLastError();
}

}  // namespace gqa
