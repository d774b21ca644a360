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
//   * K/V tiles of 64 keys are staged in LDS once per workgroup and serve all
//     128 rows (g query heads share them).
//
// Per KV tile every wavefront computes the transposed score tile
//   S^T (64 keys x 32 queries) = K (64 x d) . Q^T (d x 32)
// so the 32x32 accumulator layout puts one query column in each lane: the
// running max / sum of a query live in that lane (and its partner i^32), and
// only one cross-lane exchange per tile is needed.  The probabilities are then
// already in the B-operand layout of
//   O^T (d x 32 queries) += V^T (d x 64 keys) . P^T (64 keys x 32 queries)
// provided V is stored transposed in LDS with the keys of each 16-key group
// permuted to match the accumulator's row order; that transpose is done once
// per tile per workgroup while staging.
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

// LDS layouts (bf16 elements, 16-byte chunks XOR-swizzled against bank conflicts).
//   Ks : [64 keys][D]   chunk c of row r stored at chunk c ^ (r & 7)
//   Vt : [D][64 keys]   (keys permuted inside 16-key groups), chunk c of row r
//                       stored at chunk c ^ ((r ^ (r >> 3)) & 7)
template <int D>
struct Lds {
    uint16_t ks[kBc * D];
    uint16_t vt[D * kBc];
};

__device__ __forceinline__ int ks_off(int D, int r, int chunk) {
    return r * D + ((chunk ^ (r & 7)) << 3);
}
__device__ __forceinline__ int vt_off(int r, int chunk) {
    return r * kBc + ((chunk ^ ((r ^ (r >> 3)) & 7)) << 3);
}

// Storage slot of the first key of 4-key group `sub` inside a 16-key group:
// keys {0-3, 8-11 | 4-7, 12-15} so that lane half hh finds its 8 keys of a
// 16-key MFMA step contiguous at slots 8*hh .. 8*hh+7.
__device__ __forceinline__ int perm4(int sub) { return ((sub & 1) << 3) | ((sub & 2) << 1); }

template <int D>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    uint16_t* __restrict__ o, int Hq, int Hkv, int Sq, int Sk, int lg, int nqb,
    float scale_log2, int causal) {
    constexpr int kChunks = D / 8;          // 16-byte chunks per K row
    constexpr int kDSteps = D / 16;         // MFMA contraction steps over d
    constexpr int kDTiles = D / 32;         // 32-row output tiles of O^T
    constexpr int kKLoads = kBc * kChunks / kThreads;        // K chunks per thread
    constexpr int kVUnits = (kBc / 4) * kChunks;             // (4-key group, chunk) units
    constexpr int kVLoads = (kVUnits + kThreads - 1) / kThreads;

    __shared__ Lds<D> lds;

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int n = lane & 31;
    const int hh = lane >> 5;
    const int g = 1 << lg;
    const int P = kRowsWG >> lg;            // query positions per workgroup

    // Heaviest (latest) query blocks first: causal rows there see the most keys.
    const int qb = nqb - 1 - (int)blockIdx.x;
    const int hk = blockIdx.y;
    const int b = blockIdx.z;
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

    // Staging registers (next tile prefetch).
    u32x4 kreg[kKLoads];
    u32x4 vreg[kVLoads][4];

    auto load_tile = [&](int j0) {
#pragma unroll
        for (int x = 0; x < kKLoads; ++x) {
            const int e = tid + x * kThreads;
            const int row = e / kChunks, c = e % kChunks;
            const int key = j0 + row;
            u32x4 w = {0u, 0u, 0u, 0u};
            if (key < Sk) w = *reinterpret_cast<const u32x4*>(k + kvbase + (size_t)key * D + 8 * c);
            kreg[x] = w;
        }
#pragma unroll
        for (int x = 0; x < kVLoads; ++x) {
            const int u = tid + x * kThreads;
            const int g4 = u / kChunks, c = u % kChunks;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int key = j0 + 4 * g4 + rr;
                u32x4 w = {0u, 0u, 0u, 0u};
                if (u < kVUnits && key < Sk)
                    w = *reinterpret_cast<const u32x4*>(v + kvbase + (size_t)key * D + 8 * c);
                vreg[x][rr] = w;
            }
        }
    };

    auto store_tile = [&]() {
#pragma unroll
        for (int x = 0; x < kKLoads; ++x) {
            const int e = tid + x * kThreads;
            const int row = e / kChunks, c = e % kChunks;
            *reinterpret_cast<u32x4*>(&lds.ks[ks_off(D, row, c)]) = kreg[x];
        }
#pragma unroll
        for (int x = 0; x < kVLoads; ++x) {
            const int u = tid + x * kThreads;
            if (u < kVUnits) {
                const int g4 = u / kChunks, c = u % kChunks;
                const int slot = 16 * (g4 >> 2) + perm4(g4 & 3);     // first key's slot
                const int chunk = slot >> 3, half = (slot >> 2) & 1;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int dw = e >> 1;
                    u32x2 out;
                    if (e & 1) {
                        out.x = pack_hi16(vreg[x][0][dw], vreg[x][1][dw]);
                        out.y = pack_hi16(vreg[x][2][dw], vreg[x][3][dw]);
                    } else {
                        out.x = pack_lo16(vreg[x][0][dw], vreg[x][1][dw]);
                        out.y = pack_lo16(vreg[x][2][dw], vreg[x][3][dw]);
                    }
                    const int row = 8 * c + e;
                    *reinterpret_cast<u32x2*>(&lds.vt[vt_off(row, chunk) + 4 * half]) = out;
                }
            }
        }
    };

    f32x16 oacc[kDTiles];
#pragma unroll
    for (int t = 0; t < kDTiles; ++t) oacc[t] = f32x16{};
    float m = -INFINITY;     // running max (base-2 scaled units)
    float l = 0.f;           // running sum over this lane's keys

    if (ntiles > 0) load_tile(0);
    for (int kt = 0; kt < ntiles; ++kt) {
        const int j0 = kt * kBc;
        __syncthreads();                      // previous tile fully consumed
        store_tile();
        __syncthreads();
        if (kt + 1 < ntiles) load_tile(j0 + kBc);

        // S^T = K . Q^T for keys j0 .. j0+63 (two 32-key tiles).
        f32x16 sacc[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            sacc[u] = f32x16{};
            const int krow = 32 * u + n;
#pragma unroll
            for (int t = 0; t < kDSteps; ++t) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(&lds.ks[ks_off(D, krow, 2 * t + hh)]);
                sacc[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), qf[t],
                                                                   sacc[u], 0, 0, 0);
            }
        }

        // Scale, mask, tile max.
        const bool need_mask = (j0 + kBc - 1) > wg_first_last;
        float tmax = -INFINITY;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                float s = sacc[u][j] * scale_log2;
                if (need_mask) {
                    const int key = j0 + 32 * u + 8 * (j >> 2) + 4 * hh + (j & 3);
                    if (key > my_last) s = -INFINITY;
                }
                sacc[u][j] = s;
                tmax = fmaxf(tmax, s);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m, tmax);
        const float alpha = exp2_fast(m - m_new);      // 0 on the first tile (m = -inf)
        m = m_new;

        // P = 2^(s - m), bf16 B-operand fragments for the four 16-key steps.
        bf16x8 pf[4];
        float psum = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u) {
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                float p[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    p[e] = exp2_fast(sacc[u][8 * half + e] - m_new);
                    psum += p[e];
                }
                u32x4 w;
                w.x = pack_bf16x2(p[0], p[1]);
                w.y = pack_bf16x2(p[2], p[3]);
                w.z = pack_bf16x2(p[4], p[5]);
                w.w = pack_bf16x2(p[6], p[7]);
                pf[2 * u + half] = __builtin_bit_cast(bf16x8, w);
            }
        }
        l = l * alpha + psum;
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) oacc[t] *= alpha;

        // O^T += V^T . P^T
#pragma unroll
        for (int t = 0; t < kDTiles; ++t) {
            const int vrow = 32 * t + n;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(&lds.vt[vt_off(vrow, 2 * s + hh)]);
                oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w), pf[s],
                                                                   oacc[t], 0, 0, 0);
            }
        }
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
    dim3 grid(nqb, a.Hkv, a.B);
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
