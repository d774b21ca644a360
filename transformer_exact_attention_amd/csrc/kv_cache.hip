// Paged KV cache: writing new tokens into their pages, and copy-on-write
// block copies.
//
// The cache is cut into fixed-size blocks of 16 tokens placed anywhere in
// device memory; a token's place is its physical slot s = block * 16 + offset,
// taken from the sequence's page table when the token arrives, so nothing
// already cached ever moves [Different attention mechanisms, §5 Page
// Attention, steps 1-3].  Sequences sharing a prefix share its blocks; a
// shared, partly filled block is copied before a sequence writes into it
// (same section, advantages: copy-on-write).
//
// Both kernels only move bytes, so they are written over 16-byte units: a
// head row of d elements is U = d * element size / 16 units, and a physical
// block holds Hkv * 16 rows.  Pages are [num_blocks, Hkv, 16, d]; new tokens
// arrive as [n_tokens, Hkv, d].  They are bound by device memory: every
// source byte is read once and every destination byte written once.  The
// append streams both ways non-temporally (a bulk write of a prompt's K/V
// far exceeds the caches; measured 5 % faster than cached stores, and within
// 3 % of a plain device copy of the same bytes); the block copies keep their
// stores cached, since the next token is written into the copy right after.
// A wavefront moves 64 consecutive units of the source, i.e. whole rows
// (U = 8, 16 or 32 divides 64), and each row lands as one contiguous run of
// d * element size bytes.
#include "common.hpp"
#include "launch.hpp"

namespace gqa {

namespace {

constexpr int kThreadsKV = 256;
constexpr int kItemsKV = 4;   // units per thread per round: their loads are all issued before any store

__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }

// Token units: item i of the flattened [n_tokens, Hkv, U] source goes to
// row (slot / 16, h, slot % 16) of the pages.  Out-of-range slots (padding
// tokens carry -1) are skipped.
template <int U>
__global__ __launch_bounds__(kThreadsKV) void kv_append_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                               const u32x4* __restrict__ kn,
                                                               const u32x4* __restrict__ vn,
                                                               const int32_t* __restrict__ slots, long long total,
                                                               long long num_slots, int Hkv) {
    const long long stride = (long long)gridDim.x * kThreadsKV;
    for (long long base = (long long)blockIdx.x * kThreadsKV + threadIdx.x; base < total;
         base += stride * kItemsKV) {
        u32x4 kx[kItemsKV], vx[kItemsKV];
        long long dst[kItemsKV];
#pragma unroll
        for (int r = 0; r < kItemsKV; ++r) {
            const long long i = base + r * stride;
            dst[r] = -1;
            if (i < total) {
                const int row = (int)(i / U);                // token * Hkv + head (< 2^31)
                const int u = (int)(i - (long long)row * U);
                const int t = row / Hkv;
                const int h = row - t * Hkv;
                const long long s = slots[t];
                if (s >= 0 && s < num_slots) {
                    dst[r] = (((s >> 4) * Hkv + h) * 16 + (s & 15)) * U + u;
                    kx[r] = load_stream(kn + i);
                    vx[r] = load_stream(vn + i);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kItemsKV; ++r) {
            if (dst[r] >= 0) {
                __builtin_nontemporal_store(kx[r], kc + dst[r]);
                __builtin_nontemporal_store(vx[r], vc + dst[r]);
            }
        }
    }
}

// Block copies: unit j of pair p copies unit j of block src[p] to block
// dst[p] in both arrays (K and V codes or rows, or their per-row scales).
// Pairs with an id outside [0, num_blocks) are skipped.  total < 2^31.
__global__ __launch_bounds__(kThreadsKV) void kv_copy_blocks_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                                    const int32_t* __restrict__ src,
                                                                    const int32_t* __restrict__ dst, int total,
                                                                    int per_block, int num_blocks) {
    const int stride = (int)gridDim.x * kThreadsKV;
    for (int base = (int)blockIdx.x * kThreadsKV + (int)threadIdx.x; base < total; base += stride * kItemsKV) {
        u32x4 kx[kItemsKV], vx[kItemsKV];
        long long to[kItemsKV];
#pragma unroll
        for (int r = 0; r < kItemsKV; ++r) {
            const long long i = (long long)base + (long long)r * stride;
            to[r] = -1;
            if (i < total) {
                const int p = (int)i / per_block;
                const int j = (int)i - p * per_block;
                const int a = src[p], b = dst[p];
                if (a >= 0 && a < num_blocks && b >= 0 && b < num_blocks) {
                    to[r] = (long long)b * per_block + j;
                    const long long from = (long long)a * per_block + j;
                    kx[r] = kc[from];
                    vx[r] = vc[from];
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kItemsKV; ++r) {
            if (to[r] >= 0) {
                kc[to[r]] = kx[r];
                vc[to[r]] = vx[r];
            }
        }
    }
}

// E4M3 code (OCP 8-bit: sign, 4 exponent bits with bias 7, 3 mantissa bits,
// subnormals m * 2^-9, largest finite 448) of a finite fp32 value: the
// nearest E4M3 value, ties to the even code, magnitudes past 448 giving 448,
// the sign bit copied.  Below 2^-6 the codes are the subnormal multiples of
// 2^-9 (a * 512 is exact, rint rounds half to even); above, the fp32 pattern
// keeps 3 mantissa bits, rounded to nearest even on the 20 it drops, and the
// exponent is rebased from 127 to 7 (a carry out of the mantissa moves into
// the exponent, as it should).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fminf(fabsf(y), 448.0f);
    const uint32_t ab = __float_as_uint(a);
    const uint32_t normal = ((ab + 0x7FFFFu + ((ab >> 20) & 1u)) >> 20) - ((127u - 7u) << 3);
    const uint32_t sub = (uint32_t)__builtin_rintf(a * 512.0f);
    return sign | (a < 0.015625f ? sub : normal);
}

// Quantising append for fp8 caches (d = 128, bf16 input): 16 lanes per row,
// 8 elements each.  A row's scale is amax / 448 and its codes are those of
// x * (448 / amax), both in fp32 rounded to nearest even (zeros: scale 0).
// The 16 lanes of a row are always active together, so the row maximum is
// a butterfly within them.
__global__ __launch_bounds__(kThreadsKV) void kv_append_fp8_kernel(uint8_t* __restrict__ kc, uint8_t* __restrict__ vc,
                                                                   float* __restrict__ ks, float* __restrict__ vs,
                                                                   const u32x4* __restrict__ kn,
                                                                   const u32x4* __restrict__ vn,
                                                                   const int32_t* __restrict__ slots, int rows,
                                                                   long long num_slots, int Hkv) {
    const int stride = (int)gridDim.x * kThreadsKV;
    for (long long i = (long long)blockIdx.x * kThreadsKV + threadIdx.x; i < (long long)rows * 16; i += stride) {
        const int row = (int)(i >> 4);          // token * Hkv + head
        const int sub = (int)(i & 15);
        const int t = row / Hkv;
        const int h = row - t * Hkv;
        const long long s = slots[t];
        const u32x4 kw = load_stream(kn + i);
        const u32x4 vw = load_stream(vn + i);
        float kx[8], vx[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            kx[2 * e] = bf16_lo_to_f32(kw[e]);
            kx[2 * e + 1] = bf16_hi_to_f32(kw[e]);
            vx[2 * e] = bf16_lo_to_f32(vw[e]);
            vx[2 * e + 1] = bf16_hi_to_f32(vw[e]);
        }
        float ka = 0.f, va = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ka = fmaxf(ka, fabsf(kx[e]));
            va = fmaxf(va, fabsf(vx[e]));
        }
#pragma unroll
        for (int m = 1; m < 16; m <<= 1) {
            ka = fmaxf(ka, __shfl_xor(ka, m, 64));
            va = fmaxf(va, __shfl_xor(va, m, 64));
        }
        if (s < 0 || s >= num_slots) continue;
        const float kinv = ka > 0.f ? 448.0f / ka : 0.f;
        const float vinv = va > 0.f ? 448.0f / va : 0.f;
        u32x2 kq = {0u, 0u}, vq = {0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kq[e >> 2] |= e4m3_code(kx[e] * kinv) << (8 * (e & 3));
            vq[e >> 2] |= e4m3_code(vx[e] * vinv) << (8 * (e & 3));
        }
        const long long r = ((s >> 4) * Hkv + h) * 16 + (s & 15);     // destination row
        __builtin_nontemporal_store(kq, reinterpret_cast<u32x2*>(kc + r * 128 + 8 * sub));
        __builtin_nontemporal_store(vq, reinterpret_cast<u32x2*>(vc + r * 128 + 8 * sub));
        if (sub == 0) {
            ks[r] = ka / 448.0f;
            vs[r] = va / 448.0f;
        }
    }
}

// Enough workgroups to keep every CU busy with several rounds in flight;
// the loops stride over the rest.
int kv_grid(long long total) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    const long long need = (total + (long long)kThreadsKV * kItemsKV - 1) / ((long long)kThreadsKV * kItemsKV);
    const long long cap = (long long)cus * 16;
    return (int)(need < cap ? (need > 0 ? need : 1) : cap);
}

}  // namespace

hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream) {
    const int U = a.row_bytes / 16;
    const long long total = (long long)a.n_tokens * a.Hkv * U;
    const long long num_slots = (long long)a.num_blocks * 16;
    u32x4* kc = static_cast<u32x4*>(a.k_cache);
    u32x4* vc = static_cast<u32x4*>(a.v_cache);
    const u32x4* kn = static_cast<const u32x4*>(a.k_new);
    const u32x4* vn = static_cast<const u32x4*>(a.v_new);
    const dim3 grid(kv_grid(total));
    if (U == 8)
        hipLaunchKernelGGL(kv_append_kernel<8>, grid, dim3(kThreadsKV), 0, stream, kc, vc, kn, vn, a.slots, total,
                           num_slots, a.Hkv);
    else if (U == 16)
        hipLaunchKernelGGL(kv_append_kernel<16>, grid, dim3(kThreadsKV), 0, stream, kc, vc, kn, vn, a.slots, total,
                           num_slots, a.Hkv);
    else
        hipLaunchKernelGGL(kv_append_kernel<32>, grid, dim3(kThreadsKV), 0, stream, kc, vc, kn, vn, a.slots, total,
                           num_slots, a.Hkv);
    return hipGetLastError();
}

hipError_t launch_kv_copy_blocks(const KvCopyArgs& a, hipStream_t stream) {
    const int per_block = a.Hkv * 16 * (a.row_bytes / 16);
    const int total = a.n * per_block;
    hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3(kv_grid(total)), dim3(kThreadsKV), 0, stream,
                       static_cast<u32x4*>(a.k_cache), static_cast<u32x4*>(a.v_cache), a.src, a.dst, total, per_block,
                       a.num_blocks);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || !a.k_scale) return e;
    // per-row scales of fp8 caches: Hkv * 16 floats per block
    const int per_block_s = a.Hkv * 16 * 4 / 16;
    hipLaunchKernelGGL(kv_copy_blocks_kernel, dim3(kv_grid((long long)a.n * per_block_s)), dim3(kThreadsKV), 0, stream,
                       reinterpret_cast<u32x4*>(a.k_scale), reinterpret_cast<u32x4*>(a.v_scale), a.src, a.dst,
                       a.n * per_block_s, per_block_s, a.num_blocks);
    return hipGetLastError();
}

hipError_t launch_kv_append_fp8(const KvAppendArgs& a, hipStream_t stream) {
    const int rows = a.n_tokens * a.Hkv;
    hipLaunchKernelGGL(kv_append_fp8_kernel, dim3(kv_grid((long long)rows * 16)), dim3(kThreadsKV), 0, stream,
                       static_cast<uint8_t*>(a.k_cache), static_cast<uint8_t*>(a.v_cache), a.k_scale, a.v_scale,
                       static_cast<const u32x4*>(a.k_new), static_cast<const u32x4*>(a.v_new), a.slots, rows,
                       (long long)a.num_blocks * 16, a.Hkv);
    return hipGetLastError();
}

}  // namespace gqa
