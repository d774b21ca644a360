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

// Block copies: row j of pair p copies row j of block src[p] to block
// dst[p], for K and V.  Pairs with an id outside [0, num_blocks) are skipped.
template <int U>
__global__ __launch_bounds__(kThreadsKV) void kv_copy_blocks_kernel(u32x4* __restrict__ kc, u32x4* __restrict__ vc,
                                                                    const int32_t* __restrict__ src,
                                                                    const int32_t* __restrict__ dst,
                                                                    long long total, int rows_per_block,
                                                                    int num_blocks) {
    const long long stride = (long long)gridDim.x * kThreadsKV;
    for (long long base = (long long)blockIdx.x * kThreadsKV + threadIdx.x; base < total;
         base += stride * kItemsKV) {
        u32x4 kx[kItemsKV], vx[kItemsKV];
        long long to[kItemsKV];
#pragma unroll
        for (int r = 0; r < kItemsKV; ++r) {
            const long long i = base + r * stride;
            to[r] = -1;
            if (i < total) {
                const int row = (int)(i / U);                // pair * rows_per_block + row (< 2^31)
                const int u = (int)(i - (long long)row * U);
                const int p = row / rows_per_block;
                const int jr = row - p * rows_per_block;
                const int a = src[p], b = dst[p];
                if (a >= 0 && a < num_blocks && b >= 0 && b < num_blocks) {
                    to[r] = ((long long)b * rows_per_block + jr) * U + u;
                    const long long from = ((long long)a * rows_per_block + jr) * U + u;
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
    const int U = a.row_bytes / 16;
    const int rows_per_block = a.Hkv * 16;
    const long long total = (long long)a.n * rows_per_block * U;
    u32x4* kc = static_cast<u32x4*>(a.k_cache);
    u32x4* vc = static_cast<u32x4*>(a.v_cache);
    const dim3 grid(kv_grid(total));
    if (U == 8)
        hipLaunchKernelGGL(kv_copy_blocks_kernel<8>, grid, dim3(kThreadsKV), 0, stream, kc, vc, a.src, a.dst, total,
                           rows_per_block, a.num_blocks);
    else if (U == 16)
        hipLaunchKernelGGL(kv_copy_blocks_kernel<16>, grid, dim3(kThreadsKV), 0, stream, kc, vc, a.src, a.dst, total,
                           rows_per_block, a.num_blocks);
    else
        hipLaunchKernelGGL(kv_copy_blocks_kernel<32>, grid, dim3(kThreadsKV), 0, stream, kc, vc, a.src, a.dst, total,
                           rows_per_block, a.num_blocks);
    return hipGetLastError();
}

}  // namespace gqa
