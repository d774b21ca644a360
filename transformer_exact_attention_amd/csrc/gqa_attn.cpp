// C ABI of libgqa_attn: host-side validation, planning and kernel launch.
//
// Every check runs on the host before the first HIP call, so a rejected call
// enqueues nothing.  These calls allocate nothing; the only state is the
// per-device address of the allocation-free decode's static scratch.
#include "../../include/gqa_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <new>
#include <vector>

#include "launch.hpp"

namespace {

constexpr int64_t kMaxPlane = (int64_t)1 << 31;   // elements per (b, head) plane
static_assert(GQA_DECODE_NOALLOC_MAX_BYTES == gqa::kDecodeStaticScratchBytes,
              "the header's limit is the size of the static scratch");

bool pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool valid_scale(float s) { return std::isfinite(s) && s > 0.f; }

// Sizes shared by both calls.  Query heads must be a multiple of K/V heads
// [Attention variants deep-dive, §5 GQA code: the divisibility assertion].
int check_heads(int B, int Hq, int Hkv, int d) {
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return GQA_ERR_INVALID_ARG;
    if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
    return GQA_OK;
}

int prefill_check(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                  int Sk, int d, float scale, int causal, int dtype) {
    if (!q || !k || !v || !o) return GQA_ERR_INVALID_ARG;
    int st = check_heads(B, Hq, Hkv, d);
    if (st != GQA_OK) return st;
    if (Sq <= 0 || Sk <= 0) return GQA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return GQA_ERR_INVALID_ARG;
    if (causal != 0 && Sq > Sk) return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
    if ((int64_t)Sq * d >= kMaxPlane || (int64_t)Sk * d >= kMaxPlane) return GQA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return GQA_ERR_UNSUPPORTED;
    if (dtype == GQA_BF16) {
        const int g = Hq / Hkv;
        if (!pow2(g) || g > 128) return GQA_ERR_UNSUPPORTED;
        // one workgroup per (query block, K/V head, batch entry) in a 1-D grid
        if ((int64_t)Sq * Hkv * B >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;
    } else {
        if (Hq > 65535 || B > 65535) return GQA_ERR_UNSUPPORTED;
    }
    return GQA_OK;
}

// Everything but the workspace.
int decode_check_args(const void* q, const void* kc, const void* vc, void* o, const int32_t* seq_lens,
                      const int32_t* block_table, int B, int Hq, int Hkv, int d, int max_seq_len,
                      int block_size, int max_blocks_per_seq, float scale, int dtype) {
    if (!q || !kc || !vc || !o || !seq_lens) return GQA_ERR_INVALID_ARG;
    int st = check_heads(B, Hq, Hkv, d);
    if (st != GQA_OK) return st;
    if (max_seq_len <= 0) return GQA_ERR_INVALID_ARG;
    if (!valid_scale(scale)) return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
    if (block_table) {
        if (block_size != GQA_PAGE_BLOCK_SIZE) return GQA_ERR_INVALID_ARG;
        if (max_blocks_per_seq <= 0) return GQA_ERR_INVALID_ARG;
        if ((int64_t)max_blocks_per_seq * block_size < max_seq_len) return GQA_ERR_INVALID_ARG;
    }
    if (dtype != GQA_BF16 || (d != 64 && d != 128)) return GQA_ERR_UNSUPPORTED;
    const int g = Hq / Hkv;
    if (!pow2(g) || g > 32) return GQA_ERR_UNSUPPORTED;
    if (B > gqa::kDecodeMaxBatch || Hq > 65535) return GQA_ERR_UNSUPPORTED;
    return GQA_OK;
}

int decode_check(const void* q, const void* kc, const void* vc, void* o, const int32_t* seq_lens,
                 const int32_t* block_table, int B, int Hq, int Hkv, int d, int max_seq_len,
                 int block_size, int max_blocks_per_seq, float scale, int dtype, const void* workspace,
                 size_t workspace_bytes) {
    const int st = decode_check_args(q, kc, vc, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len, block_size,
                                     max_blocks_per_seq, scale, dtype);
    if (st != GQA_OK) return st;
    if (!workspace) return GQA_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GQA_ERR_WORKSPACE;
    if (workspace_bytes < gqa::decode_workspace_bytes(B, Hq, d, max_seq_len)) return GQA_ERR_WORKSPACE;
    return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_attn_abi_version(void) { return GQA_ATTN_ABI_VERSION; }

const char* gqa_attn_status_string(int status) {
    switch (status) {
        case GQA_OK: return "ok";
        case GQA_ERR_INVALID_ARG: return "invalid argument";
        case GQA_ERR_UNSUPPORTED: return "unsupported configuration";
        case GQA_ERR_WORKSPACE:
            return "workspace missing, misaligned or too small (attn_decode_fwd_noalloc: the sizes need more "
                   "than its static scratch of GQA_DECODE_NOALLOC_MAX_BYTES)";
        case GQA_ERR_HIP: return "HIP runtime error";
        case GQA_ERR_OUT_OF_BLOCKS: return "KV pool exhausted (free blocks or sequence ids)";
        default: return "unknown status";
    }
}

int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                     int Sk, int d, float scale, int causal, int dtype, void* stream) {
    const int st = prefill_check(q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, causal, dtype);
    if (st != GQA_OK) return st;
    gqa::PrefillArgs a{q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, causal != 0 ? 1 : 0};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == GQA_F32 ? gqa::launch_prefill_f32(a, s) : gqa::launch_prefill_bf16(a, s);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_prefill_window_fwd(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Sq,
                            int Sk, int d, float scale, int window, int dtype, void* stream) {
    const int st = prefill_check(q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, 1, dtype);
    if (st != GQA_OK) return st;
    if (window <= 0) return GQA_ERR_INVALID_ARG;
    gqa::PrefillArgs a{q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, 1, window};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == GQA_F32 ? gqa::launch_prefill_f32(a, s) : gqa::launch_prefill_bf16(a, s);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_prefill_lse_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                         int Sq, int Sk, int d, float scale, int causal, int window, int dtype, void* stream) {
    if (!lse || window < 0) return GQA_ERR_INVALID_ARG;
    const int causal_eff = causal != 0 || window > 0 ? 1 : 0;
    const int st = prefill_check(q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, causal_eff, dtype);
    if (st != GQA_OK) return st;
    gqa::PrefillArgs a{q, k, v, o, B, Hq, Hkv, Sq, Sk, d, scale, causal_eff, window, lse};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == GQA_F32 ? gqa::launch_prefill_f32(a, s) : gqa::launch_prefill_bf16(a, s);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

size_t attn_prefill_bwd_workspace_bytes(int B, int Hq, int Sq) {
    if (B <= 0 || Hq <= 0 || Sq <= 0) return 0;
    return gqa::align256((size_t)B * Hq * Sq * sizeof(float));
}

int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                     void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, float scale,
                     int causal, int window, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (!o || !lse || !dout || !dq || !dk || !dv || window < 0) return GQA_ERR_INVALID_ARG;
    const int causal_eff = causal != 0 || window > 0 ? 1 : 0;
    // o only marks the output argument of the shared check; q, k, v are read.
    const int st = prefill_check(q, k, v, dq, B, Hq, Hkv, Sq, Sk, d, scale, causal_eff, dtype);
    if (st != GQA_OK) return st;
    if ((int64_t)B * Hq * Sq >= ((int64_t)1 << 27)) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)(Sk + 127) / 128 * Hkv * B >= ((int64_t)1 << 31)) return GQA_ERR_UNSUPPORTED;   // 1-D grid
    if (!workspace || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GQA_ERR_WORKSPACE;
    if (workspace_bytes < attn_prefill_bwd_workspace_bytes(B, Hq, Sq)) return GQA_ERR_WORKSPACE;
    gqa::BackwardArgs a{q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace),
                        B, Hq, Hkv, Sq, Sk, d, scale, causal_eff, window};
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const hipError_t e = dtype == GQA_F32 ? gqa::launch_prefill_bwd_f32(a, s) : gqa::launch_prefill_bwd_bf16(a, s);
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

size_t attn_decode_workspace_bytes(int B, int Hq, int d, int max_seq_len) {
    if (B <= 0 || Hq <= 0 || d <= 0 || max_seq_len <= 0) return 0;
    return gqa::decode_workspace_bytes(B, Hq, d, max_seq_len);
}

int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o, const int32_t* seq_lens,
                    const int32_t* block_table, int B, int Hq, int Hkv, int d, int max_seq_len, int block_size,
                    int max_blocks_per_seq, float scale, int dtype, void* workspace, size_t workspace_bytes,
                    void* stream) {
    const int st = decode_check(q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                                block_size, max_blocks_per_seq, scale, dtype, workspace, workspace_bytes);
    if (st != GQA_OK) return st;
    gqa::DecodeArgs a{q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                      block_table ? max_blocks_per_seq : 0, scale, workspace};
    const hipError_t e = gqa::launch_decode_bf16(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* seq_lens, const int32_t* block_table, int B, int Hq, int Hkv, int d,
                            int max_seq_len, int block_size, int max_blocks_per_seq, float scale, int dtype,
                            void* stream) {
    const int st = decode_check_args(q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                                     block_size, max_blocks_per_seq, scale, dtype);
    if (st != GQA_OK) return st;
    if (gqa::decode_workspace_bytes(B, Hq, d, max_seq_len) > GQA_DECODE_NOALLOC_MAX_BYTES)
        return GQA_ERR_WORKSPACE;
    gqa::DecodeArgs a{q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                      block_table ? max_blocks_per_seq : 0, scale, nullptr};
    const hipError_t e = gqa::launch_decode_bf16_static(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_decode_window_fwd(const void* q, const void* k_cache, const void* v_cache, void* o, const int32_t* seq_lens,
                           const int32_t* block_table, int B, int Hq, int Hkv, int d, int max_seq_len,
                           int block_size, int max_blocks_per_seq, float scale, int window, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream) {
    const int st = decode_check(q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                                block_size, max_blocks_per_seq, scale, dtype, workspace, workspace_bytes);
    if (st != GQA_OK) return st;
    if (window <= 0) return GQA_ERR_INVALID_ARG;
    gqa::DecodeArgs a{q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                      block_table ? max_blocks_per_seq : 0, scale, workspace};
    a.window = window;
    const hipError_t e = gqa::launch_decode_bf16(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_decode_fp8_fwd(const void* q, const void* k_cache, const void* v_cache, const float* k_scale,
                        const float* v_scale, void* o, const int32_t* seq_lens, const int32_t* block_table, int B,
                        int Hq, int Hkv, int d, int max_seq_len, int block_size, int max_blocks_per_seq, float scale,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!k_scale || !v_scale) return GQA_ERR_INVALID_ARG;
    const int st = decode_check(q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                                block_size, max_blocks_per_seq, scale, GQA_BF16, workspace, workspace_bytes);
    if (st != GQA_OK) return st;
    if (d != 128) return GQA_ERR_UNSUPPORTED;
    // a contiguous cache's scale rows are read 16 at a time from block starts
    if (!block_table && max_seq_len % GQA_PAGE_BLOCK_SIZE != 0) return GQA_ERR_UNSUPPORTED;
    gqa::DecodeArgs a{q, k_cache, v_cache, o, seq_lens, block_table, B, Hq, Hkv, d, max_seq_len,
                      block_table ? max_blocks_per_seq : 0, scale, workspace, k_scale, v_scale};
    const hipError_t e = gqa::launch_decode_fp8(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_decode_validate(const int32_t* seq_lens, const int32_t* block_table, int B, int max_seq_len,
                         int block_size, int max_blocks_per_seq, int num_physical_blocks, void* stream) {
    if (!seq_lens || B <= 0 || max_seq_len < 0) return GQA_ERR_INVALID_ARG;
    if (block_table && (block_size <= 0 || max_blocks_per_seq <= 0 || num_physical_blocks <= 0))
        return GQA_ERR_INVALID_ARG;
    std::vector<int32_t> lens, table;
    try {
        lens.resize((size_t)B);
        if (block_table) table.resize((size_t)B * max_blocks_per_seq);
    } catch (const std::bad_alloc&) {
        return GQA_ERR_INVALID_ARG;
    }
    const hipStream_t s = static_cast<hipStream_t>(stream);
    if (hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, s) != hipSuccess)
        return GQA_ERR_HIP;
    if (block_table && hipMemcpyAsync(table.data(), block_table, table.size() * 4, hipMemcpyDeviceToHost, s) !=
                           hipSuccess)
        return GQA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return GQA_ERR_HIP;
    for (int b = 0; b < B; ++b) {
        const int L = lens[(size_t)b];
        if (L < 0 || L > max_seq_len) return GQA_ERR_INVALID_ARG;
        if (!block_table) continue;
        const int64_t nblk = ((int64_t)L + block_size - 1) / block_size;
        if (nblk > max_blocks_per_seq) return GQA_ERR_INVALID_ARG;
        for (int64_t j = 0; j < nblk; ++j) {
            const int32_t p = table[(size_t)b * max_blocks_per_seq + j];
            if (p < 0 || p >= num_physical_blocks) return GQA_ERR_INVALID_ARG;
        }
    }
    return GQA_OK;
}

}  // extern "C"
