// Internal launch interface between the C ABI (gqa_attn.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gqa {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int B, Hq, Hkv, Sq, Sk, d;
    float scale;
    int causal;
    int window = 0;                 // > 0: sliding window of that many keys (implies causal)
    float* lse = nullptr;           // optional: natural-log log-sum-exp per (b, head, row), fp32
};

// Backward of prefill attention (bf16 tensors, fp32 lse and row sums).
struct BackwardArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;               // natural-log log-sum-exp of the forward, [B, Hq, Sq]
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dsum;                    // workspace: rowsum(dO * O), [B, Hq, Sq] fp32
    int B, Hq, Hkv, Sq, Sk, d;
    float scale;
    int causal;
    int window;                     // > 0: sliding window (implies causal)
};

struct DecodeArgs {
    const void* q;
    const void* k_cache;
    const void* v_cache;
    void* o;
    const int32_t* seq_lens;
    const int32_t* block_table;   // nullptr: contiguous cache
    int B, Hq, Hkv, d;
    int max_seq_len;
    int max_blocks_per_seq;
    float scale;
    void* workspace;
    const float* k_scale = nullptr;   // fp8 caches: per-row scales, same row numbering as the cache
    const float* v_scale = nullptr;
    int window = 0;                   // > 0: attend only each sequence's last `window` tokens
};

// Decode work partition.  The flattened space of (sequence, K/V head, token)
// triples, W = sum_b seq_lens[b] * Hkv tokens, is cut into equal consecutive
// shares of Q tokens, one per wavefront (Q >= kDecodeMinShare, a multiple of
// 16).  A share covering part of a (sequence, K/V head) segment produces one
// partial result for that segment (merged per workgroup of four shares where
// the workgroup has room for it), so a segment of length L has at most
// ceil(L / kDecodeMinShare) + 1 partials.
constexpr int kDecodeMinShare = 256;
constexpr int kDecodeMaxBatch = 4096;     // sequence prefix sums live in LDS

inline int decode_max_partials(int max_seq_len) {
    return (max_seq_len + kDecodeMinShare - 1) / kDecodeMinShare + 1;
}
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace layout (each part 256-byte aligned):
//   fp32 partial outputs [B, Hq, P, d], P = decode_max_partials(max_seq_len)
//   fp32 base-2 log-sum-exp [B, Hq, P]
//   int64 token prefix sums over sequences [B + 1]
struct DecodeWorkspace {
    size_t part_o, part_lse, prefix, total;
};
inline DecodeWorkspace decode_workspace_layout(int B, int Hq, int d, int max_seq_len) {
    const size_t P = (size_t)decode_max_partials(max_seq_len);
    DecodeWorkspace w;
    w.part_o = 0;
    w.part_lse = align256((size_t)B * Hq * P * d * 4);
    w.prefix = w.part_lse + align256((size_t)B * Hq * P * 4);
    w.total = w.prefix + align256((size_t)(B + 1) * 8);
    return w;
}
inline size_t decode_workspace_bytes(int B, int Hq, int d, int max_seq_len) {
    return decode_workspace_layout(B, Hq, d, max_seq_len).total;
}

// Size of the static device array behind the allocation-free decode entry
// point (one copy per GPU, held until the process ends).
constexpr size_t kDecodeStaticScratchBytes = (size_t)64 << 20;

// Paged KV cache: new tokens [n_tokens, Hkv, d] to their slots, and whole
// block copies; rows are row_bytes = d * element size bytes (16 | row_bytes).
// fp8 caches add per-row fp32 scales [num_blocks, Hkv, 16] (k_scale,
// v_scale; null for bf16/fp32 caches).
struct KvAppendArgs {
    void* k_cache;
    void* v_cache;
    const void* k_new;
    const void* v_new;
    const int32_t* slots;
    int n_tokens, num_blocks, Hkv, row_bytes;
    float* k_scale = nullptr;
    float* v_scale = nullptr;
};
struct KvCopyArgs {
    void* k_cache;
    void* v_cache;
    const int32_t* src;
    const int32_t* dst;
    int n, num_blocks, Hkv, row_bytes;
    float* k_scale = nullptr;
    float* v_scale = nullptr;
};

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream);
// attn_decode_fwd with the workspace in the library's static device scratch
// (a.workspace is ignored); the caller has checked that the sizes fit.
hipError_t launch_decode_bf16_static(const DecodeArgs& a, hipStream_t stream);
hipError_t launch_kv_append(const KvAppendArgs& a, hipStream_t stream);
hipError_t launch_kv_copy_blocks(const KvCopyArgs& a, hipStream_t stream);
hipError_t launch_kv_append_fp8(const KvAppendArgs& a, hipStream_t stream);
hipError_t launch_prefill_bwd_bf16(const BackwardArgs& a, hipStream_t stream);
hipError_t launch_prefill_bwd_f32(const BackwardArgs& a, hipStream_t stream);

}  // namespace gqa
