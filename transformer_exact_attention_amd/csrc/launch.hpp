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
};

// Tokens of one decode split (one workgroup's share of a sequence) are chosen
// per call between kDecodeSplitMin and kDecodeSplitMax (powers of two).
constexpr int kDecodeSplitMin = 256;
constexpr int kDecodeSplitMax = 4096;

// Workspace layout for split size T: fp32 partial outputs [B, Hq, ns, d] then
// fp32 log-sum-exp values [B, Hq, ns], ns = ceil(max_seq_len / T), each
// 256-byte aligned.  The size query uses T = kDecodeSplitMin: an upper bound.
inline int decode_nsplit(int max_seq_len, int T) { return (max_seq_len + T - 1) / T; }
inline int decode_nsplit_max(int max_seq_len) { return decode_nsplit(max_seq_len, kDecodeSplitMin); }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline size_t decode_workspace_bytes(int B, int Hq, int d, int max_seq_len) {
    const size_t ns = (size_t)decode_nsplit_max(max_seq_len);
    return align256((size_t)B * Hq * ns * d * 4) + align256((size_t)B * Hq * ns * 4);
}

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream);

}  // namespace gqa
