/*
 * gqa_attn.h - C ABI of libgqa_attn: exact scaled-dot-product attention with
 * grouped K/V heads (MHA when Hkv == Hq, GQA when 1 < Hkv < Hq, MQA when
 * Hkv == 1) on AMD Instinct MI355X (gfx950).
 *
 * What is computed.  For batch b and query head h, with g = Hq / Hkv and K/V
 * head hk = floor(h / g):
 *     O[b,h] = softmax(Q[b,h] K[b,hk]^T * scale) V[b,hk]
 * [Different attention mechanisms (blog.gocoding.cloud), §1 MHA, step 3, for
 * one head; §3 GQA, every N/G query heads share one K/V pair].  The grouping
 * is contiguous: repeating every K/V head g times along the head axis
 * [Attention variants deep-dive (devpress.csdn.net), §5 GQA code] gives
 * query head h the K/V head floor(h / g); K/V are never copied per query head
 * [same page, the note after the §5 code].  The result is exact attention
 * computed tile by tile with an online softmax, so no Sq x Sk score matrix is
 * ever written to device memory [Attention variants deep-dive, §6.2].
 *
 * Conventions shared by every entry point:
 *  - All tensor pointers are DEVICE pointers owned by the caller; tensors are
 *    dense, row-major, with the layouts stated per call.  The library never
 *    allocates or frees device memory (the only memory it allocates is a KV
 *    pool's host-side bookkeeping, behind the pool's handle: gqa_kv_cache.h);
 *    its only global state is the static device scratch of
 *    attn_decode_fwd_noalloc (one array per GPU, loaded with the library's
 *    code) and that array's per-device address.  Calls are reentrant, except
 *    that attn_decode_fwd_noalloc calls overlapping on one GPU race.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *    on it and the call returns before the kernels finish (except
 *    attn_decode_validate, which synchronises).
 *  - Every argument is checked on the host BEFORE any HIP call; a failed
 *    check returns a status and enqueues nothing.  No C++ exception crosses
 *    this boundary.
 *  - dtype: GQA_F32 or GQA_BF16; q/k/v/o share it.  Accumulation, softmax
 *    state and decode partials are always fp32.
 */
#ifndef GQA_ATTN_H
#define GQA_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    GQA_OK = 0,
    GQA_ERR_INVALID_ARG = 1,   /* null pointer, bad size, Hq % Hkv != 0, bad scale, ... */
    GQA_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head dim, dtype, group size) */
    GQA_ERR_WORKSPACE = 3,     /* decode workspace missing or too small */
    GQA_ERR_HIP = 4,           /* a HIP launch or runtime call failed */
    GQA_ERR_OUT_OF_BLOCKS = 5  /* KV pool: not enough free blocks (see gqa_kv_cache.h) */
} gqa_status;

typedef enum { GQA_F32 = 0, GQA_BF16 = 1 } gqa_dtype;

#define GQA_ATTN_ABI_VERSION 3
#define GQA_PAGE_BLOCK_SIZE 16   /* tokens per KV page */

/* Version of this ABI (GQA_ATTN_ABI_VERSION of the built library). */
int gqa_attn_abi_version(void);

/* Static, human-readable text for a status code (never NULL). */
const char* gqa_attn_status_string(int status);

/*
 * Prefill / full attention forward.
 *
 *   q, o : [B, Hq,  Sq, d]      k, v : [B, Hkv, Sk, d]      (dtype elements)
 *
 * scale multiplies the scores q.k; pass 1/sqrt(d) for the pages' default
 * [Attention variants deep-dive, §5 GQA code].  With causal != 0, key j is
 * visible to query row i iff j <= i + (Sk - Sq) (the Sq queries are the last
 * Sq positions; j <= i when Sq == Sk).
 *
 * Supported: d in {64, 128}; GQA_F32 (any group size g) and GQA_BF16 (g in
 * {1, 2, 4, 8, 16, 32, 64, 128}).  Otherwise GQA_ERR_UNSUPPORTED.
 * GQA_ERR_INVALID_ARG for: a NULL pointer, any size <= 0, Hq % Hkv != 0,
 * causal with Sq > Sk, a non-finite or non-positive scale, a dtype outside
 * gqa_dtype, or sizes whose element counts overflow 2^31 per (b, head) plane.
 * o must not overlap q, k or v.
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d,
                     float scale, int causal, int dtype, void* stream);

/*
 * Sliding-window attention forward: attn_prefill_fwd with causal != 0 where
 * each query additionally sees only its last `window` keys -- key j is
 * visible to query row i iff i + (Sk - Sq) - window < j <= i + (Sk - Sq).
 * The pages name sliding-window attention for long sequences [Attention
 * variants deep-dive, §8 Q4] and fix nothing else; this is the plain
 * reading.  Tiles wholly before a query block's window are neither read nor
 * computed.  window >= 1 (window >= Sk is plain causal attention); otherwise
 * as attn_prefill_fwd, with GQA_ERR_INVALID_ARG for window <= 0.
 */
int attn_prefill_window_fwd(const void* q, const void* k, const void* v, void* o,
                            int B, int Hq, int Hkv, int Sq, int Sk, int d,
                            float scale, int window, int dtype, void* stream);

/*
 * Forward that also writes each query row's natural-log log-sum-exp,
 *   lse[b, h, i] = log sum_j exp(scale * q_i . k_j)   over visible keys j,
 * the one number per row the backward needs to recompute the probabilities
 * without storing them [Attention variants deep-dive, §6.2 technique 2
 * (recomputation)].  lse: fp32 [B, Hq, Sq], device, written in full (every
 * row sees at least one key under the rules below).  window == 0: exactly
 * attn_prefill_fwd (same kernels, same o bit for bit); window >= 1: exactly
 * attn_prefill_window_fwd (causal implied).  Errors as those calls, plus
 * GQA_ERR_INVALID_ARG for a NULL lse or window < 0.
 */
int attn_prefill_lse_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int Hq, int Hkv, int Sq, int Sk, int d,
                         float scale, int causal, int window, int dtype, void* stream);

/*
 * Bytes of device workspace attn_prefill_bwd needs (fp32 row sums
 * [B, Hq, Sq], rounded up to 256).  0 on invalid sizes.
 */
size_t attn_prefill_bwd_workspace_bytes(int B, int Hq, int Sq);

/*
 * Backward of attn_prefill_lse_fwd by recomputation: no attention matrix is
 * kept from the forward; the probabilities are recomputed tile by tile from
 * q, k and the saved lse, so memory stays linear in the sequence length
 * [Attention variants deep-dive, §6.2 technique 2; §8 follow-ups 2-3].
 * With P the forward's probabilities and dO = dout:
 *   dv = P^T dO,  dP = dO v^T,  dS = P * (dP - rowsum(dO * o)),
 *   dq = scale dS k,  dk = scale dS^T q,
 * and a K/V head's dk, dv sum over the g query heads that read it.
 *
 *   q, o, dout, dq : [B, Hq, Sq, d]     k, v, dk, dv : [B, Hkv, Sk, d]   (dtype)
 *   lse            : fp32 [B, Hq, Sq] from attn_prefill_lse_fwd with the same
 *                    q, k, v, scale, causal and window
 *   workspace      : device, >= attn_prefill_bwd_workspace_bytes(B, Hq, Sq)
 *                    bytes, 256-byte aligned; contents on entry are ignored.
 * dq, dk, dv are overwritten (not accumulated into) and must not overlap any
 * input.  Supported: d in {64, 128}, B * Hq * Sq < 2^27,
 * ceil(Sk / 128) * Hkv * B < 2^31, group sizes as attn_prefill_fwd; GQA_BF16
 * (matrix cores) and GQA_F32 (all tensors fp32; vector-ALU kernels, one
 * wavefront per row, meant for small problems).  GQA_ERR_INVALID_ARG as
 * attn_prefill_lse_fwd and for NULL dout/dq/dk/dv; GQA_ERR_WORKSPACE for a
 * short, NULL or misaligned workspace.
 */
int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int Hq, int Hkv, int Sq, int Sk, int d,
                     float scale, int causal, int window, int dtype,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Bytes of device workspace attn_decode_fwd needs for these sizes (an upper
 * bound valid for every Hkv dividing Hq).  0 on invalid sizes.
 */
size_t attn_decode_workspace_bytes(int B, int Hq, int d, int max_seq_len);

/*
 * Decode: one new query token per sequence attends to its cached keys.
 *
 * Query b attends every cached key t in [0, seq_lens[b]) with no mask: its
 * own K/V has already been appended at position seq_lens[b] - 1
 * [Attention variants deep-dive, §7 KV Cache].  A sequence with length 0
 * gets a zero output.
 *
 *   q, o      : [B, Hq, d]                                   (dtype elements)
 *   seq_lens  : int32 [B], device, each in [0, max_seq_len]
 *   block_table == NULL (contiguous cache):
 *       k_cache, v_cache : [B, Hkv, max_seq_len, d]
 *   block_table != NULL (paged cache, [Different attention mechanisms, §5
 *   Page Attention: fixed-size blocks, per-sequence page table]):
 *       k_cache, v_cache : [num_blocks, Hkv, block_size, d]
 *       block_table      : int32 [B, max_blocks_per_seq], device; token t of
 *                          sequence b lives in physical block
 *                          block_table[b][t / block_size], slot t % block_size.
 *                          Entries at or past ceil(seq_lens[b] / block_size)
 *                          are never read.
 *   workspace : device, >= attn_decode_workspace_bytes(B, Hq, d, max_seq_len)
 *               bytes, 256-byte aligned; contents on entry are ignored.
 *
 * Supported: GQA_BF16, d in {64, 128}, block_size == GQA_PAGE_BLOCK_SIZE,
 * g = Hq / Hkv in {1, 2, 4, 8, 16, 32}, B <= 4096.  fp32 decode returns
 * GQA_ERR_UNSUPPORTED (the decode workloads are bf16 caches; fp32 inputs
 * are served by attn_prefill_fwd with Sq = 1).
 * GQA_ERR_INVALID_ARG for: a NULL pointer (block_table may be NULL), any size
 * <= 0, Hq % Hkv != 0, a bad scale, paged with block_size != 16 or
 * max_blocks_per_seq * block_size < max_seq_len.  GQA_ERR_WORKSPACE for a
 * short or NULL workspace.  Device data (lengths, table entries in
 * [0, num_blocks)) is the caller's contract: attn_decode_validate checks it.
 */
int attn_decode_fwd(const void* q, const void* k_cache, const void* v_cache, void* o,
                    const int32_t* seq_lens, const int32_t* block_table,
                    int B, int Hq, int Hkv, int d, int max_seq_len,
                    int block_size, int max_blocks_per_seq,
                    float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): attn_decode_fwd with the same arguments, checks and results
 * (the same kernels, bit for bit), minus the workspace.  Its partial results
 * live in a static device array of GQA_DECODE_NOALLOC_MAX_BYTES bytes, one
 * per GPU the library runs on, held until the process ends; its address is
 * taken once per device at the first call on that device.  The call
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 * Sizes with attn_decode_workspace_bytes(B, Hq, d, max_seq_len) >
 * GQA_DECODE_NOALLOC_MAX_BYTES return GQA_ERR_WORKSPACE and enqueue
 * nothing.  Every call on one GPU shares that GPU's array: calls that overlap
 * on one GPU (different streams, threads or processes sharing the library
 * instance) race on it and must be ordered by the caller.  The array needs no
 * initial contents (every partial a call reads is written by that call).
 */
#define GQA_DECODE_NOALLOC_MAX_BYTES ((size_t)64 << 20)

int attn_decode_fwd_noalloc(const void* q, const void* k_cache, const void* v_cache, void* o,
                            const int32_t* seq_lens, const int32_t* block_table,
                            int B, int Hq, int Hkv, int d, int max_seq_len,
                            int block_size, int max_blocks_per_seq,
                            float scale, int dtype, void* stream);

/*
 * Sliding-window decode: attn_decode_fwd where query b attends only its
 * sequence's last `window` cached keys, [max(0, L_b - window), L_b) (the
 * reading of [Attention variants deep-dive, §8 Q4], as for
 * attn_prefill_window_fwd).  Keys before the window are never read; the
 * work split covers min(L_b, window) tokens per sequence.  window >= 1;
 * otherwise as attn_decode_fwd, with GQA_ERR_INVALID_ARG for window <= 0.
 */
int attn_decode_window_fwd(const void* q, const void* k_cache, const void* v_cache, void* o,
                           const int32_t* seq_lens, const int32_t* block_table,
                           int B, int Hq, int Hkv, int d, int max_seq_len,
                           int block_size, int max_blocks_per_seq,
                           float scale, int window, int dtype,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode over an fp8 KV cache [Attention variants deep-dive, §7 KV Cache:
 * fp16 -> fp8 halves the cache; §8 Q4: quantise the KV cache to fp8].  The
 * same computation as attn_decode_fwd with every cached row standing for
 * E4M3(code) * row scale:
 *   k_cache, v_cache : uint8 OCP E4M3 codes (sign, 4 exponent bits with bias
 *                      7, 3 mantissa bits, largest finite 448), laid out as
 *                      attn_decode_fwd's bf16 caches: [B, Hkv, max_seq_len, d]
 *                      or pages [num_blocks, Hkv, 16, d];
 *   k_scale, v_scale : fp32, one per row: [B, Hkv, max_seq_len] or
 *                      [num_blocks, Hkv, 16], device;
 *   q, o             : bf16 [B, Hq, d].
 * attn_kv_append_fp8 (gqa_kv_cache.h) writes such rows.  Supported and
 * errors as attn_decode_fwd (bf16 q/o), but d == 128 only; additionally
 * GQA_ERR_INVALID_ARG for NULL scales and GQA_ERR_UNSUPPORTED for a
 * contiguous cache whose max_seq_len is not a multiple of 16 (scales are
 * read 16 rows at a time).  Scales of rows past a sequence's length are read
 * but never used, so they may hold anything.
 */
int attn_decode_fp8_fwd(const void* q, const void* k_cache, const void* v_cache,
                        const float* k_scale, const float* v_scale, void* o,
                        const int32_t* seq_lens, const int32_t* block_table,
                        int B, int Hq, int Hkv, int d, int max_seq_len,
                        int block_size, int max_blocks_per_seq, float scale,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Debug/test helper (synchronous): copies seq_lens (and block_table, if not
 * NULL) to the host and checks 0 <= seq_lens[b] <= max_seq_len and that every
 * table entry a sequence reads lies in [0, num_physical_blocks).
 * Returns GQA_OK, GQA_ERR_INVALID_ARG on bad data, GQA_ERR_HIP on a failed copy.
 */
int attn_decode_validate(const int32_t* seq_lens, const int32_t* block_table,
                         int B, int max_seq_len, int block_size, int max_blocks_per_seq,
                         int num_physical_blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_ATTN_H */
