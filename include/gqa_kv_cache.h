/*
 * gqa_kv_cache.h - paged KV-cache management of libgqa_attn: a host-side
 * block allocator with per-sequence page tables and copy-on-write prefix
 * sharing, and the device calls that write new tokens into the pages and
 * copy blocks.  The pages this follows: [Different attention mechanisms
 * (blog.gocoding.cloud), §5 Page Attention]:
 *   step 1  the KV cache is cut into fixed-size blocks that may sit anywhere
 *           in device memory;
 *   step 2  each sequence keeps a page table from its logical blocks to
 *           physical ones;
 *   step 3  blocks are taken on demand as tokens arrive; only the page table
 *           changes, nothing already cached moves;
 *   advantages: sequences with a common prefix point their tables at the same
 *           physical blocks, shared copy-on-write.
 *
 * Layout (the paged layout of attn_decode_fwd): k_cache, v_cache are
 * [num_blocks, Hkv, 16, d]; physical slot s = block * 16 + offset holds one
 * token of every K/V head: row k_cache[s / 16][h][s % 16][:].
 *
 * Allocation rules (the pages fix none of them; these are the plain choices):
 *  - a sequence takes a new block only when its last block is full (or it
 *    has none), so a sequence of length L holds ceil(L / 16) blocks;
 *  - the lowest-numbered free block is taken first (any free block would
 *    do; the fixed rule makes every result reproducible);
 *  - fork: the child's page table is a copy of the parent's and every block
 *    in it gains a reference;
 *  - copy-on-write: before a token is written into a block that another
 *    sequence also references (only a partly filled last block inherited
 *    through a fork can be), the writer takes a new block, the old block's
 *    contents are copied into it and the writer's table entry is repointed;
 *    full shared blocks are never written and stay shared;
 *  - release: every block of the sequence loses a reference; a block with
 *    none left is free again.
 *
 * The pool is host memory owned by the library behind an opaque handle; it
 * never touches the device.  Calls on one pool are not thread-safe; distinct
 * pools are independent.  Errors are returned as gqa_status codes (see
 * gqa_attn.h); a failed call leaves the pool unchanged.
 */
#ifndef GQA_KV_CACHE_H
#define GQA_KV_CACHE_H

#include <stddef.h>
#include <stdint.h>

#include "gqa_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct gqa_kv_pool gqa_kv_pool;

/*
 * Create a pool of num_blocks physical blocks (ids 0 .. num_blocks-1) for up
 * to max_seqs live sequences of at most max_blocks_per_seq blocks each.
 * *pool_out receives the handle.  GQA_ERR_INVALID_ARG for a NULL pool_out,
 * any count <= 0 or num_blocks * 16 >= 2^31 (slots are int32).
 */
int gqa_kv_pool_create(int num_blocks, int max_seqs, int max_blocks_per_seq, gqa_kv_pool** pool_out);

/* Free the pool (NULL is ignored). */
void gqa_kv_pool_destroy(gqa_kv_pool* pool);

/* Number of free physical blocks; -1 for a NULL pool. */
int gqa_kv_pool_free_blocks(const gqa_kv_pool* pool);

/*
 * Start an empty sequence; *seq_out receives its id, the lowest id not in
 * use (ids lie in [0, max_seqs)).  GQA_ERR_OUT_OF_BLOCKS when max_seqs
 * sequences are live.
 */
int gqa_kv_seq_new(gqa_kv_pool* pool, int* seq_out);

/*
 * Start a sequence that shares every cached token of `parent` (same page
 * table, one more reference per block; no block is taken or copied).
 * GQA_ERR_INVALID_ARG for an unknown parent, GQA_ERR_OUT_OF_BLOCKS when
 * max_seqs sequences are live.
 */
int gqa_kv_seq_fork(gqa_kv_pool* pool, int parent, int* child_out);

/* End a sequence and drop its block references.  GQA_ERR_INVALID_ARG for an unknown id. */
int gqa_kv_seq_release(gqa_kv_pool* pool, int seq);

/* Cached tokens of a live sequence; -1 for an unknown id or NULL pool. */
int gqa_kv_seq_len(const gqa_kv_pool* pool, int seq);

/*
 * Reserve cache slots for new tokens: counts[i] tokens for sequence seqs[i],
 * i < n, processed in order (a sequence may appear more than once).
 *   slots_out : int32 [sum(counts)], host; the physical slot of every new
 *               token, entries of seqs[0] first, each sequence's in order.
 *   copy_src, copy_dst : int32 [n], host; the copy-on-write block copies
 *               (physical block ids) this reservation needs, *n_copies of
 *               them.  Perform them (attn_kv_copy_blocks) BEFORE writing the
 *               new tokens (attn_kv_append).
 * The sequences' lengths grow by their counts.  All or nothing:
 * GQA_ERR_INVALID_ARG (an unknown id, a negative count, n < 0, a NULL array,
 * or a sequence growing past max_blocks_per_seq blocks; checked first) and
 * GQA_ERR_OUT_OF_BLOCKS (too few free blocks) leave the pool unchanged.
 */
int gqa_kv_reserve(gqa_kv_pool* pool, const int* seqs, const int* counts, int n, int32_t* slots_out,
                   int32_t* copy_src, int32_t* copy_dst, int* n_copies);

/*
 * Page tables and lengths of n live sequences, for attn_decode_fwd:
 *   table_out : int32 [n, max_blocks], host; row i holds the physical blocks
 *               of seqs[i] in logical order, padded with -1;
 *   lens_out  : int32 [n], host.
 * GQA_ERR_INVALID_ARG for an unknown id, a NULL array, n <= 0, or a
 * sequence holding more than max_blocks blocks.
 */
int gqa_kv_block_table(const gqa_kv_pool* pool, const int* seqs, int n, int32_t* table_out, int max_blocks,
                       int32_t* lens_out);

/*
 * Device: write n_tokens new tokens into the pages.
 *   k_new, v_new : [n_tokens, Hkv, d] (dtype elements), device;
 *   slots        : int32 [n_tokens], device (from gqa_kv_reserve);
 *   k_cache[s / 16][h][s % 16][:] = k_new[t][h][:] for s = slots[t], every
 *   head h, and the same for V.  Slots outside [0, num_blocks * 16) are
 *   skipped (a negative slot marks a padding token).  Distinct tokens must
 *   have distinct slots.
 * d * element size must be a multiple of 16 bytes (d in {64, 128} for
 * GQA_BF16 and GQA_F32).  GQA_ERR_INVALID_ARG for a NULL pointer, a size
 * <= 0 (n_tokens == 0 is a no-op), a dtype outside gqa_dtype;
 * GQA_ERR_UNSUPPORTED for another d.  Enqueued on `stream`, asynchronous.
 */
int attn_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* slots,
                   int n_tokens, int num_blocks, int Hkv, int d, int dtype, void* stream);

/*
 * Device: copy whole blocks, k_cache[dst[i]] = k_cache[src[i]] and the same
 * for V (all Hkv heads, all 16 slots), for i < n.  src, dst: int32 [n],
 * device.  Pairs whose ids fall outside [0, num_blocks) are skipped.  No dst
 * may also be a src or repeat (gqa_kv_reserve's copies satisfy this).
 * Errors as attn_kv_append; n == 0 is a no-op.
 */
int attn_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n,
                        int num_blocks, int Hkv, int d, int dtype, void* stream);

/*
 * fp8 caches (read by attn_decode_fp8_fwd) [Attention variants deep-dive,
 * §7 KV Cache: fp16 -> fp8 halves the cache].  Codes are OCP E4M3 (uint8)
 * in pages [num_blocks, Hkv, 16, d] with one fp32 scale per row in
 * [num_blocks, Hkv, 16] (k_scale, v_scale).  A row x of d values is stored
 * as scale = amax / 448 (amax = max |x|) and codes E4M3(x * (448 / amax)),
 * each fp32 operation rounded to nearest even, each code the nearest E4M3
 * value with ties to the even code; an all-zero row stores scale 0.
 *
 * attn_kv_append_fp8: as attn_kv_append, quantising bf16 k_new, v_new
 * [n_tokens, Hkv, d]; attn_kv_copy_blocks_fp8: as attn_kv_copy_blocks, also
 * copying the blocks' scales.  d must be 128 (GQA_ERR_UNSUPPORTED
 * otherwise); NULL scale arrays are GQA_ERR_INVALID_ARG.
 */
int attn_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const void* k_new,
                       const void* v_new, const int32_t* slots, int n_tokens, int num_blocks, int Hkv, int d,
                       void* stream);

int attn_kv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* src,
                            const int32_t* dst, int n, int num_blocks, int Hkv, int d, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GQA_KV_CACHE_H */
