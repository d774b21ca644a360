// Paged KV-cache management behind the C ABI: the host-side block allocator
// (page tables, reference counts, copy-on-write prefix sharing) and the
// argument checks of the device calls that write tokens and copy blocks.
//
// The method [Different attention mechanisms, §5 Page Attention]: the cache
// is cut into fixed-size blocks stored anywhere (step 1), each sequence maps
// its logical blocks to physical ones through a page table (step 2), blocks
// are taken on demand as tokens arrive while nothing cached moves (step 3),
// and sequences with a common prefix point at the same physical blocks,
// shared copy-on-write (advantages).  The rules the pages leave open (one
// 16-token block holds every K/V head of a token; a block is taken only when
// the last one is full; lowest free block first; copy before writing into a
// block someone else references) are stated in gqa_kv_cache.h.
#include "../../include/gqa_kv_cache.h"

#include <hip/hip_runtime.h>

#include <cstdint>
#include <new>
#include <set>
#include <unordered_map>
#include <vector>

#include "launch.hpp"

namespace {

constexpr int kBlock = GQA_PAGE_BLOCK_SIZE;

struct Seq {
    bool live = false;
    int32_t len = 0;
    std::vector<int32_t> blocks;   // physical block of logical block j
};

}  // namespace

struct gqa_kv_pool {
    int num_blocks = 0, max_seqs = 0, max_blocks = 0;
    std::vector<int32_t> refs;         // page-table entries pointing at each block
    std::set<int32_t> free_blocks;     // refs == 0, lowest first
    std::vector<Seq> seqs;
    std::set<int> free_ids;

    bool known(int s) const { return s >= 0 && s < max_seqs && seqs[(size_t)s].live; }
    int32_t take_block() {
        const auto it = free_blocks.begin();
        const int32_t b = *it;
        free_blocks.erase(it);
        refs[(size_t)b] = 1;
        return b;
    }
    void drop(int32_t b) {
        if (--refs[(size_t)b] == 0) free_blocks.insert(b);
    }
};

namespace {

// Blocks a reservation takes, found without changing the pool: per sequence
// its running length, block count and whether its last block is one this
// reservation already made private; per shared block the references given up
// by earlier copies in the same reservation.  Returns GQA_OK and the count,
// or the error the reservation must fail with.
int plan_reserve(gqa_kv_pool& p, const int* seqs, const int* counts, int n, int64_t& need, int64_t& tokens) {
    struct View {
        int64_t len, nblk;
        int32_t last;
        bool private_last;
    };
    std::unordered_map<int, View> view;
    std::unordered_map<int32_t, int32_t> released;
    need = 0;
    tokens = 0;
    for (int i = 0; i < n; ++i) {
        const int s = seqs[i];
        const int c = counts[i];
        if (!p.known(s) || c < 0) return GQA_ERR_INVALID_ARG;
        if (c == 0) continue;
        const Seq& q = p.seqs[(size_t)s];
        auto ins = view.try_emplace(s, View{q.len, (int64_t)q.blocks.size(), q.blocks.empty() ? -1 : q.blocks.back(),
                                            false});
        View& v = ins.first->second;
        bool copy = false;
        if (v.len % kBlock != 0 && !v.private_last) {
            int32_t& gone = released[v.last];
            if (p.refs[(size_t)v.last] - gone > 1) {
                copy = true;
                ++gone;
            }
        }
        const int64_t nblk = (v.len + c + kBlock - 1) / kBlock;
        if (nblk > p.max_blocks) return GQA_ERR_INVALID_ARG;
        need += (nblk - v.nblk) + (copy ? 1 : 0);
        if (copy || nblk > v.nblk) v.private_last = true;
        v.len += c;
        v.nblk = nblk;
        tokens += c;
    }
    return GQA_OK;
}

int checked_rows(int n, int Hkv, int d, int dtype, int& row_bytes) {
    if (n < 0 || Hkv <= 0 || d <= 0) return GQA_ERR_INVALID_ARG;
    if (dtype != GQA_F32 && dtype != GQA_BF16) return GQA_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return GQA_ERR_UNSUPPORTED;
    row_bytes = d * (dtype == GQA_F32 ? 4 : 2);
    return GQA_OK;
}

}  // namespace

extern "C" {

int gqa_kv_pool_create(int num_blocks, int max_seqs, int max_blocks_per_seq, gqa_kv_pool** pool_out) {
    if (!pool_out) return GQA_ERR_INVALID_ARG;
    *pool_out = nullptr;
    if (num_blocks <= 0 || max_seqs <= 0 || max_blocks_per_seq <= 0) return GQA_ERR_INVALID_ARG;
    if ((int64_t)num_blocks * kBlock >= ((int64_t)1 << 31)) return GQA_ERR_INVALID_ARG;
    try {
        gqa_kv_pool* p = new gqa_kv_pool;
        p->num_blocks = num_blocks;
        p->max_seqs = max_seqs;
        p->max_blocks = max_blocks_per_seq;
        p->refs.assign((size_t)num_blocks, 0);
        for (int32_t b = 0; b < num_blocks; ++b) p->free_blocks.insert(p->free_blocks.end(), b);
        p->seqs.resize((size_t)max_seqs);
        for (int s = 0; s < max_seqs; ++s) p->free_ids.insert(p->free_ids.end(), s);
        *pool_out = p;
        return GQA_OK;
    } catch (const std::bad_alloc&) {
        return GQA_ERR_INVALID_ARG;
    }
}

void gqa_kv_pool_destroy(gqa_kv_pool* pool) { delete pool; }

int gqa_kv_pool_free_blocks(const gqa_kv_pool* pool) { return pool ? (int)pool->free_blocks.size() : -1; }

int gqa_kv_seq_new(gqa_kv_pool* pool, int* seq_out) {
    if (!pool || !seq_out) return GQA_ERR_INVALID_ARG;
    if (pool->free_ids.empty()) return GQA_ERR_OUT_OF_BLOCKS;
    const int s = *pool->free_ids.begin();
    pool->free_ids.erase(pool->free_ids.begin());
    Seq& q = pool->seqs[(size_t)s];
    q.live = true;
    q.len = 0;
    q.blocks.clear();
    *seq_out = s;
    return GQA_OK;
}

int gqa_kv_seq_fork(gqa_kv_pool* pool, int parent, int* child_out) {
    if (!pool || !child_out || !pool->known(parent)) return GQA_ERR_INVALID_ARG;
    if (pool->free_ids.empty()) return GQA_ERR_OUT_OF_BLOCKS;
    const int s = *pool->free_ids.begin();
    try {
        pool->seqs[(size_t)s].blocks = pool->seqs[(size_t)parent].blocks;
    } catch (const std::bad_alloc&) {
        return GQA_ERR_INVALID_ARG;
    }
    pool->free_ids.erase(pool->free_ids.begin());
    Seq& q = pool->seqs[(size_t)s];
    q.live = true;
    q.len = pool->seqs[(size_t)parent].len;
    for (const int32_t b : q.blocks) ++pool->refs[(size_t)b];
    *child_out = s;
    return GQA_OK;
}

int gqa_kv_seq_release(gqa_kv_pool* pool, int seq) {
    if (!pool || !pool->known(seq)) return GQA_ERR_INVALID_ARG;
    Seq& q = pool->seqs[(size_t)seq];
    for (const int32_t b : q.blocks) pool->drop(b);
    q.blocks.clear();
    q.len = 0;
    q.live = false;
    pool->free_ids.insert(seq);
    return GQA_OK;
}

int gqa_kv_seq_len(const gqa_kv_pool* pool, int seq) {
    if (!pool || !pool->known(seq)) return -1;
    return pool->seqs[(size_t)seq].len;
}

int gqa_kv_reserve(gqa_kv_pool* pool, const int* seqs, const int* counts, int n, int32_t* slots_out,
                   int32_t* copy_src, int32_t* copy_dst, int* n_copies) {
    if (!pool || n < 0 || !n_copies) return GQA_ERR_INVALID_ARG;
    if (n > 0 && (!seqs || !counts || !copy_src || !copy_dst)) return GQA_ERR_INVALID_ARG;
    int64_t need = 0, tokens = 0;
    try {
        const int st = plan_reserve(*pool, seqs, counts, n, need, tokens);
        if (st != GQA_OK) return st;
        if (tokens > 0 && !slots_out) return GQA_ERR_INVALID_ARG;
        if (need > (int64_t)pool->free_blocks.size()) return GQA_ERR_OUT_OF_BLOCKS;
        // Room for the new table entries first, so nothing below can fail
        // half way.
        for (int i = 0; i < n; ++i) {
            Seq& q = pool->seqs[(size_t)seqs[i]];
            q.blocks.reserve((size_t)pool->max_blocks);
        }
    } catch (const std::bad_alloc&) {
        return GQA_ERR_INVALID_ARG;
    }
    int nc = 0;
    int64_t k = 0;
    for (int i = 0; i < n; ++i) {
        Seq& q = pool->seqs[(size_t)seqs[i]];
        const int c = counts[i];
        if (c == 0) continue;
        if (q.len % kBlock != 0) {
            const int32_t last = q.blocks.back();
            if (pool->refs[(size_t)last] > 1) {          // shared and partly filled: copy on write
                const int32_t fresh = pool->take_block();
                pool->drop(last);
                copy_src[nc] = last;
                copy_dst[nc] = fresh;
                ++nc;
                q.blocks.back() = fresh;
            }
        }
        for (int t = 0; t < c; ++t) {
            const int32_t pos = q.len + t;
            if (pos % kBlock == 0) q.blocks.push_back(pool->take_block());
            slots_out[k++] = q.blocks[(size_t)(pos / kBlock)] * kBlock + pos % kBlock;
        }
        q.len += c;
    }
    *n_copies = nc;
    return GQA_OK;
}

int gqa_kv_block_table(const gqa_kv_pool* pool, const int* seqs, int n, int32_t* table_out, int max_blocks,
                       int32_t* lens_out) {
    if (!pool || !seqs || !table_out || !lens_out || n <= 0 || max_blocks <= 0) return GQA_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) {
        if (!pool->known(seqs[i])) return GQA_ERR_INVALID_ARG;
        if ((int64_t)pool->seqs[(size_t)seqs[i]].blocks.size() > max_blocks) return GQA_ERR_INVALID_ARG;
    }
    for (int i = 0; i < n; ++i) {
        const Seq& q = pool->seqs[(size_t)seqs[i]];
        int32_t* row = table_out + (size_t)i * max_blocks;
        for (int j = 0; j < max_blocks; ++j) row[j] = j < (int)q.blocks.size() ? q.blocks[(size_t)j] : -1;
        lens_out[i] = q.len;
    }
    return GQA_OK;
}

int attn_kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new, const int32_t* slots,
                   int n_tokens, int num_blocks, int Hkv, int d, int dtype, void* stream) {
    if (!k_cache || !v_cache || !k_new || !v_new || !slots || num_blocks <= 0) return GQA_ERR_INVALID_ARG;
    int row_bytes = 0;
    const int st = checked_rows(n_tokens, Hkv, d, dtype, row_bytes);
    if (st != GQA_OK) return st;
    if ((int64_t)n_tokens * Hkv >= ((int64_t)1 << 31) || (int64_t)num_blocks * kBlock >= ((int64_t)1 << 31))
        return GQA_ERR_INVALID_ARG;
    if (n_tokens == 0) return GQA_OK;
    gqa::KvAppendArgs a{k_cache, v_cache, k_new, v_new, slots, n_tokens, num_blocks, Hkv, row_bytes};
    return gqa::launch_kv_append(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src, const int32_t* dst, int n, int num_blocks,
                        int Hkv, int d, int dtype, void* stream) {
    if (!k_cache || !v_cache || !src || !dst || num_blocks <= 0) return GQA_ERR_INVALID_ARG;
    int row_bytes = 0;
    const int st = checked_rows(n, Hkv, d, dtype, row_bytes);
    if (st != GQA_OK) return st;
    if ((int64_t)n * Hkv * kBlock * (row_bytes / 16) >= ((int64_t)1 << 31)) return GQA_ERR_INVALID_ARG;
    if (n == 0) return GQA_OK;
    gqa::KvCopyArgs a{k_cache, v_cache, src, dst, n, num_blocks, Hkv, row_bytes};
    return gqa::launch_kv_copy_blocks(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_kv_append_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const void* k_new,
                       const void* v_new, const int32_t* slots, int n_tokens, int num_blocks, int Hkv, int d,
                       void* stream) {
    if (!k_cache || !v_cache || !k_scale || !v_scale || !k_new || !v_new || !slots || num_blocks <= 0)
        return GQA_ERR_INVALID_ARG;
    if (n_tokens < 0 || Hkv <= 0 || d <= 0) return GQA_ERR_INVALID_ARG;
    if (d != 128) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)n_tokens * Hkv * kBlock >= ((int64_t)1 << 31) || (int64_t)num_blocks * kBlock >= ((int64_t)1 << 31))
        return GQA_ERR_INVALID_ARG;
    if (n_tokens == 0) return GQA_OK;
    gqa::KvAppendArgs a{k_cache, v_cache, k_new, v_new, slots, n_tokens, num_blocks, Hkv, d, k_scale, v_scale};
    return gqa::launch_kv_append_fp8(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int attn_kv_copy_blocks_fp8(void* k_cache, void* v_cache, float* k_scale, float* v_scale, const int32_t* src,
                            const int32_t* dst, int n, int num_blocks, int Hkv, int d, void* stream) {
    if (!k_cache || !v_cache || !k_scale || !v_scale || !src || !dst || num_blocks <= 0) return GQA_ERR_INVALID_ARG;
    if (n < 0 || Hkv <= 0 || d <= 0) return GQA_ERR_INVALID_ARG;
    if (d != 128) return GQA_ERR_UNSUPPORTED;
    if ((int64_t)n * Hkv * kBlock * (d / 16) >= ((int64_t)1 << 31)) return GQA_ERR_INVALID_ARG;
    if (n == 0) return GQA_OK;
    gqa::KvCopyArgs a{k_cache, v_cache, src, dst, n, num_blocks, Hkv, d, k_scale, v_scale};
    return gqa::launch_kv_copy_blocks(a, static_cast<hipStream_t>(stream)) == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // extern "C"
