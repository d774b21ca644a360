"""GPU parity of the paged KV cache calls (attn_kv_append, attn_kv_copy_blocks)
and of decode over a cache built with them through the library's page pool.

Expected values come only from the oracle: rows scattered through slots and
blocks copied with numpy (``oracle.kv_pages``), the logical sequences of
``LogicalKV``, and fp64 decode over those sequences (``oracle.core``).
Byte moves are compared bit for bit.
"""
import numpy as np
import pytest

import oracle
from oracle import kv_pages as K
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

_BITS = {"bf16": np.uint16, "f32": np.uint32}


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def bits_to_gpu(bits: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int32)).view(torch.float32).cuda()


def gpu_to_bits(t, dtype: str) -> np.ndarray:
    import torch
    if dtype == "bf16":
        return t.cpu().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().view(torch.int32).numpy().view(np.uint32)


def random_bits(rng, shape, dtype):
    info = np.iinfo(_BITS[dtype])
    return rng.integers(0, int(info.max) + 1, size=shape, dtype=_BITS[dtype])


@pytest.mark.parametrize("dtype,d,Hkv,n", [("bf16", 128, 8, 1000), ("bf16", 64, 2, 77), ("f32", 128, 1, 33),
                                           ("f32", 64, 4, 1), ("bf16", 128, 32, 300), ("bf16", 128, 1, 4096)])
def test_append_matches_oracle_scatter(ga, dtype, d, Hkv, n):
    import torch
    note(f"kv append {dtype} d{d} Hkv{Hkv} n{n}")
    rng = np.random.default_rng([7, d, Hkv, n])
    nb = n // 16 + 20
    kp, vp = random_bits(rng, (nb, Hkv, 16, d), dtype), random_bits(rng, (nb, Hkv, 16, d), dtype)
    kn, vn = random_bits(rng, (n, Hkv, d), dtype), random_bits(rng, (n, Hkv, d), dtype)
    slots = rng.choice(nb * 16, size=n, replace=False).astype(np.int32)
    if n > 4:
        slots[rng.choice(n, size=max(1, n // 10), replace=False)] = -1       # padding tokens
        slots[rng.integers(0, n)] = nb * 16 + 5                              # past the pages: skipped
    keep = (slots >= 0) & (slots < nb * 16)
    want_k, want_v = kp.copy(), vp.copy()
    K.scatter_tokens(want_k, slots[keep], kn[keep])
    K.scatter_tokens(want_v, slots[keep], vn[keep])
    kc, vc = bits_to_gpu(kp, dtype), bits_to_gpu(vp, dtype)
    ga.attn_kv_append(kc, vc, bits_to_gpu(kn, dtype), bits_to_gpu(vn, dtype), to_gpu(slots, "i32"))
    torch.cuda.synchronize()
    assert np.array_equal(gpu_to_bits(kc, dtype), want_k)
    assert np.array_equal(gpu_to_bits(vc, dtype), want_v)


@pytest.mark.parametrize("dtype,d,Hkv,n", [("bf16", 128, 8, 40), ("f32", 64, 2, 3), ("bf16", 64, 32, 1),
                                           ("bf16", 128, 8, 500)])
def test_copy_blocks_match_oracle(ga, dtype, d, Hkv, n):
    import torch
    note(f"kv copy blocks {dtype} d{d} Hkv{Hkv} n{n}")
    rng = np.random.default_rng([8, d, Hkv, n])
    nb = 2 * n + 6
    kp, vp = random_bits(rng, (nb, Hkv, 16, d), dtype), random_bits(rng, (nb, Hkv, 16, d), dtype)
    ids = rng.permutation(nb).astype(np.int32)
    src, dst = ids[:n].copy(), ids[n:2 * n].copy()                      # no dst is a src or repeats
    src_all = np.concatenate([src, np.array([nb + 2], np.int32)])        # one pair out of range: skipped
    dst_all = np.concatenate([dst, np.array([ids[-1]], np.int32)])
    want_k, want_v = kp.copy(), vp.copy()
    K.copy_blocks(want_k, zip(src, dst))
    K.copy_blocks(want_v, zip(src, dst))
    kc, vc = bits_to_gpu(kp, dtype), bits_to_gpu(vp, dtype)
    ga.attn_kv_copy_blocks(kc, vc, to_gpu(src_all, "i32"), to_gpu(dst_all, "i32"))
    torch.cuda.synchronize()
    assert np.array_equal(gpu_to_bits(kc, dtype), want_k)
    assert np.array_equal(gpu_to_bits(vc, dtype), want_v)


def _write(ga, pool, kc, vc, seqs, counts, rows_k, rows_v):
    """Reserve slots, perform the copies, write the rows (bf16 bits [n, Hkv, d])."""
    import torch
    slots, src, dst = pool.reserve(seqs, counts)
    if len(src):
        ga.attn_kv_copy_blocks(kc, vc, to_gpu(src, "i32"), to_gpu(dst, "i32"))
    ga.attn_kv_append(kc, vc, bits_to_gpu(rows_k, "bf16"), bits_to_gpu(rows_v, "bf16"), to_gpu(slots, "i32"))
    torch.cuda.synchronize()
    return slots, src


@pytest.mark.parametrize("seed,Hq,Hkv", [(0, 32, 8), (1, 32, 32), (2, 32, 1), (3, 16, 4)])
def test_pool_append_then_decode_matches_definition(ga, seed, Hq, Hkv):
    """Prompts, forks sharing them, decode steps with copy-on-write, a release;
    then paged decode over the result against fp64 attention over the logical
    sequences, and the pages read back through the tables bit for bit."""
    import torch
    d, nb, max_blocks = 128, 300, 80
    rng = np.random.default_rng([9, seed])
    pool = ga.KVPool(nb, 24, max_blocks)
    logical = K.LogicalKV()
    kc = bits_to_gpu(W.normal_bf16([9, seed, 1], (nb, Hkv, 16, d)), "bf16")   # stale contents everywhere
    vc = bits_to_gpu(W.normal_bf16([9, seed, 2], (nb, Hkv, 16, d)), "bf16")
    counter = [0]

    def rows(n):
        counter[0] += 1
        return (W.normal_bf16([9, seed, 10, counter[0]], (n, Hkv, d)),
                W.normal_bf16([9, seed, 11, counter[0]], (n, Hkv, d)))

    def write(seqs, counts):
        n = int(sum(counts))
        rk, rv = rows(n)
        _, src = _write(ga, pool, kc, vc, seqs, counts, rk, rv)
        i = 0
        for s, c in zip(seqs, counts):
            logical.append(s, [(rk[j], rv[j]) for j in range(i, i + c)])
            i += c
        return len(src)

    note(f"pool + decode seed {seed} Hq{Hq} Hkv{Hkv}: prompts")
    prompts = [37] + [int(x) for x in rng.integers(1, 400, size=4)] + [16, 32]   # 37: forks must copy
    seqs = []
    for L in prompts:
        s = pool.seq_new()
        logical.new(s)
        seqs.append(s)
    write(seqs, prompts)
    copies = 0
    for parent in (seqs[0], seqs[0], seqs[2], seqs[5]):                  # forks share the prompts
        c = pool.seq_fork(parent)
        logical.fork(parent, c)
        seqs.append(c)
    for step in range(6):                                                # decode steps, one token each
        copies += write(seqs, [1] * len(seqs))
        if step == 2:
            gone = seqs.pop(1)
            pool.seq_release(gone)
            logical.release(gone)
    assert copies > 0                                                    # some writes went through a copy
    table, lens = pool.block_table(seqs, max_blocks)
    # pages read back through the tables are the logical sequences, bit for bit
    kp, vp = gpu_to_bits(kc, "bf16"), gpu_to_bits(vc, "bf16")
    S_max = int(lens.max())
    k_log = np.zeros((len(seqs), Hkv, S_max, d), np.uint16)
    v_log = np.zeros_like(k_log)
    for i, s in enumerate(seqs):
        L = int(lens[i])
        assert L == len(logical.seqs[s])
        want_k = np.array([r[0] for r in logical.seqs[s]])
        want_v = np.array([r[1] for r in logical.seqs[s]])
        assert np.array_equal(K.gather(kp, table[i], L), want_k)
        assert np.array_equal(K.gather(vp, table[i], L), want_v)
        k_log[i, :, :L] = want_k.transpose(1, 0, 2)
        v_log[i, :, :L] = want_v.transpose(1, 0, 2)
    note(f"pool + decode seed {seed}: paged decode of {len(seqs)} sequences")
    q = W.normal_bf16([9, seed, 3], (len(seqs), Hq, d))
    o = ga.attn_decode_fwd(to_gpu(q, "bf16"), kc, vc, to_gpu(lens, "i32"), block_table=to_gpu(table, "i32"))
    torch.cuda.synchronize()
    ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(k_log, "bf16"), ref_f64(v_log, "bf16"), lens)
    assert_close(to_f64(o), ref, "bf16", f"pool decode seed {seed}")
    pool.close()


@pytest.mark.slow
def test_full_size_bulk_append(ga):
    """The paged decode workload's tokens (B16, L ~ U[8192, 32768], Hkv 8)
    written in one call through the pool; sampled rows bit for bit, then decode
    over the pages against fp64 attention on sampled heads."""
    import torch
    w = W.cfg5(8)
    lens = W.seq_lengths(w.seed, w.B, w.L_lo, w.L_hi)
    N = int(lens.sum())
    nb = int(sum(-(-int(L) // 16) for L in lens)) + 8
    max_blocks = w.max_blocks
    note(f"full-size bulk append: {N} tokens, {nb} blocks")
    pool = ga.KVPool(nb, w.B, max_blocks)
    seqs = [pool.seq_new() for _ in range(w.B)]
    slots, src, _ = pool.reserve(seqs, lens.tolist())
    assert len(src) == 0 and len(slots) == N
    kn = W.normal_bf16([5, 21], (N, w.Hkv, w.d))
    vn = W.normal_bf16([5, 22], (N, w.Hkv, w.d))
    kc = torch.zeros((nb, w.Hkv, 16, w.d), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    ga.attn_kv_append(kc, vc, bits_to_gpu(kn, "bf16"), bits_to_gpu(vn, "bf16"), to_gpu(slots, "i32"))
    torch.cuda.synchronize()
    rng = np.random.default_rng(55)
    pick = np.sort(rng.choice(N, size=4096, replace=False))
    s = torch.from_numpy(slots[pick].astype(np.int64)).cuda()
    got_k = gpu_to_bits(kc[s // 16, :, s % 16, :].contiguous(), "bf16")
    got_v = gpu_to_bits(vc[s // 16, :, s % 16, :].contiguous(), "bf16")
    assert np.array_equal(got_k, kn[pick]) and np.array_equal(got_v, vn[pick])
    table, tl = pool.block_table(seqs, max_blocks)
    assert np.array_equal(tl, lens)
    q = W.normal_bf16([5, 23], (w.B, w.Hq, w.d))
    o = ga.attn_decode_fwd(to_gpu(q, "bf16"), kc, vc, to_gpu(lens, "i32"), block_table=to_gpu(table, "i32"))
    torch.cuda.synchronize()
    got = to_f64(o)
    starts = np.concatenate([[0], np.cumsum(lens)])
    for b, h in [(0, 0), (5, 17), (w.B - 1, w.Hq - 1)]:
        hk = h // (w.Hq // w.Hkv)
        kb = ref_f64(kn[starts[b]:starts[b + 1], hk], "bf16")
        vb = ref_f64(vn[starts[b]:starts[b + 1], hk], "bf16")
        ob, _, _ = oracle.attention_head(ref_f64(q[b, h], "bf16")[None, :], kb, vb, w.scale_value)
        assert_close(got[b, h][None, :], ob, "bf16", f"bulk append decode b{b} h{h}")
    pool.close()
