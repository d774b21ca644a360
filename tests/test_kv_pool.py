"""Paged KV cache on the CPU: the oracle's page pool pinned to what the pages
fix, planted mistakes in it caught, and the library's pool (host code behind
the C ABI) compared with it exactly on random operation sequences.

[Different attention mechanisms, §5 Page Attention]: fixed-size blocks
stored anywhere, one page table per sequence, blocks taken on demand as
tokens arrive, common prefixes shared copy-on-write.
"""
import random

import numpy as np
import pytest

from oracle import kv_pages as K

BLOCK = K.BLOCK


# ---- pins of the oracle ------------------------------------------------------

def refs_from_tables(pool):
    refs = [0] * pool.num_blocks
    for t in pool.tables.values():
        for b in t:
            refs[b] += 1
    return refs


def check_invariants(pool):
    # every reference count is the number of table entries naming the block
    assert pool.refs == refs_from_tables(pool)
    # a sequence of length L holds ceil(L / 16) blocks: near-zero waste
    for sid, t in pool.tables.items():
        assert len(t) == -(-pool.lens[sid] // BLOCK)
    assert pool.free_blocks() == pool.num_blocks - len({b for t in pool.tables.values() for b in t})


def test_fresh_sequence_takes_consecutive_slots():
    pool = K.PagePool(64, 4, 16)
    s = pool.new_seq()
    slots, copies = pool.reserve([s], [40])
    assert slots == list(range(40)) and copies == []
    assert pool.tables[s] == [0, 1, 2] and pool.free_blocks() == 61
    check_invariants(pool)


@pytest.mark.parametrize("chunks", [[1] * 40, [15, 1, 16, 1], [16, 16], [7, 9, 17, 3], [33]])
def test_blocks_taken_only_when_last_is_full(chunks):
    pool = K.PagePool(64, 2, 16)
    s = pool.new_seq()
    taken = 0
    for c in chunks:
        before = pool.free_blocks()
        L = pool.lens[s]
        slots, _ = pool.reserve([s], [c])
        taken = before - pool.free_blocks()
        assert taken == -(-(L + c) // BLOCK) - -(-L // BLOCK)
        t = pool.tables[s]
        assert slots == [t[p // BLOCK] * BLOCK + p % BLOCK for p in range(L, L + c)]
    check_invariants(pool)


@pytest.mark.parametrize("L,copy_expected", [(20, True), (32, False), (1, True), (16, False)])
def test_fork_shares_and_copies_only_a_shared_partial_block(L, copy_expected):
    pool = K.PagePool(64, 4, 16)
    p = pool.new_seq()
    pool.reserve([p], [L])
    free0 = pool.free_blocks()
    c = pool.fork(p)
    assert pool.free_blocks() == free0                      # a fork takes no block
    assert pool.tables[c] == pool.tables[p]
    assert all(pool.refs[b] == 2 for b in pool.tables[p])
    last = pool.tables[p][-1]
    slots, copies = pool.reserve([c], [1])
    if copy_expected:
        assert copies == [(last, pool.tables[c][-1])] and pool.tables[c][-1] != last
        assert pool.refs[last] == 1 and pool.free_blocks() == free0 - 1
        # the parent now writes into its own block without another copy
        _, copies2 = pool.reserve([p], [1])
        assert copies2 == []
    else:
        assert copies == [] and pool.tables[c][:-1] == pool.tables[p]
    assert pool.refs[pool.tables[c][-1]] == 1                # written blocks are private
    check_invariants(pool)


def test_prefix_sharing_saves_memory():
    pool = K.PagePool(256, 16, 16)
    p = pool.new_seq()
    pool.reserve([p], [100])                                 # 7 blocks, the last holds 4 tokens
    kids = [pool.fork(p) for _ in range(8)]
    pool.reserve(kids, [10] * 8)                             # each copies the partial block once
    assert pool.num_blocks - pool.free_blocks() == 7 + 8     # unshared: 7 + 8 * 7 blocks
    check_invariants(pool)


def test_release_frees_blocks_no_one_else_references():
    pool = K.PagePool(64, 4, 16)
    p = pool.new_seq()
    pool.reserve([p], [40])
    c = pool.fork(p)
    pool.reserve([c], [5])
    pool.release(p)
    check_invariants(pool)
    assert pool.num_blocks - pool.free_blocks() == 3         # blocks 0, 1 shared, c's copy of 2
    pool.release(c)
    assert pool.free_blocks() == 64 and not pool.tables


def test_failed_reservation_changes_nothing():
    pool = K.PagePool(8, 4, 8)
    a, b = pool.new_seq(), pool.new_seq()
    pool.reserve([a], [20])
    c = pool.fork(a)
    state = (dict((k, list(v)) for k, v in pool.tables.items()), dict(pool.lens), list(pool.refs))
    with pytest.raises(K.OutOfBlocks):
        pool.reserve([c, b, a], [1, 16, 100])               # needs more than the 6 free blocks
    with pytest.raises(K.InvalidRequest):
        pool.reserve([a, 3], [1, 1])                         # 3 is not a live sequence
    with pytest.raises(K.InvalidRequest):
        pool.reserve([a], [-1])
    with pytest.raises(K.InvalidRequest):
        pool.reserve([b], [8 * 16 + 1])                      # wider than its page table
    assert (pool.tables, pool.lens, pool.refs) == state


def random_ops(pool, logical, pages, rng, steps, Hkv, d, max_chunk=40, record=None):
    """Random new / fork / reserve+write / release; pages written as the pool says."""
    next_val = [1]
    for _ in range(steps):
        live = sorted(pool.tables)
        op = rng.random()
        if op < 0.15 or not live:
            try:
                s = pool.new_seq()
            except K.OutOfBlocks:
                continue
            logical.new(s)
        elif op < 0.3:
            parent = rng.choice(live)
            try:
                s = pool.fork(parent)
            except K.OutOfBlocks:
                continue
            logical.fork(parent, s)
        elif op < 0.4 and len(live) > 1:
            s = rng.choice(live)
            pool.release(s)
            logical.release(s)
        else:
            seqs = [rng.choice(live) for _ in range(rng.randint(1, 4))]
            counts = [rng.randint(0, max_chunk) for _ in seqs]
            try:
                slots, copies = pool.reserve(seqs, counts)
            except (K.OutOfBlocks, K.InvalidRequest):
                continue
            n = len(slots)
            rows = np.arange(next_val[0], next_val[0] + n * Hkv * d, dtype=np.int64).reshape(n, Hkv, d)
            next_val[0] += n * Hkv * d
            K.copy_blocks(pages, copies)
            K.scatter_tokens(pages, slots, rows)
            for blk in {s_ // BLOCK for s_ in slots}:
                assert pool.refs[blk] == 1                   # a written block is private
            i = 0
            for s, c in zip(seqs, counts):
                logical.append(s, list(rows[i:i + c]))
                i += c
            if record is not None:
                record.append((seqs, counts, slots, copies))


def check_against_definition(pool, logical, pages):
    assert sorted(pool.tables) == sorted(logical.seqs)
    for s, rows in logical.seqs.items():
        got = K.gather(pages, pool.tables[s], pool.lens[s])
        want = np.array(rows).reshape(len(rows), pages.shape[1], pages.shape[3]) if rows else got[:0]
        assert np.array_equal(got, want), f"sequence {s}"


@pytest.mark.parametrize("seed", range(6))
def test_pages_read_back_through_tables_equal_the_definition(seed):
    rng = random.Random(seed)
    Hkv, d = 2, 3
    pool = K.PagePool(96, 12, 20)
    logical = K.LogicalKV()
    pages = np.zeros((96, Hkv, BLOCK, d), dtype=np.int64)
    for _ in range(10):
        random_ops(pool, logical, pages, rng, 25, Hkv, d)
        check_invariants(pool)
        check_against_definition(pool, logical, pages)


# ---- planted mistakes in the pool must fail a pin ------------------------------

def _no_copy(self, sid):                       # writes into a shared block
    table, pos = self.tables[sid], self.lens[sid]
    if pos % BLOCK == 0:
        table.append(self._take_block())
    self.lens[sid] = pos + 1
    return table[pos // BLOCK] * BLOCK + pos % BLOCK, None


_WRITE_SLOT = K.PagePool._write_slot


def _copy_unrecorded(self, sid):               # repoints without copying the contents
    slot, copied = _WRITE_SLOT(self, sid)
    return slot, None


def _block_every_15(self, sid):                # off by one in the block size
    table, pos = self.tables[sid], self.lens[sid]
    if pos % (BLOCK - 1) == 0:
        table.append(self._take_block())
    self.lens[sid] = pos + 1
    return table[pos // (BLOCK - 1)] * BLOCK + pos % (BLOCK - 1), None


def _fork_no_ref(self, parent):                # child shares blocks without a reference
    self._check(parent)
    child = self.new_seq()
    self.tables[child] = list(self.tables[parent])
    self.lens[child] = self.lens[parent]
    return child


POOL_MUTANTS = {"no_copy_on_write": ("_write_slot", _no_copy),
                "copy_unrecorded": ("_write_slot", _copy_unrecorded),
                "block_every_15": ("_write_slot", _block_every_15),
                "fork_without_reference": ("fork", _fork_no_ref)}

POOL_PINS = [test_fresh_sequence_takes_consecutive_slots,
             lambda: [test_blocks_taken_only_when_last_is_full(c) for c in ([15, 1, 16, 1], [33])],
             lambda: [test_fork_shares_and_copies_only_a_shared_partial_block(L, e) for L, e in ((20, True), (32, False))],
             test_prefix_sharing_saves_memory,
             test_release_frees_blocks_no_one_else_references,
             lambda: [test_pages_read_back_through_tables_equal_the_definition(s) for s in range(3)]]


@pytest.mark.parametrize("name", sorted(POOL_MUTANTS))
def test_pool_mutant_fails_a_pin(name, monkeypatch):
    attr, fn = POOL_MUTANTS[name]
    monkeypatch.setattr(K.PagePool, attr, fn)
    failed = 0
    for pin in POOL_PINS:
        try:
            pin()
        except (AssertionError, IndexError):   # a pin fails, or a table lookup runs past its end
            failed += 1
    assert failed > 0, f"mutant {name} passed every pin"


# ---- the library's pool against the oracle --------------------------------------

@pytest.fixture(scope="module")
def ga():
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def _both(ga, fn_lib, fn_ref):
    """Run one operation on both pools; results and error kinds must agree."""
    err_map = {ga.OutOfBlocksError: K.OutOfBlocks, ValueError: K.InvalidRequest}
    try:
        got = fn_lib()
        got_err = None
    except (ga.OutOfBlocksError, ValueError) as e:
        got, got_err = None, err_map[type(e)]
    try:
        want = fn_ref()
        want_err = None
    except (K.OutOfBlocks, K.InvalidRequest) as e:
        want, want_err = None, type(e)
    assert got_err == want_err
    return got, want


@pytest.mark.parametrize("seed", range(8))
def test_library_pool_matches_oracle(ga, seed):
    rng = random.Random(100 + seed)
    nb, ms, mb = rng.choice([(40, 6, 12), (200, 16, 30), (17, 3, 6)])
    lib = ga.KVPool(nb, ms, mb)
    ref = K.PagePool(nb, ms, mb)
    for step in range(300):
        live = sorted(ref.tables)
        op = rng.random()
        if op < 0.12 or not live:
            got, want = _both(ga, lib.seq_new, ref.new_seq)
            assert got == want
        elif op < 0.25:
            p = rng.choice(live)
            got, want = _both(ga, lambda: lib.seq_fork(p), lambda: ref.fork(p))
            assert got == want
        elif op < 0.35 and len(live) > 1:
            s = rng.choice(live)
            lib.seq_release(s)
            ref.release(s)
        else:
            pick = live + ([ms + 3] if rng.random() < 0.05 else [])       # now and then an unknown id
            seqs = [rng.choice(pick) for _ in range(rng.randint(1, 5))]
            counts = [rng.randint(0, 50) if rng.random() > 0.03 else -1 for _ in seqs]
            got, want = _both(ga, lambda: lib.reserve(seqs, counts), lambda: ref.reserve(seqs, counts))
            if want is not None:
                slots, src, dst = got
                assert slots.tolist() == want[0]
                assert list(zip(src.tolist(), dst.tolist())) == want[1]
        assert lib.free_blocks() == ref.free_blocks()
        if ref.tables:
            ids = sorted(ref.tables)
            table, lens = lib.block_table(ids, mb)
            rt, rl = ref.block_table(ids, mb)
            assert np.array_equal(table, rt) and np.array_equal(lens, rl)
            for s in ids:
                assert lib.seq_len(s) == ref.lens[s]
    lib.close()


def test_library_pool_rejects_bad_arguments(ga):
    with pytest.raises(ValueError):
        ga.KVPool(0, 4, 4)
    with pytest.raises(ValueError):
        ga.KVPool(1 << 27, 4, 4)                  # slots would overflow int32
    pool = ga.KVPool(4, 2, 3)
    a = pool.seq_new()
    b = pool.seq_new()
    with pytest.raises(ga.OutOfBlocksError):
        pool.seq_new()                            # two live sequences is the limit
    with pytest.raises(ga.OutOfBlocksError):
        pool.seq_fork(a)
    with pytest.raises(ValueError):
        pool.seq_release(7)
    with pytest.raises(ValueError):
        pool.block_table([a, 5], 3)
    pool.reserve([a], [32])                       # two of the four blocks
    with pytest.raises(ValueError):
        pool.block_table([a], 1)                  # a holds two blocks
    with pytest.raises(ga.OutOfBlocksError):
        pool.reserve([b], [48])                   # three blocks, two are free
    with pytest.raises(ValueError):
        pool.reserve([b], [49])                   # four blocks: wider than the table (checked first)
    assert pool.free_blocks() == 2 and pool.seq_len(b) == 0
    assert pool.seq_len(a) == 32 and pool.seq_len(9) == -1
    lib = ga.load_library()
    assert lib.gqa_kv_pool_free_blocks(None) == -1
    assert lib.gqa_kv_reserve(None, None, None, 0, None, None, None, None) == ga.GQA_ERR_INVALID_ARG
    pool.close()


FAKE = 0x100000   # never dereferenced: every call below fails validation before any HIP call


@pytest.mark.parametrize("kw,status", [
    (dict(k=None), 1), (dict(slots=None), 1), (dict(n=-1), 1), (dict(Hkv=0), 1), (dict(num_blocks=0), 1),
    (dict(dtype=5), 1), (dict(d=96), 2), (dict(d=256), 2), (dict(n=1 << 28, Hkv=8), 1),
    (dict(n=0), 0),                               # nothing to do: no launch
])
def test_kv_append_rejects_on_host(ga, kw, status):
    a = dict(k=FAKE, v=FAKE, kn=FAKE, vn=FAKE, slots=FAKE, n=4, num_blocks=8, Hkv=2, d=128, dtype=1)
    a.update(kw)
    lib = ga.load_library()
    assert lib.attn_kv_append(a["k"], a["v"], a["kn"], a["vn"], a["slots"], a["n"], a["num_blocks"], a["Hkv"],
                              a["d"], a["dtype"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(src=None), 1), (dict(n=-2), 1), (dict(num_blocks=-1), 1), (dict(d=32), 2), (dict(dtype=9), 1),
    (dict(n=1 << 27, Hkv=8), 1), (dict(n=0), 0),
])
def test_kv_copy_rejects_on_host(ga, kw, status):
    a = dict(k=FAKE, v=FAKE, src=FAKE, dst=FAKE, n=3, num_blocks=8, Hkv=2, d=64, dtype=0)
    a.update(kw)
    lib = ga.load_library()
    assert lib.attn_kv_copy_blocks(a["k"], a["v"], a["src"], a["dst"], a["n"], a["num_blocks"], a["Hkv"], a["d"],
                                   a["dtype"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), 1), (dict(vs=None), 1), (dict(k=None), 1), (dict(d=64), 2), (dict(n=-1), 1), (dict(Hkv=0), 1),
    (dict(n=0), 0),
])
def test_kv_append_fp8_rejects_on_host(ga, kw, status):
    a = dict(k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, kn=FAKE, vn=FAKE, slots=FAKE, n=4, num_blocks=8, Hkv=2, d=128)
    a.update(kw)
    lib = ga.load_library()
    assert lib.attn_kv_append_fp8(a["k"], a["v"], a["ks"], a["vs"], a["kn"], a["vn"], a["slots"], a["n"],
                                  a["num_blocks"], a["Hkv"], a["d"], None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(ks=None), 1), (dict(dst=None), 1), (dict(d=64), 2), (dict(n=-1), 1), (dict(n=0), 0),
])
def test_kv_copy_fp8_rejects_on_host(ga, kw, status):
    a = dict(k=FAKE, v=FAKE, ks=FAKE, vs=FAKE, src=FAKE, dst=FAKE, n=3, num_blocks=8, Hkv=2, d=128)
    a.update(kw)
    lib = ga.load_library()
    assert lib.attn_kv_copy_blocks_fp8(a["k"], a["v"], a["ks"], a["vs"], a["src"], a["dst"], a["n"],
                                       a["num_blocks"], a["Hkv"], a["d"], None) == status
