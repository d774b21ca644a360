"""GPU parity of the fp8 KV cache: quantising append, block copies with scales,
and decode over E4M3 codes with per-row scales.

Expected values come only from the oracle: codes and scales from
``oracle.kv_fp8.quantize_rows``, attention from ``oracle.core`` on the
dequantised rows (exact in fp64).
"""
import numpy as np
import pytest

import oracle
from oracle import kv_fp8 as F
from oracle import kv_pages as K
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def u8_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def f32_gpu(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def bf16_gpu(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def quantize_bits(bits):
    """bf16 bit patterns [..., d] -> oracle codes and scales."""
    return F.quantize_rows(ref_f64(bits, "bf16").astype(np.float32))


def special_rows(n, d, seed):
    """bf16 rows: N(0,1), zeros, -0, tiny, huge, one outlier (many subnormal codes), exact ties."""
    rng = np.random.default_rng(seed)
    x = rng.normal(0, 1, (max(n, 6), d)).astype(np.float32)
    x[0] = 0
    x[1] = -0.0
    x[2] *= 1e-30
    x[3] *= 1e30
    x[4] = rng.normal(0, 1e-3, d)
    x[4, 7] = 300.0
    x[5] = np.float32(1.0625)            # with amax 448 the factor is 1: every other element is a tie
    x[5, 0] = 448.0
    return W.f32_to_bf16_bits(x[:n] if n >= 6 else x[5 - n + 1:6])


@pytest.mark.parametrize("n,Hkv", [(1, 1), (37, 8), (300, 2), (1000, 1)])
def test_fp8_append_matches_oracle_quantisation(ga, n, Hkv):
    import torch
    note(f"fp8 append n{n} Hkv{Hkv}")
    d = 128
    rng = np.random.default_rng([11, n, Hkv])
    nb = n // 16 + 8
    rows_k = special_rows(n * Hkv, d, [12, n]).reshape(n, Hkv, d)
    rows_v = special_rows(n * Hkv, d, [13, n]).reshape(n, Hkv, d)[::-1].copy()
    slots = rng.choice(nb * 16, size=n, replace=False).astype(np.int32)
    if n > 4:
        slots[rng.integers(0, n)] = -1
    kc = np.full((nb, Hkv, 16, d), 0x5A, np.uint8)
    vc = np.full_like(kc, 0xA5)
    ks = np.full((nb, Hkv, 16), 7.0, np.float32)
    vs = np.full_like(ks, -3.0)
    want = [kc.copy(), vc.copy(), ks.copy(), vs.copy()]
    keep = slots >= 0
    for rows, codes_arr, scale_arr in ((rows_k, want[0], want[2]), (rows_v, want[1], want[3])):
        codes, scales = quantize_bits(rows[keep])
        K.scatter_tokens(codes_arr, slots[keep], codes)
        for i, s in enumerate(slots[keep]):
            scale_arr[s // 16, :, s % 16] = scales[i]
    g = [u8_gpu(kc), u8_gpu(vc), f32_gpu(ks), f32_gpu(vs)]
    ga.attn_kv_append_fp8(*g, bf16_gpu(rows_k), bf16_gpu(rows_v), to_gpu(slots, "i32"))
    torch.cuda.synchronize()
    assert np.array_equal(g[0].cpu().numpy(), want[0])
    assert np.array_equal(g[1].cpu().numpy(), want[1])
    assert np.array_equal(g[2].cpu().numpy().view(np.uint32), want[2].view(np.uint32))
    assert np.array_equal(g[3].cpu().numpy().view(np.uint32), want[3].view(np.uint32))


def test_fp8_copy_blocks_copies_codes_and_scales(ga):
    import torch
    rng = np.random.default_rng(14)
    nb, Hkv, d, n = 30, 8, 128, 9
    kc = rng.integers(0, 256, (nb, Hkv, 16, d), dtype=np.uint8)
    vc = rng.integers(0, 256, (nb, Hkv, 16, d), dtype=np.uint8)
    ks = rng.normal(0, 1, (nb, Hkv, 16)).astype(np.float32)
    vs = rng.normal(0, 1, (nb, Hkv, 16)).astype(np.float32)
    ids = rng.permutation(nb).astype(np.int32)
    src, dst = ids[:n], ids[n:2 * n]
    want = [a.copy() for a in (kc, vc, ks, vs)]
    for a in want:
        K.copy_blocks(a, zip(src, dst))
    g = [u8_gpu(kc), u8_gpu(vc), f32_gpu(ks), f32_gpu(vs)]
    ga.attn_kv_copy_blocks_fp8(*g, to_gpu(src, "i32"), to_gpu(dst, "i32"))
    torch.cuda.synchronize()
    for got, w in zip(g, want):
        assert np.array_equal(got.cpu().numpy(), w)


def test_fp8_single_key_returns_every_code_value(ga):
    """One cached token: the output is its V row exactly, so a V row walking
    the E4M3 codes shows how the GPU reads each of them."""
    import torch
    d = 128
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)        # 254 finite codes
    B, Hq, Hkv, S = 2, 4, 1, 16
    vc = np.zeros((B, Hkv, S, d), np.uint8)
    vc[0, 0, 0] = codes[:d]
    vc[1, 0, 0, :codes.size - d] = codes[d:]
    kc = np.random.default_rng(15).integers(0, 0x70, (B, Hkv, S, d), dtype=np.uint8)
    ks = np.ones((B, Hkv, S), np.float32)
    vs = np.ones((B, Hkv, S), np.float32)
    q = W.normal_bf16([15, 1], (B, Hq, d))
    lens = np.array([1, 1], np.int32)
    o = ga.attn_decode_fp8_fwd(to_gpu(q, "bf16"), u8_gpu(kc), u8_gpu(vc), f32_gpu(ks), f32_gpu(vs),
                               to_gpu(lens, "i32"))
    torch.cuda.synchronize()
    got = to_f64(o)
    table = F.e4m3_table()
    for b in range(B):
        want = table[vc[b, 0, 0]]
        for h in range(Hq):
            assert np.array_equal(got[b, h], want), (b, h)


def _fp8_case(seed, B, Hq, Hkv, lens, S_max, paged):
    """Oracle-quantised caches (contiguous, or paged with a random placement);
    scales of rows past each length are NaN: they must not be used."""
    d = 128
    lens = np.asarray(lens, np.int32)
    q = W.normal_bf16([seed, 0], (B, Hq, d))
    kb = W.normal_bf16([seed, 1], (B, Hkv, S_max, d))
    vb = W.normal_bf16([seed, 2], (B, Hkv, S_max, d))
    kq, ksc = quantize_bits(kb)
    vq, vsc = quantize_bits(vb)
    for b in range(B):
        ksc[b, :, lens[b]:] = np.nan
        vsc[b, :, lens[b]:] = np.nan
    k_deq, v_deq = F.dequantize_rows(kq, np.nan_to_num(ksc)), F.dequantize_rows(vq, np.nan_to_num(vsc))
    ref = oracle.decode_contiguous(ref_f64(q, "bf16"), k_deq, v_deq, lens)
    if not paged:
        return q, (kq, vq, ksc, vsc), None, ref
    max_blocks = S_max // 16
    table, nb = W.block_placement(seed, lens, max_blocks, spare_blocks=3)
    pages = [np.zeros((nb, Hkv, 16, d), np.uint8), np.zeros((nb, Hkv, 16, d), np.uint8),
             np.full((nb, Hkv, 16), np.nan, np.float32), np.full((nb, Hkv, 16), np.nan, np.float32)]
    for b in range(B):
        for j in range(-(-int(lens[b]) // 16)):
            p = table[b, j]
            pages[0][p] = kq[b, :, 16 * j:16 * j + 16]
            pages[1][p] = vq[b, :, 16 * j:16 * j + 16]
            pages[2][p] = ksc[b, :, 16 * j:16 * j + 16]
            pages[3][p] = vsc[b, :, 16 * j:16 * j + 16]
    return q, pages, table, ref


def _run_fp8(ga, q, cache, table, lens, max_seq_len=None):
    import torch
    kq, vq, ks, vs = cache
    o = ga.attn_decode_fp8_fwd(to_gpu(q, "bf16"), u8_gpu(kq), u8_gpu(vq), f32_gpu(ks), f32_gpu(vs),
                               to_gpu(np.asarray(lens, np.int32), "i32"),
                               block_table=None if table is None else to_gpu(table, "i32"), max_seq_len=max_seq_len)
    torch.cuda.synchronize()
    return o


LENS = [0, 1, 15, 16, 17, 63, 64, 65, 255, 257, 700]


@pytest.mark.parametrize("Hq,Hkv", [(32, 8), (32, 32), (32, 1), (16, 16)])
@pytest.mark.parametrize("paged", [False, True])
def test_fp8_decode_matches_oracle(ga, Hq, Hkv, paged):
    note(f"fp8 decode Hq{Hq} Hkv{Hkv} paged={paged}")
    q, cache, table, ref = _fp8_case(16, len(LENS), Hq, Hkv, LENS, 704, paged)
    o = _run_fp8(ga, q, cache, table, LENS, 704 if paged else None)
    assert_close(to_f64(o), ref, "bf16", f"fp8 decode Hq{Hq} Hkv{Hkv} paged={paged}")


def test_fp8_paged_equals_contiguous_bitwise(ga):
    import torch
    lens = [300, 17, 64, 1000]
    q, cont, _, _ = _fp8_case(17, 4, 32, 8, lens, 1024, False)
    _, pages, table, _ = _fp8_case(17, 4, 32, 8, lens, 1024, True)
    a = _run_fp8(ga, q, cont, None, lens)
    b = _run_fp8(ga, q, pages, table, lens, 1024)
    assert torch.equal(a, b)


def test_fp8_pool_append_then_decode_matches_definition(ga):
    """Prompts, forks, decode steps with copy-on-write through the fp8 calls;
    decode against fp64 attention over the oracle-quantised logical rows, and
    the pages read back through the tables bit for bit."""
    import torch
    d, Hq, Hkv, nb, max_blocks = 128, 32, 8, 200, 40
    rng = np.random.default_rng(18)
    pool = ga.KVPool(nb, 16, max_blocks)
    logical = K.LogicalKV()
    g = [torch.zeros((nb, Hkv, 16, d), dtype=torch.uint8, device="cuda") for _ in range(2)] + \
        [torch.full((nb, Hkv, 16), float("nan"), device="cuda") for _ in range(2)]
    counter = [0]

    def write(seqs, counts):
        n = int(sum(counts))
        counter[0] += 1
        rk = W.normal_bf16([18, 1, counter[0]], (n, Hkv, d))
        rv = W.normal_bf16([18, 2, counter[0]], (n, Hkv, d))
        slots, src, dst = pool.reserve(seqs, counts)
        if len(src):
            ga.attn_kv_copy_blocks_fp8(*g, to_gpu(src, "i32"), to_gpu(dst, "i32"))
        ga.attn_kv_append_fp8(*g, bf16_gpu(rk), bf16_gpu(rv), to_gpu(slots, "i32"))
        kq, ksc = quantize_bits(rk)
        vq, vsc = quantize_bits(rv)
        i = 0
        for s, c in zip(seqs, counts):
            logical.append(s, [(kq[j], ksc[j], vq[j], vsc[j]) for j in range(i, i + c)])
            i += c
        return len(src)

    seqs = []
    prompts = [37] + [int(x) for x in rng.integers(1, 300, size=4)]
    for _ in prompts:
        s = pool.seq_new()
        logical.new(s)
        seqs.append(s)
    write(seqs, prompts)
    for parent in (seqs[0], seqs[0], seqs[3]):
        c = pool.seq_fork(parent)
        logical.fork(parent, c)
        seqs.append(c)
    copies = sum(write(seqs, [1] * len(seqs)) for _ in range(4))
    assert copies > 0
    torch.cuda.synchronize()
    table, lens = pool.block_table(seqs, max_blocks)
    host = [t.cpu().numpy() for t in g]
    S_max = -(-int(lens.max()) // 16) * 16
    k_deq = np.zeros((len(seqs), Hkv, S_max, d))
    v_deq = np.zeros_like(k_deq)
    for i, s in enumerate(seqs):
        L = int(lens[i])
        rows = logical.seqs[s]
        for t, (kq, ksc, vq, vsc) in enumerate(rows):
            blk, off = table[i, t // 16], t % 16
            assert np.array_equal(host[0][blk, :, off], kq) and np.array_equal(host[1][blk, :, off], vq)
            assert np.array_equal(host[2][blk, :, off].view(np.uint32), ksc.view(np.uint32))
            assert np.array_equal(host[3][blk, :, off].view(np.uint32), vsc.view(np.uint32))
        k_deq[i, :, :L] = np.stack([F.dequantize_rows(r[0], r[1]) for r in rows], axis=1)
        v_deq[i, :, :L] = np.stack([F.dequantize_rows(r[2], r[3]) for r in rows], axis=1)
    q = W.normal_bf16([18, 3], (len(seqs), Hq, d))
    o = ga.attn_decode_fp8_fwd(to_gpu(q, "bf16"), *g, to_gpu(lens, "i32"), block_table=to_gpu(table, "i32"))
    torch.cuda.synchronize()
    ref = oracle.decode_contiguous(ref_f64(q, "bf16"), k_deq, v_deq, lens)
    assert_close(to_f64(o), ref, "bf16", "fp8 pool decode")
    pool.close()


@pytest.mark.slow
def test_full_size_fp8_paged_decode_mqa(ga):
    """The paged MQA workload (B16, Hkv 1, L ~ U[8192, 32768]) with its pages
    quantised by the oracle; every (sequence, head)."""
    w = W.cfg5(1)
    note(f"full-size fp8 paged decode {w.name}: generating and quantising inputs")
    di = W.decode_inputs(w)
    kq, ksc = quantize_bits(di.k_cache)
    vq, vsc = quantize_bits(di.v_cache)
    o = _run_fp8(ga, di.q, (kq, vq, ksc, vsc), di.block_table, di.seq_lens, di.max_seq_len)
    got = to_f64(o)
    k_deq = F.dequantize_rows(kq, ksc)
    v_deq = F.dequantize_rows(vq, vsc)
    ref = oracle.decode_paged(ref_f64(di.q, "bf16"), k_deq, v_deq, di.block_table, di.seq_lens,
                              scale=w.scale_value)
    assert_close(got, ref, "bf16", w.name)
