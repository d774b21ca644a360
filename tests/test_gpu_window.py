"""GPU parity of sliding-window attention (attn_prefill_window_fwd,
attn_decode_window_fwd) against the fp64 oracle's window reading: each query
sees its last W keys, causal [Attention variants deep-dive, §8 Q4]."""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from tests.test_gpu_prefill import inputs, sample_rows
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def run_window(ga, q, k, v, dtype, window):
    import torch
    o = ga.attn_prefill_window_fwd(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype), window=window)
    torch.cuda.synchronize()
    return o


@pytest.mark.parametrize("dtype,d,Hq,Hkv,Sq,Sk,Wn", [
    ("bf16", 128, 32, 8, 1024, 1024, 256),      # GQA, window of 4 tiles
    ("bf16", 128, 4, 4, 700, 700, 100),         # MHA, ragged, window across tile edges
    ("bf16", 64, 8, 2, 300, 500, 64),           # Sq < Sk
    ("bf16", 128, 16, 4, 512, 512, 37),         # window not a multiple of 16
    ("bf16", 128, 8, 1, 257, 257, 1),           # one key: each row returns its own V row
    ("bf16", 64, 16, 16, 130, 130, 129),
    ("f32", 64, 4, 2, 128, 128, 17),
    ("f32", 128, 8, 4, 100, 300, 50),
])
def test_prefill_window_matches_oracle(ga, dtype, d, Hq, Hkv, Sq, Sk, Wn):
    note(f"window prefill {dtype} d{d} Hq{Hq} Hkv{Hkv} Sq{Sq} Sk{Sk} W{Wn}")
    q, k, v = inputs(40 + Wn, 1, Hq, Hkv, Sq, Sk, d, dtype)
    o = run_window(ga, q, k, v, dtype, Wn)
    ref = oracle.attention(ref_f64(q, dtype), ref_f64(k, dtype), ref_f64(v, dtype), window=Wn)
    assert_close(to_f64(o), ref, dtype, f"window {Wn}")
    if Wn == 1:                                   # exactly the diagonal V row (bf16 input, exact output)
        got = to_f64(o)[0]
        vv = ref_f64(v, dtype)[0]
        g = Hq // Hkv
        for h in range(Hq):
            assert np.array_equal(got[h], vv[h // g, Sk - Sq:])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_window_covering_everything_equals_causal_bitwise(ga, dtype):
    import torch
    q, k, v = inputs(41, 2, 8, 2, 384, 384, 128 if dtype == "bf16" else 64, dtype)
    a = run_window(ga, q, k, v, dtype, 384)
    b = ga.attn_prefill_fwd(to_gpu(q, dtype), to_gpu(k, dtype), to_gpu(v, dtype), causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def _decode_case(seed, B, Hq, Hkv, lens, S_max, paged, d=128):
    lens = np.asarray(lens, np.int32)
    q = W.normal_bf16([seed, 0], (B, Hq, d))
    if paged:
        table, nb = W.block_placement(seed, lens, -(-S_max // 16), spare_blocks=3)
        kp = W.normal_bf16([seed, 1], (nb, Hkv, 16, d))
        vp = W.normal_bf16([seed, 2], (nb, Hkv, 16, d))
        return q, kp, vp, lens, table
    kc = W.normal_bf16([seed, 1], (B, Hkv, S_max, d))
    vc = W.normal_bf16([seed, 2], (B, Hkv, S_max, d))
    return q, kc, vc, lens, None


def run_decode(ga, q, kc, vc, lens, table, S_max, window):
    import torch
    kw = dict(block_table=to_gpu(table, "i32"), max_seq_len=S_max) if table is not None else {}
    if window is not None:
        kw["window"] = window
    o = ga.attn_decode_fwd(to_gpu(q, "bf16"), to_gpu(kc, "bf16"), to_gpu(vc, "bf16"), to_gpu(lens, "i32"), **kw)
    torch.cuda.synchronize()
    return o


LENS = [0, 1, 15, 16, 17, 63, 255, 256, 700, 1024]


@pytest.mark.parametrize("paged", [False, True])
@pytest.mark.parametrize("Hq,Hkv,Wn,d", [(32, 8, 16, 128), (32, 8, 100, 128), (32, 32, 1, 128), (32, 1, 512, 128),
                                         (16, 4, 300, 128), (32, 8, 100, 64), (32, 1, 17, 64)])
def test_decode_window_matches_oracle(ga, paged, Hq, Hkv, Wn, d):
    note(f"window decode Hq{Hq} Hkv{Hkv} W{Wn} d{d} paged={paged}")
    q, kc, vc, lens, table = _decode_case(50 + Wn + d, len(LENS), Hq, Hkv, LENS, 1024, paged, d)
    o = run_decode(ga, q, kc, vc, lens, table, 1024, Wn)
    if paged:
        ref = oracle.decode_paged(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), table, lens, window=Wn)
    else:
        ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(kc, "bf16"), ref_f64(vc, "bf16"), lens, window=Wn)
    assert_close(to_f64(o), ref, "bf16", f"window decode W{Wn}")


def test_decode_window_covering_everything_equals_decode_bitwise(ga):
    import torch
    q, kc, vc, lens, table = _decode_case(60, len(LENS), 32, 8, LENS, 1024, True)
    a = run_decode(ga, q, kc, vc, lens, table, 1024, 1024)
    b = run_decode(ga, q, kc, vc, lens, table, 1024, None)
    assert torch.equal(a, b)


@pytest.mark.slow
def test_full_size_window_prefill_sampled(ga):
    """The GQA S = 8192 workload with a 4096-key window: sampled rows of every head."""
    import torch
    w = W.PREFILL_WORKLOADS[3]
    Wn = 4096
    note(f"full-size window prefill {w.name} W{Wn}")
    q, k, v = W.prefill_inputs(w)
    o = run_window(ga, q, k, v, "bf16", Wn)
    of = o.view(torch.int16).cpu().numpy()
    rng = np.random.default_rng(70)
    for b in range(w.B):
        for hq in range(0, w.Hq, 5):
            rows = sample_rows(w.Sq, rng)
            hk = oracle.kv_head_index(hq, w.Hq, w.Hkv)
            ref, _ = oracle.attention_rows(ref_f64(q[b:b + 1, hq:hq + 1], "bf16"), ref_f64(k[b:b + 1, hk:hk + 1], "bf16"),
                                           ref_f64(v[b:b + 1, hk:hk + 1], "bf16"), 0, 0, rows, w.scale_value,
                                           window=Wn)
            got = ref_f64(of[b, hq, rows].view(np.uint16), "bf16")
            assert_close(got, ref, "bf16", f"window {w.name} b{b} h{hq}")


@pytest.mark.slow
def test_full_size_window_paged_decode(ga):
    """The paged Hkv 8 decode workload with a 4096-token window, sampled heads."""
    w = W.cfg5(8)
    note(f"full-size window paged decode {w.name}")
    di = W.decode_inputs(w)
    o = run_decode(ga, di.q, di.k_cache, di.v_cache, di.seq_lens, di.block_table, di.max_seq_len, 4096)
    got = to_f64(o)
    heads = [(b, h) for b in range(w.B) for h in (0, 13, w.Hq - 1)]

    class Pages:
        def __init__(self, bits):
            self.bits, self.shape = bits, bits.shape

        def __getitem__(self, idx):
            return oracle.bf16_bits_to_f64(self.bits[idx])
    ref = oracle.decode_paged(ref_f64(di.q, "bf16"), Pages(di.k_cache), Pages(di.v_cache), di.block_table,
                              di.seq_lens, scale=w.scale_value, heads=heads, window=4096)
    idx = tuple(np.array(heads).T)
    assert_close(got[idx], ref[idx], "bf16", "window paged decode")
