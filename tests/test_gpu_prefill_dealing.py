"""Prefill work-item orders: every (plane, query block) item lands in its place.

The bf16 prefill hands its work items to workgroups in one of three orders,
chosen from the plane count (plane = one K/V head of one batch entry) and the
query blocks per plane: per-XCD plane ranges, heaviest block first across a
group of planes (groups of four, or all the XCD's planes when their count is
not a multiple of four), or plain item order.  An item dealt twice or never
would leave a block of rows unwritten, so the output is filled with NaN
before each call and compared with the fp64 oracle on every element (small
shapes) or on rows sampled from every query block (long sequences).
"""
import numpy as np
import pytest

import oracle
from tests.gpu_helpers import assert_close, note, ref_f64, to_f64, to_gpu
from transformer_exact_attention_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16_NAN = 0x7FC0


@pytest.fixture(scope="module")
def ga():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    from transformer_exact_attention_amd import gqa_attn
    gqa_attn.load_library()
    return gqa_attn


def inputs(seed, B, Hq, Hkv, Sq, Sk, d):
    q = W.normal([seed, 0], (B, Hq, Sq, d), "f32")
    k = W.normal([seed, 1], (B, Hkv, Sk, d), "f32")
    v = W.normal([seed, 2], (B, Hkv, Sk, d), "f32")
    return tuple(W.f32_to_bf16_bits(x) for x in (q, k, v))


def run_nan_filled(ga, q, k, v, causal, window=None):
    import torch
    qt, kt, vt = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16")
    o = torch.full_like(qt, float("nan"))
    assert int(o.view(torch.int16)[0, 0, 0, 0]) == BF16_NAN
    ga.attn_prefill_fwd(qt, kt, vt, o, causal=causal, window=window)
    torch.cuda.synchronize()
    return o


# (B, Hq, Hkv, S): plane counts 8, 16, 24, 32, 40, 64 with few query blocks
# select the heaviest-first order (group of 1, 2, 3, 4, 5 planes; two groups
# of four); 9 and 20 items select plain item order, 16 items (4 planes x 4
# blocks) per-XCD ranges.
@pytest.mark.parametrize("B,Hq,Hkv,S", [
    (1, 8, 8, 300), (2, 8, 8, 300), (3, 8, 8, 300), (1, 32, 32, 300), (1, 40, 40, 300), (2, 32, 32, 300),
    (1, 32, 8, 600), (1, 3, 3, 600), (2, 4, 2, 520), (1, 4, 4, 1000),
])
@pytest.mark.parametrize("causal", [True, False])
def test_every_item_written_small(ga, B, Hq, Hkv, S, causal):
    d = 64
    q, k, v = inputs(7100 + B * 100 + Hkv, B, Hq, Hkv, S, S, d)
    note(f"prefill dealing B{B} Hq{Hq} Hkv{Hkv} S{S} causal={causal}")
    o = to_f64(run_nan_filled(ga, q, k, v, causal))
    ref = oracle.attention(ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), causal=causal)
    assert_close(o, ref, "bf16", f"dealing B{B} Hq{Hq} Hkv{Hkv} S{S}")


def test_every_item_written_windowed(ga):
    B, Hq, Hkv, S, W_ = 2, 16, 16, 700, 129
    q, k, v = inputs(7200, B, Hq, Hkv, S, S, 64)
    note(f"prefill dealing window {W_} B{B} H{Hq} S{S}")
    o = to_f64(run_nan_filled(ga, q, k, v, True, window=W_))
    ref = oracle.attention(ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), causal=True, window=W_)
    assert_close(o, ref, "bf16", f"dealing window {W_}")


@pytest.mark.slow
@pytest.mark.parametrize("B,Hq,Hkv,S", [(1, 8, 8, 8192), (1, 6, 3, 3900)])
def test_every_item_written_long(ga, B, Hq, Hkv, S):
    # Planes of 32 and 31 query blocks: per-XCD plane ranges (8 planes x 32
    # blocks) and plain order (3 planes x 31 blocks).
    import torch
    d = 128
    q, k, v = inputs(7300 + Hkv, B, Hq, Hkv, S, S, d)
    note(f"prefill dealing long B{B} Hq{Hq} Hkv{Hkv} S{S}")
    o = run_nan_filled(ga, q, k, v, True)
    assert bool(torch.isfinite(o).all()), "rows left unwritten"
    of = o.view(torch.int16).cpu().numpy()
    g = Hq // Hkv
    npos = 256 // g
    rng = np.random.default_rng(7300 + Hkv)
    for b in range(B):
        for hq in range(Hq):
            # one row at each end of every query block and one inside it
            starts = np.arange(0, S, npos)
            rows = np.unique(np.concatenate([starts, np.minimum(starts + npos - 1, S - 1),
                                             starts + rng.integers(0, npos, starts.size)]))
            rows = rows[rows < S]
            ref, _ = oracle.attention_rows(ref_f64(q[b:b + 1, hq:hq + 1], "bf16"),
                                           ref_f64(k[b:b + 1, hq // g:hq // g + 1], "bf16"),
                                           ref_f64(v[b:b + 1, hq // g:hq // g + 1], "bf16"), 0, 0, rows, None, True)
            got = ref_f64(of[b, hq, rows].view(np.uint16), "bf16")
            assert_close(got, ref, "bf16", f"long dealing b{b} h{hq}")
