"""GPU: the allocation-free decode entry point (attn_decode_fwd_noalloc) through
the C ABI.  Its partial results live in the library's static device scratch;
its output must equal attn_decode_fwd's (same kernels, same plan) bit for bit,
on consecutive calls whose sizes shrink and grow again (the scratch keeps the
previous call's contents), and match the fp64 oracle within the bf16 bar."""
import numpy as np
import pytest

import oracle
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


def case(seed, B, Hq, Hkv, lens, S_max, paged, d=128):
    lens = np.asarray(lens, np.int32)
    q = W.normal_bf16([seed, 0], (B, Hq, d))
    if paged:
        max_blocks = -(-S_max // 16)
        table, nb = W.block_placement(seed, lens, max_blocks, spare_blocks=2)
        k = W.normal_bf16([seed, 1], (nb, Hkv, 16, d))
        v = W.normal_bf16([seed, 2], (nb, Hkv, 16, d))
        return q, k, v, lens, table, max_blocks * 16
    k = W.normal_bf16([seed, 1], (B, Hkv, S_max, d))
    v = W.normal_bf16([seed, 2], (B, Hkv, S_max, d))
    return q, k, v, lens, None, S_max


def run_both(ga, seed, B, Hq, Hkv, lens, S_max, paged, d=128):
    import torch
    q, k, v, lens, table, msl = case(seed, B, Hq, Hkv, lens, S_max, paged, d)
    qg, kg, vg, lg = to_gpu(q, "bf16"), to_gpu(k, "bf16"), to_gpu(v, "bf16"), to_gpu(lens, "i32")
    tg = to_gpu(table, "i32") if paged else None
    o_ref = torch.full_like(qg, float("nan"))
    o_new = torch.full_like(qg, float("nan"))
    ws = ga.decode_workspace(B, Hq, d, msl, qg.device)
    note(f"noalloc decode B{B} Hq{Hq} Hkv{Hkv} S_max{S_max} d{d} paged={paged}")
    ga.attn_decode_fwd(qg, kg, vg, lg, o_ref, block_table=tg, max_seq_len=msl, workspace=ws)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    ga.attn_decode_fwd_noalloc(qg, kg, vg, lg, o_new, block_table=tg, max_seq_len=msl)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before          # nothing allocated through torch either
    assert torch.equal(o_new.view(torch.int16), o_ref.view(torch.int16)), "noalloc != attn_decode_fwd"
    if paged:
        ref = oracle.decode_paged(ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), table, lens)
    else:
        ref = oracle.decode_contiguous(ref_f64(q, "bf16"), ref_f64(k, "bf16"), ref_f64(v, "bf16"), lens)
    assert_close(to_f64(o_new), ref, "bf16", "noalloc decode")


def test_noalloc_decode_matches_the_workspace_call_on_consecutive_calls(ga):
    big = [4096, 3000, 1, 0, 2500, 4095, 17, 1024, 2048, 700, 33, 4000, 256, 257, 3999, 1500]
    run_both(ga, 70, 16, 32, 8, big, 4096, True)                      # paged GQA, ~1 MB of partials
    run_both(ga, 71, 4, 8, 2, [300, 5, 0, 129], 300, False)           # smaller, contiguous
    run_both(ga, 72, 16, 32, 1, big, 4096, True)                      # larger again, MQA
    run_both(ga, 73, 3, 4, 4, [1, 16, 2], 16, False)                  # smallest, MHA
    run_both(ga, 74, 5, 16, 2, [700, 0, 33, 256, 1], 768, True, d=64)  # head dim 64


def test_noalloc_decode_rejects_sizes_beyond_its_scratch(ga):
    import torch
    # 64 x 32 heads x 257 partials x 128 x 4 B > 64 MiB of scratch
    B, Hq, Hkv, S = 64, 32, 8, 65536
    assert ga.attn_decode_workspace_bytes(B, Hq, 128, S) > ga.DECODE_NOALLOC_MAX_BYTES
    q = torch.zeros((B, Hq, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((1, Hkv, 16, 128), dtype=torch.bfloat16, device="cuda")
    lens = torch.zeros((B,), dtype=torch.int32, device="cuda")
    table = torch.zeros((B, S // 16), dtype=torch.int32, device="cuda")
    o = torch.empty_like(q)
    with pytest.raises(ga.GqaAttnError, match="static scratch"):
        ga.attn_decode_fwd_noalloc(q, kc, kc, lens, o, block_table=table, max_seq_len=S)
