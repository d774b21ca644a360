"""GPU: prefill and decode captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed.  The library's launches go to the caller's stream and record no
memset, so a captured call can be replayed with new input contents (new
queries, new cache lengths within max_seq_len); every replay, with the
program's own eager work and a synchronisation in between, must equal an
eager call on the same inputs bit for bit (same kernels, fixed plan and
reduction order), and the decode must match the fp64 oracle."""
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


def eager_work():
    import torch
    a = torch.randn(512, 512, device="cuda")
    (a @ a).sum().item()                          # some unrelated work and a synchronisation


def test_prefill_graph_replays_equal_eager_calls(ga):
    import torch
    B, Hq, Hkv, S, d = 1, 8, 2, 300, 128
    note("graph prefill")
    qs = [to_gpu(W.normal_bf16([9300, i], (B, Hq, S, d)), "bf16") for i in range(3)]
    k = to_gpu(W.normal_bf16([9301, 0], (B, Hkv, S, d)), "bf16")
    v = to_gpu(W.normal_bf16([9301, 1], (B, Hkv, S, d)), "bf16")
    q = qs[0].clone()
    o = torch.empty_like(q)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        ga.attn_prefill_fwd(q, k, v, o, causal=True)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ga.attn_prefill_fwd(q, k, v, o, causal=True)
    for i in range(3):
        q.copy_(qs[i])
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        eager_work()
        ref = ga.attn_prefill_fwd(qs[i], k, v, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(got, ref), f"replay {i} differs from the eager call"


@pytest.mark.parametrize("noalloc", [False, True])
def test_decode_graph_replays_follow_new_lengths(ga, noalloc):
    import torch
    B, Hq, Hkv, d, S_max = 6, 32, 8, 128, 2048
    note(f"graph decode noalloc={noalloc}")
    lens_list = [np.array([1, 700, 0, 2048, 333, 16], np.int32),
                 np.array([2048, 5, 1200, 0, 17, 999], np.int32),
                 np.array([64, 64, 64, 64, 64, 64], np.int32)]
    max_blocks = S_max // 16
    table, nb = W.block_placement(9400, np.full(B, S_max, np.int32), max_blocks)
    kp_np = W.normal_bf16([9401, 0], (nb, Hkv, 16, d))
    vp_np = W.normal_bf16([9401, 1], (nb, Hkv, 16, d))
    kp, vp, bt = to_gpu(kp_np, "bf16"), to_gpu(vp_np, "bf16"), to_gpu(table, "i32")
    q_np = [W.normal_bf16([9402, i], (B, Hq, d)) for i in range(3)]
    q = to_gpu(q_np[0], "bf16")
    lens = to_gpu(lens_list[0], "i32")
    o = torch.empty_like(q)
    ws = ga.decode_workspace(B, Hq, d, S_max)

    def call():
        if noalloc:
            ga.attn_decode_fwd_noalloc(q, kp, vp, lens, o, block_table=bt)
        else:
            ga.attn_decode_fwd(q, kp, vp, lens, o, block_table=bt, workspace=ws)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                       # warm-up (and the scratch address, first call)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(3):
        q.copy_(to_gpu(q_np[i], "bf16"))
        lens.copy_(to_gpu(lens_list[i], "i32"))
        g.replay()
        torch.cuda.synchronize()
        got = o.clone()
        eager_work()
        ref_gpu = ga.attn_decode_fwd(to_gpu(q_np[i], "bf16"), kp, vp, to_gpu(lens_list[i], "i32"), block_table=bt)
        torch.cuda.synchronize()
        assert torch.equal(got, ref_gpu), f"replay {i} differs from the eager call"
        ref = oracle.decode_paged(ref_f64(q_np[i], "bf16"), ref_f64(kp_np, "bf16"), ref_f64(vp_np, "bf16"), table,
                                  lens_list[i])
        assert_close(to_f64(got), ref, "bf16", f"graph decode replay {i}")
