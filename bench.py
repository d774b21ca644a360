"""Benchmark of the attention hot path on one MI355X; prints ONE JSON line.

A step is one pass of the whole path over one batch of synthetic inputs:
  1. prefill: causal GQA attention, B=2, Hq=32, Hkv=8, S=8192, d=128, bf16;
  2. prefill: causal MHA attention, B=4, H=32, S=2048, d=128, bf16;
  3. decode over a contiguous KV cache: B=64, Hq=32, Hkv=8, d=128, bf16,
     cached lengths uniform in [512, 4096];
  4. decode over a paged KV cache (16-token blocks, random physical placement,
     per-sequence block table): B=16, Hq=32, lengths in [8192, 32768], with
     Hkv = 8 (GQA), 32 (MHA) and 1 (MQA).
All inputs are resident in device memory before the timed region.  `value` is
the GQA prefill throughput in TFLOP/s (algorithmic FLOPs: 4*d*Hq*B per
unmasked query-key pair); the MHA prefill rate, the decode KV bandwidth
(every cached K/V byte read once) and tokens/s are reported beside it, each
with its roofline fraction.  Per-call times come from HIP events recorded on
the stream the kernels run on.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
       python bench.py --only prefill|mha|decode|paged|paged32|paged1 --steps 3 --warmup 1   (profiling runs)
"""
from __future__ import annotations

import argparse
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "prefill TFLOP/s + decode KV GB/s (GQA Hq=32 Hkv=8 d=128, bf16, 1 GPU)"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["prefill", "mha", "decode", "paged", "paged32", "paged1"], default=None)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload separately (one JSON line each) instead of the step")
    ap.add_argument("--sweep-kinds", default="prefill,long,decode,kv,fp8,window,bwd",
                    help="comma list of the sweep's parts: prefill, long (32K-context GQA prefill), decode, "
                         "kv (paged KV-cache writes), fp8 (decode over fp8 caches), window (sliding-window "
                         "prefill and decode), bwd (backward)")
    return ap.parse_args()


def kernel_traffic(name: str, source_files):
    """Per-launch HBM bytes measured by rocprofv3 counters, if still current.

    Reads profiles/<name>_pmc.txt (written from two --pmc runs, FETCH_SIZE then
    WRITE_SIZE, scaled by a plain copy's counters) and returns its bytes only
    if the recorded source digest matches the kernel sources today.
    """
    path = os.path.join(PROFILES, f"{name}_pmc.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"^source_sha256:\s*(\w+)", text, re.M)
    t = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)", text, re.M)
    if not m or not t:
        return None
    if source_digest(open(os.path.join(ROOT, f)).read() for f in source_files) != m.group(1):
        return None
    return float(t.group(1))


def source_digest(texts) -> str:
    """sha256 over the code of kernel sources, comments and blank lines removed
    (so that documentation edits do not retire measured counters)."""
    import hashlib
    h = hashlib.sha256()
    for text in texts:
        for line in text.splitlines():
            code = re.sub(r"\s*//.*$", "", line).rstrip()
            if code:
                h.update(code.encode() + b"\n")
    return h.hexdigest()


def cpu_baseline_prefill(w, q, k, v, budget_s=12.0):
    """The fp64 oracle on a bounded sample of the prefill workload (whole heads)."""
    import oracle
    threads = os.environ.get("OMP_NUM_THREADS")
    cores = int(threads) if threads else len(os.sched_getaffinity(0))
    done_flops = 0.0
    heads = 0
    t0 = time.perf_counter()
    hq = 0
    while hq < w.Hq:
        hk = oracle.kv_head_index(hq, w.Hq, w.Hkv)
        qh = oracle.bf16_bits_to_f64(q[0, hq])
        kh = oracle.bf16_bits_to_f64(k[0, hk])
        vh = oracle.bf16_bits_to_f64(v[0, hk])
        oracle.attention_head(qh, kh, vh, w.scale_value, w.causal)
        done_flops += w.flops() / (w.B * w.Hq)
        heads += 1
        hq += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": done_flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"{heads} whole query heads (b=0, heads 0..{heads - 1}) of the S=8192 causal GQA "
                      f"prefill, fp64 numpy, {dt:.1f} s"}


def sweep(args):
    """Every workload on its own: prefill (fp32 tiny, MHA S2048, GQA S8192, and the
    32K-context GQA point), contiguous decode, paged decode with Hkv in {32, 8, 1}, and
    the parts chosen by --sweep-kinds.  One JSON line per workload."""
    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()

    def gpu(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def timed(fn, reps):
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        torch.cuda.synchronize()
        for a, b in ev:
            a.record(stream)
            fn()
            b.record(stream)
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3

    kinds = set(args.sweep_kinds.split(","))
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    prefill_points = ((W.CFG1, W.CFG2, W.CFG3) if "prefill" in kinds else ()) + \
        ((W.LONG_CONTEXT,) if "long" in kinds else ())
    for w in prefill_points:
        log(f"sweep {w.name}")
        q, k, v = (gpu(x, w.dtype) for x in W.prefill_inputs(w))
        o = torch.empty_like(q)
        t = timed(lambda: gqa_attn.attn_prefill_fwd(q, k, v, o, scale=w.scale_value, causal=w.causal,
                                                    stream=stream), args.steps)
        tf = w.flops() / float(np.mean(t)) / 1e12
        print(json.dumps({"workload": w.name, "kind": "prefill", "dtype": w.dtype, "avg_us": round(float(np.mean(t)) * 1e6, 2),
                          "min_us": round(float(np.min(t)) * 1e6, 2), "TFLOPs": round(tf, 2),
                          "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4) if w.dtype == "bf16" else None}),
              flush=True)
        del q, k, v, o
    for w in (W.CFG4, W.cfg5(32), W.cfg5(8), W.cfg5(1)) if "decode" in kinds else ():
        log(f"sweep {w.name}")
        di = W.decode_inputs(w)
        q, kc, vc = gpu(di.q, "bf16"), gpu(di.k_cache, "bf16"), gpu(di.v_cache, "bf16")
        lens = gpu(di.seq_lens, "i32")
        bt = gpu(di.block_table, "i32") if w.paged else None
        o = torch.empty_like(q)
        ws = gqa_attn.decode_workspace(w.B, w.Hq, w.d, di.max_seq_len, dev)
        nbytes = W.decode_kv_bytes(di.seq_lens, w.Hkv, w.d)
        del di

        def call():
            flush.fill_(1)                      # evict the 256 MB Infinity Cache before every call
            gqa_attn.attn_decode_fwd(q, kc, vc, lens, o, block_table=bt, max_seq_len=None if not w.paged else
                                     w.max_blocks * W.BLOCK_SIZE, scale=w.scale_value, workspace=ws, stream=stream)
        ev = []
        for _ in range(args.warmup):
            call()
        torch.cuda.synchronize()
        for _ in range(args.steps):
            flush.fill_(1)
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            gqa_attn.attn_decode_fwd(q, kc, vc, lens, o, block_table=bt, max_seq_len=None if not w.paged else
                                     w.max_blocks * W.BLOCK_SIZE, scale=w.scale_value, workspace=ws, stream=stream)
            b.record(stream)
            ev.append((a, b))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        gbs = nbytes / float(np.mean(t)) / 1e9
        print(json.dumps({"workload": w.name, "kind": "decode", "kv_bytes": nbytes,
                          "avg_us": round(float(np.mean(t)) * 1e6, 2), "min_us": round(float(np.min(t)) * 1e6, 2),
                          "kv_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                          "tokens_per_s": round(w.B / float(np.mean(t)), 1)}), flush=True)
        del q, kc, vc, lens, bt, o, ws
        torch.cuda.empty_cache()
    if "kv" in kinds:
        sweep_kv(args, timed, dev, stream)
    if "fp8" in kinds:
        sweep_fp8(args, dev, stream, flush)
    if "window" in kinds:
        sweep_window(args, timed, dev, stream, flush)
    if "bwd" in kinds:
        sweep_bwd(args, timed, dev, stream)


def sweep_window(args, timed, dev, stream, flush, window=4096):
    """Sliding-window attention (each query sees its last `window` keys): the
    GQA S = 8192 prefill workload and the paged Hkv 8 decode workload.  Work
    counts only the keys inside the windows."""
    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W
    w = W.CFG3
    log(f"sweep window {window} {w.name}")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
               for x in W.prefill_inputs(w))
    o = torch.empty_like(q)
    t = timed(lambda: gqa_attn.attn_prefill_window_fwd(q, k, v, o, window=window, scale=w.scale_value,
                                                       stream=stream), args.steps)
    pairs = sum(min(i + 1, window) for i in range(w.Sq))
    flops = 4.0 * w.d * w.Hq * w.B * pairs
    tf = flops / float(np.mean(t)) / 1e12
    print(json.dumps({"workload": f"{w.name}_window{window}", "kind": "prefill_window", "dtype": "bf16",
                      "flops": flops, "avg_us": round(float(np.mean(t)) * 1e6, 2),
                      "min_us": round(float(np.min(t)) * 1e6, 2), "TFLOPs": round(tf, 2),
                      "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4)}), flush=True)
    del q, k, v, o
    torch.cuda.empty_cache()
    w = W.cfg5(8)
    log(f"sweep window {window} {w.name}")
    di = W.decode_inputs(w)
    g = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    q, kc, vc = g(di.q), g(di.k_cache), g(di.v_cache)
    lens = torch.from_numpy(di.seq_lens).to(dev)
    bt = torch.from_numpy(di.block_table).to(dev)
    o = torch.empty_like(q)
    ws = gqa_attn.decode_workspace(w.B, w.Hq, w.d, di.max_seq_len, dev)
    nbytes = int(np.minimum(di.seq_lens, window).sum()) * w.Hkv * w.d * 2 * 2
    msl = di.max_seq_len
    del di
    ev = []
    for it in range(args.warmup + args.steps):
        flush.fill_(1)                      # evict the 256 MB Infinity Cache before every call
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        gqa_attn.attn_decode_window_fwd(q, kc, vc, lens, o, window=window, block_table=bt, max_seq_len=msl,
                                        scale=w.scale_value, workspace=ws, stream=stream)
        b.record(stream)
        if it >= args.warmup:
            ev.append((a, b))
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
    gbs = nbytes / float(np.mean(t)) / 1e9
    print(json.dumps({"workload": f"{w.name}_window{window}", "kind": "decode_window", "kv_bytes": nbytes,
                      "avg_us": round(float(np.mean(t)) * 1e6, 2), "min_us": round(float(np.min(t)) * 1e6, 2),
                      "kv_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                      "tokens_per_s": round(w.B / float(np.mean(t)), 1)}), flush=True)
    del q, kc, vc, lens, bt, o, ws
    torch.cuda.empty_cache()


def sweep_bwd(args, timed, dev, stream):
    """Backward by recomputation on the two bf16 prefill workloads.  Work is
    the usual count of five products per visible (query, key) pair (S
    recomputed, dP, dV, dK, dQ: 2.5 x the forward); the kernels actually
    recompute S and dP once more for dQ (seven products), so the executed
    rate is 1.4 x the reported one."""
    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W
    for w in (W.CFG2, W.CFG3):
        log(f"sweep backward {w.name}")
        q, k, v = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
                   for x in W.prefill_inputs(w))
        do = torch.from_numpy(W.normal([w.seed, 9], (w.B, w.Hq, w.Sq, w.d), "bf16").view(np.int16)).view(
            torch.bfloat16).to(dev)
        o, lse = gqa_attn.attn_prefill_lse_fwd(q, k, v, scale=w.scale_value, causal=w.causal, stream=stream)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ws = torch.empty(gqa_attn.attn_prefill_bwd_workspace_bytes(w.B, w.Hq, w.Sq), dtype=torch.uint8, device=dev)
        tf_fwd = timed(lambda: gqa_attn.attn_prefill_lse_fwd(q, k, v, o, lse, scale=w.scale_value, causal=w.causal,
                                                             stream=stream), args.steps)
        t = timed(lambda: gqa_attn.attn_prefill_bwd(q, k, v, o, lse, do, dq, dk, dv, scale=w.scale_value,
                                                    causal=w.causal, workspace=ws, stream=stream), args.steps)
        flops = 2.5 * w.flops()
        tf = flops / float(np.mean(t)) / 1e12
        print(json.dumps({"workload": w.name, "kind": "backward", "dtype": "bf16", "flops": flops,
                          "avg_us": round(float(np.mean(t)) * 1e6, 2), "min_us": round(float(np.min(t)) * 1e6, 2),
                          "TFLOPs": round(tf, 2), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                          "lse_forward_avg_us": round(float(np.mean(tf_fwd)) * 1e6, 2)}), flush=True)
        del q, k, v, do, o, lse, dq, dk, dv, ws
        torch.cuda.empty_cache()


def sweep_fp8(args, dev, stream, flush):
    """Decode over fp8 caches (E4M3 codes + one fp32 scale per row) built from
    each decode workload's bf16 cache by the library's quantising append.
    Bytes = codes plus scales of every cached row, read once."""
    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W
    for w in (W.CFG4, W.cfg5(32), W.cfg5(8), W.cfg5(1)):
        log(f"sweep fp8 {w.name}")
        di = W.decode_inputs(w)

        def to_fp8(bits):
            # rows [..., Hkv, S, d] -> tokens [rows/Hkv.., Hkv, d] in slot order, quantised in place of the bf16
            t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)
            shape = t.shape
            if w.paged:                                  # [nb, Hkv, 16, d]: slot s = block * 16 + offset
                toks = t.permute(0, 2, 1, 3).contiguous().reshape(-1, shape[1], shape[3])
                hkv = shape[1]
            else:                                        # [B, Hkv, S, d]: one head per "block row" (Hkv = 1)
                toks = t.reshape(-1, 1, shape[3])
                hkv = 1
            n = toks.shape[0]
            codes = torch.empty((n // 16, hkv, 16, shape[3]), dtype=torch.uint8, device=dev)
            scales = torch.empty((n // 16, hkv, 16), dtype=torch.float32, device=dev)
            return toks, codes, scales, shape
        kt, kq, ksc, shape = to_fp8(di.k_cache)
        vt, vq, vsc, _ = to_fp8(di.v_cache)
        slots = torch.arange(kt.shape[0], dtype=torch.int32, device=dev)
        gqa_attn.attn_kv_append_fp8(kq, vq, ksc, vsc, kt, vt, slots, stream=stream)
        del kt, vt, slots
        kq, vq = kq.reshape(shape), vq.reshape(shape)
        ksc, vsc = ksc.reshape(shape[:3]), vsc.reshape(shape[:3])
        q = torch.from_numpy(np.ascontiguousarray(di.q).view(np.int16)).view(torch.bfloat16).to(dev)
        lens = torch.from_numpy(di.seq_lens).to(dev)
        bt = torch.from_numpy(di.block_table).to(dev) if w.paged else None
        o = torch.empty_like(q)
        ws = gqa_attn.decode_workspace(w.B, w.Hq, w.d, di.max_seq_len, dev)
        rows = int(di.seq_lens.sum()) * w.Hkv * 2
        nbytes = rows * (w.d + 4)
        msl = w.max_blocks * W.BLOCK_SIZE if w.paged else None
        del di
        ev = []
        for it in range(args.warmup + args.steps):
            flush.fill_(1)                      # evict the 256 MB Infinity Cache before every call
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            gqa_attn.attn_decode_fp8_fwd(q, kq, vq, ksc, vsc, lens, o, block_table=bt, max_seq_len=msl,
                                         scale=w.scale_value, workspace=ws, stream=stream)
            b.record(stream)
            if it >= args.warmup:
                ev.append((a, b))
        torch.cuda.synchronize()
        t = np.array([a.elapsed_time(b) for a, b in ev]) * 1e-3
        gbs = nbytes / float(np.mean(t)) / 1e9
        print(json.dumps({"workload": w.name + "_fp8", "kind": "decode_fp8", "kv_bytes": nbytes,
                          "avg_us": round(float(np.mean(t)) * 1e6, 2), "min_us": round(float(np.min(t)) * 1e6, 2),
                          "kv_GBps": round(gbs, 1), "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4),
                          "tokens_per_s": round(w.B / float(np.mean(t)), 1)}), flush=True)
        del q, kq, vq, ksc, vsc, lens, bt, o, ws
        torch.cuda.empty_cache()


def sweep_kv(args, timed, dev, stream):
    """Paged KV-cache writes: the paged Hkv 8 workload's tokens written in one
    call (a prefill's worth of K/V into the pages), one decode step's tokens
    for 64 sequences, and 64 copy-on-write block copies.  Bytes = every byte
    read once plus every byte written once."""
    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)

    def line(name, nbytes, t, tokens, extra=None):
        gbs = nbytes / float(np.mean(t)) / 1e9
        rec = {"workload": name, "kind": "kv_cache", "bytes": nbytes, "avg_us": round(float(np.mean(t)) * 1e6, 2),
               "min_us": round(float(np.min(t)) * 1e6, 2), "GBps": round(gbs, 1),
               "frac_of_hbm_peak": round(gbs / PEAK_HBM_GBS, 4), "tokens_per_s": round(tokens / float(np.mean(t)), 1)}
        rec.update(extra or {})
        print(json.dumps(rec), flush=True)

    # bulk: B16, L ~ U[8192, 32768], Hkv 8, d 128
    w = W.cfg5(8)
    log("sweep kv append (bulk)")
    lens = W.seq_lengths(w.seed, w.B, w.L_lo, w.L_hi)
    N = int(lens.sum())
    nb = int(sum(-(-int(L) // W.BLOCK_SIZE) for L in lens))
    pool = gqa_attn.KVPool(nb, w.B, w.max_blocks)
    seqs = [pool.seq_new() for _ in range(w.B)]
    slots, _, _ = pool.reserve(seqs, lens.tolist())
    kn = torch.randn((N, w.Hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((N, w.Hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    kc = torch.empty((nb, w.Hkv, W.BLOCK_SIZE, w.d), dtype=torch.bfloat16, device=dev)
    vc = torch.empty_like(kc)
    sl = torch.from_numpy(slots).to(dev)
    t = timed(lambda: gqa_attn.attn_kv_append(kc, vc, kn, vn, sl, stream=stream), args.steps)
    line("kv_append_bulk_B16_Hkv8_d128_L8192-32768", 4 * kn.numel() * 2, t, N)
    pool.close()
    del kc, vc, sl
    # practical ceiling for a read-plus-write stream: a plain device copy of the same bytes
    src = torch.cat([kn.flatten(), vn.flatten()])
    dst = torch.empty_like(src)
    del kn, vn
    t = timed(lambda: dst.copy_(src), args.steps)
    line("device_copy_same_bytes", 2 * src.numel() * 2, t, N)
    del src, dst
    torch.cuda.empty_cache()

    # decode step: 64 sequences of the contiguous decode workload's lengths, one token each
    w = W.CFG4
    log("sweep kv append (decode step) and copies")
    lens = W.seq_lengths(w.seed, w.B, w.L_lo, w.L_hi)
    nb = int(sum(-(-int(L) // W.BLOCK_SIZE) + 2 for L in lens)) + w.B
    pool = gqa_attn.KVPool(nb, 2 * w.B, w.max_blocks + 2)
    seqs = [pool.seq_new() for _ in range(w.B)]
    pool.reserve(seqs, lens.tolist())
    kids = [pool.seq_fork(s) for s in seqs]
    t0 = time.perf_counter()
    slots, src, dst = pool.reserve(seqs + kids, [1] * (2 * w.B))   # forks of partial blocks copy
    host_us = (time.perf_counter() - t0) * 1e6
    kc = torch.randn((nb, w.Hkv, W.BLOCK_SIZE, w.d), generator=gen, device=dev).to(torch.bfloat16)
    vc = torch.randn((nb, w.Hkv, W.BLOCK_SIZE, w.d), generator=gen, device=dev).to(torch.bfloat16)
    kn = torch.randn((2 * w.B, w.Hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    vn = torch.randn((2 * w.B, w.Hkv, w.d), generator=gen, device=dev).to(torch.bfloat16)
    sl = torch.from_numpy(slots).to(dev)
    t = timed(lambda: gqa_attn.attn_kv_append(kc, vc, kn, vn, sl, stream=stream), args.steps)
    line("kv_append_step_B128_Hkv8_d128", 4 * kn.numel() * 2, t, 2 * w.B,
         {"host_reserve_us": round(host_us, 1), "copies": int(len(src))})
    s_d, d_d = torch.from_numpy(src).to(dev), torch.from_numpy(dst).to(dev)
    t = timed(lambda: gqa_attn.attn_kv_copy_blocks(kc, vc, s_d, d_d, stream=stream), args.steps)
    line(f"kv_copy_blocks_{len(src)}_Hkv8_d128", 4 * len(src) * w.Hkv * W.BLOCK_SIZE * w.d * 2, t, 0)
    pool.close()


def calibration_copy(mib: int) -> int:
    """One device copy of known size: its FETCH_SIZE / WRITE_SIZE counters
    scale the same counters of the kernels into bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


# The step: every workload of the hot path once, in this order.  Each decode
# call follows at least 1.3 GB of other traffic (the 5.4 GB Hkv 32 call comes
# right before the 168 MB Hkv 1 one), which evicts the 256 MB Infinity Cache
# without a flush inside the step.
PHASES = ("prefill", "mha_prefill", "decode", "paged_decode", "paged_decode_hkv32", "paged_decode_hkv1")
ONLY = {"prefill": "prefill", "mha": "mha_prefill", "decode": "decode", "paged": "paged_decode",
        "paged32": "paged_decode_hkv32", "paged1": "paged_decode_hkv1"}
SRC_PREFILL = ["transformer_exact_attention_amd/csrc/prefill_bf16.hip",
               "transformer_exact_attention_amd/csrc/common.hpp"]
SRC_DECODE = ["transformer_exact_attention_amd/csrc/decode.hip",
              "transformer_exact_attention_amd/csrc/common.hpp",
              "transformer_exact_attention_amd/csrc/launch.hpp"]


def phase_workloads():
    from transformer_exact_attention_amd import workloads as W
    return {"prefill": W.CFG3, "mha_prefill": W.CFG2, "decode": W.CFG4, "paged_decode": W.cfg5(8),
            "paged_decode_hkv32": W.cfg5(32), "paged_decode_hkv1": W.cfg5(1)}


# counter profile (profiles/<name>_pmc.txt) of each phase
TRAFFIC_PROFILE = {"prefill": "prefill_bf16_gqa_causal_B2_Hq32_Hkv8_S8192",
                   "mha_prefill": "prefill_bf16_mha_causal_B4_H32_S2048",
                   "decode": "decode_gqa_contig_B64_Hq32_Hkv8",
                   "paged_decode": "decode_paged_B16_Hq32_Hkv8",
                   "paged_decode_hkv32": "decode_paged_B16_Hq32_Hkv32",
                   "paged_decode_hkv1": "decode_paged_B16_Hq32_Hkv1"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): "
              "the attention path runs on a single device.", file=sys.stderr)
        sys.exit(2)

    import torch
    from transformer_exact_attention_amd import gqa_attn
    from transformer_exact_attention_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    gqa_attn.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.sweep:
        sweep(args)
        if args.copy_calibration_mib:
            calibration_copy(args.copy_calibration_mib)
        return

    def gpu(a, kind):
        if kind == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    wl = phase_workloads()
    active = [p for p in PHASES if args.only is None or ONLY[args.only] == p]
    stream = torch.cuda.current_stream()
    calls = {}          # phase -> callable enqueueing one call on `stream`
    info = {}           # phase -> work figures
    t_gen = time.perf_counter()
    cpu_inputs = None
    for p in active:
        w = wl[p]
        log(f"generating {w.name}")
        if isinstance(w, W.PrefillWorkload):
            qn, kn, vn = W.prefill_inputs(w)
            q, k, v = gpu(qn, "bf16"), gpu(kn, "bf16"), gpu(vn, "bf16")
            o = torch.empty_like(q)
            if p == "prefill":
                cpu_inputs = (qn, kn, vn)
            del qn, kn, vn
            calls[p] = (lambda q=q, k=k, v=v, o=o, w=w:
                        gqa_attn.attn_prefill_fwd(q, k, v, o, scale=w.scale_value, causal=w.causal, stream=stream))
            info[p] = {"flops": w.flops(), "bytes": w.io_bytes()}
        else:
            di = W.decode_inputs(w)
            q, kc, vc = gpu(di.q, "bf16"), gpu(di.k_cache, "bf16"), gpu(di.v_cache, "bf16")
            lens = gpu(di.seq_lens, "i32")
            bt = gpu(di.block_table, "i32") if w.paged else None
            o = torch.empty_like(q)
            msl = di.max_seq_len
            ws = gqa_attn.decode_workspace(w.B, w.Hq, w.d, msl, dev)
            info[p] = {"bytes": W.decode_kv_bytes(di.seq_lens, w.Hkv, w.d), "B": w.B}
            del di
            calls[p] = (lambda q=q, kc=kc, vc=vc, lens=lens, o=o, bt=bt, msl=msl, ws=ws, w=w:
                        gqa_attn.attn_decode_fwd(q, kc, vc, lens, o, block_table=bt, max_seq_len=msl,
                                                 scale=w.scale_value, workspace=ws, stream=stream))
    torch.cuda.synchronize()
    log(f"inputs resident on the GPU ({time.perf_counter() - t_gen:.1f} s)")

    def step(ev=None):
        for i, p in enumerate(active):
            if ev:
                ev[i].record(stream)
            calls[p]()
        if ev:
            ev[len(active)].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup done ({args.warmup} steps)")

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(active) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    log(f"timed {args.steps} steps in {wall:.3f} s")

    res = {p: np.array([ev[i].elapsed_time(ev[i + 1]) for ev in events]) * 1e-3 for i, p in enumerate(active)}
    out = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(wall / args.steps * 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded iid N(0,1), bf16)"}

    def prefill_obj(p):
        w, t = wl[p], float(np.mean(res[p]))
        tf = info[p]["flops"] / t / 1e12
        return {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                "traffic": kernel_traffic(TRAFFIC_PROFILE[p], SRC_PREFILL),
                "kernel": "prefill_bf16_kernel<128, false>", "algorithmic_flops_per_launch": info[p]["flops"],
                "algorithmic_bytes_per_launch": info[p]["bytes"], "avg_launch_us": round(t * 1e6, 2),
                "min_launch_us": round(float(np.min(res[p])) * 1e6, 2)}

    def decode_obj(p):
        w, t = wl[p], float(np.mean(res[p]))
        gbs = info[p]["bytes"] / t / 1e9
        return {"workload": w.name, "kv_bytes": info[p]["bytes"], "avg_call_us": round(t * 1e6, 2),
                "min_call_us": round(float(np.min(res[p])) * 1e6, 2), "kv_GBps": round(gbs, 1),
                "tokens_per_s": round(w.B / t, 1),
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                             "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "traffic": kernel_traffic(TRAFFIC_PROFILE[p], SRC_DECODE),
                             "note": "one call = split + combine kernels; traffic counts both"}}

    if "prefill" in res:
        r = prefill_obj("prefill")
        out.update({"value": r["achieved"], "unit": "TFLOP/s"})
        out["roofline"] = r
    if "mha_prefill" in res:
        out["mha_prefill"] = {"workload": wl["mha_prefill"].name, "roofline": prefill_obj("mha_prefill")}
    for p in PHASES[2:]:
        if p in res:
            out[p] = decode_obj(p)
    if "value" not in out:
        p = active[0]
        r = prefill_obj(p) if p == "mha_prefill" else out[p]["roofline"]
        out.update({"value": r["achieved"], "unit": r["unit"]})
        out["roofline"] = r
    out["config"] = {
        "workload": ("step = causal GQA prefill B2 Hq32 Hkv8 S8192 d128 + causal MHA prefill B4 H32 S2048 d128 "
                     "+ contiguous GQA decode B64 Hq32 Hkv8 L~U[512,4096] + paged decode B16 Hq32 "
                     "L~U[8192,32768] at Hkv 8, 32 and 1 (GQA, MHA, MQA)") if args.only is None
        else f"only {ONLY[args.only]}",
        "prefill": {"B": 2, "Hq": 32, "Hkv": 8, "S": 8192, "d": 128, "causal": True},
        "mha_prefill": {"B": 4, "Hq": 32, "Hkv": 32, "S": 2048, "d": 128, "causal": True},
        "decode": {"B": 64, "Hq": 32, "Hkv": 8, "d": 128, "L": [512, 4096], "cache": "contiguous"},
        "paged_decode": {"B": 16, "Hq": 32, "Hkv": [8, 32, 1], "d": 128, "L": [8192, 32768], "block": 16}}

    if args.copy_calibration_mib:
        out["copy_calibration_bytes"] = calibration_copy(args.copy_calibration_mib)

    if not args.no_cpu_baseline and cpu_inputs is not None:
        log("timing the fp64 oracle on a sample (CPU baseline)")
        out["cpu_baseline"] = cpu_baseline_prefill(wl["prefill"], *cpu_inputs)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
