"""Shared helpers of the GPU parity tests (test infrastructure only)."""
from __future__ import annotations

import sys

import numpy as np

import oracle

BF16_TOL = 1.5e-2      # max |O_gpu - O_ref| for bf16 inputs (fp32 accumulation)
F32_TOL = 1e-4         # max |O_gpu - O_ref| for fp32 inputs
BF16_REL_FRO = 1e-2    # supplementary: ||O_gpu - O_ref||_F / ||O_ref||_F


def note(msg: str):
    """Name the case on stderr before a GPU step (survives a crash of the step)."""
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def to_gpu(arr: np.ndarray, dtype: str):
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16)
    elif dtype == "f32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32))
    elif dtype == "i32":
        t = torch.from_numpy(np.ascontiguousarray(arr, dtype=np.int32))
    else:
        raise ValueError(dtype)
    return t.cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu").to(torch.float64).numpy()


def ref_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    return oracle.to_f64(arr, dtype)


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", beyond_unit: bool = False):
    """max |got - ref| <= tol (and a relative Frobenius bound).

    ``beyond_unit``: for stress inputs whose outputs leave the O(1) range the
    tolerance is stated for, each element may also carry the rounding of the
    output to its storage type: |got - ref| <= tol + u * |ref| with u = 2^-8
    for bf16 (half a unit in the last place of an 8-bit significand is at
    most 2^-8 of the value) and u = 2^-24 for fp32.
    """
    tol = BF16_TOL if dtype == "bf16" else F32_TOL
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    rel = float(np.linalg.norm(err) / max(np.linalg.norm(ref), 1e-300))
    if beyond_unit:
        u = 2.0 ** -8 if dtype == "bf16" else 2.0 ** -24
        excess = err - u * np.abs(ref)
    else:
        excess = err
    worst = float(excess.max()) if excess.size else 0.0
    assert worst <= tol, f"{what}: max abs err {worst:.3e} > {tol:.1e} (rel fro {rel:.2e})"
    if dtype == "bf16":
        assert rel <= BF16_REL_FRO, f"{what}: relative Frobenius error {rel:.3e}"
    else:
        assert rel <= 1e-5, f"{what}: relative Frobenius error {rel:.3e}"
    return float(err.max()) if err.size else 0.0, rel
