"""Shared helpers of the GPU parity tests: device copies of seeded inputs and
the tolerance check.  The expected values always come from ``oracle/``."""
from __future__ import annotations

import sys

import numpy as np

TOL = 1e-2  # max |gpu - oracle| <= TOL * (1 + |oracle|), per element (bf16 path)


def log(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("these tests need a GPU")
    return torch


def dev_bf16(bits: np.ndarray):
    torch = torch_cuda()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_i8(vals: np.ndarray):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(vals, dtype=np.int8)).cuda()


def dev_input(t):
    """A workloads.Tensor on the GPU."""
    return dev_bf16(t.bits) if t.dtype == "bf16" else dev_i8(t.bits)


def host(x) -> np.ndarray:
    torch = torch_cuda()
    torch.cuda.synchronize()
    if x.dtype == torch.bfloat16:
        return x.float().cpu().numpy().astype(np.float64)
    return x.cpu().numpy()


def assert_close(gpu: np.ndarray, ref: np.ndarray, tol: float = TOL, what: str = "") -> float:
    """Per-element band max |gpu - ref| <= tol * (1 + |ref|); returns the worst ratio."""
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    ratio = np.abs(gpu.astype(np.float64) - ref) / (tol * (1.0 + np.abs(ref)))
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: worst |err|/band = {worst:.3f} at {idx}: gpu={gpu[idx]} ref={ref[idx]}")
    return worst


def assert_close_scaled(gpu: np.ndarray, ref: np.ndarray, scale: np.ndarray, tol_scale: float,
                        tol: float = TOL, what: str = "") -> float:
    """Per-element band |gpu - ref| <= tol (1 + |ref|) + tol_scale |scale|: the
    usual band plus, for sums whose terms cancel, a part relative to the sum
    of the terms' magnitudes (`scale`), to which the rounding error of bf16
    operands is proportional."""
    assert gpu.shape == ref.shape == scale.shape, (what, gpu.shape, ref.shape, scale.shape)
    assert np.all(np.isfinite(gpu)), f"{what}: non-finite GPU values"
    band = tol * (1.0 + np.abs(ref)) + tol_scale * np.abs(scale)
    ratio = np.abs(gpu.astype(np.float64) - ref) / band
    worst = float(ratio.max()) if ratio.size else 0.0
    if worst > 1.0:
        idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        raise AssertionError(f"{what}: worst |err|/band = {worst:.3f} at {idx}: gpu={gpu[idx]} ref={ref[idx]} "
                             f"scale={scale[idx]}")
    return worst


def assert_exact(gpu: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    ref32 = ref.astype(np.int64)
    assert np.abs(ref32).max(initial=0) < 2 ** 31, f"{what}: oracle result outside int32"
    bad = np.argwhere(gpu.astype(np.int64) != ref32)
    if bad.size:
        i = tuple(bad[0])
        raise AssertionError(f"{what}: {len(bad)} mismatches, first at {i}: gpu={gpu[i]} ref={ref[i]}")
