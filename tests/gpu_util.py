"""Helpers shared by the GPU parity tests (not collected: no test_ prefix)."""

import sys

import numpy as np
import torch


def banner(msg: str):
    """Name the case on stdout before a GPU step (kept if the run dies)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.cpu().numpy()


def assert_normalised_close(got, want, norm, tol, what=""):
    """max |got - want| / norm <= tol; where norm == 0 the values must be equal."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    norm = np.asarray(norm, np.float64)
    err = np.abs(got - want)
    zero = norm == 0
    assert np.all(err[zero] == 0), f"{what}: non-zero error where the normaliser is 0"
    rel = np.where(zero, 0.0, err / np.where(zero, 1.0, norm))
    worst = float(rel.max()) if rel.size else 0.0
    print(f"[parity] {what}: max normalised error {worst:.3e} (tolerance {tol:.1e})", flush=True)
    assert worst <= tol, f"{what}: max normalised error {worst:.3e} > {tol:.1e}"
    return worst
