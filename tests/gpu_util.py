"""Helpers for the GPU parity tests: move synthetic problems to the device and
compare against the oracle with the stated tolerance."""

from __future__ import annotations

import sys

import numpy as np
import torch

TOL = 2e-3  # |y - y_ref| <= TOL * (1 + |y_ref|)


def note(msg: str):
    """Name the case before each GPU step (flushed, so a fault still shows it)."""
    print(msg, file=sys.stderr, flush=True)


def to_dev(p, device="cuda:0"):
    sbt = torch.float16 if p.sb_dtype == "f16" else torch.bfloat16
    x = torch.from_numpy(p.x).to(device)
    w = torch.from_numpy(p.w.view(np.int32)).to(device)
    s = torch.from_numpy(p.scales.view(np.int16)).view(sbt).to(device)
    b = torch.from_numpy(p.biases.view(np.int16)).view(sbt).to(device)
    return x, w, s, b


def y_host(y: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return y.cpu().numpy()


def tol_violations(y16: np.ndarray, ref: np.ndarray):
    y = y16.astype(np.float64)
    err = np.abs(y - ref)
    bound = TOL * (1 + np.abs(ref))
    bad = ~(err <= bound)
    return int(bad.sum()), float(np.max(err / bound)) if err.size else 0.0


def assert_close(y16: np.ndarray, ref: np.ndarray, what: str):
    assert y16.shape == ref.shape, (what, y16.shape, ref.shape)
    assert np.all(np.isfinite(y16.astype(np.float64))), f"{what}: non-finite output"
    nbad, worst = tol_violations(y16, ref)
    assert nbad == 0, f"{what}: {nbad} outputs outside tolerance (worst err/bound {worst:.3g})"
    return worst
