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


# bf16 activations: y is stored in bf16, whose unit roundoff is 2^-8, so the
# comparison adds that storage rounding to the computational tolerance above.
BF16_U = 2.0 ** -8


def to_dev_act(p, device="cuda:0"):
    """to_dev for a problem whose activations may be bf16 (x held as uint16 bits)."""
    x, w, s, b = to_dev(p, device) if p.act_dtype == "f16" else (None,) + to_dev_wsb(p, device)
    if p.act_dtype == "bf16":
        x = torch.from_numpy(p.x.view(np.int16)).view(torch.bfloat16).to(device)
    return x, w, s, b


def to_dev_wsb(p, device="cuda:0"):
    sbt = torch.float16 if p.sb_dtype == "f16" else torch.bfloat16
    w = torch.from_numpy(p.w.view(np.int32)).to(device)
    s = torch.from_numpy(p.scales.view(np.int16)).view(sbt).to(device)
    b = torch.from_numpy(p.biases.view(np.int16)).view(sbt).to(device)
    return w, s, b


def assert_close_act(y: torch.Tensor, ref: np.ndarray, what: str):
    """Tolerance check for f16 or bf16 y (bf16: plus its storage rounding)."""
    torch.cuda.synchronize()
    if y.dtype == torch.float16:
        return assert_close(y.cpu().numpy(), ref, what)
    yv = y.float().cpu().numpy().astype(np.float64)
    assert yv.shape == ref.shape, (what, yv.shape, ref.shape)
    assert np.all(np.isfinite(yv)), f"{what}: non-finite output"
    err = np.abs(yv - ref)
    bound = TOL * (1 + np.abs(ref)) + BF16_U * np.abs(ref)
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside tolerance (worst {float(np.max(err / bound)):.3g})"
    return float(np.max(err / bound)) if err.size else 0.0
