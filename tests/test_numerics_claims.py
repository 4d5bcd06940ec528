"""CPU checks of the numerical facts the GPU path relies on.

* The product q*s of a code (< 256) and any finite f16 or bf16 scale is exact
  in f32, so "multiply then add" and a fused multiply-add give the same f32
  dequant bits: the kernel's choice of instruction cannot change the result.
* The fused outputs' tolerance |y - y_ref| <= 2e-3 * (1 + |y_ref|) leaves room
  for the f16 rounding of y itself (at most 2^-11 relative).
"""

import numpy as np

import synth


def _all_finite_positive(dtype: str) -> np.ndarray:
    if dtype == "f16":
        u = np.arange(1, 0x7C00, dtype=np.uint16)
        return u.view(np.float16).astype(np.float64)
    u = np.arange(1, 0x7F80, dtype=np.uint32)
    return (u << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def test_code_times_scale_exact_in_f32():
    q = np.arange(256, dtype=np.float64)
    for dt in ("f16", "bf16"):
        s = _all_finite_positive(dt)
        if dt == "bf16":
            s = s[s * 255 < np.finfo(np.float32).max]
        prod64 = q[None, :] * s[:, None]                 # exact in f64 (<= 16/19 bits)
        prod32 = (q[None, :].astype(np.float32) * s[:, None].astype(np.float32)).astype(np.float64)
        assert np.array_equal(prod64, prod32), dt


def test_mul_add_equals_single_rounding():
    rng = np.random.default_rng(3)
    s = _all_finite_positive("f16")
    for _ in range(3):
        b = rng.standard_normal(s.shape[0]).astype(np.float16).astype(np.float64)
        for q in (1, 7, 15, 200, 255):
            two_step = (np.float32(q) * s.astype(np.float32)) + b.astype(np.float32)
            single = (q * s + b).astype(np.float32)     # q*s + b exact in f64, one rounding
            assert np.array_equal(two_step, single)


def test_f16_output_rounding_within_tolerance():
    y = np.random.default_rng(4).standard_normal(100000) * 10
    y16 = y.astype(np.float16).astype(np.float64)
    assert np.all(np.abs(y16 - y) <= 0.25 * 2e-3 * (1 + np.abs(y)))


def test_synth_deterministic_and_distributed():
    a = synth.make_problem(2, 64, 2048, 4, 64, "f16", seed=11)
    b = synth.make_problem(2, 64, 2048, 4, 64, "f16", seed=11)
    c = synth.make_problem(2, 64, 2048, 4, 64, "f16", seed=12)
    for f in ("x", "w", "scales", "biases"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
        assert not np.array_equal(getattr(a, f), getattr(c, f))
    assert a.w.dtype == np.uint32 and a.w.shape == (64, 256)
    assert a.scales.shape == (64, 32) and a.scales.dtype == np.uint16
    s = a.scales.view(np.float16).astype(np.float64)
    assert s.min() >= 0.0049 and s.max() <= 0.0201
    nib = (a.w[..., None] >> (4 * np.arange(8, dtype=np.uint32))) & 0xF
    counts = np.bincount(nib.ravel(), minlength=16)
    assert counts.min() > 0.9 * counts.mean()
    bb = a.biases.view(np.float16).astype(np.float64)
    assert np.all(np.abs(bb + 8 * s) < 0.006)
    p8 = synth.make_problem(1, 8, 256, 8, 64, "bf16", seed=1)
    assert p8.w.shape == (8, 64) and p8.scales.shape == (8, 4)
    edge = list(synth.edge_cases())
    assert len(edge) == 48 and len({e["seed"] for e in edge}) == 48
