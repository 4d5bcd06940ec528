"""Seeded synthetic inputs for the affine-quantized matmul.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no unpacking, no dequantization, no matmul).  It is the
one piece shared by the oracle side (tests) and the GPU side (tests, bench).

Recipe (the pages' workload is a Llama-3.2-1B 4-bit MLX checkpoint; no trained
weights exist here, so seeded synthetic values of the same shapes stand in):

* packed payload ``w``: uint32 ``[N, K*bits/32]`` drawn uniformly over all 2**32
  words.  Every ``bits``-wide field of a uniform word is an independent uniform
  code in ``[0, 2**bits)``, so this is the same distribution as drawing uniform
  codes and packing them, without any packing arithmetic here;
* ``scales``: U[0.005, 0.02] drawn in f64 and rounded to the storage type
  (f16: numpy's round-to-nearest-even from f64; bf16: f64 -> f32 -> bf16, both
  steps round-to-nearest-even, through PyTorch);
* ``biases``: ``-2**(bits-1) * scale + N(0, 1e-3)`` (standard deviation 1e-3),
  computed in f64 from the scale as drawn (before its rounding), then rounded
  the same way as the scales;
* ``x``: standard normal ``[M, K]`` rounded to f16.

Draw order within one problem: words, scales, bias noise, x.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

# Llama-3.2-1B linear shapes (N x K = out x in): hidden 2048, intermediate
# 8192, 16 layers, vocabulary 128256.
LLAMA_1B_PROJ = (
    ("q", 2048, 2048),
    ("k", 512, 2048),
    ("v", 512, 2048),
    ("o", 2048, 2048),
    ("gate", 8192, 2048),
    ("up", 8192, 2048),
    ("down", 2048, 8192),
)
LLAMA_1B_LM_HEAD = ("lm_head", 128256, 2048)
LLAMA_1B_LAYERS = 16


@dataclass
class Problem:
    """One synthetic quantized-linear problem; arrays are host numpy."""

    x: np.ndarray          # float16 [M, K], or bf16 bit patterns (uint16) when act_dtype is "bf16"
    w: np.ndarray          # uint32 [N, K*bits/32]
    scales: np.ndarray     # uint16 bit patterns [N, K/group_size]
    biases: np.ndarray     # uint16 bit patterns [N, K/group_size]
    M: int
    N: int
    K: int
    bits: int
    group_size: int
    sb_dtype: str          # "f16" or "bf16"
    act_dtype: str = "f16"  # activations: "f16" or "bf16"


def _round_sb(v64: np.ndarray, sb_dtype: str) -> np.ndarray:
    """Store f64 values as f16 or bf16 bit patterns (uint16)."""
    if sb_dtype == "f16":
        return v64.astype(np.float16).view(np.uint16)
    if sb_dtype == "bf16":
        t = torch.from_numpy(v64.astype(np.float32)).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(f"unknown scale/bias dtype {sb_dtype!r}")


def make_weights(N: int, K: int, bits: int = 4, group_size: int = 64,
                 sb_dtype: str = "f16", rng: np.random.Generator | None = None,
                 seed: int | None = None):
    """Draw a packed payload plus scales and biases; returns (w, scales, biases)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    if bits not in (4, 8):
        raise ValueError("bits must be 4 or 8")
    if K % group_size or K % (32 // bits):
        raise ValueError("K must be a multiple of group_size and of codes per word")
    kw = K * bits // 32
    G = K // group_size
    w = rng.integers(0, 2**32, size=(N, kw), dtype=np.uint32)
    s64 = rng.uniform(0.005, 0.02, size=(N, G))
    s_bits = _round_sb(s64, sb_dtype)
    b64 = -float(2 ** (bits - 1)) * s64 + rng.normal(0.0, 1e-3, size=(N, G))
    b_bits = _round_sb(b64, sb_dtype)
    return w, s_bits, b_bits


def make_x(M: int, K: int, rng: np.random.Generator | None = None,
           seed: int | None = None, act_dtype: str = "f16") -> np.ndarray:
    """Activations N(0, 1): float16 values, or bf16 bit patterns (uint16)."""
    if rng is None:
        rng = np.random.default_rng(seed)
    v = rng.standard_normal((M, K))
    return v.astype(np.float16) if act_dtype == "f16" else _round_sb(v, act_dtype)


def make_out_bias(N: int, seed: int, act_dtype: str = "f16") -> np.ndarray:
    """A linear layer's output bias [N] as uint16 bit patterns of the
    activation type: N(0, 0.5^2)."""
    rng = np.random.default_rng(seed)
    return _round_sb(0.5 * rng.standard_normal(N), act_dtype)


def make_problem(M: int, N: int, K: int, bits: int = 4, group_size: int = 64,
                 sb_dtype: str = "f16", seed: int = 0, act_dtype: str = "f16") -> Problem:
    rng = np.random.default_rng(seed)
    w, s, b = make_weights(N, K, bits, group_size, sb_dtype, rng=rng)
    x = make_x(M, K, rng=rng, act_dtype=act_dtype)
    return Problem(x=x, w=w, scales=s, biases=b, M=M, N=N, K=K, bits=bits,
                   group_size=group_size, sb_dtype=sb_dtype, act_dtype=act_dtype)


def proj_seed(config: int, layer: int, proj_idx: int) -> int:
    """Distinct, replayable seed per (workload config, layer, projection)."""
    return 1000 * config + 10 * layer + proj_idx


def small_qmv_problem() -> Problem:
    """Single 4-bit qmv: M=1, N=512, K=2048, group 64, f16 scales/biases, seed 0."""
    return make_problem(1, 512, 2048, bits=4, group_size=64, sb_dtype="f16", seed=0)


def edge_cases():
    """The 8-bit / tail sweep: M in {1,2,4,8}, K=8192, N in {2048,1023,2050},
    bits in {4,8}, scale/bias dtype in {f16,bf16}; yields keyword dicts."""
    case = 0
    for bits in (4, 8):
        for sb in ("f16", "bf16"):
            for N in (2048, 1023, 2050):
                for M in (1, 2, 4, 8):
                    yield dict(M=M, N=N, K=8192, bits=bits, group_size=64,
                               sb_dtype=sb, seed=proj_seed(2, 0, 0) + case)
                    case += 1
