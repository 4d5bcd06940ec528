"""Plain, slow, obviously-correct CPU oracle for affine-quantized matmul.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): the product path never
imports this module, and this module imports nothing from the product path.

What the method computes (sources are the four pages of the reference):

* mlxcel epic #570 "realize low-precision / quantized performance on the
  OpenXLA (IREE) backend", section "Context": MLX 4/8-bit weights stay
  resident packed, a ``ui32`` payload plus f16 per-group scales and biases.
* mlxcel #574 "track(upstream-iree): fused dequant->matmul for the packed int8
  bandwidth win", section "What is already in-tree": the graph bit-unpacks the
  codes, then dequantizes each as ``q*scale + bias``; the result is bit-identical
  to a host dequant.  Same issue, "The blocker": a fused kernel must give the
  result of dequant followed by the matmul, without writing the f32 weight out.
* ExecuTorch PR #17187 "Metal backend: import qmv_impl from MLX",
  "Description": the operation is a linear layer with floating-point
  activations and 4-bit weights, including M = 1 with N not a multiple of 4;
  the PR's stack lists the same linear "with bias".

Readings where the pages are silent:

* Codes are packed LSB-first: code i of a word occupies bits [b*i, b*i + b).
* ``W`` is ``[N, K*b/32]`` uint32 (out-features x in-features), so
  ``y = x @ dequant(W).T``; scales and biases are ``[N, K/group_size]``.
* "Linear with bias" adds an output bias ``[N]`` (of the activation type) to
  every row of ``y``.
* Activations are f16, or bf16 (MLX's other activation format; the pages name
  only "floating-point activations"); either is widened exactly to f64.
* The native-int8 route (mlxcel #574 "Next actionable step" and "Upstream
  status refresh": a quantized dot lowered to the hardware's int8 path, dp4a /
  integer MMA, instead of scalar widening) needs int8 activations; the pages
  define no scheme, so the reading here is dynamic per-row (per-token)
  symmetric quantization: amax = max_k |x[m, k]| (f32), r = 127 / amax and
  sx = amax / 127 (f32 divisions), xq = clamp(rint(x * r), -127, 127) with the
  product and the rounding to nearest even in f32; a row with amax = 0 gives
  xq = 0, sx = 0.  The int8 path then computes exactly the dequant-matmul of
  x_hat = sx * xq.
* The fused output is compared against the f64 value before any rounding; the
  standalone dequant output is the f32 value ``RN_f32(q*s + b)``, and f16 or
  bf16 outputs are round-to-nearest-even of that f32 value (two steps).

Everything is numpy in float64; the only library primitive is numpy's matmul
(BLAS f64), whose summation order is irrelevant at the oracle's accuracy.
"""

from __future__ import annotations

import numpy as np
import torch

__all__ = [
    "unpack_codes",
    "widen_sb",
    "widen_act",
    "dequant_f64",
    "matmul_ref",
    "linear_ref",
    "quantize_act_i8",
    "matmul_ref_a8",
    "matmul_ref_rows",
    "dequant_ref_out",
    "f32_to_bf16_bits",
]


def unpack_codes(w_words: np.ndarray, K: int, bits: int) -> np.ndarray:
    """Bit-unpack a ``[N, K*bits/32]`` uint32 payload into ``[N, K]`` int64 codes.

    Follows mlxcel #574, "What is already in-tree" ("bit-unpack"), with the
    LSB-first reading: code ``k`` of row ``n`` is
    ``(W[n, k // P] >> (bits * (k % P))) & (2**bits - 1)`` with ``P = 32 // bits``.
    """
    if bits not in (4, 8):
        raise ValueError(f"bits must be 4 or 8, got {bits}")
    per_word = 32 // bits
    w = np.asarray(w_words, dtype=np.uint32)
    if w.ndim != 2 or w.shape[1] * per_word != K:
        raise ValueError(f"payload shape {w.shape} does not hold K={K} {bits}-bit codes")
    k = np.arange(K)
    word = w[:, k // per_word].astype(np.int64)
    shift = (bits * (k % per_word)).astype(np.int64)
    return (word >> shift) & ((1 << bits) - 1)


def widen_sb(sb_bits: np.ndarray, sb_dtype: str) -> np.ndarray:
    """Widen stored f16 / bf16 scale or bias bit patterns (uint16) to float64.

    epic #570 "Context" names f16 scales/biases for the packed path and bf16
    ones for dequant-at-load; #574 "Unblock criteria" asks for bf16 on the
    packed path too.  Both widen exactly: f16 through numpy's half type, bf16 by
    placing its 16 bits on top of an IEEE single (bf16 is the upper half of f32).
    """
    u = np.asarray(sb_bits, dtype=np.uint16)
    if sb_dtype == "f16":
        return u.view(np.float16).astype(np.float64)
    if sb_dtype == "bf16":
        return (u.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown scale/bias dtype {sb_dtype!r}")


def dequant_f64(w_words, scales, biases, K: int, bits: int, group_size: int,
                sb_dtype: str) -> np.ndarray:
    """Reconstruct the ``[N, K]`` weight in float64: ``w = q * scale + bias``.

    mlxcel #574 "What is already in-tree": bit-unpack, then ``q*scale + bias``
    with one (scale, bias) pair per group of ``group_size`` consecutive codes
    along K.  For f16 scale/bias the f64 result is exact (q*s has at most 19
    significant bits and the sum spans fewer than 53 bits).
    """
    if K % group_size != 0:
        raise ValueError("K must be a multiple of group_size")
    q = unpack_codes(w_words, K, bits).astype(np.float64)
    s = widen_sb(scales, sb_dtype)
    b = widen_sb(biases, sb_dtype)
    G = K // group_size
    if s.shape != (q.shape[0], G) or b.shape != (q.shape[0], G):
        raise ValueError(f"scales/biases must be [N, K/group_size] = {(q.shape[0], G)}")
    g_of_k = np.arange(K) // group_size
    return q * s[:, g_of_k] + b[:, g_of_k]


def widen_act(x, act_dtype: str = "f16") -> np.ndarray:
    """Widen activations exactly to float64: float16 values (``"f16"``), or
    bf16 bit patterns held as uint16 (``"bf16"``, decoded like a bf16 scale)."""
    if act_dtype == "f16":
        return np.asarray(x, dtype=np.float16).astype(np.float64)
    if act_dtype == "bf16":
        return widen_sb(np.asarray(x, dtype=np.uint16), "bf16")
    raise ValueError(f"unknown activation dtype {act_dtype!r}")


def matmul_ref(x, w_words, scales, biases, K: int, bits: int, group_size: int,
               sb_dtype: str, act_dtype: str = "f16") -> np.ndarray:
    """Float64 ``y = x @ dequant(W).T`` (before any output rounding).

    The fused kernel is defined (mlxcel #574 "The blocker"; epic #570 "The
    measured fusion gate") as giving the result of dequant followed by the
    matmul.  ``x`` is ``[M, K]`` activations (ExecuTorch #17187 "Description":
    floating-point activations), f16 or bf16, widened exactly to f64.
    """
    xf = widen_act(x, act_dtype)
    w = dequant_f64(w_words, scales, biases, K, bits, group_size, sb_dtype)
    return xf @ w.T


def matmul_ref_rows(x, w_words, scales, biases, rows, K: int, bits: int,
                    group_size: int, sb_dtype: str, act_dtype: str = "f16") -> np.ndarray:
    """``matmul_ref`` restricted to output columns ``rows`` (rows of W).

    Output column ``n`` depends only on row ``n`` of W, its scales and biases,
    so this equals ``matmul_ref(...)[:, rows]``; it lets tests check sampled
    outputs of full-size problems without dequantizing every row.
    """
    rows = np.asarray(rows, dtype=np.int64)
    return matmul_ref(x, np.asarray(w_words)[rows], np.asarray(scales)[rows],
                      np.asarray(biases)[rows], K, bits, group_size, sb_dtype, act_dtype)


def linear_ref(x, w_words, scales, biases, out_bias_bits, K: int, bits: int, group_size: int,
               sb_dtype: str, act_dtype: str = "f16") -> np.ndarray:
    """Float64 ``y = x @ dequant(W).T + out_bias`` (before any output rounding).

    The "linear with bias" entry of the ExecuTorch PR #17187 stack: the layer's
    output bias ``[N]`` (uint16 bit patterns of the activation type, or None for
    no bias) is added to every row of the linear layer's result.
    """
    y = matmul_ref(x, w_words, scales, biases, K, bits, group_size, sb_dtype, act_dtype)
    if out_bias_bits is None:
        return y
    ob_bits = np.asarray(out_bias_bits, dtype=np.uint16)
    ob = widen_act(ob_bits.view(np.float16), "f16") if act_dtype == "f16" else widen_act(ob_bits, act_dtype)
    return y + ob[None, :]


def quantize_act_i8(x):
    """Per-row symmetric int8 quantization of f16 activations ``[M, K]``.

    Returns ``(xq, sx)``: int8 codes ``[M, K]`` and the f32 row scales ``[M]``,
    following the steps of the reading in the module docstring, every step in
    float32 (the decisions that pick each integer are taken in f32, as in the
    kernel).
    """
    xf = np.asarray(x, dtype=np.float16).astype(np.float32)
    amax = np.max(np.abs(xf), axis=1) if xf.shape[1] else np.zeros(xf.shape[0], np.float32)
    amax = amax.astype(np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1), amax).astype(np.float32)
    r = (np.float32(127) / safe).astype(np.float32)
    sx = (safe / np.float32(127)).astype(np.float32)
    prod = (xf * r[:, None]).astype(np.float32)
    xq = np.clip(np.rint(prod), -127, 127)
    xq = np.where(zero[:, None], 0, xq).astype(np.int8)
    sx = np.where(zero, np.float32(0), sx).astype(np.float32)
    return xq, sx


def matmul_ref_a8(x, w_words, scales, biases, K: int, bits: int, group_size: int,
                  sb_dtype: str) -> np.ndarray:
    """Float64 result of the int8-activation path: ``(sx * xq) @ dequant(W).T``
    with ``(xq, sx) = quantize_act_i8(x)`` (before any output rounding)."""
    xq, sx = quantize_act_i8(x)
    xhat = xq.astype(np.float64) * sx.astype(np.float64)[:, None]
    w = dequant_f64(w_words, scales, biases, K, bits, group_size, sb_dtype)
    return xhat @ w.T


def f32_to_bf16_bits(v32: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); returns uint16 bits.

    Uses PyTorch's CPU float32 -> bfloat16 conversion as the library routine
    (round-to-nearest-even; NaN becomes the quiet NaN 0x7FC0).
    """
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def dequant_ref_out(w_words, scales, biases, K: int, bits: int, group_size: int,
                    sb_dtype: str, out_dtype: str) -> np.ndarray:
    """The standalone dequant output, which the GPU must match bit for bit.

    mlxcel #574 "What is already in-tree": the in-graph reconstruction is
    bit-identical to the host dequant, and the reconstructed weight the pages
    speak of is f32 (epic #570 "The measured fusion gate").  So:

    * ``"f32"``: ``RN_f32(q*s + b)``, returned as float32.  Rounding the exact
      f64 value once is the same as one f32 multiply-add, because ``q*s`` is
      exact in f32 and double rounding through f64 (53 >= 2*24 + 2 bits) of a
      single addition is innocuous.
    * ``"f16"``: float16 of that f32 value (round to nearest even), float16 array.
    * ``"bf16"``: bf16 of that f32 value (round to nearest even), uint16 bits.
    """
    w32 = dequant_f64(w_words, scales, biases, K, bits, group_size, sb_dtype).astype(np.float32)
    if out_dtype == "f32":
        return w32
    if out_dtype == "f16":
        return w32.astype(np.float16)
    if out_dtype == "bf16":
        return f32_to_bf16_bits(w32)
    raise ValueError(f"unknown output dtype {out_dtype!r}")
