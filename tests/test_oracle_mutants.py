"""Plant plausible mistakes in copies of the oracle; some pin must catch each.

The mistakes are planted on the CPU, in throw-away namespaces built from the
oracle's own functions; the real oracle is never modified.
"""

import types

import numpy as np
import pytest

import oracle
from oracle import qmv_oracle as Q
from tests import pins


def _namespace(**over):
    ns = types.SimpleNamespace(
        unpack_codes=Q.unpack_codes, widen_sb=Q.widen_sb, widen_act=Q.widen_act, dequant_f64=Q.dequant_f64,
        matmul_ref=Q.matmul_ref, matmul_ref_rows=Q.matmul_ref_rows, linear_ref=Q.linear_ref,
        dequant_ref_out=Q.dequant_ref_out, f32_to_bf16_bits=Q.f32_to_bf16_bits,
        quantize_act_i8=Q.quantize_act_i8)
    for k, v in over.items():
        setattr(ns, k, v)
    # re-bind the composite functions so they call the (possibly mutated) parts
    def dequant_f64(w, s, b, K, bits, gs, sb):
        if "dequant_f64" in over:
            return over["dequant_f64"](w, s, b, K, bits, gs, sb, ns)
        q = ns.unpack_codes(w, K, bits).astype(np.float64)
        sv, bv = ns.widen_sb(s, sb), ns.widen_sb(b, sb)
        g = np.arange(K) // gs
        return q * sv[:, g] + bv[:, g]

    def matmul_ref(x, w, s, b, K, bits, gs, sb, act="f16"):
        if "matmul_ref" in over:
            return over["matmul_ref"](x, w, s, b, K, bits, gs, sb, ns)
        return ns.widen_act(x, act) @ ns.dequant_f64(w, s, b, K, bits, gs, sb).T

    def matmul_ref_rows(x, w, s, b, rows, K, bits, gs, sb, act="f16"):
        rows = np.asarray(rows)
        return ns.matmul_ref(x, np.asarray(w)[rows], np.asarray(s)[rows], np.asarray(b)[rows],
                             K, bits, gs, sb, act)

    def linear_ref(x, w, s, b, ob, K, bits, gs, sb, act="f16"):
        y = ns.matmul_ref(x, w, s, b, K, bits, gs, sb, act)
        if "linear_bias" in over:
            return over["linear_bias"](y, ob)
        if ob is None:
            return y
        obits = np.asarray(ob, np.uint16)
        obv = ns.widen_act(obits.view(np.float16), "f16") if act == "f16" else ns.widen_act(obits, act)
        return y + obv[None, :]

    def dequant_ref_out(w, s, b, K, bits, gs, sb, out):
        w64 = ns.dequant_f64(w, s, b, K, bits, gs, sb)
        if "out_cast" in over:
            return over["out_cast"](w64, out, ns)
        w32 = w64.astype(np.float32)
        if out == "f32":
            return w32
        if out == "f16":
            return w32.astype(np.float16)
        return ns.f32_to_bf16_bits(w32)

    ns.dequant_f64, ns.matmul_ref = dequant_f64, matmul_ref
    ns.matmul_ref_rows, ns.dequant_ref_out = matmul_ref_rows, dequant_ref_out
    def matmul_ref_a8(x, w, s, b, K, bits, gs, sb):
        xq, sx = ns.quantize_act_i8(x)
        xhat = xq.astype(np.float64) * sx.astype(np.float64)[:, None]
        return xhat @ ns.dequant_f64(w, s, b, K, bits, gs, sb).T

    ns.linear_ref = linear_ref
    ns.matmul_ref_a8 = matmul_ref_a8
    return ns


def _msb_first(w, K, bits):
    per = 32 // bits
    k = np.arange(K)
    word = np.asarray(w, np.uint32)[:, k // per].astype(np.int64)
    return (word >> (bits * (per - 1 - k % per))) & ((1 << bits) - 1)


def _shift_off_by_one(w, K, bits):
    per = 32 // bits
    k = np.arange(K)
    word = np.asarray(w, np.uint32)[:, k // per].astype(np.int64)
    return (word >> (bits * (k % per) + 1)) & ((1 << bits) - 1)


def _mask_too_narrow(w, K, bits):
    return Q.unpack_codes(w, K, bits) & ((1 << (bits - 1)) - 1)


def _no_bias(w, s, b, K, bits, gs, sb, ns):
    q = ns.unpack_codes(w, K, bits).astype(np.float64)
    return q * ns.widen_sb(s, sb)[:, np.arange(K) // gs]


def _bias_sign(w, s, b, K, bits, gs, sb, ns):
    q = ns.unpack_codes(w, K, bits).astype(np.float64)
    g = np.arange(K) // gs
    return q * ns.widen_sb(s, sb)[:, g] - ns.widen_sb(b, sb)[:, g]


def _group_mod(w, s, b, K, bits, gs, sb, ns):
    q = ns.unpack_codes(w, K, bits).astype(np.float64)
    G = K // gs
    g = np.arange(K) % G
    return q * ns.widen_sb(s, sb)[:, g] + ns.widen_sb(b, sb)[:, g]


def _scale_bias_swapped(w, s, b, K, bits, gs, sb, ns):
    q = ns.unpack_codes(w, K, bits).astype(np.float64)
    g = np.arange(K) // gs
    return q * ns.widen_sb(b, sb)[:, g] + ns.widen_sb(s, sb)[:, g]


def _q_plus_one(w, s, b, K, bits, gs, sb, ns):
    q = ns.unpack_codes(w, K, bits).astype(np.float64) + 1
    g = np.arange(K) // gs
    return q * ns.widen_sb(s, sb)[:, g] + ns.widen_sb(b, sb)[:, g]


def _bf16_as_f16(u, sb):
    return Q.widen_sb(u, "f16")


def _bf16_truncating(v32):
    return (np.ascontiguousarray(v32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _x_reversed(x, w, s, b, K, bits, gs, sb, ns):
    xf = np.asarray(x, np.float16).astype(np.float64)[:, ::-1]
    return xf @ ns.dequant_f64(w, s, b, K, bits, gs, sb).T


def _rows_from_x(x, w, s, b, K, bits, gs, sb, ns):
    xf = np.asarray(x, np.float16).astype(np.float64)
    wf = ns.dequant_f64(w, s, b, K, bits, gs, sb)
    return (xf.sum(axis=1, keepdims=True) * np.ones((1, wf.shape[0]))) * 0 + xf @ wf.T * (1 + 1e-9)


def _f16_direct_from_f64(w64, out, ns):
    """f16 output rounded straight from the exact value (skipping the f32 step)."""
    if out == "f16":
        return w64.astype(np.float16)
    w32 = w64.astype(np.float32)
    return w32 if out == "f32" else ns.f32_to_bf16_bits(w32)


def _quant_i8(x, rounding=np.rint, qmax=127, per_row=True, zero_guard=True):
    xf = np.asarray(x, np.float16).astype(np.float32)
    amax = np.max(np.abs(xf), axis=1).astype(np.float32)
    if not per_row:
        amax = np.full_like(amax, np.max(amax))
    with np.errstate(divide="ignore", invalid="ignore"):
        safe = np.where(amax == 0, np.float32(1), amax).astype(np.float32) if zero_guard else amax
        r = (np.float32(qmax) / safe).astype(np.float32)
        sx = (safe / np.float32(qmax)).astype(np.float32)
        q = np.clip(rounding((xf * r[:, None]).astype(np.float32)), -127, 127)
    if zero_guard:
        q = np.where((amax == 0)[:, None], 0, q)
        sx = np.where(amax == 0, np.float32(0), sx).astype(np.float32)
    return np.nan_to_num(q, nan=-128).astype(np.int8), sx


def _ob(ob):
    return np.asarray(ob, np.uint16).view(np.float16).astype(np.float64)


MUTANTS = {
    "out_bias_dropped": dict(linear_bias=lambda y, ob: y),
    "out_bias_negated": dict(linear_bias=lambda y, ob: y if ob is None else y - _ob(ob)[None, :]),
    "out_bias_wrong_axis": dict(linear_bias=lambda y, ob: y if ob is None else y + _ob(ob)[:, None]),
    "out_bias_without_bias_arg": dict(linear_bias=lambda y, ob: y + 1.0 if ob is None else y + _ob(ob)[None, :]),
    "msb_first": dict(unpack_codes=_msb_first),
    "shift_off_by_one": dict(unpack_codes=_shift_off_by_one),
    "mask_too_narrow": dict(unpack_codes=_mask_too_narrow),
    "bias_dropped": dict(dequant_f64=_no_bias),
    "bias_sign": dict(dequant_f64=_bias_sign),
    "group_index_mod": dict(dequant_f64=_group_mod),
    "scale_bias_swapped": dict(dequant_f64=_scale_bias_swapped),
    "code_off_by_one": dict(dequant_f64=_q_plus_one),
    "bf16_read_as_f16": dict(widen_sb=lambda u, sb: _bf16_as_f16(u, sb) if sb == "bf16" else Q.widen_sb(u, sb)),
    "bf16_out_truncates": dict(f32_to_bf16_bits=_bf16_truncating),
    "x_k_reversed": dict(matmul_ref=_x_reversed),
    "tiny_relative_error": dict(matmul_ref=_rows_from_x),
    "f16_out_direct": dict(out_cast=_f16_direct_from_f64),
    "x_bf16_read_as_f16": dict(widen_act=lambda x, act: Q.widen_act(np.asarray(x, np.uint16).view(np.float16), "f16")
                               if act == "bf16" else Q.widen_act(x, act)),
    "out_bias_always_f16": dict(linear_bias=lambda y, ob: y if ob is None else y + _ob(ob)[None, :]),
    "i8_truncates": dict(quantize_act_i8=lambda x: _quant_i8(x, rounding=np.trunc)),
    "i8_ties_away": dict(quantize_act_i8=lambda x: _quant_i8(x, rounding=lambda v: np.sign(v) * np.floor(np.abs(v) + 0.5))),
    "i8_scale_128": dict(quantize_act_i8=lambda x: _quant_i8(x, qmax=128)),
    "i8_per_tensor": dict(quantize_act_i8=lambda x: _quant_i8(x, per_row=False)),
    "i8_zero_row_unguarded": dict(quantize_act_i8=lambda x: _quant_i8(x, zero_guard=False)),
}


def test_real_oracle_passes_all_pins():
    ns = _namespace()
    for pin in pins.ALL_PINS:
        pin(ns)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    ns = _namespace(**MUTANTS[name])
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(ns)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"planted mistake {name!r} passed every pin"
