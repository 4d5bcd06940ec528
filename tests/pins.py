"""Pins that tie the oracle to facts other than itself.

Each ``pin_*`` function takes an oracle namespace ``O`` (normally the real
``oracle`` package) and raises ``AssertionError`` on a mismatch.  They are run
against the real oracle by ``test_oracle_pins.py`` and against deliberately
broken copies of it by ``test_oracle_mutants.py``, which checks that every
planted mistake is caught by at least one pin.

Independent routes used here (none is the oracle's own vectorised formula):
* hand-derived words and values (``tests/golden/hand_dequant.txt``);
* unpacking through 32-character binary strings;
* exact rational arithmetic (``fractions.Fraction``) on tiny inputs;
* closed forms (all-ones x, one-hot x) and integer special cases checked with
  numpy's int64 matmul.
"""

from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers ---
def bitstring_unpack(word: int, bits: int) -> list[int]:
    """Codes of one uint32 word, LSB-first, read off its binary string."""
    s = format(int(word), "032b")          # s[0] is bit 31, s[31] is bit 0
    per = 32 // bits
    out = []
    for i in range(per):
        lo = bits * i                      # lowest bit of field i
        field = s[31 - (lo + bits - 1): 32 - lo]
        out.append(int(field, 2))
    return out


def f16_value(h: int) -> Fraction:
    """Exact value of an f16 bit pattern, decoded by hand from the IEEE fields."""
    sign = -1 if h & 0x8000 else 1
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    if e == 0x1F:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1024) * Fraction(2) ** (e - 15)


def bf16_value(h: int) -> Fraction:
    sign = -1 if h & 0x8000 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * Fraction(m, 128) * Fraction(2) ** (-126)
    return sign * Fraction(128 + m, 128) * Fraction(2) ** (e - 127)


def sb_value(h: int, sb_dtype: str) -> Fraction:
    return f16_value(h) if sb_dtype == "f16" else bf16_value(h)


def load_hand_dequant():
    rows = []
    with open(os.path.join(GOLDEN, "hand_dequant.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            dt, s, b, q, exact, f32b, f16b, bf16b = line.split()
            rows.append(dict(sb=dt, s=int(s, 16), b=int(b, 16), q=int(q),
                             exact=Fraction(exact), f32=int(f32b, 16),
                             f16=int(f16b, 16), bf16=int(bf16b, 16)))
    return rows


def _single_weight_payload(q: int, bits: int, K: int, slot: int) -> np.ndarray:
    """One row whose code at position ``slot`` is q and all others zero."""
    per = 32 // bits
    words = np.zeros((1, K // per), dtype=np.uint32)
    words[0, slot // per] = np.uint32(q * (2 ** (bits * (slot % per))))
    return words


# ------------------------------------------------------------------- pins ---
def pin_unpack_hand_words(O):
    """Hand-packed words, LSB-first (the layout reading for the "ui32 payload")."""
    w = np.array([[0x76543210]], dtype=np.uint32)
    assert list(O.unpack_codes(w, 8, 4)[0]) == [0, 1, 2, 3, 4, 5, 6, 7]
    w = np.array([[0x1000000F]], dtype=np.uint32)
    assert list(O.unpack_codes(w, 8, 4)[0]) == [15, 0, 0, 0, 0, 0, 0, 1]
    w = np.array([[0xAB030201]], dtype=np.uint32)
    assert list(O.unpack_codes(w, 4, 8)[0]) == [1, 2, 3, 0xAB]
    w = np.array([[0x89ABCDEF, 0x01234567]], dtype=np.uint32)
    assert list(O.unpack_codes(w, 16, 4)[0]) == [15, 14, 13, 12, 11, 10, 9, 8,
                                                  7, 6, 5, 4, 3, 2, 1, 0]


def pin_unpack_every_value_every_slot(O):
    """Brute force: each code value in each slot of a word, all other slots zero."""
    for bits in (4, 8):
        per = 32 // bits
        for slot in range(per):
            for v in range(2 ** bits):
                w = np.array([[v * 2 ** (bits * slot)]], dtype=np.uint32)
                got = O.unpack_codes(w, per, bits)[0]
                want = [0] * per
                want[slot] = v
                assert list(got) == want, (bits, slot, v, list(got))


def pin_unpack_bitstrings(O):
    """Random payloads unpacked through binary strings (independent route)."""
    rng = np.random.default_rng(12345)
    for bits in (4, 8):
        per = 32 // bits
        w = rng.integers(0, 2 ** 32, size=(3, 5), dtype=np.uint32)
        got = O.unpack_codes(w, 5 * per, bits)
        for n in range(3):
            want = []
            for j in range(5):
                want += bitstring_unpack(int(w[n, j]), bits)
            assert list(got[n]) == want


def pin_widen(O):
    """Scale/bias widening against hand decoding of the IEEE fields."""
    pats = [0x0000, 0x0001, 0x03FF, 0x0400, 0x211F, 0x3C00, 0x7BFF, 0x8001, 0xAD1F, 0xFBFF]
    got = O.widen_sb(np.array(pats, dtype=np.uint16), "f16")
    for h, g in zip(pats, got):
        assert Fraction(float(g)) == f16_value(h), (hex(h), g)
    pats = [0x0000, 0x0001, 0x007F, 0x0080, 0x3C24, 0x3F80, 0x7F7F, 0x8001, 0xBDA4, 0xFF7F]
    got = O.widen_sb(np.array(pats, dtype=np.uint16), "bf16")
    for h, g in zip(pats, got):
        assert Fraction(float(g)) == bf16_value(h), (hex(h), g)
    assert np.isinf(O.widen_sb(np.array([0x7C00], np.uint16), "f16")[0])
    assert np.isnan(O.widen_sb(np.array([0x7FC0], np.uint16), "bf16")[0])


def pin_dequant_hand_values(O):
    """Every hand-derived value in tests/golden/hand_dequant.txt, every output type."""
    for r in load_hand_dequant():
        bits = 8 if r["q"] > 15 else 4
        per = 32 // bits
        K = 64
        for slot in (0, per - 1, K - 1):
            w = _single_weight_payload(r["q"], bits, K, slot)
            s = np.array([[r["s"]]], dtype=np.uint16)
            b = np.array([[r["b"]]], dtype=np.uint16)
            wf = O.dequant_f64(w, s, b, K, bits, 64, r["sb"])
            assert Fraction(float(wf[0, slot])) == r["exact"], (r, slot)
            o32 = O.dequant_ref_out(w, s, b, K, bits, 64, r["sb"], "f32")
            assert int(o32[0, slot:slot + 1].view(np.uint32)[0]) == r["f32"], (r, slot)
            o16 = O.dequant_ref_out(w, s, b, K, bits, 64, r["sb"], "f16")
            assert int(o16[0, slot:slot + 1].view(np.uint16)[0]) == r["f16"], (r, slot)
            obf = O.dequant_ref_out(w, s, b, K, bits, 64, r["sb"], "bf16")
            assert int(obf[0, slot]) == r["bf16"], (r, slot)
            # every other position has code 0, i.e. value == bias
            other = (slot + 1) % K
            assert Fraction(float(wf[0, other])) == sb_value(r["b"], r["sb"])


def pin_group_indexing(O):
    """Scale/bias of group g applies exactly to codes [g*gs, (g+1)*gs)."""
    for gs in (32, 64, 128):
        K = 4 * gs
        G = K // gs
        for bits in (4, 8):
            per = 32 // bits
            # all codes 1: w[k] = s[g(k)] + b[g(k)], with distinct dyadic s, b per group
            w = np.full((2, K // per), sum(2 ** (bits * i) for i in range(per)), dtype=np.uint32)
            s_vals = [2.0 ** -(g + 1) for g in range(G)]
            b_vals = [float(g + 1) for g in range(G)]
            s = np.array([s_vals, s_vals[::-1]], dtype=np.float16).view(np.uint16)
            b = np.array([b_vals, b_vals[::-1]], dtype=np.float16).view(np.uint16)
            wf = O.dequant_f64(w, s, b, K, bits, gs, "f16")
            for n, (sv, bv) in enumerate(((s_vals, b_vals), (s_vals[::-1], b_vals[::-1]))):
                for k in range(K):
                    g = k // gs
                    assert wf[n, k] == sv[g] + bv[g], (gs, bits, n, k)


def _bruteforce_y(x, w, s, b, K, bits, gs, sb):
    """Exact y with Fractions: bit-string unpack, hand-decoded scales, loops."""
    M, N = x.shape[0], w.shape[0]
    per = 32 // bits
    y = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        codes = []
        for j in range(K // per):
            codes += bitstring_unpack(int(w[n, j]), bits)
        wv = [codes[k] * sb_value(int(s[n, k // gs]), sb) + sb_value(int(b[n, k // gs]), sb)
              for k in range(K)]
        for m in range(M):
            y[m][n] = sum((Fraction(float(x[m, k])) * wv[k] for k in range(K)), Fraction(0))
    return y


def pin_bruteforce_tiny(O):
    """Exact-rational brute force on tiny shapes equals the f64 oracle."""
    import synth
    shapes = [(1, 3, 64, 4, 64, "f16"), (2, 5, 128, 4, 64, "bf16"), (2, 2, 64, 8, 32, "f16"),
              (1, 4, 128, 8, 128, "bf16"), (2, 3, 96, 4, 32, "f16")]
    for i, (M, N, K, bits, gs, sb) in enumerate(shapes):
        p = synth.make_problem(M, N, K, bits, gs, sb, seed=777 + i)
        exact = _bruteforce_y(p.x, p.w, p.scales, p.biases, K, bits, gs, sb)
        got = O.matmul_ref(p.x, p.w, p.scales, p.biases, K, bits, gs, sb)
        for m in range(M):
            for n in range(N):
                e = float(exact[m][n])
                assert abs(got[m, n] - e) <= 1e-12 * (1 + abs(e)), (i, m, n, got[m, n], e)


def pin_one_hot(O):
    """x = e_k: y[:, n] is exactly the dequantized weight w[n, k]."""
    import synth
    for bits, sb in ((4, "f16"), (8, "bf16")):
        p = synth.make_problem(1, 6, 256, bits, 64, sb, seed=31 + bits)
        wf = O.dequant_f64(p.w, p.scales, p.biases, 256, bits, 64, sb)
        for k in (0, 1, 7, 63, 64, 200, 255):
            x = np.zeros((1, 256), dtype=np.float16)
            x[0, k] = 1.0
            y = O.matmul_ref(x, p.w, p.scales, p.biases, 256, bits, 64, sb)
            # and the value itself, by hand from the bit string and hand-decoded s, b
            per = 32 // bits
            for n in range(6):
                code = bitstring_unpack(int(p.w[n, k // per]), bits)[k % per]
                want = code * sb_value(int(p.scales[n, k // 64]), sb) + \
                    sb_value(int(p.biases[n, k // 64]), sb)
                assert Fraction(float(y[0, n])) == want, (bits, k, n)
                assert y[0, n] == wf[n, k]


def pin_integer_case(O):
    """scale = 1, bias = 0, x in {-1, 0, 1}: y is the integer product x @ codes^T."""
    rng = np.random.default_rng(99)
    for bits in (4, 8):
        per = 32 // bits
        K, N, M = 128, 7, 3
        w = rng.integers(0, 2 ** 32, size=(N, K // per), dtype=np.uint32)
        codes = np.array([[c for j in range(K // per) for c in bitstring_unpack(int(w[n, j]), bits)]
                          for n in range(N)], dtype=np.int64)
        xi = rng.integers(-1, 2, size=(M, K)).astype(np.int64)
        s = np.full((N, 2), 0x3C00, dtype=np.uint16)       # f16 1.0
        b = np.zeros((N, 2), dtype=np.uint16)
        y = O.matmul_ref(xi.astype(np.float16), w, s, b, K, bits, 64, "f16")
        assert np.array_equal(y, (xi @ codes.T).astype(np.float64))


def pin_all_ones_closed_form(O):
    """x = 1: y[n] = sum_g (s_g * sum_{k in g} q_k + gs * b_g), in exact rationals."""
    import synth
    for bits, gs, sb in ((4, 64, "f16"), (8, 32, "bf16"), (4, 128, "bf16")):
        K = 4 * gs
        p = synth.make_problem(1, 4, K, bits, gs, sb, seed=5 + gs)
        y = O.matmul_ref(np.ones((1, K), np.float16), p.w, p.scales, p.biases, K, bits, gs, sb)
        per = 32 // bits
        for n in range(4):
            codes = [c for j in range(K // per) for c in bitstring_unpack(int(p.w[n, j]), bits)]
            want = Fraction(0)
            for g in range(K // gs):
                qsum = sum(codes[g * gs:(g + 1) * gs])
                want += qsum * sb_value(int(p.scales[n, g]), sb) + gs * sb_value(int(p.biases[n, g]), sb)
            assert abs(y[0, n] - float(want)) <= 1e-12 * (1 + abs(float(want))), (bits, gs, n)


def pin_linearity(O):
    """y(2*x1 + x2) = 2*y(x1) + y(x2) for small-integer x (exact in f16 and f64)."""
    import synth
    p = synth.make_problem(2, 5, 128, 4, 64, "f16", seed=2024)
    rng = np.random.default_rng(7)
    x1 = rng.integers(-3, 4, size=(2, 128)).astype(np.float16)
    x2 = rng.integers(-3, 4, size=(2, 128)).astype(np.float16)
    f = lambda x: O.matmul_ref(x, p.w, p.scales, p.biases, 128, 4, 64, "f16")  # noqa: E731
    lhs = f((2 * x1 + x2).astype(np.float16))
    rhs = 2 * f(x1) + f(x2)
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-11)
    assert np.array_equal(f(np.zeros((2, 128), np.float16)), np.zeros((2, 5)))


def pin_rows_subset(O):
    """Sampled-row evaluation equals the full evaluation's columns."""
    import synth
    p = synth.make_problem(2, 9, 128, 8, 64, "bf16", seed=8)
    full = O.matmul_ref(p.x, p.w, p.scales, p.biases, 128, 8, 64, "bf16")
    rows = [8, 0, 3]
    sub = O.matmul_ref_rows(p.x, p.w, p.scales, p.biases, rows, 128, 8, 64, "bf16")
    assert np.array_equal(sub, full[:, rows])


def pin_bf16_rounding(O):
    """bf16 output rounding on hand-picked f32 patterns (ties to even, NaN, inf)."""
    pats = {0x3F808000: 0x3F80, 0x3F818000: 0x3F82, 0x3F808001: 0x3F81, 0x3F807FFF: 0x3F80,
            0x7F800000: 0x7F80, 0xFF800000: 0xFF80, 0x7F7FFFFF: 0x7F80, 0x00000001: 0x0000,
            0x80000000: 0x8000, 0x3DE00000: 0x3DE0}
    v = np.array(list(pats.keys()), dtype=np.uint32).view(np.float32)
    got = O.f32_to_bf16_bits(v)
    assert [int(g) for g in got] == list(pats.values()), [hex(int(g)) for g in got]
    nan = O.f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (int(nan) & 0x7F80) == 0x7F80 and (int(nan) & 0x7F) != 0


def pin_linear_bias_hand(O):
    """Linear with an output bias on a hand-derived case (M=2, N=3, K=32, 4-bit, g32).

    Row n of W holds the code n+1 everywhere (word (n+1) * 0x11111111), scale
    2^-4 (f16 0x2C00), bias 0; x row 0 is all ones, row 1 alternates +1 / -1;
    out_bias = (0.5, -1.25, 3.0).  Row 0: 32 * (n+1) / 16 + out_bias[n] =
    (2.5, 2.75, 9.0); row 1: the x sum is 0, so y is out_bias itself.  M != N,
    so a bias added along the wrong axis cannot broadcast.
    """
    w = np.array([[(n + 1) * 0x11111111] * 4 for n in range(3)], dtype=np.uint32)
    s = np.full((3, 1), 0x2C00, dtype=np.uint16)
    b = np.zeros((3, 1), dtype=np.uint16)
    x = np.zeros((2, 32), dtype=np.uint16)
    x[0, :] = 0x3C00
    x[1, 0::2], x[1, 1::2] = 0x3C00, 0xBC00
    ob = np.array([0x3800, 0xBD00, 0x4200], dtype=np.uint16)
    y = O.linear_ref(x.view(np.float16), w, s, b, ob, 32, 4, 32, "f16")
    assert np.array_equal(y, np.array([[2.5, 2.75, 9.0], [0.5, -1.25, 3.0]])), y
    y0 = O.linear_ref(x.view(np.float16), w, s, b, None, 32, 4, 32, "f16")
    assert np.array_equal(y0, np.array([[2.0, 4.0, 6.0], [0.0, 0.0, 0.0]])), y0


def pin_act_bf16_hand(O):
    """bf16 activations (and a bf16 output bias) on a hand-derived case
    (M=2, N=2, K=32, 4-bit, g32, f16 scale 1.0, bias 0).

    Row 0 of W holds code 1 everywhere (word 0x11111111), row 1 code 3
    (0x33333333).  x row 0: sixteen bf16 0x3F80 (1.0) then sixteen 0xC000
    (-2.0), sum -16; x row 1: all 0x3E80 (0.25), sum 8.  So y = x-sum times the
    code: [[-16, -48], [8, 24]].  With the bf16 output bias (0x4040 = 3.0,
    0xBF00 = -0.5): [[-13, -48.5], [11, 23.5]].  Read as f16, 0x3F80 is 1.875
    and 0x3E80 is 1.625, so a bf16 pattern decoded as f16 cannot pass.
    """
    w = np.array([[0x11111111] * 4, [0x33333333] * 4], dtype=np.uint32)
    s = np.full((2, 1), 0x3C00, dtype=np.uint16)
    b = np.zeros((2, 1), dtype=np.uint16)
    x = np.zeros((2, 32), dtype=np.uint16)
    x[0, :16], x[0, 16:] = 0x3F80, 0xC000
    x[1, :] = 0x3E80
    assert np.array_equal(O.widen_act(x[:, :1], "bf16"), np.array([[1.0], [0.25]]))
    y = O.matmul_ref(x, w, s, b, 32, 4, 32, "f16", "bf16")
    assert np.array_equal(y, np.array([[-16.0, -48.0], [8.0, 24.0]])), y
    ob = np.array([0x4040, 0xBF00], dtype=np.uint16)
    yb = O.linear_ref(x, w, s, b, ob, 32, 4, 32, "f16", "bf16")
    assert np.array_equal(yb, np.array([[-13.0, -48.5], [11.0, 23.5]])), yb


def pin_act_i8_hand(O):
    """int8 activations (per-row symmetric, the reading in the oracle) on a
    hand-derived case, K = 32 (x beyond column 7 is zero), 4-bit, g32, scale 1,
    bias 0; W row 0 holds code 1 everywhere, row 1 code 3.

    Row 0: x = (1, -2, 0.5, 4, -3.75, 2^-6, 0, 0), amax 4, r = 127/4 = 31.75
    (exact), products 31.75, -63.5, 15.875, 127, -119.0625, 0.49609375 ->
    rint (ties to even) 32, -64, 16, 127, -119, 0; sum -8.  Row 1 is all zero:
    xq = 0 and sx = 0.  Row 2: x = (-1/4, 1/4, 1/8, -1/8, 0, 0, 0, 1/16),
    amax 1/4, r = 508, products -127, 127, 63.5, -63.5, 0, 0, 0, 31.75 ->
    -127, 127, 64, -64, 0, 0, 0, 32; sum 32.  Row 3: amax 127/64, so r = 64 and
    sx = 2^-6 exactly; x = (127/64, 5/128, 1/128, -3/128) gives 127, 2.5, 0.5,
    -1.5 -> 127, 2, 0, -2 (ties to even; ties away from zero would give 3 and
    1); sum 127.  sx is the f32 quotient amax/127, and
    y[m, n] = sx[m] * code_n * sum(xq[m]).
    """
    x = np.zeros((4, 32), dtype=np.float16)
    x[0, :6] = [1, -2, 0.5, 4, -3.75, 2.0 ** -6]
    x[2, :8] = [-0.25, 0.25, 0.125, -0.125, 0, 0, 0, 0.0625]
    x[3, :4] = [127 / 64, 5 / 128, 1 / 128, -3 / 128]
    xq, sx = O.quantize_act_i8(x)
    want = np.zeros((4, 32), dtype=np.int8)
    want[0, :6] = [32, -64, 16, 127, -119, 0]
    want[2, :8] = [-127, 127, 64, -64, 0, 0, 0, 32]
    want[3, :4] = [127, 2, 0, -2]
    assert np.array_equal(xq, want), xq
    want_sx = np.array([np.float32(4) / np.float32(127), 0, np.float32(0.25) / np.float32(127), 2.0 ** -6],
                       dtype=np.float32)
    assert sx.dtype == np.float32 and np.array_equal(sx, want_sx), sx
    w = np.array([[0x11111111] * 4, [0x33333333] * 4], dtype=np.uint32)
    s = np.full((2, 1), 0x3C00, dtype=np.uint16)
    b = np.zeros((2, 1), dtype=np.uint16)
    y = O.matmul_ref_a8(x, w, s, b, 32, 4, 32, "f16")
    sxd = want_sx.astype(np.float64)
    want_y = np.array([[sxd[0] * -8, sxd[0] * -24], [0, 0], [sxd[2] * 32, sxd[2] * 96],
                       [sxd[3] * 127, sxd[3] * 381]])
    assert np.array_equal(y, want_y), y


ALL_PINS = [
    pin_unpack_hand_words, pin_unpack_every_value_every_slot, pin_unpack_bitstrings,
    pin_widen, pin_dequant_hand_values, pin_group_indexing, pin_bruteforce_tiny,
    pin_one_hot, pin_integer_case, pin_all_ones_closed_form, pin_linearity,
    pin_rows_subset, pin_bf16_rounding, pin_linear_bias_hand, pin_act_bf16_hand, pin_act_i8_hand,
]
