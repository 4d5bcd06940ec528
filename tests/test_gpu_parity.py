"""HIP path vs the CPU oracle, element by element, through libmxq's C ABI.

Bars: dequant bit-exact; fused outputs |y - y_ref| <= 2e-3 * (1 + |y_ref|)
against the f64 oracle value (before any rounding); integer and one-hot cases
bit-exact; repeated runs bit-identical.
"""

import numpy as np
import pytest
import torch

import dequant_matmul_qmv_amd as mxq
import oracle
import synth
from tests import pins
from tests.gpu_util import assert_close, assert_close_act, note, to_dev, to_dev_act, y_host

pytestmark = pytest.mark.gpu

OUT_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _dequant_bits(t: torch.Tensor, out: str) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu()
    if out == "f32":
        return a.numpy().view(np.uint32)
    return a.view(torch.int16).numpy().view(np.uint16)


def _oracle_bits(p, out):
    r = oracle.dequant_ref_out(p.w, p.scales, p.biases, p.K, p.bits, p.group_size, p.sb_dtype, out)
    if out == "f32":
        return r.view(np.uint32)
    if out == "f16":
        return r.view(np.uint16)
    return r


# ----------------------------------------------------------------- dequant ---
DQ_CASES = [
    (1, 32, 4, 32, "f16"), (3, 64, 4, 64, "bf16"), (5, 128, 8, 128, "f16"),
    (7, 96, 8, 32, "bf16"), (33, 256, 4, 64, "f16"), (512, 2048, 4, 64, "f16"),
    (1023, 8192, 8, 64, "bf16"), (130, 640, 4, 128, "bf16"),
]


@pytest.mark.parametrize("case", DQ_CASES, ids=str)
@pytest.mark.parametrize("out", ["f32", "f16", "bf16"])
def test_dequant_bitexact(case, out):
    N, K, bits, gs, sb = case
    p = synth.make_problem(1, N, K, bits, gs, sb, seed=N + K + bits)
    _, w, s, b = to_dev(p)
    note(f"dequant N={N} K={K} bits={bits} gs={gs} sb={sb} out={out}")
    got = _dequant_bits(mxq.mxq_dequant(w, s, b, bits=bits, group_size=gs, out_dtype=OUT_DT[out]), out)
    want = _oracle_bits(p, out)
    assert np.array_equal(got, want), f"{np.sum(got != want)} mismatching values"


def test_dequant_hand_values():
    for r in pins.load_hand_dequant():
        bits = 8 if r["q"] > 15 else 4
        per = 32 // bits
        K = 64
        codes = np.zeros((1, K), np.uint8)
        codes[0, 5] = r["q"]
        w = torch.from_numpy(mxq.mxq_pack(codes, bits).view(np.int32)).cuda()
        sbt = torch.float16 if r["sb"] == "f16" else torch.bfloat16
        s = torch.tensor([[r["s"]]], dtype=torch.int32).to(torch.int16).view(sbt).cuda()
        b = torch.tensor([[r["b"]]], dtype=torch.int32).to(torch.int16).view(sbt).cuda()
        note(f"dequant hand value {r}")
        o32 = _dequant_bits(mxq.mxq_dequant(w, s, b, bits=bits, group_size=64), "f32")
        o16 = _dequant_bits(mxq.mxq_dequant(w, s, b, bits=bits, group_size=64, out_dtype=torch.float16), "f16")
        obf = _dequant_bits(mxq.mxq_dequant(w, s, b, bits=bits, group_size=64, out_dtype=torch.bfloat16), "bf16")
        assert int(o32[0, 5]) == r["f32"] and int(o16[0, 5]) == r["f16"] and int(obf[0, 5]) == r["bf16"], r
        assert per > 0


# ------------------------------------------------------------------- fused ---
def _run(entry, p, **kw):
    x, w, s, b = to_dev(p)
    fn = mxq.mxq_qmv if entry == "qmv" else mxq.mxq_qmm
    return y_host(fn(x, w, s, b, bits=p.bits, group_size=p.group_size, **kw))


def _ref(p):
    return oracle.matmul_ref(p.x, p.w, p.scales, p.biases, p.K, p.bits, p.group_size, p.sb_dtype)


SMALL = [
    # M, N, K, bits, gs, sb
    (1, 1, 32, 4, 32, "f16"), (1, 3, 64, 4, 64, "f16"), (1, 5, 128, 8, 128, "bf16"),
    (2, 7, 96, 8, 32, "f16"), (3, 130, 2048, 4, 64, "bf16"), (4, 257, 2080, 4, 32, "f16"),
    (5, 66, 4096, 8, 64, "f16"), (6, 31, 1024, 4, 128, "bf16"), (7, 513, 2048, 8, 64, "bf16"),
    (8, 1000, 2048, 4, 64, "f16"), (9, 40, 512, 4, 64, "f16"), (17, 33, 256, 8, 32, "bf16"),
    (1, 2049, 2048, 4, 64, "f16"), (1, 64, 6144, 4, 64, "f16"),
]


@pytest.mark.parametrize("entry", ["qmv", "qmm"])
@pytest.mark.parametrize("case", SMALL, ids=str)
def test_fused_small(entry, case):
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M * 7 + N + K)
    note(f"{entry} {case}")
    assert_close(_run(entry, p), _ref(p), f"{entry} {case}")


def test_small_qmv_problem():
    """Single 4-bit qmv: M=1, N=512, K=2048, g64, f16 scales/biases, seed 0."""
    p = synth.small_qmv_problem()
    note("qmv small problem")
    assert_close(_run("qmv", p), _ref(p), "qmv small problem")


@pytest.mark.parametrize("case", [(1, 1000, 2048), (1, 2047, 2048), (1, 3000, 2048), (1, 4095, 2048),
                                  (1, 3000, 4096), (1, 4095, 4096), (1, 2048, 8192), (1, 3333, 8192),
                                  (1, 8192, 2048), (1, 12000, 2048), (1, 16383, 2048), (1, 6000, 8192),
                                  (2, 3000, 2048), (2, 12000, 4096), (1, 50000, 2048), (1, 40000, 4096)],
                         ids=str)
def test_decode_item_ring_tails(case):
    """The decode kernel's ring of item buffers (two items in flight at four
    rows per item, three below) ends with 0, 1 or 2 items left over whatever
    each wave's item count is.  N and K are chosen so that the waves of the
    small class (one row per item, x in registers, or in LDS with 2 or 4
    segment steps per row at K 4096 / 8192), of the mid class (two rows per
    item) and of the large class (four rows per item at K 2048, two at 4096)
    hold 1 to 8 items, every residue of both ring sizes; sampled outputs
    against the oracle."""
    M, N, K = case
    assert mxq.mxq_describe("qmv", M, N, K, 4, 64, "f16").startswith("qmv_kernel"), case
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=N + K + 31 * M)
    note(f"decode item ring {case}")
    y = _run("qmv", p)
    rows = _sampled_cols(N, N + K)
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, rows, K, 4, 64, "f16")
    assert_close(y[:, rows], ref, f"decode item ring {case}")


@pytest.mark.parametrize("entry", ["qmv", "qmm"])
@pytest.mark.parametrize("case", list(synth.edge_cases()), ids=lambda c: f"M{c['M']}N{c['N']}b{c['bits']}{c['sb_dtype']}")
def test_edge_cases_8bit_and_tails(entry, case):
    """M in {1,2,4,8}, K=8192, N in {2048,1023,2050}, 4/8-bit, f16/bf16 scales."""
    p = synth.make_problem(**case)
    note(f"{entry} edge {case}")
    assert_close(_run(entry, p), _ref(p), f"{entry} {case}")


QMM = [
    (64, 128, 64, 4, 64, "f16"), (64, 256, 2048, 8, 64, "bf16"), (100, 130, 512, 4, 32, "f16"),
    (128, 128, 1024, 4, 128, "bf16"), (200, 333, 2048, 4, 64, "f16"), (129, 64, 8192, 8, 64, "f16"),
    (256, 1000, 2048, 4, 64, "bf16"), (65, 1, 256, 4, 64, "f16"), (512, 96, 1024, 8, 128, "f16"),
]


# Shapes with enough 128 x 128 tiles to take the large-tile kernel (>= one per
# CU), with ragged M / N, an odd stage count and a partial bias block.
QMM_BIG = [
    (130, 32768, 256, 4, 64, "f16"), (256, 16400, 512, 8, 128, "bf16"), (200, 20000, 320, 4, 32, "f16"),
    (192, 24576, 1088, 8, 64, "f16"), (136, 33000, 192, 4, 64, "bf16"),
]


@pytest.mark.parametrize("case", QMM + QMM_BIG, ids=str)
def test_qmm_mfma(case):
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + K + 5)
    note(f"qmm mfma {case}")
    assert_close(_run("qmm", p), _ref(p), f"qmm {case}")


@pytest.mark.parametrize("case", [(128, 1024, 5760, 4, 128, "f16"), (128, 1024, 5760, 4, 64, "bf16"),
                                  (130, 1000, 5760, 8, 32, "f16")], ids=str)
def test_qmm_split_k_odd_stage_count_and_misaligned_scales(case):
    """K split into units of 9 stages (90 stages, 10 units): units start on odd
    stages, so the scale / bias block loads of groups of 64 and 128 cannot take
    aligned pairs of groups in every unit.  Scales and biases only 2-byte
    aligned give a bit-identical result."""
    M, N, K, bits, gs, sb = case
    assert ",ksplit=10>" in mxq.mxq_describe("qmm", M, N, K, bits, gs, sb)
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + gs)
    note(f"qmm split-K odd stages {case}")
    x, w, s, b = to_dev(p)
    y1 = y_host(mxq.mxq_qmm(x, w, s, b, bits=bits, group_size=gs))
    assert_close(y1, _ref(p), f"qmm split-K odd stages {case}")
    G = K // gs
    s_off = torch.empty(N * G + 1, dtype=s.dtype, device="cuda:0")
    b_off = torch.empty(N * G + 1, dtype=b.dtype, device="cuda:0")
    s_off[1:].copy_(s.reshape(-1))
    b_off[1:].copy_(b.reshape(-1))
    note(f"qmm split-K odd stages, misaligned scales {case}")
    y2 = y_host(mxq.mxq_qmm(x, w, s_off[1:].view(N, G), b_off[1:].view(N, G), bits=bits, group_size=gs))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16)), "2-byte scale loads change no bit"


def _scale_regime_problem(M, N, K, gs, sb, regime, seed):
    """4-bit problem whose scales sit in one magnitude regime, biases zero and
    x rescaled by a power of two so that y stays well inside f16.
    "big": |s| ~ U[1000, 4000], 2 % of (row, group) pairs in [4096, 30000];
    "tiny": |s| ~ U[1e-5, 1e-4] (f16 subnormals below 2^-14), 5 % log-uniform
    in [1e-8, 1e-5]; random signs."""
    p = synth.make_problem(M, N, K, 4, gs, sb, seed=seed)
    rng = np.random.default_rng(seed + 1)
    G = K // gs
    pick = rng.random((N, G)) < (0.02 if regime == "big" else 0.05)
    if regime == "big":
        s = rng.uniform(1000, 4000, (N, G))
        s[pick] = rng.uniform(4096, 30000, int(pick.sum()))
        xs = 2.0 ** -12
    else:
        s = rng.uniform(1e-5, 1e-4, (N, G))
        s[pick] = 10 ** rng.uniform(-8, -5, int(pick.sum()))
        xs = 2.0 ** 10
    s *= np.where(rng.random((N, G)) < 0.5, -1.0, 1.0)
    p.scales = synth._round_sb(s, sb)
    p.biases = synth._round_sb(np.zeros((N, G)), sb)
    p.x = (p.x.astype(np.float64) * xs).astype(np.float16)
    return p


@pytest.mark.parametrize("regime", ["big", "tiny"])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(96, 330, 1024, 64), (70, 200, 1024, 32), (100, 260, 1536, 128),
                                   (130, 32768, 512, 64)], ids=str)
def test_qmm_scale_regimes(shape, sb, regime):
    """Scales at both magnitude ends on the MFMA path (per-group f32 scale
    FMAs; the bias block's bf16 splits of a zero bias): products of large
    scales near the f16 range, f16 subnormal and zero scales, bf16 scales far
    below f16's range, random signs, on 64 x 64 and 128 x 128 tiles and group
    sizes 32, 64 and 128."""
    M, N, K, gs = shape
    p = _scale_regime_problem(M, N, K, gs, sb, regime, seed=M + N + gs)
    note(f"qmm scale regime {shape} {sb} {regime}")
    y = _run("qmm", p)
    assert np.all(np.isfinite(y))
    assert_close(y, _ref(p), f"qmm scale regime {shape} {sb} {regime}")


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
def test_qmm_subnormal_activations(bits, sb):
    """Every activation an f16 subnormal (random mantissa and sign) against
    scales of 1000-4000, so that y is O(10): on the MFMA path the 4-bit codes
    with f16 scales are themselves staged as f16 subnormals, and every product
    here has two subnormal operands.  The result must meet the same bound as
    any other input."""
    M, N, K, gs = 96, 384, 1024, 64
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=4242 + bits)
    rng = np.random.default_rng(4243 + bits)
    mant = rng.integers(1, 1024, (M, K)).astype(np.uint16)
    sign = (rng.random((M, K)) < 0.5).astype(np.uint16) << 15
    p.x = (mant | sign).view(np.float16)
    G = K // gs
    p.scales = synth._round_sb(rng.uniform(1000, 4000, (N, G)) * np.where(rng.random((N, G)) < 0.5, -1.0, 1.0), sb)
    p.biases = synth._round_sb(rng.uniform(-2e4, 2e4, (N, G)), sb)
    assert mxq.mxq_describe("qmm", M, N, K, bits, gs, sb).startswith("qmm_kernel")
    note(f"qmm subnormal activations bits={bits} sb={sb}")
    y = _run("qmm", p)
    ref = _ref(p)
    assert np.abs(ref).max() > 1.0  # the sums are not lost below f16's range
    assert_close(y, ref, f"qmm subnormal activations bits={bits} sb={sb}")


@pytest.mark.parametrize("proj", ["gate", "down"])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
def test_prefill_full_size_sampled(proj, sb):
    """M=512 prefill at gate/up (8192 x 2048) and down (2048 x 8192), sampled columns."""
    N, K = (8192, 2048) if proj == "gate" else (2048, 8192)
    p = synth.make_problem(512, N, K, 4, 64, sb, seed=synth.proj_seed(4, 0, 4 if proj == "gate" else 6))
    note(f"qmm full size {proj} {sb}")
    y = _run("qmm", p)
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(1).integers(0, N, 96)]))
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, rows, K, 4, 64, sb)
    assert_close(y[:, rows], ref, f"qmm {proj} {sb} sampled")


@pytest.mark.parametrize("name,N,K", [*synth.LLAMA_1B_PROJ, synth.LLAMA_1B_LM_HEAD])
def test_decode_projections_full_size(name, N, K):
    """Llama-3.2-1B-shaped M=1 decode projections at full size (sampled rows for lm_head)."""
    p = synth.make_problem(1, N, K, 4, 64, "f16", seed=synth.proj_seed(1, 0, 0) + N + K)
    note(f"qmv decode {name} {N}x{K}")
    y = _run("qmv", p)
    if N > 20000:
        rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(2).integers(0, N, 2048)]))
        ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, rows, K, 4, 64, "f16")
        assert_close(y[:, rows], ref, f"qmv {name} sampled")
    else:
        assert_close(y, _ref(p), f"qmv {name}")


# ------------------------------------------------------- exact special cases ---
@pytest.mark.parametrize("entry,M", [("qmv", 1), ("qmv", 8), ("qmm", 64), ("qmm", 128)])
@pytest.mark.parametrize("bits,sb", [(4, "f16"), (8, "bf16"), (4, "bf16")])
def test_one_hot_bitexact(entry, M, bits, sb):
    """x rows one-hot at k_m: y[m, n] = f16(f32(w[n, k_m])) exactly."""
    K, N = 512, 70
    p = synth.make_problem(M, N, K, bits, 64, sb, seed=400 + M + bits)
    ks = np.random.default_rng(M).integers(0, K, M)
    x = np.zeros((M, K), np.float16)
    x[np.arange(M), ks] = 1.0
    p.x = x
    note(f"one-hot {entry} M={M} bits={bits}")
    y = _run(entry, p)
    w32 = oracle.dequant_ref_out(p.w, p.scales, p.biases, K, bits, 64, sb, "f32")
    want = w32[:, ks].T.astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("entry,M", [("qmv", 3), ("qmm", 96)])
@pytest.mark.parametrize("bits", [4, 8])
def test_integer_case_bitexact(entry, M, bits):
    """scale 1, bias 0, x in {-1,0,1}: y is an integer; its f16 rounding must match."""
    K, N = 128, 50
    rng = np.random.default_rng(bits + M)
    p = synth.make_problem(M, N, K, bits, 64, "f16", seed=9)
    p.scales = np.full_like(p.scales, 0x3C00)
    p.biases = np.zeros_like(p.biases)
    p.x = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    note(f"integer {entry} M={M} bits={bits}")
    y = _run(entry, p)
    want = _ref(p).astype(np.float16)
    assert np.array_equal(y.view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("entry,M", [("qmv", 1), ("qmv", 5), ("qmm", 200)])
def test_deterministic(entry, M):
    p = synth.make_problem(M, 3000, 2048, 4, 64, "bf16", seed=77)
    x, w, s, b = to_dev(p)
    fn = mxq.mxq_qmv if entry == "qmv" else mxq.mxq_qmm
    note(f"determinism {entry} M={M}")
    y1 = y_host(fn(x, w, s, b, bits=4))
    y2 = y_host(fn(x, w, s, b, bits=4))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))


def test_empty_and_k_zero():
    dev = "cuda:0"
    x = torch.zeros((0, 64), dtype=torch.float16, device=dev)
    w = torch.zeros((5, 8), dtype=torch.int32, device=dev)
    s = torch.zeros((5, 1), dtype=torch.float16, device=dev)
    note("empty M")
    assert mxq.mxq_qmv(x, w, s, s).shape == (0, 5)
    x = torch.ones((3, 0), dtype=torch.float16, device=dev)
    w = torch.zeros((4, 0), dtype=torch.int32, device=dev)
    s = torch.zeros((4, 0), dtype=torch.float16, device=dev)
    y = torch.full((3, 4), 7.0, dtype=torch.float16, device=dev)
    note("K = 0")
    for fn in (mxq.mxq_qmv, mxq.mxq_qmm):
        y.fill_(7.0)
        fn(x, w, s, s, y)
        torch.cuda.synchronize()
        assert torch.equal(y.cpu(), torch.zeros((3, 4), dtype=torch.float16))


@pytest.mark.parametrize("M", [1, 3])
def test_nonzero_stream_and_offsets(M):
    """Work enqueued on a side stream; x passed as an unaligned slice (scalar loads)."""
    p = synth.make_problem(M, 300, 1024, 4, 64, "f16", seed=5)
    x, w, s, b = to_dev(p)
    xbig = torch.zeros((M * 1024 + 1,), dtype=torch.float16, device="cuda:0")
    xbig[1:].copy_(x.reshape(-1))
    xu = xbig[1:].view(M, 1024)
    st = torch.cuda.Stream()
    note("side stream + unaligned x")
    with torch.cuda.stream(st):
        y = mxq.mxq_qmv(xu, w, s, b, bits=4, stream=st)
    st.synchronize()
    assert_close(y.cpu().numpy(), _ref(p), "side stream")


def test_misaligned_w_rejected_on_device():
    p = synth.make_problem(1, 4, 64, 4, 64, "f16", seed=1)
    x, w, s, b = to_dev(p)
    wbig = torch.zeros((4 * 8 + 1,), dtype=torch.int32, device="cuda:0")
    wv = wbig[1:].view(4, 8)
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_qmv(x, wv, s, b, bits=4)
    assert e.value.status == mxq.MXQ_ERR_MISALIGNED


@pytest.mark.parametrize("M", [1, 3, 12])
def test_grouped_qmv(M):
    """Grouped launches: mixed N and K (one launch stages x in LDS for K=8192),
    more problems than one launch holds, and empty / K=0 problems."""
    specs = [(2048, 2048), (512, 2048), (1023, 2048), (8192, 2048), (2050, 8192), (7, 64)] * 3 + [(5, 128), (3, 256)]
    probs, dev_probs = [], []
    for i, (N, K) in enumerate(specs):
        p = synth.make_problem(M, N, K, 4, 64, "bf16" if M == 3 else "f16", seed=900 + 17 * i + M)
        probs.append(p)
        dev_probs.append(to_dev(p))
    note(f"grouped qmv M={M} count={len(specs)}")
    ys = mxq.mxq_qmv_grouped(dev_probs, bits=4)
    torch.cuda.synchronize()
    assert len(ys) == len(specs)
    for i, (p, y) in enumerate(zip(probs, ys)):
        assert_close(y.cpu().numpy(), _ref(p), f"grouped[{i}] N={p.N} K={p.K}")


def test_grouped_qmv_empty_and_k_zero():
    dev = "cuda:0"
    p = synth.make_problem(2, 300, 1024, 8, 64, "f16", seed=3)
    x, w, s, b = to_dev(p)
    x0 = torch.zeros((2, 0), dtype=torch.float16, device=dev)
    w0 = torch.zeros((4, 0), dtype=torch.int32, device=dev)
    s0 = torch.zeros((4, 0), dtype=torch.float16, device=dev)
    y0 = torch.full((2, 4), 3.0, dtype=torch.float16, device=dev)
    note("grouped with a K=0 problem")
    ys = mxq.mxq_qmv_grouped([(x, w, s, b), (x0, w0, s0, s0, y0)], bits=8)
    torch.cuda.synchronize()
    assert_close(ys[0].cpu().numpy(), _ref(p), "grouped K>0")
    assert torch.equal(y0.cpu(), torch.zeros((2, 4), dtype=torch.float16))


# ------------------------------------------------------ linear with bias ---
LINEAR = [
    (1, 1000, 2048, 4, 64, "f16"), (3, 130, 2048, 8, 32, "bf16"), (8, 2049, 4096, 4, 128, "f16"),
    (5, 1, 64, 4, 64, "f16"), (64, 256, 1024, 8, 64, "bf16"), (200, 333, 2048, 4, 64, "f16"),
    (130, 32768, 256, 4, 64, "f16"), (96, 100, 640, 4, 32, "bf16"),
]


def _bias_dev(ob):
    return torch.from_numpy(ob.view(np.int16)).view(torch.float16).cuda()


@pytest.mark.parametrize("case", LINEAR, ids=str)
def test_linear_bias(case):
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + 3 * N + K)
    ob = synth.make_out_bias(N, seed=N + 17)
    note(f"linear {case}")
    x, w, s, b = to_dev(p)
    y = y_host(mxq.mxq_linear(x, w, s, b, _bias_dev(ob), bits=bits, group_size=gs))
    ref = oracle.linear_ref(p.x, p.w, p.scales, p.biases, ob, K, bits, gs, sb)
    assert_close(y, ref, f"linear {case}")
    # without a bias the call is mxq_qmm, bit for bit
    y0 = mxq.mxq_linear(x, w, s, b, None, bits=bits, group_size=gs)
    yq = mxq.mxq_qmm(x, w, s, b, bits=bits, group_size=gs)
    assert torch.equal(y0.view(torch.int16), yq.view(torch.int16)), case


@pytest.mark.parametrize("M", [1, 7, 64, 300])
def test_linear_bias_exact_with_zero_weights(M):
    """Scales and biases 0: the weights contribute exact zeros, so y = out_bias bit for bit."""
    N, K = 1027, 512
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=M)
    ob = synth.make_out_bias(N, seed=5)
    note(f"linear zero weights M={M}")
    x, w, s, b = to_dev(p)
    s.zero_()
    b.zero_()
    y = mxq.mxq_linear(x, w, s, b, _bias_dev(ob), bits=4, group_size=64)
    want = torch.from_numpy(np.broadcast_to(ob.view(np.int16), (M, N)).copy()).cuda()
    assert torch.equal(y.view(torch.int16), want), M


def test_linear_k0_is_bias():
    M, N = 9, 77
    ob = synth.make_out_bias(N, seed=3)
    note("linear K=0")
    x = torch.empty((M, 0), dtype=torch.float16, device="cuda")
    w = torch.empty((N, 0), dtype=torch.int32, device="cuda")
    s = torch.empty((N, 0), dtype=torch.float16, device="cuda")
    y = mxq.mxq_linear(x, w, s, s, _bias_dev(ob), bits=4, group_size=64)
    want = torch.from_numpy(np.broadcast_to(ob.view(np.int16), (M, N)).copy()).cuda()
    assert torch.equal(y.view(torch.int16), want)


def test_split_k_workspace_reuse_and_streams():
    """Split-K calls keep one workspace per stream: a smaller call after a larger
    one reuses it, a larger one grows it, and a call on a second stream running
    next to one on the first uses its own.  Every result matches the oracle and a
    repeated call is bit-identical."""
    cases = {
        "a": (128, 512, 4096, 4, 64, "f16"),    # 8 splits, 2 MiB workspace
        "b": (64, 256, 8192, 8, 64, "bf16"),    # 16 splits, 1 MiB
        "c": (512, 2048, 8192, 4, 64, "f16"),   # 4 splits, 16 MiB: grows the buffer
    }
    for name, (M, N, K, bits, gs, sb) in cases.items():
        assert ",ksplit=" in mxq.mxq_describe("qmm", M, N, K, bits, gs, sb), name
    probs = {k: synth.make_problem(*c, seed=700 + i) for i, (k, c) in enumerate(cases.items())}
    dev_in = {k: to_dev(p) for k, p in probs.items()}

    def call(k):
        x, w, s, b = dev_in[k]
        p = probs[k]
        return mxq.mxq_qmm(x, w, s, b, bits=p.bits, group_size=p.group_size)

    def check(k, y):
        p = probs[k]
        if k == "c":
            cols = np.unique(np.concatenate([[0, p.N - 1], np.random.default_rng(2).integers(0, p.N, 48)]))
            ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, p.K, p.bits, p.group_size, p.sb_dtype)
            assert_close(y_host(y)[:, cols], ref, f"split-K {k}")
        else:
            assert_close(y_host(y), _ref(p), f"split-K {k}")

    note("split-K workspace: a, b, c, a on one stream")
    ya1 = call("a")
    yb = call("b")
    yc = call("c")
    ya2 = call("a")
    for k, y in (("a", ya1), ("b", yb), ("c", yc)):
        check(k, y)
    assert torch.equal(ya1.view(torch.int16), ya2.view(torch.int16))

    note("split-K workspace: c on the current stream next to a on a second stream")
    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    yc2 = call("c")
    with torch.cuda.stream(s2):
        ya3 = call("a")
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    assert torch.equal(yc.view(torch.int16), yc2.view(torch.int16))
    assert torch.equal(ya1.view(torch.int16), ya3.view(torch.int16))



# bf16 activations (x, y and the output bias in bf16) through mxq_linear_act:
# the decode kernel for M <= 8, the MFMA kernel above (split K included).
ACT_BF16 = [
    # M, N, K, bits, gs, sb
    (1, 1, 32, 4, 32, "f16"), (1, 2049, 2048, 4, 64, "f16"), (1, 513, 2048, 8, 64, "bf16"),
    (2, 1023, 8192, 4, 64, "f16"), (3, 130, 2048, 4, 64, "bf16"), (4, 2050, 8192, 8, 64, "bf16"),
    (5, 66, 4096, 8, 64, "f16"), (8, 1000, 2048, 4, 128, "f16"), (17, 33, 256, 8, 32, "bf16"),
    (64, 128, 64, 4, 64, "f16"), (100, 130, 512, 4, 32, "f16"), (200, 333, 2048, 4, 64, "bf16"),
    (129, 64, 8192, 8, 64, "f16"), (128, 512, 4096, 4, 64, "f16"), (130, 32768, 256, 4, 64, "f16"),
    (256, 16400, 512, 8, 128, "bf16"),
]


@pytest.mark.parametrize("case", ACT_BF16, ids=str)
def test_bf16_activations(case):
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M * 3 + N + K + 17, act_dtype="bf16")
    x, w, s, b = to_dev_act(p)
    note(f"bf16 activations {case}")
    y = mxq.mxq_linear_act(x, w, s, b, bits=bits, group_size=gs)
    assert y.dtype == torch.bfloat16
    ref = oracle.matmul_ref(p.x, p.w, p.scales, p.biases, K, bits, gs, sb, "bf16")
    assert_close_act(y, ref, f"bf16 act {case}")


@pytest.mark.parametrize("M", [1, 5, 96])
@pytest.mark.parametrize("bits", [4, 8])
def test_bf16_activations_with_bias(M, bits):
    N, K = 300, 1024
    p = synth.make_problem(M, N, K, bits, 64, "f16", seed=900 + M + bits, act_dtype="bf16")
    ob = synth.make_out_bias(N, seed=901 + M, act_dtype="bf16")
    x, w, s, b = to_dev_act(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    note(f"bf16 activations with bias M={M} bits={bits}")
    y = mxq.mxq_linear_act(x, w, s, b, obt, bits=bits)
    ref = oracle.linear_ref(p.x, p.w, p.scales, p.biases, ob, K, bits, 64, "f16", "bf16")
    assert_close_act(y, ref, f"bf16 act + bias M={M} bits={bits}")


@pytest.mark.parametrize("M", [1, 3, 64])
@pytest.mark.parametrize("bits", [4, 8])
def test_bf16_activations_integer_case_bitexact(M, bits):
    """Scale 1, bias 0, x in {-1, 0, 1}: every product and partial sum is an
    integer exact in f32, so y must be the round-to-nearest-even bf16 of the
    exact integer result, bit for bit (results span well past 256, where bf16
    starts rounding)."""
    N, K = 200, 512
    rng = np.random.default_rng(40 + M + bits)
    w = rng.integers(0, 2 ** 32, size=(N, K * bits // 32), dtype=np.uint32)
    s = np.full((N, K // 64), 0x3C00, dtype=np.uint16)
    b = np.zeros((N, K // 64), dtype=np.uint16)
    xv = rng.integers(-1, 2, size=(M, K)).astype(np.float64)
    xb = oracle.f32_to_bf16_bits(xv.astype(np.float32))
    p = synth.Problem(x=xb, w=w, scales=s, biases=b, M=M, N=N, K=K, bits=bits, group_size=64,
                      sb_dtype="f16", act_dtype="bf16")
    x, wt, st, bt = to_dev_act(p)
    note(f"bf16 activations integer case M={M} bits={bits}")
    y = mxq.mxq_linear_act(x, wt, st, bt, bits=bits)
    ref = oracle.matmul_ref(xb, w, s, b, K, bits, 64, "f16", "bf16")
    assert np.array_equal(ref, np.round(ref))
    want = oracle.f32_to_bf16_bits(ref.astype(np.float32))
    torch.cuda.synchronize()
    got = y.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, want), int((got != want).sum())


@pytest.mark.parametrize("M", [1, 7, 80])
def test_act_f16_matches_linear(M):
    """act_dtype f16 is mxq_linear exactly (same kernels)."""
    p = synth.make_problem(M, 260, 1024, 4, 64, "bf16", seed=950 + M)
    x, w, s, b = to_dev(p)
    ob = torch.from_numpy(synth.make_out_bias(260, seed=951).view(np.int16)).view(torch.float16).to("cuda:0")
    note(f"act f16 vs mxq_linear M={M}")
    y1 = mxq.mxq_linear(x, w, s, b, ob, bits=4)
    y2 = mxq.mxq_linear_act(x, w, s, b, ob, bits=4)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_bf16_activations_k0_and_empty():
    dev = "cuda:0"
    w = torch.zeros((5, 0), dtype=torch.int32, device=dev)
    s = torch.zeros((5, 0), dtype=torch.float16, device=dev)
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device=dev)
    ob = torch.tensor([1.5, -2.0, 0.25, 3.0, -0.5], dtype=torch.bfloat16, device=dev)
    note("bf16 activations K=0")
    y = mxq.mxq_linear_act(x, w, s, s, ob)
    torch.cuda.synchronize()
    assert torch.equal(y.float().cpu(), ob.float().cpu()[None, :].expand(3, 5))
    y0 = mxq.mxq_linear_act(torch.zeros((0, 64), dtype=torch.bfloat16, device=dev),
                            torch.zeros((5, 8), dtype=torch.int32, device=dev),
                            torch.zeros((5, 1), dtype=torch.float16, device=dev),
                            torch.zeros((5, 1), dtype=torch.float16, device=dev))
    assert tuple(y0.shape) == (0, 5)



# int8 activations (mxq_linear_a8): f16 x quantized per row inside the decode
# kernel, v_dot4 products; compared with the oracle of the same method
# (oracle.matmul_ref_a8: the same f32 quantization decisions, then f64).
A8 = [
    # M, N, K, bits, gs, sb
    (1, 1, 32, 4, 32, "f16"), (1, 2049, 2048, 4, 64, "f16"), (1, 513, 2048, 8, 64, "bf16"),
    (2, 1023, 8192, 4, 64, "f16"), (3, 130, 2048, 4, 64, "bf16"), (4, 2050, 8192, 8, 64, "bf16"),
    (5, 66, 4096, 8, 64, "f16"), (8, 1000, 2048, 4, 128, "f16"), (17, 33, 256, 8, 32, "bf16"),
    (64, 300, 1024, 4, 64, "f16"), (1, 64, 6144, 4, 64, "f16"), (2, 40, 512, 4, 32, "f16"),
]


@pytest.mark.parametrize("case", A8, ids=str)
def test_int8_activations(case):
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M * 11 + N + K + 23)
    x, w, s, b = to_dev(p)
    note(f"int8 activations {case}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=bits, group_size=gs))
    assert_close(y, oracle.matmul_ref_a8(p.x, p.w, p.scales, p.biases, K, bits, gs, sb), f"a8 {case}")


@pytest.mark.parametrize("M", [1, 2, 9])
@pytest.mark.parametrize("K", [2048, 8192])
def test_int8_activations_zero_rows_and_bias(M, K):
    """Rows of x that are all zero quantize to zero (y = output bias); a row
    whose largest |x| is 127/64 has the exact factor 64, and exact ties."""
    N = 130
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=500 + M + K)
    x = p.x.copy()
    x[0, :] = 0
    if M > 1:
        x[1, :] = np.float16(0)
        x[1, :4] = np.array([127 / 64, 5 / 128, 1 / 128, -3 / 128], dtype=np.float16)
    ob = synth.make_out_bias(N, seed=501)
    xt = torch.from_numpy(x).to("cuda:0")
    _, w, s, b = to_dev(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.float16).to("cuda:0")
    note(f"int8 activations zero rows M={M} K={K}")
    y = y_host(mxq.mxq_linear_a8(xt, w, s, b, obt, bits=4))
    ref = oracle.matmul_ref_a8(x, p.w, p.scales, p.biases, K, 4, 64, "f16") + ob.view(np.float16).astype(np.float64)
    assert_close(y, ref, f"a8 zero rows M={M} K={K}")
    assert np.array_equal(y[0], ob.view(np.float16)), "a zero row must give the output bias exactly"


@pytest.mark.parametrize("M", [1, 4])
def test_int8_activations_integer_case(M):
    """x in {-1, 0, 1} with a 1 in every row: amax 1, r = 127, xq = 127 x and
    sx = f32(1/127); with scale 1 and bias 0 every integer product and sum is
    exact, so only the row scale and the f16 store round."""
    N, K = 96, 512
    rng = np.random.default_rng(70 + M)
    w = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32)
    s = np.full((N, K // 64), 0x3C00, dtype=np.uint16)
    b = np.zeros((N, K // 64), dtype=np.uint16)
    xv = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    xv[:, 0] = 1
    p = synth.Problem(x=xv, w=w, scales=s, biases=b, M=M, N=N, K=K, bits=4, group_size=64, sb_dtype="f16")
    x, wt, st, bt = to_dev(p)
    note(f"int8 activations integer case M={M}")
    y = y_host(mxq.mxq_linear_a8(x, wt, st, bt, bits=4))
    ref = oracle.matmul_ref_a8(xv, w, s, b, K, 4, 64, "f16")
    assert_close(y, ref, f"a8 integer M={M}")


def test_int8_activations_deterministic():
    p = synth.make_problem(3, 4000, 2048, 4, 64, "f16", seed=77)
    x, w, s, b = to_dev(p)
    note("int8 activations determinism")
    y1 = mxq.mxq_linear_a8(x, w, s, b)
    y2 = mxq.mxq_linear_a8(x, w, s, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# 3..16 rows of int8 activations on shapes the K-split kernel takes (4-bit,
# K a multiple of 512 up to 4096, N >= 16 rows per CU): its integer-MFMA variant
# (rows quantized in the kernel, v_mfma_i32_16x16x64_i8 per 64-code group),
# against the same oracle; ragged N, both group sizes and scale dtypes.
A8_FEW = [
    (3, 8192, 2048, 64, "f16"), (3, 4100, 1024, 128, "bf16"), (5, 8192, 512, 64, "f16"),
    (8, 16390, 4096, 64, "bf16"), (16, 65537, 4096, 128, "f16"), (11, 128256, 2048, 64, "f16"),
    (4, 4111, 4096, 64, "f16"), (6, 8192, 3072, 64, "f16"), (13, 4100, 1536, 128, "bf16"),
]


@pytest.mark.parametrize("case", A8_FEW, ids=str)
def test_int8_few_rows_ksplit(case):
    M, N, K, gs, sb = case
    assert mxq.mxq_describe("a8", M, N, K, 4, gs, sb).startswith("qsmk_kernel"), case
    p = synth.make_problem(M, N, K, 4, gs, sb, seed=M + N + K + 41)
    x, w, s, b = to_dev(p)
    note(f"int8 few rows k-split {case}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=4, group_size=gs))
    if N * K <= 8192 * 2048:
        assert_close(y, oracle.matmul_ref_a8(p.x, p.w, p.scales, p.biases, K, 4, gs, sb), f"a8 qsmk {case}")
    else:
        cols = _sampled_cols(N, M)
        ref = oracle.matmul_ref_a8(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, 4, gs, sb)
        assert_close(y[:, cols], ref, f"a8 qsmk {case}")


# int8 activations with 8-bit codes on the integer-MFMA kernel: codes as
# signed bytes c - 128, the offset folded into the bias factor b + 128 s.
A8_FEW8 = [(3, 8192, 2048, 64, "f16"), (9, 4100, 1024, 128, "bf16"), (16, 65537, 4096, 64, "f16"),
           (7, 8192, 3584, 64, "f16"), (4, 4100, 2560, 64, "bf16")]


@pytest.mark.parametrize("case", A8_FEW8, ids=str)
def test_int8_few_rows_ksplit_8bit(case):
    M, N, K, gs, sb = case
    assert mxq.mxq_describe("a8", M, N, K, 8, gs, sb).startswith("qsmk_kernel<bits=8"), case
    p = synth.make_problem(M, N, K, 8, gs, sb, seed=M + N + K + 47)
    x, w, s, b = to_dev(p)
    note(f"int8 few rows k-split 8-bit {case}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=8, group_size=gs))
    if N * K <= 8192 * 2048:
        assert_close(y, oracle.matmul_ref_a8(p.x, p.w, p.scales, p.biases, K, 8, gs, sb), f"a8 qsmk 8-bit {case}")
    else:
        cols = _sampled_cols(N, M)
        ref = oracle.matmul_ref_a8(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, 8, gs, sb)
        assert_close(y[:, cols], ref, f"a8 qsmk 8-bit {case}")


@pytest.mark.parametrize("M", [3, 9])
def test_int8_few_rows_zero_rows_ties_and_bias(M):
    """On the integer-MFMA kernel: an all-zero row gives the output bias
    exactly; a row whose largest |x| is 127/64 has the exact factor 64 and
    exact rounding ties."""
    N, K = 8192, 2048
    assert mxq.mxq_describe("a8", M, N, K, 4, 64, "f16").startswith("qsmk_kernel")
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=600 + M)
    x = p.x.copy()
    x[0, :] = 0
    x[1, :] = np.float16(0)
    x[1, :4] = np.array([127 / 64, 5 / 128, 1 / 128, -3 / 128], dtype=np.float16)
    ob = synth.make_out_bias(N, seed=601)
    xt = torch.from_numpy(x).to("cuda:0")
    _, w, s, b = to_dev(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.float16).to("cuda:0")
    note(f"int8 few rows zero rows M={M}")
    y = y_host(mxq.mxq_linear_a8(xt, w, s, b, obt, bits=4))
    ref = oracle.matmul_ref_a8(x, p.w, p.scales, p.biases, K, 4, 64, "f16") + ob.view(np.float16).astype(np.float64)
    assert_close(y, ref, f"a8 qsmk zero rows M={M}")
    assert np.array_equal(y[0], ob.view(np.float16)), "a zero row must give the output bias exactly"


def test_int8_few_rows_integer_case_and_determinism():
    """x in {-1, 0, 1}, scale 1, bias 0 on the integer-MFMA kernel: every
    product and sum is an exact integer, only the row scale and the f16 store
    round; two runs are bit-identical."""
    M, N, K = 4, 4096, 1024
    assert mxq.mxq_describe("a8", M, N, K, 4, 64, "f16").startswith("qsmk_kernel")
    rng = np.random.default_rng(71)
    w = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint32)
    s = np.full((N, K // 64), 0x3C00, dtype=np.uint16)
    b = np.zeros((N, K // 64), dtype=np.uint16)
    xv = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    xv[:, 0] = 1
    p = synth.Problem(x=xv, w=w, scales=s, biases=b, M=M, N=N, K=K, bits=4, group_size=64, sb_dtype="f16")
    x, wt, st, bt = to_dev(p)
    note("int8 few rows integer case")
    y1 = y_host(mxq.mxq_linear_a8(x, wt, st, bt, bits=4))
    y2 = y_host(mxq.mxq_linear_a8(x, wt, st, bt, bits=4))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    assert_close(y1, oracle.matmul_ref_a8(xv, w, s, b, K, 4, 64, "f16"), "a8 qsmk integer")


# Few activation rows with K a multiple of the group size but not of 512: the
# K-split kernel's ragged variant (the last 512-code slice ends early; beyond
# 4096 in chunks, the last chunk's slices may be empty).  Sampled output
# columns against the oracle, including the ragged tail of N.
QSM = [
    (9, 65600, 2112, 4, 64, "f16"), (10, 66000, 576, 8, 64, "bf16"), (16, 65536, 4352, 4, 128, "f16"),
    (13, 70001, 2624, 8, 64, "bf16"), (12, 65540, 6272, 8, 128, "f16"), (16, 128256, 1088, 8, 64, "f16"),
    (2, 8192, 640, 4, 64, "f16"), (3, 4100, 2944, 4, 128, "bf16"), (5, 8192, 4032, 8, 64, "f16"),
    (8, 16390, 1216, 4, 64, "bf16"), (4, 4096, 4160, 4, 64, "f16"), (7, 4116, 9024, 8, 64, "bf16"),
]


def _sampled_cols(N, seed):
    return np.unique(np.concatenate([[0, 1, N - 2, N - 1], np.arange(N - 300, N - 250),
                                     np.random.default_rng(seed).integers(0, N, 150)]))


@pytest.mark.parametrize("case", QSM, ids=str)
def test_few_rows_ksplit_ragged_k(case):
    M, N, K, bits, gs, sb = case
    d = mxq.mxq_describe("qmv", M, N, K, bits, gs, sb)
    assert d.startswith("qsmk_kernel") and ",ragged" in d, (case, d)
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + K + 31)
    x, w, s, b = to_dev(p)
    note(f"few-row k-split ragged K {case}: {d}")
    y = y_host(mxq.mxq_qmv(x, w, s, b, bits=bits, group_size=gs))
    if N * K <= 8192 * 2048:
        assert_close(y, _ref(p), f"qsmk ragged {case}")
    else:
        cols = _sampled_cols(N, M)
        ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, bits, gs, sb)
        assert_close(y[:, cols], ref, f"qsmk ragged {case}")


def _shifted(t):
    """The same values in a buffer whose start is 2 bytes past a 16-byte boundary."""
    big = torch.empty(t.numel() + 1, dtype=t.dtype, device=t.device)
    v = big[1:].view(t.shape)
    v.copy_(t)
    assert v.data_ptr() % 16 == 2
    return v


@pytest.mark.parametrize("case", [(4, 8192, 2048, 4, 64, "f16"), (12, 65536, 1536, 8, 128, "bf16"),
                                  (6, 4100, 2112, 4, 64, "f16"), (9, 8192, 8192, 4, 64, "f16")], ids=str)
def test_few_rows_ksplit_unaligned_scales(case):
    """Scales and biases 2-byte but not 16-byte aligned: the ragged variant's
    2-byte scale and bias loads (before, the call left the matrix cores)."""
    M, N, K, bits, gs, sb = case
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + K + 33)
    x, w, s, b = to_dev(p)
    s2, b2 = _shifted(s), _shifted(b)
    note(f"few-row k-split unaligned scales {case}")
    y = y_host(mxq.mxq_qmv(x, w, s2, b2, bits=bits, group_size=gs))
    y_aligned = y_host(mxq.mxq_qmv(x, w, s, b, bits=bits, group_size=gs))
    if K % 512 == 0:  # the same kernel arithmetic either way: bit-identical
        assert np.array_equal(y.view(np.uint16), y_aligned.view(np.uint16)), case
    cols = _sampled_cols(N, M)
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, bits, gs, sb)
    assert_close(y[:, cols], ref, f"qsmk unaligned scales {case}")


@pytest.mark.parametrize("case", [(3, 8192, 2112, 4, 64, "f16"), (9, 4100, 1152, 8, 128, "bf16"),
                                  (16, 65540, 3008, 4, 64, "f16")], ids=str)
def test_int8_few_rows_ragged_k(case):
    M, N, K, bits, gs, sb = case
    d = mxq.mxq_describe("a8", M, N, K, bits, gs, sb)
    assert d.startswith("qsmk_kernel") and ",act=i8" in d and ",ragged" in d, (case, d)
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + K + 49)
    x, w, s, b = to_dev(p)
    note(f"int8 few rows ragged K {case}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=bits, group_size=gs))
    cols = _sampled_cols(N, M)
    ref = oracle.matmul_ref_a8(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, bits, gs, sb)
    assert_close(y[:, cols], ref, f"a8 qsmk ragged {case}")


def test_few_rows_16_row_blocks_under_capture():
    """9..16 rows at a ragged K beyond 4096 on a stream being captured (no K
    chunks inside a graph): the 16-row-block kernel, every replay against the
    oracle."""
    M, N, K, bits, gs, sb = 12, 65540, 6272, 8, 128, "f16"
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=77)
    x, w, s, b = to_dev(p)
    y = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    note("16-row-block kernel under graph capture")
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=st):
        mxq.mxq_qmv(x, w, s, b, y, bits=bits, group_size=gs)
    cols = _sampled_cols(N, M)
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, bits, gs, sb)
    for r in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_close(y.cpu().numpy()[:, cols], ref, f"qsm captured replay {r}")


# 2..16 rows, 4-bit codes, K a multiple of 512 up to 4096, at least 16 W rows per
# compute unit: the K-split few-row kernel (qsmk), for 1, 2, 4 and 8 waves per
# workgroup, group sizes 64 and 128, both scale dtypes, ragged N.
QSMK = [
    (2, 128256, 2048, 64, "f16"), (3, 4100, 512, 64, "bf16"), (5, 8192, 1024, 128, "f16"),
    (8, 8192, 2048, 64, "bf16"), (16, 16390, 4096, 64, "f16"), (11, 65537, 4096, 128, "bf16"),
    (16, 128256, 2048, 64, "f16"), (4, 4111, 4096, 64, "f16"), (6, 8192, 3072, 64, "bf16"),
    (9, 4300, 2560, 128, "f16"), (3, 8192, 3584, 64, "f16"), (2, 8200, 3072, 64, "f16"), (2, 4100, 2560, 128, "bf16"),
]


# 8-bit codes on the K-split kernel (natural-order byte unpack, 512-byte row
# slices per wave), including shapes the 16-row-block kernel used to take.
QSMK8 = [
    (2, 8192, 2048, 64, "f16"), (4, 4100, 1536, 64, "bf16"), (10, 66000, 1024, 64, "bf16"),
    (13, 70001, 512, 64, "bf16"), (12, 65540, 4096, 128, "f16"), (16, 128256, 2048, 64, "f16"),
    (7, 8192, 4096, 64, "f16"), (5, 8192, 3584, 128, "f16"), (3, 4100, 2560, 64, "bf16"), (2, 8196, 3072, 64, "f16"),
]


@pytest.mark.parametrize("case", QSMK8, ids=str)
def test_few_rows_ksplit_8bit(case):
    M, N, K, gs, sb = case
    assert mxq.mxq_describe("qmv", M, N, K, 8, gs, sb).startswith("qsmk_kernel<bits=8"), case
    p = synth.make_problem(M, N, K, 8, gs, sb, seed=M + N + K + 43)
    x, w, s, b = to_dev(p)
    note(f"few-row k-split 8-bit {case}")
    y = y_host(mxq.mxq_qmv(x, w, s, b, bits=8, group_size=gs))
    if N * K <= 8192 * 2048:
        assert_close(y, _ref(p), f"qsmk 8-bit {case}")
    else:
        cols = _sampled_cols(N, M)
        ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, 8, gs, sb)
        assert_close(y[:, cols], ref, f"qsmk 8-bit {case}")


@pytest.mark.parametrize("entry", ["qmv", "qmm"])
@pytest.mark.parametrize("case", QSMK, ids=str)
def test_few_rows_ksplit(case, entry):
    M, N, K, gs, sb = case
    assert mxq.mxq_describe(entry, M, N, K, 4, gs, sb).startswith("qsmk_kernel"), case
    p = synth.make_problem(M, N, K, 4, gs, sb, seed=M + N + K + 37)
    x, w, s, b = to_dev(p)
    note(f"few-row k-split {entry} {case}")
    fn = mxq.mxq_qmv if entry == "qmv" else mxq.mxq_qmm
    y = y_host(fn(x, w, s, b, bits=4, group_size=gs))
    if N * K <= 8192 * 2048:
        assert_close(y, _ref(p), f"qsmk {case}")
    else:
        cols = _sampled_cols(N, M)
        ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, 4, gs, sb)
        assert_close(y[:, cols], ref, f"qsmk {case}")


@pytest.mark.parametrize("regime", ["big", "tiny"])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(4, 4100, 2048, 64), (9, 8192, 1024, 128), (16, 4096, 4096, 64)], ids=str)
def test_few_rows_ksplit_scale_regimes(shape, sb, regime):
    """The K-split kernel's codes carry an offset of 1024 that leaves through
    the bias factor b - 1024 s: scales near the f16 range, f16 subnormal and
    zero scales and bf16 scales far below f16's range, random signs."""
    M, N, K, gs = shape
    assert mxq.mxq_describe("qmv", M, N, K, 4, gs, sb).startswith("qsmk_kernel"), shape
    p = _scale_regime_problem(M, N, K, gs, sb, regime, seed=M + N + gs + 3)
    note(f"qsmk scale regime {shape} {sb} {regime}")
    y = _run("qmv", p)
    assert np.all(np.isfinite(y))
    assert_close(y, _ref(p), f"qsmk scale regime {shape} {sb} {regime}")


# K beyond 4096 on the K-split kernel: K chunks of up to eight 512-code
# slices (the grid's second dimension), f32 partial tiles, fixed-order sum.
# (M, N, K, bits, group, scale dtype); chunks x waves: 2 x 8, 4 x 7, 2 x 8,
# 2 x 5, 2 x 8, 2 x 6, 2 x 8 (8-bit), 3 x 6 (8-bit)
QSMK_LONGK = [
    (4, 8192, 8192, 4, 64, "f16"), (16, 4100, 14336, 4, 128, "bf16"), (4, 2050, 8192, 4, 64, "f16"),
    (8, 4104, 5120, 4, 64, "bf16"), (12, 16400, 8192, 4, 64, "f16"), (5, 4096, 6144, 4, 128, "f16"),
    (6, 4100, 8192, 8, 64, "f16"), (9, 4104, 9216, 8, 128, "bf16"),
]


@pytest.mark.parametrize("entry", ["qmv", "qmm"])
@pytest.mark.parametrize("case", QSMK_LONGK, ids=str)
def test_few_rows_ksplit_long_k(case, entry):
    M, N, K, bits, gs, sb = case
    d = mxq.mxq_describe(entry, M, N, K, bits, gs, sb)
    assert d.startswith(f"qsmk_kernel<bits={bits}") and ",kchunks=" in d, (case, d)
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + K + 53)
    x, w, s, b = to_dev(p)
    note(f"few-row k-split, K chunks {entry} {case}")
    fn = mxq.mxq_qmv if entry == "qmv" else mxq.mxq_qmm
    y = y_host(fn(x, w, s, b, bits=bits, group_size=gs))
    cols = np.arange(N) if N * K <= 4104 * 8192 else _sampled_cols(N, M)
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, K, bits, gs, sb)
    assert_close(y[:, cols], ref, f"qsmk long K {case}")
    # the fixed-order chunk sum is deterministic
    y2 = y_host(fn(x, w, s, b, bits=bits, group_size=gs))
    assert np.array_equal(y.view(np.uint16), y2.view(np.uint16)), case


def test_few_rows_ksplit_long_k_bias_and_capture():
    """K chunks with an output bias (added once, by the reduction), and the
    same call under graph capture, which keeps the other kernels (no cached
    workspace inside a graph): both within the bar, every replay equal."""
    M, N, K, gs = 8, 4100, 8192, 64
    p = synth.make_problem(M, N, K, 4, gs, "f16", seed=611)
    ob = synth.make_out_bias(N, seed=612)
    x, w, s, b = to_dev(p)
    obd = _bias_dev(ob)
    note("few-row k-split, K chunks, bias and capture")
    ref = oracle.linear_ref(p.x, p.w, p.scales, p.biases, ob, K, 4, gs, "f16")
    y = y_host(mxq.mxq_linear(x, w, s, b, obd, bits=4, group_size=gs))
    assert_close(y, ref, "qsmk long K with bias")
    yg = torch.empty((M, N), dtype=torch.float16, device="cuda")
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        mxq.mxq_linear(x, w, s, b, obd, y=yg, bits=4, group_size=gs)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        mxq.mxq_linear(x, w, s, b, obd, y=yg, bits=4, group_size=gs)
    torch.cuda.synchronize()
    first = None
    for _ in range(3):
        yg.zero_()
        g.replay()
        torch.cuda.synchronize()
        got = yg.cpu().numpy()
        assert_close(got, ref, "qsmk long K captured")
        if first is None:
            first = got.copy()
        assert np.array_equal(got.view(np.uint16), first.view(np.uint16))


@pytest.mark.parametrize("regime", ["big", "tiny"])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
@pytest.mark.parametrize("shape", [(1, 4104, 2048, 64), (1, 2050, 8192, 128), (4, 1030, 2048, 64), (2, 514, 4096, 64)])
def test_decode_kernel_scale_regimes(shape, sb, regime):
    """The decode kernel's f16 4-bit codes carry an offset of 64 that leaves
    through the bias factor b - 64 s: scales near the f16 range, f16 subnormal
    scales and bf16 scales far below f16's range, random signs, zero biases."""
    M, N, K, gs = shape
    assert mxq.mxq_describe("qmv", M, N, K, 4, gs, sb).startswith("qmv_kernel"), shape
    p = _scale_regime_problem(M, N, K, gs, sb, regime, seed=M + N + gs + 11)
    note(f"decode kernel scale regime {shape} {sb} {regime}")
    y = _run("qmv", p)
    assert np.all(np.isfinite(y))
    assert_close(y, _ref(p), f"decode kernel scale regime {shape} {sb} {regime}")


def test_few_rows_ksplit_routing():
    """Shapes around the K-split kernel's bounds take the other kernels."""
    d = mxq.mxq_describe
    assert d("a8", 3, 8192, 2048, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=3,waves=4,act=i8>")
    assert d("a8", 2, 8192, 2048, 4, 64, "f16").startswith("qmv_kernel")       # two int8 rows: decode kernel
    assert d("a8", 12, 8192, 2048, 8, 64, "f16").startswith("qsmk_kernel<bits=8,sb=f16,gs=64,m=12,waves=4,act=i8>")
    assert d("qmv", 2, 8192, 2048, 4, 64, "f16").startswith("qsmk")
    assert not d("qmv", 2, 16384, 4096, 4, 64, "f16").startswith("qsmk")   # two rows at K > 3072: decode kernel
    assert d("qmv", 2, 65536, 3072, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=2,waves=6>")
    assert d("qmv", 3, 16384, 4096, 4, 64, "f16").startswith("qsmk")
    assert not d("qmv", 1, 128256, 2048, 4, 64, "f16").startswith("qsmk")
    assert not d("qmv", 17, 128256, 2048, 4, 64, "f16").startswith("qsmk")
    assert d("qmv", 8, 128256, 2048, 8, 64, "f16").startswith("qsmk_kernel<bits=8")   # 8-bit codes
    assert d("a8", 8, 128256, 2048, 8, 64, "f16").startswith("qsmk_kernel<bits=8")  # int8 x with 8-bit codes
    assert d("a8", 8, 128256, 1536, 8, 64, "f16").startswith("qsmk_kernel<bits=8")  # K = 3 x 512: 3 waves
    assert d("a8", 8, 128256, 2112, 8, 64, "f16").startswith("qsmk_kernel<bits=8,sb=f16,gs=64,m=8,waves=5,act=i8,ragged>")
    assert d("a8", 8, 128256, 4160, 8, 64, "f16").startswith("qmv_kernel")         # ragged K in chunks: int8 x
    assert not d("qmv", 8, 128256, 2048, 4, 32, "f16").startswith("qsmk")   # group size 32
    assert d("qmv", 8, 128256, 1536, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=8,waves=3>")
    assert d("qmv", 8, 128256, 2112, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=8,waves=5,ragged>")
    assert d("qmv", 8, 128256, 4160, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=8,waves=5,kchunks=2,ragged>")
    assert not d("qmv", 8, 128256, 448, 4, 64, "f16").startswith("qsmk")    # K below one 512-code slice
    assert d("qmv", 8, 128256, 8192, 4, 64, "f16").startswith("qsmk_kernel<bits=4,sb=f16,gs=64,m=8,waves=8,kchunks=2>")
    assert d("a8", 8, 128256, 8192, 4, 64, "f16").startswith("qmv_kernel")       # int8 x: one row scale over all K
    assert not d("qmv", 3, 128257, 8192, 4, 64, "f16").startswith("qsmk")   # chunks need M * N % 4 == 0
    assert not d("qmv", 8, 1023, 8192, 4, 64, "f16").startswith("qsmk")     # 64 x 2 blocks: too few
    assert not d("qmv", 8, 2048, 2048, 4, 64, "f16").startswith("qsmk")     # too few W rows per CU


def test_few_rows_ksplit_misaligned_scales_and_determinism():
    """Scales and biases only 2-byte aligned stay on the K-split kernel (its
    ragged variant reads them as 2-byte values) with a bit-identical result;
    the result is also bit-identical from run to run."""
    M, N, K = 6, 8192, 2048
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=77)
    x, w, s, b = to_dev(p)
    y1 = y_host(mxq.mxq_qmv(x, w, s, b, bits=4))
    y2 = y_host(mxq.mxq_qmv(x, w, s, b, bits=4))
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    G = K // 64
    s_off = torch.empty(N * G + 1, dtype=torch.float16, device="cuda:0")
    b_off = torch.empty(N * G + 1, dtype=torch.float16, device="cuda:0")
    s_off[1:].copy_(s.reshape(-1))
    b_off[1:].copy_(b.reshape(-1))
    note("few-row k-split misaligned scales")
    y3 = y_host(mxq.mxq_qmv(x, w, s_off[1:].view(N, G), b_off[1:].view(N, G), bits=4))
    ref = _ref(p)
    assert_close(y1, ref, "qsmk aligned")
    assert np.array_equal(y1.view(np.uint16), y3.view(np.uint16)), "2-byte scale loads change no bit"


@pytest.mark.parametrize("case", [(11, 32776, 2048, 4, 64, "f16", "f16"), (16, 32776, 1024, 8, 128, "bf16", "f16"),
                                  (12, 40000, 2048, 4, 64, "f16", "i8"), (10, 65544, 1536, 4, 64, "bf16", "f16")],
                         ids=str)
def test_few_rows_xcd_block_order_and_tails(case):
    """10-16 rows on the K-split kernel with a full grid (512 workgroups), whose
    blocks are taken in the XCD-grouped order within each round of the grid
    stride: N a multiple of 8 but not of 16 or 64 (a last block of 8 columns,
    a partial last round), an output bias, int8 activations; sampled columns
    against the oracle, and bit-identical to the same call with y only 2-byte
    aligned."""
    M, N, K, bits, gs, sb, act = case
    assert mxq.mxq_describe("a8" if act == "i8" else "qmv", M, N, K, bits, gs, sb).startswith("qsmk_kernel")
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + N + 77)
    ob = synth.make_out_bias(N, seed=78)
    x, w, s, b = to_dev(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.float16).to("cuda:0")
    call = mxq.mxq_linear_a8 if act == "i8" else mxq.mxq_linear
    note(f"few-row xcd block order {case}")
    y1 = torch.empty((M, N), dtype=torch.float16, device="cuda:0")
    call(x, w, s, b, obt, y1, bits=bits, group_size=gs)
    y_off = torch.empty(M * N + 1, dtype=torch.float16, device="cuda:0")
    y2 = y_off[1:].view(M, N)
    call(x, w, s, b, obt, y2, bits=bits, group_size=gs)
    y1h, y2h = y_host(y1), y_host(y2)
    assert np.array_equal(y1h.view(np.uint16), y2h.view(np.uint16)), "y alignment changes no bit"
    cols = _sampled_cols(N, 300 + M)
    if act == "i8":
        ref = oracle.matmul_ref_a8(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, bits, gs, sb)
        ref = ref + ob.view(np.float16)[cols].astype(np.float64)
    else:
        ref = oracle.linear_ref(p.x, p.w[cols], p.scales[cols], p.biases[cols], ob[cols], K, bits, gs, sb)
    assert_close(y1h[:, cols], ref, f"xcd block order {case}")


@pytest.mark.parametrize("case", [(9, 32768, 2112, 4, 64, "f16"), (13, 32768, 4096, 8, 64, "bf16"),
                                  (16, 65536, 2304, 4, 128, "f16"), (9, 40000, 2048, 8, 128, "f16")], ids=str)
def test_few_rows_staged_activations(case):
    """From 9 rows (f16 activations) the K-split kernel passes each wave's
    activation slice through LDS, whole row pieces per load, before the first
    block: 9 rows (half of the last load pair past M), a ragged K whose last
    slice holds one group, 8 waves, 8-bit codes, groups of 128; sampled
    columns against the oracle.  At 8 rows, and with int8 activations, the
    kernel loads the activations in the A layout directly."""
    M, N, K, bits, gs, sb = case
    d = mxq.mxq_describe("qmv", M, N, K, bits, gs, sb)
    assert d.startswith("qsmk_kernel") and ",xstage>" in d, d
    assert ",xstage" not in mxq.mxq_describe("qmv", 8, N, K, bits, gs, sb)
    assert ",xstage" not in mxq.mxq_describe("a8", M, N, K, bits, gs, sb)
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M + K + 91)
    x, w, s, b = to_dev(p)
    note(f"few-row staged activations {case}")
    y = y_host(mxq.mxq_qmv(x, w, s, b, bits=bits, group_size=gs))
    cols = _sampled_cols(N, 500 + M)
    ref = oracle.matmul_ref(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, bits, gs, sb)
    assert_close(y[:, cols], ref, f"staged activations {case}")


@pytest.mark.parametrize("M", list(range(2, 17)))
def test_few_rows_mfma_every_m(M):
    """Every row count the K-split few-row kernel takes, through mxq_linear
    (4-bit, with an output bias)."""
    N, K = 65792, 1024
    assert mxq.mxq_describe("qmm", M, N, K, 4, 64, "f16").startswith("qsmk_kernel"), M
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=1200 + M)
    ob = synth.make_out_bias(N, seed=1201)
    x, w, s, b = to_dev(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.float16).to("cuda:0")
    note(f"few-row mfma M={M}")
    y = y_host(mxq.mxq_linear(x, w, s, b, obt, bits=4))
    cols = _sampled_cols(N, 100 + M)
    ref = oracle.linear_ref(p.x, p.w[cols], p.scales[cols], p.biases[cols], ob[cols], K, 4, 64, "f16")
    assert_close(y[:, cols], ref, f"qsm M={M}")
