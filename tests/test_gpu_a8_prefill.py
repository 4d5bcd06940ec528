"""int8 activations at prefill sizes (M >= 17): mxq_linear_a8 on the integer
matrix-core kernel (x quantized per row once, v_mfma_i32_32x32x32_i8 per
32-code step, per-group f32 scale, bias term on bf16 MFMAs), against the
oracle of the same method (oracle.matmul_ref_a8: the same f32 quantization
decisions, then f64).

Bar: |y - y_ref| <= 2e-3 (1 + |y_ref|).
"""

import numpy as np
import pytest
import torch

import dequant_matmul_qmv_amd as mxq
import oracle
import synth
from tests.gpu_util import assert_close, note, to_dev, y_host

pytestmark = pytest.mark.gpu

# M, N, K, bits, gs, sb: tiles past M and N, every group size and scale dtype,
# K with a partial 16-group bias block (K / 64 = 40, 24; K / 32 = 36), and K
# long enough for the split into partial tiles
CASES = [
    (17, 33, 256, 4, 64, "f16"), (17, 1000, 2048, 4, 64, "f16"), (24, 300, 1152, 4, 32, "f16"),
    (64, 2050, 2560, 4, 64, "bf16"), (100, 513, 1536, 4, 128, "f16"), (128, 256, 2048, 8, 64, "f16"),
    (129, 130, 1024, 8, 32, "bf16"), (200, 777, 4096, 8, 128, "bf16"), (256, 1024, 8192, 4, 64, "f16"),
    (33, 4100, 8192, 8, 64, "f16"), (512, 384, 2048, 4, 64, "bf16"), (40, 64, 64, 4, 64, "f16"),
]


def _ref(p):
    return oracle.matmul_ref_a8(p.x, p.w, p.scales, p.biases, p.K, p.bits, p.group_size, p.sb_dtype)


@pytest.mark.parametrize("case", CASES, ids=str)
def test_a8_prefill_matches_oracle(case):
    M, N, K, bits, gs, sb = case
    desc = mxq.mxq_describe("a8", M, N, K, bits, gs, sb)
    assert "qmm_a8_kernel" in desc, desc
    p = synth.make_problem(M, N, K, bits, gs, sb, seed=M * 7 + N + K + bits + 900)
    x, w, s, b = to_dev(p)
    note(f"a8 prefill {case}: {desc}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=bits, group_size=gs))
    assert_close(y, _ref(p), f"a8 prefill {case}")


def test_a8_prefill_split_k_is_used():
    """A shape whose 128 x 128 tiles alone do not occupy the GPU runs with K
    split (f32 partial tiles summed in a fixed order)."""
    assert ",ksplit=" in mxq.mxq_describe("a8", 256, 1024, 8192, 4, 64, "f16")
    assert ",ksplit=" in mxq.mxq_describe("a8", 512, 2048, 8192, 4, 64, "f16")
    assert ",ksplit=" not in mxq.mxq_describe("a8", 512, 8192, 2048, 4, 64, "f16")


@pytest.mark.parametrize("M", [17, 130])
def test_a8_prefill_zero_rows_ties_and_bias(M):
    """An all-zero row gives the output bias exactly; a row whose largest |x|
    is 127/64 has the exact factor 64 and exact rounding ties."""
    N, K = 300, 2048
    p = synth.make_problem(M, N, K, 4, 64, "f16", seed=950 + M)
    x = p.x.copy()
    x[0, :] = 0
    x[M - 1, :] = np.float16(0)
    x[M - 1, :4] = np.array([127 / 64, 5 / 128, 1 / 128, -3 / 128], dtype=np.float16)
    ob = synth.make_out_bias(N, seed=951)
    xt = torch.from_numpy(x).to("cuda:0")
    _, w, s, b = to_dev(p)
    obt = torch.from_numpy(ob.view(np.int16)).view(torch.float16).to("cuda:0")
    note(f"a8 prefill zero rows and ties M={M}")
    y = y_host(mxq.mxq_linear_a8(xt, w, s, b, obt, bits=4))
    ref = oracle.matmul_ref_a8(x, p.w, p.scales, p.biases, K, 4, 64, "f16") + ob.view(np.float16).astype(np.float64)
    assert_close(y, ref, f"a8 prefill zero rows M={M}")
    assert np.array_equal(y[0], ob.view(np.float16)), "a zero row must give the output bias exactly"


@pytest.mark.parametrize("bits", [4, 8])
def test_a8_prefill_integer_case(bits):
    """x in {-1, 0, 1} with a 1 in every row, scale 1, bias 0: every integer
    product and sum is exact, so only the row scale and the f16 store round."""
    M, N, K = 48, 200, 1024
    rng = np.random.default_rng(960 + bits)
    w = rng.integers(0, 2 ** 32, size=(N, K * bits // 32), dtype=np.uint32)
    s = np.full((N, K // 64), 0x3C00, dtype=np.uint16)
    b = np.zeros((N, K // 64), dtype=np.uint16)
    xv = rng.integers(-1, 2, size=(M, K)).astype(np.float16)
    xv[:, 0] = 1
    p = synth.Problem(x=xv, w=w, scales=s, biases=b, M=M, N=N, K=K, bits=bits, group_size=64, sb_dtype="f16")
    x, wt, st, bt = to_dev(p)
    note(f"a8 prefill integer case bits={bits}")
    y = y_host(mxq.mxq_linear_a8(x, wt, st, bt, bits=bits))
    assert_close(y, oracle.matmul_ref_a8(xv, w, s, b, K, bits, 64, "f16"), f"a8 prefill integer bits={bits}")


@pytest.mark.parametrize("proj", ["gate", "down"])
@pytest.mark.parametrize("sb", ["f16", "bf16"])
def test_a8_prefill_full_size_sampled(proj, sb):
    """M = 512 on the Llama-3.2-1B gate (8192 x 2048) and down (2048 x 8192,
    K split) projections: sampled output columns against the oracle."""
    N, K = (8192, 2048) if proj == "gate" else (2048, 8192)
    p = synth.make_problem(512, N, K, 4, 64, sb, seed=970 + (proj == "down"))
    x, w, s, b = to_dev(p)
    note(f"a8 prefill full size {proj} {sb}: {mxq.mxq_describe('a8', 512, N, K, 4, 64, sb)}")
    y = y_host(mxq.mxq_linear_a8(x, w, s, b, bits=4))
    cols = np.unique(np.concatenate([[0, 1, 127, 128, N - 1], np.random.default_rng(5).integers(0, N, 120)]))
    ref = oracle.matmul_ref_a8(p.x, p.w[cols], p.scales[cols], p.biases[cols], K, 4, 64, sb)
    assert_close(y[:, cols], ref, f"a8 prefill {proj} {sb}")


def test_a8_prefill_deterministic():
    p = synth.make_problem(256, 1024, 8192, 4, 64, "f16", seed=980)  # split K
    x, w, s, b = to_dev(p)
    note("a8 prefill determinism")
    y1 = mxq.mxq_linear_a8(x, w, s, b).clone()
    y2 = mxq.mxq_linear_a8(x, w, s, b)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_a8_prefill_graph_replay():
    """Captured into a HIP graph (the workspace is then allocated and freed
    inside the graph): every replay, with eager work in between, equals the
    eager result bit for bit."""
    p = synth.make_problem(256, 1024, 8192, 4, 64, "f16", seed=981)
    x, w, s, b = to_dev(p)
    note("a8 prefill graph replay")
    want = mxq.mxq_linear_a8(x, w, s, b).clone()
    y = torch.empty_like(want)
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        mxq.mxq_linear_a8(x, w, s, b, y=y, stream=st)
    torch.cuda.current_stream().wait_stream(st)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        mxq.mxq_linear_a8(x, w, s, b, y=y)
    for r in range(3):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), want.view(torch.int16)), f"replay {r}"
        _ = mxq.mxq_linear_a8(x, w, s, b)  # eager work between replays
        torch.cuda.synchronize()
