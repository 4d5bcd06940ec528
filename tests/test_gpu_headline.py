"""The launches the headline decode measurement makes, and large-buffer
addressing, against the CPU oracle through libmxq's C ABI.

* Grouped launches with activations held in registers ("xreg"): the
  Llama-3.2-1B layer groups {q, k, v} and {gate, up} at one and two rows,
  plus mixed groups whose every K fits one 64-segment step.
* A weight matrix larger than 4 GiB: rows on both sides of the 4 GiB line.
* The split workspace: reuse, growth and release.

Bar: |y - y_ref| <= 2e-3 (1 + |y_ref|) against the f64 oracle.
"""

import numpy as np
import pytest
import torch

import dequant_matmul_qmv_amd as mxq
import oracle
import synth
from tests.gpu_util import assert_close, note, to_dev, y_host

pytestmark = pytest.mark.gpu

Q, K_, V, O, GATE, UP, DOWN = synth.LLAMA_1B_PROJ


def _ref(p):
    return oracle.matmul_ref(p.x, p.w, p.scales, p.biases, p.K, p.bits, p.group_size, p.sb_dtype)


GROUPS = {
    # name: (bits, scale dtype, [(N, K), ...])
    "qkv": (4, "f16", [(Q[1], Q[2]), (K_[1], K_[2]), (V[1], V[2])]),
    "gate_up": (4, "f16", [(GATE[1], GATE[2]), (UP[1], UP[2])]),
    "mixed_4bit": (4, "f16", [(2048, 2048), (513, 1024), (8192, 2048), (1023, 512), (7, 64), (2050, 2048),
                              (64, 2048), (130, 1536)]),
    "mixed_4bit_bf16": (4, "bf16", [(4100, 2048), (1, 2048), (257, 1024)]),
    "mixed_8bit": (8, "f16", [(2048, 1024), (1023, 512), (4097, 1024), (33, 64)]),
}


@pytest.mark.parametrize("M", [1, 2])
@pytest.mark.parametrize("group", list(GROUPS))
def test_grouped_register_activations(group, M):
    """mxq_qmv_grouped on groups whose activations stay in registers: the
    kernel variant behind the headline's {q,k,v} and {gate,up} launches."""
    bits, sb, shapes = GROUPS[group]
    desc = mxq.mxq_describe_grouped(shapes, M, bits, 64, sb)
    assert ",xreg>" in desc and ";" not in desc, desc  # one launch, register-resident x
    probs = [synth.make_problem(M, N, K, bits, 64, sb, seed=synth.proj_seed(1, 40 + M, i) + 7 * len(group))
             for i, (N, K) in enumerate(shapes)]
    dev = [to_dev(p) for p in probs]
    note(f"grouped xreg {group} M={M}: {desc}")
    ys = mxq.mxq_qmv_grouped(dev, bits=bits, group_size=64)
    torch.cuda.synchronize()
    for i, (p, y) in enumerate(zip(probs, ys)):
        assert_close(y.cpu().numpy(), _ref(p), f"{group}[{i}] M={M} N={p.N} K={p.K}")


def test_grouped_register_activations_deterministic():
    bits, sb, shapes = GROUPS["qkv"]
    probs = [synth.make_problem(1, N, K, bits, 64, sb, seed=50 + i) for i, (N, K) in enumerate(shapes)]
    dev = [to_dev(p) for p in probs]
    note("grouped xreg determinism")
    a = [y.clone() for y in mxq.mxq_qmv_grouped(dev, bits=bits)]
    b = mxq.mxq_qmv_grouped(dev, bits=bits)
    torch.cuda.synchronize()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.int16), v.view(torch.int16))


# ------------------------------------------------------ W beyond 4 GiB ---
# 8-bit codes, K = 16384: a row is 16 KiB, so rows from 262,144 on start past
# the 4 GiB line.  W repeats a block of P distinct rows (P does not divide
# 262,144, so a row read from an address wrapped at 4 GiB would hold another
# block row's codes and fail the comparison).
BIG_K, BIG_N, BIG_P = 16384, 262144 + 1037, 4099


@pytest.fixture(scope="module")
def big_w():
    p = synth.make_problem(1, BIG_P, BIG_K, 8, 64, "f16", seed=4242)
    w_blk, s_blk, b_blk = to_dev(p)[1:]
    reps = -(-BIG_N // BIG_P)
    note(f"building W of {BIG_N} x {BIG_K} 8-bit codes ({BIG_N * BIG_K / 2**30:.2f} GiB)")
    w = w_blk.repeat(reps, 1)[:BIG_N].contiguous()
    s = s_blk.repeat(reps, 1)[:BIG_N].contiguous()
    b = b_blk.repeat(reps, 1)[:BIG_N].contiguous()
    assert w.numel() * 4 > 2 ** 32
    yield p, w, s, b
    del w, s, b
    torch.cuda.empty_cache()


@pytest.mark.parametrize("M", [1, 2, 4, 5])
def test_weight_over_4gib(big_w, M):
    p, w, s, b = big_w
    xs = synth.make_x(M, BIG_K, seed=600 + M)
    x = torch.from_numpy(xs).cuda()
    line = 2 ** 32 // (BIG_K * 8 // 8)  # first row past 4 GiB
    rng = np.random.default_rng(M)
    rows = np.unique(np.concatenate([
        [0, 1, line - 1, line, line + 1, BIG_N - 1],
        rng.integers(0, line, 64), rng.integers(line, BIG_N, 256)]))
    desc = mxq.mxq_describe("qmv", M, BIG_N, BIG_K, 8, 64)
    note(f"qmv W over 4 GiB, M={M}: {desc}")
    y = y_host(mxq.mxq_qmv(x, w, s, b, bits=8, group_size=64))
    blk = rows % BIG_P
    ref = oracle.matmul_ref_rows(xs, p.w, p.scales, p.biases, blk, BIG_K, 8, 64, "f16")
    assert_close(y[:, rows], ref, f"W over 4 GiB, M={M}")


# ------------------------------------------------------ split workspace ---
def test_split_workspace_release_and_regrowth():
    """The split workspace grows with the call, is reused by smaller calls,
    is freed by mxq_release_workspaces, and is allocated again afterwards;
    results match the oracle and stay bit-identical across the release."""
    small = synth.make_problem(128, 512, 4096, 4, 64, "f16", seed=810)     # 8 splits, 2 MiB
    large = synth.make_problem(256, 1024, 8192, 4, 64, "f16", seed=811)    # 4 splits, 4 MiB
    for p in (small, large):
        assert ",ksplit=" in mxq.mxq_describe("qmm", p.M, p.N, p.K), (p.M, p.N, p.K)
    ds, dl = to_dev(small), to_dev(large)
    note("split workspace: release, then small, large, small")
    mxq.mxq_release_workspaces()
    assert mxq.mxq_workspace_bytes() == 0
    y1 = y_host(mxq.mxq_qmm(*ds, bits=4))
    after_small = mxq.mxq_workspace_bytes()
    assert after_small >= 8 * 128 * 512 * 4
    y2 = y_host(mxq.mxq_qmm(*dl, bits=4))
    after_large = mxq.mxq_workspace_bytes()
    assert after_large >= 4 * 256 * 1024 * 4
    y3 = y_host(mxq.mxq_qmm(*ds, bits=4))
    assert mxq.mxq_workspace_bytes() == after_large  # reused, not grown
    assert np.array_equal(y1.view(np.uint16), y3.view(np.uint16))
    assert_close(y1, _ref(small), "split small")
    cols = np.unique(np.random.default_rng(3).integers(0, large.N, 96))
    ref = oracle.matmul_ref_rows(large.x, large.w, large.scales, large.biases, cols, large.K, 4, 64, "f16")
    assert_close(y2[:, cols], ref, "split large")
    note("split workspace: release after use, call again")
    mxq.mxq_release_workspaces()
    assert mxq.mxq_workspace_bytes() == 0
    y4 = y_host(mxq.mxq_qmm(*dl, bits=4))
    assert np.array_equal(y2.view(np.uint16), y4.view(np.uint16))
    assert mxq.mxq_workspace_bytes() >= 4 * 256 * 1024 * 4


def test_split_workspace_bounded_over_many_streams():
    """Calls on more streams than the cache keeps buffers for: every result
    matches the first stream's bit for bit, and the cached bytes stay bounded
    by four buffers."""
    p = synth.make_problem(128, 512, 4096, 4, 64, "f16", seed=812)
    d = to_dev(p)
    mxq.mxq_release_workspaces()
    note("split workspace: 9 streams")
    want = y_host(mxq.mxq_qmm(*d, bits=4))
    one = mxq.mxq_workspace_bytes()
    streams = [torch.cuda.Stream() for _ in range(8)]
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(st):
            outs.append(mxq.mxq_qmm(*d, bits=4, stream=st))
        assert mxq.mxq_workspace_bytes() <= 4 * one
    torch.cuda.synchronize()
    for y in outs:
        assert np.array_equal(y.cpu().numpy().view(np.uint16), want.view(np.uint16))
    mxq.mxq_release_workspaces()
