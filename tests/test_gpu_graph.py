"""libmxq launches captured in a HIP graph: every replay equals the eager result.

The graph is replayed several times with new inputs copied into the captured
buffers between replays (eager work and synchronisation in between), and each
replay is compared bit for bit with an eager call on the same inputs.
"""

import numpy as np
import pytest
import torch

import dequant_matmul_qmv_amd as mxq
import synth
from tests.gpu_util import note, to_dev

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    dev = "cuda:0"
    pv = synth.make_problem(1, 3000, 2048, 4, 64, "f16", seed=61)
    pm = synth.make_problem(80, 500, 1024, 8, 64, "bf16", seed=62)
    # 1 x 4 tiles of 128 x 128 and 64 stages: the split-K path, whose workspace
    # comes from the stream-ordered pool inside the captured graph
    ps = synth.make_problem(128, 512, 4096, 4, 64, "f16", seed=63)
    assert mxq.mxq_describe("qmm", 128, 512, 4096, 4, 64, "f16").startswith(
        "qmm_kernel<bits=4,sb=f16,gs=64,tile=128x128,ksplit=")
    xv, wv, sv, bv = to_dev(pv)
    xm, wm, sm, bm = to_dev(pm)
    xs, ws, ss, bs = to_dev(ps)
    yv = torch.empty((1, 3000), dtype=torch.float16, device=dev)
    ym = torch.empty((80, 500), dtype=torch.float16, device=dev)
    ys = torch.empty((128, 512), dtype=torch.float16, device=dev)
    dq = torch.empty((500, 1024), dtype=torch.float32, device=dev)

    def work():
        mxq.mxq_qmv(xv, wv, sv, bv, yv, bits=4)
        mxq.mxq_qmm(xm, wm, sm, bm, ym, bits=8)
        mxq.mxq_qmm(xs, ws, ss, bs, ys, bits=4)
        mxq.mxq_dequant(wm, sm, bm, dq, bits=8)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph capture of qmv + qmm + dequant")
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    rng = np.random.default_rng(5)
    for rep in range(4):
        new_xv = torch.from_numpy(rng.standard_normal((1, 2048)).astype(np.float16)).to(dev)
        new_xm = torch.from_numpy(rng.standard_normal((80, 1024)).astype(np.float16)).to(dev)
        new_xs = torch.from_numpy(rng.standard_normal((128, 4096)).astype(np.float16)).to(dev)
        xv.copy_(new_xv)
        xm.copy_(new_xm)
        xs.copy_(new_xs)
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got_v, got_m, got_s, got_d = yv.clone(), ym.clone(), ys.clone(), dq.clone()
        ev = mxq.mxq_qmv(new_xv, wv, sv, bv, bits=4)
        em = mxq.mxq_qmm(new_xm, wm, sm, bm, bits=8)
        es = mxq.mxq_qmm(new_xs, ws, ss, bs, bits=4)
        ed = mxq.mxq_dequant(wm, sm, bm, bits=8)
        torch.cuda.synchronize()
        assert torch.equal(got_v.view(torch.int16), ev.view(torch.int16)), rep
        assert torch.equal(got_m.view(torch.int16), em.view(torch.int16)), rep
        assert torch.equal(got_s.view(torch.int16), es.view(torch.int16)), rep
        assert torch.equal(got_d.view(torch.int32), ed.view(torch.int32)), rep


def test_graph_replay_few_rows_and_dequant_layouts():
    """The K-split few-row kernel and the dequant kernel's f16 and f32 outputs
    under graph replay, each replay equal to an eager call bit for bit."""
    dev = "cuda:0"
    pk = synth.make_problem(6, 8192, 2048, 4, 64, "f16", seed=64)
    assert mxq.mxq_describe("qmv", 6, 8192, 2048, 4, 64, "f16").startswith("qsmk_kernel")
    pd = synth.make_problem(1, 700, 2048, 4, 128, "bf16", seed=65)
    xk, wk, sk, bk = to_dev(pk)
    _, wd, sd, bd = to_dev(pd)
    yk = torch.empty((6, 8192), dtype=torch.float16, device=dev)
    d16 = torch.empty((700, 2048), dtype=torch.float16, device=dev)
    d32 = torch.empty((700, 2048), dtype=torch.float32, device=dev)

    def work():
        mxq.mxq_qmv(xk, wk, sk, bk, yk, bits=4)
        mxq.mxq_dequant(wd, sd, bd, d16, bits=4, group_size=128, out_dtype=torch.float16)
        mxq.mxq_dequant(wd, sd, bd, d32, bits=4, group_size=128)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        work()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    note("graph capture of qsmk + dequant f16/f32")
    with torch.cuda.graph(g):
        work()
    torch.cuda.synchronize()

    rng = np.random.default_rng(6)
    for rep in range(3):
        new_x = torch.from_numpy(rng.standard_normal((6, 2048)).astype(np.float16)).to(dev)
        xk.copy_(new_x)
        d16.zero_()
        d32.zero_()
        torch.cuda.synchronize()
        note(f"graph replay {rep}")
        g.replay()
        torch.cuda.synchronize()
        got_k, got_16, got_32 = yk.clone(), d16.clone(), d32.clone()
        ek = mxq.mxq_qmv(new_x, wk, sk, bk, bits=4)
        e16 = mxq.mxq_dequant(wd, sd, bd, bits=4, group_size=128, out_dtype=torch.float16)
        e32 = mxq.mxq_dequant(wd, sd, bd, bits=4, group_size=128)
        torch.cuda.synchronize()
        assert torch.equal(got_k.view(torch.int16), ek.view(torch.int16)), rep
        assert torch.equal(got_16.view(torch.int16), e16.view(torch.int16)), rep
        assert torch.equal(got_32.view(torch.int32), e32.view(torch.int32)), rep


def test_describe_on_device():
    d = mxq.mxq_describe("qmv", 1, 128256, 2048, 4, 64, "f16")
    assert d.startswith("qmv_kernel<bits=4,sb=f16,mt=1,rows=4"), d
    d = mxq.mxq_describe("qmv", 20, 100, 2048, 8, 64, "bf16")
    assert d.count("qmv_kernel") == 3, d          # M=20 -> slices of 8, 8, 4
    d = mxq.mxq_describe("qmm", 512, 8192, 2048, 4, 64, "f16")
    assert d.startswith("qmm_kernel<bits=4,sb=f16,gs=64,tile=128x128> grid=256 block=512"), d
    d = mxq.mxq_describe("qmm", 512, 2048, 8192, 4, 64, "f16")
    assert d.startswith("qmm_kernel<bits=4,sb=f16,gs=64,tile=128x128,ksplit=4> grid=256 block=512"), d
    d = mxq.mxq_describe("qmm", 64, 256, 256, 4, 64, "f16")   # too few stages to split
    assert d.startswith("qmm_kernel<bits=4,sb=f16,gs=64,tile=64x64> grid=4 block=512"), d
    assert mxq.mxq_describe("qmm", 4, 100, 2048, 4, 64, "f16").startswith("qmv_kernel")
