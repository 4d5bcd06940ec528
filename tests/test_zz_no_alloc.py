"""mxq_qmm_noalloc (the entry point that allocates no device memory) against
mxq_qmm through the C ABI: two calls in a row, the second smaller, on each
route that needs scratch (split K on the matrix cores, K chunks on the
few-row kernel) and on one that needs none; outputs bit-identical to
mxq_qmm's and within 2e-3 (1 + |y_ref|) of the f64 oracle on sampled columns.
A call needing more scratch than the fixed array holds is rejected.
"""

import ctypes

import numpy as np
import pytest
import torch

import dequant_matmul_qmv_amd as mxq
import oracle
import synth
from tests.gpu_util import assert_close, note, to_dev

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 32 << 20


def _abi_call(name, p, dev_in, y):
    lib = mxq.load()
    x, w, s, b = dev_in
    st = getattr(lib, name)(x.data_ptr(), w.data_ptr(), s.data_ptr(), b.data_ptr(), y.data_ptr(),
                            p.M, p.N, p.K, p.bits, p.group_size, 0 if p.sb_dtype == "f16" else 1,
                            ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, lib.mxq_last_error().decode()


def _check_pair(p, tag):
    d = to_dev(p)
    y_ref_path = torch.empty((p.M, p.N), dtype=torch.float16, device="cuda")
    y_new = torch.full((p.M, p.N), 7.0, dtype=torch.float16, device="cuda")
    note(f"no-alloc {tag}: M={p.M} N={p.N} K={p.K} bits={p.bits} -> {mxq.mxq_describe('qmm', p.M, p.N, p.K, p.bits)}")
    st, msg = _abi_call("mxq_qmm", p, d, y_ref_path)
    assert st == mxq.MXQ_OK, msg
    st, msg = _abi_call("mxq_qmm_noalloc", p, d, y_new)
    assert st == mxq.MXQ_OK, msg
    torch.cuda.synchronize()
    a, b = y_ref_path.cpu().numpy(), y_new.cpu().numpy()
    assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"{tag}: differs from mxq_qmm"
    cols = np.unique(np.concatenate([[0, p.N - 1], np.random.default_rng(p.N).integers(0, p.N, 128)]))
    ref = oracle.matmul_ref_rows(p.x, p.w, p.scales, p.biases, cols, p.K, p.bits, p.group_size, p.sb_dtype)
    assert_close(b[:, cols], ref, f"no-alloc {tag}")


@pytest.mark.parametrize("route", ["split_k", "k_chunks", "ragged_k_chunks", "no_scratch"])
def test_noalloc_matches_qmm_twice_second_smaller(route):
    if route == "split_k":      # 4 splits x 512 x 2048 floats = 16 MiB, then 8 x 128 x 512 = 2 MiB
        first = synth.make_problem(512, 2048, 8192, 4, 64, "f16", seed=901)
        second = synth.make_problem(128, 512, 4096, 8, 64, "bf16", seed=902)
        for p in (first, second):
            assert ",ksplit=" in mxq.mxq_describe("qmm", p.M, p.N, p.K, p.bits, p.group_size, p.sb_dtype)
    elif route == "k_chunks":   # 2 chunks x 8 x 65536 floats = 4 MiB, then 2 x 3 x 8192 = 192 KiB
        first = synth.make_problem(8, 65536, 8192, 4, 64, "f16", seed=903)
        second = synth.make_problem(3, 8192, 8192, 4, 128, "bf16", seed=904)
        for p in (first, second):
            assert "kchunks=" in mxq.mxq_describe("qmm", p.M, p.N, p.K, p.bits, p.group_size, p.sb_dtype)
    elif route == "ragged_k_chunks":  # K not a multiple of 512, in chunks: 2 x 8 x 8192, then 3 x 5 x 4100 floats
        first = synth.make_problem(8, 8192, 4160, 4, 64, "f16", seed=907)
        second = synth.make_problem(5, 4100, 9024, 8, 64, "bf16", seed=908)
        for p in (first, second):
            d = mxq.mxq_describe("qmm", p.M, p.N, p.K, p.bits, p.group_size, p.sb_dtype)
            assert "kchunks=" in d and ",ragged" in d, d
    else:                       # tiles alone fill the GPU: no scratch at all
        first = synth.make_problem(512, 8192, 2048, 4, 64, "f16", seed=905)
        second = synth.make_problem(200, 4096, 1024, 8, 64, "f16", seed=906)
        assert ",ksplit=" not in mxq.mxq_describe("qmm", 512, 8192, 2048)
    _check_pair(first, f"{route} first")
    _check_pair(second, f"{route} second (smaller)")


def test_noalloc_rejects_scratch_beyond_its_size():
    """16 rows at K = 8192 on 300,000 rows of W would need 2 chunks x 16 x
    300,000 x 4 bytes (38.4 MB) of scratch: rejected before any launch."""
    p = synth.make_problem(16, 8, 8192, 4, 64, "f16", seed=907)
    N = 300000
    assert "kchunks=2" in mxq.mxq_describe("qmm", 16, N, 8192)
    need = 2 * 16 * N * 4
    assert need > SCRATCH_BYTES
    x = torch.from_numpy(p.x).cuda()
    w = torch.zeros((N, 8192 // 8), dtype=torch.int32, device="cuda")
    s = torch.zeros((N, 8192 // 64), dtype=torch.float16, device="cuda")
    y = torch.zeros((16, N), dtype=torch.float16, device="cuda")
    lib = mxq.load()
    note("no-alloc: scratch need beyond the fixed size")
    st = lib.mxq_qmm_noalloc(x.data_ptr(), w.data_ptr(), s.data_ptr(), s.data_ptr(), y.data_ptr(), 16, N, 8192, 4,
                             64, 0, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == mxq.MXQ_ERR_UNSUPPORTED
    assert str(need) in lib.mxq_last_error().decode()
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(y)) == 0  # nothing was enqueued
