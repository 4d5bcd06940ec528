"""libmxq C ABI on the CPU: symbols, host packer, and argument validation.

Nothing here launches a kernel: every fused/dequant call below is rejected by
the library's synchronous validation before any HIP call.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import dequant_matmul_qmv_amd as mxq
import oracle
from tests import pins

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "mxq.h")).read()
    return sorted(set(re.findall(r"^\s*(?:mxq_status|const char\*|int|int64_t)\s+(mxq_\w+)\s*\(", text, re.M)))


def test_header_symbols_exported():
    lib = mxq.load()
    names = _header_functions()
    assert {"mxq_qmv", "mxq_qmm", "mxq_dequant", "mxq_pack", "mxq_status_str",
            "mxq_last_error", "mxq_abi_version"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.mxq_abi_version() == 4


def test_describe_without_device_or_with_bad_args():
    lib = mxq.load()
    assert lib.mxq_describe(b"qmv", 1, 4, 48, 4, 64, 0) == b"invalid"
    assert lib.mxq_describe(b"nope", 1, 4, 64, 4, 64, 0) == b"invalid"
    assert lib.mxq_describe(b"a8", 3, 4, 48, 4, 64, 0) == b"invalid"   # K not a multiple of the group
    # valid arguments for every op, no GPU in this process: no device
    for op in (b"qmv", b"qmm", b"a8"):
        d = lib.mxq_describe(op, 3, 8192, 2048, 4, 64, 0)
        assert d in (b"no device",) or d.startswith((b"q", b"qsmk")), (op, d)


def test_status_strings():
    lib = mxq.load()
    assert lib.mxq_status_str(0) == b"MXQ_OK"
    assert lib.mxq_status_str(3) == b"MXQ_ERR_MISALIGNED"
    assert lib.mxq_status_str(99) == b"MXQ_ERR_UNKNOWN"


def test_pack_hand_words():
    assert mxq.mxq_pack(np.array([[0, 1, 2, 3, 4, 5, 6, 7]], np.uint8), 4)[0, 0] == 0x76543210
    assert mxq.mxq_pack(np.array([[15, 0, 0, 0, 0, 0, 0, 1]], np.uint8), 4)[0, 0] == 0x1000000F
    assert mxq.mxq_pack(np.array([[1, 2, 3, 0xAB]], np.uint8), 8)[0, 0] == 0xAB030201


@pytest.mark.parametrize("bits", [4, 8])
def test_pack_round_trip_through_oracle(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 2 ** bits, size=(37, 256), dtype=np.uint8)
    w = mxq.mxq_pack(codes, bits)
    assert w.shape == (37, 256 * bits // 32)
    assert np.array_equal(oracle.unpack_codes(w, 256, bits), codes)
    # and against the bit-string route, for a few words
    for n in (0, 36):
        got = [c for j in range(4) for c in pins.bitstring_unpack(int(w[n, j]), bits)]
        assert got == list(codes[n, :4 * (32 // bits)])


def test_pack_every_value_every_slot():
    for bits in (4, 8):
        per = 32 // bits
        for slot in range(per):
            for v in range(2 ** bits):
                c = np.zeros((1, per), np.uint8)
                c[0, slot] = v
                assert mxq.mxq_pack(c, bits)[0, 0] == v * 2 ** (bits * slot)


def test_pack_rejects_bad_codes():
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_pack(np.array([[16, 0, 0, 0, 0, 0, 0, 0]], np.uint8), 4)
    assert e.value.status == mxq.MXQ_ERR_INVALID_ARG
    with pytest.raises(mxq.MxqError) as e:
        mxq.mxq_pack(np.zeros((1, 6), np.uint8), 4)
    assert e.value.status == mxq.MXQ_ERR_UNSUPPORTED


FAKE = 0x10000  # a 16-byte aligned non-null address; never dereferenced (rejected first)


def _call(name, *args):
    lib = mxq.load()
    st = getattr(lib, name)(*args)
    return st, lib.mxq_last_error().decode()


@pytest.mark.parametrize("name", ["mxq_qmv", "mxq_qmm", "mxq_qmm_noalloc", "mxq_linear", "mxq_linear_act",
                                  "mxq_linear_a8"])
def test_fused_validation(name):
    P = FAKE
    ok = dict(M=1, N=4, K=64, bits=4, gs=64, sb=mxq.MXQ_F16, act=mxq.MXQ_BF16)

    def call(x=P, w=P, s=P, b=P, y=P, **kw):
        a = dict(ok, **kw)
        if name in ("mxq_linear", "mxq_linear_a8"):   # the output bias goes between biases and y
            return _call(name, x, w, s, b, a.get("ob", None), y, a["M"], a["N"], a["K"], a["bits"], a["gs"],
                         a["sb"], None)
        if name == "mxq_linear_act":   # ... and the activation dtype follows the scale dtype
            return _call(name, x, w, s, b, a.get("ob", None), y, a["M"], a["N"], a["K"], a["bits"], a["gs"],
                         a["sb"], a["act"], None)
        return _call(name, x, w, s, b, y, a["M"], a["N"], a["K"], a["bits"], a["gs"], a["sb"], None)

    if name in ("mxq_linear", "mxq_linear_act", "mxq_linear_a8"):
        st, msg = call(ob=P + 1)
        assert st == mxq.MXQ_ERR_MISALIGNED and "out_bias" in msg
    if name == "mxq_linear_act":
        st, msg = call(act=mxq.MXQ_F32)
        assert st == mxq.MXQ_ERR_UNSUPPORTED and "act_dtype" in msg
        assert call(act=9)[0] == mxq.MXQ_ERR_UNSUPPORTED

    assert call(bits=3)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(bits=2)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(gs=48)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(gs=256)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(K=96)[0] == mxq.MXQ_ERR_UNSUPPORTED          # K % group_size != 0
    assert call(sb=mxq.MXQ_F32)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(sb=7)[0] == mxq.MXQ_ERR_UNSUPPORTED
    assert call(M=-1)[0] == mxq.MXQ_ERR_INVALID_ARG
    assert call(N=-5)[0] == mxq.MXQ_ERR_INVALID_ARG
    assert call(x=None)[0] == mxq.MXQ_ERR_INVALID_ARG
    assert call(w=None)[0] == mxq.MXQ_ERR_INVALID_ARG
    assert call(s=None)[0] == mxq.MXQ_ERR_INVALID_ARG
    assert call(y=None)[0] == mxq.MXQ_ERR_INVALID_ARG
    st, msg = call(w=P + 4)
    assert st == mxq.MXQ_ERR_MISALIGNED and "16-byte" in msg
    assert call(x=P + 1)[0] == mxq.MXQ_ERR_MISALIGNED
    assert call(y=P + 1)[0] == mxq.MXQ_ERR_MISALIGNED
    assert call(M=2 ** 31)[0] == mxq.MXQ_ERR_UNSUPPORTED
    # empty problems are no-ops that touch no pointer, even null ones
    assert call(x=None, w=None, s=None, b=None, y=None, M=0)[0] == mxq.MXQ_OK
    assert call(x=None, w=None, s=None, b=None, y=None, N=0)[0] == mxq.MXQ_OK


def test_dequant_validation():
    P = FAKE

    def call(w=P, s=P, b=P, o=P, N=4, K=64, bits=4, gs=64, sb=mxq.MXQ_F16, out=mxq.MXQ_F32):
        return _call("mxq_dequant", w, s, b, o, N, K, bits, gs, sb, out, None)[0]

    assert call(bits=5) == mxq.MXQ_ERR_UNSUPPORTED
    assert call(gs=16) == mxq.MXQ_ERR_UNSUPPORTED
    assert call(K=32) == mxq.MXQ_ERR_UNSUPPORTED
    assert call(out=9) == mxq.MXQ_ERR_UNSUPPORTED
    assert call(sb=mxq.MXQ_F32) == mxq.MXQ_ERR_UNSUPPORTED
    assert call(N=-1) == mxq.MXQ_ERR_INVALID_ARG
    assert call(o=None) == mxq.MXQ_ERR_INVALID_ARG
    assert call(w=P + 8) == mxq.MXQ_ERR_MISALIGNED
    assert call(o=P + 4) == mxq.MXQ_ERR_MISALIGNED
    assert call(s=P + 1) == mxq.MXQ_ERR_MISALIGNED
    assert call(w=None, s=None, b=None, o=None, N=0) == mxq.MXQ_OK


def test_last_error_is_thread_local_and_cleared():
    import threading
    lib = mxq.load()
    lib.mxq_qmv(FAKE, FAKE, FAKE, FAKE, FAKE, 1, 4, 64, 3, 64, 0, None)
    assert b"bits" in lib.mxq_last_error()
    seen = []
    th = threading.Thread(target=lambda: seen.append(lib.mxq_last_error()))
    th.start()
    th.join()
    assert seen == [b""]
    assert lib.mxq_qmv(None, None, None, None, None, 0, 4, 64, 4, 64, 0, None) == 0
    assert lib.mxq_last_error() == b""


def test_product_path_does_not_import_oracle():
    """The product package never imports the oracle (they share no code)."""
    pkg = os.path.join(ROOT, "dequant_matmul_qmv_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("mlxcel", ""), f


def test_grouped_validation():
    lib = mxq.load()
    P = FAKE
    Q = mxq.QmvProblem
    good = Q(P, P, P, P, P, 4, 64)
    arr = (Q * 3)(good, good, Q(P, P + 4, P, P, P, 4, 64))
    assert lib.mxq_qmv_grouped(arr, 3, 1, 4, 64, 0, None) == mxq.MXQ_ERR_MISALIGNED
    assert b"mxq_qmv_grouped[2]" in lib.mxq_last_error()
    arr = (Q * 2)(good, Q(P, P, P, P, P, 4, 96))
    assert lib.mxq_qmv_grouped(arr, 2, 1, 4, 64, 0, None) == mxq.MXQ_ERR_UNSUPPORTED
    arr = (Q * 1)(good)
    assert lib.mxq_qmv_grouped(arr, 1, 1, 5, 64, 0, None) == mxq.MXQ_ERR_UNSUPPORTED
    assert lib.mxq_qmv_grouped(arr, -1, 1, 4, 64, 0, None) == mxq.MXQ_ERR_INVALID_ARG
    assert lib.mxq_qmv_grouped(None, 2, 1, 4, 64, 0, None) == mxq.MXQ_ERR_INVALID_ARG
    assert lib.mxq_qmv_grouped(None, 0, 1, 4, 64, 0, None) == mxq.MXQ_OK
    empty = (Q * 2)(Q(None, None, None, None, None, 0, 64), Q(None, None, None, None, None, 0, 0))
    assert lib.mxq_qmv_grouped(empty, 2, 1, 4, 64, 0, None) == mxq.MXQ_OK


def test_describe_grouped_without_device_or_with_bad_args():
    lib = mxq.load()
    Q = mxq.QmvProblem
    arr = (Q * 2)(Q(None, None, None, None, None, 2048, 2048), Q(None, None, None, None, None, 512, 2048))
    assert lib.mxq_describe_grouped(arr, 2, 1, 4, 64, 0) in (b"no device",) or \
        lib.mxq_describe_grouped(arr, 2, 1, 4, 64, 0).startswith(b"qmv_kernel")
    assert lib.mxq_describe_grouped(arr, 0, 1, 4, 64, 0) == b"invalid"
    assert lib.mxq_describe_grouped(arr, 2, 0, 4, 64, 0) == b"invalid"
    assert lib.mxq_describe_grouped(arr, 2, 1, 5, 64, 0) == b"invalid"
    assert lib.mxq_describe_grouped(None, 2, 1, 4, 64, 0) == b"invalid"
    bad = (Q * 1)(Q(None, None, None, None, None, 4, 96))   # K not a multiple of the group
    assert lib.mxq_describe_grouped(bad, 1, 1, 4, 64, 0) == b"invalid"
    empty = (Q * 2)(Q(None, None, None, None, None, 0, 64), Q(None, None, None, None, None, 8, 0))
    assert lib.mxq_describe_grouped(empty, 2, 1, 4, 64, 0) == b"none"


def test_read_probe_validation():
    lib = mxq.load()
    assert lib.mxq_read_probe(FAKE, 24, FAKE, None) == mxq.MXQ_ERR_INVALID_ARG
    assert lib.mxq_read_probe(FAKE, -16, FAKE, None) == mxq.MXQ_ERR_INVALID_ARG
    assert lib.mxq_read_probe(None, 32, FAKE, None) == mxq.MXQ_ERR_INVALID_ARG
    assert lib.mxq_read_probe(FAKE + 8, 32, FAKE, None) == mxq.MXQ_ERR_MISALIGNED
    assert lib.mxq_read_probe(FAKE, 32, FAKE + 2, None) == mxq.MXQ_ERR_MISALIGNED
    assert lib.mxq_read_probe(None, 0, None, None) == mxq.MXQ_OK


def test_workspace_controls_without_device():
    lib = mxq.load()
    assert lib.mxq_release_workspaces() == mxq.MXQ_OK
    assert lib.mxq_workspace_bytes() == 0
