"""The C ABI on the host: libnvfp4.so loads, exports every function that
include/nvfp4.h declares, and rejects invalid requests before touching a device.
No GPU: no call here gets past argument validation (the pointers are fakes).
"""

import ctypes
import os
import re

import pytest
import torch

from moe_nvfp4_quantize_amd import nvfp4 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails first
INVALID = B.NVFP4_ERR_INVALID_ARG


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("libnvfp4.so not built (run __graft_entry__.build())")
    return B.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for core in ("nvfp4_quantize", "nvfp4_gemm", "nvfp4_moe_grouped_gemm", "nvfp4_moe_route",
                 "nvfp4_moe_combine", "nvfp4_quantize_batched"):
        assert core in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(B.SIGNATURES), "binding and header disagree"


def test_abi_version_and_status_strings(lib):
    assert lib.nvfp4_abi_version() == 1
    for st in range(4):
        assert B.status_string(st).startswith("NVFP4")
    assert "unknown" in B.status_string(99)


def test_workspace_sizes(lib):
    base = lib.nvfp4_quantize_workspace_size(0, 16) - 256  # grid-barrier state
    assert base >= 16 + 4 * 1024 and base % 256 == 0
    assert lib.nvfp4_quantize_workspace_size(8192, 5120) == base + 1024
    assert lib.nvfp4_quantize_workspace_size(4, 15) == 0
    assert lib.nvfp4_quantize_batched_workspace_size(512, 2048, 4096) == 512 * 1024
    assert lib.nvfp4_moe_route_workspace_size(8192, 512, 10) >= 128 * 512 * 4


def _q(lib, **kw):
    a = dict(x=FAKE, t=B.NVFP4_BF16, rows=4, cols=32, ld=32, q=FAKE, s=FAKE, g=FAKE, static=0,
             ws=FAKE, wsb=4096)
    a.update(kw)
    return lib.nvfp4_quantize(a["x"], a["t"], a["rows"], a["cols"], a["ld"], a["q"], a["s"], a["g"],
                              a["static"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("bad", [
    dict(cols=24), dict(cols=0), dict(rows=-1), dict(ld=16), dict(t=7), dict(x=None),
    dict(q=None), dict(s=None), dict(g=None), dict(ws=None), dict(wsb=8),
    dict(ws=ctypes.c_void_p(0x1001)), dict(ws=ctypes.c_void_p(0x1080)), dict(rows=2 ** 31, cols=16),
])
def test_quantize_rejects(lib, bad):
    assert _q(lib, **bad) == INVALID


def test_quantize_static_empty_is_noop(lib):
    assert _q(lib, rows=0, x=None, q=None, s=None, static=1, ws=None, wsb=0) == B.NVFP4_OK


def _gemm(lib, **kw):
    a = dict(aq=FAKE, as_=FAKE, ag=FAKE, bq=FAKE, bs=FAKE, bg=FAKE, M=4, N=8, K=64, c=FAKE,
             t=B.NVFP4_F32, ldc=8)
    a.update(kw)
    return lib.nvfp4_gemm(a["aq"], a["as_"], a["ag"], a["bq"], a["bs"], a["bg"], a["M"], a["N"],
                          a["K"], a["c"], a["t"], a["ldc"], None)


@pytest.mark.parametrize("bad", [
    dict(K=24), dict(K=0), dict(M=-1), dict(ldc=4), dict(t=5), dict(aq=None), dict(bs=None),
    dict(ag=None), dict(c=None), dict(N=2 ** 31),
])
def test_gemm_rejects(lib, bad):
    assert _gemm(lib, **bad) == INVALID


def test_gemm_empty_is_noop(lib):
    assert _gemm(lib, M=0, aq=None, c=None) == B.NVFP4_OK


def test_route_rejects(lib):
    f = lib.nvfp4_moe_route
    ok = dict(lg=FAKE, T=16, E=8, k=2, ids=FAKE, w=FAKE, off=FAKE, src=FAKE, inv=FAKE, ws=FAKE,
              wsb=1 << 20)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["lg"], a["T"], a["E"], a["k"], a["ids"], a["w"], a["off"], a["src"], a["inv"],
                 a["ws"], a["wsb"], None)
    for bad in [dict(k=0), dict(k=9), dict(k=33, E=64), dict(E=1025), dict(E=0), dict(T=-1),
                dict(lg=None), dict(off=None), dict(ws=None), dict(wsb=4), dict(inv=None)]:
        assert call(**bad) == INVALID, bad


def test_grouped_gemm_rejects(lib):
    f = lib.nvfp4_moe_grouped_gemm
    ok = dict(aq=FAKE, as_=FAKE, ag=FAKE, arows=64, src=FAKE, off=FAKE, E=4, R=64, wq=FAKE, ws=FAKE,
              wg=FAKE, N=32, K=64, c=FAKE, t=B.NVFP4_F32, epi=B.NVFP4_EPI_NONE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["aq"], a["as_"], a["ag"], a["arows"], a["src"], a["off"], a["E"], a["R"], a["wq"],
                 a["ws"], a["wg"], a["N"], a["K"], a["c"], a["t"], a["epi"], None)
    for bad in [dict(K=8), dict(E=0), dict(N=0), dict(R=-1), dict(epi=2),
                dict(epi=B.NVFP4_EPI_SILU_GATE, N=33), dict(off=None), dict(wg=None), dict(c=None),
                dict(src=None, arows=8), dict(arows=0), dict(t=3)]:
        assert call(**bad) == INVALID, bad
    assert call(R=0, aq=None) == B.NVFP4_OK


def test_grouped_silu_nvfp4_rejects(lib):
    f = lib.nvfp4_moe_grouped_gemm_silu_nvfp4
    ok = dict(aq=FAKE, as_=FAKE, ag=FAKE, arows=64, src=FAKE, off=FAKE, E=4, R=64, wq=FAKE, ws=FAKE,
              wg=FAKE, N=64, K=256, hq=FAKE, hs=FAKE, hg=FAKE)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["aq"], a["as_"], a["ag"], a["arows"], a["src"], a["off"], a["E"], a["R"], a["wq"],
                 a["ws"], a["wg"], a["N"], a["K"], a["hq"], a["hs"], a["hg"], None)
    for bad in [dict(K=8), dict(E=0), dict(N=0), dict(N=48), dict(R=-1), dict(hq=None),
                dict(hs=None), dict(hg=None), dict(off=None), dict(src=None, arows=8), dict(arows=0)]:
        assert call(**bad) == INVALID, bad
    assert call(R=0, aq=None) == B.NVFP4_OK
    # valid, but K % 256 != 0 is not implemented by the fused path
    assert call(K=48) == B.NVFP4_ERR_UNSUPPORTED


def test_combine_rejects(lib):
    f = lib.nvfp4_moe_combine
    ok = dict(y=FAKE, yt=B.NVFP4_F32, w=FAKE, inv=FAKE, T=4, k=2, H=16, R=8, out=FAKE,
              ot=B.NVFP4_BF16)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["y"], a["yt"], a["w"], a["inv"], a["T"], a["k"], a["H"], a["R"], a["out"],
                 a["ot"], None)
    for bad in [dict(k=0), dict(k=33), dict(H=0), dict(R=7), dict(y=None), dict(out=None),
                dict(yt=4), dict(ot=9), dict(T=-2)]:
        assert call(**bad) == INVALID, bad


def test_fp8_quantize_rejects(lib):
    f = lib.nvfp4_fp8_quantize
    assert lib.nvfp4_fp8_quantize_workspace_size(8192, 5120) == lib.nvfp4_quantize_workspace_size(8192, 5120)
    ok = dict(x=FAKE, t=B.NVFP4_BF16, rows=4, cols=32, ld=32, q=FAKE, g=FAKE, static=0, ws=FAKE, wsb=4096)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["x"], a["t"], a["rows"], a["cols"], a["ld"], a["q"], a["g"], a["static"], a["ws"],
                 a["wsb"], None)
    for bad in [dict(cols=24), dict(cols=0), dict(rows=-1), dict(ld=16), dict(t=7), dict(x=None),
                dict(q=None), dict(q=ctypes.c_void_p(0x1008)), dict(g=None), dict(ws=None), dict(wsb=8),
                dict(ws=ctypes.c_void_p(0x1080)), dict(rows=2 ** 31, cols=16)]:
        assert call(**bad) == INVALID, bad
    assert call(rows=0, x=None, q=None, static=1, ws=None, wsb=0) == B.NVFP4_OK


def test_fp8_gemm_rejects(lib):
    f = lib.nvfp4_fp8_gemm
    ok = dict(aq=FAKE, ag=FAKE, bq=FAKE, bg=FAKE, M=4, N=8, K=64, c=FAKE, t=B.NVFP4_F32, ldc=8)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["aq"], a["ag"], a["bq"], a["bg"], a["M"], a["N"], a["K"], a["c"], a["t"], a["ldc"], None)
    for bad in [dict(K=24), dict(K=0), dict(M=-1), dict(ldc=4), dict(t=5), dict(aq=None), dict(bg=None),
                dict(c=None), dict(N=2 ** 31), dict(bq=ctypes.c_void_p(0x1004))]:
        assert call(**bad) == INVALID, bad
    assert call(M=0, aq=None, c=None) == B.NVFP4_OK


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device error path")
def test_valid_request_without_device_reports_hip_error(lib):
    # arguments pass validation; the device check then fails on a machine with no GPU
    assert _gemm(lib) in (B.NVFP4_ERR_HIP, B.NVFP4_ERR_UNSUPPORTED)


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    with pytest.raises(RuntimeError, match="no fallback"):
        B.load_library(str(tmp_path / "missing.so"))
