"""The C ABI without a GPU: the library loads, exports what include/rnq.h declares,
and rejects bad arguments before launching anything."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

import fp8_quant_amd as rnq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    if not os.path.exists(rnq.library_path()):
        pytest.skip("librnq.so not built (run `python -m fp8_quant_amd.build`)")
    return rnq.load_library()


def _declared_functions():
    names = set()
    for h in ("rnq.h", "rnq_baselines.h"):
        text = open(os.path.join(ROOT, "include", h)).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names |= set(re.findall(r"\b(rnq_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for must in ("rnq_rmsnorm_fwd", "rnq_rmsnorm_bwd", "rnq_rmsnorm_rope", "rnq_qk_norm_rope_fp8"):
        assert must in names
    assert set(names) == set(rnq.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = _lib()
    assert lib.rnq_abi_version() == 100
    for s, key in enumerate(["RNQ_OK", "NULL", "SHAPE", "UNSUPPORTED", "ARG", "WORKSPACE", "HIP"]):
        assert key in lib.rnq_status_string(s).decode()
    assert b"UNKNOWN" in lib.rnq_status_string(99)


def _qk(lib, **kw):
    a = dict(q=None, k=None, wq=None, wk=None, cos=None, sin=None, q8=None, k8=None, qs=None, ks=None,
             qy=None, ky=None, T=4, Hq=2, Hk=1, D=128, R=128, eps=1e-6, fp8_max=448.0, dt=0)
    a.update(kw)
    return lib.rnq_qk_norm_rope_fp8(a["q"], a["k"], a["wq"], a["wk"], a["cos"], a["sin"], a["q8"], a["k8"],
                                    a["qs"], a["ks"], a["qy"], a["ky"], a["T"], a["Hq"], a["Hk"], a["D"],
                                    a["R"], a["eps"], a["fp8_max"], a["dt"], None)


FAKE = ctypes.c_void_p(0x10000)  # never dereferenced: validation fails before any launch


def test_error_messages_are_per_thread():
    """rnq_last_error is thread-local: two threads that fail at the same time on
    different arguments each read their own message (the library keeps no
    shared mutable state)."""
    import threading

    lib = _lib()
    gate = threading.Barrier(2)
    seen = {}

    def worker(name, kw):
        st = _qk(lib, **kw)
        gate.wait()  # both calls have failed before either reads its message
        seen[name] = (st, lib.rnq_last_error().decode())

    threads = [threading.Thread(target=worker, args=("null", {})),
               threading.Thread(target=worker, args=("odd", dict(q=FAKE, R=63)))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    assert seen["null"][0] == 1 and seen["odd"][0] == 2
    assert seen["null"][1] != seen["odd"][1]
    assert "rope" in seen["odd"][1].lower() and "rope" not in seen["null"][1].lower()


def test_qk_argument_validation():
    lib = _lib()
    assert _qk(lib) == 1  # NULL pointers
    assert _qk(lib, T=0) == 0  # no rows: OK, nothing launched
    assert _qk(lib, T=-1) == 2
    assert _qk(lib, R=63) == 2  # odd rope_dim
    assert _qk(lib, R=256) == 2  # rope wider than the row
    assert _qk(lib, R=40) == 3  # even but not whole chunks
    assert _qk(lib, D=96, R=32) == 3  # width not built
    assert _qk(lib, fp8_max=500.0) == 4
    assert _qk(lib, fp8_max=0.0) == 4
    assert _qk(lib, eps=-1.0) == 4
    assert _qk(lib, eps=float("nan")) == 4
    assert _qk(lib, dt=7) == 4
    assert _qk(lib, T=1 << 30, Hq=4, Hk=4) == 3  # rows beyond 2^31
    full = dict(q=FAKE, k=FAKE, wq=FAKE, wk=FAKE, cos=FAKE, sin=FAKE, q8=FAKE, k8=FAKE, qs=FAKE, ks=FAKE)
    assert _qk(lib, **{**full, "k": None}) == 1  # kv heads need k
    assert _qk(lib, **{**full, "cos": None}) == 1  # rope needs the table
    assert _qk(lib, **{**full, "q": ctypes.c_void_p(0x10008)}) == 3  # misaligned
    assert _qk(lib, **{**full, "qs": ctypes.c_void_p(0x10002)}) == 3
    assert b"aligned" in lib.rnq_last_error()


def test_rmsnorm_argument_validation():
    lib = _lib()
    assert lib.rnq_rmsnorm_fwd(None, None, None, None, 4, 4096, 1e-6, 0, None) == 1
    assert lib.rnq_rmsnorm_fwd(None, None, None, None, 0, 4096, 1e-6, 0, None) == 0
    assert lib.rnq_rmsnorm_fwd(FAKE, FAKE, FAKE, None, 4, 4100, 1e-6, 0, None) == 3
    assert lib.rnq_rmsnorm_fwd(FAKE, FAKE, FAKE, None, 4, 32768, 1e-6, 0, None) == 3
    assert lib.rnq_rmsnorm_fwd(FAKE, FAKE, FAKE, None, -4, 4096, 1e-6, 0, None) == 2
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 6, 128, 64, 4, 1e-6, 0, None) == 2
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, None, None, FAKE, 6, 128, 64, 1, 1e-6, 0, None) == 1
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 6, 4100, 64, 1, 1e-6, 0, None) == 3  # not whole chunks
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 6, 16392, 64, 1, 1e-6, 0, None) == 3  # too wide
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, FAKE, FAKE, FAKE, 6, 4096, 2048, 1, 1e-6, 0, None) == 3  # tail > 1024
    assert lib.rnq_rmsnorm_rope(FAKE, FAKE, None, None, FAKE, 6, 4096, 64, 1, 1e-6, 0, None) == 1  # wide rows, no table
    need = lib.rnq_rmsnorm_bwd_workspace_size(4096, 4096)
    assert need == 512 * 4096 * 4  # 512 blocks of 8 rows: the RoPE backward with a tail above 512 columns
    assert lib.rnq_rmsnorm_bwd_workspace_size(16384, 4096) == 256 * 4096 * 4
    assert lib.rnq_rmsnorm_bwd_workspace_size(257, 1024) == 257 * 1024 * 4  # one row per block (RoPE partition)
    assert lib.rnq_rmsnorm_bwd_workspace_size(0, 4096) == 0
    assert lib.rnq_rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, need - 1, 4096, 4096, 1e-6, 0, None) == 5
    assert lib.rnq_rmsnorm_bwd(FAKE, FAKE, FAKE, None, FAKE, FAKE, None, need, 4096, 4096, 1e-6, 0, None) == 5
    assert lib.rnq_rmsnorm_bwd(FAKE, FAKE, None, None, FAKE, FAKE, FAKE, need, 4096, 4096, 1e-6, 0, None) == 1


def test_binding_refuses_cpu_tensors():
    import torch

    _lib()
    x = torch.zeros(4, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        rnq.rmsnorm(x, torch.zeros(128, dtype=torch.bfloat16))


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(rnq, "_lib", None)
    monkeypatch.setenv("RNQ_LIBRARY", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="not built"):
        rnq.load_library()


def test_grouped_argument_validation():
    lib = _lib()

    def call(x=FAKE, cos=FAKE, codes=FAKE, scales=FAKE, M=4, N=4096, R=128, rpt=1, g=128, eps=1e-6, fmax=448.0):
        return lib.rnq_rmsnorm_rope_fp8_grouped(x, FAKE, cos, cos, None, codes, scales, M, N, R, rpt, g, eps, fmax,
                                                0, None)

    assert call(x=None) == 1
    assert call(scales=None) == 1
    assert call(cos=None) == 1
    assert call(M=0, x=None) == 0  # zero rows: nothing launched, no pointer checked
    assert call(M=-1) == 2
    assert call(g=96) == 2  # does not divide 4096
    assert call(N=384, g=48) == 3  # divides, not a power of two
    assert call(N=8192, g=1024) == 3  # above 512
    assert call(N=4096, g=4) == 3  # below 8
    assert call(N=16392, g=8) == 3  # row too wide
    assert call(N=4100, g=4100, R=0) == 3  # one group per row, but N is not a multiple of 8
    assert call(N=4104, g=4104, R=0, M=0) == 0  # one group per row of any width (nothing to launch)
    assert call(R=2048) == 3  # rope tail above 1024
    assert call(R=24) == 3  # not a multiple of 16
    assert call(R=130) == 3
    assert call(R=131) == 2  # odd
    assert call(M=6, rpt=4) == 2  # rows not a multiple of rows_per_token
    assert call(rpt=0) == 2
    assert call(fmax=500.0) == 4
    assert call(eps=-1.0) == 4
    assert call(N=384, g=48) == 3 and b"power of two" in lib.rnq_last_error()


def test_rope_bwd_argument_validation():
    lib = _lib()
    need = lib.rnq_rmsnorm_bwd_workspace_size(4096, 128)

    def call(x=FAKE, cos=FAKE, ws=FAKE, wsb=need, M=4096, N=128, R=64, rpt=1, eps=1e-6, dt=0):
        return lib.rnq_rmsnorm_rope_bwd(x, FAKE, FAKE, cos, cos, None, FAKE, FAKE, ws, wsb, M, N, R, rpt, eps, dt,
                                        None)

    assert call(x=None) == 1
    assert call(cos=None) == 1
    assert call(M=0, x=None) == 0
    assert call(N=4096, R=2048) == 3  # tails above 1024 only on rows of 64..512
    assert call(N=4100, R=0) == 3
    assert call(R=24) == 3
    assert call(R=63) == 2
    assert call(R=256) == 2  # wider than the row
    assert call(M=4095, rpt=2) == 2
    assert call(rpt=0) == 2
    assert call(wsb=need - 1) == 5
    assert call(ws=None) == 5
    assert call(eps=float("nan")) == 4
    assert call(dt=7) == 4


def test_noalloc_bwd_argument_validation():
    """The allocation-free backward validates every argument before it looks up its
    static scratch (no HIP call is made for a rejected call)."""
    lib = _lib()

    def call(x=FAKE, cos=FAKE, M=4096, N=128, R=64, rpt=1, eps=1e-6, dt=0, rstd=None):
        return lib.rnq_rmsnorm_rope_bwd_noalloc(x, FAKE, FAKE, cos, cos, rstd, FAKE, FAKE, M, N, R, rpt, eps, dt,
                                                None)

    assert call(x=None) == 1
    assert call(cos=None) == 1
    assert call(M=0, x=None) == 0
    assert call(N=4096, R=2048) == 3
    assert call(N=16392, R=0) == 3  # wider than any row the backward takes
    assert call(R=24) == 3
    assert call(R=63) == 2
    assert call(M=4095, rpt=2) == 2
    assert call(M=-1) == 2
    assert call(eps=-1.0) == 4
    assert call(dt=7) == 4
    assert call(rstd=ctypes.c_void_p(0x10002)) == 3  # rstd must be 4-byte aligned
    # every shape the backward accepts fits the static scratch
    assert lib.rnq_rmsnorm_bwd_workspace_size(8192, 16384) == rnq.RNQ_NOALLOC_SCRATCH_BYTES
    assert lib.rnq_rmsnorm_bwd_workspace_size((1 << 31) - 1, 16384) <= rnq.RNQ_NOALLOC_SCRATCH_BYTES
    assert "RNQ_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)" in open(os.path.join(ROOT, "include", "rnq.h")).read()


def test_autograd_refuses_cpu_tensors():
    torch = pytest.importorskip("torch")
    from fp8_quant_amd import autograd as rag

    if not os.path.exists(rnq.library_path()):
        pytest.skip("librnq.so not built")
    x = torch.randn(4, 128, dtype=torch.bfloat16, requires_grad=True)
    w = torch.ones(128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        rag.rmsnorm(x, w)
    cos = torch.ones(4, 32)
    with pytest.raises(ValueError, match="GPU"):
        rag.rmsnorm_rope(x, w, cos, torch.zeros(4, 32))


def test_strided_entry_validation():
    lib = _lib()
    P = ctypes.c_void_p(0x20000)  # positions (never dereferenced)

    def qk(qs=0, ks=0, pos=None, rows=64, T=64, Hq=32, Hk=8, D=128, R=128):
        return lib.rnq_qk_norm_rope_fp8_ex(FAKE, qs, FAKE, ks, FAKE, FAKE, FAKE, FAKE, pos, rows, FAKE, FAKE,
                                           FAKE, FAKE, None, None, T, Hq, Hk, D, R, 1e-6, 448.0, 0, None)

    assert qk(qs=32 * 128 - 8) == 2  # below the token's rows
    assert qk(qs=48 * 128 + 4) == 3  # not a multiple of 8 elements
    assert qk(ks=8 * 128 - 8) == 2
    assert qk(pos=P, rows=0) == 2  # positions need a table
    assert qk(pos=ctypes.c_void_p(0x20002)) == 3  # positions misaligned
    assert qk(T=0) == 0
    assert lib.rnq_qk_norm_rope_fp8_ex(None, 0, None, 0, FAKE, FAKE, FAKE, FAKE, None, 0, FAKE, None, FAKE, None,
                                       None, None, 4, 1, 0, 128, 64, 1e-6, 448.0, 0, None) == 1

    def nr(xs=0, pos=None, rows=16, M=64, N=128, R=64, rpt=4):
        return lib.rnq_rmsnorm_rope_ex(FAKE, xs, FAKE, FAKE, FAKE, pos, rows, FAKE, M, N, R, rpt, 1e-6, 0, None)

    assert nr(xs=4 * 128 - 8) == 2
    assert nr(xs=4 * 128 + 12) == 3
    assert nr(pos=P, rows=-1) == 2
    assert nr(M=62) == 2
    assert nr(N=4096, R=2048) == 3  # wide rows take tails up to 1024
    assert nr(M=0) == 0


def test_stream_floor_validation():
    lib = _lib()
    f = lib.rnq_baseline_stream
    assert f(FAKE, 1000, FAKE, None) == 2  # not a multiple of 2048
    assert f(FAKE, -2048, FAKE, None) == 2
    assert f(None, 2048, FAKE, None) == 1
    assert f(ctypes.c_void_p(0x10008), 2048, ctypes.c_void_p(0x20000), None) == 3  # src not 16-byte aligned
    assert f(ctypes.c_void_p(0x10000), 4096, ctypes.c_void_p(0x10800), None) == 4  # dst inside src
    g = lib.rnq_baseline_stream_policy
    assert g(FAKE, 2048, FAKE, 2, None) == 4  # store policy other than 0 / 1
    assert g(FAKE, 2048, FAKE, -1, None) == 4
    assert g(FAKE, 1000, FAKE, 1, None) == 2
    assert g(None, 2048, FAKE, 0, None) == 1


def test_baseline_entry_validation():
    lib = _lib()

    def unf(M=64, N=4096, R=128, rpt=1, fmax=448.0):
        return lib.rnq_baseline_norm_rope_quant_unfused(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, M, N, R, rpt,
                                                        1e-6, fmax, 0, None)

    assert unf(N=4100) == 3
    assert unf(R=130) == 3
    assert unf(M=63, rpt=2) == 2
    assert unf(fmax=0.0) == 4
    assert unf(M=0) == 0
    assert lib.rnq_baseline_norm_rope_quant_unfused(FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, FAKE, 4, 4096, 128, 1,
                                                    1e-6, 448.0, 0, None) == 1

    def des(rpb=8, Hq=32, Hk=8, D=128):
        return lib.rnq_baseline_qk_design(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 16, Hq, Hk, D, D,
                                          rpb, 1e-6, 448.0, 0, None)

    assert des(rpb=3) == 2  # does not divide 40 heads
    assert des(rpb=0) == 2
    assert des(rpb=40, D=512) == 3  # 2560 threads
    assert des(D=96) == 3
