"""The C-ABI library: loads, exports what include/cskv.h declares, and
rejects bad arguments with the documented status codes before any launch
(so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cskv.h")
OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
P = ctypes.c_void_p(0x100000)        # aligned, never dereferenced on error paths
NULL = None


@pytest.fixture(scope="module")
def lib():
    from compressed_sparse_kv_overlapping_amd import binding
    return binding.library()


def declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[a-z][\w \*]*?\b(cskv_\w+)\(", text, flags=re.M)))


def test_header_functions_are_exported(lib):
    names = declared()
    assert len(names) == 25
    for n in names:
        assert hasattr(lib, n), f"{n} declared in cskv.h but not exported"
    from compressed_sparse_kv_overlapping_amd import binding
    assert set(binding.EXPORTS) == set(names)


def test_version_and_status_strings(lib):
    assert lib.cskv_version() == 10500
    assert lib.cskv_status_string(OK) == b"ok"
    for code in (INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.cskv_status_string(code) not in (b"ok", b"unknown status")


def test_compress_errors(lib):
    c = lib.cskv_compress
    assert c(P, P, P, 16, 0, 0, 1, P, 512, 1, NULL) == INVALID          # m < 1
    assert c(P, P, P, -1, 4, 0, 0, P, 512, 1, NULL) == INVALID          # T < 0
    assert c(P, P, P, 16, 4, 0, 5, P, 512, 1, NULL) == INVALID          # past N = 4
    assert c(P, P, P, 16, 4, 2, 1, P, 512, 1, NULL) == INVALID          # end < begin
    assert c(P, P, P, 16, 4, 0, 4, P, 500, 1, NULL) == INVALID          # ld_out < 512
    assert c(P, P, P, 16, 4, 0, 4, P, 516, 1, NULL) == INVALID          # ld_out % 8
    assert c(P, P, P, 16, 4, 0, 4, P, 576, 2, NULL) == UNSUPPORTED      # fp8 raw rows
    assert c(NULL, P, P, 16, 4, 0, 4, P, 576, 1, NULL) == INVALID       # null
    assert b"null" in lib.cskv_last_error()
    assert c(P, P, P, 16, 4, 0, 4, ctypes.c_void_p(0x100008), 576, 1, NULL) == INVALID  # alignment
    assert c(NULL, NULL, NULL, 3, 4, 0, 0, NULL, 512, 1, NULL) == OK    # empty range: no-op


def test_compress2_errors(lib):
    f = lib.cskv_compress2
    ws = lib.cskv_compress2_workspace_size(4096, 128)
    assert ws >= 12 * 512 * 4                                          # one block's boundary sums
    assert f(P, P, 4096, P, 4, P, 576, P, 130, P, 576, 1, P, ws, NULL) == INVALID      # 130 % 4
    assert f(P, P, 4096, P, 4, P, 576, P, 4, P, 576, 1, P, ws, NULL) == INVALID        # equal sizes
    assert f(P, P, 4096, P, 8, P, 576, P, 128, P, 576, 1, P, ws, NULL) == UNSUPPORTED  # m_small > 4
    assert f(P, P, 4096, P, 4, P, 576, P, 128, P, 576, 2, P, ws, NULL) == UNSUPPORTED  # fp8
    assert f(P, P, 4096, P, 4, P, 500, P, 128, P, 576, 1, P, ws, NULL) == INVALID      # ld
    assert f(P, P, 4096, P, 4, P, 576, P, 128, P, 576, 1, NULL, ws, NULL) == WORKSPACE
    assert f(P, P, 4096, P, 4, P, 576, P, 128, P, 576, 1, P, ws - 1, NULL) == WORKSPACE
    assert f(NULL, P, 4096, P, 4, P, 576, P, 128, P, 576, 1, P, ws, NULL) == INVALID
    assert f(NULL, NULL, 3, NULL, 4, NULL, 512, NULL, 128, NULL, 512, 1, NULL, 0, NULL) == OK  # T < m


def test_index_topk_errors(lib):
    f = lib.cskv_index_topk
    ws = lib.cskv_index_topk_workspace_size(8, 16384, 1024)
    assert ws > 8 * 8192 * 8
    assert f(P, P, 8, 16384, 0, 0, NULL, 4, 1.0, 1, P, P, ws, NULL) == INVALID       # k < 1
    assert f(P, P, 8, 16384, 4097, 0, NULL, 4, 1.0, 1, P, P, ws, NULL) == UNSUPPORTED  # k > 4096
    assert f(P, P, 8, 16384, 64, 0, P, 0, 1.0, 1, P, P, ws, NULL) == INVALID        # m with q_pos
    assert f(P, P, 8, 16384, 64, 0, NULL, 4, -1.0, 1, P, P, ws, NULL) == INVALID    # scale
    assert f(P, P, 8, 16384, 64, 0, NULL, 4, 1.0, 7, P, P, ws, NULL) == UNSUPPORTED  # dtype
    assert f(P, P, 8, 1 << 21, 64, 0, NULL, 4, 1.0, 1, P, P, ws, NULL) == UNSUPPORTED  # N
    assert f(P, P, 8, 16384, 64, 0, NULL, 4, 1.0, 1, P, NULL, ws, NULL) == WORKSPACE
    assert f(P, P, 8, 16384, 64, 0, NULL, 4, 1.0, 1, P, P, 16, NULL) == WORKSPACE
    assert f(NULL, P, 8, 16384, 64, 0, NULL, 4, 1.0, 1, P, P, ws, NULL) == INVALID


def test_index_topk_noalloc_errors(lib):
    """The allocation-free selection rejects bad arguments, and selections
    whose scratch exceeds its fixed array, before touching the device."""
    f = lib.cskv_index_topk_noalloc
    cap = lib.cskv_index_topk_noalloc_max_bytes()
    assert cap == 32 << 20
    assert lib.cskv_index_topk_workspace_size(32, 1 << 18, 1024) <= cap       # 1M-token decode fits
    assert lib.cskv_index_topk_workspace_size(4096, 1 << 18, 1024) > cap
    assert f(P, P, 4096, 1 << 18, 1024, 0, NULL, 4, 1.0, 2, P, NULL) == UNSUPPORTED
    assert b"scratch" in lib.cskv_last_error()
    assert f(P, P, 8, 16384, 0, 0, NULL, 4, 1.0, 1, P, NULL) == INVALID       # k < 1
    assert f(P, P, 8, 16384, 4097, 0, NULL, 4, 1.0, 1, P, NULL) == UNSUPPORTED  # k > 4096
    assert f(NULL, P, 8, 16384, 64, 0, NULL, 4, 1.0, 1, P, NULL) == INVALID
    assert f(P, P, 8, 16384, 64, 0, NULL, 4, 1.0, 1, NULL, NULL) == INVALID
    assert f(P, P, 8, 16384, 64, 0, P, 0, 1.0, 1, P, NULL) == INVALID        # m with q_pos


def test_index_topk_mxfp4_errors(lib):
    f = lib.cskv_index_topk_mxfp4
    ws = lib.cskv_index_topk_workspace_size(8, 16384, 1024)
    S = P  # scale arrays: any even address (no call reaches a kernel)

    def call(q=P, qs=S, kc=P, ks=S, B=8, N=16384, k=64, kb=0, qp=NULL, m=4, sc=1.0, out=P, w=P,
             wsb=ws):
        return f(q, qs, kc, ks, B, N, k, kb, qp, m, sc, out, w, wsb, NULL)
    assert call(qs=NULL) == INVALID and call(ks=NULL) == INVALID       # scales
    assert call(q=NULL) == INVALID and call(out=NULL) == INVALID
    assert call(k=0) == INVALID and call(k=4097) == UNSUPPORTED
    assert call(kb=-1) == INVALID                                      # stride in rows
    assert call(qp=P, m=0) == INVALID and call(sc=0.0) == INVALID
    assert call(N=1 << 21) == UNSUPPORTED
    assert call(w=NULL) == WORKSPACE and call(wsb=16) == WORKSPACE


def test_attend_mxfp4_errors(lib):
    s, h = lib.cskv_sparse_attend_mxfp4, lib.cskv_hca_attend_mxfp4
    ws = lib.cskv_attend_workspace_size(8, 128, 1152)

    def sp(q=P, c=P, sc=P, w=P, idx=P, B=8, H=128, N=16384, W=128, k=1024, eb=0, wr=128, wsb=ws):
        return s(q, c, sc, w, idx, B, H, N, W, k, eb, 0, wr, NULL, 0, 1.0, NULL, -1.0, P, P, P, wsb,
                 NULL)
    assert sp(sc=NULL) == INVALID and sp(c=NULL) == INVALID and sp(q=NULL) == INVALID
    assert sp(idx=NULL) == INVALID and sp(W=200) == INVALID and sp(eb=-1) == INVALID
    assert sp(B=0) == INVALID and sp(wsb=16) == WORKSPACE
    hws = lib.cskv_hca_workspace_size(8, 128, 8192)

    def hc(c=P, sc=P, B=8, N=8192, eb=0, qp=NULL, m=0, wsb=hws):
        return h(P, c, sc, B, 128, N, eb, qp, m, 1.0, NULL, -1.0, P, P, P, wsb, NULL)
    assert hc(sc=NULL) == INVALID and hc(c=NULL) == INVALID and hc(eb=-3) == INVALID
    assert hc(qp=P, m=0) == INVALID and hc(wsb=16) == WORKSPACE


def test_attend_errors(lib):
    s = lib.cskv_sparse_attend
    ws = lib.cskv_attend_workspace_size(8, 128, 1152)
    assert ws > 0
    args = dict(q=P, e=P, w=P, idx=P, B=8, H=128, N=16384, W=128, k=1024, eb=0, wb=0, wr=128,
                qp=NULL, wp0=0, sc=1.0, sink=NULL, ne=-1.0, dt=1, out=P, lse=P, ws=P, wsb=ws, st=NULL)

    def call(**kw):
        a = dict(args, **kw)
        return s(*a.values())
    assert call(W=200) == INVALID                                     # W > window rows
    assert call(dt=2) == UNSUPPORTED                                  # fp8 rows
    assert call(H=0) == INVALID
    assert call(idx=NULL) == INVALID
    assert call(ws=NULL) == WORKSPACE
    assert call(w=NULL) == INVALID
    assert call(sc=-0.5) == INVALID                                   # negative scale
    assert call(sc=float("inf")) == INVALID
    assert call(sc=float("nan")) == INVALID
    assert call(ne=float("nan")) == INVALID                           # normalisation epsilon
    assert call(ne=float("inf")) == INVALID
    h = lib.cskv_hca_attend
    hws = lib.cskv_hca_workspace_size(32, 128, 8192)
    assert h(P, P, 32, 128, 8192, 0, NULL, 0, 1.0, NULL, -1.0, 1, P, P, NULL, hws, NULL) == WORKSPACE
    assert h(P, P, 32, 128, 8192, 0, NULL, 0, 1.0, NULL, -1.0, 2, P, P, P, hws, NULL) == UNSUPPORTED
    assert h(P, P, 32, 128, 8192, 0, NULL, 0, -1.0, NULL, -1.0, 1, P, P, P, hws, NULL) == INVALID
    assert h(P, P, 32, 128, 8192, 0, P, 0, 1.0, NULL, -1.0, 1, P, P, P, hws, NULL) == INVALID  # m < 1
    assert h(P, P, 32, 128, 8192, 0, NULL, 0, 1.0, NULL, float("nan"), 1, P, P, P, hws, NULL) == INVALID
    m = lib.cskv_merge
    assert m(P, P, 2, 4, 0, NULL, P, P, 1, NULL) == INVALID
    assert m(P, P, 2, 4, 3, NULL, P, P, 2, NULL) == UNSUPPORTED


def test_csa_workspace_covers_parts(lib):
    B, H, N, W, k = 32, 128, 262144, 128, 1024
    total = lib.cskv_csa_workspace_size(B, H, N, W, k)
    assert total >= lib.cskv_index_topk_workspace_size(B, N, k) + lib.cskv_attend_workspace_size(B, H, k + W)
    assert lib.cskv_csa_attend(P, P, P, P, P, B, H, N, W, k, 4, 0, 0, 0, W, NULL, 0, 1.0, NULL, -1.0,
                               1.0, 1, 1, P, P, P, P, total - 1, NULL) == WORKSPACE


def test_binding_refuses_missing_library(monkeypatch, tmp_path):
    from compressed_sparse_kv_overlapping_amd import binding
    monkeypatch.setattr(binding, "_lib", None)
    monkeypatch.setattr(binding, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError):
        binding.library()
