"""The C-ABI library loads, exports every function include/epdc.h declares,
and rejects invalid arguments on the host before touching the GPU.  No kernel
runs here (no GPU needed)."""

import ctypes
import os
import subprocess

import pytest

from combine_ep_send_amd import _lib

pytestmark = pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH),
                                reason="libepdc.so not built")

EXPECTED = {
    "ep_abi_version", "ep_status_string", "ep_workspace_status", "ep_counts_workspace_bytes", "ep_layout_workspace_bytes",
    "ep_batched_workspace_bytes", "ep_compute_send_counts", "ep_build_send_layout",
    "ep_dispatch_layout_workspace_bytes", "ep_dispatch_layout", "ep_dispatch_layout_noalloc",
    "ep_dispatch_layout_chunked_workspace_bytes", "ep_dispatch_layout_chunked",
    "ep_regroup_workspace_bytes", "ep_regroup_by_expert",
    "ep_dispatch_permute", "ep_batched_prepare", "ep_batched_prepare_fp8", "ep_combine",
}


def test_header_declares_the_entry_points():
    assert set(_lib.header_functions()) == EXPECTED


def test_library_exports_every_header_function():
    L = ctypes.CDLL(_lib.LIB_PATH)
    for name in _lib.header_functions():
        assert hasattr(L, name), name
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    assert EXPECTED <= exported


def test_bindings_follow_the_header_version():
    import re
    text = open(_lib.HEADER).read()
    assert int(re.search(r"#define EPDC_ABI_VERSION (\d+)", text).group(1)) == _lib.ABI_VERSION


def test_version_and_status_strings():
    # version 6: ep_dispatch_layout_chunked (5: ep_dispatch_layout_noalloc,
    # 4: ep_workspace_status)
    L = _lib.lib()
    assert L.ep_abi_version() == 6
    assert L.ep_status_string(0) == b"ok"
    for s in (-1, -2, -3, -4):
        assert L.ep_status_string(s) not in (b"ok", b"unknown status")
    assert L.ep_status_string(7) == b"unknown status"


def test_workspace_sizes():
    L = _lib.lib()
    assert L.ep_counts_workspace_bytes(16384, 32, 8, 1) == 256 + (32 + 256 + 1) * 4
    assert L.ep_counts_workspace_bytes(32768, 32, 8, 4) == 256 + 4 * (32 + 256 + 1) * 4
    assert L.ep_counts_workspace_bytes(0, 2, 4, 3) == 256 + 3 * (2 + 8 + 1) * 4
    assert L.ep_layout_workspace_bytes(16384, 32) == 256 + 64 * 32 * 8
    assert L.ep_layout_workspace_bytes(0, 32) == 256 + 1 * 32 * 8
    assert L.ep_layout_workspace_bytes(-1, 32) == 0
    assert L.ep_batched_workspace_bytes(8192, 32, 8192) == 256 + 32 * 32 * 8
    assert L.ep_batched_workspace_bytes(8192, 32, 0) == 256 + 32 * 32 * 8
    assert L.ep_batched_workspace_bytes(8192, 0, 8192) == 0


def test_workspace_sizes_past_the_limits_are_zero():
    # sizes every call rejects (T >= 2^30, E > 8192) give 0, with no
    # arithmetic overflow on the way (INT64_MAX tokens, 2^16 x 2^16 experts)
    L = _lib.lib()
    big = (1 << 63) - 1
    for T in (1 << 30, big):
        assert L.ep_counts_workspace_bytes(T, 32, 8, 1) == 0
        assert L.ep_layout_workspace_bytes(T, 32) == 0
        assert L.ep_batched_workspace_bytes(T, 32, 8192) == 0
        assert L.ep_dispatch_layout_workspace_bytes(T, 32, 8) == 0
        assert L.ep_regroup_workspace_bytes(T, 256) == 0
    assert L.ep_counts_workspace_bytes(16, 1 << 16, 1 << 16, 1) == 0
    assert L.ep_dispatch_layout_workspace_bytes(16, 1 << 16, 1 << 16) == 0
    assert L.ep_counts_workspace_bytes(16, 1024, 8, 1) == 256 + (1024 + 8192 + 1) * 4
    assert L.ep_counts_workspace_bytes(16, 1024, 9, 1) == 0
    # the largest supported token count still gets a size
    assert L.ep_layout_workspace_bytes((1 << 30) - 1, 2) == 256 + (1 << 22) * 2 * 8


# Host-side validation: every call below returns before any HIP call, because
# an argument is rejected.  Pointers are fake but never dereferenced.
P = ctypes.c_void_p
A16 = P(0x10000)   # 16-byte (and 256-byte) aligned fake address
A8 = P(0x10008)
ODD = P(0x10002)


def test_counts_rejects_bad_arguments():
    L = _lib.lib()
    f = L.ep_compute_send_counts
    ok = dict(idx=A16, T=16, K=2, P=2, El=4, C=1)

    def call(idx=A16, T=16, K=2, Pn=2, El=4, C=1, dest=A16, iir=A16, sc=A16, ws=A16,
             ws_bytes=1 << 20):
        return f(idx, T, K, Pn, El, C, dest, iir, sc, None, None, ws, ws_bytes, None)
    assert call(idx=None) == _lib.EP_ERR_INVALID_ARG
    assert call(T=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(K=0) == _lib.EP_ERR_INVALID_ARG
    assert call(K=17) == _lib.EP_ERR_UNSUPPORTED
    assert call(C=0) == _lib.EP_ERR_INVALID_ARG
    assert call(Pn=2048) == _lib.EP_ERR_UNSUPPORTED
    assert call(Pn=64, El=256) == _lib.EP_ERR_UNSUPPORTED     # E > 8192
    assert call(idx=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(T=1 << 30) == _lib.EP_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=64) == _lib.EP_ERR_WORKSPACE
    assert ok


def test_layout_rejects_bad_workspace_and_capacity():
    L = _lib.lib()
    f = L.ep_build_send_layout

    def call(ws=A16, ws_bytes=1 << 20, cap=64, T=16):
        return f(A16, A16, A16, A16, T, 2, 2, 4, cap, A16, A16, A16, A16, A16, ws, ws_bytes,
                 None)
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=16) == _lib.EP_ERR_WORKSPACE
    assert call(ws=A8) == _lib.EP_ERR_WORKSPACE                # not 256-aligned
    assert call(cap=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(cap=1 << 31) == _lib.EP_ERR_UNSUPPORTED


def test_fused_layout_workspace_and_arguments():
    L = _lib.lib()
    # one row of P + E + 1 words per workgroup, min(tiles of 256, 256) rows
    assert L.ep_dispatch_layout_workspace_bytes(16384, 32, 8) == \
        256 + 64 * (32 + 256 + 1) * 4 + 64 * 32 * 4 + 32 * 4
    assert L.ep_dispatch_layout_workspace_bytes(0, 2, 4) == 256 + 1 * (2 + 8 + 1) * 4 + 2 * 4 + 2 * 4
    assert L.ep_dispatch_layout_workspace_bytes(1 << 20, 8, 8) == \
        256 + 256 * (8 + 64 + 1) * 4 + 256 * 8 * 4 + 8 * 4
    assert L.ep_dispatch_layout_workspace_bytes(-1, 2, 4) == 0
    f = L.ep_dispatch_layout

    def call(T=16, K=2, P=2, El=4, cap=64, dest=A16, ws=A16, ws_bytes=1 << 22, tpe=None):
        return f(A16, A16, T, K, P, El, cap, dest, A16, A16, tpe, None, A16, A16, A16, A16,
                 A16, ws, ws_bytes, None)
    assert call(T=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(K=0) == _lib.EP_ERR_INVALID_ARG
    assert call(K=17) == _lib.EP_ERR_UNSUPPORTED
    assert call(cap=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(cap=1 << 31) == _lib.EP_ERR_UNSUPPORTED
    assert call(dest=None) == _lib.EP_ERR_INVALID_ARG
    assert call(dest=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(tpe=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws=A8) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=64) == _lib.EP_ERR_WORKSPACE
    # LDS share over 64 KiB (1024 destinations x 8 experts): use the two calls
    assert call(T=20000, P=1024, El=8) == _lib.EP_ERR_UNSUPPORTED


def test_chunked_layout_workspace_and_arguments():
    L = _lib.lib()
    # 4 chunks x 32 destinations = 128 bins, 64 workgroups at 16384 tokens
    assert L.ep_dispatch_layout_chunked_workspace_bytes(16384, 32, 4) == \
        256 + 64 * (128 + 1) * 4 + 64 * 128 * 4 + 128 * 4
    assert L.ep_dispatch_layout_chunked_workspace_bytes(16384, 32, 33) == 0     # 1056 bins
    assert L.ep_dispatch_layout_chunked_workspace_bytes(16, 2, 0) == 0
    f = L.ep_dispatch_layout_chunked

    def call(T=16, K=2, P=2, El=4, C=2, cap=64, dest=A16, sti=A16, ws=A16, ws_bytes=1 << 22):
        return f(A16, A16, T, K, P, El, C, cap, dest, A16, A16, None, sti, A16, A16, A16, A16,
                 ws, ws_bytes, None)
    assert call(C=0) == _lib.EP_ERR_INVALID_ARG
    assert call(cap=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(P=32, C=33) == _lib.EP_ERR_UNSUPPORTED        # more than 1024 bins
    assert call(C=4, cap=1 << 29, K=2) == _lib.EP_ERR_UNSUPPORTED   # C*cap*K past int32
    assert call(dest=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(sti=None) == _lib.EP_ERR_INVALID_ARG
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=64) == _lib.EP_ERR_WORKSPACE


def test_noalloc_layout_rejects_before_touching_the_gpu():
    L = _lib.lib()
    f = L.ep_dispatch_layout_noalloc

    def call(T=16, K=2, P=2, El=4, cap=64, dest=A16, tpe=None):
        return f(A16, A16, T, K, P, El, cap, dest, A16, A16, tpe, None, A16, A16, A16, A16,
                 A16, None)
    assert call(T=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(K=17) == _lib.EP_ERR_UNSUPPORTED
    assert call(cap=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(dest=ODD) == _lib.EP_ERR_INVALID_ARG
    # a workspace need past the scratch: 256 workgroups x (1024 + 8192 + 1 + 1024) words
    need = L.ep_dispatch_layout_workspace_bytes(1 << 20, 1024, 8)
    assert need > _lib.NOALLOC_SCRATCH_BYTES
    assert call(T=1 << 20, P=1024, El=8, cap=1 << 20) == _lib.EP_ERR_WORKSPACE
    # the headline shape fits with room to spare
    assert L.ep_dispatch_layout_workspace_bytes(16384, 32, 8) < _lib.NOALLOC_SCRATCH_BYTES // 32
    st = L.ep_workspace_status
    assert st(A16, 1 << 20, None, None) == _lib.EP_ERR_INVALID_ARG
    assert st(A16, 1 << 20, ODD, None) == _lib.EP_ERR_INVALID_ARG
    assert st(A8, 1 << 20, A16, None) == _lib.EP_ERR_WORKSPACE
    assert st(A16, 128, A16, None) == _lib.EP_ERR_WORKSPACE


def test_regroup_workspace_and_arguments():
    L = _lib.lib()
    # 1000 rows: 64-row tiles, 16 workgroups
    assert L.ep_regroup_workspace_bytes(1000, 8) == 256 + 16 * (8 + 1) * 4 + 16 * 8 * 4 + 8 * 4
    assert L.ep_regroup_workspace_bytes(0, 8) == 256 + 1 * 9 * 4 + 8 * 4 + 8 * 4
    assert L.ep_regroup_workspace_bytes(10, 0) == 0
    f = L.ep_regroup_by_expert

    def call(R=16, K=2, H=64, El=4, align=1, cap=64, x=A16, idx=A16, ws=A16,
             ws_bytes=1 << 20, grp=None, G=1):
        return f(x, idx, None, grp, G, R, K, H, El, align, cap, A16, A16, None, A16, A16, A16,
                 ws, ws_bytes, None)
    assert call(G=0) == _lib.EP_ERR_INVALID_ARG
    assert call(G=2) == _lib.EP_ERR_INVALID_ARG                 # groups need row_group
    assert call(G=2, grp=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(G=300, grp=A16) == _lib.EP_ERR_UNSUPPORTED      # 1200 bins
    assert call(align=0) == _lib.EP_ERR_INVALID_ARG
    assert call(El=0) == _lib.EP_ERR_INVALID_ARG
    assert call(cap=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(H=60) == _lib.EP_ERR_INVALID_ARG
    assert call(x=A8) == _lib.EP_ERR_INVALID_ARG
    assert call(idx=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(El=2000) == _lib.EP_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=8) == _lib.EP_ERR_WORKSPACE
    # Every regrouped row index, padding included, must fit int32: at most
    # R*min(K, E_local) rows plus align-1 padding rows per bin.  1023 bins at
    # align 2^21 leave room for exactly 2098174 one-slot rows; one more row
    # is refused before the workspace is looked at (no launch either way).
    big = dict(K=1, El=1, G=1023, grp=A16, align=1 << 21, ws=None)
    fit = 2**31 - 1 - 1023 * ((1 << 21) - 1)
    assert fit == 2098174
    assert call(R=fit, **big) == _lib.EP_ERR_WORKSPACE
    assert call(R=fit + 1, **big) == _lib.EP_ERR_UNSUPPORTED
    assert call(R=(1 << 23) + 1, **big) == _lib.EP_ERR_UNSUPPORTED


def test_permute_and_combine_reject_bad_rows():
    L = _lib.lib()
    perm = L.ep_dispatch_permute
    assert perm(A16, 4, 100, A16, 2, 8, 0, A16, None, None) == _lib.EP_ERR_INVALID_ARG  # H%8
    assert perm(A16, 4, 64, A16, 2, 8, 1, A16, A16, None) == _lib.EP_ERR_INVALID_ARG   # H%128 fp8
    assert perm(A16, 4, 128, A16, 2, 8, 1, A16, None, None) == _lib.EP_ERR_INVALID_ARG  # no scale
    assert perm(A8, 4, 64, A16, 2, 8, 0, A16, None, None) == _lib.EP_ERR_INVALID_ARG   # x align
    assert perm(A16, 4, 64, A16, 2, 8, 5, A16, None, None) == _lib.EP_ERR_INVALID_ARG  # dtype
    comb = L.ep_combine
    assert comb(A16, 10, A16, A16, 4, 2, 60, None, None, A16, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(None, 10, A16, A16, 4, 2, 64, None, None, A16, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(A16, 10, A16, A16, 4, 0, 64, None, None, A16, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(A16, 10, A16, A16, 4, 2, 64, None, None, A8, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(A16, 10, A16, ODD, 4, 2, 64, None, None, A16, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(A16, 10, A16, A16, 4, 2, 64, A8, None, A16, None) == _lib.EP_ERR_INVALID_ARG
    assert comb(A16, 10, A16, None, 4, 2, 64, A16, A8, A16, None) == _lib.EP_ERR_INVALID_ARG


def test_batched_rejects_bad_arguments():
    L = _lib.lib()
    f = L.ep_batched_prepare

    def call(first=0, El=4, M=8, ws=A16, ws_bytes=1 << 20):
        return f(A16, A16, 16, 2, 64, first, El, M, A16, A16, A16, ws, ws_bytes, None)
    assert call(first=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(El=0) == _lib.EP_ERR_INVALID_ARG
    assert call(El=2000) == _lib.EP_ERR_UNSUPPORTED
    assert call(M=1 << 30) == _lib.EP_ERR_UNSUPPORTED
    # E_local * max past int64 (it once wrapped negative and passed the check)
    assert call(El=128, M=(1 << 63) - 1) == _lib.EP_ERR_UNSUPPORTED
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE


def test_batched_fp8_rejects_bad_arguments():
    L = _lib.lib()
    f = L.ep_batched_prepare_fp8

    def call(H=512, fmt=0, col=0, first=0, El=4, M=8, q=A16, sc=A16, ws=A16, ws_bytes=1 << 20):
        return f(A16, A16, 16, 2, H, first, El, M, fmt, col, q, sc, A16, A16, ws, ws_bytes, None)
    assert call(H=64) == _lib.EP_ERR_INVALID_ARG                  # H % 128
    assert call(H=640, fmt=2) == _lib.EP_ERR_INVALID_ARG          # UE8M0: H % 512
    assert call(fmt=3) == _lib.EP_ERR_INVALID_ARG
    assert call(col=2) == _lib.EP_ERR_INVALID_ARG
    assert call(first=-1) == _lib.EP_ERR_INVALID_ARG
    assert call(El=2000) == _lib.EP_ERR_UNSUPPORTED
    assert call(M=1 << 30) == _lib.EP_ERR_UNSUPPORTED
    assert call(El=128, M=(1 << 63) - 1) == _lib.EP_ERR_UNSUPPORTED
    assert call(q=A8) == _lib.EP_ERR_INVALID_ARG
    assert call(sc=None) == _lib.EP_ERR_INVALID_ARG
    assert call(sc=ODD) == _lib.EP_ERR_INVALID_ARG
    assert call(ws=None) == _lib.EP_ERR_WORKSPACE
    assert call(ws_bytes=16) == _lib.EP_ERR_WORKSPACE


def test_loader_checks_the_version_before_binding_symbols(tmp_path, monkeypatch):
    # a stub that exports only ep_abi_version, reporting an older version:
    # the loader must name the mismatch, not fail on a missing symbol
    src = tmp_path / "stub.c"
    src.write_text("int ep_abi_version(void) { return 2; }\n")
    so = tmp_path / "libepdc.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-o", str(so), str(src)], check=True)
    monkeypatch.setattr(_lib, "LIB_PATH", str(so))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(ImportError, match="ABI version 2"):
        _lib.lib()
    src.write_text("int some_other_function(void) { return 0; }\n")
    so2 = tmp_path / "libother.so"
    subprocess.run(["gcc", "-shared", "-fPIC", "-o", str(so2), str(src)], check=True)
    monkeypatch.setattr(_lib, "LIB_PATH", str(so2))
    with pytest.raises(ImportError, match="no ep_abi_version"):
        _lib.lib()
