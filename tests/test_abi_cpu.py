"""The C-ABI library loads, exports every declared entry point and rejects bad
arguments on the host before touching the GPU (CPU only: no call here
reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

from moe_layer_route_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_layer_route.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIPERR = 0, 1, 2, 3, 4
FAKE = 0x10000          # a 64 KiB-aligned non-null address that is never dereferenced


def _declared():
    src = open(HEADER).read()
    return re.findall(r"MOE_API\s+[\w\s\*]+?\b(moe_\w+)\s*\(", src)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("library not built")
    return binding.library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert len(names) >= 13, names
    raw = ctypes.CDLL(binding.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(names) == set(binding.EXPORTS)


def test_version_and_status_strings(lib):
    ver = int(re.search(r"#define MOE_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert lib.moe_abi_version() == ver
    assert lib.moe_status_str(OK) == b"ok"
    assert lib.moe_status_str(WORKSPACE) == b"workspace too small"
    assert lib.moe_status_str(99) == b"unknown status"


def test_workspace_bytes(lib):
    for T, E in ((8, 32), (64, 32), (4096, 32), (256, 128), (16384, 128)):
        n = lib.moe_workspace_bytes(T, 2880, E, 4, 2880)
        S = T * 4
        assert n >= S * 2880 * 2 + S * 2880 * 4 + 4 * S * 4 and n % 256 == 0
    assert lib.moe_workspace_bytes(0, 2880, 32, 4, 2880) == 0
    assert lib.moe_workspace_bytes(8, 2880, 4, 5, 2880) == 0            # k > E
    assert b"k=5" in lib.moe_last_error()
    assert lib.moe_workspace_bytes(8, 2884, 32, 4, 2880) == 0           # H % 8 != 0


def _fwd(lib, T=8, H=64, E=8, k=2, I=64, ptrs=None, ws_bytes=1 << 30, path=0, ws=FAKE):
    p = [FAKE] * 8 if ptrs is None else ptrs
    return lib.moe_forward_ex(*[ctypes.c_void_p(v) if v else None for v in p[:7]], T, H, E, k, I,
                              ctypes.c_void_p(p[7]) if p[7] else None, None, None,
                              ctypes.c_void_p(ws) if ws else None, ws_bytes, path, None)


@pytest.mark.parametrize("kw,err", [
    (dict(T=-1), "T=-1"), (dict(E=0), "E=0"), (dict(E=257), "E=257"), (dict(k=0), "k=0"),
    (dict(k=9, E=16), "k=9"), (dict(k=5, E=4), "k=5"), (dict(H=60), "H=60"), (dict(I=12), "I=12"),
    (dict(H=16392), "H=16392"), (dict(path=3), "path 3"), (dict(T=1 << 30, k=2), "T*k"),
])
def test_forward_rejects_bad_sizes(lib, kw, err):
    assert _fwd(lib, **kw) == INVALID
    assert err in lib.moe_last_error().decode()


def test_forward_rejects_bad_pointers(lib):
    for i in range(8):
        p = [FAKE] * 8
        p[i] = 0
        assert _fwd(lib, ptrs=p) == INVALID
        assert b"is NULL" in lib.moe_last_error()
    p = [FAKE] * 8
    p[0] = FAKE + 8                      # x must be 16-byte aligned
    assert _fwd(lib, ptrs=p) == INVALID
    assert b"aligned" in lib.moe_last_error()
    assert _fwd(lib, ws=FAKE + 64) == INVALID        # workspace must be 256-byte aligned


def test_forward_workspace_checks(lib):
    need = lib.moe_workspace_bytes(8, 64, 8, 2, 64)
    assert _fwd(lib, ws_bytes=need - 1) == WORKSPACE
    assert _fwd(lib, ws=0) == WORKSPACE
    assert b"needed" in lib.moe_last_error()


def test_zero_tokens_is_a_no_op(lib):
    assert _fwd(lib, T=0, ws=0, ws_bytes=0) == OK
    assert lib.moe_last_error() == b""
    v = ctypes.c_void_p(FAKE)
    assert lib.moe_route(v, v, v, 0, 64, 8, 2, v, v, None) == OK
    assert lib.moe_permute(v, 0, 8, 2, v, v, v, v, None) == OK
    assert lib.moe_combine(v, v, v, 0, 64, 2, v, None) == OK


def test_stage_calls_validate(lib):
    v = ctypes.c_void_p(FAKE)
    assert lib.moe_route(v, v, v, 4, 64, 8, 9, v, v, None) == INVALID
    assert lib.moe_route_ex(v, v, v, 4, 64, 8, 2, v, v, 3, None) == INVALID
    assert b"router method" in lib.moe_last_error()
    assert lib.moe_route(None, v, v, 4, 64, 8, 2, v, v, None) == INVALID
    assert lib.moe_permute(v, 4, 300, 2, v, v, v, v, None) == INVALID
    assert lib.moe_gate_up(v, v, v, v, v, v, 4, 64, 8, 2, 64, v, 7, None) == INVALID
    assert lib.moe_down(v, v, v, v, None, 4, 64, 8, 2, 64, v, 0, None) == INVALID
    assert lib.moe_combine(v, v, v, 4, 60, 2, v, None) == INVALID


def _fwd_ep(lib, e_begin, n_local, T=8, H=64, E=8, k=2, I=64):
    v = ctypes.c_void_p(FAKE)
    return lib.moe_forward_ep(*([v] * 7), T, H, E, k, I, e_begin, n_local, v, None, None, v, 1 << 30, 0, None)


@pytest.mark.parametrize("e_begin,n_local", [(-1, 2), (0, 0), (7, 2), (0, 9), (3, -1)])
def test_forward_ep_rejects_bad_ranges(lib, e_begin, n_local):
    assert _fwd_ep(lib, e_begin, n_local) == INVALID
    assert b"local experts" in lib.moe_last_error()


def test_forward_ep_accepts_every_valid_range(lib):
    v = ctypes.c_void_p(FAKE)
    for e_begin, n_local in ((0, 8), (0, 1), (7, 1), (2, 5)):
        # T = 0: validated, nothing enqueued
        assert lib.moe_forward_ep(*([v] * 7), 0, 64, 8, 2, 64, e_begin, n_local, v, None, None, None, 0, 0,
                                  None) == OK


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib
    mod = importlib.import_module("moe_layer_route_amd.binding")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(binding.MoEError, match="not built"):
            mod.library(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


def _fwd_mx(lib, T=8, H=64, E=8, k=2, I=64, ptrs=None, ws_bytes=1 << 30):
    p = [FAKE] * 10 if ptrs is None else ptrs
    vp = [ctypes.c_void_p(v) if v else None for v in p]
    return lib.moe_forward_mxfp4(*vp[:9], T, H, E, k, I, vp[9], None, None, ctypes.c_void_p(FAKE), ws_bytes, None)


def test_mxfp4_calls_validate(lib):
    v = ctypes.c_void_p(FAKE)
    # H and I must be multiples of 32 (one scale per 32 values along K)
    assert _fwd_mx(lib, H=40) == INVALID and b"multiples of 32" in lib.moe_last_error()
    assert _fwd_mx(lib, I=48) == INVALID
    for i in range(10):
        p = [FAKE] * 10
        p[i] = 0
        assert _fwd_mx(lib, ptrs=p) == INVALID
        assert b"is NULL" in lib.moe_last_error()
    assert _fwd_mx(lib, ws_bytes=16) == WORKSPACE
    assert _fwd_mx(lib, T=0) == OK
    assert lib.moe_gate_up_mxfp4(v, v, v, v, v, v, v, 4, 72, 8, 2, 64, v, 0, None) == INVALID
    assert lib.moe_down_mxfp4(v, v, None, v, v, v, 4, 64, 8, 2, 64, v, 0, None) == INVALID
    assert lib.moe_gate_up_mxfp4(v, v, v, v, v, v, v, 4, 64, 8, 2, 64, v, 3, None) == INVALID
    assert b"unknown path" in lib.moe_last_error()
    p = [ctypes.c_void_p(FAKE)] * 10
    assert lib.moe_forward_mxfp4_ex(*p[:9], 8, 64, 8, 2, 64, p[9], None, None, v, 1 << 30, 5, None) == INVALID
    # the quantiser: K % 32 == 0, N % 8 == 0, codes 16-byte aligned
    assert lib.moe_quantize_mxfp4(v, 4, 40, 64, v, v, None) == INVALID and b"K=40" in lib.moe_last_error()
    assert lib.moe_quantize_mxfp4(v, 4, 64, 12, v, v, None) == INVALID and b"N=12" in lib.moe_last_error()
    assert lib.moe_quantize_mxfp4(v, 0, 64, 64, v, v, None) == INVALID
    assert lib.moe_quantize_mxfp4(v, 4, 64, 64, ctypes.c_void_p(FAKE + 8), v, None) == INVALID
    assert b"aligned" in lib.moe_last_error()


def _fwd_fp8(lib, T=4, H=64, E=8, k=2, I=64, ptrs=None, ws_bytes=1 << 30, path=0):
    vp = [ctypes.c_void_p(p) for p in (ptrs or [FAKE] * 10)]
    return lib.moe_forward_fp8_ex(*vp[:9], T, H, E, k, I, vp[9], None, None, ctypes.c_void_p(FAKE), ws_bytes, path,
                                  None)


def test_fp8_calls_validate(lib):
    v = ctypes.c_void_p(FAKE)
    # H and I must be multiples of 16 (16-byte code rows)
    assert _fwd_fp8(lib, H=40) == INVALID and b"multiples of 16" in lib.moe_last_error()
    assert _fwd_fp8(lib, I=24) == INVALID
    for i in range(10):
        p = [FAKE] * 10
        p[i] = 0
        assert _fwd_fp8(lib, ptrs=p) == INVALID
        assert b"is NULL" in lib.moe_last_error()
    need = lib.moe_workspace_bytes_fp8(4, 64, 8, 2, 64)
    assert need > lib.moe_workspace_bytes(4, 64, 8, 2, 64)
    assert _fwd_fp8(lib, ws_bytes=need - 1) == WORKSPACE
    assert _fwd_fp8(lib, T=0) == OK
    assert _fwd_fp8(lib, path=7) == INVALID and b"unknown path" in lib.moe_last_error()
    assert lib.moe_gate_up_fp8(v, v, v, v, v, v, v, v, 4, 72, 8, 2, 64, v, 0, None) == INVALID
    assert lib.moe_down_fp8(v, None, v, v, v, v, v, 4, 64, 8, 2, 64, v, 0, None) == INVALID
    assert lib.moe_gate_up_fp8(v, v, v, v, v, v, v, v, 4, 64, 8, 2, 64, v, 3, None) == INVALID
    # the quantisers: K % 16 == 0, N % 8 == 0, codes 16-byte aligned
    assert lib.moe_quantize_fp8(v, 4, 40, 64, v, v, None) == INVALID and b"K=40" in lib.moe_last_error()
    assert lib.moe_quantize_fp8(v, 4, 64, 12, v, v, None) == INVALID and b"N=12" in lib.moe_last_error()
    assert lib.moe_quantize_fp8(v, 0, 64, 64, v, v, None) == INVALID
    assert lib.moe_quantize_fp8(v, 4, 64, 64, ctypes.c_void_p(FAKE + 8), v, None) == INVALID
    assert lib.moe_quantize_rows_fp8(v, -1, 64, v, v, None) == INVALID
    assert lib.moe_quantize_rows_fp8(v, 4, 24, v, v, None) == INVALID and b"K=24" in lib.moe_last_error()
    assert lib.moe_quantize_rows_fp8(v, 4, 64, v, ctypes.c_void_p(FAKE + 2), None) == INVALID
    assert lib.moe_workspace_bytes_fp8(4, 64, 0, 2, 64) == 0


def test_padded_calls_validate(lib):
    v = ctypes.c_void_p(FAKE)
    p = [ctypes.c_void_p(FAKE)] * 8

    def call(n_valid=None, counts=None, path=0, T=4, ws=1 << 30):
        return lib.moe_forward_padded(*p[:7], T, 64, 8, 2, 64, n_valid, p[7], None, None, counts, v, ws, path, None)

    assert call(n_valid=ctypes.c_void_p(FAKE + 2)) == INVALID and b"n_valid" in lib.moe_last_error()
    assert call(counts=ctypes.c_void_p(FAKE + 1)) == INVALID and b"expert_counts_out" in lib.moe_last_error()
    assert call(path=9) == INVALID and b"unknown path" in lib.moe_last_error()
    assert call(ws=16) == WORKSPACE
    assert call(T=0, n_valid=v, counts=v) == OK


def test_noalloc_forward_validates_before_touching_the_gpu(lib):
    v = ctypes.c_void_p(FAKE)
    p = [v] * 7
    fn = lib.moe_forward_noalloc
    assert fn(*p, 0, 2880, 32, 4, 2880, v, None, None, None) == OK
    assert fn(None, *p[1:], 4, 64, 8, 2, 64, v, None, None, None) == INVALID and b"x is NULL" in lib.moe_last_error()
    assert fn(*p, 4, 64, 8, 2, 64, None, None, None, None) == INVALID and b"y is NULL" in lib.moe_last_error()
    assert fn(*p, 4, 64, 8, 9, 64, v, None, None, None) == INVALID and b"k=9" in lib.moe_last_error()
    assert fn(*p, 4, 64, 8, 2, 64, v, ctypes.c_void_p(FAKE + 2), None, None) == INVALID
    # beyond the 64 MiB array: rejected with the size it would need
    assert fn(*p, 4096, 2880, 32, 4, 2880, v, None, None, None) == INVALID
    msg = lib.moe_last_error()
    assert b"moe_forward_noalloc" in msg and b"scratch" in msg and str(64 << 20).encode() in msg


def test_probe_calls_validate(lib):
    v = ctypes.c_void_p(FAKE)
    assert lib.moe_probe_mfma_bf16(0, 4, v, None) == INVALID and b"iters" in lib.moe_last_error()
    assert lib.moe_probe_mfma_bf16(1 << 20, 4, v, None) == INVALID
    assert lib.moe_probe_mfma_bf16(16, 0, v, None) == INVALID and b"workgroups" in lib.moe_last_error()
    assert lib.moe_probe_mfma_bf16(16, 4, None, None) == INVALID and b"out" in lib.moe_last_error()
    assert lib.moe_probe_read(v, 24, 4, v, None) == INVALID and b"multiple of 16" in lib.moe_last_error()
    assert lib.moe_probe_read(ctypes.c_void_p(FAKE + 8), 32, 4, v, None) == INVALID
    assert lib.moe_probe_read(v, 32, 70000, v, None) == INVALID and b"workgroups" in lib.moe_last_error()
    dot = lib.moe_probe_mfma_dot_bf16
    assert dot(v, v, 24, 64, v, None) == INVALID and b"M=24" in lib.moe_last_error()
    assert dot(v, v, 0, 64, v, None) == INVALID
    assert dot(v, v, 16, 48, v, None) == INVALID and b"K=48" in lib.moe_last_error()
    assert dot(v, v, 16 * 65536, 64, v, None) == INVALID
    assert dot(v, v, 16 * 40000, 1 << 16, v, None) == INVALID and b"2 GiB" in lib.moe_last_error()
    assert dot(ctypes.c_void_p(FAKE + 4), v, 16, 64, v, None) == INVALID
    assert dot(v, None, 16, 64, v, None) == INVALID
    assert dot(v, v, 16, 64, None, None) == INVALID and b"out" in lib.moe_last_error()


@pytest.mark.parametrize("name", ["moe_forward_padded_mxfp4", "moe_forward_padded_fp8"])
def test_padded_quantised_calls_validate(lib, name):
    v = ctypes.c_void_p(FAKE)
    p = [ctypes.c_void_p(FAKE)] * 10
    fn = getattr(lib, name)

    def call(n_valid=None, counts=None, path=0, T=4, ws=1 << 30, H=64, I=64):
        return fn(*p[:9], T, H, 8, 2, I, n_valid, p[9], None, None, counts, v, ws, path, None)

    assert call(n_valid=ctypes.c_void_p(FAKE + 2)) == INVALID and b"n_valid" in lib.moe_last_error()
    assert call(counts=ctypes.c_void_p(FAKE + 1)) == INVALID and b"expert_counts_out" in lib.moe_last_error()
    assert call(path=9) == INVALID and b"unknown path" in lib.moe_last_error()
    assert call(ws=16) == WORKSPACE
    assert call(H=40) == INVALID          # not a multiple of the format's block (32 for MXFP4, 16 for FP8)
    assert call(T=0, n_valid=v, counts=v) == OK


@pytest.mark.parametrize("name", ["moe_forward_ep_mxfp4", "moe_forward_ep_fp8"])
@pytest.mark.parametrize("e_begin,n_local", [(-1, 2), (0, 0), (7, 2), (0, 9)])
def test_ep_quantised_calls_reject_bad_ranges(lib, name, e_begin, n_local):
    p = [ctypes.c_void_p(FAKE)] * 10
    st = getattr(lib, name)(*p[:9], 4, 64, 8, 2, 64, e_begin, n_local, p[9], None, None, p[0], 1 << 30, 0, None)
    assert st == INVALID and b"local experts" in lib.moe_last_error()


@pytest.mark.parametrize("name", ["moe_forward_ep_mxfp4", "moe_forward_ep_fp8"])
def test_ep_quantised_calls_accept_valid_ranges(lib, name):
    p = [ctypes.c_void_p(FAKE)] * 10
    for lo, n in [(0, 8), (0, 1), (7, 1), (3, 4)]:
        # T = 0: every check passes and nothing is enqueued
        assert getattr(lib, name)(*p[:9], 0, 64, 8, 2, 64, lo, n, p[9], None, None, p[0], 1 << 30, 0, None) == OK
