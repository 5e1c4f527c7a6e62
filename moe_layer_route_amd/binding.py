"""Thin Python binding of the C ABI in ``include/moe_layer_route.h``.

Argument marshalling only: every step of the MoE block runs in the HIP kernels
of ``libmoe_layer_route.so``.  PyTorch provides device memory (``torch.empty``)
and the current stream; nothing here computes on tensor values.  If the
library has not been built, every call raises ``MoEError`` -- there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

import torch

PATH_AUTO, PATH_GEMV, PATH_GEMM = 0, 1, 2
_PATHS = {"auto": PATH_AUTO, "gemv": PATH_GEMV, "gemm": PATH_GEMM}
ROUTE_AUTO, ROUTE_EXACT, ROUTE_MFMA = 0, 1, 2
_ROUTES = {"auto": ROUTE_AUTO, "exact": ROUTE_EXACT, "mfma": ROUTE_MFMA}

# The in-tree build; MOE_LAYER_ROUTE_LIB may name another build of the same library.
LIB_PATH = os.environ.get("MOE_LAYER_ROUTE_LIB") or os.path.join(
    os.path.dirname(os.path.abspath(__file__)), "libmoe_layer_route.so")

EXPORTS = ("moe_abi_version", "moe_status_str", "moe_last_error", "moe_workspace_bytes", "moe_expert_path",
           "moe_route", "moe_route_ex",
           "moe_forward", "moe_forward_ex", "moe_forward_ep", "moe_permute", "moe_gate_up", "moe_down",
           "moe_combine", "moe_quantize_mxfp4", "moe_forward_mxfp4", "moe_forward_mxfp4_ex", "moe_gate_up_mxfp4",
           "moe_down_mxfp4", "moe_quantize_fp8", "moe_quantize_rows_fp8", "moe_workspace_bytes_fp8",
           "moe_forward_fp8", "moe_forward_fp8_ex", "moe_gate_up_fp8", "moe_down_fp8", "moe_forward_padded",
           "moe_probe_mfma_bf16", "moe_probe_read", "moe_forward_padded_mxfp4", "moe_forward_padded_fp8",
           "moe_forward_ep_mxfp4", "moe_forward_ep_fp8", "moe_probe_mfma_dot_bf16",
           "moe_forward_noalloc")


class MoEError(RuntimeError):
    """A call into the native library failed (or the library is missing)."""


_lib = None

_vp, _i64, _i32, _sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
_SIGS = {
    "moe_abi_version": (ctypes.c_int, []),
    "moe_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_workspace_bytes": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "moe_expert_path": (ctypes.c_int, [_i64, _i32, _i32]),
    "moe_route": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_route_ex": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _i32, _vp, _vp, _i32, _vp]),
    "moe_forward": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _vp]),
    "moe_forward_ex": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _i32, _vp]),
    "moe_forward_ep": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 4
                       + [_sz, _i32, _vp]),
    "moe_permute": (ctypes.c_int, [_vp, _i64, _i32, _i32, _vp, _vp, _vp, _vp, _vp]),
    "moe_gate_up": (ctypes.c_int, [_vp] * 6 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_down": (ctypes.c_int, [_vp] * 5 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_combine": (ctypes.c_int, [_vp, _vp, _vp, _i64, _i32, _i32, _vp, _vp]),
    "moe_quantize_mxfp4": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_forward_mxfp4": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _vp]),
    "moe_forward_mxfp4_ex": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _i32, _vp]),
    "moe_gate_up_mxfp4": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_down_mxfp4": (ctypes.c_int, [_vp] * 6 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_quantize_fp8": (ctypes.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp]),
    "moe_forward_padded": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 5 + [_vp, _sz, _i32, _vp]),
    "moe_quantize_rows_fp8": (ctypes.c_int, [_vp, _i64, _i32, _vp, _vp, _vp]),
    "moe_workspace_bytes_fp8": (_sz, [_i64, _i32, _i32, _i32, _i32]),
    "moe_forward_fp8": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _vp]),
    "moe_forward_fp8_ex": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4 + [_sz, _i32, _vp]),
    "moe_gate_up_fp8": (ctypes.c_int, [_vp] * 8 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_down_fp8": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32, _vp, _i32, _vp]),
    "moe_forward_padded_mxfp4": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 5
                                 + [_vp, _sz, _i32, _vp]),
    "moe_forward_padded_fp8": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 5
                               + [_vp, _sz, _i32, _vp]),
    "moe_forward_ep_mxfp4": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 4
                             + [_sz, _i32, _vp]),
    "moe_forward_ep_fp8": (ctypes.c_int, [_vp] * 9 + [_i64, _i32, _i32, _i32, _i32, _i32, _i32] + [_vp] * 4
                           + [_sz, _i32, _vp]),
    "moe_probe_mfma_bf16": (ctypes.c_int, [_i32, _i32, _vp, _vp]),
    "moe_probe_read": (ctypes.c_int, [_vp, _sz, _i32, _vp, _vp]),
    "moe_probe_mfma_dot_bf16": (ctypes.c_int, [_vp, _vp, _i32, _i32, _vp, _vp]),
    "moe_forward_noalloc": (ctypes.c_int, [_vp] * 7 + [_i64, _i32, _i32, _i32, _i32] + [_vp] * 4),
}


def library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the native library (once).  Raises MoEError if it is missing."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise MoEError(f"native library not built: {path} (run __graft_entry__.build())")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def _check(status: int, what: str):
    if status != 0:
        lib = library()
        msg = lib.moe_last_error().decode()
        raise MoEError(f"{what}: {lib.moe_status_str(status).decode()} ({status}): {msg}")


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dev(*ts):
    for t in ts:
        if t is not None:
            if not t.is_cuda:
                raise MoEError("tensors must be on the GPU")
            if not t.is_contiguous():
                raise MoEError("tensors must be contiguous")


# ---------------------------------------------------------------------------
# argument checks: shapes and dtypes are checked against the sizes the call
# passes to the library, before anything is enqueued (a short weight or a
# too-small output would otherwise be read or written out of bounds)
# ---------------------------------------------------------------------------
def _req(t, name, shape, dtype=None, bf16=False):
    """t has exactly this shape (and dtype, or 2-byte elements for bf16 bit patterns)."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise MoEError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    if dtype is not None and t.dtype != dtype:
        raise MoEError(f"{name}: expected {dtype}, got {t.dtype}")
    if bf16 and t.element_size() != 2:
        raise MoEError(f"{name}: expected a 2-byte (bf16) tensor, got {t.dtype}")


def _req_rows(t, name, min_rows, cols, dtype):
    """A buffer of at least min_rows rows of cols elements (cols None: 1-D)."""
    if t is None:
        return
    ok = t.dim() == (1 if cols is None else 2) and t.shape[0] >= min_rows and (cols is None or t.shape[1] == cols)
    if not ok:
        want = f"({min_rows}+,)" if cols is None else f"({min_rows}+, {cols})"
        raise MoEError(f"{name}: expected shape {want}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise MoEError(f"{name}: expected {dtype}, got {t.dtype}")


def _dims(t, name, n):
    if t.dim() != n:
        raise MoEError(f"{name}: expected {n} dimensions, got shape {tuple(t.shape)}")


def _route_args(x, Wr, br, k, topk_ids=None, topk_w=None):
    """x [T][H], Wr [E][H], br [E] (bf16); optional topk_ids int32 / topk_w float32 [T][k]."""
    _dims(x, "x", 2)
    _dims(Wr, "Wr", 2)
    T, H = x.shape
    E = Wr.shape[0]
    _req(x, "x", (T, H), bf16=True)
    _req(Wr, "Wr", (E, H), bf16=True)
    _req(br, "br", (E,), bf16=True)
    _req(topk_ids, "topk_ids", (T, k), torch.int32)
    _req(topk_w, "topk_w", (T, k), torch.float32)
    return T, H, E


def _bf16_experts(Wgu, bgu, Wd, bd, n, H):
    """Wgu [n][H][2I], bgu [n][2I], Wd [n][I][H], bd [n][H] (bf16); returns I."""
    _dims(Wd, "Wd", 3)
    I = Wd.shape[1]
    _req(Wgu, "Wgu", (n, H, 2 * I), bf16=True)
    _req(bgu, "bgu", (n, 2 * I), bf16=True)
    _req(Wd, "Wd", (n, I, H), bf16=True)
    _req(bd, "bd", (n, H), bf16=True)
    return I


def _mxfp4_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, n, H):
    """MXFP4 codes [n][N][K/2] and scales [n][K/32][N] (uint8), biases bf16; returns I."""
    _dims(Wd_q, "Wd_q", 3)
    I = 2 * Wd_q.shape[2]
    if H % 32 or I % 32:
        raise MoEError(f"MXFP4 weights need H and I divisible by 32, got H={H}, I={I}")
    _req(Wgu_q, "Wgu_q", (n, 2 * I, H // 2), torch.uint8)
    _req(Wgu_s, "Wgu_s", (n, H // 32, 2 * I), torch.uint8)
    _req(bgu, "bgu", (n, 2 * I), bf16=True)
    _req(Wd_q, "Wd_q", (n, H, I // 2), torch.uint8)
    _req(Wd_s, "Wd_s", (n, I // 32, H), torch.uint8)
    _req(bd, "bd", (n, H), bf16=True)
    return I


def _fp8_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, n, H):
    """FP8 codes [n][N][K] (uint8), one float32 scale per expert, biases bf16; returns I."""
    _dims(Wd_q, "Wd_q", 3)
    I = Wd_q.shape[2]
    _req(Wgu_q, "Wgu_q", (n, 2 * I, H), torch.uint8)
    _req(Wgu_s, "Wgu_s", (n,), torch.float32)
    _req(bgu, "bgu", (n, 2 * I), bf16=True)
    _req(Wd_q, "Wd_q", (n, H, I), torch.uint8)
    _req(Wd_s, "Wd_s", (n,), torch.float32)
    _req(bd, "bd", (n, H), bf16=True)
    return I


def _local_experts(e_begin, n_local, E):
    if e_begin < 0 or n_local < 1 or e_begin + n_local > E:
        raise MoEError(f"expert range [{e_begin}, {e_begin + n_local}) is not inside [0, {E})")


def _padded_args(n_valid, expert_counts, E):
    if n_valid is not None and (n_valid.dtype != torch.int32 or n_valid.numel() != 1):
        raise MoEError("n_valid must be a one-element int32 tensor")
    if expert_counts is not None and (expert_counts.dtype != torch.int32 or expert_counts.numel() != E):
        raise MoEError("expert_counts must be an int32 tensor of E elements")


def path_code(path) -> int:
    if isinstance(path, str):
        return _PATHS[path]
    return int(path)


def expert_path(T: int, E: int, k: int) -> str:
    """The expert path ("gemv" or "gemm") the library picks for these sizes."""
    return {PATH_GEMV: "gemv", PATH_GEMM: "gemm"}[int(library().moe_expert_path(T, E, k))]


def workspace_bytes(T: int, H: int, E: int, k: int, I: int) -> int:
    return int(library().moe_workspace_bytes(T, H, E, k, I))


def alloc_workspace(T: int, H: int, E: int, k: int, I: int, device=None) -> torch.Tensor:
    n = workspace_bytes(T, H, E, k, I)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def moe_route(x, Wr, br, k: int, topk_ids=None, topk_w=None, method="auto", stream=None):
    """Router: returns (topk_ids int32 [T,k], topk_w float32 [T,k]).

    method: "auto", "exact" or "mfma" (same decision; speed only)."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    _dev(x, Wr, br)
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=x.device)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=x.device)
    _dev(topk_ids, topk_w)
    m = _ROUTES[method] if isinstance(method, str) else int(method)
    _check(library().moe_route_ex(_ptr(x), _ptr(Wr), _ptr(br), T, H, E, k, _ptr(topk_ids), _ptr(topk_w), m,
                                  _stream(stream)), "moe_route")
    return topk_ids, topk_w


def moe_forward(x, Wr, br, Wgu, bgu, Wd, bd, k: int = 4, y=None, workspace=None, topk_ids=None,
                topk_w=None, path="auto", stream=None):
    """Whole MoE block forward; returns y (bf16 [T,H]).

    topk_ids / topk_w: optional preallocated outputs of the routing decision.
    workspace: optional uint8 device buffer of at least workspace_bytes(...)."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _bf16_experts(Wgu, bgu, Wd, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _dev(x, Wr, br, Wgu, bgu, Wd, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w)
    st = library().moe_forward_ex(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu), _ptr(bgu), _ptr(Wd), _ptr(bd),
                                  T, H, E, k, I, _ptr(y), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), path_code(path),
                                  _stream(stream))
    _check(st, "moe_forward")
    return y


def moe_forward_noalloc(x, Wr, br, Wgu, bgu, Wd, bd, k: int = 4, y=None, topk_ids=None, topk_w=None, stream=None):
    """moe_forward on the library's own scratch array (no workspace argument;
    the call itself allocates nothing).  For T*k*(2I + 4H + 16) bytes up to
    64 MiB; calls that overlap on one GPU race.  Returns y (bf16 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    _bf16_experts(Wgu, bgu, Wd, bd, E, H)
    I = Wd.shape[1]
    _req(y, "y", (T, H), torch.bfloat16)
    _dev(x, Wr, br, Wgu, bgu, Wd, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    _dev(y, topk_ids, topk_w)
    _check(library().moe_forward_noalloc(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu), _ptr(bgu), _ptr(Wd), _ptr(bd),
                                         T, H, E, k, I, _ptr(y), _ptr(topk_ids), _ptr(topk_w), _stream(stream)),
           "moe_forward_noalloc")
    return y


def moe_forward_ex(*args, **kw):
    return moe_forward(*args, **kw)


def moe_forward_ep(x, Wr, br, Wgu_local, bgu_local, Wd_local, bd_local, e_begin: int, k: int = 4,
                   y_partial=None, workspace=None, topk_ids=None, topk_w=None, path="auto", stream=None):
    """One expert-parallel rank's share: experts [e_begin, e_begin + n_local) of the E
    routed ones (n_local = Wgu_local.shape[0]); returns y_partial (float32 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    _dims(Wgu_local, "Wgu_local", 3)
    n_local = Wgu_local.shape[0]
    _local_experts(e_begin, n_local, E)
    I = _bf16_experts(Wgu_local, bgu_local, Wd_local, bd_local, n_local, H)
    _req(y_partial, "y_partial", (T, H), torch.float32)
    _dev(x, Wr, br, Wgu_local, bgu_local, Wd_local, bd_local)
    if y_partial is None:
        y_partial = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y_partial, workspace, topk_ids, topk_w)
    st = library().moe_forward_ep(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_local), _ptr(bgu_local),
                                  _ptr(Wd_local), _ptr(bd_local), T, H, E, k, I, e_begin, n_local,
                                  _ptr(y_partial), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), path_code(path),
                                  _stream(stream))
    _check(st, "moe_forward_ep")
    return y_partial


def moe_permute(topk_ids, E: int, stream=None):
    """Expert-contiguous order: returns (cnt [E], off [E+1], rows [T*k], pos [T*k]) int32."""
    _dims(topk_ids, "topk_ids", 2)
    T, k = topk_ids.shape
    _req(topk_ids, "topk_ids", (T, k), torch.int32)
    _dev(topk_ids)
    dev = topk_ids.device
    cnt = torch.empty(E, dtype=torch.int32, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rows = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    pos = torch.empty(max(T * k, 1), dtype=torch.int32, device=dev)
    _check(library().moe_permute(_ptr(topk_ids), T, E, k, _ptr(cnt), _ptr(off), _ptr(rows), _ptr(pos),
                                 _stream(stream)), "moe_permute")
    return cnt, off, rows[:T * k], pos[:T * k]


def moe_gate_up(x, Wgu, bgu, cnt, off, rows, k: int, path="auto", h=None, stream=None):
    """Per-expert gate_up GEMM + bias + GLU; returns h (bf16 [T*k, I], permuted order)."""
    _dims(x, "x", 2)
    _dims(Wgu, "Wgu", 3)
    T, H = x.shape
    E, I = Wgu.shape[0], Wgu.shape[2] // 2
    _req(x, "x", (T, H), bf16=True)
    _req(Wgu, "Wgu", (E, H, 2 * I), bf16=True)
    _req(bgu, "bgu", (E, 2 * I), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(rows, "rows", T * k, None, torch.int32)
    _req_rows(h, "h", T * k, I, torch.bfloat16)
    _dev(x, Wgu, bgu, cnt, off, rows)
    if h is None:
        h = torch.empty((max(T * k, 1), I), dtype=torch.bfloat16, device=x.device)
    _check(library().moe_gate_up(_ptr(x), _ptr(Wgu), _ptr(bgu), _ptr(cnt), _ptr(off), _ptr(rows), T, H, E,
                                 k, I, _ptr(h), path_code(path), _stream(stream)), "moe_gate_up")
    return h[:T * k]


def moe_down(h, Wd, bd, cnt, off, T: int, k: int, path="auto", o=None, stream=None):
    """Per-expert down GEMM + bias; returns o (float32 [T*k, H], permuted order)."""
    _dims(Wd, "Wd", 3)
    E, I, H = Wd.shape
    _req(Wd, "Wd", (E, I, H), bf16=True)
    _req(bd, "bd", (E, H), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(h, "h", T * k, I, torch.bfloat16)
    _req_rows(o, "o", T * k, H, torch.float32)
    _dev(h, Wd, bd, cnt, off)
    if o is None:
        o = torch.empty((max(T * k, 1), H), dtype=torch.float32, device=h.device)
    _check(library().moe_down(_ptr(h), _ptr(Wd), _ptr(bd), _ptr(cnt), _ptr(off), T, H, E, k, I, _ptr(o),
                              path_code(path), _stream(stream)), "moe_down")
    return o[:T * k]


def moe_combine(o, pos, topk_w, y=None, stream=None):
    """Weighted combine; returns y (bf16 [T, H])."""
    _dims(topk_w, "topk_w", 2)
    _dims(o, "o", 2)
    T, k = topk_w.shape
    H = o.shape[1]
    _req(topk_w, "topk_w", (T, k), torch.float32)
    _req_rows(o, "o", T * k, H, torch.float32)
    _req_rows(pos, "pos", T * k, None, torch.int32)
    _req(y, "y", (T, H), torch.bfloat16)
    _dev(o, pos, topk_w)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=o.device)
    _check(library().moe_combine(_ptr(o), _ptr(pos), _ptr(topk_w), T, H, k, _ptr(y), _stream(stream)),
           "moe_combine")
    return y


# ---------------------------------------------------------------------------
# MXFP4 expert weights: codes uint8 [E][N][K/2] and scales uint8 [E][K/32][N]
# (gate_up: K = H, N = 2I; down: K = I, N = H)
# ---------------------------------------------------------------------------
def _u8(*ts):
    for t in ts:
        if t.dtype != torch.uint8:
            raise MoEError(f"expected a uint8 tensor, got {t.dtype}")


def moe_quantize_mxfp4(W, codes=None, scales=None, stream=None):
    """bf16 weights [E][K][N] (x.W form) -> (codes uint8 [E][N][K/2], scales uint8 [E][K/32][N])."""
    _dims(W, "W", 3)
    E, K, N = W.shape
    _req(W, "W", (E, K, N), bf16=True)
    _req(codes, "codes", (E, N, K // 2), torch.uint8)
    _req(scales, "scales", (E, K // 32, N), torch.uint8)
    _dev(W)
    if codes is None:
        codes = torch.empty((E, N, K // 2), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((E, K // 32, N), dtype=torch.uint8, device=W.device)
    _dev(codes, scales)
    _u8(codes, scales)
    _check(library().moe_quantize_mxfp4(_ptr(W), E, K, N, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_mxfp4")
    return codes, scales


def moe_forward_mxfp4(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int = 4, y=None, workspace=None,
                      topk_ids=None, topk_w=None, path="auto", stream=None):
    """moe_forward with MXFP4 expert weights; returns y (bf16 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _mxfp4_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _dev(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w)
    st = library().moe_forward_mxfp4_ex(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu),
                                        _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), T, H, E, k, I, _ptr(y), _ptr(topk_ids),
                                        _ptr(topk_w), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        path_code(path), _stream(stream))
    _check(st, "moe_forward_mxfp4")
    return y


def moe_gate_up_mxfp4(x, Wgu_q, Wgu_s, bgu, cnt, off, rows, k: int, h=None, path="auto", stream=None):
    """MXFP4 gate_up + bias + GLU; returns h (bf16 [T*k, I], permuted order)."""
    _dims(x, "x", 2)
    _dims(Wgu_q, "Wgu_q", 3)
    T, H = x.shape
    E, I = Wgu_q.shape[0], Wgu_q.shape[1] // 2
    _req(x, "x", (T, H), bf16=True)
    _req(Wgu_q, "Wgu_q", (E, 2 * I, H // 2), torch.uint8)
    _req(Wgu_s, "Wgu_s", (E, H // 32, 2 * I), torch.uint8)
    _req(bgu, "bgu", (E, 2 * I), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(rows, "rows", T * k, None, torch.int32)
    _req_rows(h, "h", T * k, I, torch.bfloat16)
    _dev(x, Wgu_q, Wgu_s, bgu, cnt, off, rows)
    if h is None:
        h = torch.empty((max(T * k, 1), I), dtype=torch.bfloat16, device=x.device)
    _check(library().moe_gate_up_mxfp4(_ptr(x), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu), _ptr(cnt), _ptr(off),
                                       _ptr(rows), T, H, E, k, I, _ptr(h), path_code(path), _stream(stream)),
           "moe_gate_up_mxfp4")
    return h[:T * k]


def moe_down_mxfp4(h, Wd_q, Wd_s, bd, cnt, off, T: int, k: int, o=None, path="auto", stream=None):
    """MXFP4 down + bias; returns o (float32 [T*k, H], permuted order)."""
    _dims(Wd_q, "Wd_q", 3)
    E, H, I2 = Wd_q.shape
    I = 2 * I2
    _req(Wd_q, "Wd_q", (E, H, I2), torch.uint8)
    _req(Wd_s, "Wd_s", (E, I // 32, H), torch.uint8)
    _req(bd, "bd", (E, H), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(h, "h", T * k, I, torch.bfloat16)
    _req_rows(o, "o", T * k, H, torch.float32)
    _dev(h, Wd_q, Wd_s, bd, cnt, off)
    if o is None:
        o = torch.empty((max(T * k, 1), H), dtype=torch.float32, device=h.device)
    _check(library().moe_down_mxfp4(_ptr(h), _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), _ptr(cnt), _ptr(off), T, H, E,
                                    k, I, _ptr(o), path_code(path), _stream(stream)), "moe_down_mxfp4")
    return o[:T * k]


# ---------------------------------------------------------------------------
# FP8 W8A8
# ---------------------------------------------------------------------------
def workspace_bytes_fp8(T: int, H: int, E: int, k: int, I: int) -> int:
    return int(library().moe_workspace_bytes_fp8(T, H, E, k, I))


def alloc_workspace_fp8(T: int, H: int, E: int, k: int, I: int, device=None) -> torch.Tensor:
    n = workspace_bytes_fp8(T, H, E, k, I)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def moe_quantize_fp8(W, codes=None, scales=None, stream=None):
    """bf16 weights [E][K][N] (x.W form) -> (codes uint8 [E][N][K], scales float32 [E])."""
    _dims(W, "W", 3)
    E, K, N = W.shape
    _req(W, "W", (E, K, N), bf16=True)
    _req(codes, "codes", (E, N, K), torch.uint8)
    _req(scales, "scales", (E,), torch.float32)
    _dev(W)
    if codes is None:
        codes = torch.empty((E, N, K), dtype=torch.uint8, device=W.device)
    if scales is None:
        scales = torch.empty((E,), dtype=torch.float32, device=W.device)
    _dev(codes, scales)
    _check(library().moe_quantize_fp8(_ptr(W), E, K, N, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_fp8")
    return codes, scales


def moe_quantize_rows_fp8(a, codes=None, scales=None, stream=None):
    """bf16 rows [R][K] -> (codes uint8 [R][K], scales float32 [R])."""
    _dims(a, "a", 2)
    R, K = a.shape
    _req(a, "a", (R, K), bf16=True)
    _req(codes, "codes", (R, K), torch.uint8)
    _req(scales, "scales", (R,), torch.float32)
    _dev(a)
    if codes is None:
        codes = torch.empty((R, K), dtype=torch.uint8, device=a.device)
    if scales is None:
        scales = torch.empty((R,), dtype=torch.float32, device=a.device)
    _dev(codes, scales)
    _check(library().moe_quantize_rows_fp8(_ptr(a), R, K, _ptr(codes), _ptr(scales), _stream(stream)),
           "moe_quantize_rows_fp8")
    return codes, scales


def moe_forward_fp8(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int = 4, y=None, workspace=None,
                    topk_ids=None, topk_w=None, path="auto", stream=None):
    """moe_forward with FP8 W8A8 experts; returns y (bf16 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _fp8_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _dev(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace_fp8(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w)
    st = library().moe_forward_fp8_ex(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu),
                                      _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), T, H, E, k, I, _ptr(y), _ptr(topk_ids),
                                      _ptr(topk_w), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      path_code(path), _stream(stream))
    _check(st, "moe_forward_fp8")
    return y


def moe_gate_up_fp8(xq, sx, Wgu_q, Wgu_s, bgu, cnt, off, rows, k: int, h=None, path="auto", stream=None):
    """FP8 gate_up + bias + GLU from x codes and row scales; returns h (bf16 [T*k, I], permuted order)."""
    _dims(xq, "xq", 2)
    _dims(Wgu_q, "Wgu_q", 3)
    T, H = xq.shape
    E, I = Wgu_q.shape[0], Wgu_q.shape[1] // 2
    _req(xq, "xq", (T, H), torch.uint8)
    _req(sx, "sx", (T,), torch.float32)
    _req(Wgu_q, "Wgu_q", (E, 2 * I, H), torch.uint8)
    _req(Wgu_s, "Wgu_s", (E,), torch.float32)
    _req(bgu, "bgu", (E, 2 * I), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(rows, "rows", T * k, None, torch.int32)
    _req_rows(h, "h", T * k, I, torch.bfloat16)
    _dev(xq, sx, Wgu_q, Wgu_s, bgu, cnt, off, rows)
    if h is None:
        h = torch.empty((T * k, I), dtype=torch.bfloat16, device=xq.device)
    _dev(h)
    _check(library().moe_gate_up_fp8(_ptr(xq), _ptr(sx), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu), _ptr(cnt), _ptr(off),
                                     _ptr(rows), T, H, E, k, I, _ptr(h), path_code(path), _stream(stream)),
           "moe_gate_up_fp8")
    return h


def moe_down_fp8(hq, sh, Wd_q, Wd_s, bd, cnt, off, T: int, k: int, o=None, path="auto", stream=None):
    """FP8 down + bias from h codes and row scales; returns o (float32 [T*k, H], permuted order)."""
    _dims(Wd_q, "Wd_q", 3)
    E, H, I = Wd_q.shape
    _req(Wd_q, "Wd_q", (E, H, I), torch.uint8)
    _req(Wd_s, "Wd_s", (E,), torch.float32)
    _req(bd, "bd", (E, H), bf16=True)
    _req(cnt, "cnt", (E,), torch.int32)
    _req(off, "off", (E + 1,), torch.int32)
    _req_rows(hq, "hq", T * k, I, torch.uint8)
    _req_rows(sh, "sh", T * k, None, torch.float32)
    _req_rows(o, "o", T * k, H, torch.float32)
    _dev(hq, sh, Wd_q, Wd_s, bd, cnt, off)
    if o is None:
        o = torch.empty((T * k, H), dtype=torch.float32, device=hq.device)
    _dev(o)
    _check(library().moe_down_fp8(_ptr(hq), _ptr(sh), _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), _ptr(cnt), _ptr(off), T, H,
                                  E, k, I, _ptr(o), path_code(path), _stream(stream)), "moe_down_fp8")
    return o


def moe_forward_padded(x, Wr, br, Wgu, bgu, Wd, bd, k: int = 4, n_valid=None, y=None, workspace=None,
                       topk_ids=None, topk_w=None, expert_counts=None, path="auto", stream=None):
    """moe_forward over a batch whose rows from n_valid (a device int32
    tensor of one element, read when the call runs) are padding; returns y.
    expert_counts (device int32 [E]), if given, receives the per-expert loads."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _bf16_experts(Wgu, bgu, Wd, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _padded_args(n_valid, expert_counts, E)
    _dev(x, Wr, br, Wgu, bgu, Wd, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w, n_valid, expert_counts)
    st = library().moe_forward_padded(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu), _ptr(bgu), _ptr(Wd), _ptr(bd), T, H,
                                      E, k, I, _ptr(n_valid), _ptr(y), _ptr(topk_ids), _ptr(topk_w),
                                      _ptr(expert_counts), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(), path_code(path), _stream(stream))
    _check(st, "moe_forward_padded")
    return y


def moe_forward_padded_mxfp4(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int = 4, n_valid=None, y=None,
                             workspace=None, topk_ids=None, topk_w=None, expert_counts=None, path="auto",
                             stream=None):
    """moe_forward_padded with MXFP4 expert weights; returns y (bf16 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _mxfp4_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _padded_args(n_valid, expert_counts, E)
    _dev(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w, n_valid, expert_counts)
    st = library().moe_forward_padded_mxfp4(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu),
                                            _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), T, H, E, k, I, _ptr(n_valid), _ptr(y),
                                            _ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts), _ptr(workspace),
                                            workspace.numel() * workspace.element_size(), path_code(path),
                                            _stream(stream))
    _check(st, "moe_forward_padded_mxfp4")
    return y


def moe_forward_padded_fp8(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int = 4, n_valid=None, y=None,
                           workspace=None, topk_ids=None, topk_w=None, expert_counts=None, path="auto", stream=None):
    """moe_forward_padded with FP8 W8A8 experts; returns y (bf16 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    I = _fp8_experts(Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, E, H)
    _req(y, "y", (T, H), torch.bfloat16)
    _padded_args(n_valid, expert_counts, E)
    _dev(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd)
    if y is None:
        y = torch.empty((T, H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = alloc_workspace_fp8(T, H, E, k, I, x.device)
    _dev(y, workspace, topk_ids, topk_w, n_valid, expert_counts)
    st = library().moe_forward_padded_fp8(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q), _ptr(Wgu_s), _ptr(bgu),
                                          _ptr(Wd_q), _ptr(Wd_s), _ptr(bd), T, H, E, k, I, _ptr(n_valid), _ptr(y),
                                          _ptr(topk_ids), _ptr(topk_w), _ptr(expert_counts), _ptr(workspace),
                                          workspace.numel() * workspace.element_size(), path_code(path),
                                          _stream(stream))
    _check(st, "moe_forward_padded_fp8")
    return y


def moe_forward_ep_mxfp4(x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local,
                         e_begin: int, k: int = 4, y_partial=None, workspace=None, topk_ids=None, topk_w=None,
                         path="auto", stream=None):
    """moe_forward_ep with MXFP4 expert weights (the rank's n_local = Wgu_q_local.shape[0]
    experts from e_begin); returns y_partial (float32 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    _dims(Wgu_q_local, "Wgu_q_local", 3)
    n_local = Wgu_q_local.shape[0]
    _local_experts(e_begin, n_local, E)
    I = _mxfp4_experts(Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local, n_local, H)
    _req(y_partial, "y_partial", (T, H), torch.float32)
    _dev(x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local)
    if y_partial is None:
        y_partial = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace(T, H, E, k, I, x.device)
    _dev(y_partial, workspace, topk_ids, topk_w)
    st = library().moe_forward_ep_mxfp4(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q_local), _ptr(Wgu_s_local),
                                        _ptr(bgu_local), _ptr(Wd_q_local), _ptr(Wd_s_local), _ptr(bd_local), T, H,
                                        E, k, I, e_begin, n_local, _ptr(y_partial), _ptr(topk_ids), _ptr(topk_w),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        path_code(path), _stream(stream))
    _check(st, "moe_forward_ep_mxfp4")
    return y_partial


def moe_forward_ep_fp8(x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local,
                       e_begin: int, k: int = 4, y_partial=None, workspace=None, topk_ids=None, topk_w=None,
                       path="auto", stream=None):
    """moe_forward_ep with FP8 W8A8 experts (the rank's n_local = Wgu_q_local.shape[0]
    experts from e_begin); returns y_partial (float32 [T,H])."""
    T, H, E = _route_args(x, Wr, br, k, topk_ids, topk_w)
    _dims(Wgu_q_local, "Wgu_q_local", 3)
    n_local = Wgu_q_local.shape[0]
    _local_experts(e_begin, n_local, E)
    I = _fp8_experts(Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local, n_local, H)
    _req(y_partial, "y_partial", (T, H), torch.float32)
    _dev(x, Wr, br, Wgu_q_local, Wgu_s_local, bgu_local, Wd_q_local, Wd_s_local, bd_local)
    if y_partial is None:
        y_partial = torch.empty((T, H), dtype=torch.float32, device=x.device)
    if workspace is None:
        workspace = alloc_workspace_fp8(T, H, E, k, I, x.device)
    _dev(y_partial, workspace, topk_ids, topk_w)
    st = library().moe_forward_ep_fp8(_ptr(x), _ptr(Wr), _ptr(br), _ptr(Wgu_q_local), _ptr(Wgu_s_local),
                                      _ptr(bgu_local), _ptr(Wd_q_local), _ptr(Wd_s_local), _ptr(bd_local), T, H, E,
                                      k, I, e_begin, n_local, _ptr(y_partial), _ptr(topk_ids), _ptr(topk_w),
                                      _ptr(workspace), workspace.numel() * workspace.element_size(),
                                      path_code(path), _stream(stream))
    _check(st, "moe_forward_ep_fp8")
    return y_partial


# ---------------------------------------------------------------------------
# measurement probes (not part of the block)
# ---------------------------------------------------------------------------
def probe_mfma_bf16(iters: int, workgroups: int, out=None, stream=None):
    """Enqueue the MFMA rate probe; returns out (float32 [workgroups * 4], each
    2048 * iters when iters <= 8191).  Flops = workgroups * 4 * iters * 8 * 32768."""
    if out is None:
        out = torch.empty(workgroups * 4, dtype=torch.float32, device="cuda")
    _dev(out)
    _check(library().moe_probe_mfma_bf16(iters, workgroups, _ptr(out), _stream(stream)), "moe_probe_mfma_bf16")
    return out


def probe_read(buf, workgroups: int, out=None, stream=None):
    """Enqueue the streaming-read probe over buf (any dtype, contiguous, bytes % 16 == 0);
    returns out (int32 [workgroups * 4] holding uint32 XOR folds)."""
    _dev(buf)
    if out is None:
        out = torch.empty(workgroups * 4, dtype=torch.int32, device=buf.device)
    _dev(out)
    nbytes = buf.numel() * buf.element_size()
    _check(library().moe_probe_read(_ptr(buf), nbytes, workgroups, _ptr(out), _stream(stream)), "moe_probe_read")
    return out


def probe_mfma_dot_bf16(A, B, out=None, stream=None):
    """out[m][n] = A[m] . B[n] through the router's MFMA accumulation (bf16 A [M][K],
    B [16][K]; M % 16 == 0, K % 32 == 0); returns out (float32 [M][16])."""
    _dims(A, "A", 2)
    M, K = A.shape
    _req(A, "A", (M, K), bf16=True)
    _req(B, "B", (16, K), bf16=True)
    _req(out, "out", (M, 16), torch.float32)
    _dev(A, B)
    if out is None:
        out = torch.empty((M, 16), dtype=torch.float32, device=A.device)
    _dev(out)
    _check(library().moe_probe_mfma_dot_bf16(_ptr(A), _ptr(B), M, K, _ptr(out), _stream(stream)),
           "moe_probe_mfma_dot_bf16")
    return out
