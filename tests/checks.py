"""Tolerances and comparison helpers shared by the GPU parity tests.

Tolerance of y (the MoE block output): max |y - y_ref| <= 2e-2 * max |y_ref| and
mean relative error, read as the L1 ratio sum |y - y_ref| / sum |y_ref|, <= 5e-3,
with y_ref the float64 oracle and y computed from bf16 operands with float32
accumulation (h rounded to bf16 before the down GEMM, y rounded once to bf16).
topk_ids must match exactly; topk_w within 1e-4 absolute with each row summing
to 1 within 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

Y_MAX_REL = 2e-2
Y_L1_REL = 5e-3
W_ABS = 1e-4
W_SUM = 1e-5


def dev(a: np.ndarray) -> torch.Tensor:
    """Upload a uint16 (bf16 bits) numpy array as a bf16 CUDA tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def y_metrics(y: np.ndarray, ref: np.ndarray) -> dict:
    err = np.abs(y - ref)
    return {
        "max_err_rel": float(err.max() / max(np.abs(ref).max(), 1e-30)),
        "l1_rel": float(err.sum() / max(np.abs(ref).sum(), 1e-30)),
        "finite": bool(np.isfinite(y).all()),
    }


def assert_y_close(y: np.ndarray, ref: np.ndarray, what: str = "y", max_rel=Y_MAX_REL, l1=Y_L1_REL):
    m = y_metrics(y, ref)
    assert m["finite"], f"{what}: non-finite values"
    assert m["max_err_rel"] <= max_rel and m["l1_rel"] <= l1, f"{what}: {m}"
    return m


def assert_nan_rows(y: np.ndarray, ref: np.ndarray, what: str = "y"):
    """NaN exactly where the reference has NaN (some rows, all of them
    present), and the finite rows within the usual bound."""
    bad_y, bad_ref = np.isnan(y), np.isnan(ref)
    assert bad_ref.any(), f"{what}: the reference has no NaN"
    diff = np.argwhere(bad_y != bad_ref)
    assert diff.size == 0, f"{what}: NaN pattern differs at {diff[:5].tolist()}"
    rows = ~bad_ref.any(axis=1)
    assert rows.any(), f"{what}: no finite row left"
    assert_y_close(y[rows], ref[rows], what)


def assert_routing(ids_gpu: np.ndarray, w_gpu: np.ndarray, ids_ref: np.ndarray, w_ref: np.ndarray,
                   logits_ref: np.ndarray | None = None, k: int | None = None):
    bad = np.nonzero((ids_gpu != ids_ref).any(axis=1))[0]
    if bad.size:
        msg = f"{bad.size} tokens with different ids, first {bad[:5].tolist()}"
        if logits_ref is not None:
            import oracle.moe_oracle as orc
            near = set(orc.near_ties(logits_ref, k or ids_ref.shape[1]).tolist())
            msg += f"; near-tie tokens among them: {sorted(near & set(bad.tolist()))[:10]}"
        raise AssertionError(msg)
    assert np.abs(w_gpu - w_ref).max() <= W_ABS, np.abs(w_gpu - w_ref).max()
    assert np.abs(w_gpu.sum(axis=1) - 1.0).max() <= W_SUM
