"""FP8 W8A8 experts on the HIP path against the float64 oracle (needs an
MI355X).  Every call goes through the C ABI.

Inputs: activations, router and biases from the seeded generators; the FP8
weight codes and per-expert scales are drawn directly by the generator, so no
quantiser sits between the oracle and its inputs.  The GPU quantisers (weights
per expert, activation rows) are checked separately, bit for bit, against the
oracle's.  The activations are quantised inside the forward on both sides
(per token for x, per (token, slot) row for h after rounding h to bf16).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding, datagen as d  # noqa: E402
import oracle.moe_oracle as orc  # noqa: E402
from checks import assert_nan_rows, assert_routing, assert_y_close, bf16_bits, dev, host_f64  # noqa: E402

pytestmark = pytest.mark.gpu

PATHS = ["gemv", "gemm"]


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _f8_inputs(cfg, seed=0):
    x = d.make_activations(cfg, seed)
    Wr, br = d.make_router(cfg, seed)
    gq, gs, bgu, dq, ds, bd = d.make_experts_fp8(cfg, seed, threads=8)
    return (x, Wr, br, gq, gs, bgu, dq, ds, bd)


def _small(T, E, H, I, k, seed=0, router_bias="normal"):
    cfg = d.small_config(T=T, E=E, H=H, I=I, k=k, x_scale=d.scale_for_hidden(H), router_bias=router_bias)
    return cfg, _f8_inputs(cfg, seed)


def _dev_any(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda() if a.dtype != np.uint16 else dev(a)


def _run(arrays, k, **kw):
    return binding.moe_forward_fp8(*[_dev_any(a) for a in arrays], k=k, **kw)


# ---------------------------------------------------------------------------
# quantisers: codes and scales bit for bit
# ---------------------------------------------------------------------------
def _special_values(a):
    """Values that exercise the E4M3 rounding: exact midpoints between codes
    (ties), values just off them, subnormal codes, the saturation bound, zeros
    of both signs, bf16 subnormals."""
    f = d.f32_to_bf16_bits
    a = a.copy().reshape(-1)
    mids = np.array([448.0, 0.5 * (1 + 1.125), 0.5 * (1.125 + 1.25), 0.5 * (240 + 256), 3 * 2.0 ** -10,
                     2.0 ** -10, 5 * 2.0 ** -10, 1.0625, -1.0625, -0.0, 0.0, 416.0, 432.0, 440.0], np.float32)
    special = np.concatenate([f(mids), np.arange(1, 9, dtype=np.uint16) * 3])   # + bf16 subnormals
    n = min(a.size, special.size)
    a[:n] = special[:n]
    return a


@pytest.mark.parametrize("E,K,N", [(2, 96, 40), (1, 2880, 576), (3, 16, 8), (2, 80, 200)])
def test_quantize_weights_matches_oracle(E, K, N):
    _need_gpu()
    W = d.normal_bf16((E, K, N), 0.02, 0, 79, K, N)
    W[0] = _special_values(W[0]).reshape(K, N)
    if E > 1:
        W[1] = 0                                                            # an all-zero expert: scale 1
    codes, scales = binding.moe_quantize_fp8(dev(W))
    c_ref, s_ref = orc.fp8_quantize_weights(W)
    s = scales.cpu().numpy()
    assert (s == s_ref).all(), (s, s_ref)
    c = codes.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}"


@pytest.mark.parametrize("R,K", [(5, 2880), (33, 64), (1, 16), (300, 48)])
def test_quantize_rows_matches_oracle(R, K):
    _need_gpu()
    a = d.normal_bf16((R, K), 1.0, 0, 83, R, K)
    a[0] = _special_values(a[0])
    if R > 2:
        a[1] = 0                                                            # an all-zero row: scale 1
        a[2] = d.f32_to_bf16_bits(np.full(K, 3.0e38, np.float32))          # huge values
    codes, scales = binding.moe_quantize_rows_fp8(dev(a))
    c_ref, s_ref = orc.fp8_quantize_rows(orc.widen(a))
    s = scales.cpu().numpy()
    assert (s == s_ref).all(), np.nonzero(s != s_ref)
    c = codes.cpu().numpy()
    bad = np.argwhere(c != c_ref)
    assert bad.size == 0, f"codes differ at {bad[:5].tolist()}: {c[tuple(bad[0])]:#x} vs {c_ref[tuple(bad[0])]:#x}"


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,H,I,k", [
    (1, 4, 64, 64, 1),        # one token, one K step
    (5, 8, 80, 48, 2),        # K tails (80 = 64 + 16, 48 < 64)
    (33, 8, 96, 64, 4),       # 2I = 128: a partial N tile; rows past 32 per expert
    (200, 16, 256, 160, 4),   # 2I = 320, H = 256
    (300, 4, 160, 608, 4),    # 300 rows per expert: three 128-row tiles
    (17, 32, 2880, 2880, 4),  # full hidden and intermediate sizes
    (9, 40, 2880, 224, 8),    # k = 8, E not a power of two, empty experts
    (257, 8, 2880, 2880, 2),  # ragged M tiles at full size
    (60, 256, 128, 96, 8),    # largest E and k
    (1700, 256, 128, 96, 8),  # largest E and k, mean load above the tiled path's threshold
])
@pytest.mark.parametrize("path", PATHS)
def test_forward_sweep(T, E, H, I, k, path):
    _need_gpu()
    cfg, arrays = _small(T, E, H, I, k, seed=T + E)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w, path=path)
    ref = orc.moe_forward_fp8(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y T{T} E{E} H{H} I{I} k{k}")


@pytest.mark.parametrize("path", PATHS)
def test_stage_intermediates(path):
    """The stage calls alone: x codes from the GPU row quantiser equal the
    oracle's; h and o against the oracle's, matched through pos."""
    _need_gpu()
    T, E, H, I, k = 45, 8, 2880, 2880, 4
    cfg, arrays = _small(T, E, H, I, k, seed=3)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = [_dev_any(a) for a in arrays]
    ids, w = binding.moe_route(x, Wr, br, k)
    cnt, off, rows, pos = binding.moe_permute(ids, E)
    xq, sx = binding.moe_quantize_rows_fp8(x)
    h = binding.moe_gate_up_fp8(xq, sx, gq, gs, bgu, cnt, off, rows, k, path=path)
    hq, sh = binding.moe_quantize_rows_fp8(h)
    o = binding.moe_down_fp8(hq, sh, dq, ds, bd, cnt, off, T, k, path=path)
    y = binding.moe_combine(o, pos, w)
    ref = orc.moe_forward_fp8(*arrays, k=k, keep=True)
    assert (xq.cpu().numpy() == ref["xq"]).all() and (sx.cpu().numpy() == ref["sx"]).all()
    p = pos.cpu().numpy()
    assert_y_close(host_f64(h)[p], ref["h"], "h", max_rel=1e-2, l1=5e-3)
    # h codes: equal wherever the two bf16 roundings of h and the row scales
    # agree (the FP8 products are summed inside the MFMA at below float32
    # precision, so a few percent of h values round to a neighbouring bf16)
    hb = orc.bf16_round(ref["h"])
    hg = host_f64(h)[p]
    same_row = sh.cpu().numpy()[p] == ref["sh"]
    same = (hg == hb) & same_row[:, None]
    assert same_row.mean() > 0.8 and same.mean() > 0.8, (same_row.mean(), same.mean())
    assert (hq.cpu().numpy()[p][same] == ref["hq"][same]).all()
    assert_y_close(host_f64(o)[p], ref["o"], "o", max_rel=1e-2, l1=5e-3)
    assert_y_close(host_f64(y), ref["y"], "y")


def test_skipped_experts_are_never_read():
    """NaN codes, scales and biases in an expert no token selects must not reach y."""
    _need_gpu()
    T, E, H, I, k = 31, 8, 128, 96, 2
    cfg, arrays = _small(T, E, H, I, k, seed=5)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = arrays
    br = br.copy()
    br[E - 1] = d.f32_to_bf16_bits(np.array([-1e4], np.float32))[0]
    good = [x, Wr, br, gq, gs, bgu, dq, ds, bd]
    bad = [a.copy() for a in good]
    bad[3][E - 1] = 0x7F           # NaN codes
    bad[6][E - 1] = 0x7F
    bad[4][E - 1] = np.nan         # NaN scales
    bad[7][E - 1] = np.nan
    bad[5][E - 1] = 0x7FC0         # NaN biases
    bad[8][E - 1] = 0x7FC0
    for path in PATHS:
        y0 = bf16_bits(_run(good, k, path=path))
        y1 = bf16_bits(_run(bad, k, path=path))
        assert (y0 == y1).all(), path


@pytest.mark.parametrize("path", PATHS)
def test_nan_in_live_expert_propagates(path):
    """A NaN weight code in a selected expert's gate_up and down weights, and
    a NaN up bias in another: exactly the rows (or elements) of their tokens
    are NaN."""
    _need_gpu()
    T, E, H, I, k = 40, 8, 96, 160, 2
    cfg, arrays = _small(T, E, H, I, k, seed=6)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = arrays
    ids, _, _ = orc.route(x, Wr, br, k)
    live = np.unique(ids)
    gq, dq, bgu = gq.copy(), dq.copy(), bgu.copy()
    gq[live[0], 2, 7] = 0x7F       # gate column 2 (pair 1), k = 7
    dq[live[1], 5, 3] = 0xFF       # output column 5, k = 3
    bgu[live[-1], 3] = 0x7FC0      # up of pair 1
    args = (x, Wr, br, gq, gs, bgu, dq, ds, bd)
    y = host_f64(_run(args, k, path=path))
    ref = orc.moe_forward_fp8(*args, k=k)["y"]
    assert_nan_rows(y, ref)


def test_bitwise_repeat_and_poisoned_workspace():
    _need_gpu()
    T, E, H, I, k = 64, 32, 2880, 2880, 4
    cfg, arrays = _small(T, E, H, I, k, seed=9)
    args = [_dev_any(a) for a in arrays]
    ws = binding.alloc_workspace_fp8(T, H, E, k, I)
    outs = []
    for i in range(3):
        ws.fill_(0xFF if i else 0)
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        y.view(torch.int16).fill_(-1)
        outs.append(bf16_bits(binding.moe_forward_fp8(*args, k=k, y=y, workspace=ws)))
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all()


@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c3", "c5"])
def test_forward_configs(name):
    """Every workload at full size with FP8 experts, in the launch
    configuration the benchmark times; the oracle computes every token, so
    every row of every (expert, M tile) of the grouped-GEMM launches is
    compared."""
    _need_gpu()
    cfg = d.CONFIGS[name]
    arrays = _f8_inputs(cfg)
    k = cfg.k
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] FP8 {name}: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward_fp8(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y {name}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("nv", [0, 1, 37, 64, 80])
def test_padded_forward(path, nv):
    """Rows from n_valid on are padding: id -1, weight 0, y exactly 0, no
    expert load; the valid rows and the loads match the oracle's FP8
    forward of those rows alone (x and h rows are quantised per row, so the
    padding cannot change a valid row's scales)."""
    _need_gpu()
    T, E, H, I, k = 64, 16, 256, 160, 4
    cfg, arrays = _small(T, E, H, I, k, seed=13)
    n_valid = torch.tensor([nv], dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    y = binding.moe_forward_padded_fp8(*[_dev_any(a) for a in arrays], k=k, n_valid=n_valid, topk_ids=ids,
                                       topk_w=w, expert_counts=counts, path=path)
    n = min(nv, T)
    yb, idh, wh = bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy()
    assert (yb[n:] == 0).all() and (idh[n:] == -1).all() and (wh[n:] == 0).all()
    if n == 0:
        assert (counts.cpu().numpy() == 0).all()
        return
    x, Wr, br = arrays[:3]
    ids_ref, w_ref, lg = orc.route(x[:n], Wr, br, k)
    assert (counts.cpu().numpy() == orc.expert_loads(ids_ref, E)).all()
    assert_routing(idh[:n], wh[:n], ids_ref, w_ref, lg, k)
    ref = orc.moe_forward_fp8(*arrays, k=k, tokens=np.arange(n))["y"]
    assert_y_close(host_f64(y)[:n], ref, f"y n_valid={nv}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,E,H,I,k,ranges", [
    (64, 32, 2880, 2880, 4, [(0, 16), (16, 32)]),
    (300, 8, 256, 160, 2, [(0, 1), (1, 5), (5, 8)]),     # uneven ranks
])
def test_expert_parallel_ranks_sum_to_y(T, E, H, I, k, ranges, path):
    """Each rank's partial equals the oracle's forward over its expert range
    (tokens with no local expert get exactly 0), and the partials sum to y."""
    _need_gpu()
    cfg, arrays = _small(T, E, H, I, k, seed=T + 3 * E)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = arrays
    ref = orc.moe_forward_fp8(*arrays, k=k)
    total = np.zeros((T, H))
    for lo, hi in ranges:
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        local = [_dev_any(np.ascontiguousarray(a[lo:hi])) for a in (gq, gs, bgu, dq, ds, bd)]
        part = binding.moe_forward_ep_fp8(_dev_any(x), _dev_any(Wr), _dev_any(br), *local, lo, k=k, topk_ids=ids, topk_w=w,
                                        path=path).double().cpu().numpy()
        assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
        want = orc.moe_forward_fp8(*arrays, k=k, experts=(lo, hi))["y"]
        assert_y_close(part, want, f"rank [{lo},{hi}) {path}")
        none_here = ~((ref["ids"] >= lo) & (ref["ids"] < hi)).any(axis=1)
        assert (part[none_here] == 0).all()
        total += part
    assert_y_close(total, ref["y"], f"sum of ranks {path}")


def test_forward_c5_other_seed():
    """The c5 prefill workload with every tensor drawn at another seed (other
    per-expert counts, tail tiles and tile order in the tiled FP8 GEMMs);
    every token's y against the oracle."""
    _need_gpu()
    cfg = d.CONFIGS["c5"]
    arrays = _f8_inputs(cfg, seed=1)
    k = cfg.k
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] FP8 c5 seed 1: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward_fp8(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], "y c5 seed 1")
