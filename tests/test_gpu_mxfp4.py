"""MXFP4 expert weights (W4A16) on the HIP path against the float64 oracle
(needs an MI355X).  Every call goes through the C ABI.

Inputs: activations, router and biases from the seeded generators; the MXFP4
codes and scales are drawn directly by the generator (the distributions that
N(0, 0.02) weights take in the format), so no quantiser sits between the
oracle and its inputs.  The GPU quantiser is checked separately, bit for bit,
against the oracle's.
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding, datagen as d  # noqa: E402
import oracle.moe_oracle as orc  # noqa: E402
from checks import assert_nan_rows, assert_routing, assert_y_close, bf16_bits, dev, host_f64  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _mx_inputs(cfg, seed=0):
    x = d.make_activations(cfg, seed)
    Wr, br = d.make_router(cfg, seed)
    gq, gs, bgu, dq, ds, bd = d.make_experts_mxfp4(cfg, seed, threads=8)
    return (x, Wr, br, gq, gs, bgu, dq, ds, bd)


def _small(T, E, H, I, k, seed=0, router_bias="normal"):
    cfg = d.small_config(T=T, E=E, H=H, I=I, k=k, x_scale=d.scale_for_hidden(H), router_bias=router_bias)
    return cfg, _mx_inputs(cfg, seed)


PATHS = ["gemv", "gemm"]


def _run(arrays, k, **kw):
    return binding.moe_forward_mxfp4(*[dev(a) for a in arrays], k=k, **kw)


# ---------------------------------------------------------------------------
# quantiser: codes and scales bit for bit
# ---------------------------------------------------------------------------
def _special_blocks(W):
    """Blocks that exercise the rounding rule: zeros, exact midpoints (ties),
    negative zeros, subnormal maxima, huge values, a power-of-two maximum."""
    f = d.f32_to_bf16_bits
    E, K, N = W.shape
    W = W.copy()
    W[0, 0:32, 0] = 0
    mids = np.array([7.5, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, 0.3, -0.25, -0.75, -2.5, -5.0, 6.0, 4.4],
                    np.float32) * np.float32(2.0 ** -3)
    W[0, 0:16, 1] = f(mids)
    W[0, 16:32, 1] = f(-mids)
    W[0, 0:32, 2] = 0x8000                               # -0
    W[0, 5, 2] = f(np.array([-1e-3], np.float32))[0]
    W[0, 0:32, 3] = np.arange(1, 33, dtype=np.uint16) * 3  # subnormal bf16 (max 0x0060)
    W[0, 0:32, 4] = f(np.linspace(-3e38, 3e38, 32, dtype=np.float32))
    W[0, 0:32, 5] = f(np.array([4.0] + [0.125 * i for i in range(31)], np.float32))
    return W


@pytest.mark.parametrize("E,K,N", [(2, 96, 40), (1, 2880, 576), (3, 32, 8)])
def test_quantize_matches_oracle(E, K, N):
    _need_gpu()
    W = _special_blocks(d.normal_bf16((E, K, N), 0.02, 0, 77, K, N))
    codes, scales = binding.moe_quantize_mxfp4(dev(W))
    c_ref, s_ref = orc.mxfp4_quantize(np.transpose(orc.widen(W), (0, 2, 1)))
    c, s = codes.cpu().numpy(), scales.cpu().numpy()
    bad_s = np.argwhere(s != s_ref)
    assert bad_s.size == 0, f"scales differ at {bad_s[:5].tolist()}: {s[tuple(bad_s[0])]} vs {s_ref[tuple(bad_s[0])]}"
    bad_c = np.argwhere(c != c_ref)
    assert bad_c.size == 0, f"codes differ at {bad_c[:5].tolist()}"


# ---------------------------------------------------------------------------
# forward
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,H,I,k", [
    (1, 4, 32, 32, 1),        # one token, one block per row
    (5, 8, 64, 96, 2),        # K = 96: three blocks, a partial quad of blocks
    (33, 8, 96, 64, 4),       # 2I = 128: one column slice; rows past 16 per expert
    (70, 4, 160, 32, 2),      # 35 rows per expert: two passes over the weights
    (200, 16, 256, 160, 4),   # 2I = 320 and H = 256: partial column slices; two 16-row chunks a pass
    (17, 32, 2880, 2880, 4),  # full hidden and intermediate sizes
    (9, 40, 2880, 224, 8),    # k = 8, E not a power of two, empty experts
    (300, 4, 160, 608, 4),    # 300 rows per expert: three 128-row tiles; K = 160 is 1.25 quads
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
    ref = orc.moe_forward_mxfp4(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y T{T} E{E} H{H} I{I} k{k}")


@pytest.mark.parametrize("T,E,H,I,k,bias,min_max_rows", [
    (40, 16, 2880, 2880, 4, "zipf", 17),   # skewed decode batch: an expert with more than one 16-row chunk
    (3, 2, 96, 32, 2, "normal", 1),        # two experts; down N = 96: one and a half 64-column slices
    (12, 8, 2880, 64, 4, "zipf", 1),       # gate_up N = 128: two slices; down K = 64
    (24, 64, 2848, 2880, 4, "normal", 1),  # K = 2848: the last 256-value step holds one block of eight
])
def test_decode_batch_shapes(T, E, H, I, k, bias, min_max_rows):
    """Decode batches (T*k <= 10 E, the weight-streaming kernel's one-chunk regime) against the oracle, ids
    and y: an expert with more than 16 rows, very few experts, a single column quad, K cut inside a line."""
    _need_gpu()
    assert T * k <= 10 * E
    cfg, arrays = _small(T, E, H, I, k, seed=T + 7 * E, router_bias=bias)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w, path="gemv")
    ref = orc.moe_forward_mxfp4(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert np.bincount(ref["ids"].ravel(), minlength=E).max() >= min_max_rows
    assert_y_close(host_f64(y), ref["y"], f"y T{T} E{E} H{H} I{I} k{k}")


@pytest.mark.parametrize("path", PATHS)
def test_stage_intermediates(path):
    """gate_up and down alone against the oracle's h and o, matched through pos."""
    _need_gpu()
    T, E, H, I, k = 45, 8, 2880, 2880, 4
    cfg, arrays = _small(T, E, H, I, k, seed=3)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = [dev(a) for a in arrays]
    ids, w = binding.moe_route(x, Wr, br, k)
    cnt, off, rows, pos = binding.moe_permute(ids, E)
    h = binding.moe_gate_up_mxfp4(x, gq, gs, bgu, cnt, off, rows, k, path=path)
    o = binding.moe_down_mxfp4(h, dq, ds, bd, cnt, off, T, k, path=path)
    y = binding.moe_combine(o, pos, w)
    ref = orc.moe_forward_mxfp4(*arrays, k=k, keep=True)
    p = pos.cpu().numpy()
    assert_y_close(host_f64(h)[p], ref["h"], "h", max_rel=1e-2, l1=5e-3)
    assert_y_close(host_f64(o)[p], ref["o"], "o", max_rel=1e-2, l1=5e-3)
    assert_y_close(host_f64(y), ref["y"], "y")


def test_skipped_experts_are_never_read():
    """NaN scales, codes and biases in an expert no token selects must not reach y."""
    _need_gpu()
    T, E, H, I, k = 31, 8, 128, 96, 2
    cfg, arrays = _small(T, E, H, I, k, seed=5)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = arrays
    br = br.copy()
    br[E - 1] = d.f32_to_bf16_bits(np.array([-1e4], np.float32))[0]
    good = [x, Wr, br, gq, gs, bgu, dq, ds, bd]
    bad = [a.copy() for a in good]
    bad[4][E - 1] = 255          # NaN scales
    bad[7][E - 1] = 255
    bad[5][E - 1] = 0x7FC0       # NaN biases
    bad[8][E - 1] = 0x7FC0
    for path in PATHS:
        y0 = bf16_bits(_run(good, k, path=path))
        y1 = bf16_bits(_run(bad, k, path=path))
        assert (y0 == y1).all(), path


@pytest.mark.parametrize("path", PATHS)
def test_nan_scale_in_live_expert_propagates(path):
    """A NaN scale (byte 255) in a selected expert's gate_up and down
    weights, and a NaN up bias in another: exactly the rows of their tokens
    are NaN."""
    _need_gpu()
    T, E, H, I, k = 40, 8, 96, 160, 2
    cfg, arrays = _small(T, E, H, I, k, seed=6)
    x, Wr, br, gq, gs, bgu, dq, ds, bd = arrays
    ids, _, _ = orc.route(x, Wr, br, k)
    live = np.unique(ids)
    gs, ds, bgu = gs.copy(), ds.copy(), bgu.copy()
    gs[live[0], 1, 2] = 255      # block 1 of gate column 2
    ds[live[1], 2, 5] = 255      # block 2 of output column 5
    bgu[live[-1], 3] = 0x7FC0    # up of pair 1
    args = (x, Wr, br, gq, gs, bgu, dq, ds, bd)
    y = host_f64(_run(args, k, path=path))
    ref = orc.moe_forward_mxfp4(*args, k=k)["y"]
    assert_nan_rows(y, ref)


def test_bitwise_repeat_and_poisoned_workspace():
    _need_gpu()
    T, E, H, I, k = 64, 32, 2880, 2880, 4
    cfg, arrays = _small(T, E, H, I, k, seed=9)
    args = [dev(a) for a in arrays]
    ws = binding.alloc_workspace(T, H, E, k, I)
    outs = []
    for i in range(3):
        ws.fill_(0xFF if i else 0)
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        y.view(torch.int16).fill_(-1)
        outs.append(bf16_bits(binding.moe_forward_mxfp4(*args, k=k, y=y, workspace=ws)))
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all()


@pytest.mark.parametrize("name", ["c1", "c2", "c4", "c3", "c5"])
def test_forward_configs(name):
    """Every workload at full size with MXFP4 experts, in the launch
    configuration the benchmark times; the oracle computes every token, so
    every row of every (expert, M tile) of the grouped-GEMM launches is
    compared."""
    _need_gpu()
    cfg = d.CONFIGS[name]
    arrays = _mx_inputs(cfg)
    k = cfg.k
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] MXFP4 {name}: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward_mxfp4(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y {name}")


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("nv", [0, 1, 37, 64, 80])
def test_padded_forward(path, nv):
    """Rows from n_valid on are padding: id -1, weight 0, y exactly 0, no
    expert load; the valid rows and the loads match the oracle's MXFP4
    forward of those rows alone."""
    _need_gpu()
    T, E, H, I, k = 64, 16, 256, 160, 4
    cfg, arrays = _small(T, E, H, I, k, seed=13)
    n_valid = torch.tensor([nv], dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    y = binding.moe_forward_padded_mxfp4(*[dev(a) for a in arrays], k=k, n_valid=n_valid, topk_ids=ids, topk_w=w,
                                         expert_counts=counts, path=path)
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
    ref = orc.moe_forward_mxfp4(*arrays, k=k, tokens=np.arange(n))["y"]
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
    ref = orc.moe_forward_mxfp4(*arrays, k=k)
    total = np.zeros((T, H))
    for lo, hi in ranges:
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        local = [dev(np.ascontiguousarray(a[lo:hi])) for a in (gq, gs, bgu, dq, ds, bd)]
        part = binding.moe_forward_ep_mxfp4(dev(x), dev(Wr), dev(br), *local, lo, k=k, topk_ids=ids, topk_w=w,
                                        path=path).double().cpu().numpy()
        assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
        want = orc.moe_forward_mxfp4(*arrays, k=k, experts=(lo, hi))["y"]
        assert_y_close(part, want, f"rank [{lo},{hi}) {path}")
        none_here = ~((ref["ids"] >= lo) & (ref["ids"] < hi)).any(axis=1)
        assert (part[none_here] == 0).all()
        total += part
    assert_y_close(total, ref["y"], f"sum of ranks {path}")


def test_forward_c5_other_seed():
    """The c5 prefill workload with every tensor drawn at another seed (other
    per-expert counts, tail tiles and tile order in the tiled MXFP4 GEMMs);
    every token's y against the oracle."""
    _need_gpu()
    cfg = d.CONFIGS["c5"]
    arrays = _mx_inputs(cfg, seed=1)
    k = cfg.k
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = _run(arrays, k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] MXFP4 c5 seed 1: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward_mxfp4(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], "y c5 seed 1")
