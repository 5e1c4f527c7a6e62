"""HIP path against the float64 oracle on seeded inputs (needs an MI355X).

Every call goes through the C ABI (moe_layer_route_amd.binding is argument
marshalling only).  Shapes span several tiles and ragged tails: H and I take
values that are not multiples of 128 (or of 32), T takes odd values, and the
routing includes empty experts, skewed loads and k = 1 / k = E.
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


def _forward(inp_dev, k, path="auto", **kw):
    try:
        return binding.moe_forward(*inp_dev, k=k, path=path, **kw)
    except binding.MoEError as e:
        if "unsupported" in str(e):
            pytest.skip(f"path {path} not implemented")
        raise


def _small_inputs(T, E, H, I, k, seed=0, router_bias="normal"):
    cfg = d.small_config(T=T, E=E, H=H, I=I, k=k, x_scale=d.scale_for_hidden(H), router_bias=router_bias)
    return d.make_inputs(cfg, seed=seed, threads=4)


# ---------------------------------------------------------------------------
# router
# ---------------------------------------------------------------------------
ROUTE_METHODS = ["exact", "mfma"]


@pytest.mark.parametrize("method", ROUTE_METHODS)
@pytest.mark.parametrize("T,E,H,k", [
    (1, 4, 8, 1), (3, 8, 40, 2), (17, 32, 2880, 4), (65, 128, 2888, 4), (33, 256, 136, 8),
    (64, 32, 2880, 4), (5, 8, 72, 8), (200, 128, 2880, 4), (1000, 48, 2880, 4), (3, 40, 16384, 4),
    (8195, 40, 136, 4), (8256, 128, 2888, 4),   # 64-token tiles: token, expert and K tails
])
def test_route_parity(T, E, H, k, method):
    _need_gpu()
    inp = _small_inputs(T, E, H, 8, k)
    ids, w = binding.moe_route(dev(inp.x), dev(inp.Wr), dev(inp.br), k, method=method)
    torch.cuda.synchronize()
    ids_ref, w_ref, lg = orc.route(inp.x, inp.Wr, inp.br, k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, lg, k)


@pytest.mark.parametrize("method", ROUTE_METHODS)
def test_route_exact_ties_go_to_lower_index(method):
    _need_gpu()
    T, E, H, k = 9, 16, 64, 4
    rng = np.random.default_rng(1)
    x = d.f32_to_bf16_bits(rng.normal(0, 1, (T, H)).astype(np.float32))
    Wr = np.repeat(d.f32_to_bf16_bits(rng.normal(0, 0.1, (1, H)).astype(np.float32)), E, 0)
    br = np.zeros(E, np.uint16)
    ids, w = binding.moe_route(dev(x), dev(Wr), dev(br), k, method=method)
    assert (ids.cpu().numpy() == np.arange(k)).all()
    assert np.allclose(w.cpu().numpy(), 1.0 / k, atol=1e-7)
    # structured ties: one-hot router rows pick x's columns; columns 2 and 5 equal
    Wr = d.f32_to_bf16_bits(np.eye(E, H, dtype=np.float32))
    x = d.f32_to_bf16_bits(rng.normal(0, 1, (T, H)).astype(np.float32))
    x[:, 5] = x[:, 2]
    x[:, 0] = d.f32_to_bf16_bits(np.full(T, -0.0, np.float32))
    x[:, 1] = 0   # +0 ties -0 at index 0
    ids, _ = binding.moe_route(dev(x), dev(Wr), dev(br), 6, method=method)
    ids_ref, _, _ = orc.route(x, Wr, br, 6)
    assert (ids.cpu().numpy() == ids_ref).all()


@pytest.mark.parametrize("method", ROUTE_METHODS)
@pytest.mark.parametrize("E,k", [(8, 4), (32, 4), (128, 4), (256, 8)])
def test_route_near_ties_take_the_exact_decision(E, k, method):
    """Router rows that differ by a few ulps of one coordinate give logits
    closer than the float32 accumulation error: the kernel must fall back to
    the exact logits and decide as the oracle does (float32-rounded exact
    logits, lower index on equal values)."""
    _need_gpu()
    T, H = 97, 2880
    rng = np.random.default_rng(E)
    x = d.f32_to_bf16_bits((3.5 * rng.normal(0, 1, (T, H))).astype(np.float32))
    base = rng.normal(0, 0.02, H).astype(np.float32)
    W = np.repeat(base[None], E, 0)
    # a few groups of experts whose rows differ only in coordinate h0 by one
    # bf16 step; some are exact copies (exact ties)
    h0 = 7
    for e in range(E):
        W[e, h0] = base[h0] * (1.0 + (e % 3) * 2.0 ** -7)
    Wr = d.f32_to_bf16_bits(W)
    Wr[E // 2:] = d.f32_to_bf16_bits(rng.normal(0, 0.02, (E - E // 2, H)).astype(np.float32))
    br = np.zeros(E, np.uint16)
    ids, w = binding.moe_route(dev(x), dev(Wr), dev(br), k, method=method)
    ids_ref, w_ref, lg = orc.route(x, Wr, br, k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, lg, k)


@pytest.mark.parametrize("method", ROUTE_METHODS)
@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_route_configs(name, method):
    _need_gpu()
    cfg = d.CONFIGS[name]
    x = d.make_activations(cfg)
    Wr, br = d.make_router(cfg)
    ids, w = binding.moe_route(dev(x), dev(Wr), dev(br), cfg.k, method=method)
    ids_ref, w_ref, lg = orc.route(x, Wr, br, cfg.k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, lg, cfg.k)


@pytest.mark.parametrize("seed", [1, 2, 3, 7, 11])
@pytest.mark.parametrize("name", ["c3", "c4", "c5"])
def test_route_configs_other_seeds(name, seed):
    """The default router (exact at c4, the MFMA router with its exact
    near-tie recomputation at c3 and c5) on other draws of x, the router and
    its bias: every token's ids and weights against the oracle."""
    _need_gpu()
    cfg = d.CONFIGS[name]
    x = d.make_activations(cfg, seed=seed)
    Wr, br = d.make_router(cfg, seed=seed)
    ids, w = binding.moe_route(dev(x), dev(Wr), dev(br), cfg.k)
    ids_ref, w_ref, lg = orc.route(x, Wr, br, cfg.k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, lg, cfg.k)


# ---------------------------------------------------------------------------
# permutation
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("T,E,k,skew", [
    (1, 4, 1, "uniform"), (7, 8, 4, "uniform"), (64, 32, 4, "uniform"), (257, 128, 4, "uniform"),
    (4096, 32, 4, "uniform"), (16384, 128, 4, "zipf"), (1000, 256, 8, "uniform"), (300, 16, 2, "one"),
    (5000, 3, 1, "uniform"), (4097, 64, 4, "uniform"), (8193, 8, 2, "one"), (20480, 256, 8, "zipf"),
])
def test_permute_parity(T, E, k, skew):
    _need_gpu()
    rng = np.random.default_rng(T * 31 + E)
    if skew == "one":
        ids = np.zeros((T, k), np.int32)
        ids[:, 1:] = np.arange(1, k)
    elif skew == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        ids = np.stack([rng.choice(E, size=k, replace=False, p=p) for _ in range(T)]).astype(np.int32)
    else:
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    cnt, off, rows, pos = binding.moe_permute(torch.from_numpy(ids).cuda(), E)
    ref = orc.expert_permutation(ids, E)
    for got, want, name in zip((cnt, off, rows, pos), ref, ("cnt", "off", "rows", "pos")):
        assert (got.cpu().numpy() == want).all(), name


# ---------------------------------------------------------------------------
# whole forward, reduced shapes with ragged tails
# ---------------------------------------------------------------------------
SWEEP = [
    # T, E, H, I, k
    (1, 4, 8, 8, 1),
    (3, 8, 40, 24, 2),
    (17, 8, 72, 136, 4),
    (63, 16, 136, 72, 4),
    (65, 32, 2880, 40, 4),
    (33, 8, 2888, 2880, 4),
    (5, 4, 256, 264, 4),       # k = E
    (257, 8, 136, 128, 2),
    (40, 4, 128, 2888, 1),
    (3, 4, 16384, 40, 2),      # largest H: many K steps / chunk groups
    (3, 4, 40, 16384, 2),      # largest I: 2I = 32768 gate_up columns, K = 16384 for down
    (50, 256, 136, 72, 8),     # largest E and k
    (2000, 256, 136, 72, 8),   # largest E and k with a mean load above the tiled path's threshold
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,E,H,I,k", SWEEP)
def test_forward_sweep(T, E, H, I, k, path):
    _need_gpu()
    inp = _small_inputs(T, E, H, I, k, seed=T + E)
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    y = _forward([dev(a) for a in inp.arrays()], k, path, topk_ids=ids, topk_w=w)
    ref = orc.moe_forward(*inp.arrays(), k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y {T}x{E}x{H}x{I}x{k} {path}")


# ---------------------------------------------------------------------------
# expert parallelism: one rank's share per call, partials summed on the host
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("T,E,H,I,k,ranges", [
    (64, 32, 2880, 2880, 4, [(0, 16), (16, 32)]),
    (37, 16, 136, 72, 4, [(0, 4), (4, 8), (8, 12), (12, 16)]),
    (300, 8, 264, 128, 2, [(0, 1), (1, 5), (5, 8)]),            # uneven ranks
    (5, 6, 40, 24, 2, [(0, 5), (5, 6)]),
])
def test_expert_parallel_ranks_sum_to_y(T, E, H, I, k, ranges, path):
    _need_gpu()
    inp = _small_inputs(T, E, H, I, k, seed=T + 3 * E)
    x, Wr, br, Wgu, bgu, Wd, bd = [dev(a) for a in inp.arrays()]
    ref = orc.moe_forward(*inp.arrays(), k=k)
    total = np.zeros((T, H))
    for lo, hi in ranges:
        ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
        w = torch.empty((T, k), dtype=torch.float32, device="cuda")
        part = binding.moe_forward_ep(x, Wr, br, Wgu[lo:hi].contiguous(), bgu[lo:hi].contiguous(),
                                      Wd[lo:hi].contiguous(), bd[lo:hi].contiguous(), lo, k=k,
                                      topk_ids=ids, topk_w=w, path=path).double().cpu().numpy()
        assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
        want = orc.moe_forward(*inp.arrays(), k=k, experts=(lo, hi))["y"]
        assert_y_close(part, want, f"rank [{lo},{hi}) {path}")
        # tokens with no expert on this rank get exactly 0
        none_here = ~((ref["ids"] >= lo) & (ref["ids"] < hi)).any(axis=1)
        assert (part[none_here] == 0).all()
        total += part
    assert_y_close(total, ref["y"], f"sum of ranks {path}")


def test_expert_parallel_never_reads_other_ranks_experts():
    """A rank is handed only its own experts; NaN weights anywhere else in the
    full model cannot reach its partial output."""
    _need_gpu()
    T, E, H, I, k = 40, 8, 136, 72, 2
    inp = _small_inputs(T, E, H, I, k, seed=77)
    x, Wr, br, Wgu, bgu, Wd, bd = [dev(a) for a in inp.arrays()]
    lo, hi = 2, 5
    poisoned = [t.clone() for t in (Wgu, bgu, Wd, bd)]
    for t in poisoned:
        t.view(torch.int16)[:lo] = 0x7FC0
        t.view(torch.int16)[hi:] = 0x7FC0
    part = binding.moe_forward_ep(x, Wr, br, *[t[lo:hi].contiguous() for t in poisoned], lo, k=k)
    assert torch.isfinite(part).all()
    want = orc.moe_forward(*inp.arrays(), k=k, experts=(lo, hi))["y"]
    assert_y_close(part.double().cpu().numpy(), want, "rank [2,5)")


@pytest.mark.parametrize("path", PATHS)
def test_stage_intermediates(path):
    """gate_up and down alone against the oracle's h and o, matched through pos."""
    _need_gpu()
    T, E, H, I, k = 45, 8, 2880, 2880, 4
    inp = _small_inputs(T, E, H, I, k, seed=3)
    x, Wr, br, Wgu, bgu, Wd, bd = [dev(a) for a in inp.arrays()]
    ids, w = binding.moe_route(x, Wr, br, k)
    cnt, off, rows, pos = binding.moe_permute(ids, E)
    try:
        h = binding.moe_gate_up(x, Wgu, bgu, cnt, off, rows, k, path=path)
        o = binding.moe_down(h, Wd, bd, cnt, off, T, k, path=path)
    except binding.MoEError as e:
        if "unsupported" in str(e):
            pytest.skip(f"path {path} not implemented")
        raise
    y = binding.moe_combine(o, pos, w)
    ref = orc.moe_forward(*inp.arrays(), k=k, keep=True)
    p = pos.cpu().numpy()
    h_gpu = host_f64(h)[p]          # back to slot order s = t*k + j
    o_gpu = host_f64(o)[p]
    assert_y_close(h_gpu, ref["h"], "h", max_rel=1e-2, l1=5e-3)
    assert_y_close(o_gpu, ref["o"], "o", max_rel=1e-2, l1=5e-3)
    assert_y_close(host_f64(y), ref["y"], "y")


def test_identity_glu_table():
    """Wgu = 0, bgu = chosen (gate, up) pairs, Wd = identity: y = bf16(h(bgu))."""
    _need_gpu()
    pairs = [(1.0, 0.0), (-1.0, 0.0), (7.0, 7.0), (10.0, 9.0), (10.0, -9.0), (7.0, -7.0),
             (0.0, 3.0), (2.0, -1.0), (-7.0, 7.0), (2.5, 8.0), (-20.0, 3.0), (0.5, 0.5)]
    H = I = 136
    E, T, k = 4, 21, 2
    bg = np.zeros(2 * I, np.float32)
    for i, (g, u) in enumerate(pairs):
        bg[2 * i], bg[2 * i + 1] = g, u
    rng = np.random.default_rng(2)
    x = d.f32_to_bf16_bits(rng.normal(0, 1, (T, H)).astype(np.float32))
    Wr = d.f32_to_bf16_bits(rng.normal(0, 1, (E, H)).astype(np.float32))
    br = np.zeros(E, np.uint16)
    Wgu = np.zeros((E, H, 2 * I), np.uint16)
    bgu = np.repeat(d.f32_to_bf16_bits(bg)[None], E, 0)
    Wd = np.repeat(d.f32_to_bf16_bits(np.eye(I, H, dtype=np.float32))[None], E, 0)
    bd = np.zeros((E, H), np.uint16)
    arrays = (x, Wr, br, Wgu, bgu, Wd, bd)
    ref = orc.moe_forward(*arrays, k=k)["y"]
    for path in PATHS:
        try:
            y = host_f64(binding.moe_forward(*[dev(a) for a in arrays], k=k, path=path))
        except binding.MoEError as e:
            if "unsupported" in str(e):
                continue
            raise
        # h is rounded to bf16, the identity passes it through, the weights sum to 1
        assert np.allclose(y, ref, rtol=2 ** -7, atol=1e-30), (path, y[0, :12], ref[0, :12])
        assert (y[:, len(pairs):] == 0).all()


def test_skipped_experts_are_never_read():
    """NaN weights in an expert no token selects must not reach y."""
    _need_gpu()
    T, E, H, I, k = 31, 8, 136, 72, 2
    inp = _small_inputs(T, E, H, I, k, seed=5)
    br = inp.br.copy()
    br[E - 1] = d.f32_to_bf16_bits(np.array([-1e4], np.float32))[0]
    good = [dev(a) for a in (inp.x, inp.Wr, br, inp.Wgu, inp.bgu, inp.Wd, inp.bd)]
    Wgu, Wd, bgu, bd = inp.Wgu.copy(), inp.Wd.copy(), inp.bgu.copy(), inp.bd.copy()
    for a in (Wgu, Wd, bgu, bd):
        a[E - 1] = 0x7FC0
    bad = [dev(a) for a in (inp.x, inp.Wr, br, Wgu, bgu, Wd, bd)]
    for path in PATHS:
        try:
            y0 = bf16_bits(binding.moe_forward(*good, k=k, path=path))
            y1 = bf16_bits(binding.moe_forward(*bad, k=k, path=path))
        except binding.MoEError as e:
            if "unsupported" in str(e):
                continue
            raise
        assert (y0 == y1).all(), path


@pytest.mark.parametrize("path", PATHS)
def test_nan_in_live_expert_propagates(path):
    """A NaN gate bias in one selected expert and a NaN up bias in another:
    exactly the rows of their tokens are NaN (the GLU's clamps keep NaN)."""
    _need_gpu()
    T, E, H, I, k = 31, 8, 136, 72, 2
    inp = _small_inputs(T, E, H, I, k, seed=6)
    ids, _, _ = orc.route(inp.x, inp.Wr, inp.br, k)
    live = np.unique(ids)
    bgu = inp.bgu.copy()
    bgu[live[0], 0] = 0x7FC0     # gate of pair 0
    bgu[live[-1], 3] = 0x7FC0    # up of pair 1
    args = (inp.x, inp.Wr, inp.br, inp.Wgu, bgu, inp.Wd, inp.bd)
    y = host_f64(_forward([dev(a) for a in args], k, path=path))
    ref = orc.moe_forward(*args, k=k)["y"]
    assert_nan_rows(y, ref)


@pytest.mark.parametrize("path", PATHS)
def test_bitwise_repeat_and_poisoned_buffers(path):
    """Three runs give identical bytes, also with workspace and y pre-filled with 0xFF."""
    _need_gpu()
    T, E, H, I, k = 64, 32, 2880, 2880, 4
    inp = _small_inputs(T, E, H, I, k, seed=9)
    args = [dev(a) for a in inp.arrays()]
    ws = binding.alloc_workspace(T, H, E, k, I)
    outs = []
    for i in range(3):
        ws.fill_(0xFF if i else 0)
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        y.view(torch.int16).fill_(-1)
        outs.append(bf16_bits(_forward(args, k, path, y=y, workspace=ws)))
    assert (outs[0] == outs[1]).all() and (outs[1] == outs[2]).all()


def test_graph_capture_replay():
    """moe_forward captured in a HIP graph replays to the eager result, every replay."""
    _need_gpu()
    T, E, H, I, k = 64, 32, 2880, 2880, 4
    inp = _small_inputs(T, E, H, I, k, seed=11)
    args = [dev(a) for a in inp.arrays()]
    ws = binding.alloc_workspace(T, H, E, k, I)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    eager = bf16_bits(binding.moe_forward(*args, k=k, y=y, workspace=ws)).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        binding.moe_forward(*args, k=k, y=y, workspace=ws)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        binding.moe_forward(*args, k=k, y=y, workspace=ws)
    for i in range(4):
        y.view(torch.int16).fill_(-1)
        ws.fill_(0xAB)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (bf16_bits(y) == eager).all(), f"replay {i}"


# ---------------------------------------------------------------------------
# padded batches (device-side valid-row count) and expert loads
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("nv", [0, 1, 37, 64, 80])
def test_padded_forward(path, nv):
    """Rows from n_valid on are padding: id -1, weight 0, y exactly 0, no
    expert load; the valid rows and the loads match the oracle."""
    _need_gpu()
    T, E, H, I, k = 64, 16, 256, 160, 4
    inp = _small_inputs(T, E, H, I, k, seed=13)
    args = [dev(a) for a in inp.arrays()]
    n_valid = torch.tensor([nv], dtype=torch.int32, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")
    y = binding.moe_forward_padded(*args, k=k, n_valid=n_valid, topk_ids=ids, topk_w=w, expert_counts=counts,
                                   path=path)
    ref = orc.moe_forward_padded(*inp.arrays(), k=k, n_valid=nv)
    n = min(nv, T)
    yb, idh, wh = bf16_bits(y), ids.cpu().numpy(), w.cpu().numpy()
    assert (yb[n:] == 0).all() and (idh[n:] == -1).all() and (wh[n:] == 0).all()
    assert (counts.cpu().numpy() == ref["loads"]).all(), (counts.cpu().numpy(), ref["loads"])
    if n:
        assert_routing(idh[:n], wh[:n], ref["ids"][:n], ref["w"][:n], None, k)
        assert_y_close(host_f64(y)[:n], ref["y"][:n], f"y n_valid={nv}")


def test_padded_graph_replay():
    """One capture, replayed with a different n_valid each time: every replay
    equals the eager call for that n_valid (y, ids and loads, bit for bit)."""
    _need_gpu()
    T, E, H, I, k = 64, 32, 2880, 2880, 4
    inp = _small_inputs(T, E, H, I, k, seed=17)
    args = [dev(a) for a in inp.arrays()]
    ws = binding.alloc_workspace(T, H, E, k, I)
    n_valid = torch.tensor([T], dtype=torch.int32, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ids = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, k), dtype=torch.float32, device="cuda")
    counts = torch.empty((E,), dtype=torch.int32, device="cuda")

    def call():
        binding.moe_forward_padded(*args, k=k, n_valid=n_valid, y=y, workspace=ws, topk_ids=ids, topk_w=w,
                                   expert_counts=counts)

    eager = {}
    for nv in (64, 10, 0, 37):
        n_valid.fill_(nv)
        call()
        torch.cuda.synchronize()
        eager[nv] = (bf16_bits(y).copy(), ids.cpu().numpy().copy(), counts.cpu().numpy().copy())
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for nv in (37, 0, 64, 10, 37):
        y.view(torch.int16).fill_(-1)
        ws.fill_(0xAB)
        n_valid.fill_(nv)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yb, idh, ch = eager[nv]
        assert (bf16_bits(y) == yb).all() and (ids.cpu().numpy() == idh).all() and (counts.cpu().numpy() == ch).all(), nv


# ---------------------------------------------------------------------------
# the five workloads at full size
# ---------------------------------------------------------------------------
_weights_cache = {}


def _config_inputs(name, seed=0):
    """The workload's tensors; seed draws x and the router (the expert weights
    are always seed 0's, which keeps one set per E in memory)."""
    cfg = d.CONFIGS[name]
    if cfg.E not in _weights_cache:
        _weights_cache.clear()
        _weights_cache[cfg.E] = d.make_experts(cfg)
    x = d.make_activations(cfg, seed=seed)
    Wr, br = d.make_router(cfg, seed=seed)
    Wgu, bgu, Wd, bd = _weights_cache[cfg.E]
    return cfg, (x, Wr, br, Wgu, bgu, Wd, bd)


@pytest.mark.parametrize("name", ["c1", "c2", "c3", "c4", "c5"])
def test_forward_configs(name):
    """Full-size forward in the launch configuration the benchmark times; the
    oracle computes every token, so every row of every (expert, M tile) of
    the grouped-GEMM launches is compared, the last row of each expert
    segment included."""
    _need_gpu()
    cfg, arrays = _config_inputs(name)
    k = cfg.k
    args = [dev(a) for a in arrays]
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = binding.moe_forward(*args, k=k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] bf16 {name}: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y {name}")
    del args
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["c5", "c3"])
def test_forward_configs_other_seed(name):
    """The prefill workloads with x and the router drawn at another seed:
    other per-expert counts, so other tail tiles and another tile order in
    the grouped-GEMM launches; every token's y against the oracle."""
    _need_gpu()
    cfg, arrays = _config_inputs(name, seed=1)
    k = cfg.k
    args = [dev(a) for a in arrays]
    ids = torch.empty((cfg.T, k), dtype=torch.int32, device="cuda")
    w = torch.empty((cfg.T, k), dtype=torch.float32, device="cuda")
    y = binding.moe_forward(*args, k=k, topk_ids=ids, topk_w=w)
    torch.cuda.synchronize()
    print(f"[parity] bf16 {name} seed 1: GPU forward done, running the oracle over all {cfg.T} tokens", flush=True)
    ref = orc.moe_forward(*arrays, k=k)
    assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ref["ids"], ref["w"], ref["logits"], k)
    assert_y_close(host_f64(y), ref["y"], f"y {name} seed 1")
    del args
    torch.cuda.empty_cache()
