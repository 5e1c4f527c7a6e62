"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  A mutant that no pin rejects means the pins are too
weak to vouch for the oracle."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
import pins

_real = {n: getattr(orc, n) for n in ("clamped_glu", "router_logits", "select_topk",
                                      "routing_weights", "expert_mlp", "expert_permutation",
                                      "moe_forward", "widen")}


def _glu(gate_sel=0, up_sel=1, alpha=1.702, glim=(-np.inf, 7.0), ulim=(-7.0, 7.0), plus=1.0,
         clamp_after_plus=False, sig_uses_raw=False):
    def f(u):
        graw = u[..., gate_sel::2]
        gate = np.clip(graw, glim[0], glim[1])
        up = u[..., up_sel::2]
        if clamp_after_plus:
            up = np.clip(up + plus, *ulim)
        else:
            up = np.clip(up, *ulim) + plus
        z = graw if sig_uses_raw else gate
        return up * gate / (1.0 + np.exp(-alpha * z))
    return f


def _topk_high_index_on_tie(logits, k):
    T, E = logits.shape
    idx = np.arange(E)
    return np.stack([np.lexsort((-idx, -logits[t].astype(np.float64)))[:k] for t in range(T)]).astype(np.int32)


def _topk_ascending(logits, k):
    return _real["select_topk"](logits, k)[:, ::-1].copy()


def _weights_full_softmax(lg, ids):
    ex = np.exp(lg - lg.max(axis=1, keepdims=True))
    p = ex / ex.sum(axis=1, keepdims=True)
    return np.take_along_axis(p, ids.astype(np.int64), 1)


def _weights_uniform(lg, ids):
    return np.full(ids.shape, 1.0 / ids.shape[1])


def _weights_neg(lg, ids):
    return _real["routing_weights"](-lg, ids)


def _router_nobias(x, Wr, br):
    return orc.widen(x) @ orc.widen(Wr).T


def _router_minusbias(x, Wr, br):
    return orc.widen(x) @ orc.widen(Wr).T - orc.widen(br)[None, :]


def _mlp(no_bgu=False, no_bd=False, transpose_down=False):
    def f(xr, Wgu_e, bgu_e, Wd_e, bd_e):
        u = xr @ Wgu_e + (0.0 if no_bgu else bgu_e)
        h = orc.clamped_glu(u)
        o = (h @ (Wd_e.T if transpose_down else Wd_e)) + (0.0 if no_bd else bd_e)
        return u, h, o
    return f


def _perm_unstable(ids, E):
    cnt, off, rows, pos = _real["expert_permutation"](ids, E)
    rows = rows.copy()
    for e in range(E):
        rows[off[e]:off[e + 1]] = rows[off[e]:off[e + 1]][::-1]
    pos = np.empty_like(pos)
    pos[rows] = np.arange(rows.size)
    return cnt, off, rows, pos


def _perm_inclusive(ids, E):
    cnt, off, rows, pos = _real["expert_permutation"](ids, E)
    off = off.copy()
    off[:-1] = off[1:]
    return cnt, off, rows, pos


def _forward_multiply_by_zero(x, Wr, br, Wgu, bgu, Wd, bd, k, tokens=None, keep=False, experts=None):
    """Runs every expert on every token and multiplies the unselected ones by 0."""
    ids, w, lg = orc.route(x, Wr, br, k)
    xs = orc.widen(x)
    T = xs.shape[0]
    E = Wr.shape[0]
    y = np.zeros((T, Wd.shape[2]))
    for e in range(E):
        _, _, o = orc.expert_mlp(xs, orc.widen(Wgu[e]), orc.widen(bgu[e]), orc.widen(Wd[e]), orc.widen(bd[e]))
        we = np.where(ids == e, w, 0.0).sum(axis=1)
        y += we[:, None] * o
    return {"y": y, "ids": ids, "w": w, "logits": lg}


def _forward_bias_outside(x, Wr, br, Wgu, bgu, Wd, bd, k, tokens=None, keep=False, experts=None):
    """Adds the down bias once per selected expert, outside the weighted sum."""
    out = _real["moe_forward"](x, Wr, br, Wgu, bgu, Wd, bd, k, tokens, keep, experts)
    bdw = orc.widen(bd)
    for t in range(out["y"].shape[0]):
        for j in range(k):
            e = out["ids"][t, j]
            out["y"][t] += (1.0 - out["w"][t, j]) * bdw[e]
    return out


def _forward_no_weights(x, Wr, br, Wgu, bgu, Wd, bd, k, tokens=None, keep=False, experts=None):
    ids, w, lg = orc.route(x, Wr, br, k)
    out = _real["moe_forward"](x, Wr, br, Wgu, bgu, Wd, bd, k, tokens, keep, experts)
    # re-sum the expert outputs without the routing weights
    xs = orc.widen(x)
    y = np.zeros_like(out["y"])
    for t in range(xs.shape[0]):
        for j in range(k):
            e = ids[t, j]
            y[t] += orc.expert_mlp(xs[t:t + 1], orc.widen(Wgu[e]), orc.widen(bgu[e]), orc.widen(Wd[e]), orc.widen(bd[e]))[2][0]
    out["y"] = y
    return out


def _forward_range_inclusive(x, Wr, br, Wgu, bgu, Wd, bd, k, tokens=None, keep=False, experts=None):
    """An expert range that also takes its end expert."""
    if experts is not None:
        experts = (experts[0], min(experts[1] + 1, Wr.shape[0]))
    return _real["moe_forward"](x, Wr, br, Wgu, bgu, Wd, bd, k, tokens, keep, experts)


def _forward_range_ignored(x, Wr, br, Wgu, bgu, Wd, bd, k, tokens=None, keep=False, experts=None):
    """Every rank returns the whole y."""
    return _real["moe_forward"](x, Wr, br, Wgu, bgu, Wd, bd, k, tokens, keep)


def _widen_truncating(bits):
    # reads bf16 as if it were the top half of a float32 but drops the lowest mantissa bit
    b = np.asarray(bits, dtype=np.uint16) & np.uint16(0xFFFE)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


MUTANTS = {
    "glu_swap_gate_up": ("clamped_glu", _glu(gate_sel=1, up_sel=0)),
    "glu_alpha_1": ("clamped_glu", _glu(alpha=1.0)),
    "glu_alpha_1.8": ("clamped_glu", _glu(alpha=1.8)),
    "glu_no_gate_clamp": ("clamped_glu", _glu(glim=(-np.inf, np.inf))),
    "glu_two_sided_gate_clamp": ("clamped_glu", _glu(glim=(-7.0, 7.0))),
    "glu_no_up_clamp": ("clamped_glu", _glu(ulim=(-np.inf, np.inf))),
    "glu_up_clamp_one_sided": ("clamped_glu", _glu(ulim=(-np.inf, 7.0))),
    "glu_no_plus_one": ("clamped_glu", _glu(plus=0.0)),
    "glu_clamp_after_plus_one": ("clamped_glu", _glu(clamp_after_plus=True)),
    "glu_sigmoid_of_unclamped_gate": ("clamped_glu", _glu(sig_uses_raw=True)),
    "router_no_bias": ("router_logits", _router_nobias),
    "router_minus_bias": ("router_logits", _router_minusbias),
    "topk_tie_high_index": ("select_topk", _topk_high_index_on_tie),
    "topk_ascending_order": ("select_topk", _topk_ascending),
    "weights_softmax_over_all_E": ("routing_weights", _weights_full_softmax),
    "weights_uniform": ("routing_weights", _weights_uniform),
    "weights_of_negated_logits": ("routing_weights", _weights_neg),
    "mlp_no_gate_up_bias": ("expert_mlp", _mlp(no_bgu=True)),
    "mlp_no_down_bias": ("expert_mlp", _mlp(no_bd=True)),
    "mlp_down_transposed": ("expert_mlp", _mlp(transpose_down=True)),
    "perm_unstable": ("expert_permutation", _perm_unstable),
    "perm_inclusive_scan": ("expert_permutation", _perm_inclusive),
    "forward_multiply_by_zero": ("moe_forward", _forward_multiply_by_zero),
    "forward_down_bias_outside_sum": ("moe_forward", _forward_bias_outside),
    "forward_no_routing_weights": ("moe_forward", _forward_no_weights),
    "forward_expert_range_inclusive": ("moe_forward", _forward_range_inclusive),
    "forward_expert_range_ignored": ("moe_forward", _forward_range_ignored),
    "widen_drops_a_bit": ("widen", _widen_truncating),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(orc, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(orc)
        except AssertionError:
            caught.append(pin.__name__)
        except (ValueError, IndexError, FloatingPointError):
            caught.append(pin.__name__ + "(error)")
    assert caught, f"mutant {name} passed every pin"
