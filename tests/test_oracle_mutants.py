"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one of them.  A mutant that no pin rejects means the pins are too
weak to vouch for the oracle."""
import numpy as np
import pytest

import oracle.moe_oracle as orc
import pins

_real = {n: getattr(orc, n) for n in ("clamped_glu", "router_logits", "select_topk",
                                      "routing_weights", "expert_mlp", "expert_permutation",
                                      "moe_forward", "widen", "mxfp4_quantize", "mxfp4_dequantize",
                                      "moe_forward_mxfp4", "ue8m0_decode", "e2m1_decode", "e4m3_encode",
                                      "fp8_scale", "fp8_quantize_rows", "fp8_quantize_weights", "bf16_round",
                                      "moe_forward_fp8", "fp8_down", "expert_loads", "moe_forward_padded",
                                      "near_ties")}


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


def _e2m1_table_typo():
    t = np.array(orc.E2M1_VALUES, copy=True)
    t[5], t[13] = 2.5, -2.5
    return t


def _e2m1_decode_bias0(code):
    return 2.0 * _real["e2m1_decode"](code)


def _ue8m0_bias128(e):
    return _real["ue8m0_decode"](np.asarray(e) - 1)


def _dequant_nibbles_swapped(codes, scales):
    c = np.asarray(codes, np.uint8)
    return _real["mxfp4_dequantize"](((c & 15) << 4) | (c >> 4), scales)


def _dequant_scales_tiled(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],))
    q[..., 0::2] = orc.E2M1_VALUES[codes & 15]
    q[..., 1::2] = orc.E2M1_VALUES[codes >> 4]
    return q * np.tile(np.swapaxes(orc.ue8m0_decode(scales), -1, -2), 32)


def _quant_variant(ties="even", emax=2, ceil_exp=False):
    def f(w):
        w = np.asarray(w, dtype=np.float64)
        K = w.shape[-1]
        blk = w.reshape(w.shape[:-1] + (K // 32, 32))
        amax = np.abs(blk).max(axis=-1)
        _, p = np.frexp(amax)
        e = p if ceil_exp else p - 1
        shared = np.clip(np.where(amax > 0, e - emax, -127), -127, 127)
        X = np.ldexp(1.0, shared)[..., None]
        v = np.abs(blk) / X
        mags = orc.E2M1_VALUES[:8]
        dist = np.abs(v[..., None] - mags)
        best = dist.min(axis=-1, keepdims=True)
        cand = dist == best
        if ties == "even":
            pick = cand & (np.arange(8) % 2 == 0)
            code = np.where(pick.any(-1), pick.argmax(-1), cand.argmax(-1))
        else:                                     # ties to the larger magnitude
            code = 7 - cand[..., ::-1].argmax(-1)
        code = ((np.signbit(blk).astype(np.int64) << 3) | code).reshape(w.shape)
        return ((code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8),
                np.swapaxes((shared + 127).astype(np.uint8), -1, -2).copy())
    return f


def _forward_mxfp4_untransposed(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k, tokens=None, keep=False,
                                experts=None):
    def weights(e):
        return (orc.mxfp4_dequantize(Wgu_q[e], Wgu_s[e]).reshape(Wgu_q.shape[2] * 2, -1), orc.widen(bgu[e]),
                orc.mxfp4_dequantize(Wd_q[e], Wd_s[e]).reshape(Wd_q.shape[2] * 2, -1), orc.widen(bd[e]))
    return orc._forward(x, Wr, br, weights, Wgu_q.shape[1], Wd_q.shape[1], k, tokens, keep, experts)


def _e4m3_table_bias8():
    t = np.array(orc.E4M3_VALUES, copy=True)
    return t / 2.0


def _encode_variant(ties="even", saturate=True):
    def f(v):
        shape = np.shape(v)
        v = np.asarray(v, dtype=np.float32).astype(np.float64).reshape(-1)
        fin = orc.E4M3_VALUES[:0x7F]
        a = np.where(np.isnan(v), 0.0, np.abs(v))
        if saturate:
            a = np.minimum(a, 448.0)
        d = np.abs(a[:, None] - fin[None, :])
        best = d.min(axis=1, keepdims=True)
        cand = d == best
        if ties == "even":
            pick = cand & (np.arange(0x7F) % 2 == 0)
            code = np.where(pick.any(1), pick.argmax(1), cand.argmax(1))
        else:                                     # ties away from zero
            code = 0x7E - cand[:, ::-1].argmax(1)
        code = np.where(a > 464.0, 0x7F, code)    # (no saturation: overflow is NaN)
        code = code | (np.signbit(v).astype(np.int64) << 7)
        return np.where(np.isnan(v), 0x7F, code).astype(np.uint8).reshape(shape)
    return f


def _fp8_scale_inverted(amax):
    s, inv = _real["fp8_scale"](amax)
    return inv, s


def _fp8_rows_per_tensor(a):
    a = np.asarray(a, dtype=np.float32)
    s, inv = orc.fp8_scale(np.abs(a).max())
    return orc.e4m3_encode(a * inv), np.full(a.shape[:-1], s, np.float32)


def _fp8_weights_untransposed(W):
    codes, s = _real["fp8_quantize_weights"](W)
    return np.ascontiguousarray(np.swapaxes(codes, 1, 2)).reshape(codes.shape), s


def _fp8_weights_one_scale(W):
    w = orc.widen(W).astype(np.float32)
    s, inv = orc.fp8_scale(np.abs(w).max())
    codes = orc.e4m3_encode(w * inv)
    return np.ascontiguousarray(np.swapaxes(codes, 1, 2)), np.full(w.shape[0], s, np.float32)


def _bf16_round_truncating(x):
    x = np.asarray(x, dtype=np.float64)
    _, p = np.frexp(np.where(x != 0, x, 1.0))
    q = np.ldexp(1.0, np.maximum(p - 8, -133))
    return np.trunc(x / q) * q


def _forward_fp8_variant(round_h=True, weight_scale=True):
    def f(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k, tokens=None, keep=False, experts=None):
        gs = Wgu_s if weight_scale else np.ones_like(Wgu_s)
        saved = orc.bf16_round
        if not round_h:
            orc.bf16_round = lambda v: np.asarray(v, dtype=np.float64)
        try:
            return _real["moe_forward_fp8"](x, Wr, br, Wgu_q, gs, bgu, Wd_q, Wd_s, bd, k, tokens, keep, experts)
        finally:
            orc.bf16_round = saved
    return f


def _fp8_down_no_weight_scale(hb, Wd_q_e, s_d_e, bd_e64):
    return _real["fp8_down"](hb, Wd_q_e, np.float32(1.0), bd_e64)


def _loads_first_pick_only(ids, E):
    first = ids[:, 0]
    return np.bincount(first[first >= 0], minlength=E)


def _padded_variant(route_padding=False, off_by_one=False):
    def f(x, Wr, br, Wgu, bgu, Wd, bd, k, n_valid):
        T = x.shape[0]
        nv = min(max(int(n_valid), 0), T)
        if route_padding:
            nv = T
        if off_by_one:
            nv = max(nv - 1, 0)
        return _real["moe_forward_padded"](x, Wr, br, Wgu, bgu, Wd, bd, k, nv)
    return f



def _near_ties(last_boundary=True, floor=True, signed=False, ascending=False):
    def f(logits64, k, rel=1e-5):
        s = np.sort(logits64, axis=1) if ascending else -np.sort(-logits64, axis=1)
        kk = min(k + 1 if last_boundary else k, s.shape[1])
        gaps = np.abs(s[:, :kk - 1] - s[:, 1:kk])
        top = s[:, :kk - 1] if signed else np.abs(s[:, :kk - 1])
        scale = np.maximum(1.0, top) if floor else top
        return np.nonzero((gaps < rel * scale).any(axis=1))[0]
    return f


MUTANTS = {
    "loads_first_pick_only": ("expert_loads", _loads_first_pick_only),
    "padded_rows_routed": ("moe_forward_padded", _padded_variant(route_padding=True)),
    "padded_n_valid_off_by_one": ("moe_forward_padded", _padded_variant(off_by_one=True)),
    "e4m3_exponent_bias_8": ("E4M3_VALUES", _e4m3_table_bias8()),
    "e4m3_encode_ties_away": ("e4m3_encode", _encode_variant(ties="away")),
    "e4m3_encode_overflow_nan": ("e4m3_encode", _encode_variant(saturate=False)),
    "fp8_scale_inverted": ("fp8_scale", _fp8_scale_inverted),
    "fp8_rows_one_scale_per_tensor": ("fp8_quantize_rows", _fp8_rows_per_tensor),
    "fp8_weights_untransposed": ("fp8_quantize_weights", _fp8_weights_untransposed),
    "fp8_weights_one_scale_for_all_experts": ("fp8_quantize_weights", _fp8_weights_one_scale),
    "bf16_round_truncating": ("bf16_round", _bf16_round_truncating),
    "fp8_forward_h_not_rounded_to_bf16": ("moe_forward_fp8", _forward_fp8_variant(round_h=False)),
    "fp8_forward_gate_up_scale_dropped": ("moe_forward_fp8", _forward_fp8_variant(weight_scale=False)),
    "fp8_down_scale_dropped": ("fp8_down", _fp8_down_no_weight_scale),

    "e2m1_table_typo": ("E2M1_VALUES", _e2m1_table_typo()),
    "e2m1_exponent_bias_0": ("e2m1_decode", _e2m1_decode_bias0),
    "ue8m0_bias_128": ("ue8m0_decode", _ue8m0_bias128),
    "mxfp4_nibbles_swapped": ("mxfp4_dequantize", _dequant_nibbles_swapped),
    "mxfp4_scales_tiled": ("mxfp4_dequantize", _dequant_scales_tiled),
    "mxfp4_ties_away": ("mxfp4_quantize", _quant_variant(ties="away")),
    "mxfp4_emax_3": ("mxfp4_quantize", _quant_variant(emax=3)),
    "mxfp4_exponent_rounded_up": ("mxfp4_quantize", _quant_variant(ceil_exp=True)),
    "mxfp4_forward_weights_untransposed": ("moe_forward_mxfp4", _forward_mxfp4_untransposed),
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
    "near_ties_drops_last_boundary": ("near_ties", _near_ties(last_boundary=False)),
    "near_ties_no_floor_at_one": ("near_ties", _near_ties(floor=False)),
    "near_ties_signed_scale": ("near_ties", _near_ties(signed=True)),
    "near_ties_ascending": ("near_ties", _near_ties(ascending=True)),
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
