"""CPU float64 oracle of the gpt-oss MoE block forward.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The
product path (the HIP library and its Python binding) never imports it, and
this module imports nothing from the product path: its only inputs are numpy
arrays of bfloat16 bit patterns.

What it computes, and where the pages define it (xserv "Phase 19: gpt-oss-20b
MoE support" page):

* section 1, architecture table, row "MoE": a plain Linear router with bias
  over the hidden state, 32 experts, top-4, expert intermediate size 2880;
* section 1, architecture table, row for the activation: the clamped,
  interleaved GLU -- gate is the even columns of the gate_up output, up the odd
  ones, gate is clamped from above at 7, up to [-7, 7], and
  h = (up + 1) * gate * sigmoid(1.702 * gate);
* section 2, the forward pipeline: router -> top-k softmax -> gate_up GEMM ->
  bias -> GLU -> down GEMM -> bias -> weighted sum over the top-4 experts only,
  with unselected experts skipped rather than multiplied by zero.

Everything is computed in float64 from the exactly widened bf16 inputs;
nothing is rounded except where a reading below says so.

Readings where the pages are silent:

* R1  softmax over the k selected logits (softmax over all E followed by
      renormalising over the top k is the same number);
* R2  top-k order is (logit descending, expert index ascending); equal logits
      go to the lower index;
* R3  the top-k *decision* is taken on the logits rounded to float32, the
      precision the GPU kernel decides in; weights use the float64 logits;
* R4  biases are added before the clamp (gate_up) and inside the weighted sum
      (down), i.e. y = sum_j w_j * (h_j @ Wd[e_j] + bd[e_j]);
* R5  the clamped gate value is used in both factors of gate*sigmoid(1.702*gate);
      up is clamped first, then 1 is added.

The MXFP4 weight format (section 5 of the same page) and its readings M1-M3,
and the FP8 W8A8 variant (same section) and its readings F1-F6, are stated
next to their functions below.
"""
from __future__ import annotations

import numpy as np

GLU_ALPHA = 1.702     # sigmoid slope of the GLU (architecture table, activation row)
GLU_LIMIT = 7.0       # clamp bound of gate (upper) and up (both sides)


# --------------------------------------------------------------------------
# bf16 bit patterns -> float64 (exact widening: every bf16 is a float32)
# --------------------------------------------------------------------------
def widen(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Router (section 1 "MoE" row: Linear[H -> E] + bias; section 2 step 1)
# --------------------------------------------------------------------------
def router_logits(x, Wr, br) -> np.ndarray:
    """logits[t, e] = sum_h x[t, h] * Wr[e, h] + br[e], float64, shape [T, E]."""
    return widen(x) @ widen(Wr).T + widen(br)[None, :]


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k expert ids per row, ordered by (value desc, index asc).  [T, k] int32.

    The comparison uses the values as given (the caller passes the float32
    logits, reading R3).  -0.0 and +0.0 compare equal, so they tie and the
    lower index wins."""
    T, E = logits.shape
    ids = np.empty((T, k), dtype=np.int32)
    idx = np.arange(E)
    for t in range(T):
        v = logits[t]
        # lexsort sorts by the last key first: primary key -value, then index
        order = np.lexsort((idx, -v.astype(np.float64)))
        ids[t] = order[:k]
    return ids


def routing_weights(logits64: np.ndarray, ids: np.ndarray) -> np.ndarray:
    """Softmax over the k selected logits (reading R1).  [T, k] float64."""
    sel = np.take_along_axis(logits64, ids.astype(np.int64), axis=1)
    m = sel.max(axis=1, keepdims=True)
    ex = np.exp(sel - m)
    return ex / ex.sum(axis=1, keepdims=True)


def route(x, Wr, br, k: int):
    """moe_route: returns (ids [T,k] int32, w [T,k] float64, logits float64)."""
    lg = router_logits(x, Wr, br)
    ids = select_topk(lg.astype(np.float32), k)
    w = routing_weights(lg, ids)
    return ids, w, lg


# --------------------------------------------------------------------------
# Expert MLP (section 1 activation row; section 2 gate_up -> bias -> GLU ->
# down -> bias)
# --------------------------------------------------------------------------
def clamped_glu(u: np.ndarray) -> np.ndarray:
    """h[..., i] from the interleaved gate_up pre-activation u[..., 2I]."""
    gate = np.minimum(u[..., 0::2], GLU_LIMIT)
    up = np.clip(u[..., 1::2], -GLU_LIMIT, GLU_LIMIT)
    glu = gate / (1.0 + np.exp(-GLU_ALPHA * gate))
    return (up + 1.0) * glu


def expert_mlp(xrows64: np.ndarray, Wgu_e64, bgu_e64, Wd_e64, bd_e64):
    """One expert applied to rows of x: returns (u, h, o), all float64."""
    u = xrows64 @ Wgu_e64 + bgu_e64
    h = clamped_glu(u)
    o = h @ Wd_e64 + bd_e64
    return u, h, o


# --------------------------------------------------------------------------
# Expert-contiguous permutation (the device-side bookkeeping that replaces
# copying every token to every expert, section 2)
# --------------------------------------------------------------------------
def expert_permutation(ids: np.ndarray, E: int):
    """Counting sort of the T*k (token, slot) pairs by expert, stable in slot order.

    Returns cnt [E], off [E+1] (exclusive prefix sum), rows [T*k] (rows[off[e]+r]
    is the r-th slot s = t*k + j routed to e, in increasing s) and pos [T*k]
    (the inverse: rows[pos[s]] == s)."""
    flat = ids.reshape(-1).astype(np.int64)
    cnt = np.zeros(E, dtype=np.int64)
    for e in flat:
        cnt[e] += 1
    off = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):
        off[e + 1] = off[e] + cnt[e]
    fill = off[:-1].copy()
    rows = np.empty(flat.size, dtype=np.int64)
    pos = np.empty(flat.size, dtype=np.int64)
    for s, e in enumerate(flat):
        rows[fill[e]] = s
        pos[s] = fill[e]
        fill[e] += 1
    return (cnt.astype(np.int32), off.astype(np.int32), rows.astype(np.int32),
            pos.astype(np.int32))


# --------------------------------------------------------------------------
# Whole block, sparse formulation: only selected experts are read
# --------------------------------------------------------------------------
def moe_forward(x, Wr, br, Wgu, bgu, Wd, bd, k: int, tokens=None, keep=False, experts=None):
    """Full forward.  Returns a dict with y [T', H] float64, ids, w, logits,
    and, if keep, u/h/o per slot [T'*k, ...] in slot order s = t*k + j.

    tokens: optional array of token indices; the result then covers only those
    rows of x (used to check sampled outputs at full size).
    experts: optional (e_begin, e_end): y then sums only the slots whose expert
    lies in that range -- one expert-parallel rank's share (section 2 of the
    Phase 19 page: expert parallelism filters by expert range and sums the
    ranks' partial outputs).  The weights stay indexed by global expert id."""
    def weights(e):
        return widen(Wgu[e]), widen(bgu[e]), widen(Wd[e]), widen(bd[e])
    return _forward(x, Wr, br, weights, Wgu.shape[2], Wd.shape[2], k, tokens, keep, experts)


def _forward(x, Wr, br, weights, I2, Hout, k, tokens=None, keep=False, experts=None):
    """The sparse forward over a weight provider: weights(e) returns expert
    e's (Wgu [H][2I], bgu [2I], Wd [I][H], bd [H]) as float64 in x.W form."""
    ids, w, lg = route(x if tokens is None else x[np.asarray(tokens)], Wr, br, k)
    xs = widen(x if tokens is None else x[np.asarray(tokens)])
    T, H = xs.shape
    E = Wr.shape[0]
    y = np.zeros((T, Hout), dtype=np.float64)
    if keep:
        u_all = np.zeros((T * k, I2))
        h_all = np.zeros((T * k, I2 // 2))
        o_all = np.zeros((T * k, Hout))
    flat = ids.reshape(-1)
    e_lo, e_hi = (0, E) if experts is None else experts
    for e in range(e_lo, e_hi):
        slots = np.nonzero(flat == e)[0]
        if slots.size == 0:
            continue               # skipped, never multiplied by zero
        toks = slots // k
        u, h, o = expert_mlp(xs[toks], *weights(e))
        ws = w.reshape(-1)[slots]
        np.add.at(y, toks, ws[:, None] * o)
        if keep:
            u_all[slots], h_all[slots], o_all[slots] = u, h, o
    out = {"y": y, "ids": ids, "w": w, "logits": lg}
    if keep:
        out.update(u=u_all, h=h_all, o=o_all)
    return out


# --------------------------------------------------------------------------
# Padded batches and expert loads (the verify-graph page: statically sized
# buffers whose tail rows are padding; the Phase 19 page: a per-layer
# recorder of how many routed slots each expert receives)
# --------------------------------------------------------------------------
def expert_loads(ids: np.ndarray, E: int) -> np.ndarray:
    """Number of (token, slot) pairs routed to each expert; ids < 0 are not routed."""
    flat = ids.reshape(-1)
    return np.bincount(flat[flat >= 0], minlength=E)


def moe_forward_padded(x, Wr, br, Wgu, bgu, Wd, bd, k: int, n_valid: int):
    """Rows t >= n_valid (clamped to [0, T]) are padding: routed nowhere (id
    -1, weight 0), y = 0; the other rows are moe_forward of those rows alone.
    Also returns the expert loads of the valid rows."""
    T, E = x.shape[0], Wr.shape[0]
    nv = min(max(int(n_valid), 0), T)
    y = np.zeros((T, Wd.shape[2]))
    ids = np.full((T, k), -1, dtype=np.int32)
    w = np.zeros((T, k))
    if nv:
        r = moe_forward(x[:nv], Wr, br, Wgu, bgu, Wd, bd, k=k)
        y[:nv], ids[:nv], w[:nv] = r["y"], r["ids"], r["w"]
    return {"y": y, "ids": ids, "w": w, "loads": expert_loads(ids, E)}


# --------------------------------------------------------------------------
# MXFP4 expert weights (section 5 of the Phase 19 page, "MXFP4 W4A16": the
# weights are 4-bit E2M1 values with one UE8M0 power-of-two scale per 32
# values; activations stay bf16).  Readings where the page is silent:
#   M1  a block is 32 consecutive values along the contraction dimension K
#       (the dimension a dot product runs over), so the codes are stored
#       K-contiguous: codes [E][N][K/2] (byte i of row n holds k = 2i in bits
#       0-3 and k = 2i+1 in bits 4-7); the scales are stored block-major,
#       scales [E][K/32][N] (scales[e][b][n] scales k = 32b..32b+31 of
#       column n);
#   M2  the quantiser is the microscaling formats' reference conversion: per
#       block, X = 2^(floor(log2(max|v|)) - 2) (2 is the largest exponent of
#       E2M1, whose largest value is 6 = 1.5 * 2^2), each v / X rounded to the
#       nearest E2M1 value with ties to the even code and magnitudes above 6
#       saturated to 6; an all-zero block takes X = 2^-127 (code 0 stored);
#       the sign bit of a code is the sign bit of v;
#   M3  dequantisation is exact: value = E2M1(code) * 2^(scale - 127); scale
#       byte 255 is NaN.
# --------------------------------------------------------------------------
E2M1_EMAX = 2


def e2m1_decode(code: int) -> float:
    """Value of a 4-bit E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1),
    bit 0 mantissa; exponent 0 is subnormal (0 or 0.5)."""
    sign = -1.0 if (code >> 3) & 1 else 1.0
    ex = (code >> 1) & 3
    man = code & 1
    mag = 0.5 * man if ex == 0 else (1.0 + 0.5 * man) * 2.0 ** (ex - 1)
    return sign * mag


E2M1_VALUES = np.array([e2m1_decode(c) for c in range(16)], dtype=np.float64)


def ue8m0_decode(e) -> np.ndarray:
    """2^(e - 127) for scale bytes e; 255 is NaN."""
    e = np.asarray(e, dtype=np.int64)
    v = np.ldexp(1.0, e - 127)
    return np.where(e == 255, np.nan, v)


def mxfp4_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes uint8 [..., N, K/2] and scales uint8 [..., K/32, N] -> float64 [..., N, K]."""
    codes = np.asarray(codes, dtype=np.uint8)
    q = np.empty(codes.shape[:-1] + (2 * codes.shape[-1],), dtype=np.float64)
    q[..., 0::2] = E2M1_VALUES[codes & 15]
    q[..., 1::2] = E2M1_VALUES[codes >> 4]
    sc = np.repeat(np.swapaxes(ue8m0_decode(scales), -1, -2), 32, axis=-1)
    return q * sc


def mxfp4_quantize(w: np.ndarray):
    """float [..., N, K] (K % 32 == 0) -> (codes uint8 [..., N, K/2], scales uint8 [..., K/32, N])."""
    w = np.asarray(w, dtype=np.float64)
    K = w.shape[-1]
    assert K % 32 == 0
    blk = w.reshape(w.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    _, p = np.frexp(amax)                     # amax = m * 2^p, m in [0.5, 1)
    shared = np.where(amax > 0, p - 1 - E2M1_EMAX, -127)
    shared = np.clip(shared, -127, 127)
    X = np.ldexp(1.0, shared)[..., None]
    v = np.abs(blk) / X                        # exact: X is a power of two
    mags = E2M1_VALUES[:8]
    dist = np.abs(v[..., None] - mags)         # [..., 32, 8]
    best = dist.min(axis=-1, keepdims=True)
    # among the nearest magnitudes take the even code (ties to even)
    cand = (dist == best)
    even = cand & (np.arange(8) % 2 == 0)
    mag_code = np.where(even.any(axis=-1), even.argmax(axis=-1), cand.argmax(axis=-1))
    sign = np.signbit(blk).astype(np.int64)
    code = (sign << 3) | mag_code
    code = code.reshape(w.shape)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    scales = np.swapaxes((shared + 127).astype(np.uint8), -1, -2).copy()
    return packed, scales


def moe_forward_mxfp4(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int, tokens=None, keep=False,
                      experts=None):
    """The forward with MXFP4 expert weights (W4A16): gate_up codes [E][2I][H/2]
    and scales [E][H/32][2I], down codes [E][H][I/2] and scales [E][I/32][H];
    the weights are dequantised exactly and the rest is moe_forward."""
    def weights(e):
        return (mxfp4_dequantize(Wgu_q[e], Wgu_s[e]).T, widen(bgu[e]),
                mxfp4_dequantize(Wd_q[e], Wd_s[e]).T, widen(bd[e]))
    return _forward(x, Wr, br, weights, Wgu_q.shape[1], Wd_q.shape[1], k, tokens, keep, experts)


# --------------------------------------------------------------------------
# FP8 W8A8 (section 5 of the Phase 19 page: 8-bit weights with one scalar
# scale per expert, stored transposed [E][N][K]; the scales applied after the
# product).  Readings where the page is silent:
#   F1  the 8-bit format is OCP FP8 E4M3 (bias 7, no infinities, largest
#       finite 448, S.1111.111 is NaN); conversion to it rounds to nearest
#       with ties to the even code and saturates to +-448; NaN becomes 0x7F;
#   F2  a scale is s = amax / 448, and the codes are E4M3(a * (448 / amax)),
#       each of the three operations in float32 (the precision the codes are
#       decided in); amax = 0 gives s = 1 and codes of a * 1;
#   F3  weights: one scale per expert and matrix (amax over the whole
#       expert), codes stored K-contiguous [E][N][K];
#   F4  activations ("A8", not specified further): one dynamic scale per row,
#       a token's row of x for gate_up and a (token, slot) row of h for down;
#   F5  h is rounded to bf16 (RNE), the type activations are kept in between
#       the two products, before it is quantised;
#   F6  each product is sum(code_a * code_w) * s_a * s_w, i.e. the exact
#       dequantised operands, and then the bias.
# --------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(code: int) -> float:
    """Value of an OCP E4M3 code: bit 7 sign, bits 6..3 exponent (bias 7),
    bits 2..0 mantissa; exponent 0 is subnormal (m * 2^-9); 0x7F/0xFF NaN."""
    sign = -1.0 if code & 0x80 else 1.0
    ex = (code >> 3) & 15
    man = code & 7
    if ex == 15 and man == 7:
        return float("nan")
    mag = man * 2.0 ** -9 if ex == 0 else (8 + man) * 2.0 ** (ex - 10)
    return sign * mag


E4M3_VALUES = np.array([e4m3_decode(c) for c in range(256)], dtype=np.float64)


def e4m3_encode(v) -> np.ndarray:
    """float32 values -> E4M3 codes (uint8): nearest value, ties to the even
    code, magnitudes from 448 up (and infinities) saturated to 448, NaN 0x7F."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)
    a = np.where(np.isnan(v), 0.0, np.abs(v))
    # quantum of a's binade: 2^(floor(log2 a) - 3) for normals, 2^-9 below 2^-6
    _, p = np.frexp(np.where(a > 0, a, 1.0))          # a = m * 2^p, m in [0.5, 1)
    quantum = np.ldexp(1.0, np.maximum(p - 4, -9))
    q = np.rint(a / quantum) * quantum                  # exact; rint is half-even
    q = np.minimum(q, E4M3_MAX)
    _, pq = np.frexp(np.where(q > 0, q, 1.0))
    normal = q >= 2.0 ** -6
    ex = np.where(normal, pq - 1 + 7, 0)
    man = np.where(normal, q / np.ldexp(1.0, pq - 4) - 8, q / 2.0 ** -9)
    code = (ex.astype(np.int64) << 3) | man.astype(np.int64)
    code = code | (np.signbit(v).astype(np.int64) << 7)
    code = np.where(np.isnan(v), 0x7F, code)
    return code.astype(np.uint8)


def fp8_scale(amax):
    """(s, inv) for float32 maxima: s = amax / 448, inv = 448 / amax, both
    rounded to float32; amax = 0 gives (1, 1)."""
    amax = np.asarray(amax, dtype=np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(E4M3_MAX), amax)
    s = np.where(zero, np.float32(1), safe / np.float32(E4M3_MAX)).astype(np.float32)
    inv = np.where(zero, np.float32(1), np.float32(E4M3_MAX) / safe).astype(np.float32)
    return s, inv


def fp8_quantize_rows(a) -> tuple:
    """float32 [R][K] (bf16 values) -> (codes uint8 [R][K], s float32 [R]):
    one scale per row (F2, F4)."""
    a = np.asarray(a, dtype=np.float32)
    s, inv = fp8_scale(np.abs(a).max(axis=-1))
    return e4m3_encode(a * inv[..., None]), s


def fp8_quantize_weights(W) -> tuple:
    """bf16 bits [E][K][N] (x.W form) -> (codes uint8 [E][N][K], s float32 [E]):
    one scale per expert (F2, F3)."""
    w = widen(W).astype(np.float32)
    s, inv = fp8_scale(np.abs(w).reshape(w.shape[0], -1).max(axis=-1))
    codes = e4m3_encode(w * inv[:, None, None])
    return np.ascontiguousarray(np.swapaxes(codes, 1, 2)), s


def fp8_dequantize(codes, s) -> np.ndarray:
    """codes [..., R, K] with one scale per leading index -> float64."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)] * np.asarray(s, np.float64)[..., None, None]


def bf16_round(x) -> np.ndarray:
    """float64 -> the nearest bf16 value (ties to even), as float64: 8
    significant bits for normals, a quantum of 2^-133 below 2^-126."""
    x = np.asarray(x, dtype=np.float64)
    _, p = np.frexp(np.where(x != 0, x, 1.0))
    quantum = np.ldexp(1.0, np.maximum(p - 8, -133))
    return np.where(np.isfinite(x), np.rint(x / quantum) * quantum, x)


def fp8_down(hb, Wd_q_e, s_d_e, bd_e64):
    """Down product of one expert on bf16-rounded h rows (F4-F6): returns the
    row codes, row scales and o = (codes_h . codes_d^T) * s_h * s_d + bd."""
    hq, sh = fp8_quantize_rows(hb)
    o = (E4M3_VALUES[hq] @ E4M3_VALUES[Wd_q_e].T) * (sh.astype(np.float64)[:, None] * float(s_d_e)) + bd_e64
    return hq, sh, o


def moe_forward_fp8(x, Wr, br, Wgu_q, Wgu_s, bgu, Wd_q, Wd_s, bd, k: int, tokens=None, keep=False,
                    experts=None):
    """The forward with FP8 W8A8 experts: gate_up codes [E][2I][H] with scales
    [E], down codes [E][H][I] with scales [E].  x rows are quantised per token
    (F4), h rows per (token, slot) after rounding to bf16 (F5).  Returns what
    moe_forward returns, plus (keep) the h codes and scales per slot."""
    sel = slice(None) if tokens is None else np.asarray(tokens)
    ids, w, lg = route(x[sel], Wr, br, k)
    xq, sx = fp8_quantize_rows(widen(x[sel]))
    T = xq.shape[0]
    E, I2, Hout = Wr.shape[0], Wgu_q.shape[1], Wd_q.shape[1]
    y = np.zeros((T, Hout))
    if keep:
        u_all, h_all, o_all = np.zeros((T * k, I2)), np.zeros((T * k, I2 // 2)), np.zeros((T * k, Hout))
        hq_all, sh_all = np.zeros((T * k, I2 // 2), np.uint8), np.zeros(T * k, np.float32)
    flat = ids.reshape(-1)
    e_lo, e_hi = (0, E) if experts is None else experts
    for e in range(e_lo, e_hi):
        slots = np.nonzero(flat == e)[0]
        if slots.size == 0:
            continue               # skipped, never multiplied by zero
        toks = slots // k
        u = (E4M3_VALUES[xq[toks]] @ E4M3_VALUES[Wgu_q[e]].T) * (sx.astype(np.float64)[toks, None]
                                                                  * float(Wgu_s[e])) + widen(bgu[e])
        h = clamped_glu(u)
        hq, sh, o = fp8_down(bf16_round(h), Wd_q[e], Wd_s[e], widen(bd[e]))
        np.add.at(y, toks, w.reshape(-1)[slots][:, None] * o)
        if keep:
            u_all[slots], h_all[slots], o_all[slots] = u, h, o
            hq_all[slots], sh_all[slots] = hq, sh
    out = {"y": y, "ids": ids, "w": w, "logits": lg, "sx": sx}
    if keep:
        out.update(u=u_all, h=h_all, o=o_all, hq=hq_all, sh=sh_all, xq=xq)
    return out


# --------------------------------------------------------------------------
# Second formulation: every expert on every token, then select (the dense
# "replicate to all local experts" pipeline of section 2).  Small shapes only.
# --------------------------------------------------------------------------
def moe_forward_dense(x, Wr, br, Wgu, bgu, Wd, bd, k: int):
    ids, w, lg = route(x, Wr, br, k)
    xs = widen(x)
    E = Wr.shape[0]
    outs = np.stack([expert_mlp(xs, widen(Wgu[e]), widen(bgu[e]), widen(Wd[e]), widen(bd[e]))[2]
                     for e in range(E)])          # [E, T, H]
    T = xs.shape[0]
    y = np.zeros((T, Wd.shape[2]))
    for t in range(T):
        for j in range(k):
            y[t] += w[t, j] * outs[ids[t, j], t]
    return {"y": y, "ids": ids, "w": w, "logits": lg}


# --------------------------------------------------------------------------
# Diagnostics reported next to the comparisons
# --------------------------------------------------------------------------
def near_ties(logits64: np.ndarray, k: int, rel: float = 1e-5) -> np.ndarray:
    """Tokens whose float64 gap at any rank boundary 1|2 ... k|k+1 is below
    rel * max(1, |logit|): the tokens where a float32 router could differ."""
    s = -np.sort(-logits64, axis=1)
    kk = min(k + 1, s.shape[1])
    gaps = s[:, :kk - 1] - s[:, 1:kk]
    scale = np.maximum(1.0, np.abs(s[:, :kk - 1]))
    return np.nonzero((gaps < rel * scale).any(axis=1))[0]


def clamp_fraction(u: np.ndarray) -> float:
    """Fraction of gate/up pre-activations that the GLU clamps (gate > 7 or |up| > 7)."""
    g = u[..., 0::2]
    p = u[..., 1::2]
    return float(((g > GLU_LIMIT).sum() + (np.abs(p) > GLU_LIMIT).sum()) / u.size)
