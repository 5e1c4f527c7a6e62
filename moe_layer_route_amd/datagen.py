"""Seeded synthetic inputs for the gpt-oss MoE block.

This module is shared by the tests, the benchmark and the oracle-side checks.
It holds no arithmetic of the MoE method: it only draws normal samples, scales
them and rounds them to bfloat16 (round-to-nearest-even). Every tensor is
returned as a numpy ``uint16`` array holding bfloat16 bit patterns.

Streams: each tensor comes from its own ``numpy.random.Generator(PCG64(...))``
seeded with ``SeedSequence([seed, tensor_id, a, b])``.

* expert tensors (Wgu, bgu, Wd, bd) use ``a = E`` and ``b = expert``, so every
  config with the same E shares the same expert weights;
* the router weight Wr uses ``a = E, b = 0``;
* activations x and the router bias br use ``a = config id, b = T``.

Shapes follow the gpt-oss MoE block (xserv "Phase 19: gpt-oss-20b" page,
section 1, architecture table: hidden 2880, 32 experts, top-4, expert
intermediate 2880, router Linear[2880->32] with bias).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor

import numpy as np

X_ID, WR_ID, BR_ID, WGU_ID, BGU_ID, WD_ID, BD_ID, PERM_ID = 1, 2, 3, 4, 5, 6, 7, 8
MXGU_ID, MXD_ID = 9, 10
F8GU_ID, F8D_ID, F8S_ID = 11, 12, 13

# Scale of x that puts about 5% of the gate/up pre-activations past the +-7
# clamp for weights N(0, 0.02) and biases N(0, 0.01) at H = 2880: a
# pre-activation is then N(0, s^2 * H * 0.02^2 + 0.01^2); the fraction
# P(gate > 7) / 2 + P(|up| > 7) / 2 = 1.5 * Q(7 / sigma) = 0.05 gives
# sigma = 3.817 and s = 3.5562.
X_SCALE_CLAMP5 = 3.5562

WEIGHT_STD = 0.02
BIAS_STD = 0.01
ZIPF_S = 1.1
ZIPF_BETA = 2.0


@dataclasses.dataclass(frozen=True)
class MoEConfig:
    """One workload of the MoE block forward."""

    name: str
    cid: int            # config id used in the activation seed
    T: int              # tokens (rows of x)
    E: int              # experts
    H: int = 2880       # hidden size
    I: int = 2880       # expert intermediate size (gate_up has 2*I outputs)
    k: int = 4          # experts per token
    x_scale: float = X_SCALE_CLAMP5
    router_bias: str = "normal"   # "normal" | "zero" | "zipf"
    description: str = ""


CONFIGS = {
    "c1": MoEConfig("c1", 1, T=8, E=32, router_bias="normal",
                    description="gpt-oss-20b MoE block, T=8, E=32, scaled x, router bias N(0,0.01)"),
    "c2": MoEConfig("c2", 2, T=64, E=32, router_bias="zero",
                    description="gpt-oss-20b MoE block decode batch T=64, E=32, router bias 0"),
    "c3": MoEConfig("c3", 3, T=4096, E=32, x_scale=1.0, router_bias="zero",
                    description="gpt-oss-20b MoE block prefill T=4096, E=32, x N(0,1), router bias 0"),
    "c4": MoEConfig("c4", 4, T=256, E=128, router_bias="normal",
                    description="gpt-oss-120b-shaped MoE block, EAGLE verify T=256 (64 req x 4 draft), E=128"),
    "c5": MoEConfig("c5", 5, T=16384, E=128, router_bias="zipf",
                    description="gpt-oss-120b-shaped MoE block prefill T=16384, E=128, Zipf(1.1) router bias"),
}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Inputs must be finite (the generators only produce finite values); for a
    finite float32 the 32-bit sum below cannot wrap."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & np.uint32(1)
    r = u + np.uint32(0x7FFF)
    r += lsb
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int, tensor_id: int, a: int, b: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id, a, b])))


def normal_bf16(shape, std: float, seed: int, tensor_id: int, a: int, b: int) -> np.ndarray:
    """bf16(std * N(0,1)) drawn in float32 from the (tensor_id, a, b) stream."""
    g = _rng(seed, tensor_id, a, b)
    v = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return f32_to_bf16_bits(v)


def zipf_router_bias(E: int, seed: int, s: float = ZIPF_S, beta: float = ZIPF_BETA) -> np.ndarray:
    """Router bias with a Zipf(s) popularity profile over experts.

    Expert e gets popularity rank perm[e] + 1 (a seeded permutation, so the hot
    experts are not simply the first indices); its bias is
    beta * (ln p_r - mean ln p) with p_r proportional to r^-s.
    """
    perm = _rng(seed, PERM_ID, E, 0).permutation(E)
    ranks = perm.astype(np.float64) + 1.0
    lnp = -s * np.log(ranks)
    b = beta * (lnp - lnp.mean())
    return f32_to_bf16_bits(b.astype(np.float32))


@dataclasses.dataclass
class MoEInputs:
    cfg: MoEConfig
    x: np.ndarray     # [T, H] bf16 bits
    Wr: np.ndarray    # [E, H]
    br: np.ndarray    # [E]
    Wgu: np.ndarray   # [E, H, 2I], output columns interleaved gate0, up0, gate1, up1, ...
    bgu: np.ndarray   # [E, 2I] interleaved the same way
    Wd: np.ndarray    # [E, I, H]
    bd: np.ndarray    # [E, H]

    def arrays(self):
        return (self.x, self.Wr, self.br, self.Wgu, self.bgu, self.Wd, self.bd)


def make_activations(cfg: MoEConfig, seed: int = 0, T: int | None = None) -> np.ndarray:
    T = cfg.T if T is None else T
    return normal_bf16((T, cfg.H), cfg.x_scale, seed, X_ID, cfg.cid, T)


def make_router(cfg: MoEConfig, seed: int = 0):
    Wr = normal_bf16((cfg.E, cfg.H), WEIGHT_STD, seed, WR_ID, cfg.E, 0)
    if cfg.router_bias == "zero":
        br = np.zeros(cfg.E, dtype=np.uint16)
    elif cfg.router_bias == "normal":
        br = normal_bf16((cfg.E,), BIAS_STD, seed, BR_ID, cfg.cid, cfg.T)
    elif cfg.router_bias == "zipf":
        br = zipf_router_bias(cfg.E, seed)
    else:
        raise ValueError(cfg.router_bias)
    return Wr, br


def make_experts(cfg: MoEConfig, seed: int = 0, threads: int | None = None):
    """Expert weights and biases; one stream per (tensor, expert)."""
    E, H, I = cfg.E, cfg.H, cfg.I
    Wgu = np.empty((E, H, 2 * I), dtype=np.uint16)
    Wd = np.empty((E, I, H), dtype=np.uint16)
    bgu = np.empty((E, 2 * I), dtype=np.uint16)
    bd = np.empty((E, H), dtype=np.uint16)

    def one(e):
        Wgu[e] = normal_bf16((H, 2 * I), WEIGHT_STD, seed, WGU_ID, E, e)
        Wd[e] = normal_bf16((I, H), WEIGHT_STD, seed, WD_ID, E, e)
        bgu[e] = normal_bf16((2 * I,), BIAS_STD, seed, BGU_ID, E, e)
        bd[e] = normal_bf16((H,), BIAS_STD, seed, BD_ID, E, e)

    if threads is None:
        threads = min(16, max(1, len(_affinity())))
    if threads <= 1 or E == 1:
        for e in range(E):
            one(e)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(one, range(E)))
    return Wgu, bgu, Wd, bd


def _affinity():
    import os
    try:
        return os.sched_getaffinity(0)
    except AttributeError:  # pragma: no cover
        return range(os.cpu_count() or 1)


def make_inputs(cfg: MoEConfig | str, seed: int = 0, threads: int | None = None) -> MoEInputs:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    x = make_activations(cfg, seed)
    Wr, br = make_router(cfg, seed)
    Wgu, bgu, Wd, bd = make_experts(cfg, seed, threads)
    return MoEInputs(cfg, x, Wr, br, Wgu, bgu, Wd, bd)


def small_config(T: int, E: int, H: int, I: int, k: int, x_scale: float = X_SCALE_CLAMP5,
                 router_bias: str = "normal", cid: int = 100) -> MoEConfig:
    """A reduced shape for parity tests (same distributions, smaller sizes)."""
    return MoEConfig(f"T{T}_E{E}_H{H}_I{I}_k{k}", cid, T=T, E=E, H=H, I=I, k=k,
                     x_scale=x_scale, router_bias=router_bias)


def scale_for_hidden(H: int) -> float:
    """x scale that keeps the pre-activation spread of the full-size configs at hidden size H."""
    return X_SCALE_CLAMP5 * math.sqrt(2880.0 / H)


# ---------------------------------------------------------------------------
# MXFP4 expert weights drawn directly as codes and scales (no quantisation
# arithmetic here).  The distributions are those that N(0, 0.02) weights take
# in the format: magnitude codes 0..7 with the frequencies below, an even
# sign, and the block scale byte 120 (2^-7) for 92.6% of the blocks, 121 for
# 5.6% and 119 for 1.8%; the values then have a standard deviation of about
# 0.02, like the bf16 workloads.
# ---------------------------------------------------------------------------
MX_MAG_FREQ = (0.0811, 0.1587, 0.1474, 0.1312, 0.1620, 0.1505, 0.1183, 0.0508)
MX_SCALE_FREQ = {119: 0.018, 120: 0.926, 121: 0.056}


def _byte_table():
    """65536-entry table: a uniform 16-bit draw -> one code byte (two codes)."""
    p = np.array(MX_MAG_FREQ, dtype=np.float64)
    p = np.concatenate([p, p]) / (2.0 * p.sum())          # sign bit 3, either sign
    pb = np.outer(p, p).reshape(-1)                       # byte = hi * 16 + lo
    edges = np.cumsum(pb) * 65536.0
    u = np.arange(65536) + 0.5
    byte = np.minimum(np.searchsorted(edges, u), 255)
    return byte.astype(np.uint8)                          # index hi*16+lo is the byte value itself


def _scale_table():
    keys = sorted(MX_SCALE_FREQ)
    edges = np.cumsum([MX_SCALE_FREQ[k] for k in keys]) / sum(MX_SCALE_FREQ.values()) * 65536.0
    idx = np.minimum(np.searchsorted(edges, np.arange(65536) + 0.5), len(keys) - 1)
    return np.array(keys, dtype=np.uint8)[idx]


_BYTES = None
_SCALES = None


def mxfp4_draw(N: int, K: int, seed: int, tensor_id: int, a: int, b: int):
    """(codes uint8 [N][K/2], scales uint8 [K/32][N]) from the (tensor_id, a, b) stream."""
    global _BYTES, _SCALES
    if _BYTES is None:
        _BYTES, _SCALES = _byte_table(), _scale_table()
    g = _rng(seed, tensor_id, a, b)
    codes = _BYTES[g.integers(0, 65536, size=(N, K // 2), dtype=np.uint16)]
    scales = _SCALES[g.integers(0, 65536, size=(K // 32, N), dtype=np.uint16)]
    return codes, scales


def make_experts_mxfp4(cfg: MoEConfig, seed: int = 0, threads: int | None = None):
    """MXFP4 expert weights: gate_up codes [E][2I][H/2] and scales [E][H/32][2I],
    down codes [E][H][I/2] and scales [E][I/32][H] (codes K-contiguous, scales
    block-major), one stream per (tensor, expert).  The biases are those of
    make_experts."""
    E, H, I = cfg.E, cfg.H, cfg.I
    assert H % 32 == 0 and I % 32 == 0
    gq = np.empty((E, 2 * I, H // 2), np.uint8)
    gs = np.empty((E, H // 32, 2 * I), np.uint8)
    dq = np.empty((E, H, I // 2), np.uint8)
    ds = np.empty((E, I // 32, H), np.uint8)
    bgu = np.empty((E, 2 * I), dtype=np.uint16)
    bd = np.empty((E, H), dtype=np.uint16)

    def one(e):
        gq[e], gs[e] = mxfp4_draw(2 * I, H, seed, MXGU_ID, E, e)
        dq[e], ds[e] = mxfp4_draw(H, I, seed, MXD_ID, E, e)
        bgu[e] = normal_bf16((2 * I,), BIAS_STD, seed, BGU_ID, E, e)
        bd[e] = normal_bf16((H,), BIAS_STD, seed, BD_ID, E, e)

    if threads is None:
        threads = min(16, max(1, len(_affinity())))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(E)))
    return gq, gs, bgu, dq, ds, bd


# ---------------------------------------------------------------------------
# FP8 (E4M3) expert weights, drawn directly.  A code is sign | exponent field
# << 3 | mantissa field: the exponent field follows FP8_EXP_FREQ, the share
# of each binade among N(0, sigma) weights whose expert maximum (about 5.5
# sigma) is scaled to 448; mantissa and sign are uniform (the top binade
# excludes mantissa 7, the NaN pattern).  One float32 scale per expert near
# 5.5 * 0.02 / 448.
# ---------------------------------------------------------------------------
FP8_EXP_FREQ = (0.0002, 0.0002, 0.0003, 0.0006, 0.0012, 0.0025, 0.0049, 0.0098,
                0.0196, 0.039, 0.075, 0.150, 0.262, 0.316, 0.115, 0.002)
FP8_SCALE_MEAN = 5.5 * 0.02 / 448.0

_F8 = None


def _fp8_table():
    """65536-entry table: a uniform 16-bit draw -> one code."""
    p = np.zeros(256)
    for ex, f in enumerate(FP8_EXP_FREQ):
        mants = 7 if ex == 15 else 8
        for m in range(mants):
            p[(ex << 3) | m] = f / mants / 2.0
            p[0x80 | (ex << 3) | m] = f / mants / 2.0
    edges = np.cumsum(p) / p.sum() * 65536.0
    return np.minimum(np.searchsorted(edges, np.arange(65536) + 0.5), 255).astype(np.uint8)


def fp8_draw(N: int, K: int, seed: int, tensor_id: int, a: int, b: int) -> np.ndarray:
    """codes uint8 [N][K] from the (tensor_id, a, b) stream."""
    global _F8
    if _F8 is None:
        _F8 = _fp8_table()
    return _F8[_rng(seed, tensor_id, a, b).integers(0, 65536, size=(N, K), dtype=np.uint16)]


def make_experts_fp8(cfg: MoEConfig, seed: int = 0, threads: int | None = None):
    """FP8 expert weights: gate_up codes [E][2I][H] and scales [E], down codes
    [E][H][I] and scales [E] (codes K-contiguous), one stream per (tensor,
    expert).  The biases are those of make_experts."""
    E, H, I = cfg.E, cfg.H, cfg.I
    gq = np.empty((E, 2 * I, H), np.uint8)
    dq = np.empty((E, H, I), np.uint8)
    bgu = np.empty((E, 2 * I), dtype=np.uint16)
    bd = np.empty((E, H), dtype=np.uint16)
    g = _rng(seed, F8S_ID, E, 0)
    gs = (FP8_SCALE_MEAN * (1.0 + 0.05 * g.standard_normal(E))).astype(np.float32)
    ds = (FP8_SCALE_MEAN * (1.0 + 0.05 * g.standard_normal(E))).astype(np.float32)

    def one(e):
        gq[e] = fp8_draw(2 * I, H, seed, F8GU_ID, E, e)
        dq[e] = fp8_draw(H, I, seed, F8D_ID, E, e)
        bgu[e] = normal_bf16((2 * I,), BIAS_STD, seed, BGU_ID, E, e)
        bd[e] = normal_bf16((H,), BIAS_STD, seed, BD_ID, E, e)

    if threads is None:
        threads = min(16, max(1, len(_affinity())))
    with ThreadPoolExecutor(max(1, threads)) as ex:
        list(ex.map(one, range(E)))
    return gq, gs, bgu, dq, ds, bd
