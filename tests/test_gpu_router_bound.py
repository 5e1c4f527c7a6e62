"""The MFMA router's error bound against what the matrix cores actually do
(needs an MI355X).

The MFMA router (route.hip) forms each float32 logit with
v_mfma_f32_16x16x32_bf16 and trusts its top-k order only when every gap
exceeds a bound of err_steps * u * S per logit (doubled, plus two ulps), with
u = 2^-24, S = sum |x| |w| and err_steps = max(128, steps + 41) for a K slice
of `steps` 32-wide MFMA steps; otherwise it recomputes the candidates exactly.
That is only sound if the instruction's own accumulation stays inside the
bound.  moe_probe_mfma_dot_bf16 forms dot products exactly as the router does
(one accumulator over the whole of K), and these tests measure its error
against exact float64 sums on inputs built to make float32 accumulation
errors large: heavy cancellation (S >> |sum|), partial sums that grow to S/2
and return, and steps whose 32 products mix one large and many tiny terms.
Then the router itself is run on inputs whose logits cancel heavily and lie
within a few float32 ulps of each other (the Phase 19 page, section 2: the
ids never reach the host, so a wrong pick would go unnoticed downstream).
"""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding, datagen as d  # noqa: E402
import oracle.moe_oracle as orc  # noqa: E402
from checks import assert_routing, dev  # noqa: E402

pytestmark = pytest.mark.gpu
U = 2.0 ** -24


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf(a):
    return d.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _f64(bits):
    return d.bf16_bits_to_f32(bits).astype(np.float64)


def _err_steps(K):
    """The router's bound factor for one K slice of K/32 steps (before its doubling)."""
    return max(128.0, K / 32 + 41)


def _inputs(kind, M, K, rng):
    if kind == "random":
        A = _bf(3.5 * rng.standard_normal((M, K)))
        B = _bf(0.02 * rng.standard_normal((16, K)))
    elif kind == "cancel_pairs":
        # equal columns in pairs, weights of opposite sign and nearly equal size
        a = _bf(3.5 * rng.standard_normal((M, K // 2)))
        A = np.repeat(a, 2, axis=1)
        w = 0.02 * rng.standard_normal((16, K // 2)).astype(np.float32)
        eps = rng.choice([0.0, 2.0 ** -7, -(2.0 ** -7), 2.0 ** -5], size=w.shape)
        B = np.empty((16, K), np.uint16)
        B[:, 0::2] = _bf(w)
        B[:, 1::2] = _bf(-w * (1 + eps))
    elif kind == "grow_and_return":
        # positive products over the first half of K, negative over the second:
        # the partial sums climb to about S/2 and come back near 0
        A = _bf(np.abs(3.5 * rng.standard_normal((M, K))) + 0.5)
        w = np.abs(0.02 * rng.standard_normal((16, K // 2))) + 0.001
        B = np.concatenate([_bf(w), _bf(-w[:, ::-1] * (1 + 2.0 ** -8 * rng.standard_normal(w.shape)))], axis=1)
    elif kind == "one_large_many_tiny":
        # each 32-wide step: one product near 1, 31 products near 2^-24 of it
        A = _bf(1.0 + 0.01 * rng.standard_normal((M, K)))
        B = _bf(2.0 ** -24 * (1 + rng.random((16, K))))
        B[:, ::32] = _bf(1.0 + 0.01 * rng.standard_normal((16, K // 32)))
        B[8:, ::32] = _bf(-_f64(B[8:, ::32]) * (1 + 2.0 ** -8))     # and with cancellation across steps
    else:
        raise ValueError(kind)
    return A, B


@pytest.mark.parametrize("K", [2880, 32, 256, 16384])
@pytest.mark.parametrize("kind", ["random", "cancel_pairs", "grow_and_return", "one_large_many_tiny"])
def test_mfma_accumulation_stays_inside_the_router_bound(kind, K):
    _need_gpu()
    rng = np.random.default_rng(K + len(kind))
    M = 256
    A, B = _inputs(kind, M, K, rng)
    got = binding.probe_mfma_dot_bf16(dev(A), dev(B)).cpu().numpy().astype(np.float64)
    a, b = _f64(A), _f64(B)
    exact = a @ b.T                        # products exact in float64, sum error ~1e-16 S
    S = np.abs(a) @ np.abs(b).T
    ratio = np.abs(got - exact) / (U * S)
    worst = float(ratio.max())
    print(f"[router bound] {kind} K={K}: max |mfma - exact| = {worst:.2f} u S "
          f"(median {float(np.median(ratio)):.3f}); the router allows {_err_steps(K):.0f} u S, doubled")
    assert worst <= _err_steps(K), worst


def test_mfma_step_internal_precision_is_reported():
    """Not a bound check: what one instruction does with 32 products whose sum
    is not representable in float32 (printed for the record)."""
    _need_gpu()
    A = np.full((16, 32), _bf(1.0)[()], np.uint16)
    B = np.full((16, 32), _bf(2.0 ** -24)[()], np.uint16)
    B[:, 0] = _bf(1.0)
    got = binding.probe_mfma_dot_bf16(dev(A), dev(B)).cpu().numpy()
    exact = 1.0 + 31 * 2.0 ** -24
    seq = np.float32(1.0)
    for _ in range(31):
        seq = np.float32(seq + np.float32(2.0 ** -24))
    print(f"[router bound] 1 + 31 * 2^-24: mfma {float(got[0, 0])!r}, exact {exact!r}, "
          f"float32 rounded {float(np.float32(exact))!r}, sequential float32 {float(seq)!r}")
    assert abs(float(got[0, 0]) - exact) <= 32 * U * (1 + 31 * 2.0 ** -24)


def _near_tie_router(T, E, H, rng):
    """x columns equal in pairs and router rows whose pair weights nearly
    cancel (S / |logit| in the thousands); the experts of a group differ only
    by which weight of a pair sits in which column (the exact logit does not
    change, the float32 rounding does) and by a tiny term on a coordinate
    where x is tiny, which moves the logit by a few float32 ulps."""
    npair = H // 2
    xa = _bf(3.5 * rng.standard_normal((T, npair)))
    x = np.repeat(xa, 2, axis=1)
    x[:, 0] = _bf(2.0 ** -10 * rng.standard_normal(T))
    x[:, 1] = 0
    groups = 4
    base = []
    for _ in range(groups):
        w = 0.02 * rng.standard_normal(npair).astype(np.float32)
        eps = rng.choice([0.0, 2.0 ** -7, -(2.0 ** -7)], size=npair)
        row = np.empty(H, np.uint16)
        row[0::2] = _bf(w)
        row[1::2] = _bf(-w * (1 + eps))
        base.append(row)
    Wr = np.empty((E, H), np.uint16)
    for e in range(E):
        row = base[e % groups].copy()
        swap = np.nonzero(rng.random(npair) < 0.5)[0]
        swap = swap[swap > 0]
        row[2 * swap], row[2 * swap + 1] = row[2 * swap + 1].copy(), row[2 * swap].copy()
        row[0] = _bf([2.0 ** -12 * (1 + int(rng.integers(0, 4)) * 2.0 ** -7)])[0]
        Wr[e] = row
    return x, Wr


@pytest.mark.parametrize("T,E,k", [(200, 32, 4), (200, 128, 4), (8256, 128, 4), (97, 256, 8)])
def test_router_on_cancelling_near_tied_logits(T, E, k):
    _need_gpu()
    rng = np.random.default_rng(T * E)
    H = 2880
    x, Wr = _near_tie_router(T, E, H, rng)
    br = np.zeros(E, np.uint16)
    lg = orc.router_logits(x, Wr, br)
    S = d.bf16_bits_to_f32(x).astype(np.float64).__abs__() @ d.bf16_bits_to_f32(Wr).astype(np.float64).__abs__().T
    ids_ref, w_ref, _ = orc.route(x, Wr, br, k)
    near = orc.near_ties(lg, k)
    print(f"[router bound] T={T} E={E}: median S/|logit| {float(np.median(S / np.maximum(np.abs(lg), 1e-30))):.0f}, "
          f"{near.size} of {T} tokens are near ties")
    assert near.size > T // 4           # the construction does make near ties
    for method in ("mfma", "exact"):
        ids, w = binding.moe_route(dev(x), dev(Wr), dev(br), k, method=method)
        assert_routing(ids.cpu().numpy(), w.cpu().numpy(), ids_ref, w_ref, lg, k)
