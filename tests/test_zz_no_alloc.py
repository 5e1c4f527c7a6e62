"""moe_forward_noalloc (the library's own scratch array, no workspace) against
moe_forward with a caller workspace, through the C ABI (needs an MI355X).

Two calls in a row, the second smaller than the first (the array keeps the
first call's contents), on both expert paths; then a size beyond the array
is rejected, and a call after that still works."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding, datagen as d  # noqa: E402
from checks import bf16_bits, dev  # noqa: E402

pytestmark = pytest.mark.gpu


def _inputs(T, E, H, I, k, seed):
    cfg = d.small_config(T=T, E=E, H=H, I=I, k=k, x_scale=d.scale_for_hidden(H))
    return [dev(a) for a in d.make_inputs(cfg, seed=seed, threads=4).arrays()]


def _both(args, T, k):
    ids_a = torch.empty((T, k), dtype=torch.int32, device="cuda")
    w_a = torch.empty((T, k), dtype=torch.float32, device="cuda")
    ids_b = torch.full((T, k), -7, dtype=torch.int32, device="cuda")
    w_b = torch.full((T, k), -7.0, dtype=torch.float32, device="cuda")
    y_a = binding.moe_forward(*args, k=k, topk_ids=ids_a, topk_w=w_a)
    y_b = torch.empty_like(y_a)
    y_b.view(torch.int16).fill_(-1)
    binding.moe_forward_noalloc(*args, k=k, y=y_b, topk_ids=ids_b, topk_w=w_b)
    torch.cuda.synchronize()
    return (bf16_bits(y_a), ids_a.cpu().numpy(), w_a.cpu().numpy()), (bf16_bits(y_b), ids_b.cpu().numpy(),
                                                                       w_b.cpu().numpy())


def test_noalloc_matches_the_workspace_forward_on_two_calls_in_a_row():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # first call: 200 tokens over 16 experts (T*k/E = 50 rows per expert: the tiled GEMM path)
    T1, E1, k1 = 200, 16, 4
    print(f"[noalloc] call 1: T={T1} E={E1} H=I=2880 k={k1}", flush=True)
    a, b = _both(_inputs(T1, E1, 2880, 2880, k1, seed=5), T1, k1)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all() and (a[2] == b[2]).all()
    # second call, smaller: 37 tokens over 8 experts, other sizes (the streaming path)
    T2, E2, k2 = 37, 8, 2
    print(f"[noalloc] call 2: T={T2} E={E2} H=1024 I=512 k={k2}", flush=True)
    a, b = _both(_inputs(T2, E2, 1024, 512, k2, seed=6), T2, k2)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all() and (a[2] == b[2]).all()
    # beyond the 64 MiB array: rejected before anything is enqueued
    big = [dev(np.zeros(s, np.uint16)) for s in [(4096, 2880), (32, 2880), (32,)]]
    with pytest.raises(binding.MoEError, match="scratch"):
        binding.library()
        st = binding.library().moe_forward_noalloc(*[binding._ptr(t) for t in big], *[binding._ptr(big[0])] * 4,
                                                   4096, 2880, 32, 4, 2880, binding._ptr(big[0]), None, None,
                                                   binding._stream(None))
        binding._check(st, "moe_forward_noalloc")
    # and the array still serves a call after the rejection
    a, b = _both(_inputs(T2, E2, 1024, 512, k2, seed=7), T2, k2)
    assert (a[0] == b[0]).all() and (a[1] == b[1]).all()
