"""Every weight format and expert path captured in a HIP graph: each replay,
after eager work that poisons y and the workspace, reproduces the eager
result bit for bit (the verify passes replay one captured step with static
buffers).  Needs an MI355X; every call goes through the C ABI."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding, datagen as d  # noqa: E402
from checks import bf16_bits, dev  # noqa: E402

pytestmark = pytest.mark.gpu

# T*k/E = 48 is the switch between the paths; both are forced below
T, E, H, I, K = 96, 8, 256, 160, 4


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _cfg():
    return d.small_config(T=T, E=E, H=H, I=I, k=K, x_scale=d.scale_for_hidden(H))


def _tensor(a):
    return dev(a) if a.dtype == np.uint16 else torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _forward_fn(fmt, path, y, ws):
    cfg = _cfg()
    x, Wr, br = d.make_activations(cfg, 7), *d.make_router(cfg, 7)
    if fmt == "bf16":
        Wgu, bgu, Wd, bd = d.make_experts(cfg, 7, 4)
        args = [_tensor(a) for a in (x, Wr, br, Wgu, bgu, Wd, bd)]
        return lambda: binding.moe_forward(*args, k=K, y=y, workspace=ws, path=path)
    if fmt == "mxfp4":
        args = [_tensor(a) for a in (x, Wr, br, *d.make_experts_mxfp4(cfg, 7, threads=4))]
        return lambda: binding.moe_forward_mxfp4(*args, k=K, y=y, workspace=ws, path=path)
    args = [_tensor(a) for a in (x, Wr, br, *d.make_experts_fp8(cfg, 7, threads=4))]
    return lambda: binding.moe_forward_fp8(*args, k=K, y=y, workspace=ws, path=path)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "fp8"])
def test_graph_replays_match_eager(fmt, path):
    _need_gpu()
    ws = (binding.alloc_workspace_fp8 if fmt == "fp8" else binding.alloc_workspace)(T, H, E, K, I)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    fwd = _forward_fn(fmt, path, y, ws)
    fwd()
    torch.cuda.synchronize()
    eager = bf16_bits(y).copy()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for i in range(4):
        y.view(torch.int16).fill_(-1)
        ws.fill_(0xAB if i % 2 else 0x11)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert (bf16_bits(y) == eager).all(), f"{fmt} {path}: replay {i} differs from the eager result"
