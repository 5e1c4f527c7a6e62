"""The measurement probes on the GPU: their outputs are exact checks of what
they computed (the MFMA probe's all-ones sums, the read probe's XOR of the
buffer), so a probe that skipped work or read the wrong bytes fails here."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from moe_layer_route_amd import binding  # noqa: E402

pytestmark = pytest.mark.gpu


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


@pytest.mark.parametrize("iters,wg", [(1, 1), (37, 5), (8191, 3)])
def test_mfma_probe_sums(iters, wg):
    _need_gpu()
    out = binding.probe_mfma_bf16(iters, wg)
    torch.cuda.synchronize()
    assert (out.cpu().numpy() == np.float32(2048 * iters)).all()


@pytest.mark.parametrize("nbytes,wg", [(0, 2), (16, 1), (4096 + 48, 3), ((1 << 20) + 16 * 13, 7), (1 << 24, 64)])
def test_read_probe_xor(nbytes, wg):
    _need_gpu()
    words = np.random.default_rng(nbytes).integers(0, 1 << 32, nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32).copy()).cuda()
    out = binding.probe_read(buf, wg)
    torch.cuda.synchronize()
    # every 16-byte piece read exactly once: the folds XOR to the buffer's XOR (0 when empty)
    assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(words)
