"""The two measurement aids on the GPU: the streaming read returns the XOR of
exactly the bytes it was given, and the matrix-core rate probe runs, is
deterministic, and reports a rate below the published bf16 dense peak."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bit_quantized_moe_expert_amd as M  # noqa: E402

DEV = "cuda"


@pytest.mark.parametrize("nbytes,loads", [(16 * 256 * 4, 4), (16 * 1000 + 16 * 256, 1), (1 << 20, 16)])
def test_stream_read_xor(nbytes, loads):
    rng = np.random.default_rng(nbytes + loads)
    host = rng.integers(0, 1 << 32, nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(DEV)
    words = M.stream_read_sink_words(nbytes, loads)
    sink = torch.zeros(words, dtype=torch.int32, device=DEV)
    M.stream_read(buf, nbytes, sink, loads)
    torch.cuda.synchronize()
    # workgroup w reads 16-byte words [w * 256 * loads, (w + 1) * 256 * loads),
    # the last clamped to the end (a repeated word cancels in pairs only if read
    # twice by the same workgroup; the expected value repeats the same clamp)
    n16 = nbytes // 16
    v = host.reshape(n16, 4)
    want = []
    for w in range(words):
        idx = np.minimum(np.arange(w * 256 * loads, (w + 1) * 256 * loads), n16 - 1)
        want.append(np.bitwise_xor.reduce(v[idx].ravel()))
    assert np.array_equal(sink.cpu().numpy().view(np.uint32), np.array(want, np.uint32))


def test_mfma_peak_runs_and_is_deterministic():
    wg, iters = 64, 256
    a = torch.empty(wg * 512, dtype=torch.float32, device=DEV)
    b = torch.empty_like(a)
    flops = M.mfma_peak(wg, iters, a)
    M.mfma_peak(wg, iters, b)
    torch.cuda.synchronize()
    assert flops == wg * 8 * iters * 8 * 2 * 32 * 32 * 16
    assert torch.isfinite(a).all() and torch.equal(a, b)
    assert (a != 0).any()
    # full chip: the sustained rate is positive and under the published peak
    wg, iters = 256 * 4, 2048
    s = torch.empty(wg * 512, dtype=torch.float32, device=DEV)
    M.mfma_peak(wg, 64, s)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    flops = M.mfma_peak(wg, iters, s)
    e1.record()
    torch.cuda.synchronize()
    tflops = flops / (e0.elapsed_time(e1) * 1e-3) / 1e12
    assert 50.0 < tflops < 2500.0 * 1.02, tflops
