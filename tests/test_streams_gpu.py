"""liblce calls on several streams and from several host threads at once.

Each (device, stream) pair has its own scratch buffer, and the host side keeps its
tables (scratch buffers, GEMM plans and the hipBLASLt handle) under a mutex: calls issued
concurrently from different threads onto different streams (row and fused cross-entropy,
the fused backward with its library GEMMs, fused linear + JSD) must give the same results
as the same calls made one after the other.
"""
import threading

import numpy as np
import pytest

import lce_synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _cases():
    out = []
    for k in range(4):
        z = to_dev(lce_synth.f32_to_bf16_bits(lce_synth.normal_f32(300 + k, 0, 700 + 97 * k, 3001, 1.5)))
        t = torch.from_numpy(lce_synth.targets(400 + k, z.shape[0], 3001)).cuda()
        out.append(("xent", (z, t)))
        x = to_dev(lce_synth.normal_bf16_bits(500 + k, 0, 300 + 31 * k, 128, 1.0))
        w = to_dev(lce_synth.normal_bf16_bits(600 + k, 2, 2000 + 111 * k, 128, 0.1))
        tt = torch.from_numpy(lce_synth.targets(700 + k, x.shape[0], w.shape[0])).cuda()
        out.append(("fused", (x, w, tt)))
        out.append(("fused_bwd", (x, w, tt)))
        x2 = to_dev(lce_synth.normal_bf16_bits(800 + k, 0, x.shape[0], 128, 1.0))
        w2 = to_dev(lce_synth.normal_bf16_bits(900 + k, 2, w.shape[0], 128, 0.1))
        out.append(("jsd", (x, w, x2, w2)))
    return out


def _call(kind, args):
    if kind == "xent":
        z, t = args
        return torch.cat([lce.xent(z, t, "mean"), lce.xent(z, t, "none")])
    if kind == "jsd":
        x, w, x2, w2 = args
        return torch.cat([lce.fused_linear_jsd(x, w, x2, w2, 0.3, "mean"),
                          lce.fused_linear_jsd(x, w, x2, w2, 0.5, "none")])
    x, w, t = args
    if kind == "fused_bwd":
        g = torch.full((1,), 0.7, device="cuda")
        dx, dw = lce.fused_linear_xent_bwd(x, w, t, g, "mean")
        return torch.cat([dx.reshape(-1), dw.reshape(-1)])
    return torch.cat([lce.fused_linear_xent(x, w, t, "mean"), lce.fused_linear_xent(x, w, t, "none")])


def test_concurrent_threads_and_streams_match_sequential():
    cases = _cases()
    ref = [_call(k, a).clone() for k, a in cases]
    torch.cuda.synchronize()
    got = [None] * len(cases)
    errors = []

    def worker(i):
        try:
            s = torch.cuda.Stream()
            with torch.cuda.stream(s):
                for _ in range(3):
                    got[i] = _call(*cases[i])
            s.synchronize()
        except Exception as e:  # reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(i,)) for i in range(len(cases))]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for i, (r, g) in enumerate(zip(ref, got)):
        assert torch.equal(r, g), f"case {i} ({cases[i][0]})"
