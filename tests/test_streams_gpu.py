"""liblce calls on several streams and from several host threads at once.

Each (device, stream) pair has its own scratch buffer, and the host side keeps its
tables (scratch buffers, GEMM plans and the hipBLASLt handle) under a mutex: calls issued
concurrently from different threads onto different streams (row and fused cross-entropy,
the fused backward with its library GEMMs, the forward and backward in one call, fused
linear + JSD) must give the same results as the same calls made one after the other.
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
        out.append(("xent_fwd_bwd", (z, t)))
        zs = to_dev(lce_synth.f32_to_bf16_bits(lce_synth.normal_f32(350 + k, 0, 1500 + 77 * k, 512, 1.5)))
        ts = torch.from_numpy(lce_synth.targets(450 + k, zs.shape[0], 512)).cuda()
        out.append(("xent_fwd_bwd", (zs, ts)))  # short rows: several per wave
        x = to_dev(lce_synth.normal_bf16_bits(500 + k, 0, 300 + 31 * k, 128, 1.0))
        w = to_dev(lce_synth.normal_bf16_bits(600 + k, 2, 2000 + 111 * k, 128, 0.1))
        tt = torch.from_numpy(lce_synth.targets(700 + k, x.shape[0], w.shape[0])).cuda()
        out.append(("fused", (x, w, tt)))
        out.append(("fused_bwd", (x, w, tt)))
        out.append(("fused_fwd_bwd", (x, w, tt)))
        x2 = to_dev(lce_synth.normal_bf16_bits(800 + k, 0, x.shape[0], 128, 1.0))
        w2 = to_dev(lce_synth.normal_bf16_bits(900 + k, 2, w.shape[0], 128, 0.1))
        out.append(("jsd", (x, w, x2, w2)))
    return out


def _call(kind, args):
    if kind == "xent":
        z, t = args
        return torch.cat([lce.xent(z, t, "mean"), lce.xent(z, t, "none")])
    if kind == "xent_fwd_bwd":
        z, t = args
        g = torch.full((1,), 0.5, device="cuda")
        loss, d = lce.xent_fwd_bwd(z, t, g, "mean")
        lt, _ = lce.xent_fwd_bwd(z, t, torch.ones(t.shape, device="cuda"), "none")
        return torch.cat([loss, lt, d.float().reshape(-1)])
    if kind == "jsd":
        x, w, x2, w2 = args
        return torch.cat([lce.fused_linear_jsd(x, w, x2, w2, 0.3, "mean"),
                          lce.fused_linear_jsd(x, w, x2, w2, 0.5, "none")])
    x, w, t = args
    if kind == "fused_bwd":
        g = torch.full((1,), 0.7, device="cuda")
        dx, dw = lce.fused_linear_xent_bwd(x, w, t, g, "mean")
        return torch.cat([dx.reshape(-1), dw.reshape(-1)])
    if kind == "fused_fwd_bwd":
        g = torch.full((1,), 0.7, device="cuda")
        loss, dx, dw = lce.fused_linear_xent_fwd_bwd(x, w, t, g, "mean")
        return torch.cat([loss, dx.reshape(-1), dw.reshape(-1)])
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



_OOM_SCRIPT = r"""
import json, os, sys
sys.path.insert(0, sys.argv[1])
import numpy as np, torch
import lce_synth, oracle
import vocab_cross_entropy_row_amd as lce
rows, vocab = 64, 1000
f = lce_synth.normal_f32(31, 0, rows, vocab, 1.0)
tn = lce_synth.targets(32, rows, vocab)
z = torch.from_numpy(f).cuda()
t = torch.from_numpy(tn).cuda()
out = torch.full((1,), 123.0, device="cuda")
s = torch.cuda.current_stream().cuda_stream
torch.cuda.synchronize()
os.environ["LCE_TEST_FAIL_ALLOC"] = "1"
st1 = lce.lce_xent_fwd(z.data_ptr(), lce.LCE_F32, rows, vocab, t.data_ptr(),
                       lce.LCE_REDUCTION_MEAN, out.data_ptr(), s)
msg = lce.lce_last_error()
torch.cuda.synchronize()
canary = out.item()
del os.environ["LCE_TEST_FAIL_ALLOC"]
st2 = lce.lce_xent_fwd(z.data_ptr(), lce.LCE_F32, rows, vocab, t.data_ptr(),
                       lce.LCE_REDUCTION_MEAN, out.data_ptr(), s)
torch.cuda.synchronize()
want = oracle.mean(oracle.xent_rows(f, tn, dtype="f32"))
print(json.dumps({"st1": st1, "msg": msg, "canary": canary, "st2": st2,
                  "got": out.item(), "want": want}))
"""


def test_refused_scratch_allocation_reports_oom():
    """Scratch is kept per (device, stream) and grows on first use.  When that growth is
    refused (the LCE_TEST_FAIL_ALLOC hook, standing in for a failed hipMalloc) the call
    returns LCE_ERR_OOM with a message and enqueues nothing (the output keeps its canary);
    the same call succeeds once allocation is allowed again.  Runs in a child process,
    where liblce has no scratch yet on any stream."""
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = {k: v for k, v in os.environ.items() if k != "LCE_TEST_FAIL_ALLOC"}
    r = subprocess.run([sys.executable, "-c", _OOM_SCRIPT, root], capture_output=True,
                       text=True, timeout=180, env=env)
    assert r.returncode == 0, r.stderr[-2000:]
    d = json.loads(r.stdout.strip().splitlines()[-1])
    assert d["st1"] == lce.LCE_ERR_OOM, d
    assert "LCE_TEST_FAIL_ALLOC" in d["msg"], d
    assert d["canary"] == 123.0, d
    assert d["st2"] == lce.LCE_OK, d
    assert abs(d["got"] - d["want"]) <= 1e-5 * abs(d["want"]), d


def test_mean_after_fused_backward_on_one_stream():
    """The deterministic mean hands each workgroup's partial to the finishing workgroup through
    tagged 64-bit slots, which must never hold another call's data.  They live in a buffer
    that only the mean reductions write: a fused backward (which fills this stream's scratch
    with fp32 logits, the bf16 logit gradient and GEMM workspace) followed, on the same
    stream, by large-grid means of every mean-reducing entry point must give the mean of the
    same call's per-token values, on every repetition."""
    s = torch.cuda.Stream()
    x = to_dev(lce_synth.normal_bf16_bits(41, 0, 777, 256, 1.0))
    w = to_dev(lce_synth.normal_bf16_bits(42, 2, 9000, 256, 0.1))
    t = torch.from_numpy(lce_synth.targets(43, 777, 9000)).cuda()
    rows, vocab = 300_001, 64  # 18751 workgroups of 16 rows: the mean reads 18751 slots
    z = to_dev(lce_synth.f32_to_bf16_bits(lce_synth.normal_f32(44, 0, rows, vocab, 2.0)))
    tz = torch.from_numpy(lce_synth.targets(45, rows, vocab)).cuda()
    x2 = to_dev(lce_synth.normal_bf16_bits(46, 0, 777, 256, 1.0))
    w2 = to_dev(lce_synth.normal_bf16_bits(47, 2, 9000, 256, 0.1))
    with torch.cuda.stream(s):
        per_row = lce.xent(z, tz, "none").double()
        per_fused = lce.fused_linear_xent(x, w, t, "none").double()
        per_jsd = lce.fused_linear_jsd(x, w, x2, w2, 0.5, "none").double()
        for rep in range(4):
            g = torch.full((1,), 1.0 + rep, device="cuda")
            lce.fused_linear_xent_bwd(x, w, t, g, "mean")
            means = [lce.xent(z, tz, "mean"), lce.fused_linear_xent(x, w, t, "mean"),
                     lce.fused_linear_jsd(x, w, x2, w2, 0.5, "mean")]
            s.synchronize()
            for name, m, per in zip(("row", "fused", "jsd"), means, (per_row, per_fused, per_jsd)):
                want = per.mean().item()
                assert abs(m.item() - want) <= 1e-5 * abs(want), (rep, name, m.item(), want)
