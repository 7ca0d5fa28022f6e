"""liblce calls recorded into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The benchmark times graph replays, so replays must give the eager results bit for
bit: every kernel path (one wave per row, one workgroup per row, split rows, the
fused projection, fused linear + JSD with stored logits, in chunks, and recomputed,
and the forward and backward in one call, row and fused, in chunks and not)
with and without the deterministic mean, whose epoch word each replay must advance so
that the next one tells its partials from those left by earlier launches.  Between replays the program does eager
work of its own (other liblce calls on the same stream, torch kernels, host
synchronisations), and each replay first finds its outputs overwritten with NaN.
"""
import numpy as np
import pytest

import lce_synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import forced_env, to_dev  # noqa: E402

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _row_case(seed, rows, vocab, dtype, reduction, env):
    f = lce_synth.normal_f32(seed, 9, rows, vocab, 1.5)
    z = to_dev(f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f))
    t = torch.from_numpy(lce_synth.targets(seed + 1, rows, vocab)).cuda()
    out = torch.empty((1,) if reduction == "mean" else (rows,), dtype=torch.float32, device="cuda")

    def call():
        with forced_env(**env):
            lce.xent(z, t, reduction, out=out)
    return call, out


def _fused_case(seed, tokens, hidden, vocab, reduction, env):
    x = to_dev(lce_synth.normal_bf16_bits(seed, 0, tokens, hidden, 1.0))
    W = to_dev(lce_synth.normal_bf16_bits(seed + 1, 2, vocab, hidden, 0.1))
    t = torch.from_numpy(lce_synth.targets(seed + 2, tokens, vocab)).cuda()
    out = torch.empty((1,) if reduction == "mean" else (tokens,), dtype=torch.float32, device="cuda")

    def call():
        with forced_env(**env):
            lce.fused_linear_xent(x, W, t, reduction, out=out)
    return call, out


def _jsd_case(seed, tokens, hidden, vocab, reduction, env):
    xs, xt = (to_dev(lce_synth.normal_bf16_bits(seed + k, 0, tokens, hidden, 1.0)) for k in (0, 1))
    ws, wt = (to_dev(lce_synth.normal_bf16_bits(seed + k, 2, vocab, hidden, 0.1)) for k in (2, 3))
    out = torch.empty((1,) if reduction == "mean" else (tokens,), dtype=torch.float32, device="cuda")

    def call():
        with forced_env(**env):
            lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, reduction, out=out)
    return call, out


def _row_fwd_bwd_case(seed, rows, vocab, dtype, reduction, env):
    f = lce_synth.normal_f32(seed, 9, rows, vocab, 1.5)
    z = to_dev(f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f))
    t = torch.from_numpy(lce_synth.targets(seed + 1, rows, vocab)).cuda()
    g = torch.full((1,) if reduction == "mean" else (rows,), 0.75, device="cuda")
    out = torch.empty((1,) if reduction == "mean" else (rows,), dtype=torch.float32, device="cuda")
    d = torch.empty_like(z)

    def call():
        with forced_env(**env):
            lce.xent_fwd_bwd(z, t, g, reduction, out=out, dlogits=d)
    return call, (out, d)


def _fused_fwd_bwd_case(seed, tokens, hidden, vocab, reduction, env):
    x = to_dev(lce_synth.normal_bf16_bits(seed, 0, tokens, hidden, 1.0))
    W = to_dev(lce_synth.normal_bf16_bits(seed + 1, 2, vocab, hidden, 0.1))
    t = torch.from_numpy(lce_synth.targets(seed + 2, tokens, vocab)).cuda()
    g = torch.ones((1,) if reduction == "mean" else (tokens,), device="cuda")
    out = torch.empty((1,) if reduction == "mean" else (tokens,), dtype=torch.float32, device="cuda")
    dx = torch.empty((tokens, hidden), dtype=torch.float32, device="cuda")
    dw = torch.empty((vocab, hidden), dtype=torch.float32, device="cuda")

    def call():
        with forced_env(**env):
            lce.fused_linear_xent_fwd_bwd(x, W, t, g, reduction, out=out, dx=dx, dweight=dw)
    return call, (out, dx, dw)


def _cases():
    return [
        _row_fwd_bwd_case(114, 1000, 4096, "bf16", "mean", {}),
        _row_fwd_bwd_case(115, 333, 1001, "f32", "none", {}),
        _row_fwd_bwd_case(116, 200, 9000, "f32", "mean", {"LCE_BWD_PATH": "apply"}),
        _fused_fwd_bwd_case(117, 300, 64, 1000, "mean", {}),
        _fused_fwd_bwd_case(118, 600, 64, 1000, "mean", {"LCE_FUSED_BWD_STORE_BYTES": 256 * 1024 * 6}),
        _jsd_case(109, 300, 128, 2000, "mean", {}),
        _jsd_case(110, 520, 64, 1001, "none", {"LCE_JSD_STORE_BYTES": 256 * 1024 * 8}),
        _jsd_case(111, 200, 128, 1500, "mean", {"LCE_JSD_STORE_BYTES": 0}),
        _row_case(101, 1000, 3000, "bf16", "mean", {"LCE_PATH": "wave"}),
        _row_case(102, 777, 4099, "f32", "none", {"LCE_PATH": "wave"}),
        _row_case(103, 600, 20000, "f32", "mean", {"LCE_PATH": "block"}),
        _row_case(104, 300, 9001, "bf16", "none", {"LCE_PATH": "block"}),
        _row_case(105, 40, 70001, "f32", "mean", {"LCE_PATH": "split"}),
        _row_case(106, 23, 50000, "bf16", "none", {"LCE_PATH": "split"}),
        _row_case(112, 300, 70001, "f32", "mean", {"LCE_PATH": "split", "LCE_SPLITS": 9}),
        _row_case(113, 256, 131072, "f32", "mean", {}),
        _fused_case(107, 300, 128, 3000, "mean", {}),
        _fused_case(108, 130, 256, 1500, "none", {"LCE_FUSED_SEGMENTS": 3}),
    ]


def _replay_and_check(g, s, outs, refs, between):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        between(r)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        torch.cuda.synchronize()
        for i, (o, ref) in enumerate(zip(outs, refs)):
            assert torch.equal(o, ref), f"replay {r}, case {i}"


def test_graph_replays_match_eager():
    cases = _cases()
    calls = [c for c, _ in cases]
    outs = [o for _, os_ in cases for o in (os_ if isinstance(os_, tuple) else (os_,))]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in calls:  # eager reference; also grows this stream's scratch before capture
            c()
    torch.cuda.synchronize()
    refs = [o.clone() for o in outs]

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            c()
    torch.cuda.synchronize()

    other, other_out = _row_case(109, 5000, 1024, "f32", "mean", {"LCE_PATH": "wave"})

    def between(r):
        # eager liblce work on the capture stream (shares its scratch and mean state) and
        # on the default stream, plus torch kernels
        with torch.cuda.stream(s):
            other()
            calls[r % len(calls)]()
        other()
        torch.cuda.synchronize()
        assert torch.isfinite(other_out).all()
        _ = torch.randn(1 << 20, device="cuda").sum().item()

    _replay_and_check(g, s, outs, refs, between)


def test_graph_survives_scratch_growth():
    """A call captured while the stream's scratch was small still replays correctly
    after a later eager call has grown (and so replaced) that scratch."""
    s = torch.cuda.Stream()
    small, small_out = _row_case(111, 2000, 512, "bf16", "mean", {"LCE_PATH": "wave"})
    with torch.cuda.stream(s):
        small()
    torch.cuda.synchronize()
    ref = small_out.clone()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        small()
    torch.cuda.synchronize()

    # 32 segments x 8192 tokens x 8 bytes of partials: far beyond the first buffer
    big, big_out = _fused_case(112, 8192, 64, 8192, "mean", {"LCE_FUSED_SEGMENTS": 32})
    with torch.cuda.stream(s):
        big()
    torch.cuda.synchronize()
    big_ref = big_out.clone()

    def between(r):
        with torch.cuda.stream(s):
            big()
        torch.cuda.synchronize()
        assert torch.equal(big_out, big_ref)

    _replay_and_check(g, s, [small_out], [ref], between)


@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")  # the refused call enqueued nothing
def test_capture_refuses_scratch_growth():
    """A first call on a stream inside a capture cannot allocate: it fails cleanly,
    with nothing enqueued, and the library keeps working afterwards."""
    s = torch.cuda.Stream()
    # 8 MiB of partials: more than any earlier call grew any stream's scratch to
    # (torch hands out streams from a pool, so this one may have been used before)
    call, out = _fused_case(113, 32768, 64, 8192, "mean", {"LCE_FUSED_SEGMENTS": 32})
    g = torch.cuda.CUDAGraph()
    with pytest.raises(lce.LceError) as err:
        with torch.cuda.graph(g, stream=s):
            call()
    assert err.value.status == 2  # LCE_ERR_UNSUPPORTED
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        call()
    torch.cuda.synchronize()
    assert np.isfinite(out.item())
