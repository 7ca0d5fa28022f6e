"""Forward and backward in one call (lce_xent_fwd_bwd, lce_fused_linear_xent_fwd_bwd, through
the C ABI).

The gradients must be bitwise those of the backward entry points on the same inputs (the
same kernels and products run); the losses are held to the forward's tolerances against
the fp64 oracle (row: per token 1e-4, mean 1e-5 relative; fused: per token 2e-2, mean
1e-3 relative) and, where the same kernels produce them (the fused path with one chunk
or with recomputed logits), must be bitwise those of the forward entry points.
"""
import numpy as np
import pytest

import lce_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import forced_env, to_dev  # noqa: E402

TOK_ABS = 1e-4
MEAN_REL = 1e-5
FUSED_TOK_ABS = 2e-2
FUSED_MEAN_REL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _logits(seed, rows, vocab, dtype, std=2.0):
    f = lce_synth.normal_f32(seed, 9, rows, vocab, std)
    return f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f)


def _bits(t):
    """A device tensor's bytes, for bitwise comparison (NaN patterns included)."""
    return t.contiguous().view(torch.uint8).cpu().numpy()


def _check_loss(got, want, reduction, tok_abs, mean_rel, label):
    got = np.asarray(got, dtype=np.float64).reshape(-1)
    want = np.asarray(want, dtype=np.float64).reshape(-1)
    assert np.array_equal(np.isnan(got), np.isnan(want)), label
    ok = ~np.isnan(want)
    if reduction == "none":
        err = np.abs(got[ok] - want[ok])
        assert err.max(initial=0.0) <= tok_abs, f"{label}: worst {err.max()}"
    elif ok.all():
        assert abs(got[0] - want[0]) <= mean_rel * max(abs(want[0]), 1e-2), f"{label}: {got[0]} vs {want[0]}"


def _like(zd):
    """An empty tensor like zd whose data starts at the same offset modulo 16 bytes."""
    off = (zd.data_ptr() % 16) // zd.element_size()
    buf = torch.empty(zd.numel() + off, dtype=zd.dtype, device=zd.device)
    return buf[off:].view(zd.shape)


def _row_call(zd, td, gd, reduction, env=None, in_place=False):
    with forced_env(**(env or {})):
        if in_place:
            z2 = zd.clone()
            loss, d = lce.xent_fwd_bwd(z2, td, gd, reduction, dlogits=z2)
        else:
            loss, d = lce.xent_fwd_bwd(zd, td, gd, reduction, dlogits=_like(zd))
        ref = lce.xent_bwd(zd, td, gd, reduction, out=_like(zd))
    torch.cuda.synchronize()
    return loss, d, ref


# Every per-lane chunk count of the one-wave kernel (1, 2, 4, 8, 16, 32 chunks of 16
# bytes per lane) in both dtypes, rows longer than 32 KiB (statistics + apply path),
# and ragged row counts.
SHAPES = [(1, 1), (3, 7), (9, 100), (11, 500), (6, 2000), (64, 4096), (13, 4097), (5, 8193),
          (33, 1000), (7, 16384), (4, 20000), (3, 50001)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", SHAPES)
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_row_fwd_bwd(dtype, rows, vocab, reduction):
    z = _logits(rows * 5 + vocab, rows, vocab, dtype)
    t = lce_synth.targets(rows + 11, rows, vocab)
    rng = np.random.default_rng(rows * vocab)
    grad = np.float32(1.3) if reduction == "mean" else rng.normal(size=rows).astype(np.float32)
    zd = to_dev(z)
    td = torch.from_numpy(t).cuda()
    gd = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    loss, d, ref = _row_call(zd, td, gd, reduction)
    assert np.array_equal(_bits(d), _bits(ref)), f"{dtype} {rows}x{vocab} {reduction}: dlogits"
    want = oracle.xent(z, t, reduction, dtype=dtype)
    _check_loss(loss.cpu().numpy(), want, reduction, TOK_ABS, MEAN_REL,
                f"{dtype} {rows}x{vocab} {reduction}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("vocab", [37, 1001, 4099])
def test_row_fwd_bwd_unaligned_rows_and_edge_targets(dtype, reduction, vocab):
    """Rows that start off a 16-byte boundary (scalar head and tail elements), with targets
    in the head, the tail and the body, and invalid targets (NaN losses and rows)."""
    rows = 24
    z = _logits(vocab + 3, rows * vocab + 1, 1, dtype).reshape(-1)
    zd = to_dev(z)[1:].view(rows, vocab)  # one element in: no row is 16-byte aligned
    zrows = z[1:].reshape(rows, vocab)
    t = lce_synth.targets(vocab + 4, rows, vocab)
    t[0], t[1], t[2], t[3] = 0, vocab - 1, 1, vocab - 2
    if reduction == "none":
        t[4], t[5] = -1, vocab
    td = torch.from_numpy(t).cuda()
    grad = np.float32(0.7) if reduction == "mean" else np.linspace(-2, 2, rows).astype(np.float32)
    gd = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    loss, d, ref = _row_call(zd, td, gd, reduction)
    assert np.array_equal(_bits(d), _bits(ref))
    want = oracle.xent(np.ascontiguousarray(zrows), t, reduction, dtype=dtype)
    _check_loss(loss.cpu().numpy(), want, reduction, TOK_ABS, MEAN_REL, f"unaligned {dtype} {vocab}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_row_fwd_bwd_invalid_target_mean_is_nan(dtype, reduction):
    rows, vocab = 40, 3000
    z = _logits(17, rows, vocab, dtype)
    t = lce_synth.targets(18, rows, vocab)
    t[7] = -1
    t[33] = vocab
    zd, td = to_dev(z), torch.from_numpy(t).cuda()
    gd = torch.ones(1 if reduction == "mean" else rows, device="cuda")
    loss, d, ref = _row_call(zd, td, gd, reduction)
    assert np.array_equal(_bits(d), _bits(ref))
    got = loss.cpu().numpy()
    if reduction == "mean":
        assert np.isnan(got[0])
    else:
        assert np.isnan(got[[7, 33]]).all() and not np.isnan(np.delete(got, [7, 33])).any()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("rows,vocab", [(5, 3000), (300, 4096), (6, 70001)])
def test_row_fwd_bwd_apply_path(dtype, reduction, rows, vocab):
    """Rows forced through the statistics + apply path: the losses come from the
    statistics pass (merged as one shard)."""
    z = _logits(rows + 2 * vocab, rows, vocab, dtype)
    t = lce_synth.targets(rows + 5, rows, vocab)
    zd, td = to_dev(z), torch.from_numpy(t).cuda()
    gd = torch.full((1 if reduction == "mean" else rows,), 0.5, device="cuda")
    loss, d, ref = _row_call(zd, td, gd, reduction, env={"LCE_BWD_PATH": "apply"})
    assert np.array_equal(_bits(d), _bits(ref))
    want = oracle.xent(z, t, reduction, dtype=dtype)
    _check_loss(loss.cpu().numpy(), want, reduction, TOK_ABS, MEAN_REL, f"apply {dtype} {rows}x{vocab}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_row_fwd_bwd_in_place(dtype):
    rows, vocab = 96, 8000
    z = _logits(23, rows, vocab, dtype)
    t = lce_synth.targets(24, rows, vocab)
    zd, td = to_dev(z), torch.from_numpy(t).cuda()
    gd = torch.ones(1, device="cuda")
    loss, d, ref = _row_call(zd, td, gd, "mean", in_place=True)
    assert np.array_equal(_bits(d), _bits(ref))
    _check_loss(loss.cpu().numpy(), oracle.xent(z, t, "mean", dtype=dtype), "mean", TOK_ABS, MEAN_REL,
                "in place")


def test_row_fwd_bwd_empty():
    z = torch.empty(0, 16, device="cuda")
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    loss, d = lce.xent_fwd_bwd(z, t, torch.ones(1, device="cuda"), "mean")
    torch.cuda.synchronize()
    assert np.isnan(loss.item()) and d.numel() == 0
    loss, _ = lce.xent_fwd_bwd(z, t, torch.ones(0, device="cuda"), "none")
    assert loss.numel() == 0


@pytest.mark.parametrize("name", ["megatron_bf16_2048x4x4096_none", "ce_f32_16384x4096_mean"])
def test_row_fwd_bwd_full_size(name):
    """The benchmark workloads' shapes: every gradient element bitwise against the backward
    call, every loss (or the mean) against the oracle."""
    w = lce_synth.WORKLOADS[name]
    z, t = w.logits(), w.target()
    zd, td = to_dev(z), torch.from_numpy(t).cuda()
    n = t.size
    gd = (torch.ones(1, device="cuda") if w.reduction == "mean"
          else torch.linspace(0.5, 1.5, n, device="cuda").reshape(t.shape))
    loss, d, ref = _row_call(zd, td, gd, w.reduction)
    assert torch.equal(d.view(torch.int16) if d.dtype == torch.bfloat16 else d.view(torch.int32),
                       ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))
    want = oracle.xent(z, t, w.reduction, dtype=w.dtype)
    _check_loss(loss.cpu().numpy(), want, w.reduction, TOK_ABS, MEAN_REL, name)


# ------------------------------------------------------------------ fused projection

def _fused_inputs(seed, tokens, hidden, vocab, w_std=0.1):
    xb = lce_synth.normal_bf16_bits(seed, 0, tokens, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(seed + 1, 2, vocab, hidden, w_std)
    t = lce_synth.targets(seed + 2, tokens, vocab)
    return xb, wb, t


def _fused_calls(xb, wb, t, reduction, grad, env=None):
    x, W, td = to_dev(xb), to_dev(wb), torch.from_numpy(t).cuda()
    g = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    with forced_env(**(env or {})):
        loss, dx, dw = lce.fused_linear_xent_fwd_bwd(x, W, td, g, reduction)
        ref_dx, ref_dw = lce.fused_linear_xent_bwd(x, W, td, g, reduction)
    fwd = lce.fused_linear_xent(x, W, td, reduction)
    torch.cuda.synchronize()
    return loss, dx, dw, ref_dx, ref_dw, fwd


@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("tokens,hidden,vocab", [(300, 64, 1000), (256, 128, 777), (37, 64, 2000),
                                                 (513, 96, 300)])
def test_fused_fwd_bwd_one_chunk(reduction, tokens, hidden, vocab):
    xb, wb, t = _fused_inputs(tokens + vocab, tokens, hidden, vocab)
    grad = np.float32(1.0) if reduction == "mean" else np.linspace(-1, 1, tokens).astype(np.float32)
    loss, dx, dw, ref_dx, ref_dw, fwd = _fused_calls(xb, wb, t, reduction, grad)
    assert torch.equal(dx, ref_dx) and torch.equal(dw, ref_dw)
    assert np.array_equal(_bits(loss), _bits(fwd)), "losses differ from the forward call's"
    want = oracle.fused_linear_xent(xb, wb, t, reduction)
    _check_loss(loss.cpu().numpy(), want, reduction, FUSED_TOK_ABS, FUSED_MEAN_REL, "fused")


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_fused_fwd_bwd_several_chunks(reduction):
    """Stored logits in chunks of 256 tokens (3 chunks, the last ragged): per-chunk losses,
    and for the mean the fixed-order mean of the per-token losses."""
    tokens, hidden, vocab = 600, 64, 1000
    ld = (vocab + 255) // 256 * 256
    env = {"LCE_FUSED_BWD_STORE_BYTES": 256 * ld * 6}
    xb, wb, t = _fused_inputs(41, tokens, hidden, vocab)
    grad = np.float32(2.0) if reduction == "mean" else np.linspace(0.5, 1.5, tokens).astype(np.float32)
    loss, dx, dw, ref_dx, ref_dw, fwd = _fused_calls(xb, wb, t, reduction, grad, env=env)
    assert torch.equal(dx, ref_dx) and torch.equal(dw, ref_dw)
    want = oracle.fused_linear_xent(xb, wb, t, reduction)
    _check_loss(loss.cpu().numpy(), want, reduction, FUSED_TOK_ABS, FUSED_MEAN_REL, "chunks")
    _check_loss(loss.cpu().numpy(), fwd.cpu().numpy(), reduction, FUSED_TOK_ABS, FUSED_MEAN_REL,
                "chunks vs forward")
    # the chunks' launches really ran: the mean came from the per-token mean kernel
    if reduction == "mean":
        with forced_env(**env):
            lce.fused_linear_xent_fwd_bwd(to_dev(xb), to_dev(wb), torch.from_numpy(t).cuda(),
                                          torch.ones(1, device="cuda"), "mean")
        assert "mean of the chunks' losses" in lce.lce_last_launch()


@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_fused_fwd_bwd_recompute_path(reduction):
    tokens, hidden, vocab = 400, 128, 1500
    xb, wb, t = _fused_inputs(57, tokens, hidden, vocab)
    t[3] = -1
    grad = np.float32(1.0) if reduction == "mean" else np.ones(tokens, np.float32)
    loss, dx, dw, ref_dx, ref_dw, fwd = _fused_calls(xb, wb, t, reduction, grad,
                                                     env={"LCE_FUSED_BWD_STORE_BYTES": 0})
    assert np.array_equal(_bits(dx), _bits(ref_dx)) and np.array_equal(_bits(dw), _bits(ref_dw))
    assert np.array_equal(_bits(loss), _bits(fwd))
    got = loss.cpu().numpy()
    if reduction == "mean":
        assert np.isnan(got[0])
    else:
        assert np.isnan(got[3]) and not np.isnan(np.delete(got, 3)).any()


def test_fused_fwd_bwd_empty():
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    W = torch.ones(100, 64, dtype=torch.bfloat16, device="cuda")
    t = torch.empty(0, dtype=torch.int64, device="cuda")
    loss, dx, dw = lce.fused_linear_xent_fwd_bwd(x, W, t, torch.ones(1, device="cuda"), "mean")
    torch.cuda.synchronize()
    assert np.isnan(loss.item()) and dx.numel() == 0 and bool((dw == 0).all())


def test_fused_fwd_bwd_page_shape():
    """tokens 2048, hidden 4096, vocab 128256, mean: one chunk of stored logits; the loss is
    bitwise the forward call's, dx and dweight bitwise the backward call's."""
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    xb, wb, t = w.x(), w.weight(), w.target()
    print("\n[fwd_bwd] page shape", flush=True)
    loss, dx, dw, ref_dx, ref_dw, fwd = _fused_calls(xb, wb, t, "mean", np.float32(1.0))
    assert torch.equal(dx, ref_dx) and torch.equal(dw, ref_dw)
    assert np.array_equal(_bits(loss), _bits(fwd))
    del dx, dw, ref_dx, ref_dw
    torch.cuda.empty_cache()
