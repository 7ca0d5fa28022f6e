"""Gradient of the row cross-entropy (lce_xent_bwd, through the C ABI) against the fp64
oracle's softmax-minus-one-hot.

Tolerances: softmax values are at most 1, and the kernel forms each as
2^(fma(z, log2e, -M)) times a row constant in fp32, so fp32 gradients must be within
2e-6 * |g_i| of the oracle (g_i the row's output gradient); bf16 gradients are that fp32
value rounded to nearest even, so within one bf16 rounding (2^-8 relative) more.
"""
import numpy as np
import pytest

import lce_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import forced_env, to_dev  # noqa: E402

ABS_PER_G = 2e-6
BF16_REL = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _logits(seed, rows, vocab, dtype, std=2.0, shift=0.0):
    f = lce_synth.normal_f32(seed, 9, rows, vocab, std)
    if shift:
        f = (np.round(f * 64) / 64 + np.float32(shift)).astype(np.float32)
    return f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f)


def _to_host(d, dtype):
    if dtype == "f32":
        return d.cpu().numpy().astype(np.float64)
    return oracle.bf16_bits_to_f64(d.view(torch.int16).cpu().numpy().view(np.uint16))


def _check(got, want, gscale, dtype, label):
    assert np.array_equal(np.isnan(got), np.isnan(want)), label
    ok = ~np.isnan(want)
    tol = ABS_PER_G * np.abs(gscale) + (BF16_REL * np.abs(want) if dtype == "bf16" else 0.0)
    err = np.where(ok, np.abs(got - want) - tol, 0.0)
    assert err.max(initial=-1.0) <= 0.0, f"{label}: worst excess {err.max()}"


def _run(z, t, dtype, reduction, grad, env=None, in_place=False):
    zd = to_dev(z)
    td = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int64)).cuda()
    gd = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    with forced_env(**(env or {})):
        d = lce.xent_bwd(zd, td, gd, reduction, out=zd if in_place else None)
    torch.cuda.synchronize()
    return _to_host(d, dtype)


# Rows of every per-lane chunk count the one-wave kernel is instantiated for (1, 2, 4, 8,
# 16, 32 chunks of 16 bytes per lane) in both dtypes, and longer rows (two-pass path):
# fp32 vocab 100, 500, 1000, 2000, 4096, 8193 and bf16 vocab 100, 1000, 2000, 4096, 8193,
# 16384 take 1, 2, 4, 8, 16, 32 chunks per lane.
SHAPES = [(1, 1), (3, 7), (17, 64), (9, 100), (11, 500), (6, 2000), (64, 4096), (13, 4097),
          (5, 8193), (33, 1000), (7, 16384), (4, 20000), (3, 50001)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", SHAPES)
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_bwd_matches_oracle(dtype, rows, vocab, reduction):
    z = _logits(rows * 7 + vocab, rows, vocab, dtype)
    t = lce_synth.targets(rows + 3, rows, vocab)
    rng = np.random.default_rng(rows + vocab)
    grad = np.float32(1.7) if reduction == "mean" else rng.normal(size=rows).astype(np.float32)
    got = _run(z, t, dtype, reduction, grad)
    want = oracle.xent_bwd(z, t, np.asarray(grad, dtype=np.float64), reduction, dtype=dtype)
    g = (np.full(rows, float(grad) / rows) if reduction == "mean" else grad.astype(np.float64))
    _check(got, want, g[:, None], dtype, f"{dtype} {rows}x{vocab} {reduction}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(5, 3000), (40, 9000), (3, 70001)])
def test_bwd_two_pass_path(dtype, rows, vocab):
    """Rows that would stay in registers, forced through the statistics + apply path."""
    z = _logits(rows + vocab, rows, vocab, dtype)
    t = lce_synth.targets(rows, rows, vocab)
    grad = np.linspace(-1, 1, rows).astype(np.float32)
    got = _run(z, t, dtype, "none", grad, env={"LCE_BWD_PATH": "apply"})
    want = oracle.xent_bwd(z, t, grad.astype(np.float64), "none", dtype=dtype)
    _check(got, want, grad.astype(np.float64)[:, None], dtype, f"apply {dtype} {rows}x{vocab}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab", [4096, 40000])
def test_bwd_in_place(dtype, vocab):
    rows = 64
    z = _logits(3, rows, vocab, dtype)
    t = lce_synth.targets(4, rows, vocab)
    a = _run(z, t, dtype, "mean", 1.0)
    b = _run(z, t, dtype, "mean", 1.0, in_place=True)
    assert np.array_equal(a, b)


def test_bwd_large_shift_and_edge_rows():
    rows, vocab = 8, 4099
    z = _logits(5, rows, vocab, "f32", shift=-1000.0)
    z[1, :] = -np.inf
    z[1, 7] = 2.0            # one finite logit, the target: gradient 0 everywhere
    z[2, 3] += 200.0         # dominant non-target logit
    t = lce_synth.targets(6, rows, vocab)
    t[1] = 7
    t[2] = 10
    t[3] = -1                # invalid: NaN row
    got = _run(z, t, "f32", "none", np.ones(rows, np.float32))
    want = oracle.xent_bwd(z, t, np.ones(rows), "none", dtype="f32")
    _check(got, want, np.ones((rows, 1)), "f32", "edge rows")
    assert np.isnan(got[3]).all() and np.all(got[1] == 0.0)
    assert abs(got[2, 3] - 1.0) <= 2e-6 and abs(got[2, t[2]] + 1.0) <= 2e-6


@pytest.mark.parametrize("name", ["megatron_bf16_2048x4x4096_none", "ce_f32_16384x4096_mean"])
def test_bwd_full_size_sampled_rows(name):
    """Full workloads in the benchmark's launch configuration; the oracle checks a row sample."""
    w = lce_synth.WORKLOADS[name]
    z = w.logits()
    t = w.target()
    red = w.reduction
    grad = np.float32(1.0) if red == "mean" else np.linspace(0.5, 1.5, w.tokens).astype(np.float32)
    got = _run(z, t, w.dtype, red, grad)
    rows = np.r_[0:64, w.tokens - 64:w.tokens, np.arange(64, w.tokens - 64, 997)]
    g = (np.full(rows.size, 1.0 / w.tokens) if red == "mean" else grad[rows].astype(np.float64))
    # the sampled rows' gradients: per-token scale g_i (grad / tokens for the mean)
    want = oracle.xent_bwd(z[rows], t[rows], g, "none", dtype=w.dtype)
    _check(got[rows], want, g[:, None], w.dtype, name)


def test_bwd_row_longer_than_one_gib():
    """Maximum row length: a 1 GiB + 12 B fp32 row, whose statistics pass and gradient pass
    both run in slices below 1 GiB (32-bit buffer offsets); every element is checked."""
    rows, vocab = 1, (1 << 28) + 3
    print(f"\n[bwd] row above 1 GiB: f32 {rows}x{vocab}", flush=True)
    z = _logits(vocab + 21, rows, vocab, "f32")
    t = lce_synth.targets(vocab + 22, rows, vocab)
    want = oracle.xent_bwd(z, t, np.float64(1.0), "mean", dtype="f32")
    got = _run(z, t, "f32", "mean", np.float32(1.0))
    _check(got, want, np.ones((rows, 1)), "f32", "row above 1 GiB")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_bwd_unaligned_base(dtype):
    """Logits that start off a 16-byte boundary: the binding allocates the gradient at the
    same offset modulo 16 bytes, and a gradient buffer at another offset is refused."""
    rows, vocab = 12, 1000
    z = _logits(31, rows * vocab + 3, 1, dtype).reshape(-1)
    zd = to_dev(z)[3:].view(rows, vocab)
    t = lce_synth.targets(32, rows, vocab)
    td = torch.from_numpy(t).cuda()
    gd = torch.ones(1, device="cuda")
    d = lce.xent_bwd(zd, td, gd, "mean")
    torch.cuda.synchronize()
    assert (d.data_ptr() - zd.data_ptr()) % 16 == 0
    want = oracle.xent_bwd(np.ascontiguousarray(z[3:].reshape(rows, vocab)), t, np.float64(1.0), "mean",
                           dtype=dtype)
    _check(_to_host(d, dtype), want, np.full((rows, 1), 1.0 / rows), dtype, f"unaligned base {dtype}")
    with pytest.raises(lce.LceError) as e:
        lce.xent_bwd(zd, td, gd, "mean", out=torch.empty_like(zd))
    assert e.value.status == lce.LCE_ERR_UNSUPPORTED


# Rows of at most 128 16-byte chunks with no scalar edges: several rows per wave (8, 4
# or 2 rows for up to 32, 64 or 128 chunks), at and around each boundary, ragged row counts.
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(5, 4), (1, 8), (7, 64), (33, 124), (100, 128), (257, 132),
                                        (31, 256), (1001, 260), (65, 512)])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_bwd_several_rows_per_wave(dtype, rows, vocab, reduction):
    v = vocab if dtype == "f32" else 2 * vocab  # the same chunk counts in both dtypes
    z = _logits(rows * 13 + v, rows, v, dtype)
    t = lce_synth.targets(rows + 2 * v, rows, v)
    t[0] = v - 1
    if rows > 2:
        t[1], t[2] = 0, -1
    grad = np.float32(0.9) if reduction == "mean" else np.linspace(-1, 1, rows).astype(np.float32)
    got = _run(z, t, dtype, reduction, grad)
    nvec = v * (4 if dtype == "f32" else 2) // 16
    g = 8 if nvec <= 32 else 4 if nvec <= 64 else 2
    assert f"xent_bwd_group_kernel<{'float' if dtype == 'f32' else 'unsigned short'}, {g}, 4, 4, false>" \
        in lce.lce_last_launch()
    want = oracle.xent_bwd(z, t, np.asarray(grad, dtype=np.float64), reduction, dtype=dtype)
    gs = (np.full(rows, float(grad) / rows) if reduction == "mean" else grad.astype(np.float64))
    _check(got, want, gs[:, None], dtype, f"grouped {dtype} {rows}x{v} {reduction}")
    one_wave = _run(z, t, dtype, reduction, grad, env={"LCE_BWD_PATH": "wave"})
    _check(one_wave, want, gs[:, None], dtype, f"one wave {dtype} {rows}x{v} {reduction}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunks", [16, 48, 125])
@pytest.mark.parametrize("reduction", ["mean", "none"])
def test_bwd_several_rows_per_wave_special_values(dtype, chunks, reduction):
    """Special values on the several-rows-per-wave backward: rows with +inf, a NaN logit, a
    row of -inf only and invalid targets get NaN gradients, as in the oracle, and the
    finite rows that share their wave keep theirs; the one-call forward and backward gives
    the same gradient and the forward's losses."""
    vocab = chunks * (4 if dtype == "f32" else 8)
    rows = 37
    z = _logits(chunks * 11 + vocab, rows, vocab, "f32")
    z[0, 0] = np.inf
    z[1, vocab // 2] = np.inf
    z[2, vocab - 1] = np.inf
    z[3, 5] = np.nan
    z[4, :] = -np.inf
    t = lce_synth.targets(chunks + vocab, rows, vocab)
    t[5], t[6], t[7], t[8] = -1, vocab, 1 << 40, -(1 << 40)
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    grad = np.float32(1.25) if reduction == "mean" else np.linspace(-1, 1, rows).astype(np.float32)
    got = _run(z, t, dtype, reduction, grad)
    g = 8 if chunks <= 32 else 4 if chunks <= 64 else 2
    assert f"xent_bwd_group_kernel<{'float' if dtype == 'f32' else 'unsigned short'}, {g}, 4, 4, false>" \
        in lce.lce_last_launch()
    want = oracle.xent_bwd(z, t, np.asarray(grad, dtype=np.float64), reduction, dtype=dtype)
    gs = (np.full(rows, float(grad) / rows) if reduction == "mean" else grad.astype(np.float64))
    _check(got, want, gs[:, None], dtype, f"special values {dtype} {vocab} {reduction}")
    assert np.isnan(got[:9]).all() and np.isfinite(got[9:]).all()
    zd = to_dev(z)
    td = torch.from_numpy(t).cuda()
    gd = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    loss, d = lce.xent_fwd_bwd(zd, td, gd, reduction)
    fwd = lce.xent(zd, td, reduction)
    torch.cuda.synchronize()
    assert np.array_equal(_to_host(d, dtype), got, equal_nan=True)
    lw = oracle.xent_rows(z, t, dtype=dtype)
    lg = loss.cpu().numpy().astype(np.float64)
    if reduction == "mean":
        assert np.isnan(lg).all() and np.isnan(fwd.cpu().numpy()).all()
    else:
        assert np.array_equal(np.isnan(lg), np.isnan(lw))
        ok = ~np.isnan(lw)
        assert np.abs(lg[ok] - lw[ok]).max() <= 1e-4


@pytest.mark.parametrize("seed", range(2))
def test_bwd_randomized_several_rows_per_wave(seed):
    """Seeded random cases on the several-rows-per-wave backward, 8 per seed: 1-2000 rows of
    1-128 16-byte chunks, fp32 or bf16, scales 0.05 to 25, spikes, -inf entries, some invalid
    targets, either reduction; gradients against the oracle's softmax minus one-hot."""
    rng = np.random.default_rng(7500 + seed)
    for case in range(8):
        dtype = str(rng.choice(["f32", "bf16"]))
        per = 4 if dtype == "f32" else 8
        rows = int(np.exp(rng.uniform(0.0, np.log(2000.0))))
        vocab = int(rng.integers(1, 129)) * per
        std = float(rng.choice([0.05, 1.0, 4.0, 25.0]))
        z = rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)
        t = rng.integers(0, vocab, rows)
        if rng.random() < 0.5:
            for r in rng.integers(0, rows, 1 + rows // 4):
                z[r, rng.integers(0, vocab)] += np.float32(rng.uniform(5.0, 120.0))
        if rng.random() < 0.3:
            keep = z[np.arange(rows), t].copy()
            z[rng.random((rows, vocab)) < 0.2] = -np.inf
            z[np.arange(rows), t] = keep
        if rng.random() < 0.3:
            bad = rng.integers(0, rows, 1 + rows // 16)
            t[bad] = rng.choice([-1, vocab, 1 << 40], bad.size)
        host = z if dtype == "f32" else lce_synth.f32_to_bf16_bits(z)
        reduction = str(rng.choice(["mean", "none"]))
        grad = (np.float32(rng.uniform(0.5, 2.0)) if reduction == "mean"
                else rng.uniform(-1.0, 1.0, rows).astype(np.float32))
        label = f"seed {seed} case {case}: {dtype} {rows}x{vocab} std {std} {reduction}"
        got = _run(host, t, dtype, reduction, grad)
        assert "xent_bwd_group_kernel" in lce.lce_last_launch(), label
        want = oracle.xent_bwd(host, t, np.asarray(grad, dtype=np.float64), reduction, dtype=dtype)
        gs = (np.full(rows, float(grad) / rows) if reduction == "mean" else grad.astype(np.float64))
        _check(got, want, gs[:, None], dtype, label)


@pytest.mark.parametrize("seed", range(3))
def test_bwd_randomized_rows(seed):
    """Seeded random cases on every backward path, 10 per seed: 1-300 rows, vocab
    log-uniform in [1, 40000), fp32 or bf16, scales 0.05 to 25, shifts of -3000 to +1000,
    spikes 5 to 120 above the rest, -inf entries around finite targets, some invalid
    targets, the first row 0-7 elements past an aligned address, either reduction, the
    default path or one wave per row or the statistics-then-apply path; gradients against
    the oracle, the one-call forward and backward's gradient bitwise the same and its losses
    against the oracle's."""
    rng = np.random.default_rng(7700 + seed)
    for case in range(10):
        dtype = str(rng.choice(["f32", "bf16"]))
        rows = int(rng.integers(1, 301))
        vocab = max(1, int(np.exp(rng.uniform(0.0, np.log(40000.0)))))
        std = float(rng.choice([0.05, 1.0, 4.0, 25.0]))
        z = rng.standard_normal((rows, vocab), dtype=np.float32) * np.float32(std)
        z += np.float32(rng.choice([0.0, 0.0, 1000.0, -3000.0]))
        t = rng.integers(0, vocab, rows)
        if rng.random() < 0.5:
            for r in rng.integers(0, rows, 1 + rows // 4):
                z[r, rng.integers(0, vocab)] += np.float32(rng.uniform(5.0, 120.0))
        if rng.random() < 0.3:
            keep = z[np.arange(rows), t].copy()
            z[rng.random((rows, vocab)) < 0.2] = -np.inf
            z[np.arange(rows), t] = keep
        if rng.random() < 0.3:
            bad = rng.integers(0, rows, 1 + rows // 16)
            t[bad] = rng.choice([-1, vocab, 1 << 40], bad.size)
        host = z if dtype == "f32" else lce_synth.f32_to_bf16_bits(z)
        reduction = str(rng.choice(["mean", "none"]))
        grad = (np.float32(rng.uniform(0.5, 2.0)) if reduction == "mean"
                else rng.uniform(-1.0, 1.0, rows).astype(np.float32))
        path = str(rng.choice(["auto", "wave", "apply"]))
        off = int(rng.integers(0, 8))
        buf = np.zeros(off + rows * vocab, dtype=host.dtype)
        buf[off:] = host.reshape(-1)
        zd = to_dev(buf)[off:].view(rows, vocab)
        td = torch.from_numpy(t.astype(np.int64)).cuda()
        gd = torch.from_numpy(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
        label = f"seed {seed} case {case}: {dtype} {rows}x{vocab} std {std} offset {off} {path} {reduction}"
        env = {} if path == "auto" else {"LCE_BWD_PATH": path}
        with forced_env(**env):
            d = lce.xent_bwd(zd, td, gd, reduction)
            loss, d2 = lce.xent_fwd_bwd(zd, td, gd, reduction)
        torch.cuda.synchronize()
        got = _to_host(d, dtype)
        assert np.array_equal(got, _to_host(d2, dtype), equal_nan=True), label
        lw = oracle.xent_rows(host, t, dtype=dtype)
        lg = loss.cpu().numpy().astype(np.float64)
        if reduction == "none":
            assert np.array_equal(np.isnan(lg), np.isnan(lw)), label
            assert np.nanmax(np.abs(lg - lw), initial=0.0) <= 1e-4, label
        else:
            wm = oracle.mean(lw)
            assert (np.isnan(lg[0]) and np.isnan(wm)) or abs(lg[0] - wm) <= 1e-5 * abs(wm) + 1e-7, label
        want = oracle.xent_bwd(host, t, np.asarray(grad, dtype=np.float64), reduction, dtype=dtype)
        gs = (np.full(rows, float(grad) / rows) if reduction == "mean" else grad.astype(np.float64))
        _check(got, want, gs[:, None], dtype, label)
