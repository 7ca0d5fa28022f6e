"""GPU parity: liblce (through its C ABI) against the fp64 oracle, element by element.

Tolerances (fixed before any kernel was written):
  row cross-entropy, fp32 or bf16 logits: per-token |gpu - oracle| <= 1e-4,
                                          mean relative error <= 1e-5;
  fused projection + cross-entropy (bf16): per-token |gpu - oracle| <= 2e-2,
                                          mean relative error <= 1e-3.
Inputs come from the seeded generator in ``lce_synth``; the oracle sees the very
same bytes.  Small cases span several tiles, ragged tails, unaligned rows and
every kernel path; the five full-size workloads run in the launch configuration
the benchmark times.
"""
import math

import numpy as np
import pytest

import lce_synth
import oracle
from lce_synth import WORKLOADS

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import forced_env, to_dev  # noqa: E402

TOK_ABS = 1e-4
MEAN_REL = 1e-5
MEAN_ABS_FLOOR = 1e-7
FUSED_TOK_ABS = 2e-2
FUSED_MEAN_REL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def gpu_xent(logits_np, target_np, reduction, dtype):
    z = to_dev(logits_np)
    t = torch.from_numpy(np.ascontiguousarray(target_np, dtype=np.int64)).cuda()
    out = lce.xent(z, t, reduction)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def rand_logits(rng_seed, rows, vocab, dtype, std=1.0, shift=0.0):
    f = lce_synth.normal_f32(rng_seed, 9, rows, vocab, std)
    if shift:
        f = f + np.float32(shift)
    return f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f)


def check_xent(logits_np, target_np, dtype, label=""):
    want = oracle.xent_rows(logits_np, target_np, dtype=dtype)
    got = gpu_xent(logits_np, target_np, "none", dtype)
    assert got.shape == want.shape
    err = np.abs(got - want)
    assert np.array_equal(np.isnan(got), np.isnan(want)), label
    assert np.nanmax(err, initial=0.0) <= TOK_ABS, f"{label} max abs err {np.nanmax(err)}"
    gm = gpu_xent(logits_np, target_np, "mean", dtype)[0]
    wm = oracle.mean(want)
    if math.isnan(wm):
        assert math.isnan(gm), label
    else:
        # relative bound; the absolute floor only matters where the exact mean is 0
        # (vocab = 1), where a relative bound is undefined
        assert abs(gm - wm) <= MEAN_REL * abs(wm) + MEAN_ABS_FLOOR, f"{label} mean {gm} vs {wm}"
    return float(np.nanmax(err, initial=0.0))


# ------------------------------------------------------------------ small shapes, every path

SMALL = [(1, 1), (3, 2), (5, 3), (7, 7), (64, 31), (17, 64), (9, 100), (33, 255), (65, 1000),
         (40, 4096), (13, 4097), (21, 5000), (8, 8191), (5, 8193), (3, 20000)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", SMALL)
def test_small_auto_path(dtype, rows, vocab):
    z = rand_logits(rows * 7919 + vocab, rows, vocab, dtype)
    t = lce_synth.targets(vocab + 5, rows, vocab)
    check_xent(z, t, dtype, f"{dtype} {rows}x{vocab}")


@pytest.mark.parametrize("path,extra", [("wave", {}), ("block", {}), ("split", {}),
                                        ("split", {"LCE_SPLITS": 3}), ("split", {"LCE_SPLITS": 7}),
                                        ("split", {"LCE_SPLITS": 41})])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(6, 3), (11, 777), (9, 4099), (4, 33333), (2, 70001)])
def test_forced_paths(path, extra, dtype, rows, vocab):
    z = rand_logits(rows + vocab, rows, vocab, dtype, std=3.0)
    t = lce_synth.targets(vocab, rows, vocab)
    with forced_env(LCE_PATH=path, **extra):
        check_xent(z, t, dtype, f"{path} {extra} {dtype} {rows}x{vocab}")


# Rows of at most 128 16-byte chunks with no scalar edges take several rows per wave
# (8, 4 or 2 rows for up to 32, 64 or 128 chunks): chunk counts at and around each
# boundary, ragged row counts (a last wave with fewer rows than it holds).
GROUP = [(5, 4), (1, 8), (7, 64), (33, 124), (100, 128), (257, 132), (31, 256), (1001, 260), (65, 512)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", GROUP)
def test_several_rows_per_wave(dtype, rows, vocab):
    v = vocab if dtype == "f32" else 2 * vocab  # the same chunk counts in both dtypes
    z = rand_logits(rows * 31 + v, rows, v, dtype, std=2.5)
    t = lce_synth.targets(rows + v, rows, v)
    t[0] = v - 1
    if rows > 2:
        t[1], t[2] = 0, -1
    check_xent(z, t, dtype, f"{dtype} {rows}x{v}")
    lce.xent(to_dev(z), torch.from_numpy(t).cuda(), "none")
    nvec = v * (4 if dtype == "f32" else 2) // 16
    g = 8 if nvec <= 32 else 4 if nvec <= 64 else 2
    assert f"xent_group_rows_kernel<{'float' if dtype == 'f32' else 'unsigned short'}, {g}, 4, 4>" \
        in lce.lce_last_launch()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_several_rows_per_wave_edge_rows(dtype):
    """Rows held several to a wave: an all -inf row but its target, a spike far above the
    fixed reference (refolded with the running maximum), -inf entries, a row with no finite
    logit (NaN loss)."""
    rows, vocab = 24, 512 if dtype == "f32" else 1024
    z = rand_logits(77, rows, vocab, "f32", std=2.0)
    z[1, :] = -np.inf
    z[1, 5] = 3.0
    z[2, 300] = 90.0
    z[3, ::3] = -np.inf
    z[4, :] = -np.inf
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    t = lce_synth.targets(78, rows, vocab)
    t[1], t[2] = 5, 300
    check_xent(z, t, dtype, f"edge rows {dtype}")


def special_rows(seed, rows, vocab):
    """fp32 rows with the special values of the one-row tests, at the top of the batch:
    +inf at the first, an interior and the last element (NaN loss), a NaN logit, a row of
    -inf only (NaN loss), then targets at -1, at vocab, far past it and far below 0 (NaN
    loss), then finite rows.  Returns the logits, the targets and how many rows are NaN."""
    z = rand_logits(seed, rows, vocab, "f32", std=2.0)
    z[0, 0] = np.inf
    z[1, vocab // 2] = np.inf
    z[2, vocab - 1] = np.inf
    z[3, min(5, vocab - 1)] = np.nan
    z[4, :] = -np.inf
    t = lce_synth.targets(seed + 1, rows, vocab)
    t[5], t[6], t[7], t[8] = -1, vocab, 1 << 40, -(1 << 40)
    return z, t, 9


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("chunks", [16, 48, 125])
def test_several_rows_per_wave_special_values(dtype, chunks):
    """Special values on the several-rows-per-wave kernel (8, 4 and 2 rows per wave):
    the NaN rows must not leak into the finite rows that share their wave."""
    vocab = chunks * (4 if dtype == "f32" else 8)
    z, t, n_nan = special_rows(chunks * 7 + vocab, 37, vocab)
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    check_xent(z, t, dtype, f"special values {dtype} {vocab}")
    got = gpu_xent(z, t, "none", dtype)
    assert np.isnan(got[:n_nan]).all() and np.isfinite(got[n_nan:]).all()
    g = 8 if chunks <= 32 else 4 if chunks <= 64 else 2
    assert f"xent_group_rows_kernel<{'float' if dtype == 'f32' else 'unsigned short'}, {g}, 4, 4>" \
        in lce.lce_last_launch()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_large_shift_keeps_accuracy(dtype):
    """Rows shifted by -1000 (exact in both dtypes' grids) lose no accuracy."""
    z = rand_logits(4, 37, 3001, "f32", std=2.0)
    z = (np.round(z * 64) / 64 - 1000).astype(np.float32)
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    check_xent(z, lce_synth.targets(6, 37, 3001), dtype, "shift -1000")


def test_row_shift_invariance_exact_inputs():
    """Logits on a 2^-8 grid (|z| < 8) plus integer row shifts up to 2^15 are exact in
    fp32; the GPU loss must not move by more than the tolerance."""
    rng = np.random.default_rng(1)
    rows, vocab = 64, 4096
    z = (np.round(rng.uniform(-8, 8, (rows, vocab)) * 256) / 256).astype(np.float32)
    c = rng.integers(-2 ** 15, 2 ** 15, rows).astype(np.float32)
    t = rng.integers(0, vocab, rows)
    a = gpu_xent(z, t, "none", "f32")
    b = gpu_xent(z + c[:, None], t, "none", "f32")
    assert np.max(np.abs(a - b)) <= TOK_ABS


def test_uniform_logits_give_ln_vocab():
    for vocab in (1, 2, 4096, 131072):
        z = np.full((4, vocab), 37.5, dtype=np.float32)
        got = gpu_xent(z, np.arange(4) % vocab, "none", "f32")
        assert np.max(np.abs(got - math.log(vocab))) <= TOK_ABS


def test_megatron_layout_matches_flat_view():
    w = WORKLOADS["megatron_bf16_2048x4x4096_none"]
    z = to_dev(w.logits(0, 512)).view(128, 4, 4096)
    t = torch.from_numpy(w.target(0, 512)).cuda().view(128, 4)
    a = lce.xent(z, t, "none")
    b = lce.xent(z.reshape(512, 4096), t.reshape(512), "none")
    torch.cuda.synchronize()
    assert a.shape == (128, 4)
    assert torch.equal(a.reshape(512), b)


def test_invalid_targets_and_nan_logits():
    rows, vocab = 8, 1000
    z = rand_logits(3, rows, vocab, "f32")
    z[5, 17] = np.nan
    t = np.array([0, -1, 999, 1000, 5, 3, 1 << 40, 2], dtype=np.int64)
    check_xent(z, t, "f32", "invalid")
    got = gpu_xent(z, t, "none", "f32")
    assert np.isnan(got[[1, 3, 5, 6]]).all() and not np.isnan(got[[0, 2, 4, 7]]).any()
    assert math.isnan(gpu_xent(z, t, "mean", "f32")[0])


def _spiky_rows(vocab):
    """Rows that exercise the running maximum: a rising ramp, a falling ramp, single
    spikes far above the rest (more than 44 nats, past the one-pass fold's overflow
    guard) and moderately above it (rescale only) at the first, an interior and the last
    element, -inf entries, and rows that are -inf except at one or two elements."""
    rows = 14
    z = rand_logits(11, rows, vocab, "f32")
    ramp = np.linspace(0.0, 30.0, vocab, dtype=np.float32)
    z[0] += ramp
    z[1] -= ramp
    for r, pos, h in ((2, 0, 200.0), (3, 7, 200.0), (4, vocab // 2, 200.0), (5, vocab - 1, 200.0),
                      (6, 8 * 64 * 8, 60.0), (7, vocab // 3, 25.0), (8, 5 * vocab // 7, 300.0)):
        z[r, min(pos, vocab - 1)] += h
    z[8, vocab // 5] += 150.0
    z[9, ::3] = -np.inf
    z[10, :] = -np.inf
    z[10, vocab // 2] = 3.0
    z[11, :] = -np.inf
    z[11, [1, vocab - 2]] = (-5.0, 7.0)
    z[12, vocab // 4:] -= 100.0
    z[13] *= 40.0
    t = lce_synth.targets(12, rows, vocab)
    t[9] = 1  # a finite entry (every third one is -inf)
    t[10] = vocab // 2
    t[11] = vocab - 2
    return z, t


@pytest.mark.parametrize("path", ["auto", "wave", "block", "split"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab", [4099, 9000])
def test_running_maximum_edge_rows(path, dtype, vocab):
    z, t = _spiky_rows(vocab)
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    env = {} if path == "auto" else {"LCE_PATH": path}
    with forced_env(**env):
        check_xent(z, t, dtype, f"{path} {dtype} {vocab}")
        got = gpu_xent(z, t, "none", dtype)
    assert abs(got[10]) <= TOK_ABS  # one finite logit, the target: loss 0


@pytest.mark.parametrize("path", ["auto", "wave", "block", "split", "split_many"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("vocab", [4096, 20000])
def test_fixed_reference_guard_boundary(path, dtype, vocab):
    """Loss rows are first folded against each lane's first-chunk maximum, and again with
    a tracked maximum when a lane's sum reaches 2^64 (a logit about 44.4 above that
    reference).  Spikes of 40 to 48 above a flat row put lane sums on both sides of that
    bound, in the first, a middle and the last chunk a lane reads; other rows hold many
    logits 36 to 41 above the first chunk, so sums of many large terms approach it too.
    4096-wide rows take the unrolled short loop, 20000-wide the long loop (the block
    path takes its own loop, the split path its slices, with its default slice count and
    with 5 slices); every row must match the oracle."""
    heights = [40.0, 43.0, 44.0, 44.5, 45.0, 48.0]
    positions = [1024 + 5, vocab // 2 + 3, vocab - 9]
    rows = len(heights) * len(positions) + 4
    z = np.round(rand_logits(21, rows, vocab, "f32") * 64) / 64
    r = 0
    for h in heights:
        for pos in positions:
            z[r, pos] += np.float32(h)
            r += 1
    for lift in (36.0, 38.0, 40.0, 41.0):  # every element past the first 1024, lifted
        z[r, 1024:] += np.float32(lift)
        r += 1
    z = z.astype(np.float32)
    t = lce_synth.targets(22, rows, vocab)
    t[:len(positions)] = positions  # the spike itself is the target in a few rows
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    env = {} if path == "auto" else {"LCE_PATH": path}
    if path == "split_many":
        env = {"LCE_PATH": "split", "LCE_SPLITS": 5}
    with forced_env(**env):
        check_xent(z, t, dtype, f"guard {path} {dtype} {vocab}")


@pytest.mark.parametrize("seed", range(4))
def test_randomized_rows(seed):
    """Seeded random cases, 16 per seed, each checked against the oracle element by
    element: 1-79 rows, vocab log-uniform in [1, 40000), fp32 or bf16, logit scales from
    0.05 to 25, whole-matrix shifts of -3000 to +1000, spikes 5 to 120 above the rest (past
    the fixed-reference guard or not), -inf entries around finite targets, a first row
    0-7 elements past an aligned address, and every forced path."""
    rng = np.random.default_rng(7100 + seed)
    for case in range(16):
        dtype = str(rng.choice(["f32", "bf16"]))
        rows = int(rng.integers(1, 80))
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
        host = z if dtype == "f32" else lce_synth.f32_to_bf16_bits(z)
        off = int(rng.integers(0, 8))
        buf = np.zeros(off + rows * vocab, dtype=host.dtype)
        buf[off:] = host.reshape(-1)
        zd = to_dev(buf)[off:].view(rows, vocab)
        td = torch.from_numpy(t.astype(np.int64)).cuda()
        path = str(rng.choice(["auto", "wave", "block", "split"]))
        label = f"seed {seed} case {case}: {dtype} {rows}x{vocab} std {std} offset {off} {path}"
        want = oracle.xent_rows(host, t, dtype=dtype)
        env = {} if path == "auto" else {"LCE_PATH": path}
        with forced_env(**env):
            got = lce.xent(zd, td, "none").cpu().numpy().astype(np.float64)
            gm = lce.xent(zd, td, "mean").item()
        assert np.array_equal(np.isnan(got), np.isnan(want)), label
        assert np.nanmax(np.abs(got - want), initial=0.0) <= TOK_ABS, label
        wm = oracle.mean(want)
        assert abs(gm - wm) <= MEAN_REL * abs(wm) + MEAN_ABS_FLOOR, f"{label}: mean {gm} vs {wm}"


@pytest.mark.parametrize("seed", range(3))
def test_randomized_several_rows_per_wave(seed):
    """Seeded random cases on the several-rows-per-wave kernel, 16 per seed: 1-3000 rows of
    1-128 16-byte chunks (aligned, no scalar edges), fp32 or bf16, logit scales 0.05 to 25,
    shifts of -3000 to +1000, spikes 5 to 120 above the rest, -inf entries around finite
    targets, some invalid targets; per-token losses and the mean against the oracle."""
    rng = np.random.default_rng(7300 + seed)
    for case in range(16):
        dtype = str(rng.choice(["f32", "bf16"]))
        per = 4 if dtype == "f32" else 8
        rows = int(np.exp(rng.uniform(0.0, np.log(3000.0))))
        nvec = int(rng.integers(1, 129))
        vocab = nvec * per
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
        label = f"seed {seed} case {case}: {dtype} {rows}x{vocab} std {std}"
        want = oracle.xent_rows(host, t, dtype=dtype)
        zd, td = to_dev(host), torch.from_numpy(t.astype(np.int64)).cuda()
        got = lce.xent(zd, td, "none").cpu().numpy().astype(np.float64)
        assert "xent_group_rows_kernel" in lce.lce_last_launch(), label
        gm = lce.xent(zd, td, "mean").item()
        assert np.array_equal(np.isnan(got), np.isnan(want)), label
        assert np.nanmax(np.abs(got - want), initial=0.0) <= TOK_ABS, label
        wm = oracle.mean(want)
        if math.isnan(wm):
            assert math.isnan(gm), label
        else:
            assert abs(gm - wm) <= MEAN_REL * abs(wm) + MEAN_ABS_FLOOR, f"{label}: mean {gm} vs {wm}"


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_infinite_logits(dtype):
    """+inf anywhere in a row makes that row's loss NaN, and a row of -inf only is NaN,
    as in the oracle (both evaluate the max-shifted form)."""
    rows, vocab = 6, 3000
    z = rand_logits(13, rows, vocab, "f32")
    z[0, 0] = np.inf
    z[1, 1234] = np.inf
    z[2, vocab - 1] = np.inf
    z[3, :] = -np.inf
    t = lce_synth.targets(14, rows, vocab)
    if dtype == "bf16":
        z = lce_synth.f32_to_bf16_bits(z)
    check_xent(z, t, dtype, "inf")
    got = gpu_xent(z, t, "none", dtype)
    assert np.isnan(got[:4]).all() and np.isfinite(got[4:]).all()


def test_zero_tokens():
    z = torch.empty((0, 16), device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    assert math.isnan(lce.xent(z, t, "mean").item())
    assert lce.xent(z, t, "none").numel() == 0


def test_output_guard_bytes_untouched():
    rows, vocab = 100, 513
    z = to_dev(rand_logits(8, rows, vocab, "f32"))
    t = torch.from_numpy(lce_synth.targets(8, rows, vocab)).cuda()
    buf = torch.full((rows + 64,), 7.25, device="cuda")
    out = buf[32:32 + rows]
    lce.xent(z, t, "none", out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[:32] == 7.25) and torch.all(buf[32 + rows:] == 7.25)
    assert torch.isfinite(out).all()


def test_repeated_calls_bitwise_identical():
    w = WORKLOADS["ce_f32_16384x4096_mean"]
    z = to_dev(w.logits(0, 4096))
    t = torch.from_numpy(w.target(0, 4096)).cuda()
    first_mean = lce.xent(z, t, "mean").clone()
    first_none = lce.xent(z, t, "none").clone()
    for _ in range(5):
        assert torch.equal(lce.xent(z, t, "mean"), first_mean)
        assert torch.equal(lce.xent(z, t, "none"), first_none)


def test_binding_checks_shapes():
    z = torch.zeros((4, 8), device="cuda")
    with pytest.raises(ValueError):
        lce.xent(z, torch.zeros(5, dtype=torch.int64, device="cuda"))
    with pytest.raises(TypeError):
        lce.xent(z.half(), torch.zeros(4, dtype=torch.int64, device="cuda"))


# ------------------------------------------------------------------ full-size workloads

def load_workload_streaming(w, block_rows=1024):
    """Generate a row-CE workload block by block into device memory; return the device
    logits (in the workload's shape), device targets and the oracle's per-token losses."""
    tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    dev = torch.empty(w.shape, dtype=tdt, device="cuda")
    flat = dev.view(w.tokens, w.vocab)
    tgt = w.target()
    want = np.empty(w.tokens)
    for r0 in range(0, w.tokens, block_rows):
        r1 = min(w.tokens, r0 + block_rows)
        host = w.logits(r0, r1)
        flat[r0:r1].copy_(to_dev(host))
        want[r0:r1] = oracle.xent_rows(host, tgt[r0:r1], dtype=w.dtype)
        del host
    t_dev = torch.from_numpy(tgt).cuda().view(w.target_shape)
    return dev, t_dev, want


@pytest.mark.parametrize("name", ["ce_f32_16384x4096_mean", "megatron_bf16_2048x4x4096_none",
                                  "ce_f32_16384x131072_mean", "megatron_bf16_2048x4x131072_none"])
def test_full_size_row_workloads(name):
    """Every logit of the four row workloads against the oracle, per token and the mean, on
    the default path; the two 131072-wide workloads also on the split-vocab path forced
    with 8 and 32 slices per row (the path the large-vocab configuration names, which the
    default selection keeps for fewer rows than twice the CU count)."""
    w = WORKLOADS[name]
    print(f"\n[parity] workload {name} shape {w.shape}", flush=True)
    z, t, want = load_workload_streaming(w)
    wm = oracle.mean(want)
    envs = [{}]
    if w.vocab == 131072:
        envs += [{"LCE_PATH": "split", "LCE_SPLITS": 8}, {"LCE_PATH": "split", "LCE_SPLITS": 32}]
    for env in envs:
        with forced_env(**env):
            per = lce.xent(z, t, "none").cpu().numpy().reshape(-1).astype(np.float64)
            launch_none = lce.lce_last_launch()
            mean = lce.xent(z, t, "mean").item()
            launch_mean = lce.lce_last_launch()
        err = np.abs(per - want)
        print(f"[parity] {name} {env}: max abs err {err.max():.3e}; mean {mean:.8f} vs {wm:.8f}; "
              f"{launch_none} | {launch_mean}", flush=True)
        if env:
            s = env["LCE_SPLITS"]
            assert launch_none.startswith("xent_split_partial_kernel") and f"grid ({s}, " in launch_none
            assert launch_mean.startswith("xent_split_partial_kernel") and f"grid ({s}, " in launch_mean
        assert err.max() <= TOK_ABS, env
        assert abs(mean - wm) <= MEAN_REL * abs(wm), env
    del z
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["ce_f32_16384x131072_mean", "megatron_bf16_2048x4x131072_none"])
def test_few_long_rows_take_the_split_path(name):
    """256 rows of a 131072-wide workload (fewer rows than twice the CU count): the default
    selection is the split-vocab path; every row against the oracle, per token and mean."""
    w = WORKLOADS[name]
    rows = 256
    host = w.logits(0, rows)
    tg = w.target(0, rows)
    want = oracle.xent_rows(host, tg, dtype=w.dtype)
    wm = oracle.mean(want)
    z, t = to_dev(host), torch.from_numpy(tg).cuda()
    per = lce.xent(z, t, "none").cpu().numpy().astype(np.float64)
    launch = lce.lce_last_launch()
    mean = lce.xent(z, t, "mean").item()
    print(f"\n[parity] {name} rows [0, {rows}): {launch}; max abs err "
          f"{np.max(np.abs(per - want)):.3e}", flush=True)
    assert launch.startswith("xent_split_partial_kernel"), launch
    assert np.max(np.abs(per - want)) <= TOK_ABS
    assert abs(mean - wm) <= MEAN_REL * abs(wm)


@pytest.mark.parametrize("dtype,rows,vocab", [("f32", 2, (1 << 28) + 3), ("bf16", 1, (1 << 29) + 5)])
def test_rows_longer_than_one_gib(dtype, rows, vocab):
    """Maximum row length: rows of more than 1 GiB, which no kernel addresses in one piece
    (32-bit buffer offsets).  Whatever path is asked for, the host cuts each row into slices
    below 1 GiB; asked for one split, it still takes two."""
    print(f"\n[parity] rows above 1 GiB: {dtype} {rows}x{vocab}", flush=True)
    z = rand_logits(vocab + 11, rows, vocab, dtype, std=2.0)
    t = lce_synth.targets(vocab + 12, rows, vocab)
    want = oracle.xent_rows(z, t, dtype=dtype)
    wm = oracle.mean(want)
    zd = to_dev(z)
    del z
    td = torch.from_numpy(t).cuda()
    for env in ({}, {"LCE_PATH": "block"}, {"LCE_PATH": "split", "LCE_SPLITS": 1}):
        with forced_env(**env):
            got = lce.xent(zd, td, "none").cpu().numpy().astype(np.float64)
            gm = lce.xent(zd, td, "mean").item()
        err = np.max(np.abs(got - want))
        print(f"[parity] {dtype} {rows}x{vocab} {env}: max abs err {err:.3e}", flush=True)
        assert err <= TOK_ABS, env
        assert abs(gm - wm) <= MEAN_REL * abs(wm), env
    del zd
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype,vocab,paths", [("f32", 5, ({}, {"LCE_PATH": "wave"}, {"LCE_PATH": "block"})),
                                               ("bf16", 9, ({},))])
def test_many_short_rows(dtype, vocab, paths):
    """Row count far above the workloads' at small memory: 2^22 + 7 rows of a few logits
    each (grids of up to four million workgroups, and as many partials for the mean's last
    workgroup)."""
    rows = (1 << 22) + 7
    print(f"\n[parity] many short rows: {dtype} {rows}x{vocab}", flush=True)
    z = rand_logits(rows + vocab, rows, vocab, dtype, std=3.0)
    t = lce_synth.targets(vocab + 40, rows, vocab)
    want = oracle.xent_rows(z, t, dtype=dtype)
    wm = oracle.mean(want)
    zd = to_dev(z)
    td = torch.from_numpy(t).cuda()
    for env in paths:
        with forced_env(**env):
            got = lce.xent(zd, td, "none").cpu().numpy().astype(np.float64)
            gm = lce.xent(zd, td, "mean").item()
        err = np.max(np.abs(got - want))
        print(f"[parity] {dtype} {rows}x{vocab} {env}: max abs err {err:.3e}, mean {gm:.8f} vs {wm:.8f}",
              flush=True)
        assert err <= TOK_ABS, env
        assert abs(gm - wm) <= MEAN_REL * abs(wm), env
    del zd
    torch.cuda.empty_cache()


def test_fused_full_size_workload():
    w = WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    print(f"\n[parity] fused workload {w.shape}", flush=True)
    xb, wb, tg = w.x(), w.weight(), w.target()
    x, W, t = to_dev(xb), to_dev(wb), torch.from_numpy(tg).cuda()
    per = lce.fused_linear_xent(x, W, t, "none").cpu().numpy().astype(np.float64)
    mean = lce.fused_linear_xent(x, W, t, "mean").item()
    want = oracle.fused_linear_xent_rows(xb, wb, tg)
    err = np.abs(per - want)
    wm = oracle.mean(want)
    print(f"[parity] fused: max abs err {err.max():.3e}; mean {mean:.8f} vs {wm:.8f}", flush=True)
    assert err.max() <= FUSED_TOK_ABS
    assert abs(mean - wm) <= FUSED_MEAN_REL * abs(wm)
    del x, W
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ fused, small shapes

FUSED_SMALL = [(1, 8, 1), (7, 64, 5), (33, 72, 300), (300, 136, 1000), (257, 64, 4099),
               (64, 512, 513), (520, 256, 2000)]


@pytest.mark.parametrize("tokens,hidden,vocab", FUSED_SMALL)
def test_fused_small(tokens, hidden, vocab):
    xb = lce_synth.normal_bf16_bits(11 + tokens, 0, tokens, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(12 + vocab, 2, vocab, hidden, 1.0 / math.sqrt(hidden) * 3)
    tg = lce_synth.targets(13, tokens, vocab)
    x, W, t = to_dev(xb), to_dev(wb), torch.from_numpy(tg).cuda()
    want = oracle.fused_linear_xent_rows(xb, wb, tg)
    per = lce.fused_linear_xent(x, W, t, "none").cpu().numpy().astype(np.float64)
    mean = lce.fused_linear_xent(x, W, t, "mean").item()
    err = np.abs(per - want)
    assert err.max() <= FUSED_TOK_ABS, f"max abs err {err.max()}"
    # fp32 accumulation of exact bf16 products: far inside the stated tolerance
    assert err.max() <= 1e-3
    wm = oracle.mean(want)
    assert abs(mean - wm) <= FUSED_MEAN_REL * abs(wm) + MEAN_ABS_FLOOR  # floor: vocab = 1


@pytest.mark.parametrize("seed", range(3))
def test_fused_randomized(seed):
    """Seeded random fused cases, 8 per seed, each against the oracle token by token:
    1-599 tokens, hidden a multiple of 8 in [8, 1024], vocab log-uniform in [1, 6000),
    activations N(0, 1) and a head scaled to logit spreads from ~0.3 to ~12, targets
    anywhere (also the first and last vocab rows), and the vocab split into the default or
    a forced number of segments (1-9)."""
    rng = np.random.default_rng(8200 + seed)
    for case in range(8):
        tokens = int(rng.integers(1, 600))
        hidden = 8 * int(rng.integers(1, 129))
        vocab = max(1, int(np.exp(rng.uniform(0.0, np.log(6000.0)))))
        spread = float(rng.choice([0.3, 1.0, 3.0, 12.0]))
        xb = lce_synth.normal_bf16_bits(9000 + 97 * seed + case, 0, tokens, hidden, 1.0)
        wb = lce_synth.normal_bf16_bits(9500 + 97 * seed + case, 2, vocab, hidden,
                                        spread / math.sqrt(hidden))
        tg = rng.integers(0, vocab, tokens)
        tg[rng.random(tokens) < 0.1] = vocab - 1
        tg[rng.random(tokens) < 0.1] = 0
        segments = int(rng.choice([0, 1, 2, 3, 9]))
        label = f"seed {seed} case {case}: T {tokens} H {hidden} V {vocab} spread {spread} segments {segments}"
        x, W, t = to_dev(xb), to_dev(wb), torch.from_numpy(tg.astype(np.int64)).cuda()
        want = oracle.fused_linear_xent_rows(xb, wb, tg)
        env = {"LCE_FUSED_SEGMENTS": segments} if segments else {}
        with forced_env(**env):
            per = lce.fused_linear_xent(x, W, t, "none").cpu().numpy().astype(np.float64)
            mean = lce.fused_linear_xent(x, W, t, "mean").item()
        err = np.abs(per - want)
        assert err.max() <= FUSED_TOK_ABS, f"{label}: max abs err {err.max()}"
        wm = oracle.mean(want)
        assert abs(mean - wm) <= FUSED_MEAN_REL * abs(wm) + MEAN_ABS_FLOOR, f"{label}: {mean} vs {wm}"


@pytest.mark.parametrize("seed", range(2))
def test_fused_spiky_heads(seed):
    """Seeded random fused cases with a few head rows scaled 10-40x (logits up to a few
    hundred, so the tiles and segments holding them dominate their tokens' sums), 8 per
    seed; the per-token losses, the mean and the one-call forward and backward's mean
    against the oracle."""
    rng = np.random.default_rng(8800 + seed)
    for case in range(8):
        tokens = int(rng.integers(1, 400))
        hidden = 8 * int(rng.integers(1, 65))
        vocab = max(1, int(np.exp(rng.uniform(0.0, np.log(6000.0)))))
        xb = lce_synth.normal_bf16_bits(9300 + 17 * seed + case, 0, tokens, hidden, 1.0)
        w = lce_synth.normal_f32(9400 + 17 * seed + case, 2, vocab, hidden, 1.0 / math.sqrt(hidden))
        for r in rng.integers(0, vocab, 1 + vocab // 50):
            w[r] *= np.float32(rng.uniform(10.0, 40.0))
        wb = lce_synth.f32_to_bf16_bits(w)
        tg = rng.integers(0, vocab, tokens)
        segments = int(rng.choice([0, 1, 2, 3, 9]))
        label = f"seed {seed} case {case}: T {tokens} H {hidden} V {vocab} segments {segments}"
        x, W, t = to_dev(xb), to_dev(wb), torch.from_numpy(tg.astype(np.int64)).cuda()
        want = oracle.fused_linear_xent_rows(xb, wb, tg)
        env = {"LCE_FUSED_SEGMENTS": segments} if segments else {}
        with forced_env(**env):
            per = lce.fused_linear_xent(x, W, t, "none").cpu().numpy().astype(np.float64)
            mean = lce.fused_linear_xent(x, W, t, "mean").item()
            loss, _, _ = lce.fused_linear_xent_fwd_bwd(x, W, t, torch.ones(1, device="cuda"), "mean")
        err = np.abs(per - want)
        assert err.max() <= FUSED_TOK_ABS, f"{label}: max abs err {err.max()}"
        wm = oracle.mean(want)
        for name, m in (("mean", mean), ("one-call mean", loss.item())):
            assert abs(m - wm) <= FUSED_MEAN_REL * abs(wm) + MEAN_ABS_FLOOR, f"{label}: {name} {m} vs {wm}"


@pytest.mark.parametrize("segments", [1, 2, 3, 5])
def test_fused_segment_counts(segments):
    tokens, hidden, vocab = 300, 128, 3000
    xb = lce_synth.normal_bf16_bits(21, 0, tokens, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(22, 2, vocab, hidden, 0.2)
    tg = lce_synth.targets(23, tokens, vocab)
    want = oracle.fused_linear_xent_rows(xb, wb, tg)
    with forced_env(LCE_FUSED_SEGMENTS=segments):
        per = lce.fused_linear_xent(to_dev(xb), to_dev(wb), torch.from_numpy(tg).cuda(), "none")
        per = per.cpu().numpy().astype(np.float64)
    assert np.abs(per - want).max() <= 1e-3


def test_fused_identity_head_matches_row_path():
    """W = I: the fused loss equals the row kernel's loss on x."""
    tokens, hidden = 96, 256
    xb = lce_synth.normal_bf16_bits(31, 0, tokens, hidden, 2.0)
    eye = lce_synth.f32_to_bf16_bits(np.eye(hidden, dtype=np.float32))
    tg = lce_synth.targets(32, tokens, hidden)
    a = lce.fused_linear_xent(to_dev(xb), to_dev(eye), torch.from_numpy(tg).cuda(), "none")
    b = lce.xent(to_dev(xb), torch.from_numpy(tg).cuda(), "none")
    torch.cuda.synchronize()
    assert torch.max(torch.abs(a - b)).item() <= 1e-5


def test_fused_invalid_targets():
    tokens, hidden, vocab = 10, 64, 500
    xb = lce_synth.normal_bf16_bits(41, 0, tokens, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(42, 2, vocab, hidden, 0.2)
    tg = np.array([0, -1, 499, 500, 7, 1 << 33, 3, 2, 1, 0], dtype=np.int64)
    got = lce.fused_linear_xent(to_dev(xb), to_dev(wb), torch.from_numpy(tg).cuda(), "none").cpu().numpy()
    assert np.isnan(got[[1, 3, 5]]).all() and not np.isnan(got[[0, 2, 4, 6, 7, 8, 9]]).any()


def test_fused_repeated_calls_bitwise_identical():
    tokens, hidden, vocab = 512, 256, 5000
    x = to_dev(lce_synth.normal_bf16_bits(51, 0, tokens, hidden, 1.0))
    W = to_dev(lce_synth.normal_bf16_bits(52, 2, vocab, hidden, 0.1))
    t = torch.from_numpy(lce_synth.targets(53, tokens, vocab)).cuda()
    first = lce.fused_linear_xent(x, W, t, "none").clone()
    m0 = lce.fused_linear_xent(x, W, t, "mean").clone()
    for _ in range(3):
        assert torch.equal(lce.fused_linear_xent(x, W, t, "none"), first)
        assert torch.equal(lce.fused_linear_xent(x, W, t, "mean"), m0)


@pytest.mark.parametrize("path", ["wave", "block", "split"])
def test_mean_handoff_many_workgroups(path):
    """The deterministic mean's finisher sees every workgroup's partial: 30 back-to-back calls
    (thousands of workgroups each) agree bitwise, and the mean matches the average of
    the per-token losses."""
    rows, vocab = (16384, 2048) if path != "split" else (512, 40000)
    z = torch.randn((rows, vocab), device="cuda", generator=torch.Generator("cuda").manual_seed(7))
    t = torch.randint(0, vocab, (rows,), device="cuda", generator=torch.Generator("cuda").manual_seed(8))
    with forced_env(LCE_PATH=path):
        per = lce.xent(z, t, "none").double()
        means = [lce.xent(z, t, "mean").clone() for _ in range(30)]
    torch.cuda.synchronize()
    for m in means[1:]:
        assert torch.equal(m, means[0])
    ref = per.mean().item()
    assert abs(means[0].item() - ref) <= 1e-6 * abs(ref)


@pytest.mark.parametrize("unroll,waves", [(1, 4), (2, 4), (4, 4), (8, 4), (16, 4), (1, 16), (2, 16),
                                          (4, 16), (8, 16)])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vocab", [(13, 100), (40, 517), (37, 1000), (70, 4099), (9, 30001)])
def test_wave_kernel_shapes(unroll, waves, dtype, rows, vocab):
    """Every instantiated one-wave-per-row kernel shape (chunks per lane per batch,
    waves per workgroup) on ragged row counts and unaligned rows."""
    z = rand_logits(rows * 3 + vocab, rows, vocab, dtype, std=2.0)
    t = lce_synth.targets(rows + 1, rows, vocab)
    with forced_env(LCE_PATH="wave", LCE_UNROLL=unroll, LCE_WAVES_PER_BLOCK=waves):
        check_xent(z, t, dtype, f"wave U{unroll} W{waves} {dtype} {rows}x{vocab}")
