"""Vocab split across devices, emulated on one GPU: per-shard statistics
(lce_xent_partial_fwd) and their merge (lce_xent_merge), through the C ABI, against
the fp64 oracle.

Each shard is its own contiguous [tokens, shard_vocab] tensor, as on a device of a
vocab-parallel group; stacking the shards' [tokens, 3] outputs stands in for the
all-gather.  Tolerances are those of the row cross-entropy: the shard maximum and the
target logit are input values and must match exactly; ln s and the losses within 1e-4,
the mean within 1e-5 relative.
"""
import math

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


def _bounds(vocab, shards, seed):
    rng = np.random.default_rng(seed)
    cuts = sorted(rng.choice(np.arange(1, vocab), size=shards - 1, replace=False)) if shards > 1 else []
    edges = [0, *[int(c) for c in cuts], vocab]
    return list(zip(edges[:-1], edges[1:]))


def _check_stats(got, want, label):
    got = got.astype(np.float64)
    assert np.array_equal(got[:, 0], want[:, 0]), f"{label}: shard maxima differ"
    assert np.array_equal(np.isnan(got[:, 2]), np.isnan(want[:, 2])), f"{label}: target ownership"
    held = ~np.isnan(want[:, 2])
    assert np.array_equal(got[held, 2], want[held, 2]), f"{label}: target logits differ"
    finite = np.isfinite(want[:, 0])
    err = np.abs(np.log(got[finite, 1]) - np.log(want[finite, 1]))
    assert err.max(initial=0.0) <= TOK_ABS, f"{label}: ln s error {err.max()}"
    assert np.all(got[~finite, 1] == 0.0)


@pytest.mark.parametrize("path", ["auto", "wave", "block", "split", "split_many"])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,shard,start", [(37, 1000, 0), (64, 4099, 12345), (5, 20001, 7),
                                              (130, 129, 999), (130, 128, 999), (1000, 512, 3584)])
def test_partial_matches_oracle(path, dtype, rows, shard, start):
    z = _logits(rows + shard, rows, shard, dtype)
    t = lce_synth.targets(rows, rows, start + shard + 50)  # some targets past this shard
    t[:3] = (start, start + shard - 1, -5)                 # both ends, and an invalid one
    env = {} if path == "auto" else {"LCE_PATH": path}
    if path == "split_many":  # many slices per row: more partials per merged row
        env = {"LCE_PATH": "split", "LCE_SPLITS": 37}
    with forced_env(**env):
        got = lce.xent_partial(to_dev(z), torch.from_numpy(t).cuda(), start)
    torch.cuda.synchronize()
    want = oracle.xent_partial(z, t, start, dtype=dtype)
    _check_stats(got.cpu().numpy(), want, f"{path} {dtype} {rows}x{shard}@{start}")


@pytest.mark.parametrize("shards", [1, 2, 3, 8])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sharded_loss_matches_oracle_and_whole_rows(shards, dtype):
    rows, vocab = 301, 9000
    z = _logits(17 + shards, rows, vocab, dtype)
    t = lce_synth.targets(18, rows, vocab)
    t[0], t[1] = -1, vocab
    td = torch.from_numpy(t).cuda()
    parts = torch.stack([lce.xent_partial(to_dev(np.ascontiguousarray(z[:, a:b])), td, a)
                         for a, b in _bounds(vocab, shards, shards)])
    per = lce.xent_merge(parts, td, vocab, "none")
    mean = lce.xent_merge(parts, td, vocab, "mean")
    whole = lce.xent(to_dev(z), td, "none")
    torch.cuda.synchronize()
    want = oracle.xent_rows(z, t, dtype=dtype)
    got = per.cpu().numpy().astype(np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    assert np.nanmax(np.abs(got - want)) <= TOK_ABS
    assert np.nanmax(np.abs(got - whole.cpu().numpy())) <= TOK_ABS
    assert math.isnan(mean.item())  # invalid targets make the mean NaN
    # mean over the valid rows only
    parts_v = parts[:, 2:].contiguous()
    mv = lce.xent_merge(parts_v, td[2:].contiguous(), vocab, "mean").item()
    wm = oracle.mean(want[2:])
    assert abs(mv - wm) <= MEAN_REL * abs(wm)


def test_merge_of_oracle_statistics():
    """The merge alone, on statistics computed by the oracle (rounded to fp32), against
    the oracle's merge of the same fp32 values; includes a shard of -inf only."""
    rows, vocab, shards = 200, 3000, 5
    z = _logits(21, rows, vocab, "f32", std=4.0)
    bounds = _bounds(vocab, shards, 5)
    a, b = bounds[2]
    z[:50, a:b] = -np.inf
    t = lce_synth.targets(22, rows, vocab)
    t[:50] = bounds[0][0]  # those rows' targets lie in the first shard
    st = np.stack([oracle.xent_partial(np.ascontiguousarray(z[:, a:b]), t, a) for a, b in bounds])
    st32 = st.astype(np.float32)
    got = lce.xent_merge(torch.from_numpy(st32).cuda(), torch.from_numpy(t).cuda(), vocab, "none")
    want = oracle.xent_merge(st32.astype(np.float64), t, vocab)
    assert np.max(np.abs(got.cpu().numpy() - want)) <= TOK_ABS
    assert np.max(np.abs(want - oracle.xent_rows(z, t))) <= 1e-5


@pytest.mark.parametrize("shards", [2, 8])
def test_headline_shape_split_over_shards(shards):
    """bf16 [2048, 4, 4096] per-token losses with the vocab split into equal shards."""
    w = lce_synth.WORKLOADS["megatron_bf16_2048x4x4096_none"]
    z = w.logits()
    t = w.target()
    td = torch.from_numpy(t).cuda()
    step = w.vocab // shards
    parts = torch.stack([lce.xent_partial(to_dev(np.ascontiguousarray(z[:, p * step:(p + 1) * step])),
                                          td, p * step) for p in range(shards)])
    per = lce.xent_merge(parts, td, w.vocab, "none").cpu().numpy().astype(np.float64)
    want = oracle.xent_rows(z, t, dtype="bf16")
    assert np.max(np.abs(per - want)) <= TOK_ABS


def test_repeated_merge_bitwise_identical():
    rows, vocab = 4096, 2048
    z = to_dev(_logits(31, rows, vocab, "bf16"))
    td = torch.from_numpy(lce_synth.targets(32, rows, vocab)).cuda()
    parts = torch.stack([lce.xent_partial(z[:, a:b].contiguous(), td, a)
                         for a, b in ((0, 700), (700, 1500), (1500, 2048))])
    first = lce.xent_merge(parts, td, vocab, "mean").clone()
    for _ in range(10):
        assert torch.equal(lce.xent_merge(parts, td, vocab, "mean"), first)


@pytest.mark.parametrize("seed", range(3))
def test_randomized_shards(seed):
    """Seeded random cases, 8 per seed: 1-400 rows, vocab log-uniform in [2, 60000) split at
    random into 1-7 shards, fp32 or bf16, scales 0.05 to 25, spikes 5 to 120 above the rest,
    -inf entries around finite targets, some invalid targets, any row path; each shard's
    statistics against the oracle's, and the merged losses against the whole-row oracle."""
    rng = np.random.default_rng(7900 + seed)
    for case in range(8):
        dtype = str(rng.choice(["f32", "bf16"]))
        rows = int(rng.integers(1, 401))
        vocab = max(2, int(np.exp(rng.uniform(np.log(2.0), np.log(60000.0)))))
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
        shards = int(rng.integers(1, min(7, vocab) + 1))
        path = str(rng.choice(["auto", "wave", "block", "split"]))
        env = {} if path == "auto" else {"LCE_PATH": path}
        label = f"seed {seed} case {case}: {dtype} {rows}x{vocab} std {std} {shards} shards {path}"
        td = torch.from_numpy(t.astype(np.int64)).cuda()
        parts = []
        for a, b in _bounds(vocab, shards, 31 * seed + case):
            zs = np.ascontiguousarray(host[:, a:b])
            with forced_env(**env):
                p = lce.xent_partial(to_dev(zs), td, a)
            torch.cuda.synchronize()
            _check_stats(p.cpu().numpy(), oracle.xent_partial(zs, t, a, dtype=dtype), f"{label} shard {a}:{b}")
            parts.append(p)
        per = lce.xent_merge(torch.stack(parts), td, vocab, "none")
        torch.cuda.synchronize()
        got = per.cpu().numpy().astype(np.float64)
        want = oracle.xent_rows(host, t, dtype=dtype)
        assert np.array_equal(np.isnan(got), np.isnan(want)), label
        assert np.nanmax(np.abs(got - want), initial=0.0) <= TOK_ABS, label
