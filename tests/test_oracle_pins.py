"""Pins for the fp64 oracle, none of which reuses the oracle's own arithmetic.

The pages print no loss value for any input, so the oracle is pinned by what the
mathematics fixes: closed forms, invariants, 40-digit brute force on tiny shapes,
and an independent library routine.  Each test names the slip it would catch.
"""
import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np
import pytest

import lce_synth

LN = math.log


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
@pytest.mark.parametrize("vocab", [1, 2, 3, 7, 4096, 131072])
@pytest.mark.parametrize("c", [0.0, 37.5, -1000.0])
def test_uniform_logits_give_ln_vocab(oracle_mod, dtype, vocab, c):
    """All logits equal to c: loss = ln(vocab) for every target (catches a dropped
    or sign-flipped -z_t term, a missing max shift at c=-1000, log base slips)."""
    rows = 3 if vocab > 4096 else 9
    if dtype == "f32":
        z = np.full((rows, vocab), c, dtype=np.float32)
    elif dtype == "f64":
        z = np.full((rows, vocab), c, dtype=np.float64)
    else:  # 0.0, 37.5 and -1000.0 are all exact bf16 values
        z = (np.full((rows, vocab), c, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    t = _rng(vocab).integers(0, vocab, rows)
    loss = oracle_mod.xent_rows(z, t, dtype=dtype)
    assert np.allclose(loss, LN(vocab), rtol=0, atol=1e-12)
    assert oracle_mod.xent(z, t, "mean", dtype=dtype) == pytest.approx(LN(vocab), abs=1e-12)


@pytest.mark.parametrize("vocab", [2, 5, 4096])
@pytest.mark.parametrize("a", [0.0, 1.0, 5.0, 20.0, 50.0, 1000.0])
def test_dominant_target(oracle_mod, vocab, a):
    """z_t = a, all other logits 0: loss = ln(1 + (V-1) e^-a), -> 0 as a grows
    (catches an off-by-one target index and a wrong-sign exponent)."""
    rows = 4
    z = np.zeros((rows, vocab))
    t = np.array([0, vocab - 1, vocab // 2, 1 % vocab])
    z[np.arange(rows), t] = a
    want = math.log1p((vocab - 1) * math.exp(-a))
    got = oracle_mod.xent_rows(z, t)
    # m + ln(s) - z_t cancels, leaving a few ulp of |a|; the sequential fp64 sum of
    # V terms adds at most about V * 2^-53 to ln(s)
    atol = 8 * max(1.0, a) * 2.0 ** -52 + vocab * 2.0 ** -53
    assert np.allclose(got, want, rtol=1e-12, atol=atol)
    if a == 1000.0:
        assert np.all(got == 0.0)


@pytest.mark.parametrize("d", [-40.0, -3.5, -1e-3, 0.0, 0.25, 7.0, 40.0])
def test_two_classes_is_softplus(oracle_mod, d):
    """V = 2: loss = softplus(z_other - z_t) = ln(1 + e^d)."""
    z = np.array([[1.5, 1.5 + d], [1.5 + d, 1.5]])
    t = np.array([0, 1])
    want = max(d, 0.0) + math.log1p(math.exp(-abs(d)))
    assert np.allclose(oracle_mod.xent_rows(z, t), want, rtol=1e-13, atol=1e-15)


def test_single_class_is_zero(oracle_mod):
    z = np.array([[3.0], [-7.25], [0.0]])
    assert np.all(oracle_mod.xent_rows(z, np.zeros(3, dtype=np.int64)) == 0.0)


# ---------------------------------------------------------------- invariants

def test_row_shift_invariance(oracle_mod):
    """Adding a constant to a row leaves its loss unchanged.  Logits on a 2^-8
    grid with |z| < 8 and integer shifts |c| <= 2^15 stay exact in fp32."""
    rng = _rng(7)
    rows, vocab = 16, 513
    z = np.round(rng.uniform(-8, 8, (rows, vocab)) * 256) / 256
    c = rng.integers(-2 ** 15, 2 ** 15, rows).astype(np.float64)
    t = rng.integers(0, vocab, rows)
    base = oracle_mod.xent_rows(z.astype(np.float32), t)
    shifted = oracle_mod.xent_rows((z + c[:, None]).astype(np.float32), t)
    assert np.allclose(base, shifted, rtol=0, atol=1e-10)


def test_permutation_invariance(oracle_mod):
    """Permuting columns together with the target leaves the loss unchanged; permuting
    rows permutes the losses (catches row/column stride mix-ups)."""
    rng = _rng(11)
    rows, vocab = 12, 301
    z = rng.normal(size=(rows, vocab))
    t = rng.integers(0, vocab, rows)
    perm = rng.permutation(vocab)
    inv = np.argsort(perm)
    zp = z[:, perm]                      # new column j holds old column perm[j]
    tp = inv[t]
    assert np.allclose(oracle_mod.xent_rows(z, t), oracle_mod.xent_rows(zp, tp), rtol=1e-13)
    rp = rng.permutation(rows)
    assert np.allclose(oracle_mod.xent_rows(z, t)[rp], oracle_mod.xent_rows(z[rp], t[rp]),
                       rtol=0, atol=0)


def test_megatron_layout_is_row_view(oracle_mod):
    """[seq, batch, vocab] with row = s*batch + b gives the [seq*batch, vocab] losses."""
    rng = _rng(3)
    z = rng.normal(size=(5, 3, 64)).astype(np.float32)
    t = rng.integers(0, 64, (5, 3))
    a = oracle_mod.xent_rows(z, t)
    b = oracle_mod.xent_rows(z.reshape(15, 64), t.reshape(15))
    assert a.shape == (5, 3)
    assert np.array_equal(a.reshape(15), b)


# ---------------------------------------------------------------- brute force

def _brute(z_row, t):
    """-ln(e^{z_t} / sum_j e^{z_j}) at 40 digits, no max shift."""
    getcontext().prec = 40
    zs = [Decimal(float(v)) for v in z_row]
    den = sum(v.exp() for v in zs)
    return float(-((zs[t].exp() / den).ln()))


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny(oracle_mod, seed):
    rng = _rng(100 + seed)
    rows = int(rng.integers(1, 9))
    vocab = int(rng.integers(1, 17))
    z = rng.uniform(-20, 20, (rows, vocab))
    t = rng.integers(0, vocab, rows)
    want = np.array([_brute(z[i], int(t[i])) for i in range(rows)])
    assert np.allclose(oracle_mod.xent_rows(z, t), want, rtol=0, atol=1e-13)


def test_matches_library_cross_entropy(oracle_mod):
    """Independent library routine: torch CPU fp64 cross_entropy."""
    torch = pytest.importorskip("torch")
    rng = _rng(5)
    for rows, vocab in [(64, 1000), (7, 4096), (33, 3)]:
        z = rng.normal(scale=3.0, size=(rows, vocab))
        t = rng.integers(0, vocab, rows)
        ref = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(t),
                                                reduction="none").numpy()
        assert np.allclose(oracle_mod.xent_rows(z, t), ref, rtol=1e-12, atol=1e-12)
        refm = torch.nn.functional.cross_entropy(torch.from_numpy(z), torch.from_numpy(t)).item()
        assert oracle_mod.xent(z, t, "mean") == pytest.approx(refm, rel=1e-12)


# ---------------------------------------------------------------- mean and contract edges

def test_mean_is_average_of_tokens(oracle_mod):
    rng = _rng(9)
    z = rng.normal(size=(257, 99))
    t = rng.integers(0, 99, 257)
    per = oracle_mod.xent_rows(z, t)
    assert oracle_mod.mean(per) == pytest.approx(math.fsum(per) / per.size, rel=1e-13)


def test_empty_and_invalid(oracle_mod):
    z = np.zeros((0, 16), dtype=np.float32)
    assert oracle_mod.xent_rows(z, np.zeros(0, dtype=np.int64)).shape == (0,)
    assert math.isnan(oracle_mod.xent(z, np.zeros(0, dtype=np.int64), "mean"))
    z = np.zeros((4, 16), dtype=np.float32)
    got = oracle_mod.xent_rows(z, np.array([0, -1, 16, 15]))
    assert not math.isnan(got[0]) and not math.isnan(got[3])
    assert math.isnan(got[1]) and math.isnan(got[2])
    zn = np.zeros((2, 8))
    zn[1, 3] = np.nan
    got = oracle_mod.xent_rows(zn, np.array([0, 0]))
    assert got[0] == pytest.approx(LN(8)) and math.isnan(got[1])


# ---------------------------------------------------------------- bf16 decode and RNE

def test_bf16_decode_patterns(oracle_mod):
    """0x3F80 = 1.0, 0xC000 = -2.0, 0x4216 = 37.5 -- through the C decoder (V = 2
    softplus) and the Python widening used by the fused path."""
    bits = np.array([[0x3F80, 0xC000], [0xC000, 0x4216]], dtype=np.uint16)
    got = oracle_mod.xent_rows(bits, np.array([0, 1]))
    assert got[0] == pytest.approx(math.log1p(math.exp(-3.0)), rel=1e-14)
    assert got[1] == pytest.approx(math.log1p(math.exp(-39.5)), rel=1e-14)
    w = oracle_mod.bf16_bits_to_f64(np.array([0x3F80, 0xC000, 0x4216, 0x0001, 0x7F7F], np.uint16))
    assert list(w[:3]) == [1.0, -2.0, 37.5]
    assert w[3] == 2.0 ** -133
    assert w[4] == (2 - 2 ** -7) * 2.0 ** 127


def test_generator_rounds_to_nearest_even():
    vals = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, -2.0,
                     1 - 2 ** -9], dtype=np.float32)
    got = lce_synth.f32_to_bf16_bits(vals)
    assert list(got) == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC000, 0x3F80]


# ---------------------------------------------------------------- fused path

def test_fused_zero_activations_give_ln_vocab(oracle_mod):
    rng = _rng(21)
    V, H = 37, 24
    x = np.zeros((5, H), dtype=np.uint16)
    w = lce_synth.f32_to_bf16_bits(rng.normal(size=(V, H)).astype(np.float32))
    got = oracle_mod.fused_linear_xent_rows(x, w, rng.integers(0, V, 5))
    assert np.allclose(got, LN(V), rtol=0, atol=1e-13)


def test_fused_identity_head_is_plain_ce(oracle_mod):
    """W = I (vocab = hidden): fused CE of x equals plain CE of x."""
    rng = _rng(22)
    H = 40
    x = lce_synth.f32_to_bf16_bits(rng.normal(size=(6, H)).astype(np.float32))
    eye = lce_synth.f32_to_bf16_bits(np.eye(H, dtype=np.float32))
    t = rng.integers(0, H, 6)
    assert np.allclose(oracle_mod.fused_linear_xent_rows(x, eye, t),
                       oracle_mod.xent_rows(x, t, dtype="bf16"), rtol=0, atol=1e-14)


def test_fused_brute_force_tiny(oracle_mod):
    """Non-square tiny GEMM by exact rational triple loop, then 40-digit CE
    (catches a transposed operand or a swapped hidden/vocab axis)."""
    rng = _rng(23)
    T, H, V = 3, 5, 7
    x = lce_synth.f32_to_bf16_bits(rng.normal(size=(T, H)).astype(np.float32))
    w = lce_synth.f32_to_bf16_bits(rng.normal(size=(V, H)).astype(np.float32))
    t = rng.integers(0, V, T)
    xf = [[Fraction(float(v)) for v in r] for r in oracle_mod.bf16_bits_to_f64(x)]
    wf = [[Fraction(float(v)) for v in r] for r in oracle_mod.bf16_bits_to_f64(w)]
    want = []
    for i in range(T):
        z = [float(sum(xf[i][k] * wf[j][k] for k in range(H))) for j in range(V)]
        want.append(_brute(z, int(t[i])))
    got = oracle_mod.fused_linear_xent_rows(x, w, t)
    assert np.allclose(got, want, rtol=0, atol=1e-12)
    assert oracle_mod.fused_linear_xent(x, w, t, "mean") == pytest.approx(np.mean(want), abs=1e-12)


# ---------------------------------------------------------------- statistical sanity of inputs + oracle

@pytest.mark.parametrize("name,rows,expect", [
    ("ce_f32_16384x4096_mean", 1024, LN(4096) + 0.5),
    ("megatron_bf16_2048x4x4096_none", 1024, LN(4096) + 0.5),
    ("megatron_bf16_2048x4x131072_none", 64, LN(131072) + 2.0),
])
def test_mean_loss_near_ln_vocab_plus_half_variance(oracle_mod, name, rows, expect):
    """For i.i.d. N(0, s^2) logits the mean loss is about ln V + s^2/2 (catches a
    generator slip such as variance for std, or a wrong target stream)."""
    w = lce_synth.WORKLOADS[name]
    got = oracle_mod.xent(w.logits(0, rows), w.target(0, rows), "mean", dtype=w.dtype)
    assert got == pytest.approx(expect, abs=0.05)


def test_fused_workload_statistics(oracle_mod):
    """The fused workload's logits z = x W^T have variance ~ hidden * 0.02^2; on a
    vocab slice of 8192 heads the mean loss is about ln 8192 + 4096 * 0.0004 / 2."""
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    x = w.x(0, 16)
    head = w.weight(0, 8192)
    t = lce_synth.targets(77, 16, 8192)
    got = oracle_mod.fused_linear_xent(x, head, t, "mean")
    assert got == pytest.approx(LN(8192) + 4096 * 0.02 ** 2 / 2, abs=0.1)


# ---------------------------------------------------------------- vocab shards

def _shard_bounds(vocab, shards, rng):
    """Uneven split of [0, vocab) into `shards` non-empty consecutive ranges."""
    cuts = np.sort(rng.choice(np.arange(1, vocab), size=shards - 1, replace=False)) if shards > 1 else []
    edges = [0, *[int(c) for c in cuts], vocab]
    return list(zip(edges[:-1], edges[1:]))


def test_partial_uniform_shard(oracle_mod):
    z = np.full((3, 50), 2.5)
    t = np.array([10, 70, 59])
    q = oracle_mod.xent_partial(z, t, vocab_start=10)  # columns [10, 60)
    assert np.all(q[:, 0] == 2.5) and np.allclose(q[:, 1], 50.0, rtol=1e-15)
    assert q[0, 2] == 2.5 and math.isnan(q[1, 2]) and q[2, 2] == 2.5


@pytest.mark.parametrize("seed", range(4))
def test_partial_brute_force_tiny(oracle_mod, seed):
    """m is the exact shard maximum, m + ln s is the shard's log-sum-exp at 40 digits,
    and zt is the target's logit exactly when this shard holds the target."""
    rng = _rng(300 + seed)
    rows, shard, v0 = int(rng.integers(1, 7)), int(rng.integers(1, 13)), int(rng.integers(0, 20))
    z = rng.uniform(-30, 30, (rows, shard))
    t = rng.integers(0, v0 + shard + 5, rows)
    q = oracle_mod.xent_partial(z, t, vocab_start=v0)
    getcontext().prec = 40
    for i in range(rows):
        lse = float(sum(Decimal(float(v)).exp() for v in z[i]).ln())
        assert q[i, 0] == z[i].max()
        assert q[i, 0] + math.log(q[i, 1]) == pytest.approx(lse, abs=1e-13)
        if v0 <= t[i] < v0 + shard:
            assert q[i, 2] == z[i, t[i] - v0]
        else:
            assert math.isnan(q[i, 2])


def test_partial_matches_library_logsumexp(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = _rng(11)
    z = rng.normal(scale=4.0, size=(40, 3000))
    q = oracle_mod.xent_partial(z, np.zeros(40, dtype=np.int64), vocab_start=5)
    ref = torch.logsumexp(torch.from_numpy(z), dim=1).numpy()
    assert np.allclose(q[:, 0] + np.log(q[:, 1]), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("shards", [1, 2, 3, 7])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f64"])
def test_shard_merge_equals_whole_row(oracle_mod, shards, dtype):
    """Statistics of uneven vocab shards, merged, give the whole-row loss (a different
    computation: per-shard maxima and sums, then one rescaled sum)."""
    rng = _rng(400 + shards)
    rows, vocab = 33, 997
    f = rng.normal(scale=3.0, size=(rows, vocab)).astype(np.float32)
    z = {"f32": f, "f64": f.astype(np.float64), "bf16": lce_synth.f32_to_bf16_bits(f)}[dtype]
    t = rng.integers(0, vocab, rows)
    t[0], t[1] = -1, vocab  # invalid targets: NaN either way
    parts = np.stack([oracle_mod.xent_partial(np.ascontiguousarray(z[:, a:b]), t, a, dtype=dtype)
                      for a, b in _shard_bounds(vocab, shards, rng)])
    got = oracle_mod.xent_merge(parts, t, vocab)
    want = oracle_mod.xent_rows(z, t, dtype=dtype)
    assert np.array_equal(np.isnan(got), np.isnan(want)) and np.isnan(got[:2]).all()
    assert np.allclose(got[2:], want[2:], rtol=0, atol=1e-12)
    # exactly one shard reports each valid target
    held = (~np.isnan(parts[:, 2:, 2])).sum(axis=0)
    assert np.all(held == 1)


def test_merge_ignores_shard_order(oracle_mod):
    rng = _rng(12)
    rows, vocab = 20, 500
    z = rng.normal(scale=5.0, size=(rows, vocab))
    t = rng.integers(0, vocab, rows)
    parts = np.stack([oracle_mod.xent_partial(np.ascontiguousarray(z[:, a:b]), t, a)
                      for a, b in _shard_bounds(vocab, 5, rng)])
    a = oracle_mod.xent_merge(parts, t, vocab)
    b = oracle_mod.xent_merge(parts[::-1].copy(), t, vocab)
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_shard_of_minus_infinity_adds_nothing(oracle_mod):
    """A shard whose logits are all -inf contributes e^-inf = 0: (-inf, 0), and the
    merged loss equals that of the row without it."""
    rng = _rng(13)
    z = rng.normal(size=(4, 30))
    z[:, 10:20] = -np.inf
    t = np.array([0, 5, 25, 29])
    q = oracle_mod.xent_partial(np.ascontiguousarray(z[:, 10:20]), t, 10)
    assert np.all(q[:, 0] == -np.inf) and np.all(q[:, 1] == 0.0) and np.isnan(q[:, 2]).all()
    parts = np.stack([oracle_mod.xent_partial(np.ascontiguousarray(z[:, a:b]), t, a)
                      for a, b in ((0, 10), (10, 20), (20, 30))])
    assert np.allclose(oracle_mod.xent_merge(parts, t, 30), oracle_mod.xent_rows(z, t), atol=1e-13)


# ---------------------------------------------------------------- gradient

def test_bwd_uniform_logits_closed_form(oracle_mod):
    """Equal logits: softmax is 1/V, so the gradient is g (1/V - [j == t])."""
    V = 40
    z = np.full((3, V), -3.0)
    t = np.array([0, 17, 39])
    g = np.array([1.0, -2.5, 0.25])
    d = oracle_mod.xent_bwd(z, t, g, "none")
    want = g[:, None] * (np.full((3, V), 1.0 / V) - np.eye(V)[t])
    assert np.allclose(d, want, rtol=0, atol=1e-15)


def test_bwd_rows_sum_to_zero_and_mean_scaling(oracle_mod):
    rng = _rng(21)
    z = rng.normal(scale=3.0, size=(50, 777))
    t = rng.integers(0, 777, 50)
    d = oracle_mod.xent_bwd(z, t, 2.0, "mean")
    assert np.allclose(d.sum(axis=1), 0.0, atol=1e-15)
    d1 = oracle_mod.xent_bwd(z, t, np.full(50, 2.0 / 50), "none")
    assert np.allclose(d, d1, rtol=1e-15, atol=0)


def test_bwd_matches_finite_differences_of_the_loss(oracle_mod):
    """Central differences of the (separately pinned) forward oracle."""
    rng = _rng(22)
    rows, V, h = 3, 12, 1e-6
    z = rng.normal(scale=2.0, size=(rows, V))
    t = rng.integers(0, V, rows)
    g = rng.normal(size=rows)
    d = oracle_mod.xent_bwd(z, t, g, "none")
    for i in range(rows):
        for j in range(V):
            zp, zm = z.copy(), z.copy()
            zp[i, j] += h
            zm[i, j] -= h
            fd = (oracle_mod.xent_rows(zp, t)[i] - oracle_mod.xent_rows(zm, t)[i]) / (2 * h)
            assert g[i] * fd == pytest.approx(d[i, j], abs=1e-8)


def test_bwd_matches_library_autograd(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = _rng(23)
    for dt, rows, V in (("f64", 30, 2000), ("f32", 9, 4097), ("bf16", 5, 300)):
        f = rng.normal(scale=4.0, size=(rows, V)).astype(np.float32)
        z = {"f64": f.astype(np.float64), "f32": f, "bf16": lce_synth.f32_to_bf16_bits(f)}[dt]
        z64 = oracle_mod.bf16_bits_to_f64(z) if dt == "bf16" else z.astype(np.float64)
        t = rng.integers(0, V, rows)
        zt = torch.from_numpy(z64).requires_grad_(True)
        torch.nn.functional.cross_entropy(zt, torch.from_numpy(t)).mul(3.0).backward()
        d = oracle_mod.xent_bwd(z, t, 3.0, "mean", dtype=dt)
        assert np.allclose(d, zt.grad.numpy(), rtol=0, atol=1e-14)


def test_bwd_invalid_target_rows_are_nan(oracle_mod):
    z = np.zeros((3, 5))
    d = oracle_mod.xent_bwd(z, np.array([0, -1, 5]), 1.0, "mean")
    assert np.isfinite(d[0]).all() and np.isnan(d[1:]).all()


# ---------------------------------------------------------------- per-sequence log-prob sums

def test_logprob_sums_brute_force_tiny(oracle_mod):
    """Sums of 40-digit log-softmax values of an exactly computed tiny GEMM, batch != seq."""
    rng = _rng(31)
    batch, seq, hidden, vocab = 3, 4, 8, 5
    xf = rng.normal(size=(batch * seq, hidden)).astype(np.float32)
    wf = rng.normal(size=(vocab, hidden)).astype(np.float32)
    xb, wb = lce_synth.f32_to_bf16_bits(xf), lce_synth.f32_to_bf16_bits(wf)
    x, w = oracle_mod.bf16_bits_to_f64(xb), oracle_mod.bf16_bits_to_f64(wb)
    t = rng.integers(0, vocab, batch * seq)
    getcontext().prec = 40
    want = []
    for b in range(batch):
        acc = Decimal(0)
        for s in range(seq):
            r = b * seq + s
            z = [sum(Fraction(float(x[r, k])) * Fraction(float(w[j, k])) for k in range(hidden))
                 for j in range(vocab)]
            zd = [Decimal(v.numerator) / Decimal(v.denominator) for v in z]
            acc += zd[t[r]] - sum(v.exp() for v in zd).ln()
        want.append(float(acc))
    got = oracle_mod.fused_linear_logprob_sums(xb, wb, t, batch, seq)
    assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_logprob_sums_closed_forms(oracle_mod):
    """x = 0: every token's log-prob is -ln V; seq = 1: minus the per-token loss."""
    rng = _rng(32)
    wb = lce_synth.f32_to_bf16_bits(rng.normal(size=(50, 16)).astype(np.float32))
    t = rng.integers(0, 50, 12)
    zero = np.zeros((12, 16), dtype=np.uint16)
    assert np.allclose(oracle_mod.fused_linear_logprob_sums(zero, wb, t, 2, 6), -6 * math.log(50),
                       rtol=0, atol=1e-12)
    xb = lce_synth.f32_to_bf16_bits(rng.normal(size=(12, 16)).astype(np.float32))
    assert np.allclose(oracle_mod.fused_linear_logprob_sums(xb, wb, t, 12, 1),
                       -oracle_mod.fused_linear_xent_rows(xb, wb, t), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- fused linear + JSD

def _bf16(rng, shape, scale):
    return lce_synth.f32_to_bf16_bits((rng.normal(size=shape) * scale).astype(np.float32))


def test_jsd_of_identical_distributions_is_zero(oracle_mod):
    rng = _rng(41)
    x, w = _bf16(rng, (10, 32), 1.0), _bf16(rng, (300, 32), 0.3)
    for beta in (0.5, 0.2, 0.9):
        assert np.all(np.abs(oracle_mod.fused_linear_jsd_rows(x, w, x, w, beta)) <= 1e-14)


def test_jsd_of_disjoint_point_masses(oracle_mod):
    """Student all on class 0, teacher all on class 1: each KL term is -ln(beta) or
    -ln(1 - beta), so JSD = -beta ln beta - (1 - beta) ln(1 - beta) (ln 2 at 0.5)."""
    x = lce_synth.f32_to_bf16_bits(np.ones((3, 8), np.float32))
    ws = np.zeros((4, 8), np.float32)
    wt = np.zeros((4, 8), np.float32)
    ws[0], wt[1] = 100.0, 100.0          # logit 800 vs 0: the other classes vanish in fp64
    ws_b, wt_b = lce_synth.f32_to_bf16_bits(ws), lce_synth.f32_to_bf16_bits(wt)
    for beta in (0.5, 0.25):
        want = -beta * math.log(beta) - (1 - beta) * math.log(1 - beta)
        got = oracle_mod.fused_linear_jsd_rows(x, ws_b, x, wt_b, beta)
        assert np.allclose(got, want, rtol=0, atol=1e-12)


def test_jsd_symmetric_and_bounded_at_half(oracle_mod):
    rng = _rng(42)
    xs, xt = _bf16(rng, (20, 64), 1.0), _bf16(rng, (20, 64), 1.0)
    ws, wt = _bf16(rng, (500, 64), 0.4), _bf16(rng, (500, 64), 0.4)
    a = oracle_mod.fused_linear_jsd_rows(xs, ws, xt, wt, 0.5)
    b = oracle_mod.fused_linear_jsd_rows(xt, wt, xs, ws, 0.5)
    assert np.allclose(a, b, rtol=0, atol=1e-14)
    assert np.all(a >= 0.0) and np.all(a <= math.log(2) + 1e-15)


def test_jsd_brute_force_tiny(oracle_mod):
    """Exact rational GEMMs, 40-digit softmaxes and logarithms, beta = 0.3."""
    rng = _rng(43)
    T, H, V, beta = 3, 6, 5, Decimal("0.3")
    xs, xt = _bf16(rng, (T, H), 1.0), _bf16(rng, (T, H), 1.0)
    ws, wt = _bf16(rng, (V, H), 1.0), _bf16(rng, (V, H), 1.0)
    getcontext().prec = 40

    def logits(x, w, i):
        xf, wf = oracle_mod.bf16_bits_to_f64(x), oracle_mod.bf16_bits_to_f64(w)
        out = []
        for j in range(V):
            f = sum(Fraction(float(xf[i, k])) * Fraction(float(wf[j, k])) for k in range(H))
            out.append(Decimal(f.numerator) / Decimal(f.denominator))
        return out

    want = []
    for i in range(T):
        zs, zt = logits(xs, ws, i), logits(xt, wt, i)
        es, et = [v.exp() for v in zs], [v.exp() for v in zt]
        P = [v / sum(es) for v in es]
        Q = [v / sum(et) for v in et]
        M = [beta * p + (1 - beta) * q for p, q in zip(P, Q)]
        kp = sum(p * (p / m).ln() for p, m in zip(P, M))
        kq = sum(q * (q / m).ln() for q, m in zip(Q, M))
        want.append(float(beta * kp + (1 - beta) * kq))
    got = oracle_mod.fused_linear_jsd_rows(xs, ws, xt, wt, 0.3)
    assert np.allclose(got, want, rtol=0, atol=1e-13)


def test_jsd_matches_library_kl_div(oracle_mod):
    """torch kl_div (library routine, fp64) on the same fp64 logits."""
    torch = pytest.importorskip("torch")
    rng = _rng(44)
    xs, xt = _bf16(rng, (16, 48), 1.0), _bf16(rng, (16, 48), 1.0)
    ws, wt = _bf16(rng, (700, 48), 0.5), _bf16(rng, (700, 48), 0.5)
    f = oracle_mod.bf16_bits_to_f64
    lp = torch.log_softmax(torch.from_numpy(f(xs) @ f(ws).T), dim=1)
    lq = torch.log_softmax(torch.from_numpy(f(xt) @ f(wt).T), dim=1)
    beta = 0.5
    lm = torch.log(beta * lp.exp() + (1 - beta) * lq.exp())
    kl = torch.nn.functional.kl_div
    ref = beta * kl(lm, lp, reduction="batchmean", log_target=True) + \
        (1 - beta) * kl(lm, lq, reduction="batchmean", log_target=True)
    assert oracle_mod.fused_linear_jsd(xs, ws, xt, wt, beta, "mean") == pytest.approx(ref.item(), abs=1e-13)


# ---------------------------------------------------------------- fused-linear gradients

def _bf16_of(a):
    return lce_synth.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def test_fused_bwd_zero_activations_closed_form(oracle_mod):
    """x = 0: softmax is 1/V, so dx_i = g_i (mean_v W_v - W_{t_i}) and dW = 0 (catches a
    transposed product, a dropped one-hot, a wrong scale)."""
    rng = _rng(41)
    T, H, V = 5, 16, 37
    wb = _bf16_of(rng.normal(size=(V, H)))
    w = oracle_mod.bf16_bits_to_f64(wb)
    xb = np.zeros((T, H), dtype=np.uint16)
    t = rng.integers(0, V, T)
    g = rng.normal(size=T)
    dx, dw = oracle_mod.fused_linear_xent_bwd(xb, wb, t, g, "none")
    want = g[:, None] * (w.mean(axis=0)[None, :] - w[t])
    assert np.allclose(dx, want, rtol=0, atol=1e-14)
    assert np.array_equal(dw, np.zeros_like(dw))


def test_fused_bwd_matches_finite_differences(oracle_mod):
    """Central differences of the separately pinned row oracle on fp64 logits x W^T, for
    every entry of a small x and W, with a non-square head and mean reduction."""
    rng = _rng(42)
    T, H, V, h = 3, 4, 6, 1e-6
    xb, wb = _bf16_of(rng.normal(size=(T, H))), _bf16_of(rng.normal(size=(V, H)))
    x, w = oracle_mod.bf16_bits_to_f64(xb), oracle_mod.bf16_bits_to_f64(wb)
    t = rng.integers(0, V, T)
    dx, dw = oracle_mod.fused_linear_xent_bwd(xb, wb, t, 1.7, "mean")

    def loss(xx, ww):
        return 1.7 * oracle_mod.xent_rows(xx @ ww.T, t, dtype="f64").mean()

    for i in range(T):
        for k in range(H):
            xp, xm = x.copy(), x.copy()
            xp[i, k] += h
            xm[i, k] -= h
            assert (loss(xp, w) - loss(xm, w)) / (2 * h) == pytest.approx(dx[i, k], abs=1e-8)
    for v in range(V):
        for k in range(H):
            wp, wm = w.copy(), w.copy()
            wp[v, k] += h
            wm[v, k] -= h
            assert (loss(x, wp) - loss(x, wm)) / (2 * h) == pytest.approx(dw[v, k], abs=1e-8)


def test_fused_bwd_matches_library_autograd(oracle_mod):
    torch = pytest.importorskip("torch")
    rng = _rng(43)
    T, H, V = 70, 24, 301
    xb, wb = _bf16_of(rng.normal(size=(T, H))), _bf16_of(rng.normal(scale=0.3, size=(V, H)))
    t = rng.integers(0, V, T)
    g = rng.normal(size=T)
    xt = torch.from_numpy(oracle_mod.bf16_bits_to_f64(xb)).requires_grad_(True)
    wt = torch.from_numpy(oracle_mod.bf16_bits_to_f64(wb)).requires_grad_(True)
    per = torch.nn.functional.cross_entropy(xt @ wt.T, torch.from_numpy(t), reduction="none")
    (per * torch.from_numpy(g)).sum().backward()
    dx, dw = oracle_mod.fused_linear_xent_bwd(xb, wb, t, g, "none")
    assert np.allclose(dx, xt.grad.numpy(), rtol=0, atol=1e-13)
    assert np.allclose(dw, wt.grad.numpy(), rtol=0, atol=1e-13)


def test_fused_bwd_invariants(oracle_mod):
    """Rows of dZ sum to 0, so the rows of dW sum to 0; mean = none with grad / T; token
    blocks of any size give the same result; a bad target poisons its dx row and dW."""
    rng = _rng(44)
    T, H, V = 130, 8, 50
    xb, wb = _bf16_of(rng.normal(size=(T, H))), _bf16_of(rng.normal(size=(V, H)))
    t = rng.integers(0, V, T)
    dx, dw = oracle_mod.fused_linear_xent_bwd(xb, wb, t, 2.0, "mean")
    assert np.allclose(dw.sum(axis=0), 0.0, atol=1e-13)
    dx1, dw1 = oracle_mod.fused_linear_xent_bwd(xb, wb, t, np.full(T, 2.0 / T), "none")
    assert np.allclose(dx, dx1, rtol=1e-14, atol=0) and np.allclose(dw, dw1, rtol=1e-14, atol=0)
    dx2, dw2 = oracle_mod.fused_linear_xent_grads(xb, wb, t, np.full(T, 2.0 / T), block=7)
    assert np.allclose(dx, dx2, rtol=1e-13, atol=0) and np.allclose(dw, dw2, rtol=1e-13, atol=1e-16)
    t[3] = V
    dx3, dw3 = oracle_mod.fused_linear_xent_bwd(xb, wb, t, 2.0, "mean")
    assert np.isnan(dx3[3]).all() and np.isfinite(np.delete(dx3, 3, axis=0)).all()
    assert np.isnan(dw3).all()


def test_fused_dw_rows_match_full_gradient_and_autograd(oracle_mod):
    """Selected head rows of dW (any order, repeats, the targets' rows among them) equal the
    rows of the full fp64 dW, and torch autograd's, for several token block sizes; their dZ
    columns sum over the head rows to the full dZ's (catches a dropped one-hot, a column
    taken from the wrong row, a block boundary lost)."""
    torch = pytest.importorskip("torch")
    rng = _rng(45)
    T, H, V = 67, 12, 211
    xb, wb = _bf16_of(rng.normal(size=(T, H))), _bf16_of(rng.normal(scale=0.4, size=(V, H)))
    t = rng.integers(0, V, T)
    g = rng.normal(size=T)
    sel = np.array([t[5], 0, V - 1, 17, t[5], t[60], 100])
    _, dw = oracle_mod.fused_linear_xent_grads(xb, wb, t, g)
    xt = torch.from_numpy(oracle_mod.bf16_bits_to_f64(xb))
    wt = torch.from_numpy(oracle_mod.bf16_bits_to_f64(wb)).requires_grad_(True)
    per = torch.nn.functional.cross_entropy(xt @ wt.T, torch.from_numpy(t), reduction="none")
    (per * torch.from_numpy(g)).sum().backward()
    for block in (1, 16, 128):
        rows, dz = oracle_mod.fused_linear_xent_dw_rows(xb, wb, t, g, sel, block=block)
        assert rows.shape == (sel.size, H) and dz.shape == (T, sel.size)
        assert np.allclose(rows, dw[sel], rtol=0, atol=1e-13)
        assert np.allclose(rows, wt.grad.numpy()[sel], rtol=0, atol=1e-13)
    _, dz_all = oracle_mod.fused_linear_xent_dw_rows(xb, wb, t, g, np.arange(V))
    assert np.allclose(dz_all.sum(axis=1), 0.0, atol=1e-13)


def test_fused_dw_rows_edge_cases(oracle_mod):
    """x = 0 gives dW = 0; an invalid target makes every selected row NaN; an empty
    selection is an empty result; a row outside the head is refused."""
    rng = _rng(46)
    T, H, V = 9, 5, 13
    wb = _bf16_of(rng.normal(size=(V, H)))
    t = rng.integers(0, V, T)
    g = np.ones(T)
    rows, _ = oracle_mod.fused_linear_xent_dw_rows(np.zeros((T, H), np.uint16), wb, t, g, [0, 4, 12])
    assert np.array_equal(rows, np.zeros((3, H)))
    xb = _bf16_of(rng.normal(size=(T, H)))
    bad = t.copy()
    bad[2] = -1
    rows, _ = oracle_mod.fused_linear_xent_dw_rows(xb, wb, bad, g, [1, 7])
    assert np.isnan(rows).all()
    rows, dz = oracle_mod.fused_linear_xent_dw_rows(xb, wb, t, g, np.array([], dtype=np.int64))
    assert rows.shape == (0, H) and dz.shape == (T, 0)
    with pytest.raises(ValueError):
        oracle_mod.fused_linear_xent_dw_rows(xb, wb, t, g, [V])
