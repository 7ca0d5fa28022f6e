"""Fused linear + generalized JSD (lce_fused_linear_jsd_fwd, through the C ABI) against
the fp64 oracle.

Tolerance: the logits are fp32 sums of exact bf16 products (as the fused cross-entropy),
each head's log-sum-exp carries a few fp32 ulps, and each divergence term is evaluated in
fp32 with the hardware exp2/log2.  Every term beta P ln(P/M) + (1 - beta) Q ln(Q/M) is
non-negative, so the vocab sum has no cancellation; the largest absolute error comes from
ln(P/M) at P close to M, about 1e-6 per unit of probability mass.  Required here: per
token |got - want| <= 1e-4 + 1e-3 * want, and the same bound for the batch mean.

At the page's shape (tokens 1024, hidden 4096, vocab 128256) the oracle checks a sample
of tokens, and the batch mean is checked against the same call's per-token output.
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

ABS, REL = 1e-4, 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _inputs(seed, tokens, hidden, vocab, x_std=1.0, w_std=0.1):
    xs = lce_synth.normal_bf16_bits(seed, 0, tokens, hidden, x_std)
    ws = lce_synth.normal_bf16_bits(seed + 1, 2, vocab, hidden, w_std)
    xt = lce_synth.normal_bf16_bits(seed + 2, 0, tokens, hidden, x_std)
    wt = lce_synth.normal_bf16_bits(seed + 3, 2, vocab, hidden, w_std)
    return xs, ws, xt, wt


def _check(got, want):
    got = np.asarray(got, dtype=np.float64)
    err = np.abs(got - want)
    bound = ABS + REL * np.abs(want)
    i = int(np.argmax(err - bound))
    assert (err <= bound).all(), f"token {i}: got {got[i]!r}, want {want[i]!r}"


# Paths: logits stored in scratch for all tokens at once (default), stored in chunks of
# one 256-token fused tile, and recomputed tile by tile (no logit storage).
MODES = ("stored", "chunked", "recompute")


def _env(mode, vocab):
    if mode == "recompute":
        return {"LCE_JSD_STORE_BYTES": 0}
    if mode == "chunked":
        ld = -(-vocab // 256) * 256
        return {"LCE_JSD_STORE_BYTES": 256 * ld * 8}
    return {}


def _run(bits, beta=0.5, reduction="none", mode="stored"):
    xs, ws, xt, wt = (to_dev(b) for b in bits)
    with forced_env(**_env(mode, bits[1].shape[0])):
        out = lce.fused_linear_jsd(xs, ws, xt, wt, beta, reduction)
    torch.cuda.synchronize()
    return out.cpu().numpy()


# Ragged in every dimension: tokens off the 128-token tile, vocab off the 128-row
# tile, hidden off the 64-element slab; one token; several tiles per vocab segment.
@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tokens,hidden,vocab", [(1, 64, 100), (5, 128, 1000), (130, 72, 3000),
                                                 (300, 200, 515), (257, 64, 128),
                                                 (600, 64, 1001), (128, 256, 20000)])
def test_per_token_matches_oracle(tokens, hidden, vocab, mode):
    bits = _inputs(tokens + vocab, tokens, hidden, vocab)
    _check(_run(bits, mode=mode), oracle.fused_linear_jsd_rows(*bits))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("beta", [0.1, 0.5, 0.9])
def test_batchmean_matches_oracle(beta, mode):
    bits = _inputs(11, 520, 128, 1500)
    got = _run(bits, beta, "mean", mode)
    assert got.shape == (1,)
    _check(got, np.array([oracle.fused_linear_jsd(*bits, beta=beta, reduction="mean")]))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("beta", [0.2, 0.75])
def test_other_beta_per_token(beta, mode):
    bits = _inputs(21, 70, 64, 700)
    _check(_run(bits, beta, mode=mode), oracle.fused_linear_jsd_rows(*bits, beta=beta))


@pytest.mark.parametrize("mode", MODES)
def test_identical_heads_give_zero(mode):
    xs, ws, _, _ = _inputs(31, 150, 128, 2000)
    got = _run((xs, ws, xs, ws), mode=mode)
    assert np.abs(got).max() <= ABS


@pytest.mark.parametrize("mode", MODES)
def test_peaked_disjoint_distributions_approach_ln2(mode):
    # Logits of std about 16: each distribution sits on a few classes, rarely the
    # same ones, so the divergence at beta 0.5 is close to its ln 2 ceiling.
    bits = _inputs(41, 64, 256, 1000, x_std=1.0, w_std=1.0)
    got = _run(bits, mode=mode)
    want = oracle.fused_linear_jsd_rows(*bits)
    _check(got, want)
    assert np.median(want) > 0.6 and (got <= math.log(2) + ABS).all()


def test_paths_agree_on_many_tokens():
    # Stored in one piece, in 256-token chunks, and recomputed: the same values up
    # to fp32 summation order.
    bits = _inputs(71, 1100, 128, 4100)
    got = {m: _run(bits, mode=m) for m in MODES}
    assert np.abs(got["stored"] - got["chunked"]).max() <= 1e-6
    assert np.abs(got["stored"] - got["recompute"]).max() <= 1e-5


def test_symmetric_at_half():
    xs, ws, xt, wt = _inputs(51, 90, 64, 900)
    a = _run((xs, ws, xt, wt))
    b = _run((xt, wt, xs, ws))
    assert np.abs(a - b).max() <= 1e-5


def test_empty_batchmean_is_nan_and_none_writes_nothing():
    w = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    assert math.isnan(lce.fused_linear_jsd(x, w, x, w, 0.5, "mean").item())
    out = torch.full((1,), 7.0, device="cuda")
    lce.fused_linear_jsd(x, w, x, w, 0.5, "none", out=out)
    assert out.item() == 7.0


@pytest.mark.parametrize("mode", MODES)
def test_repeated_calls_bitwise_identical(mode):
    bits = _inputs(61, 400, 128, 5000)
    xs, ws, xt, wt = (to_dev(b) for b in bits)
    with forced_env(**_env(mode, 5000)):
        first_none = lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "none").clone()
        first_mean = lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "mean").clone()
        for _ in range(4):
            assert torch.equal(lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "none"), first_none)
            assert torch.equal(lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "mean"), first_mean)


def test_page_shape_sampled_against_oracle():
    w = lce_synth.JSD
    xs_b, ws_b, xt_b, wt_b = w.student_x(), w.student_weight(), w.teacher_x(), w.teacher_weight()
    xs, ws, xt, wt = (to_dev(b) for b in (xs_b, ws_b, xt_b, wt_b))
    per = lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "none").double()
    mean = lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "mean")
    with forced_env(LCE_JSD_STORE_BYTES=0):
        per_rc = lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "none").double()
    torch.cuda.synchronize()
    ref = per.mean().item()
    assert abs(mean.item() - ref) <= ABS + REL * abs(ref)
    assert torch.max(torch.abs(per - per_rc)).item() <= 1e-5
    rows = np.r_[0:6, 509:515, 1018:1024]
    want = oracle.fused_linear_jsd_rows(xs_b[rows], ws_b, xt_b[rows], wt_b)
    _check(per.cpu().numpy()[rows], want)
    _check(per_rc.cpu().numpy()[rows], want)


@pytest.mark.parametrize("seed", range(2))
def test_randomized_cases(seed):
    """Seeded random cases, 6 per seed: 1-400 tokens, hidden a multiple of 8 in [8, 512],
    vocab log-uniform in [2, 5000), each head scaled to its own logit spread (~0.3 to ~12),
    beta in (0, 1), either reduction, any of the three paths; against the oracle."""
    rng = np.random.default_rng(8600 + seed)
    for case in range(6):
        tokens = int(rng.integers(1, 401))
        hidden = 8 * int(rng.integers(1, 65))
        vocab = max(2, int(np.exp(rng.uniform(np.log(2.0), np.log(5000.0)))))
        ss, st = (float(rng.choice([0.3, 1.0, 3.0, 12.0])) for _ in range(2))
        bits = (lce_synth.normal_bf16_bits(9700 + 31 * seed + case, 0, tokens, hidden, 1.0),
                lce_synth.normal_bf16_bits(9800 + 31 * seed + case, 2, vocab, hidden, ss / math.sqrt(hidden)),
                lce_synth.normal_bf16_bits(9900 + 31 * seed + case, 0, tokens, hidden, 1.0),
                lce_synth.normal_bf16_bits(9950 + 31 * seed + case, 2, vocab, hidden, st / math.sqrt(hidden)))
        beta = float(rng.uniform(0.05, 0.95))
        reduction = str(rng.choice(["none", "mean"]))
        mode = str(rng.choice(MODES))
        got = _run(bits, beta, reduction, mode)
        want = oracle.fused_linear_jsd(*bits, beta=beta, reduction=reduction)
        _check(np.atleast_1d(got), np.atleast_1d(np.asarray(want, dtype=np.float64)))
