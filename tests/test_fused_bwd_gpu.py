"""Gradients of the fused projection + cross-entropy (lce_fused_linear_xent_bwd, through
the C ABI) against the fp64 oracle.

Tolerance, derived from the arithmetic.  The kernel's logits are fp32 sums of exact bf16
products: one rounding per 16-product MFMA step, so |z - z_exact| <= (H/16 + 2) 2^-24 S
with S = sum_k |x_k W_k|, and z and the row's log-sum-exp are held in fp32 (half an ulp
each, <= 2^-24 (|z| + |lse|)).  The softmax p = e^(z - lse) then carries a relative error
e_p of those two plus a few ulps (2^-21) of its own fp32 arithmetic.  The logit gradient
dZ_tv = g_t (p_tv - [v = t_t]) is formed in fp32, so its error is relative to g p and
not to dZ, which is near 0 where p is near 1 at the target (exactly 0 with one vocab
row); it is then rounded to bf16 (relative error <= 2^-9) before the two GEMMs, which
accumulate exact bf16 products in fp32.  So each element of dx = dZ W is within
sum_v (2^-9 |dZ_tv| + |g_t| p_tv e_p,tv + 2^-21 |g_t| [v = t_t]) |W_vh|; the tests allow
twice each term (2^-8 for the bf16 rounding, which also covers the GEMMs' fp32
accumulation), plus 1e-7 absolute.  dW = dZ^T x gets the same bound with x for W.

At the page shape (tokens 2048, hidden 4096, vocab 128256) the oracle checks dx on a
sample of tokens and dW on a sample of head rows (each row needs every token's softmax,
so the oracle takes all 2048 tokens' fp64 logits block by block); properties that hold
at any size check the rest: the columns of dW sum to ~0 (each row of dZ sums to 0), and
mean reduction equals per-token reduction with gradient 1/tokens.
"""
import numpy as np
import pytest

import lce_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import forced_env, to_dev  # noqa: E402

REL, SOFTMAX, ABS = 2.0 ** -8, 2.0 ** -20, 1e-7


def _grad_error(dz, z, lse, S, g, onehot, hidden):
    """Per-logit bound on the kernel's dZ error (twice each term of the derivation above).
    dz, z, S: [tokens, cols]; lse, g: [tokens, 1]; onehot: [tokens, cols]."""
    p = np.exp(z - lse)
    e_p = 2.0 ** -24 * (np.abs(z) + np.abs(lse)) + (hidden / 16 + 2) * 2.0 ** -24 * S + 2.0 ** -21
    return REL * np.abs(dz) + 2.0 * np.abs(g) * p * e_p + SOFTMAX * np.abs(g) * onehot


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _inputs(seed, tokens, hidden, vocab, w_std=0.1):
    xb = lce_synth.normal_bf16_bits(seed, 0, tokens, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(seed + 1, 2, vocab, hidden, w_std)
    t = lce_synth.targets(seed + 2, tokens, vocab)
    return xb, wb, t


def _row_scale(grad, reduction, tokens):
    g = np.asarray(grad, dtype=np.float64).reshape(-1)
    return np.full(tokens, g[0] / tokens) if reduction == "mean" else g


def _bounds(xb, wb, t, scale, want_dw=True):
    x64, w64 = oracle.bf16_bits_to_f64(xb), oracle.bf16_bits_to_f64(wb)
    z = x64 @ w64.T
    dz = oracle.xent_bwd(z, t, scale, "none", dtype="f64")
    m = z.max(axis=1, keepdims=True)
    lse = m + np.log(np.exp(z - m).sum(axis=1, keepdims=True))
    onehot = np.zeros_like(z)
    ok = (t >= 0) & (t < z.shape[1])
    onehot[np.nonzero(ok)[0], t[ok]] = 1.0
    g = np.asarray(scale, dtype=np.float64).reshape(-1, 1)
    e = _grad_error(dz, z, lse, np.abs(x64) @ np.abs(w64).T, g, onehot, x64.shape[1])
    bw = e.T @ np.abs(x64) + ABS if want_dw else None
    return e @ np.abs(w64) + ABS, bw


def _check(name, got, want, bound):
    err = np.abs(np.asarray(got, dtype=np.float64) - want)
    bad = np.argwhere(~(err <= bound))
    assert bad.size == 0, f"{name}: {len(bad)} elements off, first {tuple(bad[0])}: " \
        f"got {got[tuple(bad[0])]!r}, want {want[tuple(bad[0])]!r}, bound {bound[tuple(bad[0])]!r}"


def _run(xb, wb, t, grad, reduction, want_dx=True, want_dw=True, env=None):
    x, W = to_dev(xb), to_dev(wb)
    td = torch.from_numpy(t).cuda()
    g = torch.tensor(np.asarray(grad, dtype=np.float32).reshape(-1)).cuda()
    with forced_env(**(env or {})):
        dx, dw = lce.fused_linear_xent_bwd(x, W, td, g, reduction, want_dx, want_dw)
    torch.cuda.synchronize()
    return (None if dx is None else dx.cpu().numpy()), (None if dw is None else dw.cpu().numpy())


# Ragged in every dimension (tokens off the 256-token tile, vocab off the 256-row tile,
# hidden off the 64-element slab), one token, and several token chunks.
CASES = [(1, 64, 100), (5, 128, 1000), (130, 72, 3000), (300, 200, 515), (600, 64, 1001)]

# Paths: fp32 logits stored for all tokens at once (default), stored in 256-token chunks,
# and recomputed by the gradient mode of the fused kernel (no fp32 logits stored).
MODES = ("stored", "chunked", "recompute")


def _env(mode, vocab):
    ld = -(-vocab // 256) * 256
    if mode == "chunked":
        return {"LCE_FUSED_BWD_STORE_BYTES": 256 * ld * 6}
    if mode == "recompute":
        return {"LCE_FUSED_BWD_STORE_BYTES": 0}
    return {}


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("reduction", ["mean", "none"])
@pytest.mark.parametrize("tokens,hidden,vocab", CASES)
def test_grads_match_oracle(tokens, hidden, vocab, reduction, mode):
    xb, wb, t = _inputs(tokens * 7 + vocab, tokens, hidden, vocab)
    rng = np.random.default_rng(tokens)
    grad = np.array([1.7]) if reduction == "mean" else rng.normal(size=tokens)
    grad = grad.astype(np.float32).astype(np.float64)
    dx, dw = _run(xb, wb, t, grad, reduction, env=_env(mode, vocab))
    want_dx, want_dw = oracle.fused_linear_xent_bwd(xb, wb, t, grad, reduction)
    bx, bw = _bounds(xb, wb, t, _row_scale(grad, reduction, tokens))
    _check("dx", dx, want_dx, bx)
    _check("dW", dw, want_dw, bw)


@pytest.mark.parametrize("mode", ["chunked", "recompute"])
def test_token_chunks_give_the_same_grads(mode):
    """256-token chunks (dW accumulated over chunks in the GEMM's C) against one chunk;
    the stored and recomputed logit gradients are the same bf16 values, so only the
    GEMMs' chunking can differ."""
    xb, wb, t = _inputs(3, 700, 128, 2000)
    one = _run(xb, wb, t, [1.0], "mean")
    chunked = _run(xb, wb, t, [1.0], "mean", env=_env(mode, 2000))
    bx, bw = _bounds(xb, wb, t, np.full(700, 1.0 / 700))
    _check("dx chunked vs one", chunked[0], one[0], bx)
    _check("dW chunked vs one", chunked[1], one[1], bw)
    want_dx, want_dw = oracle.fused_linear_xent_bwd(xb, wb, t, 1.0, "mean")
    _check("dx chunked", chunked[0], want_dx, bx)
    _check("dW chunked", chunked[1], want_dw, bw)


def test_one_gradient_only():
    xb, wb, t = _inputs(5, 200, 64, 900)
    dx, dw = _run(xb, wb, t, [2.0], "mean")
    dx_only, none_w = _run(xb, wb, t, [2.0], "mean", want_dw=False)
    none_x, dw_only = _run(xb, wb, t, [2.0], "mean", want_dx=False)
    assert none_w is None and none_x is None
    assert np.array_equal(dx, dx_only) and np.array_equal(dw, dw_only)


@pytest.mark.parametrize("mode", ["stored", "recompute"])
def test_invalid_target_poisons_its_row_and_dweight(mode):
    xb, wb, t = _inputs(7, 40, 64, 300)
    t[11] = 300
    dx, dw = _run(xb, wb, t, [1.0], "mean", env=_env(mode, 300))
    assert np.isnan(dx[11]).all() and np.isfinite(np.delete(dx, 11, axis=0)).all()
    assert np.isnan(dw).all()


def test_empty_tokens_give_zero_dweight():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.ones((10, 64), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((0,), dtype=torch.int64, device="cuda")
    dw = torch.full((10, 64), 5.0, device="cuda")
    lce.fused_linear_xent_bwd(x, W, t, torch.ones(1, device="cuda"), "mean", want_dx=False,
                              dweight=dw)
    assert torch.equal(dw.cpu(), torch.zeros(10, 64))


@pytest.mark.parametrize("mode", MODES)
def test_repeated_calls_bitwise_identical(mode):
    xb, wb, t = _inputs(9, 520, 128, 3000)
    first = _run(xb, wb, t, [1.0], "mean", env=_env(mode, 3000))
    for _ in range(3):
        again = _run(xb, wb, t, [1.0], "mean", env=_env(mode, 3000))
        assert np.array_equal(first[0], again[0]) and np.array_equal(first[1], again[1])


def test_page_shape_sampled_and_properties():
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    xb, wb, t = w.x(), w.weight(), w.target()
    x, W = to_dev(xb), to_dev(wb)
    td = torch.from_numpy(t).cuda()
    T = w.tokens
    dx, dw = lce.fused_linear_xent_bwd(x, W, td, torch.ones(1, device="cuda"), "mean")
    dx_n, dw_n = lce.fused_linear_xent_bwd(x, W, td, torch.full((T,), 1.0 / T, device="cuda"),
                                           "none")
    with forced_env(LCE_FUSED_BWD_STORE_BYTES=0):
        dx_r, dw_r = lce.fused_linear_xent_bwd(x, W, td, torch.ones(1, device="cuda"), "mean")
    torch.cuda.synchronize()
    assert torch.equal(dx, dx_n) and torch.equal(dw, dw_n)  # 1/2048 is exact in fp32
    # Stored and recomputed logits are the same fp32 sums, so dZ is bit-identical; only
    # the recompute path's 256-token chunks change the GEMMs' shapes.
    assert torch.allclose(dx_r, dx, rtol=0, atol=1e-6) and torch.allclose(dw_r, dw, rtol=0, atol=1e-6)
    # Columns of dW sum to ~0: each dZ row sums to 0 up to its bf16 rounding.
    col = dw.double().sum(dim=0).abs()
    lim = REL * (x.double().abs().sum(dim=0) * 2.0 / T) + 1e-6
    assert bool((col <= lim).all())
    rows = np.r_[0:4, 1021:1025, 2044:2048]
    scale = np.full(len(rows), 1.0 / T)
    want_dx, _ = oracle.fused_linear_xent_grads(xb[rows], wb, t[rows], scale, want_dw=False)
    bx, _ = _bounds(xb[rows], wb, t[rows], scale, want_dw=False)
    _check("dx rows", dx.cpu().numpy()[rows], want_dx, bx)
    # Rows of dW against the oracle: the first and last head rows, two in the middle, and
    # the rows of three tokens' targets (where the one-hot term enters the sum).
    head = np.unique(np.r_[0:2, 64127:64129, w.vocab - 2:w.vocab, t[[0, 1023, 2047]]])
    want_dw, dz_cols = oracle.fused_linear_xent_dw_rows(xb, wb, t, np.full(T, 1.0 / T), head)
    x64 = oracle.bf16_bits_to_f64(xb)
    w_head = oracle.bf16_bits_to_f64(wb[head])
    z_cols = x64 @ w_head.T
    onehot = (t[:, None] == head[None, :]).astype(np.float64)
    p_cols = dz_cols * T + onehot                    # g = 1/T
    j = np.argmax(p_cols, axis=1)                    # each token's lse from its largest p here
    r = np.arange(T)
    lse = (z_cols[r, j] - np.log(p_cols[r, j]))[:, None]
    e = _grad_error(dz_cols, z_cols, lse, np.abs(x64) @ np.abs(w_head).T, np.full((T, 1), 1.0 / T),
                    onehot, x64.shape[1])
    bw = e.T @ np.abs(x64) + ABS
    _check("dW rows", dw[torch.from_numpy(head).cuda()].cpu().numpy(), want_dw, bw)


def test_graph_replays_match_eager():
    """The backward (fused kernels and hipBLASLt GEMMs) recorded into a HIP graph:
    every replay, with eager work in between, reproduces the eager gradients."""
    xb, wb, t = _inputs(13, 300, 128, 2000)
    x, W = to_dev(xb), to_dev(wb)
    td = torch.from_numpy(t).cuda()
    g = torch.full((1,), 0.5, device="cuda")
    dx = torch.empty(x.shape, device="cuda")
    dw = torch.empty(W.shape, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):  # eager reference; plans the GEMMs and grows the scratch
        lce.fused_linear_xent_bwd(x, W, td, g, "mean", dx=dx, dweight=dw)
    torch.cuda.synchronize()
    ref = (dx.clone(), dw.clone())
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr, stream=s):
        lce.fused_linear_xent_bwd(x, W, td, g, "mean", dx=dx, dweight=dw)
    torch.cuda.synchronize()
    xo, wo, to_ = _inputs(14, 100, 64, 700)
    for r in range(3):
        dx.fill_(float("nan"))
        dw.fill_(float("nan"))
        with torch.cuda.stream(s):  # other eager work on the same stream and scratch
            lce.fused_linear_xent_bwd(to_dev(xo), to_dev(wo), torch.from_numpy(to_).cuda(),
                                      torch.ones(1, device="cuda"), "mean")
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(dx, ref[0]) and torch.equal(dw, ref[1]), f"replay {r}"


def test_dw_gemm_layouts_agree():
    """dW through transposed operands (default) and through x as stored
    (LCE_FUSED_BWD_DW_NT=1): the same products in another GEMM kernel."""
    xb, wb, t = _inputs(15, 600, 136, 1700)
    a = _run(xb, wb, t, [1.0], "mean", env=_env("chunked", 1700))
    b = _run(xb, wb, t, [1.0], "mean", env={**_env("chunked", 1700), "LCE_FUSED_BWD_DW_NT": 1})
    assert np.array_equal(a[0], b[0])
    _, bw = _bounds(xb, wb, t, np.full(600, 1.0 / 600))
    _check("dW layouts", a[1], b[1], bw)
    _check("dW vs oracle", a[1], oracle.fused_linear_xent_bwd(xb, wb, t, 1.0, "mean")[1], bw)


@pytest.mark.parametrize("seed", range(2))
def test_randomized_grads(seed):
    """Seeded random cases, 6 per seed: 1-400 tokens, hidden a multiple of 8 in [8, 512],
    vocab log-uniform in [1, 4000), heads scaled to logit spreads from ~0.3 to ~12, targets
    anywhere (also the first and last vocab rows), either reduction, any of the three paths;
    dx and dW against the oracle within the bound derived above."""
    rng = np.random.default_rng(8400 + seed)
    for case in range(6):
        tokens = int(rng.integers(1, 401))
        hidden = 8 * int(rng.integers(1, 65))
        vocab = max(1, int(np.exp(rng.uniform(0.0, np.log(4000.0)))))
        spread = float(rng.choice([0.3, 1.0, 3.0, 12.0]))
        xb = lce_synth.normal_bf16_bits(9100 + 31 * seed + case, 0, tokens, hidden, 1.0)
        wb = lce_synth.normal_bf16_bits(9600 + 31 * seed + case, 2, vocab, hidden,
                                        spread / np.sqrt(hidden))
        t = rng.integers(0, vocab, tokens).astype(np.int64)
        t[rng.random(tokens) < 0.1] = vocab - 1
        t[rng.random(tokens) < 0.1] = 0
        reduction = str(rng.choice(["mean", "none"]))
        grad = (np.array([rng.uniform(0.5, 2.0)]) if reduction == "mean"
                else rng.normal(size=tokens)).astype(np.float32).astype(np.float64)
        mode = str(rng.choice(MODES))
        label = f"seed {seed} case {case}: T {tokens} H {hidden} V {vocab} spread {spread} {reduction} {mode}"
        dx, dw = _run(xb, wb, t, grad, reduction, env=_env(mode, vocab))
        want_dx, want_dw = oracle.fused_linear_xent_bwd(xb, wb, t, grad, reduction)
        bx, bw = _bounds(xb, wb, t, _row_scale(grad, reduction, tokens))
        _check(f"dx {label}", dx, want_dx, bx)
        _check(f"dW {label}", dw, want_dw, bw)
