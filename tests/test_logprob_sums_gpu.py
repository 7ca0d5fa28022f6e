"""Per-sequence sums of target log-probabilities under the fused projection
(lce_fused_linear_logprob_sums, through the C ABI) against the fp64 oracle.

The per-token fused losses carry the fused tolerance (2e-2 stated, 1e-3 required by
these tests); a sum of `seq` of them is held to seq * 1e-3.  At the full CPO-page shape
(batch 2, seq 1024, hidden 4096, vocab 128256) the oracle is too slow for every token, so
the sums are checked against the same call's per-token losses (a property that holds at
any size) and the oracle checks a sample of tokens.
"""
import math

import numpy as np
import pytest

import lce_synth
import oracle

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import to_dev  # noqa: E402

PER_TOKEN = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("batch,seq,hidden,vocab", [(1, 1, 64, 100), (3, 5, 128, 1000),
                                                    (2, 130, 256, 3000), (7, 33, 64, 515)])
def test_sums_match_oracle(batch, seq, hidden, vocab):
    xb = lce_synth.normal_bf16_bits(batch * 31 + seq, 0, batch * seq, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(vocab, 2, vocab, hidden, 0.1)
    t = lce_synth.targets(seq, batch * seq, vocab)
    got = lce.fused_linear_logprob_sums(to_dev(xb).view(batch, seq, hidden), to_dev(wb),
                                        torch.from_numpy(t).cuda().view(batch, seq))
    want = oracle.fused_linear_logprob_sums(xb, wb, t, batch, seq)
    assert np.max(np.abs(got.cpu().numpy() - want)) <= seq * PER_TOKEN


def test_invalid_target_poisons_only_its_sequence():
    batch, seq, hidden, vocab = 4, 6, 64, 200
    xb = lce_synth.normal_bf16_bits(1, 0, batch * seq, hidden, 1.0)
    wb = lce_synth.normal_bf16_bits(2, 2, vocab, hidden, 0.1)
    t = lce_synth.targets(3, batch * seq, vocab)
    t[2 * seq + 3] = vocab
    got = lce.fused_linear_logprob_sums(to_dev(xb).view(batch, seq, hidden), to_dev(wb),
                                        torch.from_numpy(t).cuda().view(batch, seq)).cpu().numpy()
    assert math.isnan(got[2]) and np.isfinite(got[[0, 1, 3]]).all()


def test_empty_sequences_sum_to_zero():
    x = torch.empty((3, 0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones((10, 64), dtype=torch.bfloat16, device="cuda")
    t = torch.empty((3, 0), dtype=torch.int64, device="cuda")
    assert torch.equal(lce.fused_linear_logprob_sums(x, w, t).cpu(), torch.zeros(3))


def test_full_cpo_shape_against_per_token_losses():
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    batch, seq = 2, 1024
    xb, wb, t = w.x(), w.weight(), w.target()
    x, W = to_dev(xb), to_dev(wb)
    td = torch.from_numpy(t).cuda()
    sums = lce.fused_linear_logprob_sums(x.view(batch, seq, w.hidden), W, td.view(batch, seq))
    per = lce.fused_linear_xent(x, W, td, "none").double()
    torch.cuda.synchronize()
    ref = -per.view(batch, seq).sum(dim=1)
    assert torch.max(torch.abs(sums.double() - ref)).item() <= 1e-3
    rows = np.r_[0:8, 1020:1028, 2040:2048]
    want = oracle.fused_linear_xent_rows(xb, wb, t, rows=rows)
    assert np.max(np.abs(per.cpu().numpy()[rows] - want)) <= PER_TOKEN


def test_repeated_sums_bitwise_identical():
    batch, seq, hidden, vocab = 8, 300, 128, 2000
    x = to_dev(lce_synth.normal_bf16_bits(5, 0, batch * seq, hidden, 1.0)).view(batch, seq, hidden)
    W = to_dev(lce_synth.normal_bf16_bits(6, 2, vocab, hidden, 0.1))
    t = torch.from_numpy(lce_synth.targets(7, batch * seq, vocab)).cuda().view(batch, seq)
    first = lce.fused_linear_logprob_sums(x, W, t).clone()
    for _ in range(5):
        assert torch.equal(lce.fused_linear_logprob_sums(x, W, t), first)
