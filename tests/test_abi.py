"""liblce C ABI on the host: the library loads, exports every declared symbol, and
rejects bad arguments with the documented status before touching the device.

None of these calls reaches a HIP API: argument validation happens first."""
import os
import re
import subprocess

import pytest

import vocab_cross_entropy_row_amd as lce

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lce.h")

FAKE = 0x7F0000000000  # a plausible, 256-byte aligned device address; never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lce.LIB_PATH):
        from vocab_cross_entropy_row_amd import build
        build.build()
    return lce.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:LCE_API\s+)?(?:const\s+)?\w+\*?\s+\**(lce_\w+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == sorted(lce.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", lce.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {ln.split()[-1] for ln in out.splitlines() if " T " in ln}
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)
    # The host code is built with hidden visibility: no internal function leaks.
    assert not [n for n in exported if "lce" in n and not n.startswith("lce_")]


def test_version_and_status_strings(lib):
    assert lce.lce_version() == 600
    names = [lce.lce_status_string(s) for s in range(6)]
    assert names == ["LCE_OK", "LCE_ERR_INVALID_ARG", "LCE_ERR_UNSUPPORTED", "LCE_ERR_ALIAS",
                     "LCE_ERR_OOM", "LCE_ERR_HIP"]
    assert lce.lce_status_string(99) == "LCE_ERR_UNKNOWN"


def _xent(logits=FAKE, dtype=lce.LCE_F32, tokens=16, vocab=32, target=FAKE + (1 << 20),
          reduction=lce.LCE_REDUCTION_NONE, out=FAKE + (2 << 20)):
    return lce.lce_xent_fwd(logits, dtype, tokens, vocab, target, reduction, out, 0)


XENT_CASES = [
    (dict(logits=0), lce.LCE_ERR_INVALID_ARG, "logits is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(out=0, tokens=0, reduction=lce.LCE_REDUCTION_MEAN), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(dtype=7), lce.LCE_ERR_INVALID_ARG, "dtype"),
    (dict(reduction=5), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(tokens=-1), lce.LCE_ERR_INVALID_ARG, "tokens"),
    (dict(vocab=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(vocab=1 << 31), lce.LCE_ERR_UNSUPPORTED, "vocab"),
    (dict(tokens=1 << 32), lce.LCE_ERR_UNSUPPORTED, "tokens"),
    (dict(logits=FAKE + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(target=FAKE + (1 << 20) + 4), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + (2 << 20) + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 64), lce.LCE_ERR_ALIAS, "logits"),
    (dict(out=FAKE + (1 << 20) + 8), lce.LCE_ERR_ALIAS, "target"),
    (dict(tokens=1 << 31, vocab=1 << 30, dtype=lce.LCE_F32), lce.LCE_ERR_INVALID_ARG, "overflow"),
    # one wave (64 work-items) per row: 2^26 rows would need 2^32 work-items in one dispatch
    (dict(tokens=1 << 26, vocab=32, out=FAKE + (1 << 40), target=FAKE + (1 << 41)),
     lce.LCE_ERR_UNSUPPORTED, "work-items"),
    # rows over 32 KiB take a 256-thread workgroup each
    (dict(tokens=1 << 24, vocab=16384, out=FAKE + (1 << 42), target=FAKE + (1 << 43)),
     lce.LCE_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,status,needle", XENT_CASES)
def test_xent_argument_errors(lib, kw, status, needle):
    assert _xent(**kw) == status
    assert needle in lce.lce_last_error()


def _xent_noalloc(logits=FAKE, dtype=lce.LCE_F32, tokens=16, vocab=32, target=FAKE + (1 << 20),
                  reduction=lce.LCE_REDUCTION_NONE, out=FAKE + (2 << 20)):
    return lce.lce_xent_fwd_noalloc(logits, dtype, tokens, vocab, target, reduction, out, 0)


@pytest.mark.parametrize("kw,status,needle", XENT_CASES)
def test_xent_noalloc_argument_errors(lib, kw, status, needle):
    # the allocation-free variant validates exactly as lce_xent_fwd
    assert _xent_noalloc(**kw) == status
    assert needle in lce.lce_last_error()
    assert lce.lce_last_launch() == ""


def test_xent_noalloc_empty_none_is_a_no_op(lib):
    assert lce.lce_xent_fwd_noalloc(0, lce.LCE_BF16, 0, 32, 0, lce.LCE_REDUCTION_NONE, 0, 0) == lce.LCE_OK
    assert lce.lce_last_error() == ""


def test_xent_bf16_alignment_is_two_bytes(lib):
    # bf16 logits only need 2-byte alignment; an odd address is rejected.
    assert _xent(logits=FAKE + 1, dtype=lce.LCE_BF16) == lce.LCE_ERR_INVALID_ARG


def test_xent_empty_none_is_a_no_op(lib):
    # tokens == 0 with no reduction writes nothing and needs no pointers.
    assert lce.lce_xent_fwd(0, lce.LCE_F32, 0, 32, 0, lce.LCE_REDUCTION_NONE, 0, 0) == lce.LCE_OK
    assert lce.lce_last_error() == ""
    assert lce.lce_last_launch() == ""  # nothing was enqueued


def test_failed_call_records_no_launch(lib):
    assert _xent(logits=0) == lce.LCE_ERR_INVALID_ARG
    assert lce.lce_last_launch() == ""


def _fused(x=FAKE, w=FAKE + (1 << 24), tokens=8, hidden=64, vocab=100, target=FAKE + (1 << 28),
           reduction=lce.LCE_REDUCTION_NONE, out=FAKE + (1 << 30)):
    return lce.lce_fused_linear_xent_fwd(x, w, tokens, hidden, vocab, target, reduction, out, 0)


FUSED_CASES = [
    (dict(x=0), lce.LCE_ERR_INVALID_ARG, "x is NULL"),
    (dict(w=0), lce.LCE_ERR_INVALID_ARG, "weight is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(hidden=0), lce.LCE_ERR_INVALID_ARG, "hidden"),
    (dict(vocab=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(hidden=60), lce.LCE_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(hidden=1 << 22), lce.LCE_ERR_UNSUPPORTED, "2^22"),
    (dict(x=FAKE + 8), lce.LCE_ERR_UNSUPPORTED, "16-byte"),
    (dict(w=FAKE + (1 << 24) + 8), lce.LCE_ERR_UNSUPPORTED, "16-byte"),
    (dict(reduction=3), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(out=FAKE + 16), lce.LCE_ERR_ALIAS, "x"),
    (dict(out=FAKE + (1 << 24) + 16), lce.LCE_ERR_ALIAS, "weight"),
    (dict(out=FAKE + (1 << 28)), lce.LCE_ERR_ALIAS, "target"),
    (dict(tokens=1 << 30, target=FAKE + (1 << 41), out=FAKE + (1 << 42)), lce.LCE_ERR_UNSUPPORTED,
     "2^30"),
]


@pytest.mark.parametrize("kw,status,needle", FUSED_CASES)
def test_fused_argument_errors(lib, kw, status, needle):
    assert _fused(**kw) == status
    assert needle in lce.lce_last_error()


def test_binding_refuses_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    z = torch.zeros(4, 8)
    t = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        lce.xent(z, t)
    with pytest.raises(ValueError):
        lce.fused_linear_xent(z.bfloat16(), z.bfloat16(), t)


def _partial(logits=FAKE, dtype=lce.LCE_F32, tokens=16, shard=32, start=64, target=FAKE + (1 << 20),
             partial=FAKE + (2 << 20)):
    return lce.lce_xent_partial_fwd(logits, dtype, tokens, shard, start, target, partial, 0)


PARTIAL_CASES = [
    (dict(logits=0), lce.LCE_ERR_INVALID_ARG, "logits is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(partial=0), lce.LCE_ERR_INVALID_ARG, "partial is NULL"),
    (dict(dtype=3), lce.LCE_ERR_INVALID_ARG, "dtype"),
    (dict(tokens=-2), lce.LCE_ERR_INVALID_ARG, "tokens"),
    (dict(shard=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(start=-1), lce.LCE_ERR_INVALID_ARG, "vocab_start"),
    (dict(start=(1 << 63) - 8), lce.LCE_ERR_INVALID_ARG, "overflows"),
    (dict(partial=FAKE + (2 << 20) + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(tokens=1 << 26, partial=FAKE + (1 << 40), target=FAKE + (1 << 41)),
     lce.LCE_ERR_UNSUPPORTED, "work-items"),
    (dict(partial=FAKE + 256), lce.LCE_ERR_ALIAS, "partial overlaps logits"),
    # 16 tokens x 12 bytes reach past the first 64 bytes of partial: overlaps the target
    (dict(partial=FAKE + (1 << 20) - 100), lce.LCE_ERR_ALIAS, "partial overlaps target"),
]


@pytest.mark.parametrize("kw,status,needle", PARTIAL_CASES)
def test_partial_argument_errors(lib, kw, status, needle):
    assert _partial(**kw) == status
    assert needle in lce.lce_last_error()


def _merge(partials=FAKE, shards=4, tokens=16, target=FAKE + (1 << 20), vocab=1000,
           reduction=lce.LCE_REDUCTION_NONE, out=FAKE + (2 << 20)):
    return lce.lce_xent_merge(partials, shards, tokens, target, vocab, reduction, out, 0)


MERGE_CASES = [
    (dict(partials=0), lce.LCE_ERR_INVALID_ARG, "partials is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(shards=0), lce.LCE_ERR_INVALID_ARG, "shards"),
    (dict(shards=1 << 31), lce.LCE_ERR_UNSUPPORTED, "shards"),
    (dict(vocab=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(reduction=9), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(partials=FAKE + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(out=FAKE + 4 * 16 * 12 - 4), lce.LCE_ERR_ALIAS, "partials"),
    (dict(out=FAKE + (1 << 20)), lce.LCE_ERR_ALIAS, "target"),
]


@pytest.mark.parametrize("kw,status,needle", MERGE_CASES)
def test_merge_argument_errors(lib, kw, status, needle):
    assert _merge(**kw) == status
    assert needle in lce.lce_last_error()


def test_partial_and_merge_empty_are_no_ops(lib):
    assert lce.lce_xent_partial_fwd(0, lce.LCE_BF16, 0, 8, 0, 0, 0, 0) == lce.LCE_OK
    assert lce.lce_xent_merge(0, 3, 0, 0, 10, lce.LCE_REDUCTION_NONE, 0, 0) == lce.LCE_OK


def _bwd(logits=FAKE, dtype=lce.LCE_F32, tokens=16, vocab=32, target=FAKE + (1 << 20),
         reduction=lce.LCE_REDUCTION_MEAN, grad=FAKE + (2 << 20), dlogits=FAKE + (3 << 20)):
    return lce.lce_xent_bwd(logits, dtype, tokens, vocab, target, reduction, grad, dlogits, 0)


BWD_CASES = [
    (dict(logits=0), lce.LCE_ERR_INVALID_ARG, "logits is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(grad=0), lce.LCE_ERR_INVALID_ARG, "grad is NULL"),
    (dict(dlogits=0), lce.LCE_ERR_INVALID_ARG, "dlogits is NULL"),
    (dict(reduction=4), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(vocab=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(grad=FAKE + (2 << 20) + 1), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(dlogits=FAKE + (3 << 20) + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(dlogits=FAKE + (3 << 20) + 4), lce.LCE_ERR_UNSUPPORTED, "modulo 16"),
    (dict(dlogits=FAKE + 64), lce.LCE_ERR_ALIAS, "same buffer"),
    (dict(dlogits=FAKE + (1 << 20) - 256), lce.LCE_ERR_ALIAS, "target"),
    (dict(dlogits=FAKE + (2 << 20) - 256), lce.LCE_ERR_ALIAS, "grad"),
    (dict(tokens=1 << 26, target=FAKE + (1 << 40), grad=FAKE + (1 << 41), dlogits=FAKE + (1 << 42)),
     lce.LCE_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,status,needle", BWD_CASES)
def test_bwd_argument_errors(lib, kw, status, needle):
    assert _bwd(**kw) == status
    assert needle in lce.lce_last_error()


def test_bwd_empty_is_a_no_op(lib):
    assert lce.lce_xent_bwd(0, lce.LCE_F32, 0, 8, 0, lce.LCE_REDUCTION_NONE, 0, 0, 0) == lce.LCE_OK


def _fwd_bwd(logits=FAKE, dtype=lce.LCE_F32, tokens=16, vocab=32, target=FAKE + (1 << 20),
             reduction=lce.LCE_REDUCTION_MEAN, grad=FAKE + (2 << 20), out=FAKE + (4 << 20),
             dlogits=FAKE + (3 << 20)):
    return lce.lce_xent_fwd_bwd(logits, dtype, tokens, vocab, target, reduction, grad, out, dlogits, 0)


# The forward's checks on out, then the backward's on grad and dlogits, then out
# against the gradient's buffers.
FWD_BWD_CASES = [
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(out=FAKE + (4 << 20) + 2), lce.LCE_ERR_INVALID_ARG, "out is not"),
    (dict(out=FAKE + 128), lce.LCE_ERR_ALIAS, "out overlaps logits"),
    (dict(out=FAKE + (1 << 20) + 8), lce.LCE_ERR_ALIAS, "out overlaps target"),
    (dict(out=FAKE + (3 << 20) + 4), lce.LCE_ERR_ALIAS, "out overlaps dlogits"),
    (dict(out=FAKE + (2 << 20)), lce.LCE_ERR_ALIAS, "out overlaps grad"),
    (dict(grad=0), lce.LCE_ERR_INVALID_ARG, "grad is NULL"),
    (dict(dlogits=0), lce.LCE_ERR_INVALID_ARG, "dlogits is NULL"),
    (dict(dlogits=FAKE + 64), lce.LCE_ERR_ALIAS, "same buffer"),
    (dict(reduction=3), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(logits=0), lce.LCE_ERR_INVALID_ARG, "logits is NULL"),
    (dict(tokens=1 << 26, target=FAKE + (1 << 40), grad=FAKE + (1 << 41), dlogits=FAKE + (1 << 42),
          out=FAKE + (1 << 43)), lce.LCE_ERR_UNSUPPORTED, "work-items"),
]


@pytest.mark.parametrize("kw,status,needle", FWD_BWD_CASES)
def test_fwd_bwd_argument_errors(lib, kw, status, needle):
    assert _fwd_bwd(**kw) == status
    assert needle in lce.lce_last_error()


def test_fwd_bwd_empty_none_is_a_no_op(lib):
    assert lce.lce_xent_fwd_bwd(0, lce.LCE_F32, 0, 8, 0, lce.LCE_REDUCTION_NONE, 0, 0, 0, 0) == lce.LCE_OK


def _sums(x=FAKE, w=FAKE + (1 << 24), batch=2, seq=4, hidden=64, vocab=100, target=FAKE + (1 << 28),
          out=FAKE + (1 << 30)):
    return lce.lce_fused_linear_logprob_sums(x, w, batch, seq, hidden, vocab, target, out, 0)


SUMS_CASES = [
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(x=0), lce.LCE_ERR_INVALID_ARG, "x is NULL"),
    (dict(batch=-1), lce.LCE_ERR_INVALID_ARG, "batch"),
    (dict(seq=-3), lce.LCE_ERR_INVALID_ARG, "seq"),
    (dict(batch=1 << 40, seq=1 << 40), lce.LCE_ERR_INVALID_ARG, "overflows"),
    (dict(hidden=12), lce.LCE_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(out=FAKE + (1 << 28) + 8), lce.LCE_ERR_ALIAS, "target"),
]


@pytest.mark.parametrize("kw,status,needle", SUMS_CASES)
def test_logprob_sums_argument_errors(lib, kw, status, needle):
    assert _sums(**kw) == status
    assert needle in lce.lce_last_error()


def _jsd(xs=FAKE, ws=FAKE + (1 << 24), xt=FAKE + (2 << 24), wt=FAKE + (3 << 24), tokens=8,
         hidden=64, vocab=100, beta=0.5, reduction=lce.LCE_REDUCTION_NONE, out=FAKE + (1 << 30)):
    return lce.lce_fused_linear_jsd_fwd(xs, ws, xt, wt, tokens, hidden, vocab, beta, reduction,
                                        out, 0)


JSD_CASES = [
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(xs=0), lce.LCE_ERR_INVALID_ARG, "student_x is NULL"),
    (dict(ws=0), lce.LCE_ERR_INVALID_ARG, "student_weight is NULL"),
    (dict(xt=0), lce.LCE_ERR_INVALID_ARG, "teacher_x is NULL"),
    (dict(wt=0), lce.LCE_ERR_INVALID_ARG, "teacher_weight is NULL"),
    (dict(tokens=-1), lce.LCE_ERR_INVALID_ARG, "tokens"),
    (dict(hidden=0), lce.LCE_ERR_INVALID_ARG, "hidden"),
    (dict(vocab=0), lce.LCE_ERR_INVALID_ARG, "vocab"),
    (dict(hidden=20), lce.LCE_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(hidden=1 << 22), lce.LCE_ERR_UNSUPPORTED, "2^22"),
    (dict(xt=FAKE + (2 << 24) + 8), lce.LCE_ERR_UNSUPPORTED, "16-byte"),
    (dict(beta=0.0), lce.LCE_ERR_INVALID_ARG, "beta"),
    (dict(beta=1.0), lce.LCE_ERR_INVALID_ARG, "beta"),
    (dict(beta=float("nan")), lce.LCE_ERR_INVALID_ARG, "beta"),
    (dict(reduction=2), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(out=FAKE + 16), lce.LCE_ERR_ALIAS, "student_x"),
    (dict(out=FAKE + (3 << 24) + 64), lce.LCE_ERR_ALIAS, "teacher_weight"),
]


@pytest.mark.parametrize("kw,status,needle", JSD_CASES)
def test_jsd_argument_errors(lib, kw, status, needle):
    assert _jsd(**kw) == status
    assert needle in lce.lce_last_error()


def test_jsd_empty_none_is_a_no_op(lib):
    assert lce.lce_fused_linear_jsd_fwd(0, FAKE, 0, FAKE, 0, 64, 100, 0.5, lce.LCE_REDUCTION_NONE,
                                        0, 0) == lce.LCE_OK


def _fbwd(x=FAKE, w=FAKE + (1 << 24), tokens=8, hidden=64, vocab=100, target=FAKE + (1 << 28),
          reduction=lce.LCE_REDUCTION_MEAN, grad=FAKE + (1 << 29), dx=FAKE + (1 << 30),
          dw=FAKE + (1 << 31)):
    return lce.lce_fused_linear_xent_bwd(x, w, tokens, hidden, vocab, target, reduction, grad, dx,
                                         dw, 0)


FBWD_CASES = [
    (dict(x=0), lce.LCE_ERR_INVALID_ARG, "x is NULL"),
    (dict(w=0), lce.LCE_ERR_INVALID_ARG, "weight is NULL"),
    (dict(target=0), lce.LCE_ERR_INVALID_ARG, "target is NULL"),
    (dict(grad=0), lce.LCE_ERR_INVALID_ARG, "grad is NULL"),
    (dict(dx=0, dw=0), lce.LCE_ERR_INVALID_ARG, "both NULL"),
    (dict(grad=FAKE + (1 << 29) + 2), lce.LCE_ERR_INVALID_ARG, "grad is not"),
    (dict(dx=FAKE + (1 << 30) + 2), lce.LCE_ERR_INVALID_ARG, "aligned"),
    (dict(hidden=12), lce.LCE_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(vocab=1 << 23), lce.LCE_ERR_UNSUPPORTED, "fused backward"),
    (dict(reduction=5), lce.LCE_ERR_INVALID_ARG, "reduction"),
    (dict(dx=FAKE + 64), lce.LCE_ERR_ALIAS, "dx overlaps x"),
    (dict(dw=FAKE + (1 << 24) + 64), lce.LCE_ERR_ALIAS, "dweight overlaps weight"),
    (dict(dx=FAKE + (1 << 28)), lce.LCE_ERR_ALIAS, "dx overlaps target"),
    (dict(dw=FAKE + (1 << 29)), lce.LCE_ERR_ALIAS, "dweight overlaps grad"),
    (dict(dw=FAKE + (1 << 30) + 1024), lce.LCE_ERR_ALIAS, "dx overlaps dweight"),
    (dict(tokens=1 << 30, target=FAKE + (1 << 40), grad=FAKE + (1 << 41), dx=FAKE + (1 << 42),
          dw=FAKE + (1 << 44)), lce.LCE_ERR_UNSUPPORTED, "2^30"),
]


@pytest.mark.parametrize("kw,status,needle", FBWD_CASES)
def test_fused_bwd_argument_errors(lib, kw, status, needle):
    assert _fbwd(**kw) == status
    assert needle in lce.lce_last_error()


def _ffb(x=FAKE, w=FAKE + (1 << 24), tokens=8, hidden=64, vocab=100, target=FAKE + (1 << 28),
         reduction=lce.LCE_REDUCTION_MEAN, grad=FAKE + (1 << 29), out=FAKE + (1 << 32),
         dx=FAKE + (1 << 30), dw=FAKE + (1 << 31)):
    return lce.lce_fused_linear_xent_fwd_bwd(x, w, tokens, hidden, vocab, target, reduction, grad,
                                             out, dx, dw, 0)


FUSED_FWD_BWD_CASES = [
    (dict(out=0), lce.LCE_ERR_INVALID_ARG, "out is NULL"),
    (dict(out=FAKE + 32), lce.LCE_ERR_ALIAS, "x"),
    (dict(out=FAKE + (1 << 28) + 16), lce.LCE_ERR_ALIAS, "target"),
    (dict(out=FAKE + (1 << 29)), lce.LCE_ERR_ALIAS, "out overlaps grad"),
    (dict(out=FAKE + (1 << 30) + 64), lce.LCE_ERR_ALIAS, "out overlaps dx"),
    (dict(out=FAKE + (1 << 31) + 64), lce.LCE_ERR_ALIAS, "out overlaps dweight"),
    (dict(grad=0), lce.LCE_ERR_INVALID_ARG, "grad is NULL"),
    (dict(dx=0, dw=0), lce.LCE_ERR_INVALID_ARG, "both NULL"),
    (dict(hidden=12), lce.LCE_ERR_UNSUPPORTED, "multiple of 8"),
    (dict(vocab=1 << 23), lce.LCE_ERR_UNSUPPORTED, "fused backward"),
    (dict(reduction=5), lce.LCE_ERR_INVALID_ARG, "reduction"),
]


@pytest.mark.parametrize("kw,status,needle", FUSED_FWD_BWD_CASES)
def test_fused_fwd_bwd_argument_errors(lib, kw, status, needle):
    assert _ffb(**kw) == status
    assert needle in lce.lce_last_error()
