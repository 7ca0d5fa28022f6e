"""lce_xent_fwd_noalloc, the row cross-entropy for callers that cannot allocate (its
scratch is a static device array), against lce_xent_fwd through the C ABI: two calls in a
row on each path, the second with a smaller input, must give bitwise the same per-token
losses and means as the allocating entry point on the same inputs; sizes beyond the
array's limits are refused."""
import numpy as np
import pytest

import lce_synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import vocab_cross_entropy_row_amd as lce  # noqa: E402
from gpu_util import to_dev  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lce.load()
    yield
    torch.cuda.synchronize()


def _inputs(seed, rows, vocab, dtype):
    f = lce_synth.normal_f32(seed, 0, rows, vocab, 2.0)
    z = to_dev(f if dtype == "f32" else lce_synth.f32_to_bf16_bits(f))
    t = torch.from_numpy(lce_synth.targets(seed + 1, rows, vocab)).cuda()
    return z, t


def _call(fn, z, t, reduction):
    dtype = lce.LCE_F32 if z.dtype == torch.float32 else lce.LCE_BF16
    red = lce.LCE_REDUCTION_MEAN if reduction == "mean" else lce.LCE_REDUCTION_NONE
    out = torch.full((1,) if reduction == "mean" else (z.shape[0],), 123.0, device="cuda")
    st = fn(z.data_ptr(), dtype, z.shape[0], z.shape[1], t.data_ptr(), red, out.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
    assert st == lce.LCE_OK, lce.lce_last_error()
    return out, lce.lce_last_launch()


# (dtype, (rows, vocab) of the first call, (rows, vocab) of the second, smaller call, the
# kernel the default selection launches).  Several rows per wave (rows of at most 2 KiB
# with no scalar edges); one wave per row; one workgroup per row (rows over 32 KiB, no
# mean: the mean takes one wave per row there); split vocab (fewer rows than twice the CU
# count).
CASES = [
    ("bf16", (65536, 512), (1001, 256), "xent_group_rows_kernel"),
    ("f32", (20000, 64), (33, 32), "xent_group_rows_kernel"),
    ("f32", (4099, 3001), (1000, 500), "xent_wave_rows_kernel"),
    ("bf16", (8192, 4096), (777, 4096), "xent_wave_rows_kernel"),
    ("f32", (600, 40000), (513, 20000), "xent_block_rows_kernel"),
    ("bf16", (300, 131072), (37, 70001), "xent_split_partial_kernel"),
    ("f32", (256, 131072), (5, 9000), "xent_split_partial_kernel"),
]


@pytest.mark.parametrize("dtype,big,small,kernel", CASES)
@pytest.mark.parametrize("reduction", ["none", "mean"])
def test_noalloc_matches_allocating_entry_point(dtype, big, small, kernel, reduction):
    for k, (rows, vocab) in enumerate((big, small)):
        z, t = _inputs(rows * 3 + vocab + k, rows, vocab, dtype)
        got, launch = _call(lce.lce_xent_fwd_noalloc, z, t, reduction)
        want, launch_ref = _call(lce.lce_xent_fwd, z, t, reduction)
        torch.cuda.synchronize()
        assert launch == launch_ref, (launch, launch_ref)
        if k == 0 and not (reduction == "mean" and kernel == "xent_block_rows_kernel"):
            assert launch.startswith(kernel), launch
        assert torch.equal(got, want), (dtype, rows, vocab, reduction,
                                        float((got - want).abs().max()))
        assert torch.isfinite(got).all()


def test_noalloc_refuses_sizes_beyond_its_array():
    # A mean over 2^23 + 1 rows of one logit needs 2^19 + 1 workgroup slots.
    rows = (1 << 23) + 1
    z = torch.zeros((rows, 1), device="cuda")
    t = torch.zeros(rows, dtype=torch.int64, device="cuda")
    out = torch.full((1,), 5.0, device="cuda")
    st = lce.lce_xent_fwd_noalloc(z.data_ptr(), lce.LCE_F32, rows, 1, t.data_ptr(),
                                  lce.LCE_REDUCTION_MEAN, out.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == lce.LCE_ERR_UNSUPPORTED
    assert "slots" in lce.lce_last_error()
    torch.cuda.synchronize()
    assert out.item() == 5.0
    # The same rows per token need no slots and are computed (loss 0 for one class).
    got, _ = _call(lce.lce_xent_fwd_noalloc, z, t, "none")
    torch.cuda.synchronize()
    assert torch.all(got == 0)


def test_noalloc_refuses_grouped_means_beyond_its_array():
    """Rows of 16 bytes take 8 rows per wave, 32 per workgroup: a mean over 2^24 + 1 such
    rows needs 2^19 + 1 workgroup slots and is refused before anything is enqueued; the
    same rows per token are computed (ln 4 for four equal logits)."""
    rows = (1 << 24) + 1
    z = torch.zeros((rows, 4), device="cuda")
    t = torch.zeros(rows, dtype=torch.int64, device="cuda")
    out = torch.full((1,), 5.0, device="cuda")
    st = lce.lce_xent_fwd_noalloc(z.data_ptr(), lce.LCE_F32, rows, 4, t.data_ptr(),
                                  lce.LCE_REDUCTION_MEAN, out.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == lce.LCE_ERR_UNSUPPORTED
    assert "slots" in lce.lce_last_error()
    torch.cuda.synchronize()
    assert out.item() == 5.0
    got, launch = _call(lce.lce_xent_fwd_noalloc, z, t, "none")
    torch.cuda.synchronize()
    assert launch.startswith("xent_group_rows_kernel"), launch
    assert torch.all((got - float(np.log(4.0))).abs() <= 1e-6)
    # 2^24 rows fill the 2^19 slots exactly
    st = lce.lce_xent_fwd_noalloc(z.data_ptr(), lce.LCE_F32, rows - 1, 4, t.data_ptr(),
                                  lce.LCE_REDUCTION_MEAN, out.data_ptr(),
                                  torch.cuda.current_stream().cuda_stream)
    assert st == lce.LCE_OK, lce.lce_last_error()
    torch.cuda.synchronize()
    assert abs(out.item() - float(np.log(4.0))) <= 1e-6
    del z, t, got
    torch.cuda.empty_cache()
