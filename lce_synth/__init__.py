"""Seeded synthetic inputs for liblce's workloads.

This module holds no cross-entropy arithmetic.  It only draws inputs, and it is
the one piece of code that both the HIP path (tests, benchmark) and the fp64
oracle consume, so both see the very same bytes.

Recipe (the pages give shapes and dtypes but no value distributions; the
KernelIndex "Cross-entropy loss" description states only that its benchmark
logits are fp32):

* Values are drawn in chunks of ``CHUNK_ROWS`` rows.  Chunk ``c`` of stream ``s``
  under seed ``k`` uses ``numpy.random.Generator(PCG64(SeedSequence([k, s, c])))``,
  so any row range can be regenerated alone, chunks can be drawn in parallel, and
  the host never holds more than the rows asked for.
* Normal values: ``standard_normal(dtype=float32) * std`` in float32.
* bf16 values: the float32 draw rounded to nearest, ties to even, on the bit
  pattern (returned as uint16 bit patterns).
* Targets: ``integers(0, vocab, dtype=int64)``, independent per token, from their
  own stream.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK_ROWS = 256

STREAM_LOGITS = 0
STREAM_TARGET = 1
STREAM_WEIGHT = 2


def _rng(seed: int, stream: int, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, chunk])))


def _workers(threads: int | None) -> int:
    if threads:
        return max(1, int(threads))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunks(rows: int, row0: int, row1: int):
    c0 = row0 // CHUNK_ROWS
    c1 = (row1 + CHUNK_ROWS - 1) // CHUNK_ROWS
    for c in range(c0, c1):
        lo = c * CHUNK_ROWS
        hi = min(rows, lo + CHUNK_ROWS)
        yield c, lo, hi


def normal_f32(seed: int, stream: int, rows: int, cols: int, std: float = 1.0,
               row0: int = 0, row1: int | None = None, threads: int | None = None,
               out: np.ndarray | None = None) -> np.ndarray:
    """Rows ``[row0, row1)`` of a seeded ``[rows, cols]`` float32 N(0, std^2) matrix."""
    row1 = rows if row1 is None else row1
    if not (0 <= row0 <= row1 <= rows):
        raise ValueError("row range outside the matrix")
    if out is None:
        out = np.empty((row1 - row0, cols), dtype=np.float32)
    std32 = np.float32(std)

    def fill(job):
        c, lo, hi = job
        blk = _rng(seed, stream, c).standard_normal(size=(hi - lo, cols), dtype=np.float32)
        if std32 != np.float32(1.0):
            blk *= std32
        a, b = max(lo, row0), min(hi, row1)
        out[a - row0:b - row0] = blk[a - lo:b - lo]

    jobs = list(_chunks(rows, row0, row1))
    if len(jobs) <= 1:
        for j in jobs:
            fill(j)
    else:
        with ThreadPoolExecutor(_workers(threads)) as ex:
            list(ex.map(fill, jobs))
    return out


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16, nearest with ties to even; returns uint16 bit patterns.

    (Inputs are finite draws; NaN/Inf handling is not needed for the generator.)
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def normal_bf16_bits(seed: int, stream: int, rows: int, cols: int, std: float = 1.0,
                     row0: int = 0, row1: int | None = None,
                     threads: int | None = None) -> np.ndarray:
    """Rows ``[row0, row1)`` of the bf16 rounding of :func:`normal_f32` (uint16 bits)."""
    row1 = rows if row1 is None else row1
    out = np.empty((row1 - row0, cols), dtype=np.uint16)

    def fill(job):
        c, lo, hi = job
        a, b = max(lo, row0), min(hi, row1)
        f = normal_f32(seed, stream, rows, cols, std, row0=a, row1=b, threads=1)
        out[a - row0:b - row0] = f32_to_bf16_bits(f)

    jobs = list(_chunks(rows, row0, row1))
    with ThreadPoolExecutor(_workers(threads)) as ex:
        list(ex.map(fill, jobs))
    return out


def targets(seed: int, rows: int, vocab: int, row0: int = 0,
            row1: int | None = None) -> np.ndarray:
    """Rows ``[row0, row1)`` of seeded int64 targets, uniform on ``[0, vocab)``."""
    row1 = rows if row1 is None else row1
    out = np.empty(row1 - row0, dtype=np.int64)
    for c, lo, hi in _chunks(rows, row0, row1):
        blk = _rng(seed, STREAM_TARGET, c).integers(0, vocab, size=hi - lo, dtype=np.int64)
        a, b = max(lo, row0), min(hi, row1)
        out[a - row0:b - row0] = blk[a - lo:b - lo]
    return out


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shapes, dtype, distribution and seeds."""
    name: str
    kind: str            # "xent" or "fused"
    dtype: str           # "f32" or "bf16" (logits, or x and W for "fused")
    shape: tuple         # logits shape ([tokens, vocab] or [seq, batch, vocab]); fused: (tokens, hidden, vocab)
    reduction: str       # "mean" or "none"
    std: float           # std of logits (xent) or of x (fused)
    seed: int            # seed of logits / x
    target_seed: int
    w_std: float = 0.0   # fused only
    w_seed: int = 0      # fused only

    @property
    def tokens(self) -> int:
        if self.kind == "fused":
            return int(self.shape[0])
        return int(np.prod(self.shape[:-1]))

    @property
    def vocab(self) -> int:
        return int(self.shape[2] if self.kind == "fused" else self.shape[-1])

    @property
    def hidden(self) -> int:
        return int(self.shape[1]) if self.kind == "fused" else 0

    @property
    def target_shape(self) -> tuple:
        return (self.tokens,) if self.kind == "fused" else tuple(self.shape[:-1])

    def logits(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        """Token rows ``[row0, row1)`` of the logits as ``[rows, vocab]`` (f32 or bf16 bits)."""
        assert self.kind == "xent"
        if self.dtype == "f32":
            return normal_f32(self.seed, STREAM_LOGITS, self.tokens, self.vocab, self.std,
                              row0, row1, threads)
        return normal_bf16_bits(self.seed, STREAM_LOGITS, self.tokens, self.vocab, self.std,
                                row0, row1, threads)

    def x(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        """Token rows of the bf16 activations ``[rows, hidden]`` (uint16 bits)."""
        assert self.kind == "fused"
        return normal_bf16_bits(self.seed, STREAM_LOGITS, self.tokens, self.hidden, self.std,
                                row0, row1, threads)

    def weight(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        """Vocab rows of the bf16 LM-head weight ``[rows, hidden]`` (uint16 bits)."""
        assert self.kind == "fused"
        return normal_bf16_bits(self.w_seed, STREAM_WEIGHT, self.vocab, self.hidden, self.w_std,
                                row0, row1, threads)

    def target(self, row0: int = 0, row1: int | None = None) -> np.ndarray:
        """Token rows of the int64 targets (flattened)."""
        return targets(self.target_seed, self.tokens, self.vocab, row0, row1)


# The five synthetic workloads.  Shapes follow the pages' benchmark sweeps:
# "Cross-entropy loss" (vocab 4096..131072, tokens 16384, fp32),
# "Vocab-parallel cross-entropy, Megatron layout" (seq 2048, batch 4,
# vocab 4096..131072, bf16) and "Fused linear + CPO loss" (batch 2, seq 1024,
# vocab 128256, hidden 4096, bf16).
WORKLOADS = {
    "ce_f32_16384x4096_mean": Workload(
        "ce_f32_16384x4096_mean", "xent", "f32", (16384, 4096), "mean", 1.0, 1001, 2001),
    "megatron_bf16_2048x4x4096_none": Workload(
        "megatron_bf16_2048x4x4096_none", "xent", "bf16", (2048, 4, 4096), "none", 1.0, 1002, 2002),
    "ce_f32_16384x131072_mean": Workload(
        "ce_f32_16384x131072_mean", "xent", "f32", (16384, 131072), "mean", 1.0, 1003, 2003),
    "megatron_bf16_2048x4x131072_none": Workload(
        "megatron_bf16_2048x4x131072_none", "xent", "bf16", (2048, 4, 131072), "none", 2.0, 1004, 2004),
    "fused_bf16_t2048_h4096_v128256_mean": Workload(
        "fused_bf16_t2048_h4096_v128256_mean", "fused", "bf16", (2048, 4096, 128256), "mean", 1.0,
        1005, 2005, w_std=0.02, w_seed=3005),
}

@dataclasses.dataclass(frozen=True)
class JsdWorkload:
    """Student and teacher activations and heads for the fused linear + JSD workload:
    four independent bf16 draws, activations N(0, x_std^2) and heads N(0, w_std^2)."""
    name: str
    tokens: int
    hidden: int
    vocab: int
    x_std: float
    w_std: float
    seeds: tuple         # (student x, student head, teacher x, teacher head)
    reduction: str = "mean"

    def student_x(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        return normal_bf16_bits(self.seeds[0], STREAM_LOGITS, self.tokens, self.hidden, self.x_std,
                                row0, row1, threads)

    def student_weight(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        return normal_bf16_bits(self.seeds[1], STREAM_WEIGHT, self.vocab, self.hidden, self.w_std,
                                row0, row1, threads)

    def teacher_x(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        return normal_bf16_bits(self.seeds[2], STREAM_LOGITS, self.tokens, self.hidden, self.x_std,
                                row0, row1, threads)

    def teacher_weight(self, row0: int = 0, row1: int | None = None, threads: int | None = None):
        return normal_bf16_bits(self.seeds[3], STREAM_WEIGHT, self.vocab, self.hidden, self.w_std,
                                row0, row1, threads)


# "Fused linear + JSD" (tokens 1024 of the page's 1024..8192 sweep, hidden 4096,
# vocab 128256, bf16, beta 0.5, batchmean).  Head std 0.02 gives logits of std
# about 1.3, as for the fused cross-entropy workload.
JSD = JsdWorkload("jsd_bf16_t1024_h4096_v128256_mean", 1024, 4096, 128256, 1.0, 0.02,
                  (1006, 3006, 1007, 3007))

# The small case the oracle finishes in seconds, and the headline benchmark workload:
# the largest configuration that fits one GPU (fp32 logits [16384, 131072], 8.6 GB).
SMALL = "ce_f32_16384x4096_mean"
HEADLINE = "ce_f32_16384x131072_mean"
