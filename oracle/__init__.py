"""Cross-entropy oracle: the slow, plain, fp64 CPU definition of what liblce computes.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code with
the HIP library (``vocab_cross_entropy_row_amd``) and imports nothing from it;
the only code both sides use is the seeded input generator in ``lce_synth``.

Sources (KernelIndex pages; the formula itself is never printed there):

* "Cross-entropy loss" -- description and Semantics block: logits
  ``float [tokens, vocab]``, target ``int64 [tokens]``, loss ``float [1]``.  Read as
  the textbook softmax cross-entropy per token, ``ln sum_j exp(z_ij) - z_{i,t_i}``,
  reduced to the mean over tokens.
* "Vocab-parallel cross-entropy, Megatron layout" -- description and Semantics
  block: logits ``[seq, batch, vocab]``, target ``[seq, batch]``, per-token fp32
  losses ``[seq, batch]`` (no reduction).  At TP=1 this is the same per-row
  formula on the contiguous ``[seq*batch, vocab]`` view.
* "Fused linear + CPO loss" -- description and Semantics block: activations
  ``[batch, seq, hidden]`` projected through a ``[vocab, hidden]`` head,
  ``z = x W^T``, with the logits never materialised.  The oracle does
  materialise them (in fp64): it computes ``z`` with a plain fp64 matrix
  product (a library primitive) and then applies the same per-row formula.

Every function here is pinned by tests that do not reuse its arithmetic:
closed forms, invariants, brute force in 40-digit decimal arithmetic, and a
library routine (see ``tests/test_oracle_pins.py``).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "xent_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_DTYPES = {"f32": 0, "bf16": 1, "f64": 2}
_lib = None


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (plain -O2, no fast-math, OpenMP over rows)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
               "-fno-fast-math", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_xent_rows.restype = ctypes.c_int
        lib.oracle_xent_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                         ctypes.c_int]
        lib.oracle_mean.restype = ctypes.c_double
        lib.oracle_mean.argtypes = [ctypes.c_void_p, ctypes.c_int64]
        lib.oracle_xent_partial.restype = ctypes.c_int
        lib.oracle_xent_partial.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                            ctypes.c_void_p, ctypes.c_int]
        lib.oracle_xent_merge.restype = ctypes.c_int
        lib.oracle_xent_merge.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                          ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_xent_bwd_rows.restype = ctypes.c_int
        lib.oracle_xent_bwd_rows.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_default_threads.restype = ctypes.c_int
        lib.oracle_default_threads.argtypes = []
        _lib = lib
    return _lib


def default_threads() -> int:
    """Host threads the oracle uses when none are given: the CPUs this process may
    run on, capped by OMP_NUM_THREADS when that is set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _dtype_of(logits: np.ndarray, dtype: str | None) -> str:
    if dtype is not None:
        return dtype
    if logits.dtype == np.float32:
        return "f32"
    if logits.dtype == np.float64:
        return "f64"
    if logits.dtype == np.uint16:
        return "bf16"
    raise TypeError(f"oracle: unsupported logits dtype {logits.dtype}")


def xent_rows(logits: np.ndarray, target: np.ndarray, dtype: str | None = None,
              nthreads: int | None = None) -> np.ndarray:
    """Per-token losses ``ln sum_j exp(z_ij) - z_{i,t_i}`` in fp64.

    ``logits`` is ``[..., vocab]`` (any leading shape, row-major): float32, float64,
    or uint16 holding bf16 bit patterns.  ``target`` has the leading shape.  The
    result has the leading shape.  Out-of-range targets give NaN.
    """
    dt = _dtype_of(logits, dtype)
    z = np.ascontiguousarray(logits)
    t = np.ascontiguousarray(target, dtype=np.int64)
    vocab = int(z.shape[-1])
    lead = z.shape[:-1]
    if t.shape != lead:
        raise ValueError(f"oracle: target shape {t.shape} != logits leading shape {lead}")
    rows = int(np.prod(lead, dtype=np.int64)) if lead else 1
    out = np.empty(rows, dtype=np.float64)
    rc = _load().oracle_xent_rows(z.ctypes.data, _DTYPES[dt], rows, vocab, t.ctypes.data,
                                  out.ctypes.data, int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: bad argument")
    return out.reshape(lead)


def xent_partial(logits: np.ndarray, target: np.ndarray, vocab_start: int,
                 dtype: str | None = None, nthreads: int | None = None) -> np.ndarray:
    """Statistics of one vocab shard, ``[rows, 3]`` fp64: (m, s, zt) per row.

    ``logits`` is ``[rows, shard]`` holding full-vocab columns
    ``[vocab_start, vocab_start + shard)``; ``target`` indexes the full vocab.
    m = max, s = sum exp(z - m), zt = the target's logit if this shard holds it,
    else NaN ("Vocab-parallel cross-entropy, Megatron layout": description).
    """
    dt = _dtype_of(logits, dtype)
    z = np.ascontiguousarray(logits)
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(-1)
    if z.ndim != 2 or t.size != z.shape[0]:
        raise ValueError("oracle: logits must be [rows, shard] and target [rows]")
    out = np.empty((z.shape[0], 3), dtype=np.float64)
    rc = _load().oracle_xent_partial(z.ctypes.data, _DTYPES[dt], z.shape[0], z.shape[1],
                                     int(vocab_start), t.ctypes.data, out.ctypes.data,
                                     int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: bad argument")
    return out


def xent_merge(partials: np.ndarray, target: np.ndarray, vocab: int) -> np.ndarray:
    """Per-token losses from ``[shards, rows, 3]`` shard statistics (fp64)."""
    q = np.ascontiguousarray(partials, dtype=np.float64)
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(-1)
    if q.ndim != 3 or q.shape[2] != 3 or q.shape[1] != t.size:
        raise ValueError("oracle: partials must be [shards, rows, 3]")
    out = np.empty(t.size, dtype=np.float64)
    rc = _load().oracle_xent_merge(q.ctypes.data, q.shape[0], q.shape[1], t.ctypes.data,
                                   int(vocab), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle: bad argument")
    return out


def xent_bwd(logits: np.ndarray, target: np.ndarray, grad, reduction: str = "mean",
             dtype: str | None = None, nthreads: int | None = None) -> np.ndarray:
    """Gradient of the loss with respect to the logits, fp64, the logits' shape.

    ``grad`` is the gradient of the loss output: a scalar for ``"mean"`` (each row
    then gets grad / tokens), one value per token for ``"none"``.  Rows with an
    out-of-range target are NaN.  (The pages give the forward only; this is its
    derivative, softmax minus the one-hot target.)
    """
    if reduction not in ("mean", "none"):
        raise ValueError(f"oracle: unknown reduction {reduction!r}")
    dt = _dtype_of(logits, dtype)
    z = np.ascontiguousarray(logits)
    t = np.ascontiguousarray(target, dtype=np.int64)
    vocab = int(z.shape[-1])
    rows = int(np.prod(z.shape[:-1], dtype=np.int64)) if z.ndim > 1 else 1
    if t.size != rows:
        raise ValueError("oracle: target must have one entry per row")
    g = np.ascontiguousarray(np.asarray(grad, dtype=np.float64).reshape(-1))
    if g.size != (1 if reduction == "mean" else rows):
        raise ValueError("oracle: grad must be a scalar (mean) or one value per token (none)")
    out = np.empty((rows, vocab), dtype=np.float64)
    rc = _load().oracle_xent_bwd_rows(z.ctypes.data, _DTYPES[dt], rows, vocab, t.ctypes.data,
                                      1 if reduction == "mean" else 0, g.ctypes.data,
                                      out.ctypes.data, int(nthreads or default_threads()))
    if rc != 0:
        raise ValueError("oracle: bad argument")
    return out.reshape(z.shape)


def mean(losses: np.ndarray) -> float:
    """Mean of per-token losses, summed in index order in fp64 (NaN for no tokens)."""
    l64 = np.ascontiguousarray(losses, dtype=np.float64).reshape(-1)
    return float(_load().oracle_mean(l64.ctypes.data, l64.size))


def xent(logits: np.ndarray, target: np.ndarray, reduction: str = "mean",
         dtype: str | None = None, nthreads: int | None = None):
    """Cross-entropy with ``reduction`` in {"mean", "none"}."""
    per_token = xent_rows(logits, target, dtype=dtype, nthreads=nthreads)
    if reduction == "none":
        return per_token
    if reduction == "mean":
        return mean(per_token)
    raise ValueError(f"oracle: unknown reduction {reduction!r}")


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64."""
    u32 = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def fused_linear_xent_rows(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray,
                           rows: np.ndarray | None = None, block: int = 128,
                           nthreads: int | None = None) -> np.ndarray:
    """Per-token losses of ``x W^T`` against ``target`` (selected rows), in fp64.

    Token rows are processed ``block`` at a time (rows are independent), so only a
    ``[block, vocab]`` slab of fp64 logits exists at once.
    """
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w_bits = np.ascontiguousarray(w_bits, dtype=np.uint16)
    target = np.ascontiguousarray(target, dtype=np.int64).reshape(-1)
    if x_bits.ndim != 2 or w_bits.ndim != 2 or x_bits.shape[1] != w_bits.shape[1]:
        raise ValueError("oracle: x must be [tokens, hidden] and W [vocab, hidden]")
    sel = np.arange(x_bits.shape[0]) if rows is None else np.asarray(rows, dtype=np.int64)
    w64t = bf16_bits_to_f64(w_bits).T
    out = np.empty(sel.size, dtype=np.float64)
    for b0 in range(0, sel.size, block):
        r = sel[b0:b0 + block]
        z = np.matmul(bf16_bits_to_f64(x_bits[r]), w64t)
        out[b0:b0 + block] = xent_rows(z, target[r], dtype="f64", nthreads=nthreads)
    return out


def fused_linear_xent(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray,
                      reduction: str = "mean", nthreads: int | None = None):
    """Fused linear + cross-entropy, ``reduction`` in {"mean", "none"}."""
    per_token = fused_linear_xent_rows(x_bits, w_bits, target, nthreads=nthreads)
    if reduction == "none":
        return per_token
    if reduction == "mean":
        return mean(per_token)
    raise ValueError(f"oracle: unknown reduction {reduction!r}")


def fused_linear_logprob_sums(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray,
                              batch: int, seq: int, nthreads: int | None = None) -> np.ndarray:
    """Per-sequence sums of target log-probabilities under ``x W^T``, fp64 ``[batch]``.

    Tokens are ordered row = b * seq + s (the CPO page's ``x [batch, seq, hidden]``,
    flattened); entry b is sum_s log softmax(z_{b,s})[t_{b,s}] = -sum_s loss_{b,s},
    summed exactly (``math.fsum``).  These sums are what the "Fused linear + CPO loss"
    page's preference loss is built from; its formula is not on the page.
    """
    import math
    per = fused_linear_xent_rows(x_bits, w_bits, target, nthreads=nthreads)
    if per.size != batch * seq:
        raise ValueError("oracle: tokens must equal batch * seq")
    per = per.reshape(batch, seq)
    return np.array([-math.fsum(per[b]) for b in range(batch)], dtype=np.float64)


def fused_linear_xent_grads(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray,
                            row_scale: np.ndarray, block: int = 64, want_dw: bool = True):
    """Gradients of the fused cross-entropy with respect to the activations and the head,
    fp64, for per-row output-gradient scales ``row_scale`` (g_i).

    The pages give only the forward; this is its derivative written out.  With
    z = x W^T (exactly widened bf16 operands, fp64 product), the logit gradient of row i
    is dZ_i = g_i (softmax(z_i) - onehot(t_i)) (``xent_bwd`` on the fp64 logits), and
    by the chain rule dx = dZ W and dW = dZ^T x (library matrix products).  Rows with an
    out-of-range target are NaN, and so is all of dW.  Returns ``(dx, dW)`` (``dW`` is
    None when ``want_dw`` is false).
    """
    x64_all = bf16_bits_to_f64(x_bits)
    w64 = bf16_bits_to_f64(w_bits)
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(-1)
    g = np.ascontiguousarray(row_scale, dtype=np.float64).reshape(-1)
    rows = x64_all.shape[0]
    if t.size != rows or g.size != rows:
        raise ValueError("oracle: target and row_scale must have one entry per row")
    dx = np.empty((rows, w64.shape[1]), dtype=np.float64)
    dw = np.zeros_like(w64) if want_dw else None
    for b0 in range(0, rows, block):
        x64 = x64_all[b0:b0 + block]
        z = np.matmul(x64, w64.T)
        dz = xent_bwd(z, t[b0:b0 + block], g[b0:b0 + block], reduction="none", dtype="f64")
        dx[b0:b0 + block] = np.matmul(dz, w64)
        if want_dw:
            dw += np.matmul(dz.T, x64)
    return dx, dw


def fused_linear_xent_dw_rows(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray,
                              row_scale: np.ndarray, head_rows: np.ndarray, block: int = 128):
    """Selected rows of the head gradient dW = dZ^T x, fp64, for per-token scales g_i.

    The same derivative as ``fused_linear_xent_grads``, for a head too large to hold
    all of dW or dZ in fp64: each block of tokens gets its full fp64 logits and their
    logit gradient (``xent_bwd``, which needs every logit of the row for the softmax),
    and only the columns of dZ for ``head_rows`` are kept.  Row r of the result is
    sum_i dZ[i, head_rows[r]] x_i.  Returns ``(dw_rows [k, hidden], dz_cols [tokens, k])``.
    """
    x64_all = bf16_bits_to_f64(x_bits)
    w64 = bf16_bits_to_f64(w_bits)
    t = np.ascontiguousarray(target, dtype=np.int64).reshape(-1)
    g = np.ascontiguousarray(row_scale, dtype=np.float64).reshape(-1)
    sel = np.asarray(head_rows, dtype=np.int64).reshape(-1)
    rows = x64_all.shape[0]
    if t.size != rows or g.size != rows:
        raise ValueError("oracle: target and row_scale must have one entry per row")
    if sel.size and (sel.min() < 0 or sel.max() >= w64.shape[0]):
        raise ValueError("oracle: head_rows outside the head")
    dz_cols = np.empty((rows, sel.size), dtype=np.float64)
    for b0 in range(0, rows, block):
        z = np.matmul(x64_all[b0:b0 + block], w64.T)
        dz = xent_bwd(z, t[b0:b0 + block], g[b0:b0 + block], reduction="none", dtype="f64")
        dz_cols[b0:b0 + block] = dz[:, sel]
    return np.matmul(dz_cols.T, x64_all), dz_cols


def fused_linear_xent_bwd(x_bits: np.ndarray, w_bits: np.ndarray, target: np.ndarray, grad,
                          reduction: str = "mean"):
    """``(dx, dW)`` of the fused cross-entropy for the output gradient ``grad``: a scalar
    for ``"mean"`` (each row then gets grad / tokens), one value per token for ``"none"``."""
    rows = int(np.asarray(x_bits).shape[0])
    g = np.asarray(grad, dtype=np.float64).reshape(-1)
    if reduction == "mean":
        if g.size != 1:
            raise ValueError("oracle: grad must be a scalar for mean")
        scale = np.full(rows, g[0] / rows)
    elif reduction == "none":
        if g.size != rows:
            raise ValueError("oracle: grad must have one value per token for none")
        scale = g
    else:
        raise ValueError(f"oracle: unknown reduction {reduction!r}")
    return fused_linear_xent_grads(x_bits, w_bits, target, scale)


def _log_softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row-wise log-softmax in fp64 by the same two plain passes as the C oracle
    (maximum, then the sum of exp(z - m)); vectorised over the rows of a block."""
    m = z.max(axis=1, keepdims=True)
    s = np.exp(z - m).sum(axis=1, keepdims=True)
    return z - (m + np.log(s))


def fused_linear_jsd_rows(xs_bits: np.ndarray, ws_bits: np.ndarray, xt_bits: np.ndarray,
                          wt_bits: np.ndarray, beta: float = 0.5, block: int = 64) -> np.ndarray:
    """Per-token generalized Jensen-Shannon divergence between the student and teacher
    distributions, fp64 ("Fused linear + JSD": description and Semantics block).

    P = softmax(x_s W_s^T) (student), Q = softmax(x_t W_t^T) (teacher), M = beta P +
    (1 - beta) Q, and per token JSD = beta KL(P || M) + (1 - beta) KL(Q || M) with
    KL(A || B) = sum_j A_j ln(A_j / B_j) (0 ln 0 = 0).  The page names "generalized JSD
    (beta 0.5)" without printing it; this is the plain reading, symmetric at beta = 0.5.
    Logits come from exactly widened bf16 operands and an fp64 matrix product.
    """
    xs_bits = np.ascontiguousarray(xs_bits, dtype=np.uint16)
    xt_bits = np.ascontiguousarray(xt_bits, dtype=np.uint16)
    ws64 = bf16_bits_to_f64(ws_bits).T
    wt64 = bf16_bits_to_f64(wt_bits).T
    rows = xs_bits.shape[0]
    out = np.empty(rows, dtype=np.float64)
    for b0 in range(0, rows, block):
        lp = _log_softmax_rows(np.matmul(bf16_bits_to_f64(xs_bits[b0:b0 + block]), ws64))
        lq = _log_softmax_rows(np.matmul(bf16_bits_to_f64(xt_bits[b0:b0 + block]), wt64))
        P, Q = np.exp(lp), np.exp(lq)
        M = beta * P + (1.0 - beta) * Q
        with np.errstate(divide="ignore", invalid="ignore"):
            logM = np.log(M)
            kp = np.where(P > 0, P * (lp - logM), 0.0).sum(axis=1)
            kq = np.where(Q > 0, Q * (lq - logM), 0.0).sum(axis=1)
        out[b0:b0 + block] = beta * kp + (1.0 - beta) * kq
    return out


def fused_linear_jsd(xs_bits, ws_bits, xt_bits, wt_bits, beta: float = 0.5,
                     reduction: str = "mean"):
    """Generalized JSD loss: "mean" is the page's batchmean (sum over tokens / tokens)."""
    per = fused_linear_jsd_rows(xs_bits, ws_bits, xt_bits, wt_bits, beta)
    if reduction == "none":
        return per
    if reduction == "mean":
        return mean(per)
    raise ValueError(f"oracle: unknown reduction {reduction!r}")
