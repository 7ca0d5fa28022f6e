"""Python binding for liblce (argument marshalling only; all compute runs in HIP kernels).

The raw C-ABI calls keep their C names and take plain integers (device addresses,
sizes, enum values, a ``hipStream_t`` as an integer) and return the ``lce_status``
code:

* :func:`lce_xent_fwd`, :func:`lce_fused_linear_xent_fwd`
* :func:`lce_xent_fwd_noalloc` (lce_xent_fwd with static scratch: allocates nothing)
* :func:`lce_xent_bwd` (gradient with respect to the logits)
* :func:`lce_fused_linear_logprob_sums` (per-sequence target log-probability sums)
* :func:`lce_xent_partial_fwd`, :func:`lce_xent_merge` (vocab split across devices)
* :func:`lce_status_string`, :func:`lce_last_error`, :func:`lce_last_launch`, :func:`lce_version`

:func:`xent`, :func:`xent_bwd`, :func:`fused_linear_xent`, :func:`xent_partial` and :func:`xent_merge`
are thin conveniences over them for
torch tensors: they check device/dtype/contiguity, allocate the fp32 output with
torch, pass ``data_ptr()`` values and torch's current HIP stream, and raise
:class:`LceError` on a non-zero status.  There is no CPU fallback: if
``liblce.so`` is not built, every call raises.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liblce.so")

LCE_F32 = 0
LCE_BF16 = 1
LCE_REDUCTION_MEAN = 0
LCE_REDUCTION_NONE = 1

LCE_OK = 0
LCE_ERR_INVALID_ARG = 1
LCE_ERR_UNSUPPORTED = 2
LCE_ERR_ALIAS = 3
LCE_ERR_OOM = 4
LCE_ERR_HIP = 5

EXPORTED = ("lce_xent_fwd", "lce_xent_fwd_noalloc", "lce_xent_bwd", "lce_xent_fwd_bwd",
            "lce_fused_linear_xent_fwd", "lce_fused_linear_xent_bwd", "lce_fused_linear_xent_fwd_bwd",
            "lce_fused_linear_logprob_sums", "lce_fused_linear_jsd_fwd", "lce_xent_partial_fwd",
            "lce_xent_merge", "lce_status_string", "lce_last_error", "lce_last_launch",
            "lce_version")

_lib = None


class LceError(RuntimeError):
    """A liblce call returned a non-zero status."""

    def __init__(self, status: int, where: str):
        self.status = int(status)
        msg = f"{where}: {lce_status_string(status)}: {lce_last_error()}"
        super().__init__(msg)


def load() -> ctypes.CDLL:
    """Load the in-tree liblce.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"liblce.so not found at {LIB_PATH}; build it with "
            "`python -m vocab_cross_entropy_row_amd.build` (there is no CPU fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    lib.lce_xent_fwd.restype = ctypes.c_int
    lib.lce_xent_fwd.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_xent_fwd_noalloc.restype = ctypes.c_int
    lib.lce_xent_fwd_noalloc.argtypes = lib.lce_xent_fwd.argtypes
    lib.lce_fused_linear_xent_fwd.restype = ctypes.c_int
    lib.lce_fused_linear_xent_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_xent_bwd.restype = ctypes.c_int
    lib.lce_xent_bwd.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                 ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                 ctypes.c_void_p]
    lib.lce_xent_fwd_bwd.restype = ctypes.c_int
    lib.lce_xent_fwd_bwd.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_fused_linear_logprob_sums.restype = ctypes.c_int
    lib.lce_fused_linear_logprob_sums.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_fused_linear_jsd_fwd.restype = ctypes.c_int
    lib.lce_fused_linear_jsd_fwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_fused_linear_xent_bwd.restype = ctypes.c_int
    lib.lce_fused_linear_xent_bwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                              ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_fused_linear_xent_fwd_bwd.restype = ctypes.c_int
    lib.lce_fused_linear_xent_fwd_bwd.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                                  ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                                  ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_xent_partial_fwd.restype = ctypes.c_int
    lib.lce_xent_partial_fwd.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_xent_merge.restype = ctypes.c_int
    lib.lce_xent_merge.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                   ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_void_p, ctypes.c_void_p]
    lib.lce_status_string.restype = ctypes.c_char_p
    lib.lce_status_string.argtypes = [ctypes.c_int]
    lib.lce_last_error.restype = ctypes.c_char_p
    lib.lce_last_error.argtypes = []
    lib.lce_last_launch.restype = ctypes.c_char_p
    lib.lce_last_launch.argtypes = []
    lib.lce_version.restype = ctypes.c_int
    lib.lce_version.argtypes = []
    _lib = lib
    return lib


# ------------------------------------------------------------------ raw C ABI

def lce_xent_fwd(logits: int, dtype: int, tokens: int, vocab: int, target: int,
                 reduction: int, out: int, stream: int) -> int:
    return load().lce_xent_fwd(logits or None, dtype, tokens, vocab, target or None, reduction,
                               out or None, stream or None)


def lce_xent_fwd_noalloc(logits: int, dtype: int, tokens: int, vocab: int, target: int,
                         reduction: int, out: int, stream: int) -> int:
    return load().lce_xent_fwd_noalloc(logits or None, dtype, tokens, vocab, target or None,
                                       reduction, out or None, stream or None)


def lce_fused_linear_xent_fwd(x: int, weight: int, tokens: int, hidden: int, vocab: int,
                              target: int, reduction: int, out: int, stream: int) -> int:
    return load().lce_fused_linear_xent_fwd(x or None, weight or None, tokens, hidden, vocab,
                                            target or None, reduction, out or None,
                                            stream or None)


def lce_xent_bwd(logits: int, dtype: int, tokens: int, vocab: int, target: int, reduction: int,
                 grad: int, dlogits: int, stream: int) -> int:
    return load().lce_xent_bwd(logits or None, dtype, tokens, vocab, target or None, reduction,
                               grad or None, dlogits or None, stream or None)


def lce_xent_fwd_bwd(logits: int, dtype: int, tokens: int, vocab: int, target: int,
                     reduction: int, grad: int, out: int, dlogits: int, stream: int) -> int:
    return load().lce_xent_fwd_bwd(logits or None, dtype, tokens, vocab, target or None, reduction,
                                   grad or None, out or None, dlogits or None, stream or None)


def lce_fused_linear_logprob_sums(x: int, weight: int, batch: int, seq: int, hidden: int,
                                  vocab: int, target: int, out: int, stream: int) -> int:
    return load().lce_fused_linear_logprob_sums(x or None, weight or None, batch, seq, hidden, vocab,
                                                target or None, out or None, stream or None)


def lce_fused_linear_xent_bwd(x: int, weight: int, tokens: int, hidden: int, vocab: int,
                              target: int, reduction: int, grad: int, dx: int, dweight: int,
                              stream: int) -> int:
    return load().lce_fused_linear_xent_bwd(x or None, weight or None, tokens, hidden, vocab,
                                            target or None, reduction, grad or None, dx or None,
                                            dweight or None, stream or None)


def lce_fused_linear_xent_fwd_bwd(x: int, weight: int, tokens: int, hidden: int, vocab: int,
                                  target: int, reduction: int, grad: int, out: int, dx: int,
                                  dweight: int, stream: int) -> int:
    return load().lce_fused_linear_xent_fwd_bwd(x or None, weight or None, tokens, hidden, vocab,
                                                target or None, reduction, grad or None, out or None,
                                                dx or None, dweight or None, stream or None)


def lce_fused_linear_jsd_fwd(student_x: int, student_weight: int, teacher_x: int,
                             teacher_weight: int, tokens: int, hidden: int, vocab: int,
                             beta: float, reduction: int, out: int, stream: int) -> int:
    return load().lce_fused_linear_jsd_fwd(student_x or None, student_weight or None,
                                           teacher_x or None, teacher_weight or None, tokens,
                                           hidden, vocab, beta, reduction, out or None,
                                           stream or None)


def lce_xent_partial_fwd(logits: int, dtype: int, tokens: int, shard_vocab: int,
                         vocab_start: int, target: int, partial: int, stream: int) -> int:
    return load().lce_xent_partial_fwd(logits or None, dtype, tokens, shard_vocab, vocab_start,
                                       target or None, partial or None, stream or None)


def lce_xent_merge(partials: int, shards: int, tokens: int, target: int, vocab: int,
                   reduction: int, out: int, stream: int) -> int:
    return load().lce_xent_merge(partials or None, shards, tokens, target or None, vocab,
                                 reduction, out or None, stream or None)


def lce_status_string(status: int) -> str:
    return load().lce_status_string(int(status)).decode()


def lce_last_error() -> str:
    return load().lce_last_error().decode()


def lce_version() -> int:
    return load().lce_version()


def lce_last_launch() -> str:
    """Kernels (with template arguments and grids) the last call on this thread enqueued."""
    return load().lce_last_launch().decode()


# ------------------------------------------------------------------ torch conveniences

_REDUCTIONS = {"mean": LCE_REDUCTION_MEAN, "none": LCE_REDUCTION_NONE}


def _stream_of(t) -> int:
    import torch
    return torch.cuda.current_stream(t.device).cuda_stream


def xent(logits, target, reduction: str = "mean", out=None):
    """Cross-entropy of ``logits`` ([..., vocab], fp32 or bf16, contiguous, on a HIP device)
    against int64 ``target`` (the leading shape).  Returns fp32: a 1-element tensor for
    ``"mean"``, the leading shape for ``"none"``."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    if not logits.is_cuda or not target.is_cuda:
        raise ValueError("logits and target must be device tensors")
    if logits.dtype == torch.float32:
        dt = LCE_F32
    elif logits.dtype == torch.bfloat16:
        dt = LCE_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if target.dtype != torch.int64:
        raise TypeError(f"target must be int64, got {target.dtype}")
    if not logits.is_contiguous() or not target.is_contiguous():
        raise ValueError("logits and target must be contiguous")
    if logits.dim() < 1 or tuple(target.shape) != tuple(logits.shape[:-1]):
        raise ValueError(f"target shape {tuple(target.shape)} must be logits shape "
                         f"{tuple(logits.shape)} without the vocab axis")
    vocab = logits.shape[-1]
    tokens = target.numel()
    if out is None:
        shape = (1,) if reduction == "mean" else tuple(target.shape)
        out = torch.empty(shape, dtype=torch.float32, device=logits.device)
    st = lce_xent_fwd(logits.data_ptr(), dt, tokens, vocab, target.data_ptr(),
                      _REDUCTIONS[reduction], out.data_ptr(), _stream_of(logits))
    if st != LCE_OK:
        raise LceError(st, "lce_xent_fwd")
    return out


def fused_linear_xent(x, weight, target, reduction: str = "mean", out=None):
    """Cross-entropy of ``x @ weight.T`` against ``target`` without storing the logits.

    ``x``: bf16 [..., hidden]; ``weight``: bf16 [vocab, hidden]; ``target``: int64 with the
    leading shape of ``x``.  Returns fp32 as :func:`xent`."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    for name, t in (("x", x), ("weight", weight), ("target", target)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("x and weight must be bfloat16")
    if target.dtype != torch.int64:
        raise TypeError("target must be int64")
    if weight.dim() != 2 or x.shape[-1] != weight.shape[1]:
        raise ValueError("weight must be [vocab, hidden] with hidden = x.shape[-1]")
    if tuple(target.shape) != tuple(x.shape[:-1]):
        raise ValueError("target shape must be x shape without the hidden axis")
    vocab, hidden = weight.shape
    tokens = target.numel()
    if out is None:
        shape = (1,) if reduction == "mean" else tuple(target.shape)
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    st = lce_fused_linear_xent_fwd(x.data_ptr(), weight.data_ptr(), tokens, hidden, vocab,
                                   target.data_ptr(), _REDUCTIONS[reduction], out.data_ptr(),
                                   _stream_of(x))
    if st != LCE_OK:
        raise LceError(st, "lce_fused_linear_xent_fwd")
    return out


def xent_partial(logits, target, vocab_start: int, out=None):
    """Vocab-shard statistics of ``logits`` ([..., shard_vocab], this device's vocab
    columns starting at ``vocab_start``) for full-vocab ``target``: fp32
    ``[..., 3]`` holding (max, sum of e^(z - max), target logit or NaN) per token."""
    import torch
    if not logits.is_cuda or not target.is_cuda:
        raise ValueError("logits and target must be device tensors")
    if logits.dtype == torch.float32:
        dt = LCE_F32
    elif logits.dtype == torch.bfloat16:
        dt = LCE_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if target.dtype != torch.int64:
        raise TypeError(f"target must be int64, got {target.dtype}")
    if not logits.is_contiguous() or not target.is_contiguous():
        raise ValueError("logits and target must be contiguous")
    if logits.dim() < 1 or tuple(target.shape) != tuple(logits.shape[:-1]):
        raise ValueError("target shape must be logits shape without the vocab axis")
    if out is None:
        out = torch.empty(tuple(target.shape) + (3,), dtype=torch.float32, device=logits.device)
    st = lce_xent_partial_fwd(logits.data_ptr(), dt, target.numel(), logits.shape[-1],
                              int(vocab_start), target.data_ptr(), out.data_ptr(),
                              _stream_of(logits))
    if st != LCE_OK:
        raise LceError(st, "lce_xent_partial_fwd")
    return out


def xent_merge(partials, target, vocab: int, reduction: str = "mean", out=None):
    """Cross-entropy from stacked shard statistics ``partials`` (fp32
    ``[shards, *target.shape, 3]``, shards in a fixed order) against full-vocab ``target``."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    if not partials.is_cuda or not target.is_cuda:
        raise ValueError("partials and target must be device tensors")
    if partials.dtype != torch.float32 or target.dtype != torch.int64:
        raise TypeError("partials must be float32 and target int64")
    if not partials.is_contiguous() or not target.is_contiguous():
        raise ValueError("partials and target must be contiguous")
    if partials.dim() < 2 or partials.shape[-1] != 3 or tuple(partials.shape[1:-1]) != tuple(target.shape):
        raise ValueError("partials must be [shards, *target.shape, 3]")
    if out is None:
        shape = (1,) if reduction == "mean" else tuple(target.shape)
        out = torch.empty(shape, dtype=torch.float32, device=partials.device)
    st = lce_xent_merge(partials.data_ptr(), partials.shape[0], target.numel(), target.data_ptr(),
                        int(vocab), _REDUCTIONS[reduction], out.data_ptr(), _stream_of(partials))
    if st != LCE_OK:
        raise LceError(st, "lce_xent_merge")
    return out


def _xent_bwd_args(logits, target, grad, reduction: str) -> int:
    """Checks shared by the row gradient calls; returns the logits' dtype code."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    if not (logits.is_cuda and target.is_cuda and grad.is_cuda):
        raise ValueError("logits, target and grad must be device tensors")
    if logits.dtype == torch.float32:
        dt = LCE_F32
    elif logits.dtype == torch.bfloat16:
        dt = LCE_BF16
    else:
        raise TypeError(f"logits must be float32 or bfloat16, got {logits.dtype}")
    if target.dtype != torch.int64 or grad.dtype != torch.float32:
        raise TypeError("target must be int64 and grad float32")
    if not (logits.is_contiguous() and target.is_contiguous() and grad.is_contiguous()):
        raise ValueError("logits, target and grad must be contiguous")
    if logits.dim() < 1 or tuple(target.shape) != tuple(logits.shape[:-1]):
        raise ValueError("target shape must be logits shape without the vocab axis")
    if grad.numel() != (1 if reduction == "mean" else target.numel()):
        raise ValueError("grad must have 1 element (mean) or one per token (none)")
    return dt


def _grad_out(logits, out):
    """The gradient buffer: ``out``, or a new tensor like ``logits`` whose data starts at
    the same offset modulo 16 bytes (the library writes gradient rows with the logits'
    16-byte cut)."""
    import torch
    if out is None:
        off = (logits.data_ptr() % 16) // logits.element_size()
        if off == 0:
            return torch.empty_like(logits)
        buf = torch.empty(logits.numel() + off, dtype=logits.dtype, device=logits.device)
        return buf[off:].view(logits.shape)
    if out.shape != logits.shape or out.dtype != logits.dtype or not out.is_contiguous():
        raise ValueError("dlogits must be a contiguous tensor like logits")
    return out


def xent_bwd(logits, target, grad, reduction: str = "mean", out=None):
    """Gradient of :func:`xent` with respect to ``logits``: softmax minus the one-hot
    target, scaled by ``grad`` (the gradient of the forward's output: a 1-element
    tensor for ``"mean"``, the target's shape for ``"none"``).  Returns a tensor like
    ``logits``; ``out`` may be ``logits`` itself (in place)."""
    dt = _xent_bwd_args(logits, target, grad, reduction)
    out = _grad_out(logits, out)
    st = lce_xent_bwd(logits.data_ptr(), dt, target.numel(), logits.shape[-1], target.data_ptr(),
                      _REDUCTIONS[reduction], grad.data_ptr(), out.data_ptr(), _stream_of(logits))
    if st != LCE_OK:
        raise LceError(st, "lce_xent_bwd")
    return out


def xent_fwd_bwd(logits, target, grad, reduction: str = "mean", out=None, dlogits=None):
    """:func:`xent` and :func:`xent_bwd` in one call (``grad`` known before the loss).
    Returns ``(loss, dlogits)``; ``dlogits`` may be ``logits`` itself (in place)."""
    import torch
    dt = _xent_bwd_args(logits, target, grad, reduction)
    dlogits = _grad_out(logits, dlogits)
    shape = (1,) if reduction == "mean" else tuple(target.shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=logits.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 tensor of shape {shape}")
    st = lce_xent_fwd_bwd(logits.data_ptr(), dt, target.numel(), logits.shape[-1],
                          target.data_ptr(), _REDUCTIONS[reduction], grad.data_ptr(),
                          out.data_ptr(), dlogits.data_ptr(), _stream_of(logits))
    if st != LCE_OK:
        raise LceError(st, "lce_xent_fwd_bwd")
    return out, dlogits


def fused_linear_logprob_sums(x, weight, target, out=None):
    """Per-sequence sums of target log-probabilities of ``x @ weight.T``: ``x`` bf16
    ``[batch, seq, hidden]``, ``weight`` bf16 ``[vocab, hidden]``, ``target`` int64
    ``[batch, seq]``; returns fp32 ``[batch]``."""
    import torch
    for name, t in (("x", x), ("weight", weight), ("target", target)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16 or target.dtype != torch.int64:
        raise TypeError("x and weight must be bfloat16, target int64")
    if x.dim() != 3 or weight.dim() != 2 or x.shape[-1] != weight.shape[1]:
        raise ValueError("x must be [batch, seq, hidden] and weight [vocab, hidden]")
    if tuple(target.shape) != tuple(x.shape[:2]):
        raise ValueError("target must be [batch, seq]")
    batch, seq, hidden = x.shape
    if out is None:
        out = torch.empty(batch, dtype=torch.float32, device=x.device)
    st = lce_fused_linear_logprob_sums(x.data_ptr(), weight.data_ptr(), batch, seq, hidden,
                                       weight.shape[0], target.data_ptr(), out.data_ptr(),
                                       _stream_of(x))
    if st != LCE_OK:
        raise LceError(st, "lce_fused_linear_logprob_sums")
    return out


def fused_linear_jsd(student_x, student_weight, teacher_x, teacher_weight, beta: float = 0.5,
                     reduction: str = "mean", out=None):
    """Generalized JSD between softmax(student_x @ student_weight.T) and
    softmax(teacher_x @ teacher_weight.T) without storing either head's logits.

    Activations bf16 [..., hidden] (same shape for both), heads bf16 [vocab, hidden].
    ``reduction="mean"`` is the batch mean (one fp32 element), ``"none"`` the
    per-token divergence with the leading shape of the activations."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    named = (("student_x", student_x), ("student_weight", student_weight),
             ("teacher_x", teacher_x), ("teacher_weight", teacher_weight))
    for name, t in named:
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16")
    if student_weight.dim() != 2 or tuple(teacher_weight.shape) != tuple(student_weight.shape):
        raise ValueError("student_weight and teacher_weight must both be [vocab, hidden]")
    if tuple(student_x.shape) != tuple(teacher_x.shape) or student_x.dim() < 1:
        raise ValueError("student_x and teacher_x must have the same shape [..., hidden]")
    vocab, hidden = student_weight.shape
    if student_x.shape[-1] != hidden:
        raise ValueError("activations' last axis must be the heads' hidden size")
    lead = tuple(student_x.shape[:-1])
    tokens = 1
    for d in lead:
        tokens *= d
    if out is None:
        shape = (1,) if reduction == "mean" else lead
        out = torch.empty(shape, dtype=torch.float32, device=student_x.device)
    st = lce_fused_linear_jsd_fwd(student_x.data_ptr(), student_weight.data_ptr(),
                                  teacher_x.data_ptr(), teacher_weight.data_ptr(), tokens, hidden,
                                  vocab, float(beta), _REDUCTIONS[reduction], out.data_ptr(),
                                  _stream_of(student_x))
    if st != LCE_OK:
        raise LceError(st, "lce_fused_linear_jsd_fwd")
    return out


def _fused_bwd_args(x, weight, target, grad, reduction: str, want_dx: bool, want_dweight: bool):
    """Checks shared by the fused gradient calls; returns (tokens, hidden, vocab)."""
    import torch
    if reduction not in _REDUCTIONS:
        raise ValueError(f"reduction must be 'mean' or 'none', got {reduction!r}")
    for name, t in (("x", x), ("weight", weight), ("target", target), ("grad", grad)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if x.dtype != torch.bfloat16 or weight.dtype != torch.bfloat16:
        raise TypeError("x and weight must be bfloat16")
    if target.dtype != torch.int64 or grad.dtype != torch.float32:
        raise TypeError("target must be int64 and grad float32")
    if weight.dim() != 2 or x.shape[-1] != weight.shape[1]:
        raise ValueError("weight must be [vocab, hidden] with hidden = x.shape[-1]")
    if tuple(target.shape) != tuple(x.shape[:-1]):
        raise ValueError("target shape must be x shape without the hidden axis")
    tokens = target.numel()
    if grad.numel() != (1 if reduction == "mean" else tokens):
        raise ValueError("grad must have 1 element (mean) or one per token (none)")
    if not (want_dx or want_dweight):
        raise ValueError("nothing to compute")
    vocab, hidden = weight.shape
    return tokens, hidden, vocab


def fused_linear_xent_bwd(x, weight, target, grad, reduction: str = "mean", want_dx: bool = True,
                          want_dweight: bool = True, dx=None, dweight=None):
    """Gradients of :func:`fused_linear_xent` with respect to ``x`` and ``weight`` for the
    loss-output gradient ``grad`` (one element for "mean", the target's shape for "none").
    Returns ``(dx, dweight)`` as fp32 tensors (``None`` for one not wanted)."""
    import torch
    tokens, hidden, vocab = _fused_bwd_args(x, weight, target, grad, reduction, want_dx, want_dweight)
    if want_dx and dx is None:
        dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    if want_dweight and dweight is None:
        dweight = torch.empty((vocab, hidden), dtype=torch.float32, device=x.device)
    st = lce_fused_linear_xent_bwd(x.data_ptr(), weight.data_ptr(), tokens, hidden, vocab,
                                   target.data_ptr(), _REDUCTIONS[reduction], grad.data_ptr(),
                                   dx.data_ptr() if want_dx else 0,
                                   dweight.data_ptr() if want_dweight else 0, _stream_of(x))
    if st != LCE_OK:
        raise LceError(st, "lce_fused_linear_xent_bwd")
    return (dx if want_dx else None), (dweight if want_dweight else None)


def fused_linear_xent_fwd_bwd(x, weight, target, grad, reduction: str = "mean",
                              want_dx: bool = True, want_dweight: bool = True, out=None, dx=None,
                              dweight=None):
    """:func:`fused_linear_xent` and :func:`fused_linear_xent_bwd` in one call (``grad``
    known before the loss).  Returns ``(loss, dx, dweight)`` (``None`` for a gradient not
    wanted)."""
    import torch
    tokens, hidden, vocab = _fused_bwd_args(x, weight, target, grad, reduction, want_dx, want_dweight)
    shape = (1,) if reduction == "mean" else tuple(target.shape)
    if out is None:
        out = torch.empty(shape, dtype=torch.float32, device=x.device)
    elif tuple(out.shape) != shape or out.dtype != torch.float32 or not out.is_contiguous():
        raise ValueError(f"out must be a contiguous float32 tensor of shape {shape}")
    if want_dx and dx is None:
        dx = torch.empty(x.shape, dtype=torch.float32, device=x.device)
    if want_dweight and dweight is None:
        dweight = torch.empty((vocab, hidden), dtype=torch.float32, device=x.device)
    st = lce_fused_linear_xent_fwd_bwd(x.data_ptr(), weight.data_ptr(), tokens, hidden, vocab,
                                       target.data_ptr(), _REDUCTIONS[reduction], grad.data_ptr(),
                                       out.data_ptr(), dx.data_ptr() if want_dx else 0,
                                       dweight.data_ptr() if want_dweight else 0, _stream_of(x))
    if st != LCE_OK:
        raise LceError(st, "lce_fused_linear_xent_fwd_bwd")
    return out, (dx if want_dx else None), (dweight if want_dweight else None)
