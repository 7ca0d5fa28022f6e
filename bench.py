"""liblce benchmark: µs per forward cross-entropy on one MI355X, with roofline and CPU oracle.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workloads all|headline|NAME,...]

A step is one forward call of the hot path on one batch of synthetic input already
resident in HBM.  The headline workload is the largest configuration that fits one GPU:
fp32 logits [16384, 131072] (8.6 GB) with the mean loss.  Inputs are replicated so that
the replicas together exceed the 256 MB Infinity Cache, and step i reads replica i mod R:
every step streams its logits from HBM.

Timing (graph_replays): W eager warmup steps, then the K timed steps are captured into
one HIP graph (liblce launches on torch's current stream; nothing in the call allocates
or memsets once warm), replayed once untimed (its outputs are checked against the eager
ones), then replayed SPREAD_REPLAYS times, each replay timed between two events recorded
on the capture stream, bracketed by torch.cuda.synchronize().  `value` is the median µs
per step over those replays, with p10 and p90 beside it.  The graph removes host launch
overhead, which is longer than the shortest kernels; the eager per-call time is reported
next to it.

Prints ONE JSON line (rank 0, N = 1).  Other workloads are measured the same way and
reported under "workloads".  The roofline is for the dominant kernel, named from what the
library reports it launched (lce_last_launch): algorithmic bytes (each input and output
tensor read or written once) or flops per step over the median step time.  Every
headline step is one launch of that kernel, so the step time is its average launch
duration.
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs per forward CE (and achieved HBM GB/s / % roofline) at tokens×vocab"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, datasheet
BF16_DENSE_TFLOPS = 2500.0     # MI355X dense bf16 MFMA, datasheet
INFINITY_CACHE_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


# ------------------------------------------------------------------ work model

def tensor_bytes(tensors) -> int:
    """Bytes of a list of (numel, itemsize) tensors, each read or written once."""
    return int(sum(int(n) * int(s) for n, s in tensors))


def xent_bytes(tokens: int, vocab: int, esize: int, reduction: str) -> int:
    """Algorithmic bytes of one row cross-entropy: logits + int64 targets + fp32 output."""
    out = 1 if reduction == "mean" else tokens
    return tensor_bytes([(tokens * vocab, esize), (tokens, 8), (out, 4)])


def fused_bytes(tokens: int, hidden: int, vocab: int, reduction: str) -> int:
    """Algorithmic bytes of one fused projection + cross-entropy: x + W + targets + output."""
    out = 1 if reduction == "mean" else tokens
    return tensor_bytes([(tokens * hidden, 2), (vocab * hidden, 2), (tokens, 8), (out, 4)])


def fused_flops(tokens: int, hidden: int, vocab: int) -> int:
    """Multiply-adds of z = x W^T, counted as 2 flops each."""
    return 2 * int(tokens) * int(hidden) * int(vocab)


CSRC = os.path.join(ROOT, "vocab_cross_entropy_row_amd", "csrc")
# Sources that define each workload's dominant kernel (plus the build flags).
SPREAD_REPLAYS = 10  # graph replays timed for the median / p10 / p90 per step

KERNEL_SOURCES = {  # kernel sources, and lce_api.cpp, which picks the instantiation and launch shape
    "xent": ["xent_kernels.hip", "row_stream.h", "lce_device.h", "lce_internal.h", "lce_api.cpp"],
    "fused": ["fused_kernel.hip", "mfma_common.h", "lce_device.h", "lce_internal.h", "lce_api.cpp"],
}


def source_digest(kind: str) -> str:
    """sha256 over the sources of a workload kind's kernels and the device compiler flags:
    ties counter data to the kernel build it was taken on."""
    from vocab_cross_entropy_row_amd import build as lce_build
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kind]:
        h.update(f.encode())
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    # the flags name the repository's include directory: hash it relative to the root
    h.update(" ".join(lce_build.common_flags()).replace(lce_build.ROOT, "<root>").encode())
    return h.hexdigest()


def traffic_for(workload: str, kind: str):
    """HBM traffic per launch from the committed counter summary, or None if absent or
    if the kernel's sources changed since the counters were taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != source_digest(kind):
        return None
    return d.get("traffic_bytes_per_launch")


# ------------------------------------------------------------------ device inputs

def _to_dev(arr, torch):
    import numpy as np
    if arr.dtype == np.uint16:
        return torch.from_numpy(arr.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(arr).cuda()


# Device inputs of the workloads named in KEEP are kept here after their own timing,
# for the measurements that reuse them (split path, sweeps).
KEEP = set()
_KEPT = {}


def make_inputs(w, torch, replicas: int):
    """Device replicas of a workload's inputs (generated once on the host, in row blocks)."""
    if w.name in _KEPT:
        base = _KEPT[w.name]
        return [base] + [tuple(a.clone() for a in base) for _ in range(replicas - 1)]
    reps = _make_inputs(w, torch, replicas)
    if w.name in KEEP:
        _KEPT[w.name] = reps[0]
    return reps


def _make_inputs(w, torch, replicas: int):
    if w.kind == "xent":
        tdt = torch.float32 if w.dtype == "f32" else torch.bfloat16
        z = torch.empty(w.shape, dtype=tdt, device="cuda")
        flat = z.view(w.tokens, w.vocab)
        blk = max(1, (512 << 20) // (w.vocab * (4 if w.dtype == "f32" else 2)))
        for r0 in range(0, w.tokens, blk):
            r1 = min(w.tokens, r0 + blk)
            flat[r0:r1].copy_(_to_dev(w.logits(r0, r1), torch))
        t = torch.from_numpy(w.target()).cuda().view(w.target_shape)
        reps = [(z, t)] + [(z.clone(), t.clone()) for _ in range(replicas - 1)]
        return reps
    x = _to_dev(w.x(), torch)
    W = torch.empty((w.vocab, w.hidden), dtype=torch.bfloat16, device="cuda")
    blk = 16384
    for r0 in range(0, w.vocab, blk):
        r1 = min(w.vocab, r0 + blk)
        W[r0:r1].copy_(_to_dev(w.weight(r0, r1), torch))
    t = torch.from_numpy(w.target()).cuda()
    return [(x, W, t)] + [(x.clone(), W.clone(), t.clone()) for _ in range(replicas - 1)]


def replicas_for(w) -> int:
    """Enough replicas that their logits/weights exceed 4x the Infinity Cache (<= 16)."""
    per = (w.tokens * w.vocab * (4 if w.dtype == "f32" else 2)) if w.kind == "xent" \
        else (w.vocab * w.hidden * 2)
    r = 1
    while r < 16 and r * per < 4 * INFINITY_CACHE_BYTES:
        r += 1
    return r


# ------------------------------------------------------------------ timing

def spread_of(per) -> dict:
    """Median, p10, p90, min, max and last of per-replay µs per step."""
    s = sorted(per)
    q = lambda f: s[min(len(s) - 1, int(round(f * (len(s) - 1))))]
    return {"replays": len(per), "median_us": round(statistics.median(s), 3),
            "p10_us": round(q(0.1), 3), "p90_us": round(q(0.9), 3), "min_us": round(s[0], 3),
            "max_us": round(s[-1], 3), "last_us": round(per[-1], 3)}


def graph_replays(step, steps: int, warmup: int, replays: int = None):
    """The timing protocol of every measurement here: `warmup` eager calls step(i), then
    `steps` calls captured into one HIP graph on a side stream (after one eager call on
    that stream, so liblce's per-stream scratch exists before capture), one untimed
    replay, then `replays` replays each timed between two events recorded on the capture
    stream.  Returns the µs per step of each timed replay, in order."""
    import torch
    replays = SPREAD_REPLAYS if replays is None else replays
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(replays):
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            t0.record(s)
            g.replay()
            t1.record(s)
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) * 1000.0 / steps)
    del g
    return per


def time_workload(w, steps: int, warmup: int, torch, lce, eager_only: bool = False):
    reps = make_inputs(w, torch, replicas_for(w))
    R = len(reps)
    outs = [torch.empty((1,) if w.reduction == "mean" else w.target_shape, dtype=torch.float32,
                        device="cuda") for _ in range(R)]

    def step(i):
        r = i % R
        if w.kind == "xent":
            z, t = reps[r]
            lce.xent(z, t, w.reduction, out=outs[r])
        else:
            x, W, t = reps[r]
            lce.fused_linear_xent(x, W, t, w.reduction, out=outs[r])

    for i in range(max(warmup, R)):  # every replica's output is written at least once
        step(i)
    torch.cuda.synchronize()
    eager_ref = [o.clone() for o in outs]
    step(0)
    launch = lce.lce_last_launch()  # what the library enqueued for one step

    # eager per-call time (host launch overhead included)
    n_eager = min(steps, 50)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n_eager):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    eager_us = e0.elapsed_time(e1) * 1000.0 / n_eager
    if eager_only:
        torch.cuda.synchronize()
        e0.record()
        for i in range(steps):
            step(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / steps
        del reps, outs
        torch.cuda.empty_cache()
        return {"us_per_step": us, "eager_us_per_call": eager_us, "replicas": R,
                "graph_matches_eager": None, "spread": None, "launch": launch}

    # exactly `steps` steps in one graph; after the replays, every output must equal the
    # eager one bitwise
    per = graph_replays(step, steps, 0)
    ok = all(torch.equal(a, b) for a, b in zip(outs, eager_ref))
    spread = spread_of(per)
    del reps, outs
    torch.cuda.empty_cache()
    return {"us_per_step": spread["median_us"], "eager_us_per_call": eager_us, "replicas": R,
            "graph_matches_eager": bool(ok), "spread": spread, "launch": launch}


def roofline_entry(w, us: float) -> dict:
    if w.kind == "xent":
        esize = 4 if w.dtype == "f32" else 2
        b = xent_bytes(w.tokens, w.vocab, esize, w.reduction)
        gbs = b / (us * 1e-6) / 1e9
        return {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic_for(w.name, w.kind),
                "algorithmic_bytes": b}
    fl = fused_flops(w.tokens, w.hidden, w.vocab)
    tf = fl / (us * 1e-6) / 1e12
    return {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_DENSE_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_DENSE_TFLOPS, 4),
            "traffic": traffic_for(w.name, w.kind), "algorithmic_flops": fl,
            "algorithmic_bytes": fused_bytes(w.tokens, w.hidden, w.vocab, w.reduction)}


def time_backward(w, torch, lce, steps: int, warmup: int) -> dict:
    """Gradient of a row workload's loss with respect to its logits (lce_xent_bwd), timed
    as a HIP graph of `steps` calls over rotating replicas (logits and gradient buffers)
    that exceed the Infinity Cache.  Algorithmic bytes: the logits read once, the gradient
    written once, targets and the output gradient."""
    reps = make_inputs(w, torch, replicas_for(w))
    R = len(reps)
    outs = [torch.empty_like(z) for z, _ in reps]
    grad = torch.ones((1,) if w.reduction == "mean" else w.target_shape, dtype=torch.float32,
                      device="cuda")

    def step(i):
        z, t = reps[i % R]
        lce.xent_bwd(z, t, grad, w.reduction, out=outs[i % R])

    step(0)
    launch = lce.lce_last_launch()
    sp = spread_of(graph_replays(step, steps, max(warmup, R)))
    us = sp["median_us"]
    esize = 4 if w.dtype == "f32" else 2
    b = tensor_bytes([(w.tokens * w.vocab, esize), (w.tokens * w.vocab, esize), (w.tokens, 8),
                      (1 if w.reduction == "mean" else w.tokens, 4)])
    # A training step's two halves: the forward then the backward (two calls), against
    # both in one call (lce_xent_fwd_bwd), on the same replicas.
    losses = [torch.empty((1,) if w.reduction == "mean" else w.target_shape, dtype=torch.float32,
                          device="cuda") for _ in range(R)]

    def fwd(i):
        z, t = reps[i % R]
        lce.xent(z, t, w.reduction, out=losses[i % R])

    def fwd_bwd(i):
        z, t = reps[i % R]
        lce.xent_fwd_bwd(z, t, grad, w.reduction, out=losses[i % R], dlogits=outs[i % R])
    fwd_bwd(0)
    fb_launch = lce.lce_last_launch()
    fwd_us = spread_of(graph_replays(fwd, steps, max(warmup, R)))["median_us"]
    fb = spread_of(graph_replays(fwd_bwd, steps, max(warmup, R)))
    del reps, outs, losses
    torch.cuda.empty_cache()
    gbs = b / (us * 1e-6) / 1e9
    fb_gbs = b / (fb["median_us"] * 1e-6) / 1e9
    return {"us_per_step": round(us, 3), "replicas": R, "spread": sp, "launch": launch,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": b},
            "training_step": {"forward_us": round(fwd_us, 3),
                              "forward_then_backward_us": round(fwd_us + us, 3),
                              "fwd_bwd_us": round(fb["median_us"], 3), "fwd_bwd_spread": fb,
                              "fwd_bwd_launch": fb_launch,
                              "fwd_bwd_roofline": {"bound": "hbm", "achieved": round(fb_gbs, 1),
                                                   "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                   "frac": round(fb_gbs / HBM_PEAK_GBS, 4)}}}


def time_logprob_sums(torch, lce, lce_synth, steps: int, warmup: int) -> dict:
    """Per-sequence target log-probability sums at the fused workload's shape read as the
    CPO page's [batch 2, seq 1024] (lce_fused_linear_logprob_sums), timed as a HIP graph."""
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    batch, seq = 2, w.tokens // 2
    (x, W, t), = make_inputs(w, torch, 1)
    x3, t2 = x.view(batch, seq, w.hidden), t.view(batch, seq)
    out = torch.empty(batch, dtype=torch.float32, device="cuda")
    sp = spread_of(graph_replays(lambda i: lce.fused_linear_logprob_sums(x3, W, t2, out=out), steps,
                                 max(1, warmup), replays=5))
    us = sp["median_us"]
    tf = fused_flops(w.tokens, w.hidden, w.vocab) / (us * 1e-6) / 1e12
    del x, W, t
    torch.cuda.empty_cache()
    return {"shape": f"batch {batch} x seq {seq}, hidden {w.hidden}, vocab {w.vocab}",
            "us_per_step": round(us, 1), "spread": sp,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_DENSE_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_DENSE_TFLOPS, 4)}}


def time_fused_bwd(torch, lce, lce_synth, steps: int, warmup: int) -> dict:
    """Gradients of the fused projection + cross-entropy at the fused workload's shape
    (lce_fused_linear_xent_bwd, mean reduction, dx and dW in fp32), timed as a HIP graph of
    `steps` calls.  Algorithmic flops: the logits once plus the two products, 3 * 2*T*H*V
    (the call executes 4 * 2*T*H*V: a log-sum-exp pass, the logit-gradient pass and the
    two GEMMs)."""
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    (x, W, t), = make_inputs(w, torch, 1)
    g = torch.ones(1, dtype=torch.float32, device="cuda")
    dx = torch.empty(x.shape, dtype=torch.float32, device="cuda")
    dw = torch.empty(W.shape, dtype=torch.float32, device="cuda")

    def call(i=0):
        lce.fused_linear_xent_bwd(x, W, t, g, "mean", dx=dx, dweight=dw)
    call()
    launch = lce.lce_last_launch()
    torch.cuda.synchronize()
    ref = (dx.clone(), dw.clone())
    sp = spread_of(graph_replays(call, steps, max(1, warmup), replays=5))
    us = sp["median_us"]
    same = bool(torch.equal(dx, ref[0]) and torch.equal(dw, ref[1]))
    flops = 3 * fused_flops(w.tokens, w.hidden, w.vocab)
    tf = flops / (us * 1e-6) / 1e12
    # A training step: the forward call then this one, against the loss and both
    # gradients from one call (lce_fused_linear_xent_fwd_bwd).
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    fwd_us = spread_of(graph_replays(lambda i: lce.fused_linear_xent(x, W, t, "mean", out=loss),
                                     steps, max(1, warmup), replays=5))["median_us"]

    def fwd_bwd(i=0):
        lce.fused_linear_xent_fwd_bwd(x, W, t, g, "mean", out=loss, dx=dx, dweight=dw)
    fwd_bwd()
    fb_launch = lce.lce_last_launch()
    fb = spread_of(graph_replays(fwd_bwd, steps, max(1, warmup), replays=5))
    fb_same = bool(torch.equal(dx, ref[0]) and torch.equal(dw, ref[1]))
    fb_tf = flops / (fb["median_us"] * 1e-6) / 1e12
    del x, W, t, dx, dw, ref
    torch.cuda.empty_cache()
    return {"shape": f"tokens {w.tokens}, hidden {w.hidden}, vocab {w.vocab}, mean; dx and dW fp32",
            "us_per_step": round(us, 1), "spread": sp, "launch": launch,
            "graph_matches_eager": same, "algorithmic_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_DENSE_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_DENSE_TFLOPS, 4)},
            "training_step": {"forward_us": round(fwd_us, 1),
                              "forward_then_backward_us": round(fwd_us + us, 1),
                              "fwd_bwd_us": round(fb["median_us"], 1), "fwd_bwd_spread": fb,
                              "fwd_bwd_launch": fb_launch, "fwd_bwd_gradients_match": fb_same,
                              "fwd_bwd_roofline": {"bound": "mfma", "achieved": round(fb_tf, 1),
                                                   "peak": BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                                                   "frac": round(fb_tf / BF16_DENSE_TFLOPS, 4)}}}


def time_jsd(torch, lce, lce_synth, steps: int, warmup: int) -> dict:
    """Fused linear + JSD at the JSD page's shape (tokens 1024, hidden 4096, vocab 128256,
    beta 0.5, batchmean), timed as a HIP graph of `steps` calls, on the default path
    (logits stored in scratch) and on the recompute path (LCE_JSD_STORE_BYTES=0).
    Algorithmic flops: both heads' logits once, 2 * 2*T*H*V."""
    w = lce_synth.JSD
    xs, ws, xt, wt = (_to_dev(b, torch) for b in (w.student_x(), w.student_weight(),
                                                   w.teacher_x(), w.teacher_weight()))
    out = torch.empty(1, dtype=torch.float32, device="cuda")
    flops = 2 * fused_flops(w.tokens, w.hidden, w.vocab)
    res = {"shape": f"tokens {w.tokens}, hidden {w.hidden}, vocab {w.vocab}, beta 0.5, batchmean",
           "algorithmic_flops": flops}
    for label, env in (("stored", None), ("recompute", "0")):
        old = os.environ.get("LCE_JSD_STORE_BYTES")
        if env is not None:
            os.environ["LCE_JSD_STORE_BYTES"] = env
        try:
            lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "mean", out=out)
            launch = lce.lce_last_launch()
            torch.cuda.synchronize()
            val = out.item()
            sp = spread_of(graph_replays(
                lambda i: lce.fused_linear_jsd(xs, ws, xt, wt, 0.5, "mean", out=out), steps,
                max(1, warmup), replays=5))
            us = sp["median_us"]
        finally:
            if env is not None:
                if old is None:
                    os.environ.pop("LCE_JSD_STORE_BYTES", None)
                else:
                    os.environ["LCE_JSD_STORE_BYTES"] = old
        tf = flops / (us * 1e-6) / 1e12
        res[label] = {"us_per_step": round(us, 1), "batchmean": val, "spread": sp,
                      "launch": launch,
                      "roofline": {"bound": "mfma", "achieved": round(tf, 1),
                                   "peak": BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                                   "frac": round(tf / BF16_DENSE_TFLOPS, 4)}}
    # The page's token sweep (stored path, eager calls between events): the same heads,
    # activations drawn N(0, 1) on the device (torch generator seeded by the token
    # count) and rounded to bf16.
    scaling = {}
    for tokens in (2048, 4096, 8192):
        xs2 = torch.randn(tokens, w.hidden, device="cuda", generator=torch.Generator(
            device="cuda").manual_seed(tokens)).to(torch.bfloat16)
        xt2 = torch.randn(tokens, w.hidden, device="cuda", generator=torch.Generator(
            device="cuda").manual_seed(tokens + 1)).to(torch.bfloat16)
        for _ in range(2):
            lce.fused_linear_jsd(xs2, ws, xt2, wt, 0.5, "mean", out=out)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            lce.fused_linear_jsd(xs2, ws, xt2, wt, 0.5, "mean", out=out)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / 3
        tf = 2 * fused_flops(tokens, w.hidden, w.vocab) / (us * 1e-6) / 1e12
        scaling[str(tokens)] = {"us_per_call": round(us, 1), "tflops": round(tf, 1)}
        del xs2, xt2
    res["stored_by_tokens"] = scaling
    del xs, ws, xt, wt
    torch.cuda.empty_cache()
    return res


def time_vocab_shard(torch, lce, lce_synth, tp: int, steps: int, warmup: int) -> dict:
    """The headline workload with its vocab split over `tp` devices, as one device sees it:
    statistics of its [tokens, vocab/tp] shard (lce_xent_partial_fwd, timed over rotating
    replicas that exceed the Infinity Cache), and the merge of all `tp` shards' statistics
    (lce_xent_merge, after the all-gather that one GPU cannot show).  Both are timed as HIP
    graphs of `steps` calls; the merged losses are checked against the unsplit call."""
    w = lce_synth.WORKLOADS["megatron_bf16_2048x4x4096_none"]
    T, V = w.tokens, w.vocab
    sv = V // tp
    z = torch.empty((T, V), dtype=torch.bfloat16, device="cuda")
    blk = 2048
    for r0 in range(0, T, blk):
        z[r0:r0 + blk].copy_(_to_dev(w.logits(r0, min(T, r0 + blk)), torch))
    t = torch.from_numpy(w.target()).cuda()
    shards = [z[:, p * sv:(p + 1) * sv].contiguous() for p in range(tp)]
    shard_bytes = T * sv * 2
    R = max(1, min(128, -(-4 * INFINITY_CACHE_BYTES // shard_bytes)))
    reps = [shards[0]] + [shards[0].clone() for _ in range(R - 1)]
    part = torch.empty((T, 3), dtype=torch.float32, device="cuda")
    stats = torch.stack([lce.xent_partial(sh, t, p * sv) for p, sh in enumerate(shards)])
    out = torch.empty(T, dtype=torch.float32, device="cuda")

    def graph_us(fn, k):
        return spread_of(graph_replays(fn, k, max(warmup, R)))["median_us"]

    p_us = graph_us(lambda i: lce.xent_partial(reps[i % R], t, 0, out=part), steps)
    m_us = graph_us(lambda i: lce.xent_merge(stats, t, V, "none", out=out), steps)
    # The same shard bytes read by bench_probe's plain read (nothing else): the floor a
    # read of this size has on this part (launch and memory latency included).
    read_us = probe_read_us(torch, reps, steps) if os.path.exists(PROBE_LIB) else None
    lce.xent_merge(stats, t, V, "none", out=out)
    whole = lce.xent(z, t.view(-1), "none")
    torch.cuda.synchronize()
    diff = float(torch.max(torch.abs(out - whole)).item())
    p_bytes = shard_bytes + T * 8 + T * 12
    m_bytes = tp * T * 12 + T * 8 + T * 4
    del reps, shards, z
    torch.cuda.empty_cache()
    return {"shard": f"bf16 [{T}, {sv}] = vocab columns [0, {sv}) of {w.name}, tp={tp}",
            "partial_us": round(p_us, 3), "merge_us": round(m_us, 3),
            "partial_roofline": {"bound": "hbm", "achieved": round(p_bytes / (p_us * 1e3), 1),
                                 "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                 "frac": round(p_bytes / (p_us * 1e3) / HBM_PEAK_GBS, 4),
                                 "algorithmic_bytes": p_bytes, "replicas": R},
            "shard_read_only_us": round(read_us, 3) if read_us else None,
            "partial_us_over_read_only_us": round(p_us / read_us, 4) if read_us else None,
            "merge_algorithmic_bytes": m_bytes,
            "max_abs_diff_vs_unsplit": diff}


# ------------------------------------------------------------------ split path and sweeps

def _xent_point(torch, lce, z_all, t_all, rows: int, vocab: int, reduction: str, steps: int,
                warmup: int, target_seed: int, lce_synth) -> dict:
    """One row cross-entropy measurement on [rows, vocab] views cut from a kept workload's
    logit buffer (seeded synthetic values; disjoint slices serve as the rotating replicas,
    as many as fit, up to enough to exceed 4x the Infinity Cache) with targets drawn
    uniform on [0, vocab) from their own seed."""
    flat = z_all.reshape(-1)
    esize = flat.element_size()
    per = rows * vocab
    R = 1
    while R < 16 and R * per * esize < 4 * INFINITY_CACHE_BYTES and (R + 1) * per <= flat.numel():
        R += 1
    views = [flat[r * per:(r + 1) * per].view(rows, vocab) for r in range(R)]
    t = torch.from_numpy(lce_synth.targets(target_seed, rows, vocab)).cuda()
    outs = [torch.empty((1,) if reduction == "mean" else (rows,), dtype=torch.float32,
                        device="cuda") for _ in range(R)]

    def step(i):
        lce.xent(views[i % R], t, reduction, out=outs[i % R])

    step(0)
    launch = lce.lce_last_launch()
    sp = spread_of(graph_replays(step, steps, max(warmup, R)))
    b = xent_bytes(rows, vocab, esize, reduction)
    gbs = b / (sp["median_us"] * 1e-6) / 1e9
    return {"tokens": rows, "vocab": vocab, "reduction": reduction, "replicas": R,
            "us_per_step": sp["median_us"], "spread": sp, "launch": launch,
            "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                         "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                         "algorithmic_bytes": b}}


def time_split(torch, lce, lce_synth, steps: int, warmup: int) -> dict:
    """Few rows of 131072 logits, where the split-vocab path is the default (fewer rows
    than twice the CU count): 256 rows of the fp32 [16384, 131072] workload's logits with
    the mean, and 256 rows of the bf16 [2048, 4, 131072] workload's logits per token."""
    res = {}
    for name, red, tseed in (("ce_f32_16384x131072_mean", "mean", 2101),
                             ("megatron_bf16_2048x4x131072_none", "none", 2102)):
        z, _t = _KEPT[name]
        w = lce_synth.WORKLOADS[name]
        key = f"split_{w.dtype}_256x{w.vocab}_{red}"
        res[key] = _xent_point(torch, lce, z, None, 256, w.vocab, red, steps, warmup, tseed,
                               lce_synth)
        print(f"[bench] {key}: {res[key]['us_per_step']:.2f} µs/step "
              f"({res[key]['roofline']['achieved']} GB/s) via {res[key]['launch']}",
              file=sys.stderr, flush=True)
    return res


SWEEP_VOCABS = (4096, 8192, 16384, 32768, 65536, 131072)
FUSED_SWEEP_BATCHES = (2, 4, 8, 16)


def time_sweeps(torch, lce, lce_synth, steps: int, warmup: int) -> dict:
    """The pages' own workload axes: vocab 4096..131072 at tokens 16384 fp32 with the mean
    ("Cross-entropy loss", Current records) and at seq 2048 x batch 4 bf16 per token
    ("Vocab-parallel cross-entropy, Megatron layout", Current records), each cut from the
    kept 131072-wide workload's logit buffer; and the fused projection at batch 2/4/8/16 x
    seq 1024 ("Fused linear + CPO loss", Scaling by batch) with the fused workload's head
    and activations drawn by its recipe (seed 1005) for the larger token counts."""
    res = {"ce_f32_tokens16384_mean": {}, "megatron_bf16_2048x4_none": {}, "fused_by_batch": {}}
    zf, _ = _KEPT["ce_f32_16384x131072_mean"]
    zb, _ = _KEPT["megatron_bf16_2048x4x131072_none"]
    for v in SWEEP_VOCABS:
        k = min(steps, 30) if v >= 65536 else steps
        res["ce_f32_tokens16384_mean"][str(v)] = _xent_point(
            torch, lce, zf, None, 16384, v, "mean", k, warmup, 2200 + v % 997, lce_synth)
        res["megatron_bf16_2048x4_none"][str(v)] = _xent_point(
            torch, lce, zb, None, 8192, v, "none", k, warmup, 2300 + v % 991, lce_synth)
        print(f"[bench] sweep vocab {v}: fp32 mean "
              f"{res['ce_f32_tokens16384_mean'][str(v)]['us_per_step']:.2f} µs, bf16 none "
              f"{res['megatron_bf16_2048x4_none'][str(v)]['us_per_step']:.2f} µs",
              file=sys.stderr, flush=True)
    w = lce_synth.WORKLOADS["fused_bf16_t2048_h4096_v128256_mean"]
    x0, W, _t = _KEPT[w.name]
    for b in FUSED_SWEEP_BATCHES:
        T = b * 1024
        x = x0 if T == w.tokens else _to_dev(lce_synth.normal_bf16_bits(
            w.seed, lce_synth.STREAM_LOGITS, T, w.hidden, w.std), torch)
        t = torch.from_numpy(lce_synth.targets(w.target_seed, T, w.vocab)).cuda()
        out = torch.empty(1, dtype=torch.float32, device="cuda")
        sp = spread_of(graph_replays(lambda i: lce.fused_linear_xent(x, W, t, "mean", out=out),
                                     max(3, min(steps, 30) * 2 // b), 1, replays=5))
        tf = fused_flops(T, w.hidden, w.vocab) / (sp["median_us"] * 1e-6) / 1e12
        res["fused_by_batch"][str(b)] = {
            "tokens": T, "us_per_step": sp["median_us"], "spread": sp,
            "roofline": {"bound": "mfma", "achieved": round(tf, 1), "peak": BF16_DENSE_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tf / BF16_DENSE_TFLOPS, 4)}}
        print(f"[bench] sweep fused batch {b}: {sp['median_us']:.1f} µs ({tf:.1f} TFLOP/s)",
              file=sys.stderr, flush=True)
        del x, t
    torch.cuda.empty_cache()
    return res


# ------------------------------------------------------------------ CPU baseline (oracle)

def cpu_baseline(w, budget_s: float = 10.0) -> dict:
    """Time the fp64 oracle on the host cores over a bounded sample of the workload and
    scale to µs per full forward call."""
    import oracle
    threads = oracle.default_threads()
    if w.kind == "xent":
        rows = w.tokens
        per_row_elems = w.vocab
        # sample: leading rows, at most ~2^28 elements
        sample_rows = min(rows, max(1, (1 << 28) // per_row_elems))
        z = w.logits(0, sample_rows)
        t = w.target(0, sample_rows)
        times = []
        t_end = time.perf_counter() + budget_s
        while len(times) < 5 and (not times or time.perf_counter() < t_end):
            t0 = time.perf_counter()
            oracle.xent_rows(z, t, dtype=w.dtype, nthreads=threads)
            times.append(time.perf_counter() - t0)
        per_call = statistics.median(times) * rows / sample_rows
        sample = (f"rows [0, {sample_rows}) of {rows} ({sample_rows * per_row_elems} logits), "
                  f"median of {len(times)} runs, scaled to all rows")
    else:
        rows = w.tokens
        sample_rows = min(rows, 16)
        xb, wb, tg = w.x(0, sample_rows), w.weight(), w.target(0, sample_rows)
        t0 = time.perf_counter()
        oracle.fused_linear_xent_rows(xb, wb, tg, nthreads=threads)
        per_call = (time.perf_counter() - t0) * rows / sample_rows
        sample = f"{sample_rows} of {rows} token rows (full head), one run, scaled to all rows"
    return {"value": round(per_call * 1e6, 1), "unit": "µs", "cores": threads, "kind": "oracle",
            "sample": sample, "cpu_model": _cpu_model()}


def _cpu_model() -> str:
    """The host CPU's model name from /proc/cpuinfo ("unknown" if not readable)."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# ------------------------------------------------------------------ streaming-read probe

PROBE_SRC = os.path.join(ROOT, "bench_probe.hip")
PROBE_LIB = os.path.join(ROOT, "bench_probe.so")


def build_probe() -> str:
    """Compile bench_probe.so (gfx950) from bench_probe.hip: the plain-read and VALU-rate probes."""
    import subprocess
    from vocab_cross_entropy_row_amd import build as B
    tmp = PROBE_LIB + ".tmp"
    subprocess.run([B.hipcc(), "-x", "hip", "-O3", "-std=c++17", "-fPIC", f"--offload-arch={B.ARCH}",
                    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-shared",
                    PROBE_SRC, "-o", tmp], check=True, capture_output=True)
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


def _probe_lib():
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(PROBE_LIB)
    lib.bench_stream_read.restype = ctypes.c_int
    lib.bench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                      ctypes.c_void_p]
    return lib


def probe_read_us(torch, bufs, k: int) -> float:
    """bench_probe's plain read of each device buffer in `bufs` in turn (rotating), timed as
    a graph of `k` reads on a side stream: median µs per read over the timed replays."""
    lib = _probe_lib()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())

    def call(i):
        b = bufs[i % len(bufs)]
        rc = lib.bench_stream_read(b.data_ptr(), b.numel() * b.element_size(), sink.data_ptr(),
                                   s.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"bench_stream_read failed (hipError {rc})")
    with torch.cuda.stream(s):
        for i in range(len(bufs)):
            call(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(k):
            call(i)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = []
    for _ in range(SPREAD_REPLAYS):
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            t0.record(s)
            g.replay()
            t1.record(s)
        torch.cuda.synchronize()
        per.append(t0.elapsed_time(t1) * 1000.0 / k)
    del g
    return statistics.median(per)


def time_stream_read(torch, head_bytes: int, head_replicas: int, steps: int) -> dict:
    """A plain streaming read for comparison (not a peak: the long row kernels read faster):
    bench_probe's kernel (16-byte nontemporal loads, nothing else) over one 2 GiB buffer,
    and over `head_bytes` (the logit bytes of a short-row workload) with as many rotating
    replicas as that workload's timing uses, each timed as a graph of `steps` reads
    (median of the replays)."""
    big = [torch.ones(1 << 31, dtype=torch.uint8, device="cuda")]
    us_big = probe_read_us(torch, big, max(5, min(steps, 20)))
    del big
    small = [torch.ones(head_bytes, dtype=torch.uint8, device="cuda") for _ in range(head_replicas)]
    us_small = probe_read_us(torch, small, steps)
    del small
    torch.cuda.empty_cache()
    return {"kernel": "bench_probe.hip stream_read_kernel (16-byte nt buffer loads, 8 per lane "
                      "in flight, 32 KiB contiguous per workgroup, 2048 x 256 threads)",
            "bytes_2GiB_us": round(us_big, 2), "gbs_2GiB": round((1 << 31) / (us_big * 1e-6) / 1e9, 1),
            "bytes": head_bytes, "replicas": head_replicas, "read_us": round(us_small, 3),
            "gbs": round(head_bytes / (us_small * 1e-6) / 1e9, 1)}


def time_valu_rate(torch) -> dict:
    """bench_probe's vector-arithmetic rates: 8 independent chains per lane of v_exp_f32,
    of v_fma_f32 and of the bf16 row-fold step (decode, FMA, exponential, add) in 2048
    workgroups of 256 threads (every wave slot of 256 CUs), each timed with events (median of
    three launches after one untimed), as SIMD cycles per wave instruction (per element for
    the fold step) at the 2.4 GHz datasheet clock."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.bench_valu_rate.restype = ctypes.c_int
    lib.bench_valu_rate.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p]
    blocks, iters = 2048, 4096
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    steps_per_simd = blocks * 4 / 1024 * iters * 8  # 4 waves per workgroup, 1024 SIMDs
    res = {}
    for mode, name in ((0, "exp_f32"), (1, "fma_f32"), (2, "bf16_fold_step")):
        s = torch.cuda.current_stream()
        per = []
        for _ in range(4):
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(s)
            rc = lib.bench_valu_rate(mode, out.data_ptr(), blocks, iters, s.cuda_stream)
            t1.record(s)
            if rc != 0:
                raise RuntimeError(f"bench_valu_rate failed (hipError {rc})")
            torch.cuda.synchronize()
            per.append(t0.elapsed_time(t1) * 1e3)
        us = statistics.median(per[1:])
        res[name] = {"us": round(us, 1),
                     "cycles_per_wave_instruction_at_2_4_GHz": round(us * 1e-6 * 2.4e9 / steps_per_simd, 2)}
    return res


def time_fused_skeleton(torch) -> dict:
    """bench_probe's skeleton of the fused kernel's inner loop (mfma_lds_kernel): per wave and
    k-step 8 MFMAs 32x32x16 bf16 on a 128 x 64 tile with its 6 fragment reads from LDS, a
    barrier every 4 k-steps and 8 direct-to-LDS 1 KiB loads per wave every 4 k-steps, in 256
    workgroups of 8 waves (one per CU), the parts added one at a time.  Cycles are s_memtime
    cycles per wave, the per-workgroup maximum, median over workgroups; MFMA busy is 32
    cycles (the datasheet rate of one 32x32x16 bf16 MFMA per SIMD) over the measured cycles
    per MFMA per SIMD (two waves per SIMD).  Beside it, bench_probe's lds_read_kernel: LDS
    read throughput alone (ds_read_b128, nothing else) at 4, 8 and 16 waves per CU."""
    import ctypes
    lib = ctypes.CDLL(PROBE_LIB)
    lib.bench_mfma_lds.restype = ctypes.c_int
    lib.bench_mfma_lds.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_int, ctypes.c_void_p]
    iters = 8192
    cycles = torch.zeros(256 * 16, dtype=torch.int64, device="cuda")  # 2048 waves; 4096 for the LDS probe
    sink = torch.empty(256 * 512, dtype=torch.float32, device="cuda")
    src = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    names = ("mfma_only", "fragment_reads_only", "mfma_and_fragment_reads",
             "plus_barrier_every_4_ksteps", "plus_lds_dmas")
    lds_bytes = (0, 6 * 1024, 6 * 1024, 6 * 1024, 8 * 1024)  # per wave per k-step
    res = {}
    s = torch.cuda.current_stream()
    for v, name in enumerate(names):
        med = []
        for _ in range(3):
            rc = lib.bench_mfma_lds(v, cycles.data_ptr(), sink.data_ptr(), src.data_ptr(), iters,
                                    s.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"bench_mfma_lds failed (hipError {rc})")
            torch.cuda.synchronize()
            per_wg = cycles[:2048].view(256, 8).max(dim=1).values.double()
            med.append(float(per_wg.median()))
        c = statistics.median(med)
        entry = {"cycles_per_wave": round(c)}
        if v != 1:
            per_mfma = c / (2 * 8 * iters)
            entry["cycles_per_mfma_per_simd"] = round(per_mfma, 2)
            entry["mfma_busy"] = round(32.0 / per_mfma, 4)
        entry["lds_bytes_per_clk_per_cu"] = round(8 * iters * lds_bytes[v] / c, 1)
        res[name] = entry
    # LDS read throughput alone at 1, 2 and 4 waves per SIMD (bench_probe's lds_read_kernel)
    lib.bench_lds_read.restype = ctypes.c_int
    lib.bench_lds_read.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                   ctypes.c_void_p]
    lds_read = {}
    rsink = torch.empty(256 * 64 * 16, dtype=torch.int32, device="cuda")
    for w in (4, 8, 16):
        med = []
        for _ in range(3):
            rc = lib.bench_lds_read(w, cycles.data_ptr(), rsink.data_ptr(), 4096, s.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"bench_lds_read failed (hipError {rc})")
            torch.cuda.synchronize()
            med.append(float(cycles[:256 * w].view(256, w).max(dim=1).values.double().median()))
        lds_read[f"{w}_waves_per_cu"] = round(w * 4096 * 8 * 1024 / statistics.median(med), 1)
    # the datasheet's 2.5 PFLOP/s is 256 CUs x 4096 flop per clock x 2.4 GHz: the MFMA-only
    # variant measures the flop per clock a CU's four SIMDs issue
    per_clk = 4 * 32 * 32 * 16 * 2 / res["mfma_only"]["cycles_per_mfma_per_simd"]
    return {"kernel": "bench_probe.hip mfma_lds_kernel (256 x 8 waves, 8192 k-steps per wave)",
            "bf16_flop_per_clk_per_cu": round(per_clk, 1), "variants": res,
            "lds_read_bytes_per_clk_per_cu": lds_read}


# ------------------------------------------------------------------ HBM counter calibration

COPY_BYTES = 1 << 30


def copy_calibration(torch, reps: int = 5) -> None:
    """A plain device copy of COPY_BYTES (torch's copy kernel): under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch should read COPY_BYTES; the ratio scales the
    counters of our kernels to bytes."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()


def _pmc_rows(d: str):
    import csv
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    for f in files:
        with open(f) as fh:
            yield from csv.DictReader(fh)


def _per_dispatch(d: str, counter: str):
    """{kernel name: [counter value per dispatch]} for one rocprofv3 --pmc run."""
    vals = {}
    per = {}
    for r in _pmc_rows(d):
        if r.get("Counter_Name") != counter:
            continue
        key = (r.get("Dispatch_Id") or r.get("Correlation_Id"), r["Kernel_Name"])
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    for (_, name), v in per.items():
        vals.setdefault(name, []).append(v)
    return vals


def summarize_pmc(fetch_dir: str, write_dir: str, workload: str, kernel_substr: str,
                  commands: dict, kind: str) -> dict:
    """Traffic per launch of the kernel whose name contains `kernel_substr`, from a
    FETCH_SIZE run and a WRITE_SIZE run (KiB per dispatch), each scaled by the same
    counter's reading for the COPY_BYTES copy kernel in the same run."""
    out = {"workload": workload, "kernel_match": kernel_substr, "commands": commands,
           "copy_bytes": COPY_BYTES, "source_files": KERNEL_SOURCES[kind] + ["(compile flags)"],
           "source_sha256": source_digest(kind)}
    total = 0.0
    for label, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        vals = _per_dispatch(d, counter)
        # the calibration copies are the largest copy dispatches of the run
        copy = sorted((v for k, vs in vals.items() if "copy" in k.lower() for v in vs),
                      reverse=True)[:5]
        mine = [v for k, vs in vals.items() if kernel_substr in k for v in vs]
        if not copy or not mine:
            raise SystemExit(f"{counter}: kernels seen: {sorted(vals)}")
        copy_kib = statistics.median(copy)
        mine_kib = statistics.median(mine)
        scale = (COPY_BYTES / 1024.0) / copy_kib
        bytes_ = mine_kib * 1024.0 * scale
        out[label] = {"counter": counter, "kernel_kib_per_dispatch_median": round(mine_kib, 1),
                      "dispatches": len(mine), "copy_kib_per_dispatch_median": round(copy_kib, 1),
                      "scale": round(scale, 5), "bytes_per_launch": round(bytes_)}
        total += bytes_
    out["traffic_bytes_per_launch"] = round(total)
    return out


def _work_of(w):
    """(algorithmic bytes, algorithmic flops or None) of one step of a workload."""
    if w.kind == "xent":
        return xent_bytes(w.tokens, w.vocab, 4 if w.dtype == "f32" else 2, w.reduction), None
    return (fused_bytes(w.tokens, w.hidden, w.vocab, w.reduction),
            fused_flops(w.tokens, w.hidden, w.vocab))


def summarize_trace(trace_dir: str, workload: str, kernel_substr: str, command: str) -> str:
    """profiles/kernel_trace_<workload>.md from one rocprofv3 --kernel-trace --stats run:
    the busiest kernels, and the duration spread of the dispatches of the kernel whose
    name contains `kernel_substr`, with its roofline at the median and mean duration."""
    import csv
    import lce_synth
    w = lce_synth.WORKLOADS[workload]
    tf = glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True)
    sf = glob.glob(os.path.join(trace_dir, "**", "*kernel_stats.csv"), recursive=True)
    if not tf or not sf:
        raise SystemExit(f"no kernel_trace.csv / kernel_stats.csv under {trace_dir}")
    rows = [r for r in csv.DictReader(open(tf[0])) if kernel_substr in r["Kernel_Name"]]
    if not rows:
        raise SystemExit(f"no dispatch of {kernel_substr} in {tf[0]}")
    d = sorted((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0 for r in rows)
    q = lambda f: d[min(len(d) - 1, int(round(f * (len(d) - 1))))]
    med, mean = statistics.median(d), statistics.fmean(d)
    r0 = rows[0]
    b, fl = _work_of(w)
    lines = [f"# Kernel trace: {workload}", "",
             "Command (run from /tmp on one MI355X, repository at $R):", "", f"    {command}", "",
             "Busiest kernels (run_kernel_stats.csv; every launch of the process, durations in µs):",
             "", "| kernel | calls | average | min | max |", "|---|---|---|---|---|"]
    for s in list(csv.DictReader(open(sf[0])))[:5]:
        lines.append(f"| `{s['Name'][:90]}` | {s['Calls']} | {float(s['AverageNs']) / 1000:.2f} | "
                     f"{float(s['MinNs']) / 1000:.2f} | {float(s['MaxNs']) / 1000:.2f} |")
    lines += ["", f"Dispatches of `{kernel_substr}` (run_kernel_trace.csv: eager warm-up and reference "
              "calls and graph replays): " + f"{len(d)} dispatches, grid {r0['Grid_Size_X']} x "
              f"{r0['Grid_Size_Y']} work-items in workgroups of {r0['Workgroup_Size_X']}, "
              f"{r0['LDS_Block_Size']} bytes of LDS.", "",
              "| statistic | µs |", "|---|---|"]
    for k, v in (("median", med), ("mean", mean), ("p10", q(0.1)), ("p90", q(0.9)),
                 ("min", d[0]), ("max", d[-1])):
        lines.append(f"| {k} | {v:.2f} |")
    lines.append("")
    if fl is None:
        lines.append(f"Algorithmic bytes per launch: {b:,} (each input and output tensor once). At the "
                     f"median duration that is {b / (med * 1e3):.1f} GB/s = "
                     f"{b / (med * 1e3) / HBM_PEAK_GBS:.4f} of 8 TB/s; at the mean, "
                     f"{b / (mean * 1e3):.1f} GB/s = {b / (mean * 1e3) / HBM_PEAK_GBS:.4f}.")
    else:
        lines.append(f"Algorithmic flops per launch: {fl:,} (2·T·H·V). At the median duration that is "
                     f"{fl / (med * 1e6):.1f} TFLOP/s = {fl / (med * 1e6) / BF16_DENSE_TFLOPS:.4f} of "
                     f"2.5 PFLOP/s; at the mean, {fl / (mean * 1e6):.1f} TFLOP/s.")
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"kernel_trace_{workload}.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def traffic_markdown(d: dict) -> str:
    """profiles/traffic_<workload>.md beside the JSON summary of summarize_pmc."""
    import lce_synth
    w = lce_synth.WORKLOADS[d["workload"]]
    b, _ = _work_of(w)
    lines = [f"# HBM traffic: {d['kernel_match']} on {d['workload']}", "",
             f"Two counter runs, each with a {COPY_BYTES >> 30} GiB device copy (`--copy-calibration`) "
             "in the same process (run from /tmp, repository at $R):", ""]
    lines += [f"    {c}" for c in d["commands"].get("runs", [])]
    lines += ["", f"Summary (traffic_{d['workload']}.json, written by `python bench.py --summarize-pmc "
              f"<fetch dir> <write dir> --workloads {d['workload']} --kernel {d['kernel_match']}`; it "
              "is used by bench.py only while the kernel's sources hash to its `source_sha256`).", "",
              "| counter | kernel, KiB per dispatch (median) | dispatches | copy, KiB per dispatch | "
              "scale | bytes per launch |", "|---|---|---|---|---|---|"]
    for k in ("fetch", "write"):
        e = d[k]
        lines.append(f"| {e['counter']} | {e['kernel_kib_per_dispatch_median']} | {e['dispatches']} | "
                     f"{e['copy_kib_per_dispatch_median']} | {e['scale']} | {e['bytes_per_launch']:,} |")
    t = d["traffic_bytes_per_launch"]
    lines += ["", f"Traffic per launch: {t:,} B against {b:,} algorithmic bytes: "
              f"{t / b:.4f}x.", ""]
    return "\n".join(lines)


# ------------------------------------------------------------------ main

def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workloads", default="all",
                    help="'all', 'headline', or a comma list of workload names")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extras", default=None,
                    help="comma list of extra measurements (backward, shard, sums, jsd, "
                         "fused_bwd, split, sweep, stream_read, skeleton); default: all of them "
                         "when --workloads is all")
    ap.add_argument("--eager", action="store_true",
                    help="time plain launches instead of a graph replay (for profiler runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 1 GiB device copy (counter calibration for rocprofv3 --pmc)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<workload>.json from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-trace", metavar="TRACE_DIR",
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 --kernel-trace run")
    ap.add_argument("--kernel", default="xent_wave_rows_kernel",
                    help="kernel name substring for --summarize-pmc / --summarize-trace")
    ap.add_argument("--pmc-command", action="append", default=[],
                    help="command lines of the profiler runs, recorded in the summary")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        import lce_synth
        wl = lce_synth.HEADLINE if args.workloads in ("all", "headline") else args.workloads
        d = summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], wl, args.kernel,
                          {"runs": args.pmc_command}, lce_synth.WORKLOADS[wl].kind)
        os.makedirs(PROFILES, exist_ok=True)
        path = os.path.join(PROFILES, f"traffic_{wl}.json")
        with open(path, "w") as fh:
            json.dump(d, fh, indent=1)
        with open(os.path.join(PROFILES, f"traffic_{wl}.md"), "w") as fh:
            fh.write(traffic_markdown(d))
        print(json.dumps(d))
        return 0
    if args.summarize_trace:
        import lce_synth
        wl = lce_synth.HEADLINE if args.workloads in ("all", "headline") else args.workloads
        print(summarize_trace(args.summarize_trace, wl, args.kernel, " ".join(args.pmc_command)))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: liblce has no multi-GPU path "
              "(rows would shard across GPUs with one 8-byte all-reduce for the mean). "
              "Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch
    import lce_synth
    import vocab_cross_entropy_row_amd as lce

    lce.load()
    torch.cuda.set_device(0)
    if args.workloads == "all":
        names = list(lce_synth.WORKLOADS)
    elif args.workloads == "headline":
        names = [lce_synth.HEADLINE]
    else:
        names = args.workloads.split(",")
        unknown = [n for n in names if n not in lce_synth.WORKLOADS]
        if unknown:
            raise SystemExit(f"unknown workloads {unknown}; choose from {list(lce_synth.WORKLOADS)}")
    # The line's head: the headline workload when it is measured, else the first named.
    head_name = lce_synth.HEADLINE if lce_synth.HEADLINE in names else names[0]
    head = lce_synth.WORKLOADS[head_name]

    all_extras = ("backward", "shard", "sums", "jsd", "fused_bwd", "split", "sweep", "stream_read",
                  "skeleton")
    if args.extras is not None:
        extras = [e for e in args.extras.split(",") if e]
        unknown = [e for e in extras if e not in all_extras]
        if unknown:
            raise SystemExit(f"unknown extras {unknown}; choose from {all_extras}")
    else:
        extras = list(all_extras) if args.workloads == "all" and not args.eager else []
    if "split" in extras or "sweep" in extras:
        KEEP.update({"ce_f32_16384x131072_mean", "megatron_bf16_2048x4x131072_none"})
        names += [n for n in sorted(KEEP) if n not in names]
    if "sweep" in extras:
        KEEP.add("fused_bf16_t2048_h4096_v128256_mean")
        if "fused_bf16_t2048_h4096_v128256_mean" not in names:
            names.append("fused_bf16_t2048_h4096_v128256_mean")

    results = {}
    for name in names:
        w = lce_synth.WORKLOADS[name]
        big = w.kind == "fused" or w.tokens * w.vocab >= (1 << 30)
        k = args.steps if not big else max(5, min(args.steps, 30))
        print(f"[bench] {name}: {k} steps", file=sys.stderr, flush=True)
        r = time_workload(w, k, args.warmup, torch, lce, eager_only=args.eager)
        r["steps"] = k
        r["roofline"] = roofline_entry(w, r["us_per_step"])
        if not args.no_cpu and name != head_name:
            r["cpu_oracle"] = cpu_baseline(w, budget_s=5.0)
        results[name] = r
        print(f"[bench] {name}: {r['us_per_step']:.2f} µs/step (median; "
              f"{r['roofline']['achieved']} {r['roofline']['unit']}) via {r['launch']}",
              file=sys.stderr, flush=True)

    shard = sums = jsd = fbwd = split = sweeps = None
    backward = {}
    if "backward" in extras:
        for bname in ("megatron_bf16_2048x4x4096_none", "ce_f32_16384x4096_mean"):
            bw = lce_synth.WORKLOADS[bname]
            backward[bname] = time_backward(bw, torch, lce, min(args.steps, 200), args.warmup)
            ts = backward[bname]["training_step"]
            print(f"[bench] backward {bname}: {backward[bname]['us_per_step']:.2f} µs/step "
                  f"({backward[bname]['roofline']['achieved']} GB/s); forward + backward "
                  f"{ts['forward_then_backward_us']:.2f} µs in two calls, {ts['fwd_bwd_us']:.2f} µs "
                  f"in one", file=sys.stderr, flush=True)
    if "shard" in extras:
        shard = time_vocab_shard(torch, lce, lce_synth, 8, min(args.steps, 200), args.warmup)
        print(f"[bench] vocab shard tp=8: partial {shard['partial_us']:.2f} µs (plain read of "
              f"its bytes {shard['shard_read_only_us']} µs), merge {shard['merge_us']:.2f} µs, "
              f"max |diff| vs unsplit {shard['max_abs_diff_vs_unsplit']:.2e}",
              file=sys.stderr, flush=True)
    if "split" in extras:
        split = time_split(torch, lce, lce_synth, min(args.steps, 200), args.warmup)
    if "sweep" in extras:
        sweeps = time_sweeps(torch, lce, lce_synth, min(args.steps, 100), args.warmup)
    _KEPT.clear()
    torch.cuda.empty_cache()
    if "sums" in extras:
        sums = time_logprob_sums(torch, lce, lce_synth, min(args.steps, 10), 2)
        print(f"[bench] fused log-prob sums: {sums['us_per_step']:.1f} µs "
              f"({sums['roofline']['achieved']} TFLOP/s)", file=sys.stderr, flush=True)
    if "jsd" in extras:
        jsd = time_jsd(torch, lce, lce_synth, min(args.steps, 10), 2)
        print(f"[bench] fused linear + JSD: stored {jsd['stored']['us_per_step']:.1f} µs "
              f"({jsd['stored']['roofline']['achieved']} TFLOP/s), recompute "
              f"{jsd['recompute']['us_per_step']:.1f} µs", file=sys.stderr, flush=True)
    if "fused_bwd" in extras:
        fbwd = time_fused_bwd(torch, lce, lce_synth, min(args.steps, 5), 2)
        print(f"[bench] fused backward: {fbwd['us_per_step']:.1f} µs "
              f"({fbwd['roofline']['achieved']} TFLOP/s over 3*2THV); forward + backward "
              f"{fbwd['training_step']['forward_then_backward_us']:.1f} µs in two calls, "
              f"{fbwd['training_step']['fwd_bwd_us']:.1f} µs in one", file=sys.stderr, flush=True)

    probe = None
    if "stream_read" in extras and "megatron_bf16_2048x4x4096_none" in results:
        pw = lce_synth.WORKLOADS["megatron_bf16_2048x4x4096_none"]
        hb = pw.tokens * pw.vocab * 2
        probe = time_stream_read(torch, hb, results[pw.name]["replicas"], min(args.steps, 200))
        probe["workload"] = pw.name
        probe["kernel_us_over_read_only_us"] = round(results[pw.name]["us_per_step"] / probe["read_us"], 4)
        probe["valu_rate"] = time_valu_rate(torch)
        print(f"[bench] streaming read: {probe['gbs_2GiB']} GB/s over 2 GiB, "
              f"{probe['read_us']:.2f} µs for {pw.name}'s {hb} logit bytes",
              file=sys.stderr, flush=True)

    skeleton = None
    if "skeleton" in extras:
        skeleton = time_fused_skeleton(torch)
        sv = skeleton["variants"]
        print("[bench] fused-loop skeleton, MFMA busy: " + ", ".join(
            f"{k} {v['mfma_busy']:.3f}" for k, v in sv.items() if "mfma_busy" in v) +
            "; LDS reads alone (B/clk/CU) at 4, 8, 16 waves per CU: " +
            ", ".join(str(v) for v in skeleton["lds_read_bytes_per_clk_per_cu"].values()),
            file=sys.stderr, flush=True)

    if args.copy_calibration:
        copy_calibration(torch)

    h = results[head_name]
    cfg = {"workload": head.name}
    if head.kind == "xent":
        cfg.update({"tokens": head.tokens, "vocab": head.vocab, "logits_dtype": head.dtype,
                    "logits_shape": list(head.shape)})
    else:
        cfg.update({"tokens": head.tokens, "hidden": head.hidden, "vocab": head.vocab})
    cfg.update({"reduction": head.reduction,
                "timing": ("eager launches" if args.eager else
                           f"hip graph of K steps; median over {SPREAD_REPLAYS} timed replays"),
                "eager_us_per_call": round(h["eager_us_per_call"], 3),
                "replicas": h["replicas"], "graph_matches_eager": h["graph_matches_eager"],
                "spread": h.get("spread")})
    roof = {k: v for k, v in h["roofline"].items() if k in
            ("bound", "achieved", "peak", "unit", "frac", "traffic")}
    roof["kernel"] = h["launch"].split(" + ")[0]
    roof["launch"] = h["launch"]
    roof["duration_us"] = h["us_per_step"]
    roof["algorithmic_bytes"] = h["roofline"].get("algorithmic_bytes")
    if "algorithmic_flops" in h["roofline"]:
        roof["algorithmic_flops"] = h["roofline"]["algorithmic_flops"]
    line = {
        "metric": METRIC,
        "value": round(h["us_per_step"], 3),
        "unit": "µs",
        "n_gpus": 1,
        "steps": h["steps"],
        "warmup": args.warmup,
        "ms_per_step": round(h["us_per_step"] / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head.dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(head)
    line["workloads"] = {n: {"us_per_step": round(r["us_per_step"], 3),
                             "rows_per_s": round(lce_synth.WORKLOADS[n].tokens / (r["us_per_step"] * 1e-6)),
                             "spread": r.get("spread"), "launch": r["launch"],
                             "eager_us_per_call": round(r["eager_us_per_call"], 3),
                             "steps": r["steps"], "replicas": r["replicas"],
                             "graph_matches_eager": r["graph_matches_eager"],
                             "roofline": r["roofline"],
                             **({"cpu_oracle": r["cpu_oracle"]} if "cpu_oracle" in r else {})}
                         for n, r in results.items()}
    if split is not None:
        line["split_path"] = split
    if sweeps is not None:
        line["sweeps"] = sweeps
    if shard is not None:
        line["vocab_shard_tp8"] = shard
    if backward:
        line["backward"] = backward
    if sums is not None:
        line["fused_logprob_sums"] = sums
    if jsd is not None:
        line["fused_linear_jsd"] = jsd
    if fbwd is not None:
        line["fused_backward"] = fbwd
    if probe is not None:
        line["stream_read_probe"] = probe
    if skeleton is not None:
        line["fused_skeleton_probe"] = skeleton
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
