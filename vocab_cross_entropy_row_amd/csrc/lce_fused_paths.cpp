// liblce entry points built on the fused projection: its backward
// (lce_fused_linear_xent_bwd) and fused linear + generalized JSD
// (lce_fused_linear_jsd_fwd), with their chunking and scratch plans.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <cstdint>

#include "fused_grad.h"
#include "lce.h"
#include "lce_host.h"
#include "lce_internal.h"

namespace lce {
namespace host {

// Gradients of the fused projection + cross-entropy, for chunks of tokens.
// Stored path (default): the forward kernel's store mode gives each chunk's
// log-sum-exp and writes its fp32 logits [chunk, ld] into scratch, then
// fused_grad_rows_kernel turns them into the bf16 logit gradient dZ [chunk,
// ld].  Recompute path (when not even 256 tokens of fp32 logits and dZ fit):
// the forward kernel gives every token's log-sum-exp, then for each chunk
// the fused kernel's gradient mode recomputes the logits and writes dZ.
// Either way two library GEMMs consume dZ: dx[chunk] = dZ W and
// dW (+)= dZ^T x[chunk].  With `out`, the pass that gives the log-sum-exps
// also gives the forward's losses: per token into out, or their mean (the
// merge's own mean when one pass covers every token, else a mean kernel over
// per-token losses kept in scratch).  Chunks are the largest multiple of 256 tokens whose
// buffers (6 or 2 bytes per logit) fit in LCE_FUSED_BWD_STORE_BYTES (default
// 2 GiB), at least 256.
constexpr size_t kGemmWorkspace = size_t(128) << 20;
// Most tokens per chunk: the per-token streaming kernels launch 256 work-items
// per token, and a dispatch counts its work-items in 32 bits.
constexpr int64_t kMaxChunk = (int64_t(1) << 24) - 256;

// The stored path also needs the store mode's 32-bit addressing: a token
// tile's fp32 rows (block_tokens * ld * 4 bytes) go through one buffer
// resource.  Beyond that (vocab >= 2^22 - 256 with the tile of 256 tokens)
// the recompute path is taken whatever the cap, since its bf16 dZ rows need
// half the bytes (the entry point refuses vocab >= 2^23 - 256).
FusedBwdPlan plan_fused_bwd(int64_t tokens, int64_t vocab, int64_t cap) {
  FusedBwdPlan p;
  const lce::FusedGeometry geo = lce::fused_geometry();
  p.ld = (vocab + geo.block_vocab - 1) / geo.block_vocab * geo.block_vocab;
  const bool addressable = p.ld * geo.block_tokens * 4 < (int64_t(1) << 32);
  p.stored = addressable && cap / (p.ld * 6) >= geo.block_tokens;
  int64_t chunk = cap / (p.ld * (p.stored ? 6 : 2)) / geo.block_tokens * geo.block_tokens;
  if (chunk < geo.block_tokens) chunk = geo.block_tokens;
  if (chunk > kMaxChunk) chunk = kMaxChunk;
  if (chunk > tokens) chunk = tokens;
  p.chunk = chunk;
  return p;
}

lce_status run_fused_bwd(const void* x, const void* weight, int64_t tokens, int64_t hidden,
                         int64_t vocab, const int64_t* target, bool mean, const float* grad,
                         float* dx, float* dw, float* out, hipStream_t stream) {
  lce_status s = LCE_OK;
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;
  const FusedBwdPlan plan =
      plan_fused_bwd(tokens, vocab, env_int64("LCE_FUSED_BWD_STORE_BYTES", int64_t(2) << 30));
  const int64_t ld = plan.ld, chunk = plan.chunk;
  const bool stored = plan.stored;

  Carve cv;
  const size_t off_lse = cv.take((size_t)tokens * 4u);
  const size_t off_ws = cv.take(kGemmWorkspace);
  const size_t off_dz = cv.take((size_t)chunk * (size_t)ld * 2u);
  const size_t off_z = cv.take(stored ? (size_t)chunk * (size_t)ld * 4u : 0u);
  // dW = x^T dZ as a product of two transposed operands: x^T [hidden, chunk]
  // is written once per chunk (hipBLASLt's NT kernels for this shape, dZ read
  // as stored, measured slower).
  const bool dw_tt = dw && env_int("LCE_FUSED_BWD_DW_NT", 0) == 0;
  const size_t off_xt = cv.take(dw_tt ? (size_t)chunk * (size_t)hidden * 2u : 0u);
  // A mean over several stored chunks: their per-token losses first.
  const bool chunk_losses = out && mean && stored && chunk < tokens;
  const size_t off_loss = cv.take(chunk_losses ? (size_t)tokens * 4u : 0u);
  const size_t reserved = cv.off - Carve().off;
  const int64_t last = tokens - (tokens - 1) / chunk * chunk;
  size_t need = cv.off;
  for (int64_t n : {stored ? chunk : tokens, last}) {
    const FusedPlan fp = plan_fused(n, vocab, cus, reserved);
    if (fp.end > need) need = fp.end;
  }
  char* base = nullptr;
  if ((s = get_scratch(stream, need, &base)) != LCE_OK) return s;
  float* lse = (float*)(base + off_lse);
  void* ws = base + off_ws;
  void* dz = base + off_dz;
  float* z = (float*)(base + off_z);
  uint16_t* xt = (uint16_t*)(base + off_xt);
  float* losses = (float*)(base + off_loss);

  if (!stored && (s = run_fused(x, weight, tokens, hidden, vocab, target, mean, out, stream,
                                reserved, lse)) != LCE_OK)
    return s;
  const uint16_t* x16 = (const uint16_t*)x;
  for (int64_t c0 = 0; c0 < tokens; c0 += chunk) {
    const int64_t n = tokens - c0 < chunk ? tokens - c0 : chunk;
    hipError_t e = hipSuccess;
    if (stored) {
      float* chunk_out = !out ? nullptr : chunk_losses ? losses + c0 : mean ? out : out + c0;
      if ((s = run_fused(x16 + c0 * hidden, weight, n, hidden, vocab, target + c0,
                         mean && !chunk_losses, chunk_out, stream, reserved, lse + c0, z, ld)) != LCE_OK)
        return s;
      lce::FusedGradRowsArgs g{};
      g.z = z;
      g.lse = lse + c0;
      g.target = target + c0;
      g.grad = mean ? grad : grad + c0;
      g.grad_mean = mean ? 1 : 0;
      g.grad_tokens = tokens;
      g.rows = n;
      g.vocab = vocab;
      g.ld = ld;
      g.dz = (uint16_t*)dz;
      e = lce::launch_fused_grad_rows(g, stream);
      if (e == hipSuccess) note_launch("fused_grad_rows_kernel grid %lld x 256", (long long)n);
    } else {
      lce::FusedGradArgs g{};
      g.x = x16 + c0 * hidden;
      g.w = weight;
      g.tokens = n;
      g.hidden = hidden;
      g.vocab = vocab;
      g.target = target + c0;
      g.lse = lse + c0;
      g.grad = mean ? grad : grad + c0;
      g.grad_mean = mean ? 1 : 0;
      g.grad_tokens = tokens;
      g.dz = dz;
      g.dz_ld = ld;
      g.segments = lce::fused_segments(n, vocab, cus);
      e = lce::launch_fused_grad(g, stream);
      if (e == hipSuccess) note_launch("fused_xent_partial_kernel (logit gradient)");
    }
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    // Row-major [r, c] is column-major [c, r]: dx^T[H, n] = W^T[H, V] dZ^T[V, n],
    // dW^T[H, V] (+)= x^T[H, n] dZ[n, V].
    if (dx && (s = gemm_bf16_f32(HIPBLAS_OP_N, HIPBLAS_OP_N, hidden, n, vocab, weight, hidden, dz,
                                 ld, 0.0f, dx + c0 * hidden, hidden, ws, kGemmWorkspace,
                                 stream)) != LCE_OK)
      return s;
    if (dw && dw_tt) {
      // x^T[H, n] as column-major [n, H] (row-major [H, n]) read transposed,
      // dZ row-major [n, ld] (column-major [ld, n]) read transposed.
      e = lce::launch_transpose_u16(x16 + c0 * hidden, n, hidden, xt, stream);
      if (e != hipSuccess) return hip_fail(e, "kernel launch");
      note_launch("transpose_u16_kernel");
      if ((s = gemm_bf16_f32(HIPBLAS_OP_T, HIPBLAS_OP_T, hidden, vocab, n, xt, n, dz, ld,
                             c0 == 0 ? 0.0f : 1.0f, dw, hidden, ws, kGemmWorkspace, stream)) != LCE_OK)
        return s;
    } else if (dw && (s = gemm_bf16_f32(HIPBLAS_OP_N, HIPBLAS_OP_T, hidden, vocab, n,
                                        x16 + c0 * hidden, hidden, dz, ld, c0 == 0 ? 0.0f : 1.0f,
                                        dw, hidden, ws, kGemmWorkspace, stream)) != LCE_OK) {
      return s;
    }
  }
  if (chunk_losses) {
    MeanState ms;
    if ((s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
      return s;
    hipError_t e = lce::launch_jsd_mean(tokens, losses, out, ms.slots, ms.epoch, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    note_launch("fused_jsd_merge_kernel (mean of the chunks' losses)");
  }
  return LCE_OK;
}

// Fused linear + JSD.  Both paths first take each head's per-token
// log-sum-exp with the fused cross-entropy kernel.  The stored path has that
// kernel also write both heads' fp32 logits for a chunk of tokens into scratch
// and then streams them once (jsd_stored_rows_kernel); the recompute path
// multiplies both heads again, tile by tile (the fused kernel's JSD mode), and
// needs no logit storage.  The stored path is taken when a chunk of at least
// one fused token tile fits in LCE_JSD_STORE_BYTES (default 2 GiB) of scratch.
struct JsdPlan {
  int64_t chunk = 0;  // tokens per chunk; 0: recompute path
  int64_t ld = 0;     // stored row length (vocab rounded up to the fused tile)
};

JsdPlan plan_jsd(int64_t tokens, int64_t vocab) {
  JsdPlan p;
  const lce::FusedGeometry g = lce::fused_geometry();
  const int64_t ld = (vocab + g.block_vocab - 1) / g.block_vocab * g.block_vocab;
  // Byte offsets within a token tile's rows are 32-bit.
  if (ld * g.block_tokens * 4 >= (int64_t(1) << 32)) return p;
  const int64_t cap = env_int64("LCE_JSD_STORE_BYTES", int64_t(2) << 30);
  const int64_t per_token = ld * 8;  // both heads' rows
  int64_t max_chunk = cap / per_token / g.block_tokens * g.block_tokens;
  if (max_chunk < g.block_tokens) return p;
  if (max_chunk > kMaxChunk) max_chunk = kMaxChunk;
  if (tokens <= max_chunk) {
    p.chunk = tokens;
  } else {
    const int64_t n = (tokens + max_chunk - 1) / max_chunk;
    const int64_t even = (tokens + n - 1) / n;
    p.chunk = (even + g.block_tokens - 1) / g.block_tokens * g.block_tokens;  // <= max_chunk
  }
  p.ld = ld;
  return p;
}

lce_status run_jsd_stored(const void* xs, const void* ws, const void* xt, const void* wt,
                          int64_t tokens, int64_t hidden, int64_t vocab, float beta, bool mean,
                          float* out, hipStream_t stream, int cus, const JsdPlan& plan) {
  lce_status s = LCE_OK;
  Carve cv;
  const size_t off_ls = cv.take((size_t)tokens * 4u);
  const size_t off_lt = cv.take((size_t)tokens * 4u);
  const size_t off_per = cv.take(mean ? (size_t)tokens * 4u : 0u);
  const size_t zbytes = (size_t)plan.chunk * (size_t)plan.ld * 4u;
  const size_t off_zs = cv.take(zbytes);
  const size_t off_zt = cv.take(zbytes);
  const size_t reserved = cv.off - Carve().off;
  // The fused kernel's own regions follow; size them for the largest chunk
  // and for the last (smaller) one, whose plan may differ.
  const int64_t last = tokens - (tokens - 1) / plan.chunk * plan.chunk;
  size_t need = cv.off;
  for (int64_t n : {plan.chunk, last}) {
    const FusedPlan fp = plan_fused(n, vocab, cus, reserved);
    if (fp.end > need) need = fp.end;
  }
  char* base = nullptr;
  if ((s = get_scratch(stream, need, &base)) != LCE_OK) return s;
  MeanState ms;
  if (mean && (s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
    return s;
  float* lse_s = (float*)(base + off_ls);
  float* lse_t = (float*)(base + off_lt);
  float* per = mean ? (float*)(base + off_per) : out;
  float* zs = (float*)(base + off_zs);
  float* zt = (float*)(base + off_zt);

  const uint16_t* xs16 = (const uint16_t*)xs;
  const uint16_t* xt16 = (const uint16_t*)xt;
  for (int64_t c0 = 0; c0 < tokens; c0 += plan.chunk) {
    const int64_t n = tokens - c0 < plan.chunk ? tokens - c0 : plan.chunk;
    if ((s = run_fused(xs16 + c0 * hidden, ws, n, hidden, vocab, nullptr, false, nullptr, stream,
                       reserved, lse_s + c0, zs, plan.ld)) != LCE_OK)
      return s;
    if ((s = run_fused(xt16 + c0 * hidden, wt, n, hidden, vocab, nullptr, false, nullptr, stream,
                       reserved, lse_t + c0, zt, plan.ld)) != LCE_OK)
      return s;
    lce::JsdRowsArgs r{};
    r.zs = zs;
    r.zt = zt;
    r.z_ld = plan.ld;
    r.rows = n;
    r.vocab = vocab;
    r.lse_s = lse_s + c0;
    r.lse_t = lse_t + c0;
    r.beta = beta;
    r.dst = per + c0;
    hipError_t e = lce::launch_jsd_rows(r, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    note_launch("jsd_stored_rows_kernel grid %lld x 256", (long long)n);
  }
  if (mean) {
    hipError_t e = lce::launch_jsd_mean(tokens, per, out, ms.slots, ms.epoch, stream);
    if (e != hipSuccess) return hip_fail(e, "kernel launch");
    note_launch("fused_jsd_merge_kernel (mean)");
  }
  return LCE_OK;
}

lce_status run_jsd_recompute(const void* xs, const void* ws, const void* xt, const void* wt,
                             int64_t tokens, int64_t hidden, int64_t vocab, float beta, bool mean,
                             float* out, hipStream_t stream, int cus) {
  lce_status s = LCE_OK;
  // Scratch: both heads' log-sum-exp, the divergence kernel's per-segment
  // sums and mean slots, then the cross-entropy kernel's own regions.
  lce::JsdArgs a{};
  a.xs = xs;
  a.ws = ws;
  a.xt = xt;
  a.wt = wt;
  a.tokens = tokens;
  a.hidden = hidden;
  a.vocab = vocab;
  a.beta = beta;
  a.out = out;
  a.reduce_mean = mean ? 1 : 0;
  a.segments = lce::jsd_segments(tokens, vocab, cus);
  Carve cv;
  const size_t off_ls = cv.take((size_t)tokens * 4u);
  const size_t off_lt = cv.take((size_t)tokens * 4u);
  const size_t off_part = cv.take((size_t)a.segments * (size_t)tokens * 4u);
  const size_t reserved = cv.off - Carve().off;
  const FusedPlan fp = plan_fused(tokens, vocab, cus, reserved);
  char* base = nullptr;
  if ((s = get_scratch(stream, fp.end > cv.off ? fp.end : cv.off, &base)) != LCE_OK) return s;
  float* lse_s = (float*)(base + off_ls);
  float* lse_t = (float*)(base + off_lt);
  a.lse_s = lse_s;
  a.lse_t = lse_t;
  a.partials = (float*)(base + off_part);
  if (mean) {
    MeanState ms;
    if ((s = get_mean_state(stream, (tokens + lce::kRowThreads - 1) / lce::kRowThreads, &ms)) != LCE_OK)
      return s;
    a.mean_slots = ms.slots;
    a.epoch = ms.epoch;
  }

  if ((s = run_fused(xs, ws, tokens, hidden, vocab, nullptr, false, nullptr, stream, reserved,
                     lse_s)) != LCE_OK)
    return s;
  if ((s = run_fused(xt, wt, tokens, hidden, vocab, nullptr, false, nullptr, stream, reserved,
                     lse_t)) != LCE_OK)
    return s;
  hipError_t e = lce::launch_jsd(a, stream);
  if (e != hipSuccess) return hip_fail(e, "kernel launch");
  const lce::FusedGeometry jg = lce::jsd_geometry();
  note_launch("fused_xent_partial_kernel<JSD mode> grid %lld x 512 + fused_jsd_merge_kernel",
              (long long)((tokens + jg.block_tokens - 1) / jg.block_tokens * a.segments));
  return LCE_OK;
}

}  // namespace host
}  // namespace lce

using namespace lce::host;

extern "C" {

lce_status lce_fused_linear_jsd_fwd(const void* student_x, const void* student_weight,
                                    const void* teacher_x, const void* teacher_weight,
                                    int64_t tokens, int64_t hidden, int64_t vocab, float beta,
                                    lce_reduction reduction, float* out, hipStream_t stream) {
  begin_call();
  lce_status s = validate_common(tokens, nullptr, (int)reduction, out, "out", false);
  if (s != LCE_OK) return s;
  const uint64_t ob = out_bytes(tokens, (int)reduction);
  if ((s = validate_head(student_x, student_weight, tokens, hidden, vocab, out, ob, "student_x",
                         "student_weight")) != LCE_OK)
    return s;
  if ((s = validate_head(teacher_x, teacher_weight, tokens, hidden, vocab, out, ob, "teacher_x",
                         "teacher_weight")) != LCE_OK)
    return s;
  if (!(beta > 0.0f && beta < 1.0f))
    return fail(LCE_ERR_INVALID_ARG, "beta must be in (0, 1) (got %g)", (double)beta);
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (tokens == 0) {
    if (!mean) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  int cus = 0;
  if ((s = num_cus(&cus)) != LCE_OK) return s;
  const JsdPlan plan = plan_jsd(tokens, vocab);
  if (plan.chunk > 0)
    return run_jsd_stored(student_x, student_weight, teacher_x, teacher_weight, tokens, hidden,
                          vocab, beta, mean, out, stream, cus, plan);
  return run_jsd_recompute(student_x, student_weight, teacher_x, teacher_weight, tokens, hidden,
                           vocab, beta, mean, out, stream, cus);
}

// Both fused gradient entry points: arguments checked here, `out` (the
// forward's output) only when non-null.
static lce_status fused_bwd_call(const void* x, const void* weight, int64_t tokens, int64_t hidden,
                                 int64_t vocab, const int64_t* target, lce_reduction reduction,
                                 const float* grad, float* out, float* dx, float* dweight,
                                 hipStream_t stream) {
  lce_status s = out ? validate_fused(x, weight, tokens, hidden, vocab, target, (int)reduction, out)
                     : validate_common(tokens, target, (int)reduction, nullptr, nullptr);
  if (s != LCE_OK) return s;
  if ((s = validate_head(x, weight, tokens, hidden, vocab, nullptr, 0)) != LCE_OK) return s;
  const bool mean = reduction == LCE_REDUCTION_MEAN;
  if (!dx && !dweight) return fail(LCE_ERR_INVALID_ARG, "dx and dweight are both NULL");
  if (tokens > 0 && !grad) return fail(LCE_ERR_INVALID_ARG, "grad is NULL");
  if (grad && !aligned(grad, 4)) return fail(LCE_ERR_INVALID_ARG, "grad is not 4-byte aligned");
  if ((dx && !aligned(dx, 4)) || (dweight && !aligned(dweight, 4)))
    return fail(LCE_ERR_INVALID_ARG, "dx and dweight must be 4-byte aligned");
  const int64_t ld = (vocab + 255) / 256 * 256;
  if (ld * 256 * 2 >= (int64_t(1) << 32))
    return fail(LCE_ERR_UNSUPPORTED, "vocab must be < 2^23 - 256 for the fused backward (got %lld)",
                (long long)vocab);
  const uint64_t xb = (uint64_t)(tokens * hidden * 2), wb = (uint64_t)(vocab * hidden * 2);
  const uint64_t dxb = dx ? (uint64_t)(tokens * hidden * 4) : 0, dwb = dweight ? (uint64_t)(vocab * hidden * 4) : 0;
  const uint64_t gb = mean ? 4u : (uint64_t)tokens * 4u, tb = (uint64_t)tokens * 8u;
  const struct { const void* p; uint64_t n; const char* name; } outs[2] = {{dx, dxb, "dx"}, {dweight, dwb, "dweight"}};
  for (const auto& o : outs) {
    if (!o.p) continue;
    if (overlaps(o.p, o.n, x, xb)) return fail(LCE_ERR_ALIAS, "%s overlaps x", o.name);
    if (overlaps(o.p, o.n, weight, wb)) return fail(LCE_ERR_ALIAS, "%s overlaps weight", o.name);
    if (overlaps(o.p, o.n, target, tb)) return fail(LCE_ERR_ALIAS, "%s overlaps target", o.name);
    if (overlaps(o.p, o.n, grad, gb)) return fail(LCE_ERR_ALIAS, "%s overlaps grad", o.name);
  }
  if (overlaps(dx, dxb, dweight, dwb)) return fail(LCE_ERR_ALIAS, "dx overlaps dweight");
  if (out) {
    const uint64_t ob = out_bytes(tokens, (int)reduction);
    if (overlaps(out, ob, grad, gb)) return fail(LCE_ERR_ALIAS, "out overlaps grad");
    if (overlaps(out, ob, dx, dxb)) return fail(LCE_ERR_ALIAS, "out overlaps dx");
    if (overlaps(out, ob, dweight, dwb)) return fail(LCE_ERR_ALIAS, "out overlaps dweight");
  }
  if (tokens == 0) {  // no token contributes: dweight is zero, dx is empty, a mean is NaN
    if (out && mean) {
      hipError_t e = lce::launch_fill_f32(out, 1, __builtin_nanf(""), stream);
      if (e != hipSuccess) return hip_fail(e, "launch");
    }
    if (!dweight) return LCE_OK;
    hipError_t e = lce::launch_fill_f32(dweight, vocab * hidden, 0.0f, stream);
    return e == hipSuccess ? LCE_OK : hip_fail(e, "launch");
  }
  return run_fused_bwd(x, weight, tokens, hidden, vocab, target, mean, grad, dx, dweight, out, stream);
}

lce_status lce_fused_linear_xent_bwd(const void* x, const void* weight, int64_t tokens,
                                     int64_t hidden, int64_t vocab, const int64_t* target,
                                     lce_reduction reduction, const float* grad, float* dx,
                                     float* dweight, hipStream_t stream) {
  begin_call();
  return fused_bwd_call(x, weight, tokens, hidden, vocab, target, reduction, grad, nullptr, dx,
                        dweight, stream);
}

lce_status lce_fused_linear_xent_fwd_bwd(const void* x, const void* weight, int64_t tokens,
                                         int64_t hidden, int64_t vocab, const int64_t* target,
                                         lce_reduction reduction, const float* grad, float* out,
                                         float* dx, float* dweight, hipStream_t stream) {
  begin_call();
  if (!out) return fail(LCE_ERR_INVALID_ARG, "out is NULL");
  return fused_bwd_call(x, weight, tokens, hidden, vocab, target, reduction, grad, out, dx, dweight,
                        stream);
}

}  // extern "C"
