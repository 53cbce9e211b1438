// C ABI of libvc: argument validation, split planning and dispatch.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/vc.h"
#include "launch.h"

namespace {

thread_local std::string g_err;

vc_status fail(vc_status s, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

constexpr int64_t kMaxTokens = int64_t(1) << 30;   // per (request, KV head) slot

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

vc_status hip_status(hipError_t e, const char *what) {
  if (e == hipSuccess) return VC_OK;
  return fail(VC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

#define REQ(cond, ...) \
  do {                 \
    if (!(cond)) return fail(VC_EINVAL, __VA_ARGS__); \
  } while (0)

vc_status check_heads(int B, int Hq, int Hkv, int D) {
  REQ(B >= 0 && Hq > 0 && Hkv > 0, "B, Hq, Hkv must be positive (B may be 0)");
  REQ(Hq % Hkv == 0, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  REQ(Hq / Hkv <= 16, "at most 16 query heads per KV head (got %d)", Hq / Hkv);
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call (got %lld)", (long long)B * Hkv);
  if (D != 64 && D != 128) return fail(VC_ENOTSUP, "head_dim %d not compiled (64 or 128)", D);
  return VC_OK;
}

vc_status check_draft_shape(const vc_draft_args *a) {
  REQ(a, "null argument struct");
  vc_status st = check_heads(a->B, a->Hq, a->Hkv, a->D);
  if (st != VC_OK) return st;
  REQ(a->dtype == VC_BF16 || a->dtype == VC_FP32, "unknown dtype %d", a->dtype);
  REQ(a->fmt == VC_KV_DENSE || a->fmt == VC_KV_INT4 || a->fmt == VC_KV_INT4_PACKED, "unknown kv format %d", a->fmt);
  const bool i4 = a->fmt != VC_KV_DENSE;
  if (i4 && a->dtype != VC_BF16) return fail(VC_ENOTSUP, "int4 main segment is compiled for bf16 queries only");
  if (i4 && a->D != 128) return fail(VC_ENOTSUP, "int4 main segment is compiled for head_dim 128");
  REQ(a->cap >= 0 && a->cap % 64 == 0, "cap (%lld) must be a non-negative multiple of 64", (long long)a->cap);
  REQ(a->tcap >= 0, "tcap must be non-negative");
  // token indices inside the kernels are 32-bit
  REQ(a->cap + a->tcap <= kMaxTokens, "cap + tcap (%lld) above 2^30 tokens", (long long)(a->cap + a->tcap));
  return VC_OK;
}

vc_status check_draft(const vc_draft_args *a) {
  vc_status st = check_draft_shape(a);
  if (st != VC_OK || a->B == 0) return st;
  REQ(a->q && a->out && a->main_len, "q, out and main_len are required");
  if (a->fmt == VC_KV_INT4_PACKED) {
    REQ(a->cap == 0 || a->k, "k (the packed int4 blocks) is required when cap > 0");
    REQ(!a->v && !a->k_scale && !a->k_zero && !a->v_scale && !a->v_zero,
        "a packed int4 main segment lives in k alone: v and the scale/zero pointers must be NULL");
  } else {
    REQ(a->cap == 0 || (a->k && a->v), "k and v are required when cap > 0");
  }
  REQ(aligned16(a->q) && aligned16(a->out) && aligned16(a->k) && aligned16(a->v),
      "q, k, v and out must be 16-byte aligned");
  if (a->fmt == VC_KV_INT4) {
    REQ(a->cap == 0 || (a->k_scale && a->k_zero && a->v_scale && a->v_zero),
        "int4 main segment needs k_scale, k_zero, v_scale and v_zero");
    REQ(aligned16(a->k_scale) && aligned16(a->k_zero) && aligned16(a->v_scale) && aligned16(a->v_zero),
        "int4 scales and zeros must be 16-byte aligned");
  }
  if (a->tail_len) {
    REQ(a->tcap > 0 && a->tail_k && a->tail_v, "tail_len given without tail_k/tail_v/tcap");
    REQ(aligned16(a->tail_k) && aligned16(a->tail_v), "tail_k and tail_v must be 16-byte aligned");
  }
  if (a->degree) {
    REQ(aligned16(a->degree), "degree must be 16-byte aligned");
    REQ(a->degree_h_stride == 0 || a->degree_h_stride == a->cap,
        "degree_h_stride must be 0 (shared) or cap (per KV head)");
  }
  REQ(a->scale > 0.f && a->scale == a->scale, "scale must be positive and finite");
  return VC_OK;
}

vc_status check_verify_shape(const vc_verify_args *a) {
  REQ(a, "null argument struct");
  vc_status st = check_heads(a->B, a->Hq, a->Hkv, a->D);
  if (st != VC_OK) return st;
  REQ(a->dtype == VC_BF16 || a->dtype == VC_FP32, "unknown dtype %d", a->dtype);
  REQ(a->M >= 1, "M must be >= 1");
  REQ(a->ccap >= 0 && a->ccap % 64 == 0, "ccap (%lld) must be a non-negative multiple of 64", (long long)a->ccap);
  REQ(a->ccap <= kMaxTokens, "ccap (%lld) above 2^30 tokens", (long long)a->ccap);
  // packed rows M*G index row groups of at least 64 on a grid dimension capped at 65535
  REQ((int64_t)a->M * (a->Hq / a->Hkv) <= 65535 * 64, "M * Hq/Hkv (%lld) above 65535 * 64",
      (long long)a->M * (a->Hq / a->Hkv));
  REQ((int64_t)a->B * a->M * a->Hq <= INT32_MAX, "B * M * Hq above 2^31 - 1");
  return VC_OK;
}

vc_status check_verify(const vc_verify_args *a) {
  vc_status st = check_verify_shape(a);
  if (st != VC_OK || a->B == 0) return st;
  REQ(a->q && a->out && a->ctx_len && a->blk_k && a->blk_v, "q, out, ctx_len, blk_k and blk_v are required");
  REQ(a->ccap == 0 || (a->ctx_k && a->ctx_v), "ctx_k and ctx_v are required when ccap > 0");
  REQ(aligned16(a->q) && aligned16(a->out) && aligned16(a->ctx_k) && aligned16(a->ctx_v) &&
          aligned16(a->blk_k) && aligned16(a->blk_v),
      "tensor pointers must be 16-byte aligned");
  REQ(a->scale > 0.f && a->scale == a->scale, "scale must be positive and finite");
  return VC_OK;
}

}  // namespace

namespace vc {
vc_status set_error(vc_status s, const char *msg) { return fail(s, "%s", msg); }

vc_status validate_draft_call(const vc_draft_args *a) {
  vc_status st = check_draft(a);
  if (st != VC_OK || a->B == 0) return st;
  const SplitPlan pl = plan_draft(*a);
  if (pl.ws_bytes) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes)
      return fail(VC_EINVAL, "workspace of %zu bytes required (got %zu)", pl.ws_bytes, a->workspace_bytes);
    if (!aligned16(a->workspace)) return fail(VC_EINVAL, "workspace must be 16-byte aligned");
  }
  return VC_OK;
}

vc_status validate_verify_call(const vc_verify_args *a) {
  vc_status st = check_verify(a);
  if (st != VC_OK || a->B == 0) return st;
  const SplitPlan pl = plan_verify(*a);
  if (pl.ws_bytes) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes)
      return fail(VC_EINVAL, "workspace of %zu bytes required (got %zu)", pl.ws_bytes, a->workspace_bytes);
    if (!aligned16(a->workspace)) return fail(VC_EINVAL, "workspace must be 16-byte aligned");
  }
  return VC_OK;
}
}  // namespace vc

extern "C" {

const char *vc_status_string(vc_status s) {
  switch (s) {
    case VC_OK: return "VC_OK";
    case VC_EINVAL: return "VC_EINVAL";
    case VC_ENOTSUP: return "VC_ENOTSUP";
    case VC_EHIP: return "VC_EHIP";
    default: break;
  }
  return "unknown vc_status";
}

const char *vc_last_error(void) { return g_err.c_str(); }

const char *vc_build_info(void) {
  return "libvc gfx950 (HIP " HIP_VERSION_GITHASH "), MFMA bf16 draft/verify, fp32 VALU draft/verify";
}

size_t vc_draft_workspace_size(const vc_draft_args *a) {
  if (check_draft_shape(a) != VC_OK) return 0;
  return vc::plan_draft(*a).ws_bytes;
}

size_t vc_verify_workspace_size(const vc_verify_args *a) {
  if (check_verify_shape(a) != VC_OK) return 0;
  return vc::plan_verify(*a).ws_bytes;
}

vc_status vc_draft_attn(const vc_draft_args *a, void *stream) {
  vc_status st = vc::validate_draft_call(a);
  if (st != VC_OK || a->B == 0) return st;
  return hip_status(vc::launch_draft(*a, vc::plan_draft(*a), (hipStream_t)stream), "vc_draft_attn launch");
}

vc_status vc_verify_attn(const vc_verify_args *a, void *stream) {
  vc_status st = vc::validate_verify_call(a);
  if (st != VC_OK || a->B == 0) return st;
  return hip_status(vc::launch_verify(*a, vc::plan_verify(*a), (hipStream_t)stream), "vc_verify_attn launch");
}

vc_status vc_accept(const vc_accept_args *a, void *stream) {
  if (!a) return fail(VC_EINVAL, "null argument struct");
  REQ(a->B >= 0 && a->M >= 1 && a->V >= 1, "B >= 0, M >= 1 and V >= 1 required");
  REQ(a->logit_dtype == VC_BF16 || a->logit_dtype == VC_FP32, "unknown logit dtype %d", a->logit_dtype);
  if (a->B == 0) return VC_OK;
  REQ(a->logits && a->argmax && a->accept_len && a->out_tokens && a->n_out, "null output or logits pointer");
  REQ(a->M == 1 || a->draft, "draft is required when M > 1");
  REQ(aligned16(a->logits), "logits must be 16-byte aligned");
  return hip_status(vc::launch_accept(*a, (hipStream_t)stream), "vc_accept launch");
}

vc_status vc_next_input(int32_t B, int32_t M, const int32_t *out_tokens, const int32_t *n_out, int32_t *dst,
                        int64_t dst_stride, void *stream) {
  REQ(B >= 0 && M >= 1 && dst_stride >= 1, "B >= 0, M >= 1 and dst_stride >= 1 required");
  if (B == 0) return VC_OK;
  REQ(out_tokens && n_out && dst, "null pointer");
  return hip_status(vc::launch_next_input(B, M, out_tokens, n_out, dst, dst_stride, (hipStream_t)stream),
                    "vc_next_input launch");
}

vc_status vc_argmax(int32_t R, int32_t V, int32_t logit_dtype, const void *logits, int32_t *out,
                    int32_t out_stride, void *stream) {
  REQ(R >= 0 && V >= 1 && out_stride >= 1, "R >= 0, V >= 1, out_stride >= 1 required");
  REQ(logit_dtype == VC_BF16 || logit_dtype == VC_FP32, "unknown logit dtype %d", logit_dtype);
  if (R == 0) return VC_OK;
  REQ(logits && out, "null logits or output");
  REQ(aligned16(logits), "logits must be 16-byte aligned");
  return hip_status(vc::launch_argmax(R, V, logit_dtype, logits, out, out_stride, (hipStream_t)stream),
                    "vc_argmax launch");
}

size_t vc_lm_head_argmax_workspace_size(int32_t R, int32_t V) {
  if (R <= 0 || V <= 0) return 0;
  return vc::lm_argmax_workspace(R, V);
}

}  // extern "C"

namespace vc {
vc_status check_lm_argmax(int32_t R, int32_t Dm, int32_t V, const void *h, const void *w, const void *out,
                          void *ws, size_t ws_bytes) {
  REQ(R >= 0 && V >= 1 && Dm >= 32, "R >= 0, V >= 1 and Dm >= 32 required");
  if (Dm % 32) return fail(VC_ENOTSUP, "Dm (%d) must be a multiple of 32", Dm);
  REQ(Dm <= (1 << 20), "Dm (%d) above 2^20", Dm);
  REQ(V <= (1 << 30), "V (%d) above 2^30", V);
  if (R == 0) return VC_OK;
  REQ(h && w && out && ws, "null h, w, output or workspace");
  REQ(aligned16(h) && aligned16(w) && aligned16(ws), "h, w and workspace must be 16-byte aligned");
  REQ(ws_bytes >= vc::lm_argmax_workspace(R, V), "workspace of %zu bytes is below the %zu required", ws_bytes,
      vc::lm_argmax_workspace(R, V));
  return VC_OK;
}
}  // namespace vc

extern "C" {

vc_status vc_lm_head_argmax(int32_t R, int32_t Dm, int32_t V, const void *h, const void *w, int32_t *out,
                            int32_t out_stride, void *workspace, size_t workspace_bytes, void *stream) {
  REQ(out_stride >= 1, "out_stride must be >= 1");
  vc_status st = vc::check_lm_argmax(R, Dm, V, h, w, out, workspace, workspace_bytes);
  if (st != VC_OK || R == 0) return st;
  return hip_status(vc::launch_lm_argmax(R, Dm, V, h, w, out, out_stride, workspace, (hipStream_t)stream),
                    "vc_lm_head_argmax launch");
}

vc_status vc_lm_head_accept(int32_t B, int32_t M, int32_t Dm, int32_t V, const void *h, const void *w,
                            const int32_t *draft, int32_t *argmax, int32_t *accept_len, int32_t *out_tokens,
                            int32_t *n_out, void *workspace, size_t workspace_bytes, void *stream) {
  REQ(B >= 0 && M >= 1, "B >= 0 and M >= 1 required");
  REQ((int64_t)B * M <= 0x7fffffff, "B * M overflows");
  vc_status st = vc::check_lm_argmax(B * M, Dm, V, h, w, argmax, workspace, workspace_bytes);
  if (st != VC_OK || B == 0) return st;
  REQ(accept_len && out_tokens && n_out, "null accept output");
  REQ(M == 1 || draft, "draft is required when M > 1");
  hipStream_t s = (hipStream_t)stream;
  st = hip_status(vc::launch_lm_argmax(B * M, Dm, V, h, w, argmax, 1, workspace, s), "vc_lm_head_accept launch");
  if (st != VC_OK) return st;
  return hip_status(vc::launch_accept_rows(B, M, draft, argmax, accept_len, out_tokens, n_out, s),
                    "vc_lm_head_accept launch");
}

}  // extern "C"

namespace vc {
vc_status check_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, int64_t cap, int32_t dst_v_blocked,
                       const void *blk_k, const void *blk_v, const int32_t *n_out, const void *dst_k,
                       const void *dst_v, const int32_t *len, const float *degree, int64_t degree_h_stride) {
  REQ(B >= 0 && Hkv >= 1 && D >= 1 && M >= 1 && cap >= 0, "bad commit shape");
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  REQ(dtype == VC_BF16 || dtype == VC_FP32, "unknown dtype %d", dtype);
  REQ(dst_v_blocked == 0 || dst_v_blocked == 1, "dst_v_blocked must be 0 or 1");
  REQ(!dst_v_blocked || cap % 32 == 0, "a blocked V cache needs cap %% 32 == 0");
  if (B == 0) return VC_OK;
  REQ(blk_k && blk_v && n_out && dst_k && dst_v && len, "null pointer");
  REQ(!degree || degree_h_stride == 0 || degree_h_stride == cap, "degree_h_stride must be 0 or cap");
  return VC_OK;
}
}  // namespace vc

extern "C" {

vc_status vc_commit_rows(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, int64_t cap,
                         int32_t dst_v_blocked, const void *blk_k, const void *blk_v, const int32_t *n_out,
                         void *dst_k, void *dst_v,
                         int32_t *len, float *degree, int64_t degree_h_stride, void *stream) {
  vc_status st = vc::check_commit(B, Hkv, D, M, dtype, cap, dst_v_blocked, blk_k, blk_v, n_out, dst_k, dst_v, len,
                                  degree, degree_h_stride);
  if (st != VC_OK || B == 0) return st;
  const int64_t deg_b = degree_h_stride ? degree_h_stride * Hkv : cap;
  return hip_status(vc::launch_commit(B, Hkv, D, M, dtype == VC_BF16 ? 2 : 4, cap, dst_v_blocked, blk_k, blk_v, n_out, dst_k,
                                      dst_v, len, degree, deg_b, degree_h_stride, (hipStream_t)stream),
                    "vc_commit_rows launch");
}

vc_status vc_compact_kv(int32_t B, int32_t Hkv, int32_t D, int32_t dtype, const void *src_k, const void *src_v,
                        int64_t src_cap, const int32_t *idx, int64_t idx_stride, const int32_t *n_kept,
                        void *dst_k, void *dst_v, int64_t cap, int32_t *dst_len, void *stream) {
  REQ(B >= 0 && Hkv >= 1 && src_cap >= 0 && cap >= 0 && idx_stride >= 0, "bad compaction shape");
  REQ(dtype == VC_BF16 || dtype == VC_FP32, "unknown dtype %d", dtype);
  if (D != 64 && D != 128) return fail(VC_ENOTSUP, "head_dim %d not compiled (64 or 128)", D);
  REQ(cap % 32 == 0, "cap (%lld) must be a multiple of 32", (long long)cap);
  REQ(cap <= kMaxTokens, "cap (%lld) above 2^30 tokens", (long long)cap);
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  if (B == 0 || cap == 0) return VC_OK;
  REQ(idx_stride >= 1, "idx_stride must be >= 1");
  REQ(src_k && src_v && idx && n_kept && dst_k && dst_v, "null pointer");
  REQ(aligned16(src_k) && aligned16(src_v) && aligned16(dst_k) && aligned16(dst_v),
      "K/V buffers must be 16-byte aligned");
  return hip_status(vc::launch_compact_kv(B, Hkv, D, dtype == VC_BF16 ? 2 : 4, src_k, src_v, src_cap, idx, idx_stride,
                                          n_kept, dst_k, dst_v, cap, dst_len, (hipStream_t)stream),
                    "vc_compact_kv launch");
}

vc_status vc_quantize_int4(int32_t B, int32_t Hkv, int32_t D, const void *src_k, const void *src_v,
                           int64_t src_cap, const int32_t *src_start, int32_t n_groups, int64_t cap,
                           const int32_t *dst_start, void *k_codes, void *k_scale, void *k_zero, void *v_codes,
                           void *v_scale, void *v_zero, void *stream) {
  REQ(B >= 0 && Hkv >= 1 && n_groups >= 0 && src_cap >= 0 && cap >= 0, "bad quantize shape");
  REQ(cap <= kMaxTokens && src_cap <= kMaxTokens, "cap or src_cap above 2^30 tokens");
  if (D != 128) return fail(VC_ENOTSUP, "the int4 cache is compiled for head_dim 128 (got %d)", D);
  REQ(cap % 32 == 0, "cap (%lld) must be a multiple of 32", (long long)cap);
  REQ(n_groups <= 65535, "at most 65535 groups per call (got %d)", n_groups);
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  if (B == 0 || n_groups == 0) return VC_OK;
  REQ(src_k && src_v && src_start && dst_start && k_codes && k_scale && k_zero && v_codes && v_scale && v_zero,
      "null pointer");
  REQ(aligned16(k_codes) && aligned16(v_codes) && aligned16(src_k) && aligned16(src_v),
      "source and int4 code buffers must be 16-byte aligned");
  REQ(aligned16(k_scale) && aligned16(k_zero) && aligned16(v_scale) && aligned16(v_zero),
      "int4 scale and zero buffers must be 16-byte aligned");
  vc::QuantParams p;
  p.code_bs = 32 * D / 2;   // 2048 bytes of codes per 32-token block
  p.par_bs = 2 * D;         // 256 bytes of binary16 per block
  p.BH = B * Hkv;
  p.src_cap = src_cap;
  p.cap = cap;
  p.src_k = static_cast<const uint16_t *>(src_k);
  p.src_v = static_cast<const uint16_t *>(src_v);
  p.src_start = src_start;
  p.dst_start = dst_start;
  p.k_codes = static_cast<uint8_t *>(k_codes);
  p.v_codes = static_cast<uint8_t *>(v_codes);
  p.k_scale = static_cast<uint16_t *>(k_scale);
  p.k_zero = static_cast<uint16_t *>(k_zero);
  p.v_scale = static_cast<uint16_t *>(v_scale);
  p.v_zero = static_cast<uint16_t *>(v_zero);
  return hip_status(vc::launch_quantize_int4(p, n_groups, (hipStream_t)stream), "vc_quantize_int4 launch");
}

vc_status vc_quantize_int4_packed(int32_t B, int32_t Hkv, int32_t D, const void *src_k, const void *src_v,
                                  int64_t src_cap, const int32_t *src_start, int32_t n_groups, int64_t cap,
                                  const int32_t *dst_start, void *packed, void *stream) {
  REQ(B >= 0 && Hkv >= 1 && n_groups >= 0 && src_cap >= 0 && cap >= 0, "bad quantize shape");
  REQ(cap <= kMaxTokens && src_cap <= kMaxTokens, "cap or src_cap above 2^30 tokens");
  if (D != 128) return fail(VC_ENOTSUP, "the int4 cache is compiled for head_dim 128 (got %d)", D);
  REQ(cap % 32 == 0, "cap (%lld) must be a multiple of 32", (long long)cap);
  REQ(n_groups <= 65535, "at most 65535 groups per call (got %d)", n_groups);
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  if (B == 0 || n_groups == 0) return VC_OK;
  REQ(src_k && src_v && src_start && dst_start && packed, "null pointer");
  REQ(aligned16(packed) && aligned16(src_k) && aligned16(src_v), "source and packed buffers must be 16-byte aligned");
  uint8_t *blk = static_cast<uint8_t *>(packed);
  vc::QuantParams p;
  p.BH = B * Hkv;
  p.src_cap = src_cap;
  p.cap = cap;
  p.src_k = static_cast<const uint16_t *>(src_k);
  p.src_v = static_cast<const uint16_t *>(src_v);
  p.src_start = src_start;
  p.dst_start = dst_start;
  p.k_codes = blk + vc::kPackedKCodes;
  p.v_codes = blk + vc::kPackedVCodes;
  p.k_scale = reinterpret_cast<uint16_t *>(blk + vc::kPackedKScale);
  p.k_zero = reinterpret_cast<uint16_t *>(blk + vc::kPackedKZero);
  p.v_scale = reinterpret_cast<uint16_t *>(blk + vc::kPackedVScale);
  p.v_zero = reinterpret_cast<uint16_t *>(blk + vc::kPackedVZero);
  p.code_bs = p.par_bs = vc::kPackedBlock;
  return hip_status(vc::launch_quantize_int4(p, n_groups, (hipStream_t)stream), "vc_quantize_int4_packed launch");
}

}  // extern "C"

namespace vc {
vc_status check_int4_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, const void *blk_k,
                            const void *blk_v, const int32_t *n_out, const void *tail_k, const void *tail_v,
                            int64_t tcap, const int32_t *tail_len, const void *packed, int64_t cap,
                            const int32_t *main_len) {
  REQ(B >= 0 && Hkv >= 1 && M >= 1 && cap >= 0 && tcap >= 32, "bad int4 commit shape (tcap >= 32, M >= 1)");
  if (D != 128 || dtype != VC_BF16) return fail(VC_ENOTSUP, "the int4 cache is compiled for bf16, head_dim 128");
  REQ(cap % 32 == 0 && cap <= kMaxTokens && tcap <= kMaxTokens, "cap must be a multiple of 32; caps <= 2^30");
  REQ(tcap / 32 <= 65535, "tcap above 65535 groups");
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  if (B == 0) return VC_OK;
  REQ(blk_k && blk_v && n_out && tail_k && tail_v && tail_len && packed && main_len, "null pointer");
  REQ(aligned16(blk_k) && aligned16(blk_v) && aligned16(tail_k) && aligned16(tail_v) && aligned16(packed),
      "K/V, tail and packed buffers must be 16-byte aligned");
  return VC_OK;
}
}  // namespace vc

extern "C" {

vc_status vc_int4_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, const void *blk_k, const void *blk_v,
                         const int32_t *n_out, void *tail_k, void *tail_v, int64_t tcap, int32_t *tail_len,
                         void *packed, int64_t cap, int32_t *main_len, void *stream) {
  vc_status st = vc::check_int4_commit(B, Hkv, D, M, VC_BF16, blk_k, blk_v, n_out, tail_k, tail_v, tcap, tail_len,
                                       packed, cap, main_len);
  if (st != VC_OK || B == 0) return st;
  return hip_status(vc::launch_int4_commit(B, Hkv, M, blk_k, blk_v, n_out, tail_k, tail_v, tcap, tail_len, packed,
                                           cap, main_len, (hipStream_t)stream),
                    "vc_int4_commit launch");
}

vc_status vc_csm_round(int32_t B, int32_t Hkv, int32_t D, int32_t n_in, int32_t n_sink, int32_t n_recent,
                       int32_t chunk, double r, const void *in_k, const void *in_v, const float *in_deg,
                       int64_t cap_in, void *out_k, void *out_v, float *out_deg, int64_t cap_out, int32_t *n_out,
                       int32_t *out_len, void *stream) {
  REQ(n_out, "null n_out");
  REQ(B >= 0 && Hkv >= 1 && n_in >= 0 && n_sink >= 0 && n_recent >= 0, "bad CSM shape");
  REQ((int64_t)B * Hkv <= 65535, "at most 65535 (request, KV head) slices per call");
  if (D != 128) return fail(VC_ENOTSUP, "the CSM round is compiled for head_dim 128 (got %d)", D);
  REQ(chunk >= 2 && chunk <= 128, "chunk must lie in 2..128 (got %d)", chunk);
  REQ(r >= 0.f && r <= 1.f, "r must lie in [0, 1]");
  REQ(n_in <= kMaxTokens, "n_in (%d) above 2^30 tokens", n_in);
  REQ((int64_t)n_sink + n_recent <= n_in, "sinks + recent tokens (%lld) exceed n_in (%d)",
      (long long)n_sink + n_recent, n_in);
  REQ(n_in <= cap_in && cap_in % 32 == 0 && cap_out % 32 == 0, "n_in <= cap_in; caps multiples of 32");
  // one 256-thread workgroup per chunk on the x dimension of the grid, whose work-item count is 32-bit
  REQ(((int64_t)n_in - n_sink - n_recent + chunk - 1) / chunk + 2 <= (1 << 24) - 1,
      "too many chunks: at most 2^24 - 3 per (request, KV head)");
  const int out = vc::csm_survivors(n_in, n_sink, n_recent, chunk, r);
  REQ(out <= cap_out, "the round keeps %d tokens; cap_out is %lld", out, (long long)cap_out);
  *n_out = out;
  if (B == 0) return VC_OK;
  REQ(in_k && in_v && out_k && out_v && out_deg, "null pointer");
  REQ(aligned16(in_k) && aligned16(out_k), "K buffers must be 16-byte aligned");
  vc::CsmParams p;
  p.n_in = n_in; p.n_sink = n_sink; p.n_recent = n_recent; p.chunk = chunk; p.n_out = out; p.r = r;
  p.cap_in = cap_in; p.cap_out = cap_out;
  p.in_k = static_cast<const uint16_t *>(in_k);
  p.in_v = static_cast<const uint16_t *>(in_v);
  p.in_deg = in_deg;
  p.out_k = static_cast<uint16_t *>(out_k);
  p.out_v = static_cast<uint16_t *>(out_v);
  p.out_deg = out_deg;
  p.out_len = out_len;
  return hip_status(vc::launch_csm_round(p, B * Hkv, (hipStream_t)stream), "vc_csm_round launch");
}

int32_t vc_csm_round_due(int64_t n_tokens, int64_t budget, int32_t decode_step, int32_t every) {
  if (every < 1 || decode_step < 0) return -1;
  if (decode_step > 0 && decode_step % every != 0) return 0;
  return n_tokens > budget ? 1 : 0;
}

double vc_csm_schedule_ratio(double r_init, double delta_r, int32_t round) {
  const double r = r_init - (double)round * delta_r;
  return r < 0.0 ? 0.0 : (r > 1.0 ? 1.0 : r);
}

}  // extern "C"
