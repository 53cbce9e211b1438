// Kernel launchers (internal).  Arguments were validated by api.cpp.
#pragma once

#include <hip/hip_runtime.h>

#include "../../include/vc.h"

#define VC_DEVICE_HOST_INLINE __host__ __device__ inline

namespace vc {

// Launch plan of a split attention call: `splits` partial results per
// (row, head) are merged by the combine kernel when splits > 1.
struct SplitPlan {
  int splits;
  size_t ws_bytes;
};

SplitPlan plan_draft(const vc_draft_args &a);
SplitPlan plan_verify(const vc_verify_args &a);

// Host-side validation of one call, as the entry point does it before any
// launch (used by the round scheduler to check a whole round up front).
vc_status validate_draft_call(const vc_draft_args *a);
vc_status validate_verify_call(const vc_verify_args *a);
vc_status check_lm_argmax(int32_t R, int32_t Dm, int32_t V, const void *h, const void *w, const void *out,
                          void *ws, size_t ws_bytes);
vc_status check_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, int64_t cap, int32_t dst_v_blocked,
                       const void *blk_k, const void *blk_v, const int32_t *n_out, const void *dst_k,
                       const void *dst_v, const int32_t *len, const float *degree, int64_t degree_h_stride);
vc_status check_int4_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, const void *blk_k,
                            const void *blk_v, const int32_t *n_out, const void *tail_k, const void *tail_v,
                            int64_t tcap, const int32_t *tail_len, const void *packed, int64_t cap,
                            const int32_t *main_len);
vc_status set_error(vc_status s, const char *msg);

hipError_t launch_accept(const vc_accept_args &a, hipStream_t s);
hipError_t launch_argmax(int rows, int V, int dtype, const void *logits, int *out, int out_stride,
                         hipStream_t s);
// Acceptance over precomputed argmax rows (argmax [B][M], draft [B][M-1]).
hipError_t launch_next_input(int B, int M, const int32_t *out_tokens, const int32_t *n_out, int32_t *dst,
                             int64_t dst_stride, hipStream_t s);
hipError_t launch_accept_rows(int B, int M, const int32_t *draft, const int32_t *argmax, int32_t *accept_len,
                              int32_t *out_tokens, int32_t *n_out, hipStream_t s);
// LM head fused with the argmax (see lmhead_argmax.hip).
size_t lm_argmax_workspace(int R, int V);
hipError_t launch_lm_argmax(int R, int Dm, int V, const void *h, const void *w, int *out, int out_stride,
                            void *ws, hipStream_t s);
hipError_t launch_commit(int B, int Hkv, int D, int M, int elem_bytes, int64_t cap, int v_blocked, const void *blk_k,
                         const void *blk_v, const int32_t *n_out, void *dst_k, void *dst_v, int32_t *len,
                         float *degree, int64_t deg_b_stride, int64_t deg_h_stride, hipStream_t s);
hipError_t launch_compact_kv(int B, int Hkv, int D, int elem_bytes, const void *src_k, const void *src_v,
                             int64_t src_cap, const int32_t *idx, int64_t idx_stride, const int32_t *n_kept,
                             void *dst_k, void *dst_v, int64_t cap, int32_t *dst_len, hipStream_t s);
// after_kernel (optional): an event recorded once the attention kernel is
// enqueued and before the split merge, so a caller can time the kernel alone.
hipError_t launch_draft(const vc_draft_args &a, const SplitPlan &p, hipStream_t s, hipEvent_t after_kernel = nullptr);
hipError_t launch_verify(const vc_verify_args &a, const SplitPlan &p, hipStream_t s, hipEvent_t after_kernel = nullptr);

// The interleaved int4 block (fmt = VC_KV_INT4_PACKED, head_dim 128): byte
// offsets of a 32-token block's six pieces and the block size.
constexpr int kPackedKCodes = 0, kPackedVCodes = 2048, kPackedKScale = 4096, kPackedKZero = 4352,
              kPackedVScale = 4608, kPackedVZero = 4864, kPackedBlock = 5120;

// Int4 group quantization (see quant.hip): BH = B * Hkv slices.  Block j of
// slice bh of a piece starts at base + (bh * cap/32 + j) * stride bytes.
struct QuantParams {
  int BH;
  int64_t src_cap, cap;
  const uint16_t *src_k, *src_v;
  const int32_t *src_start, *dst_start;
  uint8_t *k_codes, *v_codes;
  uint16_t *k_scale, *k_zero, *v_scale, *v_zero;
  int code_bs, par_bs;   // bytes per block: codes, scales/zeros
  // tail mode (vc_int4_commit): when tail_len is set, slice bh quantizes the
  // full groups of its bf16 tail after the append of n_add[b] rows, from
  // token 0 of the tail to dst_start[bh]; the grid's group count is a bound
  const int32_t *tail_len = nullptr, *n_add = nullptr;
  int Hkv = 1, M = 0;
};

// Rows of a request's bf16 tail after appending n_out of a block of M rows:
// the length clamped to [0, tcap], then at most M rows, at most up to tcap.
VC_DEVICE_HOST_INLINE int tail_total(int tail_len, int n_out, int M, int64_t tcap) {
  const int L = tail_len < 0 ? 0 : (tail_len > tcap ? (int)tcap : tail_len);
  int n = n_out < 0 ? 0 : (n_out > M ? M : n_out);
  if (n > tcap - L) n = (int)(tcap - L);
  return L + n;
}
hipError_t launch_int4_commit(int B, int Hkv, int M, const void *blk_k, const void *blk_v, const int32_t *n_out,
                              void *tail_k, void *tail_v, int64_t tcap, int32_t *tail_len, void *packed,
                              int64_t cap, int32_t *main_len, hipStream_t s);
hipError_t launch_quantize_int4(const QuantParams &p, int n_groups, hipStream_t s);

// One Chunked Soft Matching round (see csm.hip).
struct CsmParams {
  int n_in, n_sink, n_recent, chunk, n_out;
  double r;   // merge count floor(r * |A|) is taken in double, as the caller wrote r
  int64_t cap_in, cap_out;
  const uint16_t *in_k, *in_v;
  const float *in_deg;
  uint16_t *out_k, *out_v;
  float *out_deg;
  int32_t *out_len;   // optional [BH]: set to n_out (the drafter's main_len)
};
int csm_survivors(int n_in, int n_sink, int n_recent, int chunk, double r);
hipError_t launch_csm_round(const CsmParams &p, int BH, hipStream_t s);

// Merge `splits` partials (o normalised per split, lse in log2 units) of
// `rows` (row, head) pairs into out (bf16 or fp32) and optional lse (ln).
hipError_t launch_combine(const float *part_o, const float *part_lse, int splits, int rows, int D,
                          int dtype, void *out, float *out_lse, hipStream_t s);

}  // namespace vc
