// Greedy argmax over the vocabulary and accept-until-first-mismatch.
//
// "Riepilogo Tecnico: VeriCache", section "Algoritmo Principale", step 3:
// drafted tokens are accepted up to the first disagreement with the
// full-cache prediction; a full match also accepts the prediction after the
// last draft (the bonus token).  The prediction emitted after the accepted
// prefix is the full-cache argmax, so every round emits n + 1 tokens.
//
// Kernel 1 (argmax_rows): one 256-thread workgroup per logit row; 16-byte
// loads, per-thread running best, then a wave shuffle reduction and a
// 4-wave LDS reduction.  Ties go to the lowest index.  The pass reads each
// logit once, so it is HBM-bound.
// Kernel 2 (accept_rows): one wave per request; a ballot over
// "draft != prediction" finds the first mismatch.
#include "common.h"
#include "launch.h"

namespace vc {

namespace {

constexpr int kArgmaxThreads = 256;

VC_DEVICE void better(float &bv, int &bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

template <typename T, bool kVec>
__global__ __launch_bounds__(kArgmaxThreads) void argmax_rows(const T *__restrict__ logits,
                                                              int V, int *__restrict__ out,
                                                              int out_stride) {
  const int row = blockIdx.x;
  const T *p = logits + (size_t)row * V;
  float bv = kNegInf;
  int bi = 0x7fffffff;
  const int tid = threadIdx.x;
  if constexpr (kVec) {
    // 16 bytes per load: 8 bf16 or 4 fp32 logits.
    constexpr int kPer = 16 / sizeof(T);
    const int nvec = V / kPer;
    const u32x4 *pv = reinterpret_cast<const u32x4 *>(p);
    for (int j = tid; j < nvec; j += kArgmaxThreads) {
      const u32x4 w = pv[j];
      const int base = j * kPer;
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          better(bv, bi, bf16_lo(w[e]), base + 2 * e);
          better(bv, bi, bf16_hi(w[e]), base + 2 * e + 1);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) better(bv, bi, u32_as_f32(w[e]), base + e);
      }
    }
  } else {
    for (int j = tid; j < V; j += kArgmaxThreads) {
      float v;
      if constexpr (sizeof(T) == 2) v = bf16_to_f32(reinterpret_cast<const uint16_t *>(p)[j]);
      else v = reinterpret_cast<const float *>(p)[j];
      better(bv, bi, v, j);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(bv, o, 64);
    int oi = __shfl_xor(bi, o, 64);
    better(bv, bi, ov, oi);
  }
  __shared__ float sv[kArgmaxThreads / 64];
  __shared__ int si[kArgmaxThreads / 64];
  const int wave = tid >> 6, lane = tid & 63;
  if (lane == 0) { sv[wave] = bv; si[wave] = bi; }
  __syncthreads();
  if (tid == 0) {
    for (int w = 1; w < kArgmaxThreads / 64; ++w) better(bv, bi, sv[w], si[w]);
    out[(size_t)row * out_stride] = (bi < V) ? bi : 0;
  }
}

__global__ __launch_bounds__(64) void accept_rows(const int *__restrict__ draft,
                                                  const int *__restrict__ am, int M,
                                                  int *__restrict__ accept_len,
                                                  int *__restrict__ out_tokens,
                                                  int *__restrict__ n_out) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int k = M - 1;
  const int *d = draft + (size_t)b * k;
  const int *y = am + (size_t)b * M;
  int n = k;
  for (int base = 0; base < k; base += 64) {
    const int j = base + lane;
    const bool miss = (j < k) && (d[j] != y[j]);
    const unsigned long long mask = __ballot(miss);
    if (mask) { n = base + __builtin_ctzll(mask); break; }
  }
  int *o = out_tokens + (size_t)b * M;
  for (int j = lane; j < M; j += 64) o[j] = (j < n) ? d[j] : (j == n ? y[n] : -1);
  if (lane == 0) { accept_len[b] = n; n_out[b] = n + 1; }
}

__global__ __launch_bounds__(64) void next_input(int B, int M, const int *__restrict__ out_tokens,
                                                 const int *__restrict__ n_out, int *__restrict__ dst,
                                                 int64_t dst_stride) {
  const int b = blockIdx.x * 64 + threadIdx.x;
  if (b >= B) return;
  int n = n_out[b];
  n = n < 1 ? 1 : (n > M ? M : n);
  dst[b * dst_stride] = out_tokens[(size_t)b * M + n - 1];
}

}  // namespace

hipError_t launch_next_input(int B, int M, const int32_t *out_tokens, const int32_t *n_out, int32_t *dst,
                             int64_t dst_stride, hipStream_t s) {
  next_input<<<(B + 63) / 64, 64, 0, s>>>(B, M, out_tokens, n_out, dst, dst_stride);
  return hipGetLastError();
}

hipError_t launch_argmax(int rows, int V, int dtype, const void *logits, int *out, int out_stride,
                         hipStream_t s) {
  if (rows == 0) return hipSuccess;
  if (dtype == VC_BF16) {
    if (V % 8 == 0)
      argmax_rows<uint16_t, true><<<rows, kArgmaxThreads, 0, s>>>((const uint16_t *)logits, V, out, out_stride);
    else
      argmax_rows<uint16_t, false><<<rows, kArgmaxThreads, 0, s>>>((const uint16_t *)logits, V, out, out_stride);
  } else {
    if (V % 4 == 0)
      argmax_rows<float, true><<<rows, kArgmaxThreads, 0, s>>>((const float *)logits, V, out, out_stride);
    else
      argmax_rows<float, false><<<rows, kArgmaxThreads, 0, s>>>((const float *)logits, V, out, out_stride);
  }
  return hipGetLastError();
}

hipError_t launch_accept(const vc_accept_args &a, hipStream_t s) {
  hipError_t e = launch_argmax(a.B * a.M, a.V, a.logit_dtype, a.logits, a.argmax, 1, s);
  if (e != hipSuccess) return e;
  return launch_accept_rows(a.B, a.M, a.draft, a.argmax, a.accept_len, a.out_tokens, a.n_out, s);
}

hipError_t launch_accept_rows(int B, int M, const int32_t *draft, const int32_t *argmax, int32_t *accept_len,
                              int32_t *out_tokens, int32_t *n_out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  accept_rows<<<B, 64, 0, s>>>(draft, argmax, M, accept_len, out_tokens, n_out);
  return hipGetLastError();
}

}  // namespace vc
