// Commit of verified rows into a cache (after acceptance).
//
// "Riepilogo Tecnico: VeriCache", "Algoritmo Principale", step 3: decoding
// restarts from the last accepted token, so the verified K/V rows of the
// accepted block prefix (x0, d_1..d_n: n_out = n + 1 rows) join the cache.
// One workgroup per (request, KV head): it reads the current length, copies
// the rows (K token-major; V channel-major for a full cache, or in 32-token
// blocks for a compressed main segment) and advances the length.  Rows
// beyond the capacity are dropped.  Reads n_out from device memory, so no
// host synchronisation sits between acceptance and commit.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void commit_rows(int Hkv, int D, int M, int64_t cap, int v_blocked,
                                                   const T *__restrict__ blk_k, const T *__restrict__ blk_v,
                                                   const int32_t *__restrict__ n_out, T *__restrict__ dst_k,
                                                   T *__restrict__ dst_v, int32_t *__restrict__ len,
                                                   float *__restrict__ degree, int64_t deg_b_stride,
                                                   int64_t deg_h_stride) {
  const int bh = blockIdx.x;
  const int b = bh / Hkv, h = bh % Hkv;
  int L = len[bh];
  L = L < 0 ? 0 : (L > cap ? (int)cap : L);
  int n = n_out[b];
  n = n < 0 ? 0 : (n > M ? M : n);
  if (n > cap - L) n = (int)(cap - L);
  const T *sk = blk_k + (size_t)bh * M * D;
  const T *sv = blk_v + (size_t)bh * D * M;
  T *dk = dst_k + ((size_t)bh * cap + L) * D;
  T *dv = dst_v + (size_t)bh * D * cap;
  for (int e = threadIdx.x; e < n * D; e += blockDim.x) dk[e] = sk[e];
  for (int e = threadIdx.x; e < n * D; e += blockDim.x) {
    const int d = e / n, r = e % n, t = L + r;
    const size_t at = v_blocked ? (size_t)(t >> 5) * D * 32 + d * 32 + (t & 31) : (size_t)d * cap + t;
    dv[at] = sv[(size_t)d * M + r];
  }
  if (degree) {
    float *dg = degree + b * deg_b_stride + h * deg_h_stride + L;
    for (int r = threadIdx.x; r < n; r += blockDim.x) dg[r] = 1.0f;
  }
  __syncthreads();
  if (threadIdx.x == 0) len[bh] = L + n;
}

}  // namespace

hipError_t launch_commit(int B, int Hkv, int D, int M, int elem_bytes, int64_t cap, int v_blocked, const void *blk_k,
                         const void *blk_v, const int32_t *n_out, void *dst_k, void *dst_v, int32_t *len,
                         float *degree, int64_t deg_b_stride, int64_t deg_h_stride, hipStream_t s) {
  if (B == 0) return hipSuccess;
  if (elem_bytes == 2)
    commit_rows<uint16_t><<<B * Hkv, 256, 0, s>>>(Hkv, D, M, cap, v_blocked, (const uint16_t *)blk_k, (const uint16_t *)blk_v,
                                                  n_out, (uint16_t *)dst_k, (uint16_t *)dst_v, len, degree,
                                                  deg_b_stride, deg_h_stride);
  else
    commit_rows<float><<<B * Hkv, 256, 0, s>>>(Hkv, D, M, cap, v_blocked, (const float *)blk_k, (const float *)blk_v, n_out,
                                               (float *)dst_k, (float *)dst_v, len, degree, deg_b_stride,
                                               deg_h_stride);
  return hipGetLastError();
}

}  // namespace vc
