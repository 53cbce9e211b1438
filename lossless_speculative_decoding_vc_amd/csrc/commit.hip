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

// Compaction for a token-eviction compressor: row j of the compacted cache is
// row idx[b][j] of the full cache, for every KV head of request b (the kept
// set is per token, shared by the heads).  One 256-thread workgroup per
// (32-row block, b, KV head): K rows are copied in 16-byte pieces, V is
// gathered channel by channel into the 32-token block [D][32] the drafter
// reads.  An index outside the source writes a zero row; rows at or past
// n_kept are left untouched.
namespace vc {
namespace {

template <typename T>
__global__ __launch_bounds__(256) void compact_kv(int Hkv, int D, int64_t src_cap, const T *__restrict__ src_k,
                                                  const T *__restrict__ src_v, const int32_t *__restrict__ idx,
                                                  int64_t idx_stride, const int32_t *__restrict__ n_kept,
                                                  T *__restrict__ dst_k, T *__restrict__ dst_v, int64_t cap,
                                                  int32_t *__restrict__ dst_len) {
  constexpr int kPer = 16 / sizeof(T);   // elements per 16-byte piece
  __shared__ int64_t rows[32];
  const int bh = blockIdx.y, b = bh / Hkv;
  const int j0 = blockIdx.x * 32;
  int n = n_kept[b];
  n = n < 0 ? 0 : (n > cap ? (int)cap : n);
  if (n > idx_stride) n = (int)idx_stride;   // never read past the request's index row
  if (blockIdx.x == 0 && threadIdx.x == 0 && dst_len) dst_len[bh] = n;
  if (j0 >= n) return;
  const int m = min(32, n - j0);
  if (threadIdx.x < 32) {
    const int t = threadIdx.x;
    int64_t r = -1;
    if (t < m) {
      const int64_t x = idx[(size_t)b * idx_stride + j0 + t];
      r = (x >= 0 && x < src_cap) ? x : -1;
    }
    rows[t] = r;
  }
  __syncthreads();
  const T *sk = src_k + (size_t)bh * src_cap * D;
  const T *sv = src_v + (size_t)bh * D * src_cap;
  T *dk = dst_k + ((size_t)bh * cap + j0) * D;
  T *dv = dst_v + ((size_t)bh * (cap / 32) + blockIdx.x) * D * 32;
  const int pieces = D / kPer;
  for (int e = threadIdx.x; e < m * pieces; e += blockDim.x) {
    const int t = e / pieces, c = e % pieces;
    u32x4 w = u32x4{0, 0, 0, 0};
    if (rows[t] >= 0) w = *reinterpret_cast<const u32x4 *>(sk + rows[t] * D + c * kPer);
    *reinterpret_cast<u32x4 *>(dk + (size_t)t * D + c * kPer) = w;
  }
  for (int e = threadIdx.x; e < D * 32; e += blockDim.x) {
    const int d = e / 32, t = e % 32;
    if (t < m) dv[e] = rows[t] >= 0 ? sv[(size_t)d * src_cap + rows[t]] : T(0);
  }
}

}  // namespace

hipError_t launch_compact_kv(int B, int Hkv, int D, int elem_bytes, const void *src_k, const void *src_v,
                             int64_t src_cap, const int32_t *idx, int64_t idx_stride, const int32_t *n_kept,
                             void *dst_k, void *dst_v, int64_t cap, int32_t *dst_len, hipStream_t s) {
  if (B == 0 || cap == 0) return hipSuccess;
  const dim3 grid((unsigned)(cap / 32), B * Hkv);
  if (elem_bytes == 2)
    compact_kv<uint16_t><<<grid, 256, 0, s>>>(Hkv, D, src_cap, (const uint16_t *)src_k, (const uint16_t *)src_v, idx,
                                              idx_stride, n_kept, (uint16_t *)dst_k, (uint16_t *)dst_v, cap, dst_len);
  else
    compact_kv<float><<<grid, 256, 0, s>>>(Hkv, D, src_cap, (const float *)src_k, (const float *)src_v, idx,
                                           idx_stride, n_kept, (float *)dst_k, (float *)dst_v, cap, dst_len);
  return hipGetLastError();
}

}  // namespace vc
