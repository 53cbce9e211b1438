// Log-sum-exp merge of split attention partials.
//
// A split covers a contiguous range of the key sequence and stores its
// softmax-normalised output o_s and its log-sum-exp lse_s (base 2).  The
// attention over the union of the ranges is
//   o = sum_s 2^(lse_s - L) o_s,   L = log2 sum_s 2^lse_s,
// the standard flash-decoding reduction.  One workgroup per output row with
// up to 16 waves: wave w takes the splits w, w + nw, ... eight at a time, and
// every lane its D/64 channels.  Each batch of eight issues all its loads at
// once (eight log-sum-exps and eight partial rows) and folds them into a
// running maximum and rescaled sums, so a merge of up to eight splits costs
// one round trip to memory; the waves' (max, sum, row) triples meet in LDS.
// Spreading one row over several waves keeps the loads of a many-split,
// few-row merge (one long request) in flight.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kMaxCombineWaves = 16;

template <int D, bool kBf16>
__global__ __launch_bounds__(kMaxCombineWaves * 64) void combine_splits(const float *__restrict__ part_o,
                                                                        const float *__restrict__ part_lse,
                                                                        int splits, int rows, void *__restrict__ out,
                                                                        float *__restrict__ out_lse) {
  constexpr int kPer = D / 64;
  __shared__ float red_o[kMaxCombineWaves][D];
  __shared__ float red_w[kMaxCombineWaves];
  __shared__ float red_m[kMaxCombineWaves];
  const int row = blockIdx.x;
  const int nw = blockDim.x >> 6;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;

  float m = kNegInf;   // running reference (base 2) of this wave's sums
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s0 = wave; s0 < splits; s0 += 8 * nw) {
    float l[8], v[8][kPer];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * nw;
      const bool ok = s < splits;
      const int sc = ok ? s : s0;
      l[u] = ok ? part_lse[(size_t)sc * rows + row] : kNegInf;
      const float *po = part_o + ((size_t)sc * rows + row) * D + lane * kPer;
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[u][e] = po[e];
    }
    float mb = m;
#pragma unroll
    for (int u = 0; u < 8; ++u) mb = fmaxf(mb, l[u]);
    const float mu = (mb == kNegInf) ? 0.f : mb;
    const float alpha = fast_exp2(m - mu);   // 0 while nothing was summed (m = -inf)
    wsum *= alpha;
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = fast_exp2(l[u] - mu);   // 0 for an empty split or past the end
      wsum += w;
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] += w * v[u][e];
    }
    m = mb;
  }
  if (nw == 1) {
    const float inv = 1.f / wsum;   // wsum == 0 only for an empty key set -> NaN output
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const float x = acc[e] * inv;
      if constexpr (kBf16) reinterpret_cast<uint16_t *>(out)[(size_t)row * D + lane * kPer + e] = f32_to_bf16(x);
      else reinterpret_cast<float *>(out)[(size_t)row * D + lane * kPer + e] = x;
    }
    if (out_lse && lane == 0) out_lse[row] = (wsum > 0.f) ? (m + fast_log2(wsum)) * kLn2 : kNegInf;
    return;
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) red_o[wave][lane * kPer + e] = acc[e];
  if (lane == 0) {
    red_w[wave] = wsum;
    red_m[wave] = m;
  }
  __syncthreads();
  if (wave != 0) return;
  float M = kNegInf;
  for (int w = 0; w < nw; ++w) M = fmaxf(M, red_m[w]);
  const float Mu = (M == kNegInf) ? 0.f : M;
  float tot = 0.f;
  float o[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) o[e] = 0.f;
  for (int w = 0; w < nw; ++w) {
    const float f = fast_exp2(red_m[w] - Mu);
    tot += f * red_w[w];
#pragma unroll
    for (int e = 0; e < kPer; ++e) o[e] += f * red_o[w][lane * kPer + e];
  }
  const float inv = 1.f / tot;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float x = o[e] * inv;
    if constexpr (kBf16) reinterpret_cast<uint16_t *>(out)[(size_t)row * D + lane * kPer + e] = f32_to_bf16(x);
    else reinterpret_cast<float *>(out)[(size_t)row * D + lane * kPer + e] = x;
  }
  if (out_lse && lane == 0) out_lse[row] = (tot > 0.f) ? (M + fast_log2(tot)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_combine(const float *part_o, const float *part_lse, int splits, int rows, int D,
                          int dtype, void *out, float *out_lse, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const bool bf = dtype == VC_BF16;
  // one wave per eight splits, at most kMaxCombineWaves
  int nw = (splits + 7) / 8;
  nw = nw < 1 ? 1 : (nw > kMaxCombineWaves ? kMaxCombineWaves : nw);
  const dim3 block(64 * nw);
  if (D == 128) {
    if (bf) combine_splits<128, true><<<rows, block, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
    else combine_splits<128, false><<<rows, block, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
  } else {
    if (bf) combine_splits<64, true><<<rows, block, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
    else combine_splits<64, false><<<rows, block, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
  }
  return hipGetLastError();
}

}  // namespace vc
