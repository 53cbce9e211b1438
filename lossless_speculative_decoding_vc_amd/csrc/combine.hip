// Log-sum-exp merge of split attention partials.
//
// A split covers a contiguous range of the key sequence and stores its
// softmax-normalised output o_s and its log-sum-exp lse_s (base 2).  The
// attention over the union of the ranges is
//   o = sum_s 2^(lse_s - L) o_s,   L = log2 sum_s 2^lse_s,
// the standard flash-decoding reduction.  One workgroup per output row with
// up to 16 waves: wave w takes the splits w, w + nw, ... eight at a time (all
// eight partial rows in flight), every lane its D/64 channels, and the waves'
// sums meet in LDS.  Spreading one row over several waves keeps the loads of
// a many-split, few-row merge (one long request) in flight instead of
// walking the splits one batch after another.
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

  // reference: the largest split lse of the row
  float mx = kNegInf;
  for (int s = threadIdx.x; s < splits; s += blockDim.x) mx = fmaxf(mx, part_lse[(size_t)s * rows + row]);
  mx = wave_max(mx);
  if (lane == 0) red_m[wave] = mx;
  __syncthreads();
  mx = red_m[0];
  for (int w = 1; w < nw; ++w) mx = fmaxf(mx, red_m[w]);
  const float mu = (mx == kNegInf) ? 0.f : mx;

  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s0 = wave; s0 < splits; s0 += 8 * nw) {
    float w[8], v[8][kPer];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int s = s0 + u * nw;
      const bool ok = s < splits;
      const int sc = ok ? s : s0;
      w[u] = ok ? fast_exp2(part_lse[(size_t)sc * rows + row] - mu) : 0.f;
      const float *po = part_o + ((size_t)sc * rows + row) * D + lane * kPer;
#pragma unroll
      for (int e = 0; e < kPer; ++e) v[u][e] = ok ? po[e] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      wsum += w[u];
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] += w[u] * v[u][e];
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) red_o[wave][lane * kPer + e] = acc[e];
  if (lane == 0) red_w[wave] = wsum;
  __syncthreads();
  if (wave != 0) return;
  for (int w = 1; w < nw; ++w) {
#pragma unroll
    for (int e = 0; e < kPer; ++e) acc[e] += red_o[w][lane * kPer + e];
    wsum += red_w[w];
  }
  const float inv = 1.f / wsum;   // wsum == 0 only for an empty key set -> NaN output
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const float v = acc[e] * inv;
    if constexpr (kBf16) reinterpret_cast<uint16_t *>(out)[(size_t)row * D + lane * kPer + e] = f32_to_bf16(v);
    else reinterpret_cast<float *>(out)[(size_t)row * D + lane * kPer + e] = v;
  }
  if (out_lse && lane == 0) out_lse[row] = (wsum > 0.f) ? (mx + fast_log2(wsum)) * kLn2 : kNegInf;
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
