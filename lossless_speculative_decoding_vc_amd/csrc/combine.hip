// Log-sum-exp merge of split attention partials.
//
// A split covers a contiguous range of the key sequence and stores its
// softmax-normalised output o_s and its log-sum-exp lse_s (base 2).  The
// attention over the union of the ranges is
//   o = sum_s 2^(lse_s - L) o_s,   L = log2 sum_s 2^lse_s,
// the standard flash-decoding reduction.  One wave per (row, head): the
// lanes first read all split weights in one coalesced pass, then every lane
// accumulates its D/64 channels over the splits with the weight broadcast
// from the lane that read it (8 splits in flight).
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

template <int D, bool kBf16>
__global__ __launch_bounds__(64) void combine_splits(const float *__restrict__ part_o,
                                                     const float *__restrict__ part_lse,
                                                     int splits, int rows, void *__restrict__ out,
                                                     float *__restrict__ out_lse) {
  constexpr int kPer = D / 64;
  const int row = blockIdx.x;
  const int lane = threadIdx.x;
  float mx = kNegInf;
  for (int s = lane; s < splits; s += 64) mx = fmaxf(mx, part_lse[(size_t)s * rows + row]);
  mx = wave_max(mx);
  const float mu = (mx == kNegInf) ? 0.f : mx;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  for (int s0 = 0; s0 < splits; s0 += 64) {
    const int sl = s0 + lane;
    const float w_mine = (sl < splits) ? fast_exp2(part_lse[(size_t)sl * rows + row] - mu) : 0.f;
    wsum += w_mine;
    const int n = min(64, splits - s0);
    for (int j0 = 0; j0 < n; j0 += 8) {
      float w[8], v[8][kPer];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j0 + u;
        w[u] = __shfl(w_mine, j < n ? j : 0, 64);
        const float *po = part_o + ((size_t)(s0 + (j < n ? j : 0)) * rows + row) * D + lane * kPer;
#pragma unroll
        for (int e = 0; e < kPer; ++e) v[u][e] = (j < n) ? po[e] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
#pragma unroll
        for (int e = 0; e < kPer; ++e) acc[e] += w[u] * v[u][e];
    }
  }
  wsum = wave_sum(wsum);
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
  if (D == 128) {
    if (bf) combine_splits<128, true><<<rows, 64, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
    else combine_splits<128, false><<<rows, 64, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
  } else {
    if (bf) combine_splits<64, true><<<rows, 64, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
    else combine_splits<64, false><<<rows, 64, 0, s>>>(part_o, part_lse, splits, rows, out, out_lse);
  }
  return hipGetLastError();
}

}  // namespace vc
