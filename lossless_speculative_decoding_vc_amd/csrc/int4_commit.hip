// Commit of verified rows into an int4 compressed cache through its bf16
// tail (vc_int4_commit).
//
// "Riepilogo Tecnico: VeriCache", "Algoritmo Principale", step 3: the
// verified rows of the accepted prefix join the caches; "Supporto
// Architetturale": the drafter's cache may be a quantized one.  Int4 groups
// span 32 tokens, so verified rows wait in a short bf16 tail (which the
// drafter reads after the int4 segment) until a whole group is there:
//   1. tail_append: the block's first n_out[b] rows go to the tail after its
//      tail_len[b] rows (one workgroup per (request, KV head));
//   2. quantize_int4 in tail mode: every full 32-token group of the tail is
//      quantized into the packed cache at main_len (one workgroup per group);
//   3. tail_finish: per request, main_len advances by the groups written, the
//      remaining rows (fewer than 32) move to the front of the tail and
//      tail_len becomes their count.
// Every kernel derives the tail's row count with tail_total(), so they agree
// without a host round trip.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kD = 128, kGroup = 32;

__global__ __launch_bounds__(256) void tail_append(int Hkv, int M, int64_t tcap, const uint16_t *__restrict__ blk_k,
                                                   const uint16_t *__restrict__ blk_v,
                                                   const int32_t *__restrict__ n_out, uint16_t *__restrict__ tail_k,
                                                   uint16_t *__restrict__ tail_v,
                                                   const int32_t *__restrict__ tail_len) {
  const int bh = blockIdx.x, b = bh / Hkv;
  const int L0 = tail_total(tail_len[b], 0, M, tcap);
  const int n = tail_total(tail_len[b], n_out[b], M, tcap) - L0;
  const uint16_t *sk = blk_k + (size_t)bh * M * kD;
  const uint16_t *sv = blk_v + (size_t)bh * kD * M;
  uint16_t *dk = tail_k + ((size_t)bh * tcap + L0) * kD;
  uint16_t *dv = tail_v + (size_t)bh * kD * tcap + L0;
  for (int e = threadIdx.x; e < n * kD; e += blockDim.x) dk[e] = sk[e];
  for (int e = threadIdx.x; e < n * kD; e += blockDim.x) {
    const int d = e / n, r = e % n;
    dv[(size_t)d * tcap + r] = sv[(size_t)d * M + r];
  }
}

__global__ __launch_bounds__(256) void tail_finish(int Hkv, int M, int64_t tcap, int64_t cap,
                                                   const int32_t *__restrict__ n_out, uint16_t *__restrict__ tail_k,
                                                   uint16_t *__restrict__ tail_v, int32_t *__restrict__ tail_len,
                                                   int32_t *__restrict__ main_len) {
  const int b = blockIdx.x;
  const int tot = tail_total(tail_len[b], n_out[b], M, tcap);
  const int g = tot / kGroup, rem = tot - kGroup * g;
  __syncthreads();   // every thread has read tail_len[b] before it changes
  for (int h = 0; h < Hkv; ++h) {
    const int bh = b * Hkv + h;
    const int d0 = main_len[bh];
    // the quantizer wrote the groups only where the cache had room for all of them
    const bool wrote = d0 >= 0 && d0 % kGroup == 0 && (int64_t)d0 + (int64_t)kGroup * g <= cap;
    if (g > 0) {
      // rows [32 g, tot) to [0, rem): disjoint ranges, since rem < 32 <= 32 g
      uint16_t *tk = tail_k + (size_t)bh * tcap * kD;
      uint16_t *tv = tail_v + (size_t)bh * kD * tcap;
      for (int e = threadIdx.x; e < rem * kD; e += blockDim.x) tk[e] = tk[(size_t)kGroup * g * kD + e];
      for (int e = threadIdx.x; e < rem * kD; e += blockDim.x) {
        const int d = e / rem, r = e % rem;
        tv[(size_t)d * tcap + r] = tv[(size_t)d * tcap + kGroup * g + r];
      }
    }
    __syncthreads();
    if (threadIdx.x == 0 && wrote) main_len[bh] = d0 + kGroup * g;
  }
  if (threadIdx.x == 0) tail_len[b] = rem;
}

}  // namespace

hipError_t launch_int4_commit(int B, int Hkv, int M, const void *blk_k, const void *blk_v, const int32_t *n_out,
                              void *tail_k, void *tail_v, int64_t tcap, int32_t *tail_len, void *packed,
                              int64_t cap, int32_t *main_len, hipStream_t s) {
  if (B == 0) return hipSuccess;
  tail_append<<<B * Hkv, 256, 0, s>>>(Hkv, M, tcap, (const uint16_t *)blk_k, (const uint16_t *)blk_v, n_out,
                                      (uint16_t *)tail_k, (uint16_t *)tail_v, tail_len);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint8_t *blk = static_cast<uint8_t *>(packed);
  QuantParams p;
  p.BH = B * Hkv;
  p.src_cap = tcap;
  p.cap = cap;
  p.src_k = static_cast<const uint16_t *>(tail_k);
  p.src_v = static_cast<const uint16_t *>(tail_v);
  p.src_start = main_len;   // unused in tail mode (the source starts at the tail's first row)
  p.dst_start = main_len;
  p.k_codes = blk + kPackedKCodes;
  p.v_codes = blk + kPackedVCodes;
  p.k_scale = reinterpret_cast<uint16_t *>(blk + kPackedKScale);
  p.k_zero = reinterpret_cast<uint16_t *>(blk + kPackedKZero);
  p.v_scale = reinterpret_cast<uint16_t *>(blk + kPackedVScale);
  p.v_zero = reinterpret_cast<uint16_t *>(blk + kPackedVZero);
  p.code_bs = p.par_bs = kPackedBlock;
  p.tail_len = tail_len;
  p.n_add = n_out;
  p.Hkv = Hkv;
  p.M = M;
  e = launch_quantize_int4(p, (int)(tcap / kGroup), s);   // at most tcap / 32 full groups
  if (e != hipSuccess) return e;
  tail_finish<<<B, 256, 0, s>>>(Hkv, M, tcap, cap, n_out, (uint16_t *)tail_k, (uint16_t *)tail_v, tail_len, main_len);
  return hipGetLastError();
}

}  // namespace vc
