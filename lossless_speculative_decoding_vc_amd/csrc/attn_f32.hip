// fp32 attention for the small fp32 mode (draft and verify share it).
//
// One 1024-thread workgroup per (request, block row, query head).  The key
// sequence is two segments: A (compressed main segment, or the full-cache
// context) followed by B (draft tail, or the verify block keys 0..i).
// Segment A may carry merge degrees whose logarithm is added to the score
// ("Riassunto Tecnico: CentroidKV", "Componenti Chiave", item 4).  Keys are
// processed 1024 at a time: thread = key for the scores (its key row read with
// 16-byte loads), a running maximum and sum shared by the workgroup (online
// softmax in base 2), then each wave accumulates the weighted values of its
// 64 keys with lane = channel, 32 value loads in flight together; the 16
// waves' sums are added in wave order at the end.  Used for the tiny fp32
// decoder, whose caches hold a few thousand tokens: the workgroup size only
// shortens the chain of dependent loads (one chunk covers most contexts).
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kAT = 1024;   // threads per workgroup = keys per chunk

struct F32Params {
  int Hq, Hkv, G, M, D;
  float qk_scale;
  const float *q;                    // [B][M][Hq][D]
  const float *ak, *av;              // segment A: K [acap][D] per (b, kvh); V [D][acap] (verify
  int64_t acap;                      // context) or [acap/32][D][32] (draft main segment)
  int av_blocked;
  const int32_t *alen;               // per (b, kvh) if alen_per_head else per b
  int alen_per_head;
  const float *deg;                  // optional, per token of segment A
  int64_t deg_b_stride, deg_h_stride;
  const float *bk, *bv;              // segment B: K [bcap][D], V [D][bcap] per (b, kvh)
  int64_t bcap;
  const int32_t *blen;               // per b (draft tail); NULL -> causal block (i + 1)
  int causal;
  float *out;                        // [B][M][Hq][D]
  float *out_lse;                    // [B][M][Hq]
};

__global__ __launch_bounds__(kAT) void attn_f32(F32Params p) {
  const int b = blockIdx.y;
  const int i = blockIdx.x / p.Hq;
  const int h = blockIdx.x % p.Hq;
  const int kvh = h / p.G;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int D = p.D;
  __shared__ __attribute__((aligned(16))) float qs[128];
  __shared__ float ps[kAT];
  __shared__ float red_m[kAT / 64], red_s[kAT / 64];
  __shared__ float acc_w[kAT / 64][128];
  const float *qrow = p.q + (((size_t)b * p.M + i) * p.Hq + h) * D;
  if (tid < D) qs[tid] = qrow[tid];
  __syncthreads();

  int la = p.alen[p.alen_per_head ? b * p.Hkv + kvh : b];
  la = la < 0 ? 0 : (la > p.acap ? (int)p.acap : la);
  int lb = 0;
  if (p.bk) {
    lb = p.causal ? i + 1 : (p.blen ? p.blen[b] : 0);
    lb = lb < 0 ? 0 : (lb > p.bcap ? (int)p.bcap : lb);
  }
  const int total = la + lb;
  const size_t bh = (size_t)b * p.Hkv + kvh;
  const float *ak = p.ak + bh * p.acap * D, *av = p.av + bh * D * p.acap;
  const float *bk = p.bk ? p.bk + bh * p.bcap * D : nullptr;
  const float *bv = p.bv ? p.bv + bh * D * p.bcap : nullptr;
  const float *dg = p.deg ? p.deg + b * p.deg_b_stride + kvh * p.deg_h_stride : nullptr;
  const f32x4 *q4 = reinterpret_cast<const f32x4 *>(qs);

  float m_run = kNegInf, l_run = 0.f;
  float acc[2] = {0.f, 0.f};
  for (int t0 = 0; t0 < total; t0 += kAT) {
    const int t = t0 + tid;
    float s = kNegInf;
    if (t < total) {
      const f32x4 *kr = reinterpret_cast<const f32x4 *>((t < la) ? ak + (size_t)t * D : bk + (size_t)(t - la) * D);
      float dot = 0.f;
      for (int d4 = 0; d4 < D / 4; ++d4) {
        const f32x4 kv = kr[d4], qv = q4[d4];
        dot = fmaf(qv[0], kv[0], dot);
        dot = fmaf(qv[1], kv[1], dot);
        dot = fmaf(qv[2], kv[2], dot);
        dot = fmaf(qv[3], kv[3], dot);
      }
      s = dot * p.qk_scale;
      if (dg && t < la) s += fast_log2(dg[t]);
    }
    const float wm = wave_max(s);
    if (lane == 0) red_m[wv] = wm;
    __syncthreads();
    float cmax = red_m[0];
    for (int ww = 1; ww < kAT / 64; ++ww) cmax = fmaxf(cmax, red_m[ww]);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    const float pr = (t < total) ? fast_exp2(s - m_new) : 0.f;
    const float ws = wave_sum(pr);
    if (lane == 0) red_s[wv] = ws;
    ps[tid] = pr;
    __syncthreads();
    float csum = red_s[0];
    for (int ww = 1; ww < kAT / 64; ++ww) csum += red_s[ww];
    l_run = l_run * alpha + csum;
    m_run = m_new;
    const int j0 = t0 + wv * 64;
    const int n = min(64, total - j0);   // this wave's keys (may be <= 0)
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d >= D) break;
      float a2 = acc[e] * alpha;
#pragma unroll 1
      for (int jh = 0; jh < n; jh += 32) {
        float v[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const int tt = j0 + jh + j;
          v[j] = jh + j >= n ? 0.f
                             : (tt < la) ? av[p.av_blocked ? (size_t)(tt >> 5) * D * 32 + d * 32 + (tt & 31)
                                                           : (size_t)d * p.acap + tt]
                                         : bv[(size_t)d * p.bcap + (tt - la)];
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) a2 = fmaf(ps[wv * 64 + jh + j], v[j], a2);
      }
      acc[e] = a2;
    }
    __syncthreads();
  }
  for (int e = 0; e < 2; ++e) {
    const int d = lane + 64 * e;
    if (d < D) acc_w[wv][d] = acc[e];
  }
  __syncthreads();
  float *orow = p.out + (((size_t)b * p.M + i) * p.Hq + h) * D;
  if (tid < D) {
    float o = acc_w[0][tid];
    for (int ww = 1; ww < kAT / 64; ++ww) o += acc_w[ww][tid];
    orow[tid] = o / l_run;
  }
  if (p.out_lse && tid == 0)
    p.out_lse[((size_t)b * p.M + i) * p.Hq + h] = (l_run > 0.f) ? (m_run + fast_log2(l_run)) * kLn2 : kNegInf;
}

}  // namespace

hipError_t launch_draft_f32(const vc_draft_args &a, hipStream_t s) {
  F32Params p{};
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv; p.M = 1; p.D = a.D;
  p.qk_scale = a.scale * kLog2e;
  p.q = (const float *)a.q;
  p.ak = (const float *)a.k; p.av = (const float *)a.v; p.acap = a.cap; p.av_blocked = 1;
  p.alen = a.main_len; p.alen_per_head = 1;
  p.deg = a.degree;
  p.deg_h_stride = a.degree_h_stride;
  p.deg_b_stride = a.degree_h_stride ? a.degree_h_stride * a.Hkv : a.cap;
  p.bk = (const float *)a.tail_k; p.bv = (const float *)a.tail_v; p.bcap = a.tcap;
  p.blen = a.tail_len; p.causal = 0;
  if (!a.tail_len) p.bk = p.bv = nullptr;
  p.out = (float *)a.out; p.out_lse = a.out_lse;
  attn_f32<<<dim3(a.Hq, a.B), kAT, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_verify_f32(const vc_verify_args &a, hipStream_t s) {
  F32Params p{};
  p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv; p.M = a.M; p.D = a.D;
  p.qk_scale = a.scale * kLog2e;
  p.q = (const float *)a.q;
  p.ak = (const float *)a.ctx_k; p.av = (const float *)a.ctx_v; p.acap = a.ccap;
  p.alen = a.ctx_len; p.alen_per_head = 0;
  p.bk = (const float *)a.blk_k; p.bv = (const float *)a.blk_v; p.bcap = a.M;
  p.blen = nullptr; p.causal = 1;
  p.out = (float *)a.out; p.out_lse = a.out_lse;
  attn_f32<<<dim3(a.M * a.Hq, a.B), kAT, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vc
