// fp32 attention for the small fp32 mode (draft and verify share it).
//
// One wave per (request, block row, query head).  The key sequence is two
// segments: A (compressed main segment, or the full-cache context) followed
// by B (draft tail, or the verify block keys 0..i).  Segment A may carry
// merge degrees whose logarithm is added to the score ("Riassunto Tecnico:
// CentroidKV", "Componenti Chiave", item 4).  Keys are processed 64 at a
// time: lane = key for the scores, lane = channel for the weighted sum, with
// an online (running-max) softmax in base 2.  Used for the tiny fp32 decoder,
// where every tensor is a few hundred KB; it is not a bandwidth kernel.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

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

__global__ __launch_bounds__(64) void attn_f32(F32Params p) {
  const int b = blockIdx.y;
  const int i = blockIdx.x / p.Hq;
  const int h = blockIdx.x % p.Hq;
  const int kvh = h / p.G;
  const int lane = threadIdx.x;
  const int D = p.D;
  __shared__ float qs[128];
  __shared__ float ps[64];
  const float *qrow = p.q + (((size_t)b * p.M + i) * p.Hq + h) * D;
  for (int d = lane; d < D; d += 64) qs[d] = qrow[d];
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

  float m_run = kNegInf, l_run = 0.f;
  float acc[2] = {0.f, 0.f};
  for (int t0 = 0; t0 < total; t0 += 64) {
    const int t = t0 + lane;
    float s = kNegInf;
    if (t < total) {
      const float *kr = (t < la) ? ak + (size_t)t * D : bk + (size_t)(t - la) * D;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
      s = dot * p.qk_scale;
      if (dg && t < la) s += fast_log2(dg[t]);
    }
    const float cmax = wave_max(s);
    const float m_new = fmaxf(m_run, cmax);
    const float alpha = fast_exp2(m_run - m_new);
    const float pr = (t < total) ? fast_exp2(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(pr);
    m_run = m_new;
    ps[lane] = pr;
    __syncthreads();
    const int n = min(64, total - t0);
    for (int e = 0; e < 2; ++e) {
      const int d = lane + 64 * e;
      if (d >= D) break;
      float a2 = acc[e] * alpha;
      for (int j = 0; j < n; ++j) {
        const int tt = t0 + j;
        const float v = (tt < la) ? av[p.av_blocked ? (size_t)(tt >> 5) * D * 32 + d * 32 + (tt & 31)
                                                   : (size_t)d * p.acap + tt]
                                  : bv[(size_t)d * p.bcap + (tt - la)];
        a2 = fmaf(ps[j], v, a2);
      }
      acc[e] = a2;
    }
    __syncthreads();
  }
  float *orow = p.out + (((size_t)b * p.M + i) * p.Hq + h) * D;
  for (int e = 0; e < 2; ++e) {
    const int d = lane + 64 * e;
    if (d < D) orow[d] = acc[e] / l_run;
  }
  if (p.out_lse && lane == 0)
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
  attn_f32<<<dim3(a.Hq, a.B), 64, 0, s>>>(p);
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
  attn_f32<<<dim3(a.M * a.Hq, a.B), 64, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vc
