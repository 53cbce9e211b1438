// Draft decode attention over the compressed cache (bf16, MFMA).
//
// "Riepilogo Tecnico: VeriCache", "Algoritmo Principale", step 1: the target
// model drafts over KV_comp; "Innovazioni Chiave del Sistema" (P1): drafting
// is bound by HBM bandwidth.  The compressed main segment may carry merge
// degrees n_t whose logarithm is added to the softmax score ("Riassunto
// Tecnico: CentroidKV", "Componenti Chiave", item 4 "Aggregazione").
//
// Design (gfx950):
//  * grid (splits, B*Hkv); 4 waves per workgroup; every wave serves ALL
//    G = Hq/Hkv query heads of its KV head, so each K/V byte is read from
//    HBM exactly once per call.
//  * a wave walks 32-token chunks, the next chunk's loads in flight while
//    the current one is computed.  Both contractions run on
//    v_mfma_f32_16x16x32_bf16 with operands loaded straight from HBM into
//    registers (no LDS): S^T = K Q^T (A = 16 token rows of K, 16 bytes per
//    lane; B = Q^T, one column per query head) and O^T = V^T P^T (A = 16
//    channel rows of the channel-major V, 16 bytes = 8 consecutive tokens
//    per lane; B = the probabilities, already in the lanes that produced
//    them).  Token rows of the S^T tiles are permuted so that each lane's
//    four score registers of the two S^T tiles are 8 consecutive
//    tokens -- exactly the k-slots the PV MFMA needs; no data moves between
//    lanes except two max-shuffles per chunk.
//  * online softmax in base 2 (scores pre-multiplied by log2 e; the degree
//    term becomes log2 n_t), one running max per query head.
//  * the 4 waves merge through LDS; with more than one split the workgroup
//    writes a normalised partial and its log-sum-exp for the combine kernel.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kDraftWaves = 4;
constexpr int kChunk = 32;   // tokens per wave step

struct DraftParams {
  int B, Hq, Hkv, G, splits;
  float qk_scale;   // scale * log2(e)
  int64_t cap, tcap;
  const uint16_t *q;
  const int32_t *main_len;
  const uint16_t *k, *v;
  const float *degree;
  int64_t deg_b_stride, deg_h_stride;
  const uint16_t *tail_k, *tail_v;
  const int32_t *tail_len;
  uint16_t *out;
  float *out_lse;
  float *part_o, *part_lse;
};

VC_DEVICE u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Registers of one 32-token chunk: K A-operands of the two S^T tiles, V^T
// A-operands of the PV k-step, log2 degrees of the lane's 8 tokens.
template <int D>
struct DraftChunk {
  u32x4 ka[2][D / 32];
  u32x4 va[D / 16];
  float lg[8];
};

template <int D>
__global__ __launch_bounds__(kDraftWaves * 64) void draft_bf16_dense(DraftParams p) {
  constexpr int KS = D / 32;   // k-steps of the QK contraction
  constexpr int DT = D / 16;   // 16-channel output tiles
  const int bh = blockIdx.y;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int split = blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.G;

  int mlen = p.main_len[bh];
  mlen = mlen < 0 ? 0 : (mlen > p.cap ? (int)p.cap : mlen);
  int tlen = 0;
  if (p.tail_len && p.tail_k) {
    tlen = p.tail_len[b];
    tlen = tlen < 0 ? 0 : (tlen > p.tcap ? (int)p.tcap : tlen);
  }
  const int total = mlen + tlen;
  const int nchunks = (total + kChunk - 1) / kChunk;
  const int cps = (nchunks + p.splits - 1) / p.splits;
  const int c0 = split * cps;
  const int c1 = min(c0 + cps, nchunks);

  bf16x8 qb[KS];
  if (col < G) {
    const uint16_t *qp = p.q + ((size_t)b * p.Hq + kvh * G + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(ld16(qp + 32 * ks + 8 * grp));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
  }

  const uint16_t *kb = p.k + (size_t)bh * p.cap * D;
  const uint16_t *vb = p.v + (size_t)bh * D * p.cap;
  const uint16_t *tkb = p.tail_k ? p.tail_k + (size_t)bh * p.tcap * D : nullptr;
  const uint16_t *tvb = p.tail_v ? p.tail_v + (size_t)bh * D * p.tcap : nullptr;
  const float *db = p.degree ? p.degree + b * p.deg_b_stride + kvh * p.deg_h_stride : nullptr;

  // S^T tile tau, row m (= lane col) holds token base + 8*(m>>2) + 4*tau + (m&3),
  // so the lane's 4+4 score registers are tokens base + 8*grp + 0..7.
  auto fetch = [&](int c, DraftChunk<D> &ch) __attribute__((always_inline)) {
    const int base = c * kChunk;
    if (base + kChunk <= mlen) {
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int t = base + 8 * (col >> 2) + 4 * tau + (col & 3);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ch.ka[tau][ks] = ld16(kb + (size_t)t * D + 32 * ks + 8 * grp);
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) ch.va[dt] = ld16(vb + (size_t)(16 * dt + col) * p.cap + base + 8 * grp);
      if (db) {
        const f32x4 *dp = reinterpret_cast<const f32x4 *>(db + base + 8 * grp);
        const f32x4 d0 = dp[0], d1 = dp[1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ch.lg[e] = fast_log2(d0[e]);
          ch.lg[4 + e] = fast_log2(d1[e]);
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ch.lg[e] = 0.f;
      }
    } else {
      // Chunk crossing the end of the main segment: per-row source select
      // for K, per-element select for V (tail tokens, zero past the end).
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
        const int t = base + 8 * (col >> 2) + 4 * tau + (col & 3);
        const uint16_t *row = nullptr;
        if (t < mlen) row = kb + (size_t)t * D;
        else if (t < total) row = tkb + (size_t)(t - mlen) * D;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) ch.ka[tau][ks] = row ? ld16(row + 32 * ks + 8 * grp) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + col;
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          uint32_t h[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int t = base + 8 * grp + 2 * e2 + u;
            uint16_t x = 0;
            if (t < mlen) x = vb[(size_t)d * p.cap + t];
            else if (t < total) x = tvb[(size_t)d * p.tcap + (t - mlen)];
            h[u] = x;
          }
          w[e2] = h[0] | (h[1] << 16);
        }
        ch.va[dt] = u32x4{w[0], w[1], w[2], w[3]};
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = base + 8 * grp + e;
        ch.lg[e] = (db && t < mlen) ? fast_log2(db[t]) : 0.f;
      }
    }
  };

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int c, const DraftChunk<D> &ch) __attribute__((always_inline)) {
    const int base = c * kChunk;
    f32x4 s[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      s[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[tau] = mfma16x16x32(as_bf16x8(ch.ka[tau][ks]), qb[ks], s[tau]);
    }
    float sc[8];
    float cmax = kNegInf;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * tau + i;
        float x = s[tau][i] * p.qk_scale + ch.lg[e];
        x = (base + 8 * grp + e < total) ? x : kNegInf;
        sc[e] = x;
        cmax = fmaxf(cmax, x);
      }
    cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
    const float m_new = fmaxf(m_run, cmax);
    const float m_use = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(sc[e] - m_use);
      psum += pr[e];
    }
    l_run = l_run * alpha + psum;
    if (__any(m_new != m_run)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
    }
    m_run = m_new;
    const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = mfma16x16x32(as_bf16x8(ch.va[dt]), pb, o[dt]);
  };

  // Software pipeline: the next chunk's loads are in flight while the
  // current one is computed (unrolled by two so the buffers stay static).
  DraftChunk<D> ca, cb;
  int c = c0 + wave;
  if (c < c1) fetch(c, ca);
  for (; c < c1; c += 2 * kDraftWaves) {
    const int cn = c + kDraftWaves;
    if (cn < c1) fetch(cn, cb);
    compute(c, ca);
    if (cn >= c1) break;
    if (cn + kDraftWaves < c1) fetch(cn + kDraftWaves, ca);
    compute(cn, cb);
  }

  // Merge the lane groups' partial sums, then the 4 waves through LDS.
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __shared__ float sm[kDraftWaves][16], sl[kDraftWaves][16];
  __shared__ float so[kDraftWaves][D][17];
  if (grp == 0) { sm[wave][col] = m_run; sl[wave][col] = l_run; }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) so[wave][16 * dt + 4 * grp + i][col] = o[dt][i];
  __syncthreads();

  const int rows = p.B * p.Hq;
  for (int idx = threadIdx.x; idx < G * D; idx += kDraftWaves * 64) {
    const int g = idx / D, d = idx % D;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < kDraftWaves; ++w) M = fmaxf(M, sm[w][g]);
    const float Mu = (M == kNegInf) ? 0.f : M;
    float L = 0.f, acc = 0.f;
#pragma unroll
    for (int w = 0; w < kDraftWaves; ++w) {
      const float f = fast_exp2(sm[w][g] - Mu);
      L += f * sl[w][g];
      acc += f * so[w][d][g];
    }
    const int row = b * p.Hq + kvh * G + g;
    if (p.splits == 1) {
      p.out[(size_t)row * D + d] = f32_to_bf16(acc / L);
      if (p.out_lse && d == 0) p.out_lse[row] = (L > 0.f) ? (M + fast_log2(L)) * kLn2 : kNegInf;
    } else {
      p.part_o[((size_t)split * rows + row) * D + d] = (L > 0.f) ? acc / L : 0.f;
      if (d == 0) p.part_lse[(size_t)split * rows + row] = (L > 0.f) ? M + fast_log2(L) : kNegInf;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// Split plan: enough workgroups to cover the 256 CUs a few times over, while
// keeping every split at >= 8 chunks so the partials stay small next to the
// K/V bytes.
SplitPlan plan_draft(const vc_draft_args &a) {
  SplitPlan p{1, 0};
  if (a.dtype == VC_FP32) return p;   // fp32 mode runs unsplit
  const int64_t pairs = (int64_t)a.B * a.Hkv;
  const int64_t chunks = (a.cap + a.tcap + kChunk - 1) / kChunk;
  int s = a.num_splits;
  if (s <= 0) {
    s = 1;
    while (pairs * s < 1024 && chunks / (s * 2) >= 16) s *= 2;
  }
  if (s > chunks && chunks > 0) s = (int)chunks;
  if (s < 1) s = 1;
  p.splits = s;
  if (s > 1) p.ws_bytes = (size_t)s * a.B * a.Hq * (a.D + 1) * sizeof(float);
  return p;
}

hipError_t launch_draft_f32(const vc_draft_args &a, hipStream_t s);

hipError_t launch_draft(const vc_draft_args &a, const SplitPlan &pl, hipStream_t s) {
  if (a.dtype == VC_FP32) return launch_draft_f32(a, s);
  DraftParams p;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv; p.splits = pl.splits;
  p.qk_scale = a.scale * kLog2e;
  p.cap = a.cap; p.tcap = a.tcap;
  p.q = (const uint16_t *)a.q; p.main_len = a.main_len;
  p.k = (const uint16_t *)a.k; p.v = (const uint16_t *)a.v;
  p.degree = a.degree;
  p.deg_h_stride = a.degree_h_stride;
  p.deg_b_stride = a.degree_h_stride ? a.degree_h_stride * a.Hkv : a.cap;
  p.tail_k = (const uint16_t *)a.tail_k; p.tail_v = (const uint16_t *)a.tail_v;
  p.tail_len = a.tail_len;
  p.out = (uint16_t *)a.out; p.out_lse = a.out_lse;
  const size_t rows = (size_t)a.B * a.Hq;
  p.part_o = (float *)a.workspace;
  p.part_lse = p.part_o ? p.part_o + (size_t)pl.splits * rows * a.D : nullptr;
  dim3 grid(pl.splits, a.B * a.Hkv);
  if (a.fmt == VC_KV_INT4) return hipErrorInvalidValue;   // separate kernel
  if (a.D == 128) draft_bf16_dense<128><<<grid, kDraftWaves * 64, 0, s>>>(p);
  else draft_bf16_dense<64><<<grid, kDraftWaves * 64, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_combine(p.part_o, p.part_lse, pl.splits, (int)rows, a.D, a.dtype, a.out, a.out_lse, s);
}

}  // namespace vc
