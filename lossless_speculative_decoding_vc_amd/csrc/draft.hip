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
constexpr float kSlack = 8.f;  // lazy-rescale threshold (base 2)

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
  // int4 main segment
  const uint8_t *kq, *vq;                    // codes
  const uint16_t *ks, *kz, *vs, *vz;         // binary16 scales / zeros
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
        float x = fmaf(s[tau][i], p.qk_scale, ch.lg[e]);
        x = (base + 8 * grp + e < total) ? x : kNegInf;
        sc[e] = x;
        cmax = fmaxf(cmax, x);
      }
    // Lazy reference max: the lane groups exchange maxima (two cross-lane
    // shuffles) and rescale only when some score in the wave exceeds the
    // reference by more than kSlack; probabilities stay <= 2^kSlack.
    if (__any(cmax - m_run > kSlack)) {   // false when both are -inf
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(sc[e] - m_use);
      psum += pr[e];
    }
    l_run += psum;
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

// ---------------------------------------------------------------------------
// Int4 main segment ("Supporto Architetturale": quantizing drafters plug into
// the same interface).  Same MFMA pipeline as the dense kernel; each lane
// dequantises its own operands in registers right before the MFMAs:
//  * K: the lane's S^T row is a token; its 16-byte code load covers channels
//    32*grp .. 32*grp+31 (k-step ks takes 8*ks..8*ks+7 of them), with the
//    chunk's per-channel scales/zeros (the chunk is exactly one 32-token
//    group);
//  * V: the lane's row is a channel; its 4-byte code load covers the 8 tokens
//    of its k-slots, with their per-token scales/zeros of the channel's
//    32-channel group.
// x = code * scale + zero in fp32, rounded to bf16 for the MFMA.
VC_DEVICE void unpack8(uint32_t w, float *out) {
  // byte i of w holds element 2i (low nibble) and 2i+1 (high nibble)
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  // (float)(byte k) compiles to v_cvt_f32_ubyte<k>
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    out[2 * k] = (float)((lo >> (8 * k)) & 0xffu);
    out[2 * k + 1] = (float)((hi >> (8 * k)) & 0xffu);
  }
}
VC_DEVICE void f16x8(const u32x4 &w, float *out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t u = w[i];
    out[2 * i] = f16_to_f32((uint16_t)(u & 0xffffu));
    out[2 * i + 1] = f16_to_f32((uint16_t)(u >> 16));
  }
}

template <int D>
struct Int4Raw {
  u32x4 kc[2];          // K codes of the two S^T tiles (32 channels each)
  u32x4 ks[4], kz[4];   // K scales / zeros of channels 32*grp .. +31
  uint32_t vc[D / 16];  // V codes: 8 tokens of channel 16*dt + col
  u32x4 vs[D / 32], vz[D / 32];   // V scales / zeros of the lane's 8 tokens per channel group
  float lg[8];
};

template <int D>
__global__ __launch_bounds__(kDraftWaves * 64) void draft_bf16_int4(DraftParams p) {
  constexpr int KS = D / 32, DT = D / 16, NG = D / 32;
  static_assert(D == 128, "int4 draft is compiled for head_dim 128");
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

  // Q^T operand, channel order d = 32*grp + 8*ks + e (the K code layout).
  bf16x8 qb[KS];
  if (col < G) {
    const uint16_t *qp = p.q + ((size_t)b * p.Hq + kvh * G + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(ld16(qp + 32 * grp + 8 * ks));
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qb[ks] = as_bf16x8(u32x4{0, 0, 0, 0});
  }

  const uint8_t *kqb = p.kq + (size_t)bh * p.cap * (D / 2);
  const uint8_t *vqb = p.vq + (size_t)bh * D * (p.cap / 2);
  const uint16_t *ksb = p.ks + (size_t)bh * (p.cap / 32) * D;
  const uint16_t *kzb = p.kz + (size_t)bh * (p.cap / 32) * D;
  const uint16_t *vsb = p.vs + (size_t)bh * NG * p.cap;
  const uint16_t *vzb = p.vz + (size_t)bh * NG * p.cap;
  const uint16_t *tkb = p.tail_k ? p.tail_k + (size_t)bh * p.tcap * D : nullptr;
  const uint16_t *tvb = p.tail_v ? p.tail_v + (size_t)bh * D * p.tcap : nullptr;
  const float *db = p.degree ? p.degree + b * p.deg_b_stride + kvh * p.deg_h_stride : nullptr;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto fetch = [&](int c, Int4Raw<D> &r) __attribute__((always_inline)) {
    const int base = c * kChunk;
    const int g32 = base / 32;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = base + 8 * (col >> 2) + 4 * tau + (col & 3);
      r.kc[tau] = *reinterpret_cast<const u32x4 *>(kqb + (size_t)t * (D / 2) + 16 * grp);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r.ks[i] = ld16(ksb + (size_t)g32 * D + 32 * grp + 8 * i);
      r.kz[i] = ld16(kzb + (size_t)g32 * D + 32 * grp + 8 * i);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      r.vc[dt] = *reinterpret_cast<const uint32_t *>(vqb + (size_t)(16 * dt + col) * (p.cap / 2) + (base + 8 * grp) / 2);
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      r.vs[j] = ld16(vsb + (size_t)j * p.cap + base + 8 * grp);
      r.vz[j] = ld16(vzb + (size_t)j * p.cap + base + 8 * grp);
    }
    if (db) {
      const f32x4 *dp = reinterpret_cast<const f32x4 *>(db + base + 8 * grp);
      const f32x4 d0 = dp[0], d1 = dp[1];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        r.lg[e] = fast_log2(d0[e]);
        r.lg[4 + e] = fast_log2(d1[e]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) r.lg[e] = 0.f;
    }
  };

  // Dequantise into MFMA operands (main chunk) -- full chunks only.
  auto decode = [&](const Int4Raw<D> &r, u32x4 (&ka)[2][KS], u32x4 (&va)[DT]) __attribute__((always_inline)) {
    float sf[32], zf[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f16x8(r.ks[i], sf + 8 * i);
      f16x8(r.kz[i], zf + 8 * i);
    }
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        float cv[8];
        unpack8(r.kc[tau][ks], cv);
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2)
          w[e2] = pack_bf16x2(fmaf(cv[2 * e2], sf[8 * ks + 2 * e2], zf[8 * ks + 2 * e2]),
                              fmaf(cv[2 * e2 + 1], sf[8 * ks + 2 * e2 + 1], zf[8 * ks + 2 * e2 + 1]));
        ka[tau][ks] = u32x4{w[0], w[1], w[2], w[3]};
      }
    float vsf[NG][8], vzf[NG][8];
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      f16x8(r.vs[j], vsf[j]);
      f16x8(r.vz[j], vzf[j]);
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int j = dt >> 1;
      float cv[8];
      unpack8(r.vc[dt], cv);
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2)
        w[e2] = pack_bf16x2(fmaf(cv[2 * e2], vsf[j][2 * e2], vzf[j][2 * e2]),
                            fmaf(cv[2 * e2 + 1], vsf[j][2 * e2 + 1], vzf[j][2 * e2 + 1]));
      va[dt] = u32x4{w[0], w[1], w[2], w[3]};
    }
  };

  // Chunk that reaches the tail or the end: element-wise, from the int4 main
  // segment, the bf16 tail, or zero.
  auto slow_ops = [&](int c, u32x4 (&ka)[2][KS], u32x4 (&va)[DT], float (&lg)[8]) __attribute__((always_inline)) {
    const int base = c * kChunk;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = base + 8 * (col >> 2) + 4 * tau + (col & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint32_t w[4];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          float x[2];
#pragma unroll
          for (int u = 0; u < 2; ++u) {
            const int d = 32 * grp + 8 * ks + 2 * e2 + u;
            float v = 0.f;
            if (t < mlen) {
              const uint8_t byte = kqb[(size_t)t * (D / 2) + d / 2];
              const float code = (float)((d & 1) ? (byte >> 4) : (byte & 15));
              v = fmaf(code, f16_to_f32(ksb[(size_t)(t / 32) * D + d]), f16_to_f32(kzb[(size_t)(t / 32) * D + d]));
            } else if (t < total) {
              v = bf16_to_f32(tkb[(size_t)(t - mlen) * D + d]);
            }
            x[u] = v;
          }
          w[e2] = pack_bf16x2(x[0], x[1]);
        }
        ka[tau][ks] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + col, j = d / 32;
      uint32_t w[4];
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        float x[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int t = base + 8 * grp + 2 * e2 + u;
          float v = 0.f;
          if (t < mlen) {
            const uint8_t byte = vqb[(size_t)d * (p.cap / 2) + t / 2];
            const float code = (float)((t & 1) ? (byte >> 4) : (byte & 15));
            v = fmaf(code, f16_to_f32(vsb[(size_t)j * p.cap + t]), f16_to_f32(vzb[(size_t)j * p.cap + t]));
          } else if (t < total) {
            v = bf16_to_f32(tvb[(size_t)d * p.tcap + (t - mlen)]);
          }
          x[u] = v;
        }
        w[e2] = pack_bf16x2(x[0], x[1]);
      }
      va[dt] = u32x4{w[0], w[1], w[2], w[3]};
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int t = base + 8 * grp + e;
      lg[e] = (db && t < mlen) ? fast_log2(db[t]) : 0.f;
    }
  };

  auto compute = [&](int c, const u32x4 (&ka)[2][KS], const u32x4 (&va)[DT], const float (&lg)[8])
      __attribute__((always_inline)) {
    const int base = c * kChunk;
    f32x4 s[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      s[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[tau] = mfma16x16x32(as_bf16x8(ka[tau][ks]), qb[ks], s[tau]);
    }
    float sc[8];
    float cmax = kNegInf;
#pragma unroll
    for (int tau = 0; tau < 2; ++tau)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * tau + i;
        float x = fmaf(s[tau][i], p.qk_scale, lg[e]);
        x = (base + 8 * grp + e < total) ? x : kNegInf;
        sc[e] = x;
        cmax = fmaxf(cmax, x);
      }
    // Lazy reference max: the lane groups exchange maxima (two cross-lane
    // shuffles) and rescale only when some score in the wave exceeds the
    // reference by more than kSlack; probabilities stay <= 2^kSlack.
    if (__any(cmax - m_run > kSlack)) {   // false when both are -inf
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
      m_run = m_new;
    }
    const float m_use = (m_run == kNegInf) ? 0.f : m_run;
    float pr[8];
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pr[e] = fast_exp2(sc[e] - m_use);
      psum += pr[e];
    }
    l_run += psum;
    const bf16x8 pb = as_bf16x8(u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                                      pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = mfma16x16x32(as_bf16x8(va[dt]), pb, o[dt]);
  };

  // Pipeline: raw loads of the next chunk in flight while the current
  // chunk's dequantised operands go through the MFMAs.
  Int4Raw<D> raw;
  u32x4 ka[2][KS], va[DT];
  float lg[8];
  int c = c0 + wave;
  auto prepare = [&](int cc) __attribute__((always_inline)) {
    if (cc * kChunk + kChunk <= mlen) {
      decode(raw, ka, va);
#pragma unroll
      for (int e = 0; e < 8; ++e) lg[e] = raw.lg[e];
    } else {
      slow_ops(cc, ka, va, lg);
    }
  };
  if (c < c1) {
    if (c * kChunk + kChunk <= mlen) fetch(c, raw);
    prepare(c);
  }
  for (; c < c1; c += kDraftWaves) {
    const int cn = c + kDraftWaves;
    const bool have_next = cn < c1;
    if (have_next && cn * kChunk + kChunk <= mlen) fetch(cn, raw);
    compute(c, ka, va, lg);
    if (have_next) prepare(cn);
  }

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
  p.kq = (const uint8_t *)a.k; p.vq = (const uint8_t *)a.v;
  p.ks = a.k_scale; p.kz = a.k_zero; p.vs = a.v_scale; p.vz = a.v_zero;
  dim3 grid(pl.splits, a.B * a.Hkv);
  if (a.fmt == VC_KV_INT4) draft_bf16_int4<128><<<grid, kDraftWaves * 64, 0, s>>>(p);
  else if (a.D == 128) draft_bf16_dense<128><<<grid, kDraftWaves * 64, 0, s>>>(p);
  else draft_bf16_dense<64><<<grid, kDraftWaves * 64, 0, s>>>(p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_combine(p.part_o, p.part_lse, pl.splits, (int)rows, a.D, a.dtype, a.out, a.out_lse, s);
}

}  // namespace vc
