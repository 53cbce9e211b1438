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
//  * the main segment's V is stored in 32-token blocks (channel-major inside
//    a block), so one chunk's V is a contiguous 8 KB run at head_dim 128.
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
  // int4 main segment (packed: kq is the array of 5120-byte blocks)
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
      for (int dt = 0; dt < DT; ++dt) ch.va[dt] = ld16(vb + (size_t)base * D + (16 * dt + col) * kChunk + 8 * grp);
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
            if (t < mlen) x = vb[(size_t)(t / kChunk) * D * kChunk + d * kChunk + (t % kChunk)];
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
  // Columns past the G heads are MFMA padding: with no visible token their
  // probabilities are 0, so their P operand columns are zeros (less
  // switching in the matrix cores; nothing reads those columns).
  const int lane_total = (col < G) ? total : 0;

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
        x = (base + 8 * grp + e < lane_total) ? x : kNegInf;
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
// the same interface).  K codes are grouped per channel over 32 tokens -- one
// group is exactly one 32-token chunk -- and V codes per token over 32
// channels.  Design:
//  * every wave streams its own chunks through a private ring of kI4Stages
//    LDS stages filled by direct global->LDS loads: per chunk 2 KB of K
//    codes, 2 KB of V codes and 1 KB of scales/zeros (plus 128 B of merge
//    degrees when present), two chunks in flight per wave.  No barrier is
//    needed: a wave only reads what it loaded itself.  Two workgroups share
//    a CU (63 KB of LDS each, at most 256 registers per lane), so every SIMD
//    interleaves two waves and 16 chunks (80 KB) per CU are in flight.
//  * the quantisation is folded into the other MFMA operand, so the VALU
//    never multiplies an individual code by its scale:
//      S_t   = sum_d (q_d s_d) c_td + sum_d q_d z_d
//      O_d  += sum_t (p_t s_tg) c_td + sum_t p_t z_tg
//    with c read as an exact fp16 "magic" value (1024 + c or 64 + c, one
//    shift and four and-or per eight codes).  On the score side the magic
//    offsets are removed by an extra MFMA against the constant -1024/-64
//    operand and the zero-point term is an MFMA whose A operand repeats z
//    along the rows.  On the value side both are the same for every channel
//    of a 32-channel group (V's magic depends on the token's slot, its zero
//    point on the token and group), so they collect in one running sum per
//    head and group, W_g = sum_t p_t (z_tg - magic_t s_tg), by two MFMAs per
//    group whose A operands (the zero points, the -magic constant) repeat
//    along the rows, added to the group's channels once after the loop.  All
//    operands are fp16 (v_mfma_f32_16x16x32_f16) with fp32 accumulation; Q
//    is brought into fp16 range with an exact per-head power-of-two scale.
//  * chunks that reach the bf16 tail or the end of the sequence are
//    dequantised element-wise after the main loop.
constexpr int kI4Stages = 3;
constexpr int kI4Stage = 5 * 1024 + 256;   // K codes, V codes, scales/zeros, degree (bytes)

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

VC_DEVICE f16x8 as_f16x8(const u32x4 &u) { return __builtin_bit_cast(f16x8, u); }
VC_DEVICE f32x4 mfma_f16(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}
VC_DEVICE uint32_t pk_mul_f16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b));
}
// acc + lo + hi of a packed fp16 pair (the word is taken by value: a bit
// cast applied to an ext_vector element would read element 0).
VC_DEVICE float sum_f16x2(uint32_t w, float acc) {
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, w), f16x2{(_Float16)1.0f, (_Float16)1.0f}, acc, false);
}
VC_DEVICE uint32_t pack_f16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
// One 32-bit word of eight 4-bit codes (code 2j in bits 4j..4j+3, code 2j+1
// in bits 16+4j..16+4j+3) as four fp16 pairs in code order:
//   (1024 + c0, 1024 + c1), (64 + c2, 64 + c3), (1024 + c4, 1024 + c5),
//   (64 + c6, 64 + c7).
// A code in bits 0..3 of a half lands in the low mantissa bits of an fp16
// whose ulp is 1, one in bits 4..7 in those of an fp16 whose ulp is 1/16:
// both exact.  One shift and four v_and_or_b32 per eight codes: a
// three-operand instruction takes no 32-bit literal here and at most one
// scalar operand, so the caller keeps the masks (lo = 0x000F000F,
// hi = 0x00F000F0) in SGPRs and the magics in VGPRs, values the compiler
// cannot fold into literals.  Plain C, not inline asm: the compiler must see
// these writes to insert the wait states an MFMA reading them needs.
VC_DEVICE u32x4 magic_codes(uint32_t w, uint32_t lo, uint32_t hi, uint32_t m1024, uint32_t m64) {
  const uint32_t w8 = w >> 8;
  return u32x4{(w & lo) | m1024, (w & hi) | m64, (w8 & lo) | m1024, (w8 & hi) | m64};
}
// The magic offsets of magic_codes, negated (fp16 pairs, same slot order).
constexpr uint32_t kNegMagic1024 = 0xE400E400u, kNegMagic64 = 0xD400D400u;

// Direct global->LDS load of 16 bytes per lane (lane i lands at lds + 16 i).
VC_DEVICE void dma16(const void *gptr, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}
// The same load from a wave-uniform 64-bit base plus a 32-bit lane offset
// (no per-lane 64-bit address arithmetic).
VC_DEVICE void dma16_s(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

template <int D, bool DEG, bool PACKED>
__global__ __launch_bounds__(kDraftWaves * 64, 2) void draft_int4(DraftParams p) {
  constexpr int KS = D / 32, DT = D / 16, NG = D / 32;
  static_assert(D == 128, "int4 draft is compiled for head_dim 128");
  constexpr int kBlk = DEG ? 6 : 5;   // direct loads per chunk per wave
  constexpr int kStages = kI4Stages, kStage = kI4Stage;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kDraftWaves * kStages * kStage];

  const int bh = blockIdx.y;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int split = blockIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.G;

  int mlen = p.main_len[bh];
  mlen = mlen < 0 ? 0 : (mlen > p.cap ? (int)p.cap : mlen);
  int tlen = 0;
  if (p.tail_len && p.tail_k) {
    tlen = p.tail_len[b];
    tlen = tlen < 0 ? 0 : (tlen > p.tcap ? (int)p.tcap : tlen);
  }
  // Chunks 0 .. nmain-1 cover the int4 segment (the last one masked at
  // mlen), chunks nmain .. nmain+ntail-1 the bf16 tail from token mlen on.
  const int nmain = (mlen + kChunk - 1) / kChunk;
  const int nchunks = nmain + (tlen + kChunk - 1) / kChunk;
  const int cps = (nchunks + p.splits - 1) / p.splits;
  const int c0 = split * cps;
  const int c1 = min(c0 + cps, nchunks);
  const int cf = max(c0, min(c1, nmain));   // [c0, cf): int4 chunks of this split

  // Q^T operand in fp16, channel order d = 32*grp + 8*ks + e (the K code
  // layout), scaled per head by 2^-E so that max |q| lies in [0.5, 1).
  float qf[KS][8];
  float qmax = 0.f;
  if (col < G) {
    const uint16_t *qp = p.q + ((size_t)b * p.Hq + kvh * G + col) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 w = ld16(qp + 32 * grp + 8 * ks);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        qf[ks][2 * j] = bf16_lo(w[j]);
        qf[ks][2 * j + 1] = bf16_hi(w[j]);
      }
    }
  } else {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 8; ++e) qf[ks][e] = 0.f;
  }
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) qmax = fmaxf(qmax, fabsf(qf[ks][e]));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 16, 64));
  qmax = fmaxf(qmax, __shfl_xor(qmax, 32, 64));
  const int qexp = (qmax > 0.f) ? __builtin_amdgcn_frexp_expf(qmax) : 0;
  const float qs = ldexpf(p.qk_scale, qexp);   // score scale of this lane's head (base 2)
  // Columns past the G heads are MFMA padding: a score of -inf there makes
  // their probabilities 0, so the value-side operands of those columns are
  // zeros (less switching in the matrix cores; nothing reads those columns).
  const float pad = (col < G) ? 0.f : kNegInf;
  u32x4 qh[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int j = 0; j < 4; ++j)
      qh[ks][j] = pack_f16x2(ldexpf(qf[ks][2 * j], -qexp), ldexpf(qf[ks][2 * j + 1], -qexp));
  // Make the compiler wait for the Q loads here: its wait counts do not see
  // the direct loads below and would otherwise count them.
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) __asm__ volatile("" ::"v"(qh[ks]));

  const uint8_t *kqb = p.kq + (size_t)bh * p.cap * (D / 2);
  const uint8_t *vqb = p.vq + (size_t)bh * D * (p.cap / 2);
  const uint16_t *ksb = p.ks + (size_t)bh * (p.cap / 32) * D;
  const uint16_t *kzb = p.kz + (size_t)bh * (p.cap / 32) * D;
  const uint16_t *vsb = p.vs + (size_t)bh * NG * p.cap;
  const uint16_t *vzb = p.vz + (size_t)bh * NG * p.cap;
  // packed: one 5120-byte block per 32 tokens (p.kq is the block array)
  const uint8_t *pkb = p.kq + (size_t)bh * (p.cap / kChunk) * kPackedBlock;
  const uint16_t *tkb = p.tail_k ? p.tail_k + (size_t)bh * p.tcap * D : nullptr;
  const uint16_t *tvb = p.tail_v ? p.tail_v + (size_t)bh * D * p.tcap : nullptr;
  const float *db = p.degree ? p.degree + b * p.deg_b_stride + kvh * p.deg_h_stride : nullptr;

  float m_run = kNegInf, l_run = 0.f;
  f32x4 o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // W_g of this lane's head: what the zero points and the magic offsets add
  // to every channel of V group g, accumulated by MFMAs whose A operand is
  // the same in every row (so all four rows of a lane hold the same sum)
  f32x4 wz[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) wz[g] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The lane's reference as the scores are taken relative to it: m_run,
  // or 0 while it is -inf.
  auto ref_use = [&]() __attribute__((always_inline)) { return (m_run == kNegInf) ? 0.f : m_run; };
  // Online softmax of one chunk's 8 scores per lane (token 8*grp + e), given
  // relative to m_use = ref_use() (the subtraction folded into the scores'
  // FMA).  Returns the probabilities relative to the lane's reference max.
  // Lazy reference: the lane groups exchange maxima and rescale only when
  // some score in the wave exceeds it by more than kSlack.
  auto softmax = [&](float (&x)[8], float (&pr)[8], float m_use) __attribute__((always_inline)) {
    float cmax = vmax(vmax(vmax(x[0], x[1]), vmax(x[2], x[3])), vmax(vmax(x[4], x[5]), vmax(x[6], x[7])));
    // m_run - m_use is 0, or -inf before the first finite score (then any
    // finite score takes the reference over; all -inf gives NaN: no)
    if (__any(cmax - (m_run - m_use) > kSlack)) {
      cmax += m_use;   // the scores' own maximum
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run, cmax);
      const float alpha = (m_new == kNegInf) ? 1.f : fast_exp2(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[dt] *= alpha;
#pragma unroll
      for (int g = 0; g < NG; ++g) wz[g] *= alpha;
      m_run = m_new;
      const float shift = ref_use() - m_use;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] -= shift;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(x[e]);
  };

  // ---- main loop: whole int4 chunks through the wave's LDS ring ----------
  uint8_t *ring = lds + wave * (kStages * kStage);
  const uint32_t ring_addr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)ring;
  const int first = c0 + wave;
  const int nmine = (cf > first) ? (cf - first + kDraftWaves - 1) / kDraftWaves : 0;
  // Direct loads of chunk c into stage st (lane i writes 16 bytes at 16 i):
  //  blocks 0-1: K codes, token row t at 64 t, its 16-byte slot s holding
  //              global slot s ^ ((t >> 3) & 3) (bank-conflict-free reads);
  //  blocks 2-3: V codes, channel d at 2048 + 16 d (the chunk's 32 tokens);
  //  block 4:    K scales (4096 + 2 ch), K zeros (4352 + 2 ch), V scales
  //              (4608 + 64 g + 2 t), V zeros (4864 + 64 g + 2 t);
  //  block 5:    merge degrees (5120 + 4 t), lanes 0..7 only.
  // Every piece is a contiguous run of the 32-token-blocked int4 layout, so
  // each load uses whole cache lines.
  // Lane byte offsets of the loads, the same for every chunk: K code rows
  // 16 h + lane/4 (slot swizzled), and 16 bytes per lane for the rest.
  uint32_t koff[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = 16 * h + (lane >> 2);
    koff[h] = (uint32_t)(t * (D / 2) + 16 * ((lane & 3) ^ ((t >> 3) & 3)));
  }
  const uint32_t loff = 16u * (uint32_t)lane;
  auto issue = [&](int k) __attribute__((always_inline)) {
    const int c = first + kDraftWaves * k;
    const int base = c * kChunk;
    const uint32_t st = ring_addr + (uint32_t)((k % kStages) * kStage);
    if constexpr (PACKED) {
      // the block's K codes, V codes and its four 256-byte parameter pieces
      // are one contiguous 5120-byte run
      const uint8_t *blk = pkb + (size_t)c * kPackedBlock;
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16_s(koff[h], blk, st + 1024 * h);
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16_s(loff, blk + kPackedVCodes + 1024 * h, st + 2048 + 1024 * h);
      dma16_s(loff, blk + kPackedKScale, st + 4096);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16_s(koff[h], kqb + (size_t)base * (D / 2), st + 1024 * h);
#pragma unroll
      for (int h = 0; h < 2; ++h) dma16_s(loff, vqb + (size_t)base * (D / 2) + 1024 * h, st + 2048 + 1024 * h);
      const uint16_t *src;
      const int q = lane & 15;
      if (lane < 16) src = ksb + (size_t)(base / 32) * D + 8 * q;
      else if (lane < 32) src = kzb + (size_t)(base / 32) * D + 8 * q;
      else if (lane < 48) src = vsb + (size_t)base * NG + 8 * q;
      else src = vzb + (size_t)base * NG + 8 * q;
      dma16(src, st + 4096);
    }
    if (DEG) {
      if (lane < 8) dma16_s(loff, db + base, st + 5120);
    }
  };
  auto wait_chunks_after = [&](int n) __attribute__((always_inline)) {   // n = 0..kStages-2
    if (n >= 3) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(3 * kBlk) : "memory");
    else if (n == 2) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kBlk) : "memory");
    else if (n == 1) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(kBlk) : "memory");
    else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  static_assert(kStages <= 5, "wait_chunks_after covers up to 3 chunks in flight");
  u32x4 negm = u32x4{kNegMagic1024, kNegMagic64, kNegMagic1024, kNegMagic64};
  uint32_t m1024 = 0x64006400u, m64 = 0x54005400u, mlo = 0x000F000Fu, mhi = 0x00F000F0u;
  __asm__ volatile("" : "+v"(m1024), "+v"(m64), "+v"(negm));   // the magics stay in VGPRs
  __asm__ volatile("" : "+s"(mlo), "+s"(mhi));     // and the masks in SGPRs

  // One int4 chunk from its LDS stage; `masked` drops tokens at or past mlen.
  auto main_chunk = [&](const uint8_t *st, int c, bool masked) __attribute__((always_inline)) {
    // operands of this chunk
    u32x4 kc[2], ksc[KS], kzr[KS], vsc[NG], vzr[NG];
    uint32_t vc[DT];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = 8 * (col >> 2) + 4 * tau + (col & 3);
      kc[tau] = *reinterpret_cast<const u32x4 *>(st + 64 * t + 16 * (grp ^ ((t >> 3) & 3)));
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      ksc[ks] = *reinterpret_cast<const u32x4 *>(st + 4096 + 2 * (32 * grp + 8 * ks));
      kzr[ks] = *reinterpret_cast<const u32x4 *>(st + 4352 + 2 * (32 * grp + 8 * ks));
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) vc[dt] = *reinterpret_cast<const uint32_t *>(st + 2048 + 16 * (16 * dt + col) + 4 * grp);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      vsc[g] = *reinterpret_cast<const u32x4 *>(st + 4608 + 64 * g + 16 * grp);
      vzr[g] = *reinterpret_cast<const u32x4 *>(st + 4864 + 64 * g + 16 * grp);
    }
    float lg[8];
    if (DEG) {
      const f32x4 d0 = *reinterpret_cast<const f32x4 *>(st + 5120 + 32 * grp);
      const f32x4 d1 = *reinterpret_cast<const f32x4 *>(st + 5120 + 32 * grp + 16);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lg[e] = fast_log2(d0[e]);
        lg[4 + e] = fast_log2(d1[e]);
      }
    }
    // scores: S = C + codes . q' with q' = q s and the row-constant
    // C = sum_d q_d z_d - (magic offsets) . q'
    u32x4 qp[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 4; ++j) qp[ks][j] = pk_mul_f16(qh[ks][j], ksc[ks][j]);
    f32x4 cst = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      cst = mfma_f16(negm, qp[ks], cst);
      cst = mfma_f16(kzr[ks], qh[ks], cst);
    }
    f32x4 s[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      s[tau] = cst;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[tau] = mfma_f16(magic_codes(kc[tau][ks], mlo, mhi, m1024, m64), qp[ks], s[tau]);
    }
    float sc[8], pr[8];
    const float m_use = ref_use(), bias = pad - m_use;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sc[e] = fmaf(s[e >> 2][e & 3], qs, DEG ? lg[e] + bias : bias);
      if (masked && c * kChunk + 8 * grp + e >= mlen) sc[e] = kNegInf;
    }
    softmax(sc, pr, m_use);
    // O += (magic + codes) . (p s) per 32-channel group g of the V scales;
    // W_g += p . z - (p s) . magic, the part shared by the group's channels:
    // the zero points (the same for every channel row of the group) and the
    // constant -magic operand against P and P s, exact fp16 products in fp32
    u32x4 pp;
#pragma unroll
    for (int j = 0; j < 4; ++j) pp[j] = pack_f16x2(pr[2 * j], pr[2 * j + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      l_run = sum_f16x2(pp[j], l_run);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      u32x4 pg;
#pragma unroll
      for (int j = 0; j < 4; ++j) pg[j] = pk_mul_f16(pp[j], vsc[g][j]);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int dt = 2 * g + h;
        o[dt] = mfma_f16(magic_codes(vc[dt], mlo, mhi, m1024, m64), pg, o[dt]);
      }
      wz[g] = mfma_f16(vzr[g], pp, wz[g]);
      wz[g] = mfma_f16(negm, pg, wz[g]);
    }
  };

  auto step = [&](int k, bool masked) __attribute__((always_inline)) {
    wait_chunks_after(min(nmine - 1 - k, kStages - 2));
    if (k + kStages - 1 < nmine) issue(k + kStages - 1);
    main_chunk(ring + (k % kStages) * kStage, first + kDraftWaves * k, masked);
  };
  // Only the chunk that holds token mlen-1 can be partial, and it is the
  // wave's last: whole chunks run in a loop of their own, so the loop holds a
  // single copy of the chunk code and the accumulators stay in place.
  const int nwhole = (nmine > 0 && (first + kDraftWaves * (nmine - 1) + 1) * kChunk > mlen) ? nmine - 1 : nmine;
  for (int k = 0; k < min(kStages - 1, nmine); ++k) issue(k);
  for (int k = 0; k < nwhole; ++k) step(k, false);
  for (int k = nwhole; k < nmine; ++k) step(k, true);

  // ---- bf16 tail chunks (tokens mlen + 32 j ...): loads clamped in range and
  // masked afterwards, so they issue back to back ---------------------------
  // (The wave's chunks are first + 4 k; those past its int4 ones all lie in
  // [nmain, c1).)
  for (int c = first + kDraftWaves * nmine; c < c1; c += kDraftWaves) {
    const int tb = kChunk * (c - nmain);   // first tail index of this chunk
    u32x4 ka[2][KS], va[DT];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t = tb + 8 * (col >> 2) + 4 * tau + (col & 3);
      const int tc = min(t, tlen - 1);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4 w = ld16(tkb + (size_t)tc * D + 32 * grp + 8 * ks);
#pragma unroll
        for (int j = 0; j < 4; ++j) ka[tau][ks][j] = pack_f16x2(bf16_lo(w[j]), bf16_hi(w[j]));
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + col;
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = bf16_to_f32(tvb[(size_t)d * p.tcap + min(tb + 8 * grp + e, tlen - 1)]);
#pragma unroll
      for (int j = 0; j < 4; ++j) va[dt][j] = pack_f16x2(x[2 * j], x[2 * j + 1]);
    }
    f32x4 s[2];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      s[tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) s[tau] = mfma_f16(ka[tau][ks], qh[ks], s[tau]);
    }
    float sc[8], pr[8];
    const float m_use = ref_use(), bias = pad - m_use;
#pragma unroll
    for (int e = 0; e < 8; ++e) sc[e] = (tb + 8 * grp + e < tlen) ? fmaf(s[e >> 2][e & 3], qs, bias) : kNegInf;
    softmax(sc, pr, m_use);
    u32x4 pp;
#pragma unroll
    for (int j = 0; j < 4; ++j) pp[j] = pack_f16x2(pr[2 * j], pr[2 * j + 1]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      l_run = sum_f16x2(pp[j], l_run);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt] = mfma_f16(va[dt], pp, o[dt]);
  }

  // ---- W_g onto every channel of group g --------------------------------
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] += wz[dt >> 1];

  // ---- merge the 4 waves through LDS (reusing the ring) ------------------
  l_run += __shfl_xor(l_run, 16, 64);
  l_run += __shfl_xor(l_run, 32, 64);
  __syncthreads();   // every wave is done with its ring
  float (*sm)[16] = reinterpret_cast<float (*)[16]>(lds);
  float (*sl)[16] = reinterpret_cast<float (*)[16]>(lds + kDraftWaves * 16 * sizeof(float));
  static_assert(2 * kDraftWaves * 16 * sizeof(float) + kDraftWaves * D * 17 * sizeof(float) <= sizeof(lds),
                "the merge area fits the ring");
  float (*so)[D][17] = reinterpret_cast<float (*)[D][17]>(lds + 2 * kDraftWaves * 16 * sizeof(float));
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

hipError_t launch_draft(const vc_draft_args &a, const SplitPlan &pl, hipStream_t s, hipEvent_t after_kernel) {
  if (a.dtype == VC_FP32) {
    const hipError_t e = launch_draft_f32(a, s);
    return (e != hipSuccess || !after_kernel) ? e : hipEventRecord(after_kernel, s);
  }
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
  p.kq = (const uint8_t *)a.k; p.vq = (const uint8_t *)a.v;   // packed: k holds the blocks
  p.ks = a.k_scale; p.kz = a.k_zero; p.vs = a.v_scale; p.vz = a.v_zero;
  const bool pk = a.fmt == VC_KV_INT4_PACKED;
  dim3 grid(pl.splits, a.B * a.Hkv);
  if (a.fmt != VC_KV_DENSE) {
    if (pk && a.degree) draft_int4<128, true, true><<<grid, kDraftWaves * 64, 0, s>>>(p);
    else if (pk) draft_int4<128, false, true><<<grid, kDraftWaves * 64, 0, s>>>(p);
    else if (a.degree) draft_int4<128, true, false><<<grid, kDraftWaves * 64, 0, s>>>(p);
    else draft_int4<128, false, false><<<grid, kDraftWaves * 64, 0, s>>>(p);
  } else if (a.D == 128) {
    draft_bf16_dense<128><<<grid, kDraftWaves * 64, 0, s>>>(p);
  } else {
    draft_bf16_dense<64><<<grid, kDraftWaves * 64, 0, s>>>(p);
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && after_kernel) e = hipEventRecord(after_kernel, s);
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_combine(p.part_o, p.part_lse, pl.splits, (int)rows, a.D, a.dtype, a.out, a.out_lse, s);
}

}  // namespace vc
