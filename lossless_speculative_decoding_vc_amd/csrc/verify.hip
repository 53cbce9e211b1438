// Verify block attention against the full cache (bf16, MFMA).
//
// "Riepilogo Tecnico: VeriCache", "Algoritmo Principale", step 2: one forward
// pass over KV_full checks all drafted tokens in parallel; "Innovazioni
// Chiave del Sistema" (P1): verification is compute- and interconnect-bound.
// Row i of a request's block (the last accepted token and the drafts) sees
// the whole context and the block keys 0..i.
//
// Design (gfx950):
//  * the M block rows times the G = Hq/Hkv query heads that share a KV head
//    are packed into R = M*G query rows, so one pass over a KV head's keys
//    serves all of them (the contraction that makes verify dense).
//  * grid (splits, row tiles, B*Hkv); W waves per workgroup, 32 rows per
//    wave; the workgroup streams 32-token tiles of K (token-major) and V
//    (channel-major) through double-buffered LDS, every wave reading the
//    same tile, so K/V leave HBM once per row tile.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16; the token
//    rows of the two S^T tiles are permuted so that each lane's scores are
//    the 8 consecutive tokens the PV MFMA consumes as its k-slots: P never
//    leaves the registers it was computed in.
//  * fp32 online softmax in base 2, one running max per packed row; causal
//    masking only in tiles that reach the block.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kTile = 32;   // tokens per LDS tile

struct VerifyParams {
  int B, Hq, Hkv, G, M, R, splits;
  float qk_scale;
  int64_t ccap;
  const uint16_t *q;
  const uint16_t *ck, *cv;
  const int32_t *ctx_len;
  const uint16_t *bk, *bv;
  uint16_t *out;
  float *out_lse;
  float *part_o, *part_lse;
};

template <int D>
struct VerifyLds {
  static constexpr int kKStride = D * 2 + 16;   // bytes per K row (padded)
  static constexpr int kVStride = kTile * 2 + 16;   // bytes per V channel row (padded)
  static constexpr int kKBytes = kTile * kKStride;
  static constexpr int kVBytes = D * kVStride;
  static constexpr int kBuf = kKBytes + kVBytes;
};

template <int D, int W>
__global__ __launch_bounds__(W * 64) void verify_bf16(VerifyParams p) {
  using L = VerifyLds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int kPieces = 8 * D;   // 16-byte pieces per tile: K 4D + V 4D
  constexpr int kThreads = W * 64;
  constexpr int kPer = (kPieces + kThreads - 1) / kThreads;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * L::kBuf];

  const int bh = blockIdx.z;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.G, M = p.M;
  const int r0 = blockIdx.y * (32 * W) + 32 * wave;

  int cl = p.ctx_len[b];
  cl = cl < 0 ? 0 : (cl > p.ccap ? (int)p.ccap : cl);
  const int total = cl + M;
  const int nchunks = (total + kTile - 1) / kTile;
  const int cps = (nchunks + p.splits - 1) / p.splits;
  const int c0 = split * cps;
  const int c1 = min(c0 + cps, nchunks);

  // Q^T operands: column = packed row r = i*G + g.
  bf16x8 qb[2][KS];
  int row_i[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r = r0 + 16 * c + col;
    row_i[c] = r / G;
    if (r < p.R) {
      const int i = r / G, g = r % G;
      const uint16_t *qp = p.q + (((size_t)b * M + i) * p.Hq + kvh * G + g) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[c][ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * grp));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[c][ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  const uint16_t *ckb = p.ck + (size_t)bh * p.ccap * D;
  const uint16_t *cvb = p.cv + (size_t)bh * D * p.ccap;
  const uint16_t *bkb = p.bk + (size_t)bh * M * D;
  const uint16_t *bvb = p.bv + (size_t)bh * D * M;

  auto fetch = [&](int c, u32x4 *reg) {
    const int base = c * kTile;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = tid + u * kThreads;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (pc < 4 * D) {   // K piece: row, 16-byte segment
        const int row = pc / (D / 8), seg = pc % (D / 8);
        const int j = base + row;
        if (j < cl) v = *reinterpret_cast<const u32x4 *>(ckb + (size_t)j * D + 8 * seg);
        else if (j < total) v = *reinterpret_cast<const u32x4 *>(bkb + (size_t)(j - cl) * D + 8 * seg);
      } else if (pc < kPieces) {   // V piece: channel, 8 tokens
        const int pv = pc - 4 * D;
        const int d = pv >> 2, q4 = pv & 3;
        const int j0 = base + 8 * q4;
        if (j0 + 8 <= cl) {
          v = *reinterpret_cast<const u32x4 *>(cvb + (size_t)d * p.ccap + j0);
        } else {
          uint32_t w[4];
#pragma unroll
          for (int e2 = 0; e2 < 4; ++e2) {
            uint32_t h[2];
#pragma unroll
            for (int uu = 0; uu < 2; ++uu) {
              const int j = j0 + 2 * e2 + uu;
              uint16_t x = 0;
              if (j < cl) x = cvb[(size_t)d * p.ccap + j];
              else if (j < total) x = bvb[(size_t)d * M + (j - cl)];
              h[uu] = x;
            }
            w[e2] = h[0] | (h[1] << 16);
          }
          v = u32x4{w[0], w[1], w[2], w[3]};
        }
      }
      reg[u] = v;
    }
  };
  auto stash = [&](int buf, const u32x4 *reg) {
    uint8_t *base = lds + buf * L::kBuf;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int pc = tid + u * kThreads;
      if (pc < 4 * D) {
        const int row = pc / (D / 8), seg = pc % (D / 8);
        *reinterpret_cast<u32x4 *>(base + row * L::kKStride + 16 * seg) = reg[u];
      } else if (pc < kPieces) {
        const int pv = pc - 4 * D;
        const int d = pv >> 2, q4 = pv & 3;
        *reinterpret_cast<u32x4 *>(base + L::kKBytes + d * L::kVStride + 16 * q4) = reg[u];
      }
    }
  };

  float m_run[2] = {kNegInf, kNegInf}, l_run[2] = {0.f, 0.f};
  f32x4 o[2][DT];
#pragma unroll
  for (int c = 0; c < 2; ++c)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[c][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 pre[kPer];
  if (c0 < c1) {
    fetch(c0, pre);
    stash(0, pre);
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int buf = (c - c0) & 1;
    if (c + 1 < c1) fetch(c + 1, pre);
    const uint8_t *kt = lds + buf * L::kBuf;
    const uint8_t *vt = kt + L::kKBytes;
    const int base = c * kTile;

    f32x4 s[2][2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc)
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) s[cc][tau] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int kr = 8 * (col >> 2) + 4 * tau + (col & 3);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 ka = as_bf16x8(*reinterpret_cast<const u32x4 *>(kt + kr * L::kKStride + (32 * ks + 8 * grp) * 2));
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) s[cc][tau] = mfma16x16x32(ka, qb[cc][ks], s[cc][tau]);
      }
    }
    const bool need_mask = base + kTile > cl;
    bf16x8 pb[2];
#pragma unroll
    for (int cc = 0; cc < 2; ++cc) {
      float sc[8];
      float cmax = kNegInf;
#pragma unroll
      for (int tau = 0; tau < 2; ++tau)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[cc][tau][i] * p.qk_scale;
          if (need_mask) {
            const int j = base + 8 * grp + 4 * tau + i;
            if (j >= cl + row_i[cc] + 1) x = kNegInf;
          }
          sc[4 * tau + i] = x;
          cmax = fmaxf(cmax, x);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      const float m_new = fmaxf(m_run[cc], cmax);
      const float m_use = (m_new == kNegInf) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[cc] - m_use);
      float pr[8], psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pr[e] = fast_exp2(sc[e] - m_use);
        psum += pr[e];
      }
      l_run[cc] = l_run[cc] * alpha + psum;
      m_run[cc] = m_new;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[cc][dt] *= alpha;
      pb[cc] = as_bf16x8(u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                               pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])});
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const bf16x8 va = as_bf16x8(*reinterpret_cast<const u32x4 *>(vt + (16 * dt + col) * L::kVStride + 16 * grp));
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) o[cc][dt] = mfma16x16x32(va, pb[cc], o[cc][dt]);
    }
    if (c + 1 < c1) stash(buf ^ 1, pre);
    __syncthreads();
  }

  const int rows = p.B * M * p.Hq;
#pragma unroll
  for (int cc = 0; cc < 2; ++cc) {
    float l = l_run[cc];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = r0 + 16 * cc + col;
    if (r >= p.R) continue;
    const int i = r / G, g = r % G;
    const int orow = (b * M + i) * p.Hq + kvh * G + g;
    const float inv = (l > 0.f) ? 1.f / l : 0.f;
    if (p.splits == 1) {
      const float invo = 1.f / l;   // NaN for an empty key set
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        u32x2 w = u32x2{pack_bf16x2(o[cc][dt][0] * invo, o[cc][dt][1] * invo),
                        pack_bf16x2(o[cc][dt][2] * invo, o[cc][dt][3] * invo)};
        *reinterpret_cast<u32x2 *>(p.out + (size_t)orow * D + d) = w;
      }
      if (p.out_lse && grp == 0) p.out_lse[orow] = (l > 0.f) ? (m_run[cc] + fast_log2(l)) * kLn2 : kNegInf;
    } else {
      float *po = p.part_o + ((size_t)split * rows + orow) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        *reinterpret_cast<f32x4 *>(po + d) = o[cc][dt] * inv;
      }
      if (grp == 0) p.part_lse[(size_t)split * rows + orow] = (l > 0.f) ? m_run[cc] + fast_log2(l) : kNegInf;
    }
  }
}

int verify_waves(int R) { return R <= 64 ? 2 : (R <= 128 ? 4 : (R <= 192 ? 6 : 8)); }

template <int D>
void launch_verify_d(const VerifyParams &p, int W, int row_tiles, hipStream_t s) {
  dim3 grid(p.splits, row_tiles, p.B * p.Hkv);
  switch (W) {
    case 2: verify_bf16<D, 2><<<grid, 128, 0, s>>>(p); break;
    case 4: verify_bf16<D, 4><<<grid, 256, 0, s>>>(p); break;
    case 6: verify_bf16<D, 6><<<grid, 384, 0, s>>>(p); break;
    default: verify_bf16<D, 8><<<grid, 512, 0, s>>>(p); break;
  }
}

}  // namespace

SplitPlan plan_verify(const vc_verify_args &a) {
  SplitPlan p{1, 0};
  if (a.dtype == VC_FP32) return p;
  const int R = a.M * (a.Hq / a.Hkv);
  const int W = verify_waves(R);
  const int64_t row_tiles = (R + 32 * W - 1) / (32 * W);
  const int64_t wgs = (int64_t)a.B * a.Hkv * row_tiles;
  const int64_t chunks = (a.ccap + a.M + kTile - 1) / kTile;
  int s = a.num_splits;
  if (s <= 0) {
    s = 1;
    while (wgs * s < 512 && chunks / (s * 2) >= 16) s *= 2;
  }
  if (s > chunks && chunks > 0) s = (int)chunks;
  if (s < 1) s = 1;
  p.splits = s;
  if (s > 1) p.ws_bytes = (size_t)s * a.B * a.M * a.Hq * (a.D + 1) * sizeof(float);
  return p;
}

hipError_t launch_verify_f32(const vc_verify_args &a, hipStream_t s);

hipError_t launch_verify(const vc_verify_args &a, const SplitPlan &pl, hipStream_t s) {
  if (a.dtype == VC_FP32) return launch_verify_f32(a, s);
  VerifyParams p;
  p.B = a.B; p.Hq = a.Hq; p.Hkv = a.Hkv; p.G = a.Hq / a.Hkv; p.M = a.M; p.R = a.M * p.G;
  p.splits = pl.splits;
  p.qk_scale = a.scale * kLog2e;
  p.ccap = a.ccap;
  p.q = (const uint16_t *)a.q;
  p.ck = (const uint16_t *)a.ctx_k; p.cv = (const uint16_t *)a.ctx_v; p.ctx_len = a.ctx_len;
  p.bk = (const uint16_t *)a.blk_k; p.bv = (const uint16_t *)a.blk_v;
  p.out = (uint16_t *)a.out; p.out_lse = a.out_lse;
  const size_t rows = (size_t)a.B * a.M * a.Hq;
  p.part_o = (float *)a.workspace;
  p.part_lse = p.part_o ? p.part_o + (size_t)pl.splits * rows * a.D : nullptr;
  const int W = verify_waves(p.R);
  const int row_tiles = (p.R + 32 * W - 1) / (32 * W);
  if (a.D == 128) launch_verify_d<128>(p, W, row_tiles, s);
  else launch_verify_d<64>(p, W, row_tiles, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_combine(p.part_o, p.part_lse, pl.splits, (int)rows, a.D, a.dtype, a.out, a.out_lse, s);
}

}  // namespace vc
