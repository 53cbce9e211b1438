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
//  * grid (splits, row groups, B*Hkv); K/V leave HBM once per row group.
//    Up to 64 packed rows: four waves (one per SIMD) of one 16-row column
//    tile.  Up to 192 rows (token split, verify_ts): eight waves, the two
//    waves of a SIMD hold the same 32 or 48 rows and take alternate
//    32-token halves of every tile, so each reads only its half of the tile
//    from LDS and the two carry equal work; their softmax states are merged
//    through LDS at the end.  Up to 256 rows (row split, verify_pp): eight
//    waves of two column tiles, the two waves of a SIMD on different rows.
//  * the workgroup streams 64-token tiles of K (token-major) and V
//    (channel-major) through a ring of LDS stages (four, or five for the
//    token split: 160 KB at head_dim 128) filled by direct global->LDS
//    loads (global_load_lds_dwordx4), two to three tiles in flight without
//    holding any of them in registers.  Each wave-wide load lands as 1 KB of
//    contiguous LDS, so bank conflicts are avoided by XOR-swizzling which
//    16-byte piece a lane fetches instead of padding rows.  Tiles that reach
//    the block keys or the end of the key sequence are staged through
//    registers after the main loop.
//  * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16; the token
//    rows of the S^T tiles are permuted so each lane's scores are the 8
//    consecutive tokens the PV MFMA consumes as its k-slots: P never leaves
//    the registers it was computed in.
//  * the two waves of a SIMD run a ping-pong: one issues an MFMA cluster
//    (PV, then QK) while the other computes probabilities on the VALU,
//    separated by workgroup barriers.
//  * fp32 online softmax in base 2 with a lazily updated reference max per
//    packed row (rescale only when a score exceeds it by more than 2^8);
//    causal masking only in tiles that reach the block.
#include <float.h>

#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kTile = 64;      // tokens per LDS tile
constexpr int kStages = 4;     // LDS ring depth
constexpr int kStagesTs = 5;   // LDS ring depth of the token-split schedule (160 KB at head_dim 128)
constexpr float kSlack = 8.f;  // lazy-rescale threshold (base 2)

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
struct Lds {
  static constexpr int kKRow = D * 2;                   // bytes per K token row
  static constexpr int kKBytes = kTile * kKRow;
  static constexpr int kVRow = kTile * 2;               // bytes per V channel row (128)
  static constexpr int kVBytes = D * kVRow;
  static constexpr int kStage = kKBytes + kVBytes;      // 256 * D bytes
  static constexpr int kBlocks = kStage / 1024;         // 1 KB per wave-wide load
  static constexpr int kKBlocks = kKBytes / 1024;
  static constexpr int kSlots = kKRow / 16;             // 16-byte slots per K row
  static constexpr int kRowsPerBlock = 1024 / kKRow;
};

// LDS row r of a K tile holds token ktok(r) of S^T tile r/16, row r%16, so
// the 16 lanes of one operand read hit 16 consecutive rows.
VC_DEVICE int ktok(int r) {
  const int tau = r >> 4, m = r & 15;
  return 32 * (tau >> 1) + 8 * (m >> 2) + 4 * (tau & 1) + (m & 3);
}
// XOR swizzle of 16-byte slots (an involution: maps logical <-> physical).
template <int D>
VC_DEVICE int kswz(int r, int slot) {
  return (D == 128) ? (slot ^ (r & 15)) : (slot ^ ((r >> 1) & 7));
}
VC_DEVICE int vswz(int d, int slot) { return slot ^ ((d >> 1) & 7); }

// One 16-byte direct global->LDS load per lane: lane i's piece lands at
// LDS byte address lds_addr + 16*i.  Issued through inline assembly so the
// compiler does not serialise it against later LDS accesses; completion is
// tracked explicitly with s_waitcnt vmcnt and a workgroup barrier.
VC_DEVICE void load_lds16(const void *gptr, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}

// The same load with a scalar 64-bit base and a 32-bit per-lane byte offset.
VC_DEVICE void load_lds16_s(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr) : "memory", "m0");
}

// Tile that reaches the block keys or the end of the key sequence: staged
// through registers with the same swizzled layout (zero past the end).
template <int D>
VC_DEVICE void stage_slow(uint8_t *st, int base, int cl, int total, int M, int64_t ccap,
                                        const uint16_t *ckb, const uint16_t *cvb, const uint16_t *bkb,
                                        const uint16_t *bvb, int tid, int nthreads) {
  using L = Lds<D>;
  for (int pc = tid; pc < L::kBlocks * 64; pc += nthreads) {
    const int q = pc >> 6, ln = pc & 63;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (q < L::kKBlocks) {
      const int r = q * L::kRowsPerBlock + ln / L::kSlots;
      const int seg = kswz<D>(r, ln % L::kSlots);
      const int j = base + ktok(r);
      if (j < cl) v = *reinterpret_cast<const u32x4 *>(ckb + (size_t)j * D + 8 * seg);
      else if (j < total) v = *reinterpret_cast<const u32x4 *>(bkb + (size_t)(j - cl) * D + 8 * seg);
    } else {
      const int d = (q - L::kKBlocks) * 8 + ln / 8;
      const int j0 = base + 8 * vswz(d, ln % 8);
      uint32_t w[4];
      for (int e2 = 0; e2 < 4; ++e2) {
        uint32_t h[2];
        for (int uu = 0; uu < 2; ++uu) {
          const int j = j0 + 2 * e2 + uu;
          uint16_t x = 0;
          if (j < cl) x = cvb[(size_t)d * ccap + j];
          else if (j < total) x = bvb[(size_t)d * M + (j - cl)];
          h[uu] = x;
        }
        w[e2] = h[0] | (h[1] << 16);
      }
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    *reinterpret_cast<u32x4 *>(st + q * 1024 + ln * 16) = v;
  }
}

template <int D, int W, int CT>
__global__ __launch_bounds__(W * 64) void verify_bf16(VerifyParams p) {
  using L = Lds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int kThreads = W * 64;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * L::kStage];

  const int bh = blockIdx.z;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.G, M = p.M;
  const int r0 = blockIdx.y * (16 * CT * W) + 16 * CT * wave;   // first packed row of this wave

  int cl = p.ctx_len[b];
  cl = cl < 0 ? 0 : (cl > p.ccap ? (int)p.ccap : cl);
  const int total = cl + M;
  const int nchunks = (total + kTile - 1) / kTile;
  const int cps = (nchunks + p.splits - 1) / p.splits;
  const int c0 = split * cps;
  const int c1 = min(c0 + cps, nchunks);

  // Q^T operands: column = packed row r = i*G + g.
  bf16x8 qb[CT][KS];
  int row_lim[CT];   // row r sees key j iff j < row_lim = cl + i + 1
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = r0 + 16 * ct + col;
    row_lim[ct] = cl + r / G + 1;
    if (r < p.R) {
      const int i = r / G, g = r % G;
      const uint16_t *qp = p.q + (((size_t)b * M + i) * p.Hq + kvh * G + g) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * grp));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  // The direct loads below are invisible to the compiler's wait-count
  // tracking: if a Q load were still outstanding inside the main loop, the
  // compiler's wait for it would count the tile prefetches too and drain the
  // ring.  Consuming Q in an empty asm makes it wait here, once.
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __asm__ volatile("" ::"v"(qb[ct][ks]));

  const uint16_t *ckb = p.ck + (size_t)bh * p.ccap * D;
  const uint16_t *cvb = p.cv + (size_t)bh * D * p.ccap;
  const uint16_t *bkb = p.bk + (size_t)bh * M * D;
  const uint16_t *bvb = p.bv + (size_t)bh * D * M;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;

  // Tiles [c0, cf) hold only context tokens ("full"): each wave fetches whole
  // 1 KB blocks of them straight into LDS (block q: 4 K rows or 8 V channel
  // rows, lanes ordered by physical slot).  Tiles [cf, c1) reach the block
  // keys or the end of the key sequence; they are staged after the main loop.
  const int cf = max(c0, min(c1, cl / kTile));
  auto issue = [&](int c) __attribute__((always_inline)) {
    const int stage = c & (kStages - 1);
    const int base = c * kTile;
#pragma unroll
    for (int j = 0; j < (L::kBlocks + W - 1) / W; ++j) {
      const int q = wave + j * W;
      if (q >= L::kBlocks) break;
      const uint16_t *src;
      if (q < L::kKBlocks) {
        const int r = q * L::kRowsPerBlock + lane / L::kSlots;
        src = ckb + (size_t)(base + ktok(r)) * D + 8 * kswz<D>(r, lane % L::kSlots);
      } else {
        const int d = (q - L::kKBlocks) * 8 + lane / 8;
        src = cvb + (size_t)d * p.ccap + base + 8 * vswz(d, lane % 8);
      }
      load_lds16(src, lds_base + (uint32_t)(stage * L::kStage + q * 1024));
    }
  };

  float m_run[CT], l_run[CT], mq[CT];   // mq = scaled reference (0 while it is -inf)
  f32x4 o[CT][DT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    // a padding row (r >= R) starts with a reference of +inf: its
    // probabilities are 0, so its P operand columns are zeros (less switching
    // in the matrix cores); padding rows are never stored
    const bool real = r0 + 16 * ct + col < p.R;
    m_run[ct] = real ? kNegInf : -kNegInf;
    mq[ct] = real ? 0.f : -kNegInf;
    l_run[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Pieces of one 32-token half h of a 64-token tile (S^T tiles tau = 2h,
  // 2h+1, then the PV k-step h).
  const float qs = p.qk_scale;
  using KOps = u32x4[2][KS];
  using Scores = f32x4[CT][2];
  // K operands of half h (16 token rows per S^T tile, 32 channels per k-step).
  auto load_k = [&](const uint8_t *kt, int h, KOps &ka) __attribute__((always_inline)) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int kr = 16 * (2 * h + t2) + col;   // token 8*(col>>2) + 4*t2 + (col&3) of the half
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        ka[t2][ks] = *reinterpret_cast<const u32x4 *>(kt + kr * L::kKRow + 16 * kswz<D>(kr, 4 * ks + grp));
    }
  };
  auto qk = [&](const KOps &ka, Scores &sc) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) sc[ct][0] = sc[ct][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) sc[ct][t2] = mfma16x16x32(as_bf16x8(ka[t2][ks]), qb[ct][ks], sc[ct][t2]);
  };
  // Lazy reference max per packed row: each lane compares its own 8 scores
  // with the row's reference; only when some score in the wave exceeds it by
  // more than kSlack (base 2) do the lane groups exchange their maxima (two
  // cross-lane shuffles) and rescale.  After the first tiles that branch is
  // rarely taken, and probabilities stay <= 2^kSlack.
  auto row_max = [&](const Scores &sc, float (&lmax)[CT]) __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      lmax[ct] = vmax(vmax(vmax(sc[ct][0][0], sc[ct][0][1]), vmax(sc[ct][0][2], sc[ct][0][3])),
                      vmax(vmax(sc[ct][1][0], sc[ct][1][1]), vmax(sc[ct][1][2], sc[ct][1][3])));
      need |= (lmax[ct] - m_run[ct]) * qs > kSlack;   // false when both are -inf
    }
    return need;
  };
  auto rescale = [&](bool need, const float (&lmax)[CT]) __attribute__((always_inline)) {
    if (__any(need)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float cmax = lmax[ct];
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
        const float m_new = fmaxf(m_run[ct], cmax);
        // 1 when the reference does not move (also at -inf, and at +inf for padding rows)
        const float alpha = (m_new == m_run[ct]) ? 1.f : fast_exp2((m_run[ct] - m_new) * qs);
        l_run[ct] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
        m_run[ct] = m_new;
        mq[ct] = (m_new == kNegInf) ? 0.f : m_new * qs;
      }
    }
  };
  auto update_max = [&](const Scores &sc) __attribute__((always_inline)) {
    float lmax[CT];
    rescale(row_max(sc, lmax), lmax);
  };
  // Probabilities relative to the reference, packed to bf16 as the B operand
  // of the PV MFMA (k-slot e of lane group grp = token 8*grp + e of the half).
  // The row sum accumulates the bf16-rounded probabilities, i.e. exactly the
  // weights the PV MFMA applies.
  auto exp_pack = [&](const Scores &sc, bf16x8 (&pb)[CT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sc[ct][e >> 2][e & 3], qs, -mq[ct]));
      const u32x4 w = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                            pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
      l_run[ct] = sum_bf16x2(w[3], sum_bf16x2(w[2], sum_bf16x2(w[1], sum_bf16x2(w[0], l_run[ct]))));
      pb[ct] = as_bf16x8(w);
    }
  };
  // V^T operands of half h (16 channels per output tile, 32 tokens).
  using VOps = u32x4[DT];
  auto load_v = [&](const uint8_t *kt, int h, VOps &va) __attribute__((always_inline)) {
    const uint8_t *vt = kt + L::kKBytes;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + col;
      va[dt] = *reinterpret_cast<const u32x4 *>(vt + d * L::kVRow + 16 * vswz(d, 4 * h + grp));
    }
  };
  auto pv = [&](const VOps &va, const bf16x8 (&pb)[CT]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct][dt] = mfma16x16x32(as_bf16x8(va[dt]), pb[ct], o[ct][dt]);
  };
  auto stage_ptr = [&](int c) __attribute__((always_inline)) { return lds + (c & (kStages - 1)) * L::kStage; };

  // Main loop over the full tiles, software-pipelined by halves: while the
  // QK MFMAs of half n+1 run, the VALU computes the probabilities of half n;
  // while the PV MFMAs of half n run, it takes the maxima of half n+1.  K
  // and V operands are read from LDS one half-step before their MFMAs.
  //
  // Ring of kStages LDS stages filled by direct loads.  At the top of tile
  // c the wave waits for tile c+1 (direct loads complete in issue order per
  // wave, so "landed" is vmcnt <= the loads issued after it), and a barrier
  // publishes all waves' pieces and guarantees that tile c-1's stage is no
  // longer read, so tile c+3 can be issued into it.  The loop holds no call
  // and no other memory load, so nothing else moves vmcnt.
  constexpr int kMine = L::kBlocks / W;   // fewest direct loads per wave per tile
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {   // n = 0, 1, 2 tiles may stay in flight
    if (n >= 2) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kMine) : "memory");
    else if (n == 1) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(kMine) : "memory");
    else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  if (c0 < cf) {
    for (int c = c0; c < min(c0 + kStages - 1, cf); ++c) issue(c);
    wait_tiles_after(min(cf - 1 - c0, kStages - 2));
    __syncthreads();
    KOps ka;
    VOps va;
    Scores s_cur, s_nxt;
    bf16x8 pb[CT];
    load_k(stage_ptr(c0), 0, ka);
    qk(ka, s_cur);
    load_k(stage_ptr(c0), 1, ka);
    load_v(stage_ptr(c0), 0, va);
    update_max(s_cur);
    for (int it = c0; it + 1 < cf; ++it) {
      wait_tiles_after(it + 2 < cf ? 1 : 0);
      __syncthreads();
      if (it + kStages - 1 < cf) issue(it + kStages - 1);
      const uint8_t *kt = stage_ptr(it), *kn = stage_ptr(it + 1);
      // half 2*it: S(2it+1) = QK, P(2it) -> PV.  The scheduling fences keep
      // each operand refill after the MFMAs that still read the old one, so
      // only one copy of the K and V operands is live.
      float lmax[CT];
      qk(ka, s_nxt);
      exp_pack(s_cur, pb);
      __builtin_amdgcn_sched_barrier(0);
      load_k(kn, 0, ka);
      pv(va, pb);
      bool need = row_max(s_nxt, lmax);
      __builtin_amdgcn_sched_barrier(0);
      load_v(kt, 1, va);
      rescale(need, lmax);
      // half 2*it+1: S(2it+2) = QK, P(2it+1) -> PV
      qk(ka, s_cur);
      exp_pack(s_nxt, pb);
      __builtin_amdgcn_sched_barrier(0);
      load_k(kn, 1, ka);
      pv(va, pb);
      need = row_max(s_cur, lmax);
      __builtin_amdgcn_sched_barrier(0);
      load_v(kn, 0, va);
      rescale(need, lmax);
    }
    const uint8_t *kt = stage_ptr(cf - 1);
    qk(ka, s_nxt);
    exp_pack(s_cur, pb);
    pv(va, pb);
    load_v(kt, 1, va);
    update_max(s_nxt);
    exp_pack(s_nxt, pb);
    pv(va, pb);
  }

  // Tiles with block keys or past the end: staged through registers, causal
  // mask applied to the scores, not pipelined.
  for (int it = cf; it < c1; ++it) {
    uint8_t *st = stage_ptr(it);
    __syncthreads();
    stage_slow<D>(st, it * kTile, cl, total, M, p.ccap, ckb, cvb, bkb, bvb, tid, kThreads);
    __syncthreads();
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      KOps ka;
      Scores sc;
      bf16x8 pb[CT];
      load_k(st, h, ka);
      qk(ka, sc);
      const int jb = it * kTile + 32 * h + 8 * grp;   // key index of score (t2, i): jb + 4*t2 + i
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jb + 4 * t2 + i >= row_lim[ct]) sc[ct][t2][i] = kNegInf;
      VOps va;
      load_v(st, h, va);
      update_max(sc);
      exp_pack(sc, pb);
      pv(va, pb);
    }
  }

  const int rows = p.B * M * p.Hq;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float l = l_run[ct];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = r0 + 16 * ct + col;
    if (r >= p.R) continue;
    const int i = r / G, g = r % G;
    const int orow = (b * M + i) * p.Hq + kvh * G + g;
    if (p.splits == 1) {
      const float invo = 1.f / l;   // NaN for an empty key set
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        u32x2 w = u32x2{pack_bf16x2(o[ct][dt][0] * invo, o[ct][dt][1] * invo),
                        pack_bf16x2(o[ct][dt][2] * invo, o[ct][dt][3] * invo)};
        *reinterpret_cast<u32x2 *>(p.out + (size_t)orow * D + d) = w;
      }
      if (p.out_lse && grp == 0) p.out_lse[orow] = (l > 0.f) ? (m_run[ct] * p.qk_scale + fast_log2(l)) * kLn2 : kNegInf;
    } else {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      float *po = p.part_o + ((size_t)split * rows + orow) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        *reinterpret_cast<f32x4 *>(po + d) = o[ct][dt] * inv;
      }
      if (grp == 0) p.part_lse[(size_t)split * rows + orow] = (l > 0.f) ? m_run[ct] * p.qk_scale + fast_log2(l) : kNegInf;
    }
  }
}

// The rows [r0, r0 + 16*CT) of one workgroup of eight waves (two per SIMD),
// run by one wave.  Row split (verify_pp): the two waves of a SIMD hold
// different rows, possibly different CT, and each takes both 32-token halves
// of every tile.  Token split (verify_ts, kTokens): both waves of a SIMD hold
// the same rows; wave w takes the first half of every tile and wave w+4 the
// second, and their softmax states are merged at the end.
template <int D, int CT, bool kTokens>
VC_DEVICE void pp_rows(const VerifyParams &p, uint8_t *lds, const int wave, const int r0) {
  constexpr int W = 8;
  using L = Lds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int kThreads = W * 64;

  const int bh = blockIdx.z;
  const int b = bh / p.Hkv, kvh = bh % p.Hkv;
  const int split = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int G = p.G, M = p.M;

  int cl = p.ctx_len[b];
  cl = cl < 0 ? 0 : (cl > p.ccap ? (int)p.ccap : cl);
  const int total = cl + M;
  const int nchunks = (total + kTile - 1) / kTile;
  const int cps = (nchunks + p.splits - 1) / p.splits;
  const int c0 = split * cps;
  const int c1 = min(c0 + cps, nchunks);

  // Q^T operands: column = packed row r = i*G + g.
  bf16x8 qb[CT][KS];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    const int r = r0 + 16 * ct + col;
    if (r < p.R) {
      const int i = r / G, g = r % G;
      const uint16_t *qp = p.q + (((size_t)b * M + i) * p.Hq + kvh * G + g) * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = as_bf16x8(*reinterpret_cast<const u32x4 *>(qp + 32 * ks + 8 * grp));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qb[ct][ks] = as_bf16x8(u32x4{0, 0, 0, 0});
    }
  }

  // The direct loads below are invisible to the compiler's wait-count
  // tracking: if a Q load were still outstanding inside the main loop, the
  // compiler's wait for it would count the tile prefetches too and drain the
  // ring.  Consuming Q in an empty asm makes it wait here, once.
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) __asm__ volatile("" ::"v"(qb[ct][ks]));

  const uint16_t *ckb = p.ck + (size_t)bh * p.ccap * D;
  const uint16_t *cvb = p.cv + (size_t)bh * D * p.ccap;
  const uint16_t *bkb = p.bk + (size_t)bh * M * D;
  const uint16_t *bvb = p.bv + (size_t)bh * D * M;
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;

  // Tiles [c0, cf) hold only context tokens ("full"): each wave fetches whole
  // 1 KB blocks of them straight into LDS (block q: 4 K rows or 8 V channel
  // rows, lanes ordered by physical slot).  Tiles [cf, c1) reach the block
  // keys or the end of the key sequence; they are staged after the main loop.
  const int cf = max(c0, min(c1, cl / kTile));
  // Per-lane byte offsets of this wave's direct loads, relative to the
  // tile's first K row / first V column (scalar bases, so each load holds one
  // 32-bit VGPR).  K blocks come first: W divides the K block count.  The
  // wave's j-th K block lies W*kRowsPerBlock rows (a multiple of 32, so the
  // same row permutation and swizzle) below its first, and its j-th V block
  // 8*W channel rows below its first: one offset per kind, with the block's
  // distance added to the scalar base.
  constexpr int kJobs = L::kBlocks / W, kKJobs = L::kKBlocks / W;
  static_assert(L::kBlocks % W == 0 && L::kKBlocks % W == 0, "even split of a tile's loads");
  static_assert((W * L::kRowsPerBlock) % 32 == 0, "K blocks of one wave share the row permutation");
  uint32_t doff_k, doff_v;
  {
    const int r = wave * L::kRowsPerBlock + lane / L::kSlots;
    doff_k = (uint32_t)(ktok(r) * D + 8 * kswz<D>(r, lane % L::kSlots)) * 2u;
    const int d = wave * 8 + lane / 8;
    doff_v = (uint32_t)((size_t)d * p.ccap + 8 * vswz(d, lane % 8)) * 2u;
  }
  // LDS stage of tile c: a ring of kStages tiles (row split) or of
  // kStagesTs (token split), counted from the split's first tile
  auto stage_of = [&](int c) __attribute__((always_inline)) {
    return kTokens ? (c - c0) % kStagesTs : (c & (kStages - 1));
  };
  auto issue = [&](int c) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (uint32_t)(stage_of(c) * L::kStage);
    const uint16_t *kb = ckb + (size_t)c * kTile * D, *vb = cvb + (size_t)c * kTile;
#pragma unroll
    for (int j = 0; j < kJobs; ++j) {
      const uint32_t dst = st + (uint32_t)((wave + j * W) * 1024);
      if (j < kKJobs) load_lds16_s(doff_k, kb + (size_t)j * W * L::kRowsPerBlock * D, dst);
      else load_lds16_s(doff_v, vb + (size_t)(j - kKJobs) * 8 * W * p.ccap, dst);
    }
  };

  float m_run[CT], l_run[CT];
  f32x4 o[CT][DT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    // A real row starts with the reference -FLT_MAX: every finite score
    // reaches it, so the first tile with a finite score takes the reference
    // over before any probability is formed, and the scaled reference is
    // plain m_run * qs (finite) throughout.  Until then l and o are 0, so the
    // rescale weight applied to them (exp2 of a non-positive number) does
    // not matter.  A padding row (r >= R) starts with +inf: its
    // probabilities are 0, so its P operand columns are zeros (less
    // switching in the matrix cores); padding rows are never stored.
    const bool real = r0 + 16 * ct + col < p.R;
    m_run[ct] = real ? -FLT_MAX : -kNegInf;
    l_run[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Pieces of one 32-token half h of a 64-token tile (S^T tiles tau = 2h,
  // 2h+1, then the PV k-step h).
  const float qs = p.qk_scale;
  using KOps = u32x4[2][KS];
  using Scores = f32x4[CT][2];
  // K operands of half h (16 token rows per S^T tile, 32 channels per k-step).
  // (k-steps [ks0, ks1) only, when given)
  auto load_k = [&](const uint8_t *kt, int h, KOps &ka, int ks0 = 0, int ks1 = D / 32) __attribute__((always_inline)) {
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
      const int kr = 16 * (2 * h + t2) + col;   // token 8*(col>>2) + 4*t2 + (col&3) of the half
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        if (ks >= ks0 && ks < ks1)
          ka[t2][ks] = *reinterpret_cast<const u32x4 *>(kt + kr * L::kKRow + 16 * kswz<D>(kr, 4 * ks + grp));
    }
  };
  auto qk = [&](const KOps &ka, Scores &sc) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) sc[ct][0] = sc[ct][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) sc[ct][t2] = mfma16x16x32(as_bf16x8(ka[t2][ks]), qb[ct][ks], sc[ct][t2]);
  };
  // Lazy reference max per packed row: each lane compares its own 8 scores
  // with the row's reference; only when some score in the wave exceeds it by
  // more than kSlack (base 2) do the lane groups exchange their maxima (two
  // cross-lane shuffles) and rescale.  After the first tiles that branch is
  // rarely taken, and probabilities stay <= 2^kSlack.
  auto row_max = [&](const Scores &sc, float (&lmax)[CT]) __attribute__((always_inline)) {
    bool need = false;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      lmax[ct] = vmax(vmax(vmax(sc[ct][0][0], sc[ct][0][1]), vmax(sc[ct][0][2], sc[ct][0][3])),
                      vmax(vmax(sc[ct][1][0], sc[ct][1][1]), vmax(sc[ct][1][2], sc[ct][1][3])));
      need |= (lmax[ct] - m_run[ct]) * qs > kSlack;   // false when both are -inf
    }
    return need;
  };
  auto rescale = [&](bool need, const float (&lmax)[CT]) __attribute__((always_inline)) {
    if (__any(need)) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        float cmax = lmax[ct];
        cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
        cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
        const float m_new = fmaxf(m_run[ct], cmax);
        // 1 when the reference does not move (also at +inf for padding rows)
        const float alpha = (m_new == m_run[ct]) ? 1.f : fast_exp2((m_run[ct] - m_new) * qs);
        l_run[ct] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[ct][dt] *= alpha;
        m_run[ct] = m_new;
      }
    }
  };
  auto update_max = [&](const Scores &sc) __attribute__((always_inline)) {
    float lmax[CT];
    rescale(row_max(sc, lmax), lmax);
  };
  // Probabilities relative to the reference, packed to bf16 as the B operand
  // of the PV MFMA (k-slot e of lane group grp = token 8*grp + e of the half).
  // The row sum accumulates the bf16-rounded probabilities, i.e. exactly the
  // weights the PV MFMA applies.
  auto exp_pack = [&](const Scores &sc, bf16x8 (&pb)[CT]) __attribute__((always_inline)) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float mq = m_run[ct] * qs;   // scaled reference (+inf for padding rows)
      float pr[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pr[e] = fast_exp2(fmaf(sc[ct][e >> 2][e & 3], qs, -mq));
      const u32x4 w = u32x4{pack_bf16x2(pr[0], pr[1]), pack_bf16x2(pr[2], pr[3]),
                            pack_bf16x2(pr[4], pr[5]), pack_bf16x2(pr[6], pr[7])};
      l_run[ct] = sum_bf16x2(w[3], sum_bf16x2(w[2], sum_bf16x2(w[1], sum_bf16x2(w[0], l_run[ct]))));
      pb[ct] = as_bf16x8(w);
    }
  };
  // V^T operands of half h (16 channels per output tile, 32 tokens).
  using VOps = u32x4[DT];
  auto load_v = [&](const uint8_t *kt, int h, VOps &va) __attribute__((always_inline)) {
    const uint8_t *vt = kt + L::kKBytes;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d = 16 * dt + col;
      va[dt] = *reinterpret_cast<const u32x4 *>(vt + d * L::kVRow + 16 * vswz(d, 4 * h + grp));
    }
  };
  auto pv = [&](const VOps &va, const bf16x8 (&pb)[CT]) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) o[ct][dt] = mfma16x16x32(as_bf16x8(va[dt]), pb[ct], o[ct][dt]);
  };
  auto stage_ptr = [&](int c) __attribute__((always_inline)) { return lds + stage_of(c) * L::kStage; };

  // Main loop over the full tiles as a two-group ping-pong.  Each 32-token
  // half n is an MFMA cluster M_n (O += PV of half n-1, then S_n = QK of
  // half n; between the two it reads the V operands of half n from LDS)
  // followed by a VALU cluster V_n (softmax of S_n into P_n; it reads the K
  // operands of half n+1).  The two waves that share a SIMD (w and w+4) run
  // the same sequence one cluster apart, separated by a workgroup barrier
  // after every cluster, so one of them issues MFMAs while the other runs
  // the softmax on the VALU (a single wave cannot overlap the two: an MFMA
  // blocks its own issue for its whole duration), and both read LDS in every
  // phase.
  //
  // Ring: in global phase f (wave group g runs its cluster f - g), relative
  // tile u is read from phase 4u-1 to 4u+3 and is waited for (each wave its
  // own direct loads, vmcnt) at the end of phase 4u-2; tile v is issued at
  // the start of phase 4v-11 into the stage of tile v-4, whose last reads
  // completed before the barrier ending phase 4v-13 (the barrier waits for
  // outstanding LDS reads).  Two tiles stay in flight behind the one waited
  // for.
  constexpr int kMine = kJobs;   // direct loads per wave per tile
  auto wait_tiles_after = [&](int n) __attribute__((always_inline)) {   // n = 0, 1, 2 tiles may stay in flight
    if (n >= 2) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kMine) : "memory");
    else if (n == 1) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(kMine) : "memory");
    else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  };
  auto bar = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  };
  const int grp2 = wave >> 2;   // 0 leads, 1 lags by one cluster
  // A wave whose rows are all past R (row-group padding) keeps to the
  // barrier and load schedule but skips its LDS reads and arithmetic.
  const bool active = r0 < p.R;
  if constexpr (kTokens) {
    // Token split: a wave's tile t is two clusters, V_t (P of tile t) and
    // M_t+1 (V operands and PV of tile t, then K operands and S of tile
    // t+1); wave group 1 lags group 0 by one cluster.  The operands are read
    // from LDS inside the MFMA cluster that consumes them, so none is held
    // through the softmax (a wave holds up to 48 rows).  Ring of five
    // stages: in global phase f (group g runs its cluster f - g), tile u is
    // read from phase 2u to 2u+3 and waited for at the end of phase 2u-1;
    // tile u is issued at the start of phase 2u-6 into the stage of tile
    // u-5, last read in phase 2u-7.  Two tiles stay in flight behind the
    // one waited for.
    const int h = grp2;
    if (c0 < cf) {
      const int T = cf - c0;
      for (int t = 0; t < min(3, T); ++t) issue(c0 + t);
      wait_tiles_after(min(T - 1, 2));
      __syncthreads();
      KOps ka;
      VOps va;
      Scores sc;
      bf16x8 pb[CT];
      if (grp2 == 1) {   // phase 0 (group 1's cluster "V_-1")
        if (3 < T) issue(c0 + 3);
        bar();
      }
      // M_0: S of tile 0
      if (grp2 == 0 && 3 < T) issue(c0 + 3);
      __builtin_amdgcn_sched_barrier(0);
      if (active) {
        load_k(stage_ptr(c0), h, ka);
        qk(ka, sc);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (grp2 == 1 && 1 < T) wait_tiles_after(min(2, T - 2));
      bar();
      for (int t = 0; t < T; ++t) {
        // V_t
        if (grp2 == 1 && t + 4 < T) issue(c0 + t + 4);
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
          update_max(sc);
          exp_pack(sc, pb);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (grp2 == 0 && t + 1 < T) wait_tiles_after(min(2, T - 2 - t));
        bar();
        // M_t+1
        if (grp2 == 0 && t + 4 < T) issue(c0 + t + 4);
        __builtin_amdgcn_sched_barrier(0);
        if (active) {
          // the V operands and the first half of the K operands are read
          // first (one LDS latency per cluster), the rest of K behind PV
          const uint8_t *kn = stage_ptr(c0 + min(t + 1, T - 1));
          load_v(stage_ptr(c0 + t), h, va);
          load_k(kn, h, ka, 0, KS / 2);
          __builtin_amdgcn_sched_barrier(0);
          pv(va, pb);
          __builtin_amdgcn_sched_barrier(0);
          load_k(kn, h, ka, KS / 2, KS);
          __builtin_amdgcn_sched_barrier(0);
          if (t + 1 < T) qk(ka, sc);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (grp2 == 1 && t + 2 < T) wait_tiles_after(min(2, T - 3 - t));
        bar();
      }
      if (grp2 == 0) bar();
    }
  } else if (c0 < cf) {
    const int T = cf - c0;
    for (int t = 0; t < min(3, T); ++t) issue(c0 + t);
    wait_tiles_after(min(T - 1, 2));
    __syncthreads();
    KOps ka;
    VOps va;
    Scores sc;
    bf16x8 pb[CT];
    load_k(stage_ptr(c0), 0, ka);
    if (grp2 == 1) bar();
    // M_0
    if (grp2 == 1 && 3 < T) issue(c0 + 3);
    __builtin_amdgcn_sched_barrier(0);
    if (active) load_v(stage_ptr(c0), 0, va);
    if (active) qk(ka, sc);
    bar();
    for (int t = 0; t < T; ++t) {
      const uint8_t *st = stage_ptr(c0 + t);
      const uint8_t *sn = stage_ptr(c0 + min(t + 1, T - 1));
      // V_2t: P of half 0; K operands of half 1
      if (grp2 == 0 && t + 3 < T) issue(c0 + t + 3);
      if (active) load_k(st, 1, ka);
      __builtin_amdgcn_sched_barrier(0);
      if (active) {
        update_max(sc);
        exp_pack(sc, pb);
      }
      __builtin_amdgcn_sched_barrier(0);
      if (grp2 == 1 && t + 1 < T) wait_tiles_after(min(2, T - 2 - t));
      bar();
      // M_2t+1: PV of half 0; V operands of half 1; S of half 1
      if (active) pv(va, pb);
      __builtin_amdgcn_sched_barrier(0);
      if (active) load_v(st, 1, va);
      if (active) qk(ka, sc);
      __builtin_amdgcn_sched_barrier(0);
      if (grp2 == 0 && t + 1 < T) wait_tiles_after(min(2, T - 2 - t));
      bar();
      // V_2t+1: P of half 1; K operands of half 0 of tile t+1 (after the
      // last tile these repeat tile t and the scores they give are unused)
      if (active) load_k(sn, 0, ka);
      __builtin_amdgcn_sched_barrier(0);
      if (active) {
        update_max(sc);
        exp_pack(sc, pb);
      }
      bar();
      // M_2t+2: PV of half 1; V operands and S of half 0 of tile t+1
      if (grp2 == 1 && t + 4 < T) issue(c0 + t + 4);
      __builtin_amdgcn_sched_barrier(0);
      if (active) pv(va, pb);
      __builtin_amdgcn_sched_barrier(0);
      if (active) load_v(sn, 0, va);
      if (active) qk(ka, sc);
      bar();
    }
    if (grp2 == 0) bar();
  }

  // Tiles with block keys or past the end: staged through registers, causal
  // mask applied to the scores, not pipelined (token split: each wave its
  // own half of the tile).
  for (int it = cf; it < c1; ++it) {
    uint8_t *st = stage_ptr(it);
    __syncthreads();
    stage_slow<D>(st, it * kTile, cl, total, M, p.ccap, ckb, cvb, bkb, bvb, tid, kThreads);
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < (kTokens ? 1 : 2); ++hh) {
      const int h = kTokens ? grp2 : hh;
      KOps ka;
      Scores sc;
      bf16x8 pb[CT];
      load_k(st, h, ka);
      qk(ka, sc);
      const int jb = it * kTile + 32 * h + 8 * grp;   // key index of score (t2, i): jb + 4*t2 + i
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int row_lim = cl + (r0 + 16 * ct + col) / G + 1;   // row r = i*G + g sees key j < cl + i + 1
#pragma unroll
        for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (jb + 4 * t2 + i >= row_lim) sc[ct][t2][i] = kNegInf;
      }
      VOps va;
      load_v(st, h, va);
      update_max(sc);
      exp_pack(sc, pb);
      pv(va, pb);
    }
  }

  if constexpr (kTokens) {
    // Merge the pair's states: wave w+4 leaves its reference, row sums and
    // unnormalised outputs in LDS (lane-major, per component), wave w
    // rescales both to the larger reference and stores the rows.
    constexpr int kComp = DT * 4 + 2;
    static_assert(4 * CT * kComp * 64 * 4 <= kStagesTs * L::kStage, "merge area fits the ring");
    float *xs = reinterpret_cast<float *>(lds) + (size_t)(wave & 3) * CT * kComp * 64 + lane;
    __syncthreads();   // every wave is done with the ring and the tail stages
    if (grp2 == 1) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) xs[(ct * kComp + 4 * dt + i) * 64] = o[ct][dt][i];
        xs[(ct * kComp + DT * 4) * 64] = m_run[ct];
        xs[(ct * kComp + DT * 4 + 1) * 64] = l_run[ct];
      }
    }
    __syncthreads();
    if (grp2 == 1) return;
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      const float mb = xs[(ct * kComp + DT * 4) * 64];
      const float mm = fmaxf(m_run[ct], mb);
      // weight of a state kept relative to reference m: 1 at the common
      // reference (also for padding rows, +inf in both), exp2 of a
      // non-positive number otherwise (a state still at -FLT_MAX has l = 0
      // and o = 0)
      const float wa = (m_run[ct] == mm) ? 1.f : fast_exp2((m_run[ct] - mm) * qs);
      const float wb = (mb == mm) ? 1.f : fast_exp2((mb - mm) * qs);
      l_run[ct] = l_run[ct] * wa + xs[(ct * kComp + DT * 4 + 1) * 64] * wb;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) o[ct][dt][i] = o[ct][dt][i] * wa + xs[(ct * kComp + 4 * dt + i) * 64] * wb;
      m_run[ct] = mm;
    }
  }

  const int rows = p.B * M * p.Hq;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) {
    float l = l_run[ct];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const int r = r0 + 16 * ct + col;
    if (r >= p.R) continue;
    const int i = r / G, g = r % G;
    const int orow = (b * M + i) * p.Hq + kvh * G + g;
    if (p.splits == 1) {
      const float invo = 1.f / l;   // NaN for an empty key set
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        u32x2 w = u32x2{pack_bf16x2(o[ct][dt][0] * invo, o[ct][dt][1] * invo),
                        pack_bf16x2(o[ct][dt][2] * invo, o[ct][dt][3] * invo)};
        *reinterpret_cast<u32x2 *>(p.out + (size_t)orow * D + d) = w;
      }
      if (p.out_lse && grp == 0) p.out_lse[orow] = (l > 0.f) ? (m_run[ct] * p.qk_scale + fast_log2(l)) * kLn2 : kNegInf;
    } else {
      const float inv = (l > 0.f) ? 1.f / l : 0.f;
      float *po = p.part_o + ((size_t)split * rows + orow) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int d = 16 * dt + 4 * grp;
        *reinterpret_cast<f32x4 *>(po + d) = o[ct][dt] * inv;
      }
      if (grp == 0) p.part_lse[(size_t)split * rows + orow] = (l > 0.f) ? m_run[ct] * p.qk_scale + fast_log2(l) : kNegInf;
    }
  }
}


// Eight waves, two per SIMD (waves w and w+4), in the ping-pong schedule of
// pp_rows.  A row group is 64*(CTA+CTB) packed rows: waves 0-3 take 16*CTA
// rows each, waves 4-7 the next 16*CTB each.
template <int D, int CTA, int CTB>
__global__ __launch_bounds__(512) void verify_pp(VerifyParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStages * Lds<D>::kStage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = blockIdx.y * 64 * (CTA + CTB);
  if (wave < 4) pp_rows<D, CTA, false>(p, lds, wave, rg + 16 * CTA * wave);
  else pp_rows<D, CTB, false>(p, lds, wave, rg + 64 * CTA + 16 * CTB * (wave - 4));
}

// Eight waves, two per SIMD, in the token-split schedule of pp_rows: a row
// group is 64*CT packed rows, 16*CT per SIMD, shared by its two waves.
template <int D, int CT>
__global__ __launch_bounds__(512) void verify_ts(VerifyParams p) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kStagesTs * Lds<D>::kStage];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  pp_rows<D, CT, true>(p, lds, wave, blockIdx.y * 64 * CT + 16 * CT * (wave & 3));
}

// Kernel and row split for R packed rows.  Up to 64 rows: verify_bf16 with
// four waves of one 16-row column tile.  Up to 192 rows the token-split
// kernel: 32 or 48 rows per SIMD, shared by its two waves.  Beyond that the
// row-split ping-pong kernel with 256-row groups as 32 + 32 rows per SIMD
// (two waves per SIMD cap a wave at 256 registers, i.e. 48 rows at head_dim
// 128).  The ping-pong kernels address a V row through a 32-bit byte offset,
// so a context capacity of 2^31 bytes per channel row and beyond uses
// verify_bf16 with 48-row waves.
struct VerifyShape {
  enum Kind { kFour, kTokenSplit, kRowSplit } kind;
  int CT;   // column tiles per wave (kFour, kTokenSplit)
  int rows() const { return kind == kFour ? 64 * CT : kind == kTokenSplit ? 64 * CT : 256; }
};
VerifyShape verify_shape(int R, int64_t ccap) {
  if (R <= 64) return {VerifyShape::kFour, 1};
  if ((int64_t)2 * ccap * 128 >= ((int64_t)1 << 31)) return {VerifyShape::kFour, R <= 128 ? 2 : 3};
  if (R <= 128) return {VerifyShape::kTokenSplit, 2};
  if (R <= 192) return {VerifyShape::kTokenSplit, 3};
  return {VerifyShape::kRowSplit, 2};
}

template <int D>
void launch_verify_d(const VerifyParams &p, VerifyShape sh, int row_groups, hipStream_t s) {
  dim3 grid(p.splits, row_groups, p.B * p.Hkv);
  switch (sh.kind) {
    case VerifyShape::kTokenSplit:
      if (sh.CT == 2) verify_ts<D, 2><<<grid, 512, 0, s>>>(p);
      else verify_ts<D, 3><<<grid, 512, 0, s>>>(p);
      break;
    case VerifyShape::kRowSplit: verify_pp<D, 2, 2><<<grid, 512, 0, s>>>(p); break;
    default:
      if (sh.CT == 1) verify_bf16<D, 4, 1><<<grid, 256, 0, s>>>(p);
      else if (sh.CT == 2) verify_bf16<D, 4, 2><<<grid, 256, 0, s>>>(p);
      else verify_bf16<D, 4, 3><<<grid, 256, 0, s>>>(p);
  }
}

}  // namespace

// One workgroup per CU (its LDS ring): pick the split count so that the grid
// is about one full wave of workgroups over the 256 CUs, with every split at
// least 8 tiles long.
SplitPlan plan_verify(const vc_verify_args &a) {
  SplitPlan p{1, 0};
  if (a.dtype == VC_FP32) return p;
  const int R = a.M * (a.Hq / a.Hkv);
  const VerifyShape sh = verify_shape(R, a.ccap);
  const int64_t row_groups = (R + sh.rows() - 1) / sh.rows();
  const int64_t wgs = (int64_t)a.B * a.Hkv * row_groups;
  const int64_t chunks = (a.ccap + a.M + kTile - 1) / kTile;
  int s = a.num_splits;
  if (s <= 0) {
    s = (int)((256 + wgs - 1) / wgs);
    const int64_t max_s = chunks / 8 > 0 ? chunks / 8 : 1;
    if (s > max_s) s = (int)max_s;
  }
  if (s > chunks && chunks > 0) s = (int)chunks;
  if (s < 1) s = 1;
  p.splits = s;
  if (s > 1) p.ws_bytes = (size_t)s * a.B * a.M * a.Hq * (a.D + 1) * sizeof(float);
  return p;
}

hipError_t launch_verify_f32(const vc_verify_args &a, hipStream_t s);

hipError_t launch_verify(const vc_verify_args &a, const SplitPlan &pl, hipStream_t s, hipEvent_t after_kernel) {
  if (a.dtype == VC_FP32) {
    const hipError_t e = launch_verify_f32(a, s);
    return (e != hipSuccess || !after_kernel) ? e : hipEventRecord(after_kernel, s);
  }
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
  const VerifyShape sh = verify_shape(p.R, p.ccap);
  const int row_groups = (p.R + sh.rows() - 1) / sh.rows();
  if (a.D == 128) launch_verify_d<128>(p, sh, row_groups, s);
  else launch_verify_d<64>(p, sh, row_groups, s);
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && after_kernel) e = hipEventRecord(after_kernel, s);
  if (e != hipSuccess || pl.splits == 1) return e;
  return launch_combine(p.part_o, p.part_lse, pl.splits, (int)rows, a.D, a.dtype, a.out, a.out_lse, s);
}

}  // namespace vc
