// LM head fused with the greedy choice: for every hidden row, the argmax over
// the vocabulary of h W^T, without writing the logits.
//
// "Riepilogo Tecnico: VeriCache", "Algoritmo Principale": the drafter picks
// each draft token greedily (step 1) and the verify pass takes the full-cache
// greedy prediction at every block row (steps 2-3).  Both only need the
// index of the largest logit, so the [rows][vocab] logit matrix (69 MB at
// 528 rows x 32768 fp32) never has to reach HBM.
//
// Design (gfx950):
//  * W is vocab-major [V][Dm] (a linear layer's weight) and h is [R][Dm], so
//    both MFMA operands reduce along their contiguous axis and load as 16-byte
//    vectors: logits^T tile = W_tile (A, 16 vocab x 32 k) x h_tile^T (B,
//    32 k x 16 rows) on v_mfma_f32_16x16x32_bf16, fp32 accumulation.
//  * a workgroup owns a tile of BV vocab entries x BR hidden rows and walks
//    the whole Dm axis in 32-wide k-steps through a ring of S LDS stages
//    filled by direct global->LDS loads (global_load_lds_dwordx4: no
//    registers held for prefetch).  One wave-wide load moves 1 KB (16 rows x
//    64 B, or 4 rows x 256 B when a stage spans four k-steps) into contiguous
//    LDS; which 16-byte piece a lane fetches is XOR-swizzled by row so the
//    operand reads are free of bank conflicts.
//    Each wave reads the next step's MFMA operands from LDS between the
//    current step's MFMAs.
//  * verify-sized row counts (R > 64) use 8 waves (two per SIMD, so one
//    wave's LDS reads overlap the other's MFMAs), 4 along vocab x 2 along
//    rows, each wave 64 vocab x 144 rows (36 accumulator tiles): BV = 256,
//    BR = 288.  At 528 rows x 32768 vocab that is 2 x 128 = 256 workgroups,
//    one per CU; the two row tiles of a vocab tile sit on the same XCD so W
//    leaves HBM once and the second read hits that XCD's L2.
//  * drafter-sized row counts (R <= 64) stream W once with one row tile:
//    4 waves of 32 vocab x R rows (HBM-bound).  A ring stage there spans
//    four k-steps, i.e. 256 contiguous bytes of every weight row (3 stages
//    in flight), which reads HBM faster than 64-byte pieces of more rows.
//    Verify-sized tiles keep one k-step per stage: their 34 KB stages
//    would leave a ring of only two.
//  * epilogue: each lane scans its accumulators in vocab order, lanes and
//    waves that share a row meet by shuffles and LDS, and the tile writes
//    one (max, index) pair per row; a second kernel reduces the pairs of a
//    row over the vocab tiles.  Ties go to the lowest vocab index and NaN
//    logits never win, as in the unfused argmax.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

struct Best {
  float v;
  int i;
};

struct LmParams {
  int R, Dm, V, n_vt;
  const uint16_t *h, *w;   // h [R][Dm], w [V][Dm]
  Best *part;              // [R][n_vt]
};

VC_DEVICE void better(float &bv, int &bi, float v, int i) {
  if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
}

// One 16-byte direct global->LDS load per lane with a scalar 64-bit base and
// a 32-bit per-lane byte offset: lane i's piece lands at lds_addr + 16*i.
// Completion is tracked with s_waitcnt vmcnt and a workgroup barrier.
VC_DEVICE void lds_load16(uint32_t voff, const void *sbase, uint32_t lds_addr) {
  __asm__ volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds_addr)
                   : "memory", "m0");
}

// Physical 16-byte slot of logical slot s in LDS row r when a row holds KS
// k-steps (4*KS slots of 8 k): the 16 rows one operand read touches land on
// distinct bank groups.
template <int KS>
VC_DEVICE int swz(int r, int s) {
  constexpr int kShift = KS == 1 ? 2 : (KS == 2 ? 1 : 0);
  return s ^ ((r >> kShift) & (4 * KS - 1));
}

// Tile of NV x NR 16x16 logit blocks per wave, WV x WR waves, a ring of S
// LDS stages of KS 32-wide k-steps each.
template <int NV, int NR, int WV, int WR, int S, int KS>
__global__ __launch_bounds__(WV *WR * 64) void lm_argmax(LmParams p) {
  constexpr int W = WV * WR;
  constexpr int BV = 16 * NV * WV, BR = 16 * NR * WR;
  constexpr int kRowB = 64 * KS;                            // bytes of a row in one stage
  constexpr int kRpb = 1024 / kRowB;                        // rows per 1 KB load block
  constexpr int kSlots = 4 * KS;                            // 16-byte slots per row
  constexpr int kBlkW = BV / kRpb, kBlk = kBlkW + BR / kRpb;   // 1 KB blocks per stage
  constexpr int kStage = kBlk * 1024;
  constexpr int kMine = (kBlk + W - 1) / W;                 // load slots per wave per stage
  constexpr int kMinLoads = kBlk / W;                       // loads every wave issues per stage
  static_assert(S * kStage <= 160 * 1024, "ring exceeds LDS");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[S * kStage];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, col = lane & 15, grp = lane >> 4;
  const int wv = wave % WV, wr = wave / WV;

  // Tile of this workgroup.  Workgroups are dealt round-robin to the 8 XCDs;
  // when the grid divides evenly, XCD x takes a contiguous run of tiles in
  // (vocab tile, row tile) order, so the row tiles sharing a vocab tile
  // share that XCD's L2.
  const int n_rt = (p.R + BR - 1) / BR;
  const int nb = gridDim.x;
  int t = blockIdx.x;
  if ((nb & 7) == 0) t = (t & 7) * (nb >> 3) + (t >> 3);
  const int vt = t / n_rt, rt = t % n_rt;
  const int v0 = vt * BV, r0 = rt * BR;

  // Per-lane byte offsets of this wave's load slots (fixed across stages);
  // rows past the end are clamped to the last row (loaded, never used).
  const char *wtile = reinterpret_cast<const char *>(p.w + (size_t)v0 * p.Dm);
  const char *htile = reinterpret_cast<const char *>(p.h + (size_t)r0 * p.Dm);
  uint32_t voff[kMine];
#pragma unroll
  for (int j = 0; j < kMine; ++j) {
    const int q = wave + j * W;
    const int r = kRpb * (q < kBlkW ? q : q - kBlkW) + lane / kSlots;   // row within its tile
    const int lim = q < kBlkW ? p.V - v0 : p.R - r0;
    const int rc = r < lim ? r : lim - 1;
    voff[j] = (uint32_t)(rc * p.Dm * 2 + 16 * swz<KS>(r, lane % kSlots));
  }
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t *)lds;
  const int NSt = p.Dm / (32 * KS);   // stages

  auto issue = [&](int u) __attribute__((always_inline)) {
    const uint32_t st = lds_base + (uint32_t)((u % S) * kStage);
    const char *wb = wtile + u * kRowB, *hb = htile + u * kRowB;
#pragma unroll
    for (int j = 0; j < kMine; ++j) {
      const int q = wave + j * W;
      if (q < kBlk) lds_load16(voff[j], q < kBlkW ? wb : hb, st + q * 1024);
    }
  };
  // MFMA operands of k-step kk of the stage at st.
  auto read_a = [&](const uint8_t *st, int kk, int i) __attribute__((always_inline)) {
    const int r = 16 * (wv * NV + i) + col;
    return as_bf16x8(*reinterpret_cast<const u32x4 *>(st + r * kRowB + 16 * swz<KS>(r, 4 * kk + grp)));
  };
  auto read_b = [&](const uint8_t *st, int kk, int j) __attribute__((always_inline)) {
    const int r = 16 * (wr * NR + j) + col;
    return as_bf16x8(
        *reinterpret_cast<const u32x4 *>(st + BV * kRowB + r * kRowB + 16 * swz<KS>(r, 4 * kk + grp)));
  };

  f32x4 acc[NV][NR];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int j = 0; j < NR; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Ring protocol.  The operands of each k-step are read from LDS into
  // registers during the previous k-step's MFMAs.  Stage u's last operands
  // are read while its second-to-last k-step computes, so at the top of its
  // last k-step every wave waits for stage u+1, passes a barrier, and stage
  // u+S refills u's slot.  LDS read latency thus stays off the critical
  // path: after a barrier a wave starts its MFMAs at once, and each row
  // block's MFMAs are followed by the read of that block's next operand
  // into the registers they free.
#pragma unroll
  for (int u = 0; u < S; ++u)
    if (u < NSt) issue(u);
  if (S <= NSt) __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 1) * kMinLoads) : "memory");
  else __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  bf16x8 a[NV], b[NR];
#pragma unroll
  for (int i = 0; i < NV; ++i) a[i] = read_a(lds, 0, i);
#pragma unroll
  for (int j = 0; j < NR; ++j) b[j] = read_b(lds, 0, j);

  for (int u = 0; u < NSt; ++u) {
    const uint8_t *cur = lds + (u % S) * kStage;
    // on the last stage a stale in-bounds slot whose values are never used
    const uint8_t *nxt = lds + ((u + 1) % S) * kStage;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk == KS - 1) {
        // Stage u+1 has landed once at most the later stages issued so far
        // (u+2 .. u+S-1) are outstanding (counting the fewest loads a wave
        // issues per stage only waits longer); this wave's reads of stage
        // u are complete, so after the barrier its slot may be refilled.
        if (u + S <= NSt) __asm__ volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((S - 2) * kMinLoads) : "memory");
        else __asm__ volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
        __syncthreads();
        if (u + S < NSt) issue(u + S);
      }
      const uint8_t *pst = kk == KS - 1 ? nxt : cur;
      const int pk = kk == KS - 1 ? 0 : kk + 1;
      bf16x8 na[NV], nb[NR];
#pragma unroll
      for (int i = 0; i < NV; ++i) na[i] = read_a(pst, pk, i);
#pragma unroll
      for (int j = 0; j < NR; ++j) {
#pragma unroll
        for (int i = 0; i < NV; ++i) acc[i][j] = mfma16x16x32(a[i], b[j], acc[i][j]);
        nb[j] = read_b(pst, pk, j);
      }
      // Issue order: the NV reads of na between the first row block's
      // MFMAs, then one nb read after each row block's NV MFMAs.
#pragma unroll
      for (int g = 0; g < NV; ++g) {
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int j = 1; j < NR; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, NV, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) a[i] = na[i];
#pragma unroll
      for (int j = 0; j < NR; ++j) b[j] = nb[j];
    }
  }

  // Epilogue.  acc[i][j][e] is the logit of vocab v0 + 16*(wv*NV + i) +
  // 4*grp + e at row r0 + 16*(wr*NR + j) + col.
  __syncthreads();   // the ring is reused for the cross-wave exchange
  Best *xch = reinterpret_cast<Best *>(lds);   // [BR][WV]
#pragma unroll
  for (int j = 0; j < NR; ++j) {
    float bv = kNegInf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int v = v0 + 16 * (wv * NV + i) + 4 * grp + e;
        if (v < p.V) better(bv, bi, acc[i][j][e], v);
      }
    better(bv, bi, __shfl_xor(bv, 16, 64), __shfl_xor(bi, 16, 64));
    better(bv, bi, __shfl_xor(bv, 32, 64), __shfl_xor(bi, 32, 64));
    if (grp == 0) xch[(16 * (wr * NR + j) + col) * WV + wv] = Best{bv, bi};
  }
  __syncthreads();
  for (int rr = tid; rr < BR; rr += W * 64) {
    if (r0 + rr >= p.R) break;
    float bv = kNegInf;
    int bi = 0x7fffffff;
#pragma unroll
    for (int x = 0; x < WV; ++x) better(bv, bi, xch[rr * WV + x].v, xch[rr * WV + x].i);
    p.part[(size_t)(r0 + rr) * p.n_vt + vt] = Best{bv, bi};
  }
}

// Row argmax from the per-tile pairs: one wave per row.
__global__ __launch_bounds__(256) void argmax_partials(const Best *__restrict__ part, int n_vt, int R, int V,
                                                       int *__restrict__ out, int out_stride) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= R) return;
  float bv = kNegInf;
  int bi = 0x7fffffff;
  for (int j = lane; j < n_vt; j += 64) {
    const Best b = part[(size_t)row * n_vt + j];
    better(bv, bi, b.v, b.i);
  }
  for (int o = 32; o > 0; o >>= 1) better(bv, bi, __shfl_xor(bv, o, 64), __shfl_xor(bi, o, 64));
  if (lane == 0) out[(size_t)row * out_stride] = (bi < V) ? bi : 0;
}

// Configurations: verify-sized (R > 64) and drafter-sized (R <= 64, NR row
// blocks of 16).  A stage spans KS k-steps (64*KS contiguous bytes of every
// row) when Dm allows it, else one.
constexpr int kBigNV = 4, kBigNR = 9, kBigWV = 4, kBigWR = 2, kBigS = 4;
constexpr int kSmallNV = 2, kSmallWV = 4, kSmallKS = 4, kSmallS = 3;

template <int NV, int NR, int WV, int WR, int S, int KS>
hipError_t launch_cfg(const LmParams &p0, hipStream_t s) {
  constexpr int BV = 16 * NV * WV, BR = 16 * NR * WR;
  LmParams p = p0;
  p.n_vt = (p.V + BV - 1) / BV;
  const int n_rt = (p.R + BR - 1) / BR;
  lm_argmax<NV, NR, WV, WR, S, KS><<<p.n_vt * n_rt, WV * WR * 64, 0, s>>>(p);
  return hipGetLastError();
}

template <int NR>
hipError_t launch_small(const LmParams &p, hipStream_t s) {
  if ((p.Dm / 32) % kSmallKS == 0) return launch_cfg<kSmallNV, NR, kSmallWV, 1, kSmallS, kSmallKS>(p, s);
  return launch_cfg<kSmallNV, NR, kSmallWV, 1, 8, 1>(p, s);
}

int vocab_tile(int R) { return R > 64 ? 16 * kBigNV * kBigWV : 16 * kSmallNV * kSmallWV; }

}  // namespace

size_t lm_argmax_workspace(int R, int V) {
  const int bv = vocab_tile(R);
  return (size_t)R * (((int64_t)V + bv - 1) / bv) * sizeof(Best);
}

hipError_t launch_lm_argmax(int R, int Dm, int V, const void *h, const void *w, int *out, int out_stride,
                            void *ws, hipStream_t s) {
  if (R == 0) return hipSuccess;
  LmParams p{R, Dm, V, 0, (const uint16_t *)h, (const uint16_t *)w, (Best *)ws};
  hipError_t e;
  if (R > 64) e = launch_cfg<kBigNV, kBigNR, kBigWV, kBigWR, kBigS, 1>(p, s);
  else if (R > 48) e = launch_small<4>(p, s);
  else if (R > 32) e = launch_small<3>(p, s);
  else if (R > 16) e = launch_small<2>(p, s);
  else e = launch_small<1>(p, s);
  if (e != hipSuccess) return e;
  const int bv = vocab_tile(R);
  argmax_partials<<<(R + 3) / 4, 256, 0, s>>>((const Best *)ws, (V + bv - 1) / bv, R, V, out, out_stride);
  return hipGetLastError();
}

}  // namespace vc
