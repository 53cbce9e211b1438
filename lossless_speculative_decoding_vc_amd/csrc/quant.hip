// Int4 group quantization of bf16 K/V rows into the compressed-cache format
// vc_draft_attn reads with fmt = VC_KV_INT4 (six arrays) or VC_KV_INT4_PACKED
// (one interleaved 5120-byte block per 32 tokens).
//
// "Riepilogo Tecnico: VeriCache", "Supporto Architetturale": the drafter's
// compressed cache may come from a quantizer, behind the same interface as
// eviction.  The pages fix no scheme; this library's reading is asymmetric
// min/max per group:
//   K: one group = one channel over 32 consecutive tokens,
//   V: one group = one token over 32 consecutive channels,
//   s = (max - min) / 15 and z = min, each rounded to binary16 (nearest even),
//   code c = clip(rint((x - z) / s), 0, 15) (ties to even), c = 0 if s == 0.
// Appending drafted-and-verified tokens to an int4 cache is this operation on
// each full 32-token group of the bf16 tail; building the cache from a full
// bf16 cache is the same call over all its groups.
//
// One workgroup of 256 threads per (32-token group, b, KV head): threads
// 0..127 own one K channel each (32 tokens), threads 128..255 one (token, V
// channel group) pair.  The bf16 tiles arrive in LDS through 16-byte loads;
// codes meet in LDS and leave as 32-bit words of eight.
// The code decision is taken in fp32 and re-taken in fp64 when the quotient
// lies within 1e-5 of a rounding tie (the fp32 quotient is within 2^-19 of
// the exact one for |q| <= 16 when taken with one reciprocal per group), so
// every code equals the one an exact
// evaluation gives.  Scales and zeros are rounded from fp64 to binary16 in
// one step.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kGroup = 32;

// fp64 -> binary16, round to nearest even, in one rounding step (the
// hardware path goes through fp32 and could round twice).
VC_DEVICE uint16_t f64_to_f16_rne(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int ex = (int)((b >> 52) & 0x7FF);
  const uint64_t man = b & ((1ull << 52) - 1);
  if (ex == 0x7FF) return sign | 0x7C00u | (man ? 0x200u : 0u);   // inf / nan
  if (ex == 0) return sign;                                         // fp64 subnormal: far below fp16
  const int e = ex - 1023;
  const uint64_t full = (1ull << 52) | man;
  if (e >= -14) {                                                   // normal fp16 range (or overflow)
    uint32_t m = (uint32_t)(man >> 42);
    const uint64_t rem = man & ((1ull << 42) - 1), half = 1ull << 41;
    int he = e + 15;
    if (rem > half || (rem == half && (m & 1u))) ++m;
    if (m == 1024u) { m = 0; ++he; }
    if (he >= 31) return sign | 0x7C00u;
    return sign | (uint16_t)(he << 10) | (uint16_t)m;
  }
  const int shift = 28 - e;                                         // subnormal fp16: units of 2^-24
  if (shift >= 64) return sign;
  uint32_t m = (uint32_t)(full >> shift);
  const uint64_t rem = full & ((1ull << shift) - 1), half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1u))) ++m;                 // m == 1024 is the smallest normal
  return sign | (uint16_t)m;
}

// clip(rint((x - z) / s), 0, 15) for x, z, s exact in fp32, rs = rcp(s).
// (x - z) * rs is within 3 ulp of the exact quotient, i.e. within 3e-6 for
// |q| <= 16; when it lies within 1e-5 of a tie the code is decided in fp64.
VC_DEVICE uint32_t code_of(float x, float z, float s, float rs) {
  const float q = (x - z) * rs;
  float r = rintf(q);
  if (fabsf(q - r) > 0.5f - 1e-5f) r = (float)rint(((double)x - (double)z) / (double)s);
  r = fminf(fmaxf(r, 0.f), 15.f);
  return (s > 0.f) ? (uint32_t)r : 0u;
}

// Word of eight codes c0..c7: c_2j in bits 4j..4j+3, c_2j+1 in 16+4j..16+4j+3.
VC_DEVICE uint32_t pack8(const uint8_t *c) {
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) w |= ((uint32_t)c[2 * j] << (4 * j)) | ((uint32_t)c[2 * j + 1] << (16 + 4 * j));
  return w;
}

template <int D>
__global__ __launch_bounds__(256) void quantize_int4(QuantParams p) {
  static_assert(D == 128, "int4 cache is compiled for head_dim 128");
  __shared__ __attribute__((aligned(16))) uint16_t ktile[kGroup][D];   // [token][channel]
  __shared__ __attribute__((aligned(16))) uint16_t vtile[D][kGroup];   // [channel][token]
  __shared__ uint8_t kcode[kGroup][D];
  __shared__ uint8_t vcode[D][kGroup];
  // each XCD runs a contiguous run of groups, so the two groups whose V runs
  // share a 128-byte line read it through one L2
  int grp, bh;
  xcd_order(grp, bh);
  const int tid = threadIdx.x;
  int s0, d0;
  int64_t span;   // tokens of the whole call per (b, KV head)
  if (p.tail_len) {
    // tail mode: the full groups of the slice's tail once n_add rows are appended
    const int b = bh / p.Hkv;
    const int g = tail_total(p.tail_len[b], p.n_add[b], p.M, p.src_cap) / kGroup;
    if (grp >= g) return;
    s0 = 0;
    d0 = p.dst_start[bh];
    span = (int64_t)g * kGroup;
  } else {
    s0 = p.src_start[bh];
    d0 = p.dst_start[bh];
    span = (int64_t)gridDim.x * kGroup;
  }
  // every workgroup of a (b, KV head) sees the same starts, so a slice whose
  // call would leave the source or the cache is skipped as a whole
  if (s0 < 0 || d0 < 0 || (d0 % kGroup) != 0 || s0 + span > p.src_cap || d0 + span > p.cap) return;
  const int64_t st = (int64_t)s0 + (int64_t)grp * kGroup, dt = (int64_t)d0 + (int64_t)grp * kGroup;
  const int64_t blk = dt / kGroup;
  const size_t gblk = (size_t)bh * (p.cap / kGroup) + blk;   // block index over all slices

  // The K tile is 8 KB contiguous and read in 16-byte pieces; the V tile is
  // 128 channel runs of 64 B, read in 16-byte pieces when the first token and
  // the channel stride are multiples of 8 (else element by element).
  const uint16_t *sk = p.src_k + ((size_t)bh * p.src_cap + st) * D;
  const uint16_t *sv = p.src_v + (size_t)bh * D * p.src_cap + st;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = 8 * (tid + 256 * i);   // element of the K tile
    *reinterpret_cast<u32x4 *>(&ktile[e / D][e % D]) = *reinterpret_cast<const u32x4 *>(sk + e);
  }
  if (((st | p.src_cap) & 7) == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int e = tid + 256 * i, d = e / 4, c = e % 4;   // channel d, 8-token piece c
      *reinterpret_cast<u32x4 *>(&vtile[d][8 * c]) = *reinterpret_cast<const u32x4 *>(sv + (size_t)d * p.src_cap + 8 * c);
    }
  } else {
    for (int e = tid; e < D * kGroup; e += 256) vtile[e / kGroup][e % kGroup] = sv[(size_t)(e / kGroup) * p.src_cap + e % kGroup];
  }
  __syncthreads();

  if (tid < D) {
    // K channel tid over the group's 32 tokens
    const int d = tid;
    float x[kGroup];
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int t = 0; t < kGroup; ++t) {
      x[t] = bf16_to_f32(ktile[t][d]);
      mn = fminf(mn, x[t]);
      mx = fmaxf(mx, x[t]);
    }
    const uint16_t s16 = f64_to_f16_rne(((double)mx - (double)mn) / 15.0), z16 = f64_to_f16_rne((double)mn);
    const float s = f16_to_f32(s16), z = f16_to_f32(z16), rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int t = 0; t < kGroup; ++t) kcode[t][d] = (uint8_t)code_of(x[t], z, s, rs);
    const size_t o = gblk * p.par_bs + 2 * d;   // bytes
    *reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(p.k_scale) + o) = s16;
    *reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(p.k_zero) + o) = z16;
  } else {
    // V token t, channel group g
    const int t = (tid - D) % kGroup, g = (tid - D) / kGroup;
    float x[kGroup];
    float mn = __builtin_huge_valf(), mx = -__builtin_huge_valf();
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      x[j] = bf16_to_f32(vtile[kGroup * g + j][t]);
      mn = fminf(mn, x[j]);
      mx = fmaxf(mx, x[j]);
    }
    const uint16_t s16 = f64_to_f16_rne(((double)mx - (double)mn) / 15.0), z16 = f64_to_f16_rne((double)mn);
    const float s = f16_to_f32(s16), z = f16_to_f32(z16), rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int j = 0; j < kGroup; ++j) vcode[kGroup * g + j][t] = (uint8_t)code_of(x[j], z, s, rs);
    const size_t o = gblk * p.par_bs + 2 * (g * kGroup + t);   // bytes
    *reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(p.v_scale) + o) = s16;
    *reinterpret_cast<uint16_t *>(reinterpret_cast<uint8_t *>(p.v_zero) + o) = z16;
  }
  __syncthreads();
  // K codes: token row t of the group, D/8 words; V codes: channel d's 32 tokens, 4 words
  uint32_t *kq = reinterpret_cast<uint32_t *>(p.k_codes + gblk * p.code_bs);
  uint32_t *vq = reinterpret_cast<uint32_t *>(p.v_codes + gblk * p.code_bs);
  for (int w = tid; w < kGroup * D / 8; w += 256) {
    const int t = w / (D / 8), c = w % (D / 8);
    kq[w] = pack8(&kcode[t][8 * c]);
    vq[w] = pack8(&vcode[w / 4][8 * (w % 4)]);
  }
}

}  // namespace

hipError_t launch_quantize_int4(const QuantParams &p, int n_groups, hipStream_t s) {
  if (n_groups == 0 || p.BH == 0) return hipSuccess;
  quantize_int4<128><<<dim3(n_groups, p.BH), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vc
