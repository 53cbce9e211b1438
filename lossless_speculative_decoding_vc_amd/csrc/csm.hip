// One clustering round of Chunked Soft Matching over the compressed cache.
//
// "Riassunto Tecnico: CentroidKV", "Componenti Chiave": attention sinks and
// recent tokens stay out of the partition (item 2); the rest is cut into
// chunks, each chunk's tokens are split alternately into sets A and B, each
// token is paired with a highly similar token of the other set, the pairs are
// ranked by similarity and only the top fraction r is merged (item 3); the
// similarity is the cosine of the key states (item 1); a cluster's key and
// value are the degree-weighted mean of its members and its degree their sum
// (item 4).  Readings where the page is silent: A = even positions of the
// chunk, B = odd; an A token's match is the B token of its chunk with the
// largest key cosine (lowest index on equal values); the floor(r |A|) A
// tokens with the largest cosine (lower index first on equal values) merge;
// survivors keep ascending position.
//
// Layouts are those of vc_draft_attn's dense main segment: K [cap][D]
// token-major, V in 32-token blocks [cap/32][D][32], degrees [cap] (fp32, one
// row per KV head), so rounds compose and the output feeds the drafter.
//
// One workgroup of 256 threads per (chunk, b, KV head), plus two per (b, KV
// head) that copy the sinks and the recent tokens; chunks up to 64 tokens use
// a 40 KB LDS footprint, up to 128 an 89 KB one.  A chunk's keys and values
// are staged in LDS (bf16).  The |A| x |B| key dot products run on MFMA
// (exact bf16 products, fp32 sums) and scaled by the inverse fp32 norms; each A
// token's argmax and rank come from eight lanes and a shuffle reduction; a B
// token's members are one ballot (a bit mask over the A tokens).  Each
// survivor is written once, by one wave with lane = channel pair, so member
// loops never diverge within a wave: unmerged tokens bit-exactly, clusters as
// the fp32 degree-weighted mean rounded to bf16, V through an LDS tile
// [channel][survivor] so the blocked writes coalesce.  Every chunk before the
// last is full, so a chunk's output offset follows from its index alone.
#include "common.h"
#include "launch.h"

namespace vc {
namespace {

constexpr int kD = 128;

VC_DEVICE float dot8(const u32x4 &a, const u32x4 &b, float acc) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = fmaf(bf16_lo(a[j]), bf16_lo(b[j]), acc);
    acc = fmaf(bf16_hi(a[j]), bf16_hi(b[j]), acc);
  }
  return acc;
}

template <int kMaxChunk>
__global__ __launch_bounds__(256) void csm_round_kernel(CsmParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t ks[kMaxChunk][kD + 8];   // rows padded by 16 B: lanes reading different rows spread over the banks
  // channel-major, as in the source; rows padded by 8 bytes so that lanes reading one token of 64 different
  // channels spread over the banks
  __shared__ __attribute__((aligned(16))) uint16_t vs[kD][kMaxChunk + 4];
  __shared__ float dg[kMaxChunk];
  __shared__ __attribute__((aligned(16))) float sim[kMaxChunk / 2][kMaxChunk / 2];
  __shared__ float score[kMaxChunk / 2];
  __shared__ int match[kMaxChunk / 2], mergedA[kMaxChunk / 2];
  __shared__ int surv[kMaxChunk];
  __shared__ unsigned long long amask[kMaxChunk / 2];   // B token j: bit i set iff A token i merges into it
  // each XCD runs a contiguous run of chunks, so the 32-token V blocks two
  // neighbouring chunks share are fetched and written through one L2
  const int tid = threadIdx.x;
  const int nchunks = (int)gridDim.x - 2;
  int bh, c;
  xcd_order(c, bh);
  c -= 1;   // -1: sinks, nchunks: recent tokens
  const uint16_t *ik = p.in_k + (size_t)bh * p.cap_in * kD;
  const uint16_t *iv = p.in_v + (size_t)bh * p.cap_in * kD;
  const float *idg = p.in_deg ? p.in_deg + (size_t)bh * p.cap_in : nullptr;
  uint16_t *ok = p.out_k + (size_t)bh * p.cap_out * kD;
  uint16_t *ov = p.out_v + (size_t)bh * p.cap_out * kD;
  float *odg = p.out_deg + (size_t)bh * p.cap_out;
  auto vidx = [](int64_t t, int d) { return (size_t)(t >> 5) * kD * 32 + (size_t)d * 32 + (t & 31); };

  if (c < 0 || c >= nchunks) {
    if (c < 0 && tid == 0 && p.out_len) p.out_len[bh] = p.n_out;
    // pass-through of the sinks (to the front) or the recent tokens (to the end)
    const int n = c < 0 ? p.n_sink : p.n_recent;
    const int64_t src0 = c < 0 ? 0 : p.n_in - p.n_recent, dst0 = c < 0 ? 0 : p.n_out - p.n_recent;
    for (int e = tid; e < n * (kD / 8); e += 256) {   // K rows in 16-byte pieces
      const int t = e / (kD / 8), q = e % (kD / 8);
      *reinterpret_cast<u32x4 *>(ok + (size_t)(dst0 + t) * kD + 8 * q) =
          *reinterpret_cast<const u32x4 *>(ik + (size_t)(src0 + t) * kD + 8 * q);
    }
    for (int d = 0; d < kD; ++d)                      // V: consecutive lanes, consecutive tokens
      for (int t = tid; t < n; t += 256) ov[vidx(dst0 + t, d)] = iv[vidx(src0 + t, d)];
    for (int t = tid; t < n; t += 256) odg[dst0 + t] = idg ? idg[src0 + t] : 1.f;
    return;
  }

  const int64_t s0 = (int64_t)p.n_sink + (int64_t)c * p.chunk;
  const int L = (int)min((int64_t)p.chunk, p.n_in - p.n_recent - s0);
  const int nA = (L + 1) / 2, nB = L / 2;
  const int m = nB > 0 ? (int)floor(p.r * nA) : 0;
  const int m_full = (int)floor(p.r * ((p.chunk + 1) / 2));
  const int64_t base = (int64_t)p.n_sink + (int64_t)c * (p.chunk - m_full);   // earlier chunks are full

  // stage the chunk: every load of a thread is issued before any of them is
  // written to LDS (compile-time trip counts, predicated on the chunk length),
  // so the loads overlap instead of each waiting for its own round trip.
  // K rows in 16-byte pieces; V in 8-byte pieces of four tokens (which never
  // straddle a 32-token block) when the chunk starts on a multiple of 4.
  {
    constexpr int KP = kMaxChunk * (kD / 8) / 256;   // K pieces per thread
    u32x4 kr[KP];
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int e = tid + 256 * j, t = e / (kD / 8), q = e % (kD / 8);
      kr[j] = t < L ? *reinterpret_cast<const u32x4 *>(ik + (size_t)(s0 + t) * kD + 8 * q) : u32x4{0, 0, 0, 0};
    }
    if ((s0 & 3) == 0) {
      constexpr int G4 = kMaxChunk / 4, VP = kD / (256 / G4);   // 4-token groups per channel, pieces per thread
      const int g = tid % G4, t = 4 * g;
      u32x2 vr[VP];
#pragma unroll
      for (int j = 0; j < VP; ++j) {
        const int d = tid / G4 + (256 / G4) * j;
        vr[j] = t + 3 < L ? *reinterpret_cast<const u32x2 *>(iv + vidx(s0 + t, d)) : u32x2{0, 0};
      }
#pragma unroll
      for (int j = 0; j < VP; ++j) {
        const int d = tid / G4 + (256 / G4) * j;
        if (t + 3 < L) *reinterpret_cast<u32x2 *>(&vs[d][t]) = vr[j];
        else
          for (int u = t; u < L; ++u) vs[d][u] = iv[vidx(s0 + u, d)];
      }
    } else {
      for (int e = tid; e < L * kD; e += 256) {
        const int d = e / L, t = e % L;
        vs[d][t] = iv[vidx(s0 + t, d)];
      }
    }
#pragma unroll
    for (int j = 0; j < KP; ++j) {
      const int e = tid + 256 * j, t = e / (kD / 8), q = e % (kD / 8);
      if (t < L) *reinterpret_cast<u32x4 *>(&ks[t][8 * q]) = kr[j];
    }
  }
  for (int t = tid; t < L; t += 256) dg[t] = idg ? idg[s0 + t] : 1.f;
  __syncthreads();
  // cosines of A token i (position 2i) with B token j (position 2j+1): the
  // dot products as 16x16 tiles of v_mfma_f32_16x16x32_bf16 (bf16 products
  // are exact in its fp32 accumulation) times the two inverse norms, one tile
  // per wave in turn; rows past nA / nB read row 0 and are not stored.  The
  // norms come from the same operand registers: lane (col, grp) holds a
  // quarter of row col's channels over the four k-steps, the four quarters
  // meet by two shuffles (in a fixed order).
  {
    const int wave = tid >> 6, lane = tid & 63, col = lane & 15, grp = lane >> 4;
    const int tA = (nA + 15) / 16, tB = (nB + 15) / 16;
    for (int tile = wave; tile < tA * tB; tile += 4) {
      const int ti = tile / tB, tj = tile % tB;
      const int ia = 16 * ti + col, jb = 16 * tj + col;
      const int ra = ia < nA ? 2 * ia : 0, rb = jb < nB ? 2 * jb + 1 : 0;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      float na = 0.f, nb = 0.f;
#pragma unroll
      for (int k = 0; k < kD / 32; ++k) {
        const u32x4 a = *reinterpret_cast<const u32x4 *>(&ks[ra][32 * k + 8 * grp]);
        const u32x4 b = *reinterpret_cast<const u32x4 *>(&ks[rb][32 * k + 8 * grp]);
        acc = mfma16x16x32(as_bf16x8(a), as_bf16x8(b), acc);
        na = dot8(a, a, na);
        nb = dot8(b, b, nb);
      }
      na += __shfl_xor(na, 16, 64);
      na += __shfl_xor(na, 32, 64);
      nb += __shfl_xor(nb, 16, 64);
      nb += __shfl_xor(nb, 32, 64);
      const float rna = 1.f / sqrtf(na), rnb = 1.f / sqrtf(nb);   // rows ia and jb
      // lane holds S[16 ti + 4 grp + i][16 tj + col]
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int ii = 16 * ti + 4 * grp + i, jj = 16 * tj + col;
        const float ra_i = __shfl(rna, 4 * grp + i, 64);   // inverse norm of A row 4 grp + i of the tile
        if (ii < nA && jj < nB) sim[ii][jj] = acc[i] * (ra_i * rnb);
      }
    }
  }
  __syncthreads();
  // argmax (lowest B index on equal values) and rank of every A token, eight
  // lanes per A token and a shuffle reduction
  for (int base_i = 0; base_i < nA; base_i += 32) {
    const int i = base_i + (tid >> 3), sub = tid & 7;
    float bs = -2.f;
    int best = 0x7fffffff;
    if (i < nA)
      for (int j = sub; j < nB; j += 8)
        if (sim[i][j] > bs) { bs = sim[i][j]; best = j; }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float ob = __shfl_xor(bs, o, 64);
      const int oj = __shfl_xor(best, o, 64);
      if (ob > bs || (ob == bs && oj < best)) { bs = ob; best = oj; }
    }
    if (i < nA && sub == 0) {
      match[i] = nB > 0 ? best : 0;
      score[i] = bs;
    }
  }
  __syncthreads();
  for (int base_i = 0; base_i < nA; base_i += 32) {
    const int i = base_i + (tid >> 3), sub = tid & 7;
    int rank = 0;
    if (i < nA) {
      const float si = score[i];
      for (int k = sub; k < nA; k += 8) rank += (score[k] > si) || (score[k] == si && k < i);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) rank += __shfl_xor(rank, o, 64);
    if (i < nA && sub == 0) mergedA[i] = rank < m;
  }
  __syncthreads();
  // survivors (B tokens and unmerged A tokens) in position order: surv[k] is
  // the chunk position of output slot base + k; amask[j] holds the A tokens
  // merged into B token j.  Every wave takes the merge flags of all A tokens
  // (at most 64) as one ballot, so a survivor's slot is a popcount.
  {
    const int wave = tid >> 6, lane = tid & 63;
    const bool mg = lane < nA && mergedA[lane];
    const unsigned long long mm = __ballot(mg);
    if (tid < L) {
      const int t = tid;
      if ((t & 1) || !((mm >> (t >> 1)) & 1ull)) {
        const int na_below = (t + 1) >> 1;   // A tokens at positions below t
        const unsigned long long msk = na_below >= 64 ? ~0ull : ((1ull << na_below) - 1);
        surv[t - __popcll(mm & msk)] = t;
      }
    }
    // members of each B token as a bit mask over the A tokens (ascending bit = ascending position): one
    // ballot per B token, the B tokens dealt round-robin to the four waves
    const int mt = lane < nA ? match[lane] : -1;
    for (int j = wave; j < nB; j += 4) {
      const unsigned long long bal = __ballot(mg && mt == j);
      if (lane == 0) amask[j] = bal;
    }
  }
  __syncthreads();
  const int ns = L - m;
  // Output: survivor k (chunk position surv[k]) goes to slot base + k.  A
  // cluster (a B token with merged A tokens) is its own degree-weighted value
  // plus its members' in ascending position, times the inverse total degree;
  // other survivors are copied bit-exactly.  The K rows go first, 16 lanes per
  // survivor (16-byte pieces), 16 survivors at a time; lane 0 of a survivor
  // also keeps its member mask and inverse degree for the V pass (in the
  // similarity matrix's space, no longer read) and writes its degree.
  static_assert(sizeof(sim) >= kMaxChunk * (sizeof(unsigned long long) + sizeof(float)), "per-survivor data fits");
  unsigned long long *smask = reinterpret_cast<unsigned long long *>(&sim[0][0]);
  float *sinv = reinterpret_cast<float *>(smask + kMaxChunk);
  for (int k = tid >> 4; k < ns; k += 16) {
    const int t = surv[k], q = tid & 15;
    const unsigned long long mk = (t & 1) ? amask[t >> 1] : 0ull;
    const u32x4 xt = *reinterpret_cast<const u32x4 *>(&ks[t][8 * q]);
    u32x4 *dst = reinterpret_cast<u32x4 *>(ok + (size_t)(base + k) * kD + 8 * q);
    const float dt = dg[t];
    if (!mk) {
      *dst = xt;
      if (q == 0) {
        smask[k] = 0ull;
        odg[base + k] = dt;
      }
      continue;
    }
    float w = dt, acc[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] = dt * bf16_lo(xt[j]);
      acc[2 * j + 1] = dt * bf16_hi(xt[j]);
    }
    for (unsigned long long b = mk; b; b &= b - 1) {
      const int a2 = 2 * __builtin_ctzll(b);
      const u32x4 xa = *reinterpret_cast<const u32x4 *>(&ks[a2][8 * q]);
      const float wa = dg[a2];
      w += wa;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = fmaf(wa, bf16_lo(xa[j]), acc[2 * j]);
        acc[2 * j + 1] = fmaf(wa, bf16_hi(xa[j]), acc[2 * j + 1]);
      }
    }
    const float inv = 1.f / w;
    u32x4 kw;
#pragma unroll
    for (int j = 0; j < 4; ++j) kw[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
    *dst = kw;
    if (q == 0) {
      smask[k] = mk;
      sinv[k] = inv;
      odg[base + k] = w;
    }
  }
  __syncthreads();
  // V: the output tile [channel][survivor] is formed in LDS (over the key
  // buffer, no longer read), each wave on whole survivors (uniform member
  // loops within a wave); it then leaves in pieces of four consecutive tokens (8 bytes, never straddling a
  // 32-token block) when the first output slot is a multiple of 4, else
  // element by element.
  static_assert(sizeof(ks) >= sizeof(uint16_t) * kD * (kMaxChunk + 4), "V tile fits over the key buffer");
  uint16_t (*vo)[kMaxChunk + 4] = reinterpret_cast<uint16_t (*)[kMaxChunk + 4]>(&ks[0][0]);
  {
    // lane = channel pair (d, d + 64), wave w takes survivors w, w + 4, ...
    const int lane = tid & 63;
    for (int k = tid >> 6; k < ns; k += 4) {
      const int t = surv[k];
      const unsigned long long mk = smask[k];
      uint16_t v0 = vs[lane][t], v1 = vs[lane + 64][t];
      if (mk) {
        const float dt = dg[t];
        float acc0 = dt * bf16_to_f32(v0), acc1 = dt * bf16_to_f32(v1);
        for (unsigned long long b = mk; b; b &= b - 1) {
          const int a2 = 2 * __builtin_ctzll(b);
          const float wa = dg[a2];
          acc0 = fmaf(wa, bf16_to_f32(vs[lane][a2]), acc0);
          acc1 = fmaf(wa, bf16_to_f32(vs[lane + 64][a2]), acc1);
        }
        const float inv = sinv[k];
        v0 = f32_to_bf16(acc0 * inv);
        v1 = f32_to_bf16(acc1 * inv);
      }
      vo[lane][k] = v0;
      vo[lane + 64][k] = v1;
    }
  }
  __syncthreads();
  if ((base & 3) == 0) {
    constexpr int G4 = kMaxChunk / 4, CPP = 256 / G4;   // 4-token groups per channel, channels per pass
    const int g = tid % G4;
    if (4 * g < ns)
      for (int d = tid / G4; d < kD; d += CPP) {
        if (4 * g + 3 < ns) {
          *reinterpret_cast<u32x2 *>(ov + vidx(base + 4 * g, d)) = *reinterpret_cast<const u32x2 *>(&vo[d][4 * g]);
        } else {
          for (int u = 4 * g; u < ns; ++u) ov[vidx(base + u, d)] = vo[d][u];
        }
      }
  } else {
    for (int k0 = 0; k0 < ns; k0 += 64) {
      const int k = k0 + (tid & 63);
      if (k < ns)
        for (int d = tid >> 6; d < kD; d += 4) ov[vidx(base + k, d)] = vo[d][k];
    }
  }
}

}  // namespace

int csm_survivors(int n_in, int n_sink, int n_recent, int chunk, double r) {
  int out = n_in;
  for (int64_t s = n_sink; s < (int64_t)n_in - n_recent; s += chunk) {
    const int L = (int)std::min<int64_t>(chunk, (int64_t)n_in - n_recent - s);
    if (L > 1) out -= (int)floor((double)r * ((L + 1) / 2));
  }
  return out;
}

hipError_t launch_csm_round(const CsmParams &p, int BH, hipStream_t s) {
  const int mid = p.n_in - p.n_recent - p.n_sink;
  const int nchunks = mid > 0 ? (mid + p.chunk - 1) / p.chunk : 0;
  if (BH == 0) return hipSuccess;
  if (p.chunk <= 64) csm_round_kernel<64><<<dim3(nchunks + 2, BH), 256, 0, s>>>(p);
  else csm_round_kernel<128><<<dim3(nchunks + 2, BH), 256, 0, s>>>(p);
  return hipGetLastError();
}

}  // namespace vc
