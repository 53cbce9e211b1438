// A small fp32 decoder run entirely on the GPU (support for end-to-end
// checks of the draft-then-verify loop; see include/vc_tiny.h).
//
// A forward is twelve launches for two layers: the embedding gather, then
// per layer five fused kernels -- RMSNorm + QKV projection + RoPE + scatter
// of K/V into the block (verify) or draft tail, attention through the
// library's fp32 path, output projection + residual, RMSNorm + gate/up
// projections + SwiGLU, down projection + residual -- and RMSNorm + the LM
// head.  The row counts are 1 (a draft step) to k + 1 (a verify block), so a
// projection is a few hundred KB of weights read by a few workgroups: each
// workgroup takes a 64- or 128-column slice, splits the reduction over 16
// waves that each keep their weight loads in flight together, and sums the
// 16 partials in a fixed order.  Positions can come from device memory (the
// committed length), so a whole round can be replayed from a graph.
#include <cmath>

#include "../../include/vc_tiny.h"
#include "common.h"
#include "launch.h"

namespace vc {

hipError_t launch_draft_f32(const vc_draft_args &a, hipStream_t s);
hipError_t launch_verify_f32(const vc_verify_args &a, hipStream_t s);

namespace {

constexpr int kRT = 8;                  // rows per workgroup
constexpr int kPW = 16;                 // waves splitting the reduction
constexpr int kPT = 64 * kPW;           // threads per projection workgroup
constexpr int kMaxK = 4096;             // largest reduction length (ffn)
constexpr int kXsFloats = kRT * 1024;   // LDS rows of X (K <= 1024 per LDS tile pass)

__global__ __launch_bounds__(256) void embed_rows(const float *__restrict__ emb, const int32_t *__restrict__ tok,
                                                  int vocab, int dm, float *__restrict__ h, int32_t *tail_len,
                                                  int tail_val) {
  const int r = blockIdx.x;
  int t = tok[r];
  t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
  for (int i = threadIdx.x; i < dm; i += blockDim.x) h[(size_t)r * dm + i] = emb[(size_t)t * dm + i];
  if (tail_len && r == 0 && threadIdx.x == 0) *tail_len = tail_val;
}

enum Epi { kPlain = 0, kSwiglu = 1, kQkvRope = 2 };

struct ProjParams {
  const float *X;          // [R][K]
  int R, K, norm;          // norm: RMSNorm (unit gain) each X row first
  float eps;
  const float *W[2];       // [K][ldw] each (W[1]: the up projection of SwiGLU)
  int ldw, N;              // N output columns
  const float *Res;        // plain: Y = X W (+ Res), Res may alias Y
  float *Y;                // [R][N]
  // QKV + RoPE: workgroup x < Hq is q head x, then Hkv k heads, then Hkv v heads
  const float *wq, *wk, *wv;
  int Hq, Hkv, D;
  const float *cs, *sn;    // RoPE table [rope_rows][D/2]
  int rope_rows;
  const int32_t *pos_base; // optional device [1]
  int pos0;                // position of row r: (pos_base ? *pos_base : 0) + pos0 + r
  float *q_out;            // [R][Hq][D]
  float *kd, *vd;          // K [Hkv] x krow_stride_h, rows row_base + r; V [Hkv] x vcol_stride_h, [D][vrow_stride]
  int64_t krow_stride_h, vcol_stride_h, vrow_stride;
  int row_base;
};

// One workgroup: rows r0 .. r0 + rows - 1, columns col0 + lane + 64 e (e < E) of
// X W[m] for m < NMAT; the reduction over K is split in kPW contiguous
// ranges (one per wave) whose partial sums are added in wave order.
template <int E, int NMAT, int EPI>
__global__ __launch_bounds__(kPT) void proj(ProjParams p) {
  __shared__ float xs[kXsFloats];
  __shared__ float part[NMAT][kPW][kRT][64 * E];
  __shared__ float inv_rms[kRT];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r0 = blockIdx.y * kRT;
  const int rows = min(kRT, p.R - r0);
  const int K = p.K;

  // the workgroup's weight slice
  const float *W0, *W1 = nullptr;
  int ldw, col0, ncols;
  int head = 0, kind = 0;   // QKV: 0 q, 1 k, 2 v
  if constexpr (EPI == kQkvRope) {
    const int x = blockIdx.x;
    kind = x < p.Hq ? 0 : (x < p.Hq + p.Hkv ? 1 : 2);
    head = kind == 0 ? x : (kind == 1 ? x - p.Hq : x - p.Hq - p.Hkv);
    W0 = kind == 0 ? p.wq : (kind == 1 ? p.wk : p.wv);
    ldw = (kind == 0 ? p.Hq : p.Hkv) * p.D;
    col0 = head * p.D;
    ncols = col0 + p.D;
  } else {
    W0 = p.W[0];
    W1 = p.W[1];
    ldw = p.ldw;
    col0 = blockIdx.x * 64 * E;
    ncols = p.N;
  }

  float acc[NMAT][E][kRT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int r = 0; r < kRT; ++r) acc[m][e][r] = 0.f;

  // The reduction runs over LDS tiles of at most 1024 columns of X.
  for (int kt = 0; kt < K; kt += 1024) {
    const int kl = min(1024, K - kt);
    __syncthreads();
    for (int i = tid; i < rows * kl; i += kPT) {
      const int r = i / kl, c = i - r * kl;
      xs[r * kl + c] = p.X[(size_t)(r0 + r) * K + kt + c];
    }
    if (p.norm && kt == 0) {
      // RMSNorm needs the whole row: K <= 1024 when norm is set (host-checked)
      __syncthreads();
      if (w < rows) {
        float ss = 0.f;
        for (int i = lane; i < K; i += 64) ss = fmaf(xs[w * kl + i], xs[w * kl + i], ss);
        ss = wave_sum(ss);
        if (lane == 0) inv_rms[w] = 1.0f / sqrtf(ss / (float)K + p.eps);
      }
      __syncthreads();
      for (int i = tid; i < rows * kl; i += kPT) xs[i] *= inv_rms[i / kl];
    }
    __syncthreads();
    const int per = (kl + kPW - 1) / kPW;
    const int k0 = w * per, k1 = min(kl, k0 + per);
#pragma unroll 16
    for (int k = k0; k < k1; ++k) {
      float wv[NMAT][E];
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int c = col0 + lane + 64 * e;
        const bool ok = c < ncols;
        wv[0][e] = ok ? W0[(size_t)(kt + k) * ldw + c] : 0.f;
        if constexpr (NMAT == 2) wv[1][e] = ok ? W1[(size_t)(kt + k) * ldw + c] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < kRT; ++r) {
        if (r < rows) {
          const float x = xs[r * kl + k];
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int e = 0; e < E; ++e) acc[m][e][r] = fmaf(x, wv[m][e], acc[m][e][r]);
        }
      }
    }
  }
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e)
#pragma unroll
      for (int r = 0; r < kRT; ++r)
        if (r < rows) part[m][w][r][lane + 64 * e] = acc[m][e][r];
  __syncthreads();

  constexpr int TW = 64 * E;
  float *outs = xs;   // [kRT][TW]: the summed tile (QKV epilogue)
  for (int i = tid; i < rows * TW; i += kPT) {
    const int r = i / TW, cc = i - r * TW;
    float s0 = 0.f, s1 = 0.f;
    for (int ww = 0; ww < kPW; ++ww) {
      s0 += part[0][ww][r][cc];
      if constexpr (NMAT == 2) s1 += part[NMAT - 1][ww][r][cc];
    }
    const int c = col0 + cc;
    if constexpr (EPI == kPlain) {
      if (c < ncols) {
        const size_t o = (size_t)(r0 + r) * p.N + c;
        p.Y[o] = p.Res ? p.Res[o] + s0 : s0;
      }
    } else if constexpr (EPI == kSwiglu) {
      if (c < ncols) p.Y[(size_t)(r0 + r) * p.N + c] = s0 / (1.0f + expf(-s0)) * s1;
    } else {
      outs[r * TW + cc] = s0;
    }
  }
  if constexpr (EPI == kQkvRope) {
    __syncthreads();
    const int D = p.D, half = D / 2;
    const int base = p.pos_base ? *p.pos_base : 0;
    for (int i = tid; i < rows * D; i += kPT) {
      const int r = i / D, cc = i - r * D;
      const float x = outs[r * TW + cc];
      if (kind == 2) {
        p.vd[head * p.vcol_stride_h + (size_t)cc * p.vrow_stride + p.row_base + r0 + r] = x;
        continue;
      }
      int pos = base + p.pos0 + r0 + r;
      pos = pos < 0 ? 0 : (pos >= p.rope_rows ? p.rope_rows - 1 : pos);
      const int j = cc < half ? cc : cc - half;
      const float c = p.cs[(size_t)pos * half + j], s = p.sn[(size_t)pos * half + j];
      const float y = cc < half ? x * c - outs[r * TW + cc + half] * s : x * c + outs[r * TW + cc - half] * s;
      if (kind == 0)
        p.q_out[((size_t)(r0 + r) * p.Hq + head) * D + cc] = y;
      else
        p.kd[head * p.krow_stride_h + (size_t)(p.row_base + r0 + r) * D + cc] = y;
    }
  }
}

// Eviction rule of the tiny loop's compressor: the first `sinks` positions,
// the last `recent`, and the multiples of `stride` in between (ascending);
// everything when T <= sinks + recent.
// The middle range [sinks, T - recent) is non-empty; sums are taken in 64
// bits so that no argument in int32 range wraps, and every result is at most T.
VC_DEVICE_HOST_INLINE int evict_mid(int T, int sinks, int recent, int stride, int *first) {
  const int64_t lo = sinks, hi = (int64_t)T - recent;
  const int64_t f = (lo + stride - 1) / stride, last = (hi - 1) / stride;
  *first = (int)f;
  return last >= f ? (int)(last - f + 1) : 0;
}
VC_DEVICE_HOST_INLINE bool evict_all(int T, int sinks, int recent) { return (int64_t)T <= (int64_t)sinks + recent; }
VC_DEVICE_HOST_INLINE int evict_count(int T, int sinks, int recent, int stride) {
  if (evict_all(T, sinks, recent)) return T;
  int first;
  return sinks + evict_mid(T, sinks, recent, stride, &first) + recent;
}

// Compacted cache rows j0 .. j0 + 31 of KV head blockIdx.y (one 32-row block
// of the blocked V layout per workgroup).  The kept positions come from idx
// (a list) or, with idx == NULL, from the eviction rule at T = *src_len.
__global__ __launch_bounds__(256) void gather_tile(int D, int n_list, const int32_t *__restrict__ idx,
                                                   const int32_t *__restrict__ src_len, int sinks, int recent,
                                                   int stride, const float *__restrict__ sk,
                                                   const float *__restrict__ sv, int64_t scap,
                                                   float *__restrict__ dk, float *__restrict__ dv, int64_t dcap,
                                                   int32_t *__restrict__ dlen) {
  const int h = blockIdx.y, j0 = blockIdx.x * 32, tid = threadIdx.x;
  int n, T = 0, mid = 0, first = 0;
  if (idx) {
    n = n_list;
  } else {
    T = *src_len;
    T = T < 0 ? 0 : (T > scap ? (int)scap : T);
    n = evict_count(T, sinks, recent, stride);
    if (!evict_all(T, sinks, recent)) mid = evict_mid(T, sinks, recent, stride, &first);
  }
  n = n > dcap ? (int)dcap : n;
  if (blockIdx.x == 0 && tid == 0) dlen[h] = n;
  if (j0 >= n) return;
  __shared__ int pos[32];
  if (tid < 32) {
    const int j = j0 + tid;
    int p = j;
    if (idx) {
      p = j < n ? idx[j] : 0;
    } else if (!evict_all(T, sinks, recent)) {
      p = j < sinks ? j : (j < sinks + mid ? (first + (j - sinks)) * stride : T - recent + (j - sinks - mid));
    }
    pos[tid] = p < 0 ? 0 : (p >= scap ? (int)scap - 1 : p);
  }
  __syncthreads();
  const int rows = min(32, n - j0);
  const float *skh = sk + (size_t)h * scap * D, *svh = sv + (size_t)h * D * scap;
  float *dkh = dk + (size_t)h * dcap * D, *dvt = dv + (size_t)h * D * dcap + (size_t)(j0 / 32) * D * 32;
  for (int e = tid; e < rows * D; e += 256) {
    const int j = e / D, d = e - j * D;
    dkh[(size_t)(j0 + j) * D + d] = skh[(size_t)pos[j] * D + d];
  }
  for (int e = tid; e < 32 * D; e += 256) {
    const int d = e >> 5, j = e & 31;
    if (j < rows) dvt[e] = svh[(size_t)d * scap + pos[j]];
  }
}

struct TinyWs {
  float *h, *q, *o, *g;
};

TinyWs carve(const vc_tiny_model &m, int R, void *ws) {
  const size_t dm = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim;
  float *p = (float *)ws;
  TinyWs w;
  w.h = p; p += R * dm;
  w.q = p; p += R * qd;
  w.o = p; p += R * qd;
  w.g = p; p += R * (size_t)m.ffn;
  return w;
}

size_t ws_floats(const vc_tiny_model &m, int R) {
  const size_t dm = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim;
  return (size_t)R * (dm + 2 * qd + (size_t)m.ffn);
}

hipError_t plain(const float *X, int R, int K, bool norm, float eps, const float *W, int N, const float *Res,
                 float *Y, hipStream_t s) {
  ProjParams p{};
  p.X = X; p.R = R; p.K = K; p.norm = norm; p.eps = eps;
  p.W[0] = W; p.ldw = N; p.N = N; p.Res = Res; p.Y = Y;
  proj<1, 1, kPlain><<<dim3((N + 63) / 64, (R + kRT - 1) / kRT), kPT, 0, s>>>(p);
  return hipGetLastError();
}

hipError_t launch_gather(int Hkv, int D, int n_list, const int32_t *idx, const int32_t *src_len, int sinks,
                         int recent, int stride, const float *sk, const float *sv, int64_t scap, float *dk,
                         float *dv, int64_t dcap, int32_t *dlen, hipStream_t s) {
  gather_tile<<<dim3((unsigned)(dcap / 32), Hkv), 256, 0, s>>>(D, n_list, idx, src_len, sinks, recent, stride, sk,
                                                              sv, scap, dk, dv, dcap, dlen);
  return hipGetLastError();
}

}  // namespace
}  // namespace vc

namespace vc {
vc_status set_error(vc_status s, const char *msg);
}

extern "C" {

vc_status vc_tiny_rope_table(int32_t rows, int32_t head_dim, float base, float *cos_out, float *sin_out) {
  if (rows < 0 || head_dim <= 0 || head_dim % 2 || !cos_out || !sin_out)
    return vc::set_error(VC_EINVAL, "bad rope table arguments");
  const int half = head_dim / 2;
  for (int p = 0; p < rows; ++p)
    for (int i = 0; i < half; ++i) {
      const double theta = std::pow((double)base, -2.0 * i / head_dim);
      const double ang = (double)p * theta;
      cos_out[(size_t)p * half + i] = (float)std::cos(ang);
      sin_out[(size_t)p * half + i] = (float)std::sin(ang);
    }
  return VC_OK;
}

size_t vc_tiny_workspace_size(const vc_tiny_model *m, int32_t R) {
  if (!m || R <= 0) return 0;
  return vc::ws_floats(*m, R) * sizeof(float);
}

vc_status vc_tiny_forward(const vc_tiny_model *m, int32_t R, const int32_t *tokens, int32_t pos0,
                          const vc_tiny_attn *at, float *logits, void *workspace, size_t workspace_bytes,
                          void *stream) {
  using namespace vc;
  if (!m || !at || !tokens || !logits || R <= 0) return set_error(VC_EINVAL, "bad tiny forward arguments");
  if (m->n_layers < 1 || m->n_layers > VC_TINY_MAX_LAYERS) return set_error(VC_EINVAL, "bad layer count");
  if (m->n_q_heads < 1 || m->n_kv_heads < 1 || m->n_q_heads % m->n_kv_heads)
    return set_error(VC_EINVAL, "Hq must be a positive multiple of Hkv");
  if (m->head_dim != 64 && m->head_dim != 128) return set_error(VC_ENOTSUP, "head_dim must be 64 or 128");
  if (m->d_model < 1 || m->d_model > 1024 || m->ffn < 1 || m->ffn > kMaxK || m->vocab < 1 ||
      (size_t)m->n_q_heads * m->head_dim > 1024)
    return set_error(VC_ENOTSUP, "tiny model too wide (d_model and Hq * head_dim <= 1024, ffn <= 4096)");
  if (pos0 < 0 || (!at->pos_base && (int64_t)pos0 + R > m->rope_rows))
    return set_error(VC_EINVAL, "positions exceed the RoPE table");
  if (!workspace || workspace_bytes < vc_tiny_workspace_size(m, R)) return set_error(VC_EINVAL, "workspace too small");
  if (at->mode == VC_TINY_DRAFT && (R != 1 || at->tail_pos < 0 || at->tail_pos >= at->tcap || !at->tail_len))
    return set_error(VC_EINVAL, "draft mode needs R = 1 and 0 <= tail_pos < tcap");
  hipStream_t s = (hipStream_t)stream;
  const int dm = m->d_model, Hq = m->n_q_heads, Hkv = m->n_kv_heads, D = m->head_dim, F = m->ffn;
  const int qd = Hq * D;
  const dim3 rtiles(1, (R + kRT - 1) / kRT);
  TinyWs w = carve(*m, R, workspace);
  hipError_t e;
#define TRY(x)                                                      \
  do {                                                              \
    e = (x);                                                        \
    if (e != hipSuccess) return set_error(VC_EHIP, hipGetErrorString(e)); \
  } while (0)
  const bool draft = at->mode == VC_TINY_DRAFT;
  embed_rows<<<R, 256, 0, s>>>(m->emb, tokens, m->vocab, dm, w.h, draft ? at->tail_len : nullptr,
                               at->tail_pos + 1);
  TRY(hipGetLastError());
  for (int l = 0; l < m->n_layers; ++l) {
    ProjParams p{};
    p.X = w.h; p.R = R; p.K = dm; p.norm = 1; p.eps = m->eps;
    p.wq = m->wq[l]; p.wk = m->wk[l]; p.wv = m->wv[l];
    p.Hq = Hq; p.Hkv = Hkv; p.D = D;
    p.cs = m->rope_cos; p.sn = m->rope_sin; p.rope_rows = m->rope_rows;
    p.pos_base = at->pos_base; p.pos0 = pos0;
    p.q_out = w.q;
    p.kd = (float *)at->blk_k[l];
    p.vd = (float *)at->blk_v[l];
    if (!draft) {
      p.krow_stride_h = (int64_t)R * D; p.vcol_stride_h = (int64_t)D * R; p.vrow_stride = R; p.row_base = 0;
    } else {
      p.krow_stride_h = at->tcap * D; p.vcol_stride_h = (int64_t)D * at->tcap; p.vrow_stride = at->tcap;
      p.row_base = at->tail_pos;
    }
    const dim3 grid(Hq + 2 * Hkv, rtiles.y);
    if (D == 64)
      proj<1, 1, kQkvRope><<<grid, kPT, 0, s>>>(p);
    else
      proj<2, 1, kQkvRope><<<grid, kPT, 0, s>>>(p);
    TRY(hipGetLastError());
    if (!draft) {
      vc_verify_args va{};
      va.B = 1; va.Hq = Hq; va.Hkv = Hkv; va.D = D; va.M = R; va.dtype = VC_FP32;
      va.scale = 1.0f / sqrtf((float)D);
      va.ccap = at->cap; va.q = w.q; va.ctx_k = at->k[l]; va.ctx_v = at->v[l]; va.ctx_len = at->len;
      va.blk_k = at->blk_k[l]; va.blk_v = at->blk_v[l]; va.out = w.o;
      TRY(launch_verify_f32(va, s));
    } else {
      vc_draft_args da{};
      da.B = 1; da.Hq = Hq; da.Hkv = Hkv; da.D = D; da.dtype = VC_FP32; da.fmt = VC_KV_DENSE;
      da.scale = 1.0f / sqrtf((float)D);
      da.cap = at->cap; da.tcap = at->tcap; da.q = w.q; da.main_len = at->len; da.k = at->k[l]; da.v = at->v[l];
      da.tail_k = at->blk_k[l]; da.tail_v = at->blk_v[l]; da.tail_len = at->tail_len; da.out = w.o;
      TRY(launch_draft_f32(da, s));
    }
    TRY(plain(w.o, R, qd, false, 0.f, m->wo[l], dm, w.h, w.h, s));
    ProjParams g{};
    g.X = w.h; g.R = R; g.K = dm; g.norm = 1; g.eps = m->eps;
    g.W[0] = m->wg[l]; g.W[1] = m->wu[l]; g.ldw = F; g.N = F; g.Y = w.g;
    proj<1, 2, kSwiglu><<<dim3((F + 63) / 64, rtiles.y), kPT, 0, s>>>(g);
    TRY(hipGetLastError());
    TRY(plain(w.g, R, F, false, 0.f, m->wd[l], dm, w.h, w.h, s));
  }
  TRY(plain(w.h, R, dm, true, m->eps, m->w_lm, m->vocab, nullptr, logits, s));
#undef TRY
  return VC_OK;
}

vc_status vc_gather_rows(int32_t Hkv, int32_t D, int32_t n, const int32_t *idx, const float *src_k,
                         const float *src_v, int64_t src_cap, float *dst_k, float *dst_v, int64_t dst_cap,
                         int32_t *dst_len, void *stream) {
  if (Hkv < 1 || D < 1 || n < 0 || n > dst_cap || dst_cap % 32 != 0 || src_cap < 1 || !idx || !src_k || !src_v ||
      !dst_k || !dst_v || !dst_len)
    return vc::set_error(VC_EINVAL, "bad gather arguments");
  if (dst_cap == 0) return VC_OK;
  hipError_t e = vc::launch_gather(Hkv, D, n, idx, nullptr, 0, 0, 1, src_k, src_v, src_cap, dst_k, dst_v, dst_cap,
                                   dst_len, (hipStream_t)stream);
  return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, hipGetErrorString(e));
}

int32_t vc_evict_kept_count(int32_t T, int32_t sinks, int32_t recent, int32_t stride) {
  if (T < 0 || sinks < 0 || recent < 0 || stride < 1) return -1;
  return vc::evict_count(T, sinks, recent, stride);
}

vc_status vc_gather_evict(int32_t Hkv, int32_t D, const int32_t *src_len, int32_t sinks, int32_t recent,
                          int32_t stride, const float *src_k, const float *src_v, int64_t src_cap, float *dst_k,
                          float *dst_v, int64_t dst_cap, int32_t *dst_len, void *stream) {
  if (Hkv < 1 || D < 1 || sinks < 0 || recent < 0 || stride < 1 || src_cap < 1 || src_cap > INT32_MAX ||
      dst_cap % 32 != 0 || !src_len || !src_k || !src_v || !dst_k || !dst_v || !dst_len)
    return vc::set_error(VC_EINVAL, "bad eviction gather arguments");
  if (vc::evict_count((int)src_cap, sinks, recent, stride) > dst_cap)
    return vc::set_error(VC_EINVAL, "the compacted cache cannot hold the kept rows of a full source cache");
  if (dst_cap == 0) return VC_OK;
  hipError_t e = vc::launch_gather(Hkv, D, 0, nullptr, src_len, sinks, recent, stride, src_k, src_v, src_cap, dst_k,
                                   dst_v, dst_cap, dst_len, (hipStream_t)stream);
  return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, hipGetErrorString(e));
}

}  // extern "C"
