// A small fp32 decoder run entirely on the GPU (support for end-to-end
// checks of the draft-then-verify loop; see include/vc_tiny.h).
//
// Each forward is a fixed sequence of small kernels per layer: RMSNorm,
// QKV GEMM, RoPE + scatter of K/V into the block (verify) or draft tail,
// attention through the library's own draft/verify paths, output GEMM with
// the residual, RMSNorm, gate/up GEMMs, SwiGLU, down GEMM with the residual;
// then RMSNorm and the LM head.  Every reduction runs in a fixed order.
#include <cmath>

#include "../../include/vc_tiny.h"
#include "common.h"
#include "launch.h"

namespace vc {

hipError_t launch_draft_f32(const vc_draft_args &a, hipStream_t s);
hipError_t launch_verify_f32(const vc_verify_args &a, hipStream_t s);

namespace {

__global__ __launch_bounds__(256) void embed_rows(const float *__restrict__ emb, const int32_t *__restrict__ tok,
                                                  int vocab, int dm, float *__restrict__ h) {
  const int r = blockIdx.x;
  int t = tok[r];
  t = t < 0 ? 0 : (t >= vocab ? vocab - 1 : t);
  for (int i = threadIdx.x; i < dm; i += blockDim.x) h[(size_t)r * dm + i] = emb[(size_t)t * dm + i];
}

// out = x / sqrt(mean(x^2) + eps), one wave per row.
__global__ __launch_bounds__(64) void rmsnorm_rows(const float *__restrict__ x, int dm, float eps,
                                                   float *__restrict__ out) {
  const int r = blockIdx.x, lane = threadIdx.x;
  const float *xr = x + (size_t)r * dm;
  float ss = 0.f;
  for (int i = lane; i < dm; i += 64) ss = fmaf(xr[i], xr[i], ss);
  ss = wave_sum(ss);
  const float inv = 1.0f / sqrtf(ss / (float)dm + eps);
  for (int i = lane; i < dm; i += 64) out[(size_t)r * dm + i] = xr[i] * inv;
}

// Y[R][N] = X[R][K] W[K][N] (+ Res[R][N]); a row tile of 8 staged in LDS,
// one output column per thread, k ascending.
constexpr int kRowTile = 8;
__global__ __launch_bounds__(256) void gemm_rows(const float *__restrict__ X, const float *__restrict__ W,
                                                 const float *Res, float *Y, int R, int K, int N) {
  extern __shared__ float xs[];   // [kRowTile][K]
  const int r0 = blockIdx.y * kRowTile;
  const int rows = min(kRowTile, R - r0);
  for (int i = threadIdx.x; i < rows * K; i += blockDim.x) xs[i] = X[(size_t)r0 * K + i];
  __syncthreads();
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  float acc[kRowTile];
#pragma unroll
  for (int r = 0; r < kRowTile; ++r) acc[r] = 0.f;
  for (int k = 0; k < K; ++k) {
    const float w = W[(size_t)k * N + n];
#pragma unroll
    for (int r = 0; r < kRowTile; ++r)
      if (r < rows) acc[r] = fmaf(xs[r * K + k], w, acc[r]);
  }
  for (int r = 0; r < rows; ++r) {
    const size_t o = (size_t)(r0 + r) * N + n;
    Y[o] = Res ? Res[o] + acc[r] : acc[r];
  }
}

// RoPE on q and k of row r (position pos0 + r), q to q_out[r][Hq][D],
// k/v scattered into the K (token-major) / V (channel-major) destination.
// Sources: xq [R][Hq*D], xk [R][Hkv*D], xv [R][Hkv*D].
__global__ __launch_bounds__(256) void rope_scatter(const float *__restrict__ xq, const float *__restrict__ xk,
                                                    const float *__restrict__ xv, int Hq, int Hkv, int D,
                                                    const float *__restrict__ cs, const float *__restrict__ sn,
                                                    int pos0, float *__restrict__ q_out, float *__restrict__ kd,
                                                    float *__restrict__ vd, int64_t krow_stride_h,
                                                    int64_t vcol_stride_h, int64_t vrow_stride, int row_base) {
  const int r = blockIdx.x;
  const int half = D / 2;
  const int p = pos0 + r;
  const int row = row_base + r;   // destination row / column
  for (int e = threadIdx.x; e < (Hq + Hkv) * half; e += blockDim.x) {
    const int h = e / half, i = e % half;
    const float c = cs[(size_t)p * half + i], s = sn[(size_t)p * half + i];
    const float *src = (h < Hq) ? xq + ((size_t)r * Hq + h) * D : xk + ((size_t)r * Hkv + (h - Hq)) * D;
    const float x1 = src[i], x2 = src[i + half];
    const float y1 = x1 * c - x2 * s, y2 = x2 * c + x1 * s;
    if (h < Hq) {
      q_out[((size_t)r * Hq + h) * D + i] = y1;
      q_out[((size_t)r * Hq + h) * D + i + half] = y2;
    } else {
      const int kh = h - Hq;
      kd[kh * krow_stride_h + (size_t)row * D + i] = y1;
      kd[kh * krow_stride_h + (size_t)row * D + i + half] = y2;
    }
  }
  for (int e = threadIdx.x; e < Hkv * D; e += blockDim.x) {
    const int kh = e / D, d = e % D;
    vd[kh * vcol_stride_h + (size_t)d * vrow_stride + row] = xv[(size_t)r * Hkv * D + e];
  }
}

__global__ __launch_bounds__(256) void swiglu(const float *__restrict__ g, const float *__restrict__ u,
                                              float *__restrict__ out, size_t n) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) {
    const float x = g[i];
    out[i] = x / (1.0f + expf(-x)) * u[i];
  }
}

__global__ void set_i32(int32_t *p, int v) { *p = v; }

__global__ __launch_bounds__(256) void gather_rows(int D, int n, const int32_t *__restrict__ idx,
                                                   const float *__restrict__ sk, const float *__restrict__ sv,
                                                   int64_t scap, float *__restrict__ dk, float *__restrict__ dv,
                                                   int64_t dcap, int32_t *__restrict__ dlen) {
  const int h = blockIdx.x;
  const float *skh = sk + (size_t)h * scap * D, *svh = sv + (size_t)h * D * scap;
  float *dkh = dk + (size_t)h * dcap * D, *dvh = dv + (size_t)h * D * dcap;
  for (int e = threadIdx.x; e < n * D; e += blockDim.x) {
    const int j = e / D, d = e % D;
    int p = idx[j];
    p = p < 0 ? 0 : (p >= scap ? (int)scap - 1 : p);
    dkh[(size_t)j * D + d] = skh[(size_t)p * D + d];
    dvh[(size_t)(j >> 5) * D * 32 + d * 32 + (j & 31)] = svh[(size_t)d * scap + p];
  }
  if (threadIdx.x == 0) dlen[h] = n;
}

struct TinyWs {
  float *h, *a, *qkv, *q, *o, *g, *u;
};

TinyWs carve(const vc_tiny_model &m, int R, void *ws) {
  const size_t dm = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim, kd = (size_t)m.n_kv_heads * m.head_dim;
  float *p = (float *)ws;
  TinyWs w;
  w.h = p; p += R * dm;
  w.a = p; p += R * dm;
  w.qkv = p; p += R * (qd + 2 * kd);
  w.q = p; p += R * qd;
  w.o = p; p += R * qd;
  w.g = p; p += R * (size_t)m.ffn;
  w.u = p; p += R * (size_t)m.ffn;
  return w;
}

size_t ws_floats(const vc_tiny_model &m, int R) {
  const size_t dm = m.d_model, qd = (size_t)m.n_q_heads * m.head_dim, kd = (size_t)m.n_kv_heads * m.head_dim;
  return (size_t)R * (2 * dm + qd + 2 * kd + 2 * qd + 2 * (size_t)m.ffn);
}

hipError_t gemm(const float *X, const float *W, const float *Res, float *Y, int R, int K, int N, hipStream_t s) {
  dim3 grid((N + 255) / 256, (R + kRowTile - 1) / kRowTile);
  gemm_rows<<<grid, 256, kRowTile * K * sizeof(float), s>>>(X, W, Res, Y, R, K, N);
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
  if (m->n_q_heads % m->n_kv_heads) return set_error(VC_EINVAL, "Hq must be a multiple of Hkv");
  if (m->head_dim != 64 && m->head_dim != 128) return set_error(VC_ENOTSUP, "head_dim must be 64 or 128");
  if (m->d_model > 1024 || m->ffn > 4096) return set_error(VC_ENOTSUP, "tiny model too wide");
  if (pos0 < 0 || pos0 + R > m->rope_rows) return set_error(VC_EINVAL, "positions exceed the RoPE table");
  if (!workspace || workspace_bytes < vc_tiny_workspace_size(m, R)) return set_error(VC_EINVAL, "workspace too small");
  if (at->mode == VC_TINY_DRAFT && (R != 1 || at->tail_pos < 0 || at->tail_pos >= at->tcap || !at->tail_len))
    return set_error(VC_EINVAL, "draft mode needs R = 1 and 0 <= tail_pos < tcap");
  hipStream_t s = (hipStream_t)stream;
  const int dm = m->d_model, Hq = m->n_q_heads, Hkv = m->n_kv_heads, D = m->head_dim, F = m->ffn;
  const int qd = Hq * D, kd = Hkv * D;
  TinyWs w = carve(*m, R, workspace);
  hipError_t e;
#define TRY(x)                                                      \
  do {                                                              \
    e = (x);                                                        \
    if (e != hipSuccess) return set_error(VC_EHIP, hipGetErrorString(e)); \
  } while (0)
  embed_rows<<<R, 256, 0, s>>>(m->emb, tokens, m->vocab, dm, w.h);
  TRY(hipGetLastError());
  if (at->mode == VC_TINY_DRAFT) {
    set_i32<<<1, 1, 0, s>>>(at->tail_len, at->tail_pos + 1);
    TRY(hipGetLastError());
  }
  for (int l = 0; l < m->n_layers; ++l) {
    rmsnorm_rows<<<R, 64, 0, s>>>(w.h, dm, m->eps, w.a);
    TRY(hipGetLastError());
    // projections: qkv holds xq [R][qd], then xk [R][kd], then xv [R][kd]
    float *xq = w.qkv, *xk = w.qkv + (size_t)R * qd, *xv = xk + (size_t)R * kd;
    TRY(gemm(w.a, m->wq[l], nullptr, xq, R, dm, qd, s));
    TRY(gemm(w.a, m->wk[l], nullptr, xk, R, dm, kd, s));
    TRY(gemm(w.a, m->wv[l], nullptr, xv, R, dm, kd, s));
    float *kdst = (float *)at->blk_k[l];
    float *vdst = (float *)at->blk_v[l];
    if (at->mode == VC_TINY_VERIFY) {
      rope_scatter<<<R, 256, 0, s>>>(xq, xk, xv, Hq, Hkv, D, m->rope_cos, m->rope_sin, pos0, w.q, kdst, vdst,
                                     (int64_t)R * D, (int64_t)D * R, R, 0);
      TRY(hipGetLastError());
      vc_verify_args va{};
      va.B = 1; va.Hq = Hq; va.Hkv = Hkv; va.D = D; va.M = R; va.dtype = VC_FP32;
      va.scale = 1.0f / sqrtf((float)D);
      va.ccap = at->cap; va.q = w.q; va.ctx_k = at->k[l]; va.ctx_v = at->v[l]; va.ctx_len = at->len;
      va.blk_k = kdst; va.blk_v = vdst; va.out = w.o;
      TRY(launch_verify_f32(va, s));
    } else {
      rope_scatter<<<1, 256, 0, s>>>(xq, xk, xv, Hq, Hkv, D, m->rope_cos, m->rope_sin, pos0, w.q, kdst, vdst,
                                     at->tcap * D, (int64_t)D * at->tcap, at->tcap, at->tail_pos);
      TRY(hipGetLastError());
      vc_draft_args da{};
      da.B = 1; da.Hq = Hq; da.Hkv = Hkv; da.D = D; da.dtype = VC_FP32; da.fmt = VC_KV_DENSE;
      da.scale = 1.0f / sqrtf((float)D);
      da.cap = at->cap; da.tcap = at->tcap; da.q = w.q; da.main_len = at->len; da.k = at->k[l]; da.v = at->v[l];
      da.tail_k = kdst; da.tail_v = vdst; da.tail_len = at->tail_len; da.out = w.o;
      TRY(launch_draft_f32(da, s));
    }
    TRY(gemm(w.o, m->wo[l], w.h, w.h, R, qd, dm, s));
    rmsnorm_rows<<<R, 64, 0, s>>>(w.h, dm, m->eps, w.a);
    TRY(hipGetLastError());
    TRY(gemm(w.a, m->wg[l], nullptr, w.g, R, dm, F, s));
    TRY(gemm(w.a, m->wu[l], nullptr, w.u, R, dm, F, s));
    const size_t n = (size_t)R * F;
    swiglu<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(w.g, w.u, w.g, n);
    TRY(hipGetLastError());
    TRY(gemm(w.g, m->wd[l], w.h, w.h, R, F, dm, s));
  }
  rmsnorm_rows<<<R, 64, 0, s>>>(w.h, dm, m->eps, w.a);
  TRY(hipGetLastError());
  TRY(gemm(w.a, m->w_lm, nullptr, logits, R, dm, m->vocab, s));
#undef TRY
  return VC_OK;
}

vc_status vc_gather_rows(int32_t Hkv, int32_t D, int32_t n, const int32_t *idx, const float *src_k,
                         const float *src_v, int64_t src_cap, float *dst_k, float *dst_v, int64_t dst_cap,
                         int32_t *dst_len, void *stream) {
  if (Hkv < 1 || D < 1 || n < 0 || n > dst_cap || dst_cap % 32 != 0 || src_cap < 1 || !idx || !src_k || !src_v ||
      !dst_k || !dst_v || !dst_len)
    return vc::set_error(VC_EINVAL, "bad gather arguments");
  vc::gather_rows<<<Hkv, 256, 0, (hipStream_t)stream>>>(D, n, idx, src_k, src_v, src_cap, dst_k, dst_v, dst_cap,
                                                        dst_len);
  hipError_t e = hipGetLastError();
  return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, hipGetErrorString(e));
}

}  // extern "C"
