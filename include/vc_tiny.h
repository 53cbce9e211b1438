/*
 * vc_tiny.h -- support entry points that run a small fp32 decoder entirely
 * on the GPU, so the draft-then-verify loop ("Riepilogo Tecnico: VeriCache",
 * section "Algoritmo Principale") can be exercised end to end and compared
 * token for token with full-KV greedy decoding (section "Risultati
 * Sperimentali": the output is identical to full-cache greedy decoding).
 *
 * The decoder (a plain Llama-family block stack; the pages name no model):
 *   h = E[token]; per layer: a = RMSNorm(h); q,k,v = a Wq, a Wk, a Wv;
 *   RoPE (rotate-half, pairs (i, i + D/2)) on q and k; GQA attention;
 *   h += o Wo; m = RMSNorm(h); h += (SiLU(m Wg) * (m Wu)) Wd;
 *   logits = RMSNorm(h) W_lm.   RMSNorm has unit gain.
 * All tensors fp32, row-major; weights are [in][out] (x W).
 *
 * Conventions as in vc.h: device pointers unless stated, caller-owned
 * buffers, work enqueued on `stream`, no allocation, no synchronisation.
 */
#ifndef VC_TINY_H
#define VC_TINY_H

#include <stddef.h>
#include <stdint.h>

#include "vc.h"

#ifdef __cplusplus
extern "C" {
#endif

#define VC_TINY_MAX_LAYERS 16

typedef struct vc_tiny_model {
  int32_t n_layers, d_model, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
  float eps;
  float rope_base;
  const float *emb;                              /* [vocab][d_model]               */
  const float *wq[VC_TINY_MAX_LAYERS];           /* [d_model][Hq*D]                */
  const float *wk[VC_TINY_MAX_LAYERS];           /* [d_model][Hkv*D]               */
  const float *wv[VC_TINY_MAX_LAYERS];           /* [d_model][Hkv*D]               */
  const float *wo[VC_TINY_MAX_LAYERS];           /* [Hq*D][d_model]                */
  const float *wg[VC_TINY_MAX_LAYERS];           /* [d_model][ffn]                 */
  const float *wu[VC_TINY_MAX_LAYERS];           /* [d_model][ffn]                 */
  const float *wd[VC_TINY_MAX_LAYERS];           /* [ffn][d_model]                 */
  const float *w_lm;                             /* [d_model][vocab]               */
  const float *rope_cos, *rope_sin;              /* [rope_rows][D/2] (vc_tiny_rope_table) */
  int32_t rope_rows;                             /* positions covered by the table */
} vc_tiny_model;

typedef enum { VC_TINY_VERIFY = 0, VC_TINY_DRAFT = 1 } vc_tiny_mode;

/* Attention context of one forward call (batch 1).
 * VERIFY (also prefill): the R rows are a causal block at positions
 *   pos0..pos0+R-1 after a full cache of ctx_len (device [1]) rows; the
 *   forward writes each layer's block K/V (post-RoPE) into blk_k[l]
 *   [Hkv][R][D] and blk_v[l] [Hkv][D][R], then attends over cache + block.
 * DRAFT: R = 1 row at position pos0 attends over a compressed main segment
 *   (main_k[l] [Hkv][cap][D], main_v[l] [Hkv][D][cap], main_len device
 *   [Hkv]) and a tail; the forward writes the row's K/V into the tail at
 *   index tail_pos (tail_k[l] [Hkv][tcap][D], tail_v[l] [Hkv][D][tcap]) and
 *   attends with tail length tail_pos + 1 (tail_len, device [1], is set).
 * Positions: row r sits at pos0 + r, or at pos_base[0] + pos0 + r when
 *   pos_base is set (a device value such as the committed length, so that a
 *   captured round can be replayed as the sequence grows).  With pos_base the
 *   host cannot check the RoPE table's range: the caller keeps positions
 *   below rope_rows (the forward clamps them into the table).             */
typedef struct vc_tiny_attn {
  int32_t mode;
  int64_t cap;                                   /* ctx capacity (VERIFY) / main capacity (DRAFT) */
  void *k[VC_TINY_MAX_LAYERS];                   /* ctx_k (VERIFY) / main_k (DRAFT)               */
  void *v[VC_TINY_MAX_LAYERS];                   /* ctx_v (VERIFY) / main_v (DRAFT)               */
  int32_t *len;                                  /* ctx_len [1] (VERIFY) / main_len [Hkv] (DRAFT)  */
  void *blk_k[VC_TINY_MAX_LAYERS];               /* VERIFY block K/V, or DRAFT tail K/V           */
  void *blk_v[VC_TINY_MAX_LAYERS];
  int64_t tcap;                                  /* DRAFT tail capacity                           */
  int32_t tail_pos;                              /* DRAFT: tail index of this row                 */
  int32_t *tail_len;                             /* DRAFT: device [1], set to tail_pos + 1        */
  const int32_t *pos_base;                       /* optional device [1]: see below                */
} vc_tiny_attn;

/* Host-side RoPE table: cos/sin[p][i] of p * base^(-2i/D), computed in double
 * and rounded to float, for p < rows, i < D/2 (host buffers).               */
vc_status vc_tiny_rope_table(int32_t rows, int32_t head_dim, float base, float *cos_out, float *sin_out);

/* Bytes of workspace one forward of R rows needs.                           */
size_t vc_tiny_workspace_size(const vc_tiny_model *m, int32_t R);

/* One forward pass of R rows: tokens (device [R]) at positions pos0..;
 * logits [R][vocab] out.                                                    */
vc_status vc_tiny_forward(const vc_tiny_model *m, int32_t R, const int32_t *tokens, int32_t pos0,
                          const vc_tiny_attn *attn, float *logits, void *workspace, size_t workspace_bytes,
                          void *stream);

/* Compressed-cache construction for a token-eviction compressor: copy the
 * rows at positions idx[0..n-1] (device, ascending) of a cache into a
 * compacted cache, per KV head: dst_k[h][j] = src_k[h][idx[j]], dst_v of
 * row j = column idx[j] of src_v; sets dst_len[h] = n (device [Hkv]).
 * K token-major [Hkv][cap][D]; source V channel-major [Hkv][D][src_cap]
 * (a full cache), destination V in the draft main-segment layout
 * [Hkv][dst_cap/32][D][32] (dst_cap % 32 == 0); fp32.                       */
vc_status vc_gather_rows(int32_t Hkv, int32_t D, int32_t n, const int32_t *idx, const float *src_k,
                         const float *src_v, int64_t src_cap, float *dst_k, float *dst_v, int64_t dst_cap,
                         int32_t *dst_len, void *stream);

/* The tiny loop's eviction compressor ("Riassunto Tecnico: CentroidKV",
 * "Componenti Chiave", item 2: attention sinks and recent tokens are kept):
 * of a cache of T committed tokens keep the first `sinks` positions, the
 * last `recent`, and every multiple of `stride` in between; every position
 * when T <= sinks + recent.  vc_evict_kept_count returns how many positions
 * that keeps (-1 on negative arguments or stride < 1); it grows with T.     */
int32_t   vc_evict_kept_count(int32_t T, int32_t sinks, int32_t recent, int32_t stride);

/* vc_gather_rows over the kept positions of the eviction rule at the
 * committed length T = src_len[0] (device), computed on the device: the
 * compacted cache gets the kept rows in ascending order and dst_len[h] the
 * kept count, so a round can be captured once and replayed.  T is clamped
 * to [0, src_cap].  VC_EINVAL unless dst_cap % 32 == 0 and dst_cap holds the
 * kept rows of a full source cache (vc_evict_kept_count(src_cap, ...)).     */
vc_status vc_gather_evict(int32_t Hkv, int32_t D, const int32_t *src_len, int32_t sinks, int32_t recent,
                          int32_t stride, const float *src_k, const float *src_v, int64_t src_cap, float *dst_k,
                          float *dst_v, int64_t dst_cap, int32_t *dst_len, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* VC_TINY_H */
