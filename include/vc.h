/*
 * vc.h -- C ABI of the VeriCache draft-then-verify hot path on MI355X (gfx950).
 *
 * The method ("Riepilogo Tecnico: VeriCache", gist.science paper 2605.17613,
 * section "Algoritmo Principale"): the target model drafts candidate tokens
 * over a compressed KV cache (KV_comp), one forward pass over the full cache
 * (KV_full) verifies all drafted tokens at once, and tokens are accepted up to
 * the first mismatch, plus one bonus token when every draft matches.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Tensor pointers are DEVICE pointers unless stated otherwise; arrays are
 *    dense, row-major, in the index order written ([B][Hkv][cap][D] means D
 *    fastest).  Base pointers of bf16/fp32 tensors must be 16-byte aligned.
 *  - K is token-major ([..][tokens][D]); V is CHANNEL-major ([..][D][tokens]).
 *    Both contractions of attention (q.k over channels, p.v over tokens)
 *    then reduce along the contiguous axis.
 *  - The caller owns every buffer (e.g. allocated by torch).  These calls
 *    never allocate device memory, never synchronize, never modify inputs;
 *    work is enqueued on `stream` (a hipStream_t; NULL = null stream) and the
 *    call returns.  Calls on distinct streams with distinct outputs may run
 *    concurrently.
 *  - Lengths that live in device memory (main_len, tail_len, ctx_len) are
 *    clamped by the kernels to their capacities, so out-of-range values can
 *    not cause out-of-bounds accesses.  A query whose key set is empty gets
 *    NaN output and -inf lse.
 *  - Return: VC_OK, or VC_EINVAL (bad pointer/shape/alignment), VC_ENOTSUP
 *    (a head_dim / dtype / format combination that is not compiled),
 *    VC_EHIP (a HIP launch error).  On a non-OK status nothing was enqueued
 *    (except for VC_EHIP), and vc_last_error() returns a message for the
 *    calling thread.
 */
#ifndef VC_H
#define VC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The last enumerator keeps the type int-sized and makes every non-negative
 * int a valid value, so a caller may pass any such code to vc_status_string. */
typedef enum { VC_OK = 0, VC_EINVAL = 1, VC_ENOTSUP = 2, VC_EHIP = 3, VC_STATUS_MAX_ = 0x7fffffff } vc_status;
typedef enum { VC_BF16 = 0, VC_FP32 = 1 } vc_dtype;
typedef enum { VC_KV_DENSE = 0, VC_KV_INT4 = 1, VC_KV_INT4_PACKED = 2 } vc_kv_format;

/* ------------------------------------------------------------------------ */
/* Draft decode attention ("Algoritmo Principale", step 1: drafting over the
 * compressed cache).  One query token per request; for query head h (KV head
 * g = h / (Hq/Hkv)) the output is
 *   o = sum_t softmax_t(scale * q.k_t + beta_t) v_t
 * over the main (compressed) segment t < main_len[b][g] followed by the tail
 * segment t < tail_len[b] (beta = 0).  beta_t = ln(degree_t) when degrees are
 * given: a centroid that merged n_t tokens enters the softmax with the
 * logarithm of its degree ("Riassunto Tecnico: CentroidKV", gist.science paper
 * 2506.11418, "Componenti Chiave", item 4 "Aggregazione"); otherwise 0.
 * The main segment is either dense (bf16/fp32) or int4 group-quantized
 * (the quantizing drafters of "Supporto Architetturale"):
 *   K_hat[t][d] = ck[t][d] * k_scale[t/32][d] + k_zero[t/32][d]
 *   V_hat[t][d] = cv[t][d] * v_scale[t/32][d/32][t%32] + v_zero[t/32][d/32][t%32]
 * (one K group = one channel over 32 tokens, one V group = one token over 32
 * channels; codes 0..15, scales/zeros binary16).  Everything int4 is laid out
 * in 32-token blocks, so one block's codes and parameters are contiguous.
 * Range of the int4 path: its MFMA operands are fp16 (q * k_scale with q
 * brought to [0.5, 1) by a power of two, and p * v_scale with p <= 2^8), so
 * every k_scale and v_scale must lie below 2^9 (reconstructions within about
 * +-7000); larger scales overflow to inf and the output is NaN.  Nothing checks
 * this on the device: a cache built by vc_quantize_int4 from values that
 * large must not be drafted over.                                          */
typedef struct vc_draft_args {
  int32_t B, Hq, Hkv, D;          /* D in {64, 128}; Hq % Hkv == 0, Hq/Hkv <= 16   */
  int32_t dtype;                  /* vc_dtype of q, dense K/V, tail K/V and out    */
  int32_t fmt;                    /* vc_kv_format of the main segment              */
  float   scale;                  /* softmax scale, normally 1/sqrt(D)             */
  int32_t num_splits;             /* token splits per (b, KV head); 0 = automatic  */
  int64_t cap;                    /* main capacity per (b, KV head); multiple of 64 */
  int64_t tcap;                   /* tail capacity (0 when no tail); cap + tcap    */
                                  /* <= 2^30                                       */
  const void    *q;               /* [B][Hq][D]                                    */
  const int32_t *main_len;        /* [B][Hkv] valid main tokens                    */
  const void    *k;               /* DENSE [B][Hkv][cap][D]; INT4 u8 [B][Hkv][cap][D/2]:
                                     a token's D codes in channel order, packed
                                     eight per 32-bit word (see below)             */
  const void    *v;               /* DENSE [B][Hkv][cap/32][D][32]: 32-token
                                     blocks, channel-major inside a block; INT4 u8
                                     [B][Hkv][cap/32][D][16]: per 32-token block,
                                     channel d's 32 codes in token order, packed
                                     eight per 32-bit word (see below)             */
  /* INT4 code words: eight consecutive 4-bit codes c0..c7 per little-endian
     32-bit word, c_2j in bits 4j..4j+3 and c_2j+1 in bits 16+4j..16+4j+3
     (j = 0..3): bytes c0|c2<<4, c4|c6<<4, c1|c3<<4, c5|c7<<4.               */
  const uint16_t *k_scale, *k_zero; /* INT4 only: fp16 [B][Hkv][cap/32][D]         */
  const uint16_t *v_scale, *v_zero; /* INT4 only: fp16 [B][Hkv][cap/32][D/32][32]  */
  /* INT4_PACKED: the same codes and parameters with each 32-token block's six
     pieces interleaved into one 5120-byte block, k = u8 [B][Hkv][cap/32][5120]:
     bytes 0..2047 K codes (as INT4 k), 2048..4095 V codes (as INT4 v),
     4096..4351 K scales, 4352..4607 K zeros, 4608..4863 V scales, 4864..5119
     V zeros (each as the INT4 arrays' block); v and the four scale/zero
     pointers must be NULL.  One block is then one contiguous read.          */
  const float   *degree;          /* optional [B][Hd][cap] merge degrees n_t >= 1  */
  int64_t degree_h_stride;        /* 0: one row per request shared by all KV heads;
                                     cap: one row per KV head                      */
  const void    *tail_k;          /* optional [B][Hkv][tcap][D] (dtype)            */
  const void    *tail_v;          /* optional [B][Hkv][D][tcap] (dtype)            */
  const int32_t *tail_len;        /* optional [B]; NULL means 0                    */
  void  *out;                     /* [B][Hq][D] (dtype)                            */
  float *out_lse;                 /* optional [B][Hq], natural log                 */
  void  *workspace;               /* split partials; >= vc_draft_workspace_size()  */
  size_t workspace_bytes;
} vc_draft_args;

vc_status vc_draft_attn(const vc_draft_args *a, void *stream);
size_t    vc_draft_workspace_size(const vc_draft_args *a);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * call as vc_draft_attn, with a->workspace ignored.  The split partials live
 * in a static device array of vc_draft_noalloc_max_scratch() bytes (16 MiB),
 * one per GPU, held until the process ends; this call allocates nothing.  A
 * call whose vc_draft_workspace_size() exceeds the array fails with
 * VC_EINVAL before anything is enqueued.  Every call on one GPU shares that
 * GPU's array and the array keeps the last call's partials: calls that
 * overlap in time on one GPU (e.g. on two streams) race and must not be
 * made.  Nothing in it needs clearing: a call writes its partials before it
 * reads them.                                                              */
vc_status vc_draft_attn_noalloc(const vc_draft_args *a, void *stream);
size_t    vc_draft_noalloc_max_scratch(void);

/* ------------------------------------------------------------------------ */
/* Verify block attention ("Algoritmo Principale", step 2: one forward pass
 * with the full cache checks every drafted token in parallel).  Each request
 * has a block of M query rows (the last accepted token followed by the k
 * drafts, M = k + 1).  Row i of request b sees every context key
 * t < ctx_len[b] and the block keys 0..i (causal inside the block):
 *   o[b][i][h] = sum_t softmax_t(scale * q.k_t) v_t.
 * With ctx_len = 0 and the prompt as the block this is causal prefill.     */
typedef struct vc_verify_args {
  int32_t B, Hq, Hkv, D, M;       /* D in {64, 128}; M >= 1; Hq % Hkv == 0;        */
                                  /* M*Hq/Hkv <= 65535*64, B*M*Hq < 2^31           */
  int32_t dtype;                  /* vc_dtype of every tensor below                */
  float   scale;
  int32_t num_splits;             /* key splits per (b, KV head); 0 = automatic    */
  int64_t ccap;                   /* context capacity; multiple of 64, <= 2^30     */
  const void    *q;               /* [B][M][Hq][D]                                 */
  const void    *ctx_k;           /* [B][Hkv][ccap][D]                             */
  const void    *ctx_v;           /* [B][Hkv][D][ccap]                             */
  const int32_t *ctx_len;         /* [B]                                           */
  const void    *blk_k;           /* [B][Hkv][M][D]                                */
  const void    *blk_v;           /* [B][Hkv][D][M]                                */
  void  *out;                     /* [B][M][Hq][D]                                 */
  float *out_lse;                 /* optional [B][M][Hq], natural log              */
  void  *workspace;               /* >= vc_verify_workspace_size()                 */
  size_t workspace_bytes;
} vc_verify_args;

vc_status vc_verify_attn(const vc_verify_args *a, void *stream);
size_t    vc_verify_workspace_size(const vc_verify_args *a);

/* ------------------------------------------------------------------------ */
/* Greedy acceptance ("Algoritmo Principale", step 3).  For each request the
 * M = k + 1 logit rows are the full-cache predictions after x0, d_1..d_k:
 *   y_{j+1} = argmax(logits[b][j])   (lowest index among equal maxima;
 *                                     logits must be finite)
 *   n       = number of leading j with d_j == y_j          (0..k)
 *   emitted = d_1..d_n, y_{n+1}      (y_{k+1} is the bonus when n = k)
 * Outputs: argmax [B][M], accept_len [B] = n, out_tokens [B][M] = emitted
 * then -1 padding, n_out [B] = n + 1.  Any M >= 1 is accepted.              */
typedef struct vc_accept_args {
  int32_t B, M, V;
  int32_t logit_dtype;            /* VC_BF16 or VC_FP32                            */
  const void    *logits;          /* [B][M][V]                                     */
  const int32_t *draft;           /* [B][M-1] (may be NULL when M == 1)            */
  int32_t *argmax;                /* [B][M]                                        */
  int32_t *accept_len;            /* [B]                                           */
  int32_t *out_tokens;            /* [B][M]                                        */
  int32_t *n_out;                 /* [B]                                           */
} vc_accept_args;

vc_status vc_accept(const vc_accept_args *a, void *stream);

/* The next round's first input ("Algoritmo Principale", step 3: decoding
 * resumes from the last emitted token): dst[b * dst_stride] =
 * out_tokens[b][n_out[b] - 1] for out_tokens [B][M] and n_out [B] as
 * vc_accept writes them (n_out clamped to [1, M]); int32, device.  Lets a
 * round's inputs be chained on the device without a host round trip.
 * VC_EINVAL on B < 0, M < 1, dst_stride < 1 or null pointers.               */
vc_status vc_next_input(int32_t B, int32_t M, const int32_t *out_tokens, const int32_t *n_out, int32_t *dst,
                        int64_t dst_stride, void *stream);

/* ------------------------------------------------------------------------ */
/* Greedy token choice of the drafter (the draft step's argmax): for each of
 * R rows of logits[R][V], out[r * out_stride] = lowest index of the row
 * maximum (same rule as vc_accept).  out_stride >= 1 lets a caller write the
 * i-th draft of every request straight into draft[B][k] (stride k).        */
vc_status vc_argmax(int32_t R, int32_t V, int32_t logit_dtype, const void *logits,
                    int32_t *out, int32_t out_stride, void *stream);

/* LM head fused with the greedy choice ("Algoritmo Principale", steps 1
 * and 3: the drafter and the verifier keep only the argmax of each logit
 * row): out[r * out_stride] = lowest index of the maximum over v of
 *   logit[r][v] = sum_k h[r][k] * w[v][k]
 * computed in fp32 from bf16 products (MFMA) without writing the logits.
 *   h [R][Dm] bf16, w [V][Dm] bf16 (vocab-major: a linear layer's weight),
 *   both 16-byte aligned; Dm % 32 == 0, Dm <= 2^20, V <= 2^30; out int32 (device).
 * NaN logits never win (a row of NaN gives 0).  The summation order is the
 * kernel's own, so at a near tie (logits equal to fp32 rounding) another
 * GEMM followed by vc_argmax may pick a different maximum.  workspace: device buffer of
 * at least vc_lm_head_argmax_workspace_size(R, V) bytes (per-tile maxima),
 * 16-byte aligned, owned by the caller and not read across calls.
 * VC_EINVAL on bad shapes, null or misaligned pointers or a short
 * workspace; nothing is enqueued then.                                     */
size_t    vc_lm_head_argmax_workspace_size(int32_t R, int32_t V);
vc_status vc_lm_head_argmax(int32_t R, int32_t Dm, int32_t V, const void *h, const void *w,
                            int32_t *out, int32_t out_stride, void *workspace,
                            size_t workspace_bytes, void *stream);

/* The verify step's logits, greedy acceptance and emitted tokens in one
 * call: vc_lm_head_argmax over the B*M block rows h [B][M][Dm] into
 * argmax [B][M], then the acceptance of vc_accept (same outputs, same rule)
 * against draft [B][M-1].  The workspace is that of
 * vc_lm_head_argmax_workspace_size(B * M, V).                              */
vc_status vc_lm_head_accept(int32_t B, int32_t M, int32_t Dm, int32_t V, const void *h, const void *w,
                            const int32_t *draft, int32_t *argmax, int32_t *accept_len,
                            int32_t *out_tokens, int32_t *n_out, void *workspace,
                            size_t workspace_bytes, void *stream);

/* Commit after acceptance ("Algoritmo Principale", step 3: the process
 * restarts from the last accepted token): append the verified K/V rows of
 * x0, d_1..d_n -- the first n_out[b] rows of the block -- to a cache at its
 * current length, and advance the length.
 *   blk_k [B][Hkv][M][D], blk_v [B][Hkv][D][M]        (dtype)
 *   dst_k [B][Hkv][cap][D]                            (dtype)
 *   dst_v [B][Hkv][D][cap] when dst_v_blocked = 0 (a full cache, as
 *         vc_verify_attn reads it), [B][Hkv][cap/32][D][32] when it is 1 (a
 *         compressed main segment, as vc_draft_attn reads it; cap % 32 == 0)
 *   len [B][Hkv] (in/out), n_out [B]
 *   degree: optional [B][Hd][cap] (Hd = 1 when degree_h_stride = 0, else
 *   Hkv); appended rows get degree 1.
 * Rows past cap are dropped (the length saturates at cap).                 */
vc_status vc_commit_rows(int32_t B, int32_t Hkv, int32_t D, int32_t M, int32_t dtype, int64_t cap,
                         int32_t dst_v_blocked, const void *blk_k, const void *blk_v, const int32_t *n_out,
                         void *dst_k, void *dst_v, int32_t *len, float *degree,
                         int64_t degree_h_stride, void *stream);

/* ------------------------------------------------------------------------ */
/* Compressed-cache construction for a token-eviction compressor ("Riepilogo
 * Tecnico: VeriCache", "Supporto Architetturale": eviction policies sit
 * behind the same compression interface; the kept set is per token, shared
 * by a request's KV heads).  For request b, KV head h and j < n_kept[b]:
 *   dst_k[b][h][j] = src_k[b][h][idx[b][j]]
 *   token j of dst_v[b][h] = token idx[b][j] of src_v[b][h]
 *   src_k [B][Hkv][src_cap][D], src_v [B][Hkv][D][src_cap]   (a full cache,
 *         as vc_verify_attn reads it)
 *   dst_k [B][Hkv][cap][D], dst_v [B][Hkv][cap/32][D][32]    (the main segment
 *         of vc_draft_attn)
 *   idx int32 [B][idx_stride] (device; any order, ascending keeps positions in
 *   order), n_kept int32 [B] (device, clamped to [0, min(cap, idx_stride)]),
 *   dst_len int32 [B][Hkv] (device, optional) set to the clamped n_kept.
 * dtype VC_BF16 or VC_FP32; D in {64, 128}; cap % 32 == 0; all K/V buffers
 * 16-byte aligned.  An index outside [0, src_cap) writes a zero row; rows at
 * or past n_kept are not written.  Source and destination must not overlap.*/
vc_status vc_compact_kv(int32_t B, int32_t Hkv, int32_t D, int32_t dtype, const void *src_k, const void *src_v,
                        int64_t src_cap, const int32_t *idx, int64_t idx_stride, const int32_t *n_kept,
                        void *dst_k, void *dst_v, int64_t cap, int32_t *dst_len, void *stream);

/* ------------------------------------------------------------------------ */
/* Int4 group quantization into the compressed-cache format vc_draft_attn
 * reads with fmt = VC_KV_INT4 ("Riepilogo Tecnico: VeriCache", "Supporto
 * Architetturale": the drafter's cache may come from a quantizer behind the
 * same interface as eviction; the pages fix no scheme, this library reads it
 * as asymmetric min/max over 32-element groups).  For every (b, KV head) and
 * group j < n_groups, the 32 bf16 tokens src_start[bh] + 32 j .. + 31 of the
 * source are quantized into tokens dst_start[bh] + 32 j .. of the cache:
 *   K: one group = one channel over the 32 tokens; V: one group = one token
 *   over 32 channels;  s = (max - min) / 15 and z = min, each rounded to
 *   binary16 (nearest even);  code = clip(rint((x - z) / s), 0, 15), ties to
 *   even, 0 when s == 0 (exactly, as an exact evaluation decides).
 *   src_k [B][Hkv][src_cap][D], src_v [B][Hkv][D][src_cap]  bf16 (the tail
 *         layouts of vc_draft_attn)
 *   src_start, dst_start [B][Hkv] int32 (device); dst_start % 32 == 0; a
 *         (b, KV head) whose groups would leave [0, src_cap) or [0, cap), or
 *         whose dst_start is negative or not a multiple of 32, is skipped
 *   k_codes, k_scale, k_zero, v_codes, v_scale, v_zero: the INT4 layouts of
 *         vc_draft_args with capacity cap (a multiple of 32); only the
 *         written groups' bytes change.
 * D = 128; n_groups <= 65535; inputs finite with |x| <= 65504; src_k, src_v
 * and the code buffers 16-byte aligned.  vc_draft_attn reads the result only
 * while every scale stays below 2^9, i.e. groups spanning less than about
 * 7680 (see the range note of vc_draft_args).  Appending
 * verified tokens to an int4 cache (flushing full 32-token groups of the bf16
 * tail) and building the cache from a full bf16 cache are both this call.    */
vc_status vc_quantize_int4(int32_t B, int32_t Hkv, int32_t D, const void *src_k, const void *src_v,
                           int64_t src_cap, const int32_t *src_start, int32_t n_groups, int64_t cap,
                           const int32_t *dst_start, void *k_codes, void *k_scale, void *k_zero, void *v_codes,
                           void *v_scale, void *v_zero, void *stream);

/* Commit of verified rows into a packed int4 cache through its bf16 tail
 * ("Algoritmo Principale", step 3, with the quantizing drafter of "Supporto
 * Architetturale"): int4 groups span 32 tokens, so verified rows wait in a
 * bf16 tail -- the tail segment vc_draft_attn reads after the int4 main
 * segment -- until a whole group is there.  Per request b and KV head h:
 *   rows = tail[0 .. tail_len[b]) followed by the block's first n_out[b]
 *   rows (at most M, and only as many as fit tcap); its full 32-token groups
 *   are quantized (exactly as vc_quantize_int4_packed) into the packed cache
 *   at token main_len[b][h], which advances by their tokens; the remaining
 *   rows (< 32) move to the front of the tail and tail_len[b] becomes their
 *   count.  When the cache has no room for all the groups of a (b, h) (or
 *   main_len is not a multiple of 32) they are dropped and main_len stays.
 *   blk_k [B][Hkv][M][D], blk_v [B][Hkv][D][M] bf16 (the verify block);
 *   n_out [B] (device); tail_k [B][Hkv][tcap][D], tail_v [B][Hkv][D][tcap]
 *   bf16; tail_len [B] (device, in/out); packed u8 [B][Hkv][cap/32][5120];
 *   main_len [B][Hkv] (device, in/out).
 * D = 128; cap % 32 == 0; tcap >= 32 (tcap >= 31 + M keeps every row);
 * buffers 16-byte aligned.  Three launches on `stream`, no host round trip.  */
vc_status vc_int4_commit(int32_t B, int32_t Hkv, int32_t D, int32_t M, const void *blk_k, const void *blk_v,
                         const int32_t *n_out, void *tail_k, void *tail_v, int64_t tcap, int32_t *tail_len,
                         void *packed, int64_t cap, int32_t *main_len, void *stream);

/* The same quantization into the interleaved fmt = VC_KV_INT4_PACKED cache:
 * packed u8 [B][Hkv][cap/32][5120] (block layout as in vc_draft_args).
 * Arguments, decisions and errors as vc_quantize_int4.                      */
vc_status vc_quantize_int4_packed(int32_t B, int32_t Hkv, int32_t D, const void *src_k, const void *src_v,
                                  int64_t src_cap, const int32_t *src_start, int32_t n_groups, int64_t cap,
                                  const int32_t *dst_start, void *packed, void *stream);

/* ------------------------------------------------------------------------ */
/* One clustering round of Chunked Soft Matching ("Riassunto Tecnico:
 * CentroidKV", "Componenti Chiave" items 1-4) over a compressed cache in the
 * dense main-segment layout of vc_draft_args, producing the merged subset and
 * its degrees n_t for the log-degree term of vc_draft_attn.  Per (b, KV head)
 * over the first n_in tokens:
 *   tokens [0, n_sink) and [n_in - n_recent, n_in) pass through unchanged;
 *   the rest is cut into chunks of `chunk` tokens (the last may be shorter);
 *   in a chunk, A = even positions, B = odd positions; each A token's match
 *   is the B token of its chunk with the largest key cosine (lowest index on
 *   equal values); the floor(r * |A|) A tokens with the largest cosine
 *   (lower index first on equal values) merge into their matches;
 *   a cluster's key and value are the degree-weighted means of its members
 *   (fp32, rounded to bf16), its degree the sum; unmerged tokens are copied
 *   bit-exactly; survivors keep ascending position.
 * One call is one round (the schedule that decides when rounds run and with
 * which r is vc_csm_round_due / vc_csm_schedule_ratio below).  The survivor
 * count, the same for every (b, KV head), is returned in *n_out (host)
 * before launch, and written to out_len[b][h] (device, optional) by the
 * launch; output tokens past it are not written.
 *   in_k [B][Hkv][cap_in][D], in_v [B][Hkv][cap_in/32][D][32]   bf16
 *   in_deg [B][Hkv][cap_in] fp32 (NULL: every degree 1)
 *   out_k [B][Hkv][cap_out][D], out_v [B][Hkv][cap_out/32][D][32]   bf16
 *   out_deg [B][Hkv][cap_out] fp32 (feed vc_draft_attn with
 *           degree_h_stride = cap_out; the drafter takes cap_out % 64 == 0)
 * D = 128; 2 <= chunk <= 128; 0 <= r <= 1; n_in <= 2^30; caps multiples of 32; K buffers
 * 16-byte aligned; in and out must not overlap.                              */
vc_status vc_csm_round(int32_t B, int32_t Hkv, int32_t D, int32_t n_in, int32_t n_sink, int32_t n_recent,
                       int32_t chunk, double r, const void *in_k, const void *in_v, const float *in_deg,
                       int64_t cap_in, void *out_k, void *out_v, float *out_deg, int64_t cap_out, int32_t *n_out,
                       int32_t *out_len, void *stream);

/* The CentroidKV schedule around vc_csm_round ("Riassunto Tecnico:
 * CentroidKV", "Componenti Chiave" item 2 "Pipeline di Inferenza": a first
 * round after the prefill when the cache exceeds the budget, then a round
 * every `every` decode steps to keep it within the budget; item 3 "Scheduling
 * Progressivo": the ratio decays linearly over rounds).  Host-only.
 *   vc_csm_round_due: 1 when a round is due after decode step `decode_step`
 *     (0 = right after the prefill; a check every `every` steps after that)
 *     for a cache of n_tokens, i.e. n_tokens > budget; 0 otherwise; -1 for
 *     every < 1 or a negative step.
 *   vc_csm_schedule_ratio: r_j = r_init - j * delta_r for round j (0-based,
 *     counting the rounds run so far), kept within [0, 1].
 * A round removes at most half of its middle segment (only one of the two
 * alternating sets merges away).                                            */
int32_t vc_csm_round_due(int64_t n_tokens, int64_t budget, int32_t decode_step, int32_t every);
double  vc_csm_schedule_ratio(double r_init, double delta_r, int32_t round);

/* ------------------------------------------------------------------------ */
/* Cross-resource staggering ("Innovazioni Chiave del Sistema", P1): while
 * some requests draft from HBM, the full cache of the requests that verify
 * is loaded from host memory over PCIe, so transfer overlaps compute.  The
 * stagger object owns a host-to-device copy stream and a device-to-host
 * write-back stream (both non-blocking, default priority) and the events of
 * a ring of `nslots` device staging slots:
 *   vc_stagger_stream_layer(l)  copy stream: wait until slot l % nslots is
 *                               released, copy `bytes` from pinned host
 *                               memory into it, mark layer l copied;
 *   vc_stagger_acquire(l)       `stream` waits for layer l's copy; returns
 *                               the slot holding it;
 *   vc_stagger_release(l)       marks (in `stream` order) that the slot of
 *                               layer l may be overwritten;
 *   vc_stagger_writeback        device-to-host copy on the write-back
 *                               stream, ordered after the work already
 *                               enqueued on `after` (commit of verified rows
 *                               to the host-resident full cache);
 *   vc_stagger_copy_ms          duration of layer l's last host-to-device
 *                               copy (valid after vc_stagger_sync).
 * Slots are caller-owned device buffers; host sources must be pinned
 * (hipHostMalloc) for the host-to-device copies to run on the copy (SDMA)
 * engines.  The runtime carries out the device-to-host write-backs, small
 * here, as blit kernels on the compute units.                              */
typedef struct vc_stagger vc_stagger;
vc_status vc_stagger_create(vc_stagger **out, void *const *slots, int32_t nslots, size_t slot_bytes,
                            int32_t max_layers);
vc_status vc_stagger_stream_layer(vc_stagger *s, int32_t layer, const void *host_src, size_t bytes);
vc_status vc_stagger_acquire(vc_stagger *s, int32_t layer, void *stream, void **slot);
vc_status vc_stagger_release(vc_stagger *s, int32_t layer, void *stream);
vc_status vc_stagger_writeback(vc_stagger *s, void *host_dst, const void *dev_src, size_t bytes, void *after);
vc_status vc_stagger_after(vc_stagger *s, void *stream);   /* copy stream waits for `stream` */
vc_status vc_stagger_sync(vc_stagger *s);
vc_status vc_stagger_copy_ms(vc_stagger *s, int32_t layer, float *ms);
vc_status vc_stagger_destroy(vc_stagger *s);

/* ------------------------------------------------------------------------ */
/* One round of the staggered schedule ("Innovazioni Chiave del Sistema",
 * P1: the runtime staggers requests so that while some draft from HBM the
 * others verify against a full cache brought over PCIe; the two cohorts
 * swap roles every round).  In one call the library enqueues, on the
 * caller's two compute streams and the stagger object's copy streams:
 *   drafting cohort (draft_stream): `steps` draft steps; step i runs the
 *     draft attention of every layer (draft[l], with tail_len replaced by
 *     step_tail_len[i] when given), then the LM head fused with the argmax
 *     over draft_hidden[i], writing draft column i of drafts [Bd][steps];
 *   verifying cohort (verify_stream): per layer l, the full cache is
 *     streamed from host_kv[l] into the slot ring (K at the slot's start, V
 *     at v_offset), verify[l] runs against it (its ctx_k/ctx_v are ignored),
 *     and the slot is released for layer l + nslots; then the LM head fused
 *     with the argmax and the acceptance over verify_hidden [Bv][M][Dm]
 *     against verify_drafts [Bv][M-1] ("Algoritmo Principale", steps 2-3);
 *     then per layer the commit of the verified rows: vc_commit_rows of
 *     verify[l]'s block into commit[l] and the write-back of the block's K
 *     and V rows to commit[l].host_k / host_v.
 * mode VC_ROUND_STAGGERED enqueues the first nslots layer copies, then every
 * draft step back to back on the draft stream, then the verify layers, with
 * no wait between the two compute streams: the copies run while the drafting
 * cohort computes.  The verify kernels that free the slots queue behind the
 * draft kernels for the CUs, so the ring needs enough slots to keep the link
 * busy through the drafting (six of 8 GiB at the 128K shape; two stall it).
 * VC_ROUND_BULK is the bulk-synchronous comparison: every draft step first,
 * and the copy and verify streams wait for them.  Both modes run the same kernels on the same
 * inputs, so their outputs are identical bit for bit.  VC_ROUND_CHAINED is
 * one cohort in both roles (a long context: "Supporto Architetturale"):
 * the verify stream waits for the draft steps, since it verifies the drafts
 * they write (verify_drafts may be drafts), while the copies of the first
 * layers already stream during the drafting; with `fetch` the compressed
 * cache itself comes over the link first (remote prefix caching) and each
 * layer's first draft call waits for its part.
 * Every argument of every call is validated before anything is enqueued; on
 * VC_EINVAL nothing was enqueued (VC_EHIP: a launch failed part-way; the
 * caller synchronizes and discards the round).  The call returns without
 * synchronizing; vc_stagger_sync and the caller's streams tell completion.
 * `before_verify` (optional) is called on the host just before layer l's
 * verify is enqueued, with the verify stream (e.g. to insert markers or a
 * bounded stall).  Workspaces: each cohort's draft[l].workspace,
 * verify[l].workspace and LM-head workspaces as their entry points require;
 * the draft calls of one round may share one workspace (they run in order
 * on draft_stream), and so may the verify calls.                            */
#define VC_ROUND_STAGGERED 0
#define VC_ROUND_BULK 1
#define VC_ROUND_CHAINED 2

#define VC_COMMIT_ROWS 0          /* vc_commit_rows into a dense cache               */
#define VC_COMMIT_INT4_TAIL 1     /* vc_int4_commit into a packed int4 cache         */

typedef struct vc_round_commit {
  int32_t  kind;                  /* VC_COMMIT_ROWS or VC_COMMIT_INT4_TAIL           */
  void    *dst_k, *dst_v;         /* ROWS: the layer's cache the rows go to          */
  int32_t *len;                   /* ROWS: [Bv][Hkv], advanced by n_out              */
  float   *degree;                /* ROWS: optional merge degrees (appended rows: 1) */
  int64_t  degree_h_stride;       /* ROWS: 0 or cap                                  */
  int64_t  cap;                   /* ROWS: dense capacity; INT4_TAIL: int4 capacity  */
  int32_t  dst_v_blocked;         /* ROWS: 1 a compressed main segment, 0 full cache */
  void    *tail_k, *tail_v;       /* INT4_TAIL: the bf16 tail and its capacity       */
  int64_t  tcap;
  int32_t *tail_len;              /* INT4_TAIL: [Bv] (in/out)                        */
  void    *packed;                /* INT4_TAIL: [Bv][Hkv][cap/32][5120]              */
  int32_t *main_len;              /* INT4_TAIL: [Bv][Hkv] (in/out)                   */
  void    *host_k, *host_v;       /* optional pinned destinations of the block rows  */
} vc_round_commit;

typedef void (*vc_round_hook)(void *ctx, int32_t layer, void *verify_stream);

/* What a timed round measures (vc_round_desc::time_kernels).
 *   VC_TIME_DRAFT_STEPS: each draft step's run of `layers` draft attention
 *     calls (their split merges included), and each layer's verify call.
 *   VC_TIME_ATTENTION_KERNELS: each draft and verify attention kernel alone,
 *     the split merge that follows it left outside the event pair.        */
typedef enum { VC_TIME_NONE = 0, VC_TIME_DRAFT_STEPS = 1, VC_TIME_ATTENTION_KERNELS = 2 } vc_round_timing;

/* A copy a chained round starts before any other: the compressed cache of a
 * request whose prefix is held in host memory ("Supporto Architetturale",
 * remote prefix caching: the drafter needs only the compressed cache, so it
 * starts once that has arrived while the full cache is still on its way).
 * `bytes` from pinned host memory to a device buffer; the first draft step's
 * call for `layer` waits for every fetch of that layer.                     */
typedef struct vc_round_fetch {
  const void *host_src;           /* pinned host                                     */
  void       *dev_dst;            /* device, e.g. the layer's packed int4 cache      */
  size_t      bytes;
  int32_t     layer;              /* 0 .. layers-1                                   */
} vc_round_fetch;

typedef struct vc_round_desc {
  int32_t layers;                 /* 1 .. the stagger object's max_layers            */
  int32_t steps;                  /* draft steps (0: no drafting cohort)             */
  int32_t mode;                   /* VC_ROUND_STAGGERED, _BULK or _CHAINED           */
  /* LM head of the model, vocab-major [V][Dm] bf16 */
  const void *lm_w;
  int32_t Dm, V;
  /* drafting cohort */
  const vc_draft_args *draft;     /* [layers]                                        */
  const int32_t *const *step_tail_len; /* optional [steps] device [Bd]               */
  const void *const *draft_hidden;     /* [steps] device [Bd][Dm] bf16               */
  int32_t *drafts;                /* device [Bd][steps]                              */
  void   *draft_lm_ws;            /* vc_lm_head_argmax_workspace_size(Bd, V)         */
  size_t  draft_lm_ws_bytes;
  /* verifying cohort (verify == NULL: none) */
  const vc_verify_args *verify;   /* [layers]                                        */
  const void *const *host_kv;     /* [layers] pinned host: the layer's full K then V */
  size_t  kv_bytes;               /* bytes streamed per layer (<= slot bytes)        */
  size_t  v_offset;               /* offset of V in the slot, multiple of 16         */
  const void    *verify_hidden;   /* device [Bv][M][Dm] bf16                         */
  const int32_t *verify_drafts;   /* device [Bv][M-1]                                */
  int32_t *argmax, *accept_len, *out_tokens, *n_out;   /* as vc_lm_head_accept       */
  void   *verify_lm_ws;           /* vc_lm_head_argmax_workspace_size(Bv * M, V)     */
  size_t  verify_lm_ws_bytes;
  const vc_round_commit *commit;  /* optional [layers]                               */
  vc_round_hook before_verify;    /* optional                                        */
  void   *hook_ctx;
  int32_t time_kernels;           /* vc_round_timing: events on the compute streams
                                     (vc_stagger_round_times)                        */
  const vc_round_fetch *fetch;    /* optional [n_fetch], VC_ROUND_CHAINED with steps
                                     > 0 only: enqueued in order on the copy stream
                                     ahead of the layer copies                       */
  int32_t n_fetch;
} vc_round_desc;

vc_status vc_stagger_round(vc_stagger *s, const vc_round_desc *d, void *draft_stream, void *verify_stream);

/* Durations (ms) of the last timed round, valid once its streams have
 * completed.  VC_TIME_DRAFT_STEPS: draft_ms[i] spans draft step i's `layers`
 * back-to-back draft attention calls (the LM head excluded), verify_ms[l]
 * layer l's verify call.  VC_TIME_ATTENTION_KERNELS: draft_ms[i * layers + l]
 * is layer l's draft attention kernel in step i and verify_ms[l] layer l's
 * verify attention kernel, each without its split merge.  *n_draft and
 * *n_verify are set to the counts; the arrays (host, may be NULL to query
 * the counts) must hold at least that many entries.                        */
vc_status vc_stagger_round_times(vc_stagger *s, float *draft_ms, int32_t *n_draft, float *verify_ms,
                                 int32_t *n_verify);

/* ------------------------------------------------------------------------ */
const char *vc_status_string(vc_status s);
const char *vc_last_error(void);   /* thread-local message of the last failure */
const char *vc_build_info(void);   /* target, compile flags                    */

#ifdef __cplusplus
}
#endif
#endif /* VC_H */
