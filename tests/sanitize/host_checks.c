/*
 * Host-side checks of libvc's argument validation and error paths, built with
 * AddressSanitizer and UndefinedBehaviorSanitizer on the host code (see
 * tests/test_host_sanitizers.py).  Every call here is refused by the host
 * before any GPU work -- malformed shapes, null pointers, sizes past a
 * limit, a stagger object on a machine without a usable device -- or is a
 * pure host function; a sanitizer report or a wrong status fails the run.
 * Device pointers are never dereferenced by the host code, so stand-in
 * addresses are used where a call must get past its null checks.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "vc.h"
#include "vc_tiny.h"

static int failures = 0;

#define EXPECT(cond, what)                                                        \
  do {                                                                            \
    if (!(cond)) {                                                                \
      fprintf(stderr, "FAILED: %s (line %d): %s\n", what, __LINE__, vc_last_error()); \
      ++failures;                                                                 \
    }                                                                             \
  } while (0)

#define EXPECT_ERR(call, what)                                      \
  do {                                                              \
    vc_status st_ = (call);                                         \
    EXPECT(st_ != VC_OK, what);                                     \
    EXPECT(vc_last_error() && vc_last_error()[0], what " (message)"); \
  } while (0)

/* a stand-in device address: aligned, never dereferenced by the host */
#define FAKE ((void *)(uintptr_t)0x10000000u)

static vc_draft_args draft_ok(void) {
  vc_draft_args a;
  memset(&a, 0, sizeof a);
  a.B = 2; a.Hq = 8; a.Hkv = 2; a.D = 128; a.dtype = VC_BF16; a.fmt = VC_KV_DENSE; a.scale = 0.088f;
  a.cap = 1024; a.q = FAKE; a.main_len = (int32_t *)FAKE; a.k = FAKE; a.v = FAKE; a.out = FAKE;
  return a;
}

static vc_verify_args verify_ok(void) {
  vc_verify_args a;
  memset(&a, 0, sizeof a);
  a.B = 1; a.Hq = 8; a.Hkv = 2; a.D = 128; a.M = 9; a.dtype = VC_BF16; a.scale = 0.088f;
  a.ccap = 1024; a.q = FAKE; a.ctx_k = FAKE; a.ctx_v = FAKE; a.ctx_len = (int32_t *)FAKE;
  a.blk_k = FAKE; a.blk_v = FAKE; a.out = FAKE;
  return a;
}

static void draft_checks(void) {
  vc_draft_args a;
  EXPECT_ERR(vc_draft_attn(NULL, NULL), "draft: null struct");
  a = draft_ok(); a.Hq = 7;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: Hq not a multiple of Hkv");
  a = draft_ok(); a.D = 96;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: head_dim");
  a = draft_ok(); a.cap = 1000;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: cap not a multiple of the block");
  a = draft_ok(); a.cap = (int64_t)1 << 40;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: capacity past 2^30");
  a = draft_ok(); a.B = 70000;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: too many slices");
  a = draft_ok(); a.q = NULL;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: null q");
  a = draft_ok(); a.scale = 0.f;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: zero scale");
  a = draft_ok(); a.dtype = 9;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: dtype");
  a = draft_ok(); a.fmt = VC_KV_INT4; a.dtype = VC_FP32;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: int4 in fp32");
  a = draft_ok(); a.tail_len = (int32_t *)FAKE; a.tail_k = NULL;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: tail length without a tail");
  a = draft_ok(); a.cap = 65536; a.workspace = NULL; a.workspace_bytes = 0; a.num_splits = 64;
  EXPECT_ERR(vc_draft_attn(&a, NULL), "draft: forced splits without a workspace");
  a = draft_ok(); a.q = NULL;
  EXPECT_ERR(vc_draft_attn_noalloc(&a, NULL), "draft noalloc: null q");
  EXPECT_ERR(vc_draft_attn_noalloc(NULL, NULL), "draft noalloc: null struct");
  EXPECT(vc_draft_workspace_size(NULL) == 0, "draft workspace of a null struct");
  EXPECT(vc_draft_noalloc_max_scratch() > 0, "noalloc scratch size");
  a = draft_ok(); a.B = 0;
  EXPECT(vc_draft_attn(&a, NULL) == VC_OK, "draft: empty batch is a no-op");
}

static void verify_checks(void) {
  vc_verify_args a;
  EXPECT_ERR(vc_verify_attn(NULL, NULL), "verify: null struct");
  a = verify_ok(); a.M = 0;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: empty block");
  a = verify_ok(); a.Hkv = 3;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: Hq not a multiple of Hkv");
  a = verify_ok(); a.ccap = (int64_t)1 << 40;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: context past 2^30");
  a = verify_ok(); a.M = 1 << 24; a.Hq = 64; a.Hkv = 1;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: packed rows past the grid");
  a = verify_ok(); a.blk_v = NULL;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: null block V");
  a = verify_ok(); a.ccap = 65536; a.num_splits = 3; a.workspace = NULL;
  EXPECT_ERR(vc_verify_attn(&a, NULL), "verify: splits without a workspace");
  EXPECT(vc_verify_workspace_size(NULL) == 0, "verify workspace of a null struct");
  a = verify_ok(); a.B = 0;
  EXPECT(vc_verify_attn(&a, NULL) == VC_OK, "verify: empty batch is a no-op");
}

static void accept_checks(void) {
  vc_accept_args a;
  EXPECT_ERR(vc_accept(NULL, NULL), "accept: null struct");
  memset(&a, 0, sizeof a);
  a.B = 2; a.M = 0; a.V = 10;
  EXPECT_ERR(vc_accept(&a, NULL), "accept: M = 0");
  a.M = 3; a.logit_dtype = 5;
  EXPECT_ERR(vc_accept(&a, NULL), "accept: logit dtype");
  a.logit_dtype = VC_FP32;
  EXPECT_ERR(vc_accept(&a, NULL), "accept: null outputs");
  a.logits = FAKE; a.argmax = (int32_t *)FAKE; a.accept_len = (int32_t *)FAKE;
  a.out_tokens = (int32_t *)FAKE; a.n_out = (int32_t *)FAKE; a.draft = NULL;
  EXPECT_ERR(vc_accept(&a, NULL), "accept: drafts required when M > 1");
  a.draft = (const int32_t *)FAKE; a.logits = (const void *)((uintptr_t)FAKE + 4);
  EXPECT_ERR(vc_accept(&a, NULL), "accept: misaligned logits");
  EXPECT_ERR(vc_argmax(-1, 10, VC_FP32, FAKE, (int32_t *)FAKE, 1, NULL), "argmax: negative rows");
  EXPECT_ERR(vc_argmax(4, 10, VC_FP32, FAKE, (int32_t *)FAKE, 0, NULL), "argmax: zero stride");
  EXPECT_ERR(vc_argmax(4, 10, VC_FP32, NULL, (int32_t *)FAKE, 1, NULL), "argmax: null logits");
  EXPECT(vc_argmax(0, 10, VC_FP32, NULL, NULL, 1, NULL) == VC_OK, "argmax: no rows is a no-op");
  EXPECT_ERR(vc_next_input(-1, 3, (const int32_t *)FAKE, (const int32_t *)FAKE, (int32_t *)FAKE, 1, NULL),
             "next input: negative batch");
  EXPECT_ERR(vc_next_input(2, 0, (const int32_t *)FAKE, (const int32_t *)FAKE, (int32_t *)FAKE, 1, NULL),
             "next input: empty block");
  EXPECT_ERR(vc_next_input(2, 3, NULL, (const int32_t *)FAKE, (int32_t *)FAKE, 1, NULL), "next input: null tokens");
  EXPECT_ERR(vc_next_input(2, 3, (const int32_t *)FAKE, (const int32_t *)FAKE, (int32_t *)FAKE, 0, NULL),
             "next input: zero stride");
}

static void lmhead_checks(void) {
  EXPECT_ERR(vc_lm_head_argmax(4, 100, 1000, FAKE, FAKE, (int32_t *)FAKE, 1, FAKE, 1 << 20, NULL),
             "LM head: Dm not a multiple of 32");
  EXPECT_ERR(vc_lm_head_argmax(4, 128, 1000, FAKE, FAKE, (int32_t *)FAKE, 1, FAKE, 4, NULL),
             "LM head: short workspace");
  EXPECT_ERR(vc_lm_head_argmax(4, 128, 1000, NULL, FAKE, (int32_t *)FAKE, 1, FAKE, 1 << 20, NULL),
             "LM head: null hidden rows");
  EXPECT_ERR(vc_lm_head_accept(2, 0, 128, 1000, FAKE, FAKE, (const int32_t *)FAKE, (int32_t *)FAKE,
                               (int32_t *)FAKE, (int32_t *)FAKE, (int32_t *)FAKE, FAKE, 1 << 20, NULL),
             "LM head accept: empty block");
  EXPECT(vc_lm_head_argmax_workspace_size(0, 1000) == 0, "LM head workspace of zero rows");
  EXPECT(vc_lm_head_argmax_workspace_size(4, 1000) >= 4 * sizeof(int32_t), "LM head workspace of four rows");
  /* the largest vocabulary: the tile count must not overflow */
  EXPECT(vc_lm_head_argmax_workspace_size(1, INT32_MAX) > 0, "LM head workspace of a 2^31 - 1 vocabulary");
}

static void cache_checks(void) {
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 0, VC_BF16, 1024, 0, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: empty block");
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 9, 7, 1024, 0, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: dtype");
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 9, VC_BF16, 1024, 2, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: V layout flag");
  EXPECT_ERR(vc_commit_rows(70000, 2, 128, 9, VC_BF16, 1024, 0, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: too many slices");
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 9, VC_BF16, 1024, 0, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, (float *)FAKE, 7, NULL),
             "commit: degree stride");
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 9, VC_BF16, 1000, 1, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: blocked V with cap not a multiple of 32");
  EXPECT_ERR(vc_commit_rows(2, 2, 128, 9, VC_BF16, 1024, 0, NULL, FAKE, (const int32_t *)FAKE, FAKE, FAKE,
                            (int32_t *)FAKE, NULL, 0, NULL),
             "commit: null block K");
  EXPECT_ERR(vc_compact_kv(2, 2, 128, VC_BF16, FAKE, FAKE, 4096, (const int32_t *)FAKE, 4096,
                           (const int32_t *)FAKE, FAKE, FAKE, 1000, NULL, NULL),
             "compaction: cap not a multiple of 32");
  EXPECT_ERR(vc_compact_kv(70000, 1, 128, VC_BF16, FAKE, FAKE, 4096, (const int32_t *)FAKE, 4096,
                           (const int32_t *)FAKE, FAKE, FAKE, 1024, NULL, NULL),
             "compaction: too many slices");
  EXPECT_ERR(vc_quantize_int4(1, 2, 128, FAKE, FAKE, 4096, (const int32_t *)FAKE, 70000, 4096,
                              (const int32_t *)FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL),
             "quantizer: too many groups");
  EXPECT_ERR(vc_quantize_int4(1, 2, 64, FAKE, FAKE, 4096, (const int32_t *)FAKE, 4, 4096, (const int32_t *)FAKE,
                              FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, NULL),
             "quantizer: head_dim 64");
  EXPECT_ERR(vc_quantize_int4_packed(1, 2, 128, FAKE, FAKE, 4096, (const int32_t *)FAKE, 4, 4016,
                                     (const int32_t *)FAKE, FAKE, NULL),
             "packed quantizer: cap not a multiple of 32");
  EXPECT_ERR(vc_int4_commit(1, 2, 128, 9, FAKE, FAKE, (const int32_t *)FAKE, FAKE, FAKE, 16, (int32_t *)FAKE,
                            FAKE, 4096, (int32_t *)FAKE, NULL),
             "int4 commit: tail shorter than a group");
  EXPECT_ERR(vc_int4_commit(1, 2, 128, 9, FAKE, FAKE, NULL, FAKE, FAKE, 64, (int32_t *)FAKE, FAKE, 4096,
                            (int32_t *)FAKE, NULL),
             "int4 commit: null n_out");
  int32_t n_out = -1;
  EXPECT_ERR(vc_csm_round(1, 2, 128, 600, 4, 64, 1, 0.5, FAKE, FAKE, NULL, 640, FAKE, FAKE, (float *)FAKE, 640,
                          &n_out, NULL, NULL),
             "CSM: chunk below 2");
  EXPECT_ERR(vc_csm_round(1, 2, 128, 600, 4, 64, 64, 1.5, FAKE, FAKE, NULL, 640, FAKE, FAKE, (float *)FAKE, 640,
                          &n_out, NULL, NULL),
             "CSM: ratio above 1");
  EXPECT_ERR(vc_csm_round(1, 2, 128, 600, 4, 64, 64, 0.5, FAKE, FAKE, NULL, 640, FAKE, FAKE, (float *)FAKE, 64,
                          &n_out, NULL, NULL),
             "CSM: output capacity too small");
  EXPECT_ERR(vc_csm_round(1, 2, 128, 1 << 30, 0, 0, 2, 0.5, FAKE, FAKE, NULL, (int64_t)1 << 30, FAKE, FAKE,
                          (float *)FAKE, (int64_t)1 << 30, &n_out, NULL, NULL),
             "CSM: more chunks than a grid row");
  /* sums of large counts must be rejected, not wrap */
  EXPECT_ERR(vc_csm_round(1, 2, 128, INT32_MAX - 64, INT32_MAX - 64, INT32_MAX - 64, 128, 0.5, FAKE, FAKE, NULL,
                          (int64_t)1 << 31, FAKE, FAKE, (float *)FAKE, (int64_t)1 << 31, &n_out, NULL, NULL),
             "CSM: sinks + recent past 2^31");
  EXPECT_ERR(vc_csm_round(1, 2, 128, INT32_MAX, 0, 0, 128, 0.5, FAKE, FAKE, NULL, (int64_t)1 << 31, FAKE, FAKE,
                          (float *)FAKE, (int64_t)1 << 31, &n_out, NULL, NULL),
             "CSM: n_in of 2^31 - 1");
  n_out = -1;
  EXPECT(vc_csm_round(0, 2, 128, 600, 4, 64, 64, 0.5, NULL, NULL, NULL, 640, NULL, NULL, NULL, 640, &n_out, NULL,
                      NULL) == VC_OK && n_out > 0 && n_out < 600,
         "CSM: survivor count of an empty batch");
  EXPECT(vc_csm_round_due(10, 5, 3, 0) == -1, "CSM schedule: period 0");
  EXPECT(vc_csm_round_due(10, 5, 0, 4) == 1 && vc_csm_round_due(4, 5, 0, 4) == 0, "CSM schedule: after prefill");
  EXPECT(vc_csm_round_due(10, 5, 3, 4) == 0 && vc_csm_round_due(10, 5, 8, 4) == 1, "CSM schedule: decode steps");
  EXPECT(vc_csm_schedule_ratio(0.5, 0.25, 3) == 0.0 && vc_csm_schedule_ratio(1.5, 0.0, 0) == 1.0,
         "CSM schedule: ratio clamped");
}

static void stagger_checks(void) {
  vc_stagger *s = NULL;
  void *slots[2] = {FAKE, FAKE};
  EXPECT_ERR(vc_stagger_create(NULL, slots, 2, 1 << 20, 4), "stagger: null output");
  EXPECT_ERR(vc_stagger_create(&s, NULL, 2, 1 << 20, 4), "stagger: null slots");
  EXPECT_ERR(vc_stagger_create(&s, slots, 0, 1 << 20, 4), "stagger: no slots");
  EXPECT_ERR(vc_stagger_create(&s, slots, 2, 1 << 20, 0), "stagger: no layers");
  EXPECT_ERR(vc_stagger_stream_layer(NULL, 0, FAKE, 16), "stagger: null object (stream)");
  EXPECT_ERR(vc_stagger_acquire(NULL, 0, NULL, NULL), "stagger: null object (acquire)");
  EXPECT_ERR(vc_stagger_release(NULL, 0, NULL), "stagger: null object (release)");
  EXPECT_ERR(vc_stagger_writeback(NULL, FAKE, FAKE, 16, NULL), "stagger: null object (writeback)");
  EXPECT_ERR(vc_stagger_after(NULL, NULL), "stagger: null object (after)");
  EXPECT_ERR(vc_stagger_sync(NULL), "stagger: null object (sync)");
  float ms = 0.f;
  EXPECT_ERR(vc_stagger_copy_ms(NULL, 0, &ms), "stagger: null object (copy_ms)");
  EXPECT(vc_stagger_destroy(NULL) == VC_OK, "stagger: destroying nothing");
  vc_round_desc d;
  memset(&d, 0, sizeof d);
  EXPECT_ERR(vc_stagger_round(NULL, &d, NULL, NULL), "round: null object");
  int32_t nd = 0, nv = 0;
  EXPECT_ERR(vc_stagger_round_times(NULL, NULL, &nd, NULL, &nv), "round times: null object");
  /* a real object needs streams: on a machine without a usable GPU the
     create fails and must leave nothing behind (the leak checker sees) */
  vc_status st = vc_stagger_create(&s, slots, 2, 1 << 20, 4);
  if (st == VC_OK) {
    EXPECT_ERR(vc_stagger_round(s, NULL, NULL, NULL), "round: null descriptor");
    d.layers = 9;
    EXPECT_ERR(vc_stagger_round(s, &d, NULL, NULL), "round: more layers than the object holds");
    d.layers = 2; d.mode = 7;
    EXPECT_ERR(vc_stagger_round(s, &d, NULL, NULL), "round: unknown mode");
    d.mode = VC_ROUND_STAGGERED; d.n_fetch = 1;
    EXPECT_ERR(vc_stagger_round(s, &d, NULL, NULL), "round: a fetch outside the chained mode");
    EXPECT(vc_stagger_destroy(s) == VC_OK, "stagger: destroy");
  }
}

static void tiny_checks(void) {
  float c[4 * 4], sn[4 * 4];
  EXPECT(vc_tiny_rope_table(4, 8, 10000.f, c, sn) == VC_OK, "RoPE table on the host");
  EXPECT(c[0] == 1.f && sn[0] == 0.f, "RoPE table: position 0");
  EXPECT_ERR(vc_tiny_rope_table(4, 7, 10000.f, c, sn), "RoPE table: odd head_dim");
  EXPECT_ERR(vc_tiny_rope_table(4, 8, 10000.f, NULL, sn), "RoPE table: null output");
  EXPECT_ERR(vc_tiny_forward(NULL, 1, (const int32_t *)FAKE, 0, NULL, (float *)FAKE, FAKE, 0, NULL),
             "tiny forward: null model");
  vc_tiny_model m;
  memset(&m, 0, sizeof m);
  m.n_layers = 2; m.d_model = 256; m.n_q_heads = 4; m.n_kv_heads = 2; m.head_dim = 64; m.ffn = 1024;
  m.vocab = 512; m.rope_rows = 16;
  vc_tiny_attn at;
  memset(&at, 0, sizeof at);
  EXPECT_ERR(vc_tiny_forward(&m, 1, (const int32_t *)FAKE, 20, &at, (float *)FAKE, FAKE, 1 << 20, NULL),
             "tiny forward: positions past the RoPE table");
  EXPECT_ERR(vc_tiny_forward(&m, 4, (const int32_t *)FAKE, INT32_MAX - 1, &at, (float *)FAKE, FAKE, 1 << 20, NULL),
             "tiny forward: positions near 2^31");
  m.ffn = 8192;
  EXPECT_ERR(vc_tiny_forward(&m, 1, (const int32_t *)FAKE, 0, &at, (float *)FAKE, FAKE, 1 << 20, NULL),
             "tiny forward: ffn too wide");
  EXPECT(vc_tiny_workspace_size(NULL, 4) == 0, "tiny workspace of a null model");
  EXPECT(vc_evict_kept_count(1024, 4, 128, 8) == 243, "eviction count");
  EXPECT(vc_evict_kept_count(10, 4, 128, 0) == -1, "eviction count: stride 0");
  /* extreme arguments: sinks + recent and the stride rounding must not wrap */
  EXPECT(vc_evict_kept_count(INT32_MAX, INT32_MAX - 1, INT32_MAX - 1, 1) == INT32_MAX, "eviction count: huge keeps");
  EXPECT(vc_evict_kept_count(INT32_MAX, 1000, 0, INT32_MAX) == 1000, "eviction count: huge stride");
  EXPECT(vc_evict_kept_count(INT32_MAX, 0, 0, 1) == INT32_MAX, "eviction count: stride 1");
  EXPECT_ERR(vc_gather_rows(2, 64, 40, (const int32_t *)FAKE, (const float *)FAKE, (const float *)FAKE, 100,
                            (float *)FAKE, (float *)FAKE, 32, (int32_t *)FAKE, NULL),
             "gather: more rows than the destination holds");
  EXPECT_ERR(vc_gather_evict(2, 64, (const int32_t *)FAKE, 4, 128, 8, (const float *)FAKE, (const float *)FAKE,
                             1088, (float *)FAKE, (float *)FAKE, 64, (int32_t *)FAKE, NULL),
             "eviction gather: destination too small for a full source");
}

int main(void) {
  for (int st = 0; st < 4; ++st) EXPECT(strncmp(vc_status_string((vc_status)st), "VC_", 3) == 0, "status string");
  EXPECT(strcmp(vc_status_string((vc_status)99), "unknown vc_status") == 0, "unknown status string");
  EXPECT(vc_build_info() && vc_build_info()[0], "build info");
  draft_checks();
  verify_checks();
  accept_checks();
  lmhead_checks();
  cache_checks();
  stagger_checks();
  tiny_checks();
  if (failures) {
    fprintf(stderr, "%d host check(s) failed\n", failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
