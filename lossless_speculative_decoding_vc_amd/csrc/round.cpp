// One round of the staggered schedule, enqueued natively.
//
// "Riepilogo Tecnico: VeriCache", "Innovazioni Chiave del Sistema", P1:
// drafting is bound by HBM bandwidth and verification by the interconnect
// that brings the full cache from host memory; the runtime staggers requests
// so that one cohort drafts while the other verifies, and the cohorts swap
// roles every round.  "Algoritmo Principale": draft k tokens over the
// compressed cache, verify them in one pass over the full cache, accept up to
// the first mismatch (plus the bonus), restart from the last accepted token.
//
// vc_stagger_round checks every call of the round first and then enqueues
// the whole round from the host in one pass: the first layers' copies into
// the slot ring, the drafting cohort's k steps back to back (every layer's
// draft attention, then the LM head fused with the argmax) on the draft
// stream, the verifying cohort's layers on the verify stream, each after its
// layer's host-to-device copy, then the fused LM head + acceptance and the
// commit of the verified rows.  The draft stream never waits for a copy, so
// the copy engines stream the next layers while the drafting cohort
// computes; in the bulk-synchronous mode every draft step comes first and the
// copy and verify streams wait for them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <string>
#include <vector>

#include "launch.h"
#include "stagger_impl.h"

namespace {

vc_status bad(const std::string &m) { return vc::set_error(VC_EINVAL, m.c_str()); }

vc_status with_layer(vc_status st, const char *what, int i) {
  if (st == VC_OK) return st;
  const std::string m = std::string(what) + " " + std::to_string(i) + ": " + vc_last_error();
  return vc::set_error(st, m.c_str());
}

size_t elem_bytes(int32_t dtype) { return dtype == VC_BF16 ? 2 : 4; }

// Everything the round will call, checked before the first enqueue.
vc_status validate(const vc_stagger *s, const vc_round_desc *d) {
  if (!s || !d) return bad("null stagger or round descriptor");
  const int L = d->layers, k = d->steps;
  if (L < 1 || L > (int)s->copied.size())
    return bad("layers must lie in 1.." + std::to_string(s->copied.size()) + " (got " + std::to_string(L) + ")");
  if (k < 0) return bad("steps must be >= 0");
  if (d->mode != VC_ROUND_STAGGERED && d->mode != VC_ROUND_BULK && d->mode != VC_ROUND_CHAINED)
    return bad("unknown round mode");
  if (d->time_kernels < VC_TIME_NONE || d->time_kernels > VC_TIME_ATTENTION_KERNELS)
    return bad("unknown timing mode");
  if ((k > 0 || d->verify) && !d->lm_w) return bad("lm_w is required");
  if (k > 0) {
    if (!d->draft || !d->draft_hidden || !d->drafts) return bad("a drafting cohort needs draft, draft_hidden, drafts");
    const int Bd = d->draft[0].B;
    for (int l = 0; l < L; ++l) {
      if (d->draft[l].B != Bd) return bad("every layer's draft call must have the same batch");
      vc_draft_args a = d->draft[l];
      for (int i = 0; i < (d->step_tail_len ? k : 1); ++i) {
        if (d->step_tail_len) a.tail_len = d->step_tail_len[i];
        vc_status st = with_layer(vc::validate_draft_call(&a), "draft layer", l);
        if (st != VC_OK) return st;
      }
    }
    for (int i = 0; i < k; ++i) {
      vc_status st = with_layer(vc::check_lm_argmax(Bd, d->Dm, d->V, d->draft_hidden[i], d->lm_w, d->drafts,
                                                    d->draft_lm_ws, d->draft_lm_ws_bytes),
                                "drafting LM head, step", i);
      if (st != VC_OK) return st;
    }
  }
  if (d->n_fetch < 0) return bad("n_fetch must be >= 0");
  if (d->n_fetch > 0) {
    if (d->mode != VC_ROUND_CHAINED || k == 0) return bad("fetches need the chained mode with draft steps");
    if (!d->fetch) return bad("null fetch list");
    for (int j = 0; j < d->n_fetch; ++j) {
      const vc_round_fetch &f = d->fetch[j];
      if (!f.host_src || !f.dev_dst || f.bytes == 0 || f.layer < 0 || f.layer >= L)
        return bad("fetch " + std::to_string(j) + ": null pointer, no bytes or layer outside 0.." +
                   std::to_string(L - 1));
    }
  }
  if (d->verify) {
    if (!d->host_kv) return bad("a verifying cohort needs host_kv");
    if (d->kv_bytes > s->slot_bytes || d->v_offset >= d->kv_bytes || d->v_offset % 16)
      return bad("kv_bytes must fit a slot and v_offset lie inside it, a multiple of 16");
    const int Bv = d->verify[0].B, M = d->verify[0].M;
    for (int l = 0; l < L; ++l) {
      vc_verify_args a = d->verify[l];
      if (a.B != Bv || a.M != M) return bad("every layer's verify call must have the same batch and block");
      if (!d->host_kv[l]) return bad("null host_kv for layer " + std::to_string(l));
      const size_t need_k = (size_t)a.B * a.Hkv * a.ccap * a.D * elem_bytes(a.dtype);
      if (need_k > d->v_offset || d->v_offset + need_k > d->kv_bytes)
        return bad("layer " + std::to_string(l) + ": the context K and V do not fit kv_bytes at v_offset");
      a.ctx_k = s->slots[0];
      a.ctx_v = static_cast<char *>(s->slots[0]) + d->v_offset;
      vc_status st = with_layer(vc::validate_verify_call(&a), "verify layer", l);
      if (st != VC_OK) return st;
      if (d->commit) {
        const vc_round_commit &c = d->commit[l];
        if (c.kind == VC_COMMIT_ROWS) {
          st = with_layer(vc::check_commit(a.B, a.Hkv, a.D, a.M, a.dtype, c.cap, c.dst_v_blocked, a.blk_k, a.blk_v,
                                           d->n_out, c.dst_k, c.dst_v, c.len, c.degree, c.degree_h_stride),
                          "commit layer", l);
        } else if (c.kind == VC_COMMIT_INT4_TAIL) {
          st = with_layer(vc::check_int4_commit(a.B, a.Hkv, a.D, a.M, a.dtype, a.blk_k, a.blk_v, d->n_out, c.tail_k,
                                                c.tail_v, c.tcap, c.tail_len, c.packed, c.cap, c.main_len),
                          "int4 commit layer", l);
        } else {
          st = bad("unknown commit kind for layer " + std::to_string(l));
        }
        if (st != VC_OK) return st;
      }
    }
    if (!d->accept_len || !d->out_tokens || !d->n_out) return bad("null acceptance output");
    if (M > 1 && !d->verify_drafts) return bad("verify_drafts is required when M > 1");
    vc_status st = vc::check_lm_argmax(Bv * M, d->Dm, d->V, d->verify_hidden, d->lm_w, d->argmax, d->verify_lm_ws,
                                       d->verify_lm_ws_bytes);
    if (st != VC_OK) return st;
  }
  return VC_OK;
}

#define CHK(x)                           \
  do {                                   \
    vc_status st_ = (x);                 \
    if (st_ != VC_OK) return st_;        \
  } while (0)

// Event pairs for the timed calls of one round, taken from the object's pool.
struct RoundTimer {
  vc_stagger *s;
  int every;
  int next = 0;
  vc_status begin(hipStream_t st, bool on) {
    if (!on) return VC_OK;
    return hipEventRecord(s->round_ev[2 * next], st) == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, "timing event");
  }
  vc_status end(hipStream_t st, bool on) {
    if (!on) return VC_OK;
    const hipError_t e = hipEventRecord(s->round_ev[2 * next + 1], st);
    ++next;
    return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, "timing event");
  }
  // the closing event of the current pair, for a launch to record itself
  hipEvent_t take_end() { return s->round_ev[2 * next++ + 1]; }
};

// One draft attention call (validated with the round); with per-kernel
// timing its kernel alone sits between an event pair, the split merge after.
vc_status draft_call(const vc_draft_args &a, hipStream_t st, RoundTimer &tm) {
  if (tm.every != VC_TIME_ATTENTION_KERNELS) return vc_draft_attn(&a, st);
  CHK(tm.begin(st, true));
  if (a.B == 0) return tm.end(st, true);
  const hipError_t e = vc::launch_draft(a, vc::plan_draft(a), st, tm.take_end());
  return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, hipGetErrorString(e));
}

vc_status verify_call(const vc_verify_args &a, hipStream_t st, RoundTimer &tm) {
  if (tm.every != VC_TIME_ATTENTION_KERNELS) {
    CHK(tm.begin(st, tm.every > 0));
    CHK(vc_verify_attn(&a, st));
    return tm.end(st, tm.every > 0);
  }
  CHK(tm.begin(st, true));
  if (a.B == 0) return tm.end(st, true);
  const hipError_t e = vc::launch_verify(a, vc::plan_verify(a), st, tm.take_end());
  return e == hipSuccess ? VC_OK : vc::set_error(VC_EHIP, hipGetErrorString(e));
}

vc_status draft_step(const vc_round_desc *d, int i, void *ds, RoundTimer &tm, const vc_stagger *s) {
  // VC_TIME_DRAFT_STEPS: one event pair around the step's back-to-back draft
  // attention calls; VC_TIME_ATTENTION_KERNELS: one pair per kernel
  const bool step_pair = tm.every == VC_TIME_DRAFT_STEPS;
  CHK(tm.begin((hipStream_t)ds, step_pair));
  for (int l = 0; l < d->layers; ++l) {
    if (i == 0)   // the first use of each layer's compressed cache waits for its fetches
      for (int j = 0; j < d->n_fetch; ++j)
        if (d->fetch[j].layer == l && hipStreamWaitEvent((hipStream_t)ds, s->fetch_ev[j], 0) != hipSuccess)
          return vc::set_error(VC_EHIP, "waiting for a fetch");
    vc_draft_args a = d->draft[l];
    if (d->step_tail_len) a.tail_len = d->step_tail_len[i];
    CHK(draft_call(a, (hipStream_t)ds, tm));
  }
  CHK(tm.end((hipStream_t)ds, step_pair));
  return vc_lm_head_argmax(d->draft[0].B, d->Dm, d->V, d->draft_hidden[i], d->lm_w, d->drafts + i, d->steps,
                           d->draft_lm_ws, d->draft_lm_ws_bytes, ds);
}

}  // namespace

extern "C" vc_status vc_stagger_round(vc_stagger *s, const vc_round_desc *d, void *draft_stream,
                                      void *verify_stream) {
  CHK(validate(s, d));
  const int L = d->layers, k = d->steps;
  const int ns = (int)s->slots.size();
  // the slot ring must be free: the previous round released its layers
  for (int sl = 0; sl < ns; ++sl)
    if (!s->released[sl]) return bad("a staging slot still holds an unreleased layer");

  // timing events: the draft pairs first (one per step, or one per layer and
  // step), then one pair per verify layer
  RoundTimer tm{s, d->time_kernels};
  s->timed_drafts = s->timed_verifies = 0;
  if (tm.every) {
    const int n_draft = tm.every == VC_TIME_ATTENTION_KERNELS ? k * L : k;
    const int n_ver = d->verify ? L : 0;
    const size_t need = 2 * (size_t)(n_draft + n_ver);
    while (s->round_ev.size() < need) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return vc::set_error(VC_EHIP, "creating timing events");
      s->round_ev.push_back(e);
    }
    s->timed_drafts = n_draft;
    s->timed_verifies = n_ver;
  }
  RoundTimer vt{s, tm.every, tm.every ? s->timed_drafts : 0};

  if (d->n_fetch > 0) {
    // the compressed cache first, each copy followed by its completion event
    while ((int)s->fetch_ev.size() < d->n_fetch) {
      hipEvent_t e;
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess)
        return vc::set_error(VC_EHIP, "creating fetch events");
      s->fetch_ev.push_back(e);
    }
    for (int j = 0; j < d->n_fetch; ++j) {
      const vc_round_fetch &f = d->fetch[j];
      if (hipMemcpyAsync(f.dev_dst, f.host_src, f.bytes, hipMemcpyHostToDevice, s->h2d) != hipSuccess ||
          hipEventRecord(s->fetch_ev[j], s->h2d) != hipSuccess)
        return vc::set_error(VC_EHIP, "enqueueing a fetch");
    }
  }
  // the first layers' copies (staggered and chained: they overlap the drafting), then every draft step back
  // to back on the draft stream
  const bool early_copies = k > 0 && d->verify && d->mode != VC_ROUND_BULK;
  for (int i = 0; early_copies && i < (ns < L ? ns : L); ++i)
    CHK(vc_stagger_stream_layer(s, i, d->host_kv[i], d->kv_bytes));
  for (int i = 0; i < k; ++i) CHK(draft_step(d, i, draft_stream, tm, s));
  if (k > 0 && d->mode == VC_ROUND_BULK) CHK(vc_stagger_after(s, draft_stream));   // no copy overlaps the drafting
  if (!d->verify) return VC_OK;
  if (k > 0 && d->mode != VC_ROUND_STAGGERED) {
    // the verify stream starts after the drafting cohort as well
    hipEvent_t ev;
    if (hipEventCreateWithFlags(&ev, hipEventDisableTiming) != hipSuccess)
      return vc::set_error(VC_EHIP, "event for the bulk-synchronous order");
    hipError_t e = hipEventRecord(ev, (hipStream_t)draft_stream);
    if (e == hipSuccess) e = hipStreamWaitEvent((hipStream_t)verify_stream, ev, 0);
    (void)hipEventDestroy(ev);
    if (e != hipSuccess) return vc::set_error(VC_EHIP, hipGetErrorString(e));
  }
  if (!early_copies)
    for (int l = 0; l < (ns < L ? ns : L); ++l) CHK(vc_stagger_stream_layer(s, l, d->host_kv[l], d->kv_bytes));
  for (int l = 0; l < L; ++l) {
    void *slot = nullptr;
    CHK(vc_stagger_acquire(s, l, verify_stream, &slot));
    if (d->before_verify) d->before_verify(d->hook_ctx, l, verify_stream);
    vc_verify_args a = d->verify[l];
    a.ctx_k = slot;
    a.ctx_v = static_cast<char *>(slot) + d->v_offset;
    CHK(verify_call(a, (hipStream_t)verify_stream, vt));
    CHK(vc_stagger_release(s, l, verify_stream));
    if (l + ns < L) CHK(vc_stagger_stream_layer(s, l + ns, d->host_kv[l + ns], d->kv_bytes));
  }
  const vc_verify_args &v0 = d->verify[0];
  CHK(vc_lm_head_accept(v0.B, v0.M, d->Dm, d->V, d->verify_hidden, d->lm_w, d->verify_drafts, d->argmax,
                        d->accept_len, d->out_tokens, d->n_out, d->verify_lm_ws, d->verify_lm_ws_bytes,
                        verify_stream));
  if (d->commit) {
    for (int l = 0; l < L; ++l) {
      const vc_verify_args &a = d->verify[l];
      const vc_round_commit &c = d->commit[l];
      if (c.kind == VC_COMMIT_ROWS)
        CHK(vc_commit_rows(a.B, a.Hkv, a.D, a.M, a.dtype, c.cap, c.dst_v_blocked, a.blk_k, a.blk_v, d->n_out,
                           c.dst_k, c.dst_v, c.len, c.degree, c.degree_h_stride, verify_stream));
      else
        CHK(vc_int4_commit(a.B, a.Hkv, a.D, a.M, a.blk_k, a.blk_v, d->n_out, c.tail_k, c.tail_v, c.tcap, c.tail_len,
                           c.packed, c.cap, c.main_len, verify_stream));
      const size_t blk_bytes = (size_t)a.B * a.Hkv * a.M * a.D * elem_bytes(a.dtype);
      if (c.host_k) CHK(vc_stagger_writeback(s, c.host_k, a.blk_k, blk_bytes, verify_stream));
      if (c.host_v) CHK(vc_stagger_writeback(s, c.host_v, a.blk_v, blk_bytes, verify_stream));
    }
  }
  return VC_OK;
}

extern "C" vc_status vc_stagger_round_times(vc_stagger *s, float *draft_ms, int32_t *n_draft, float *verify_ms,
                                            int32_t *n_verify) {
  if (!s || !n_draft || !n_verify) return bad("null stagger or count");
  *n_draft = s->timed_drafts;
  *n_verify = s->timed_verifies;
  for (int i = 0; draft_ms && i < s->timed_drafts; ++i)
    if (hipEventElapsedTime(&draft_ms[i], s->round_ev[2 * i], s->round_ev[2 * i + 1]) != hipSuccess)
      return vc::set_error(VC_EHIP, "reading a draft timing event (has the round completed?)");
  for (int l = 0; verify_ms && l < s->timed_verifies; ++l) {
    const int j = s->timed_drafts + l;
    if (hipEventElapsedTime(&verify_ms[l], s->round_ev[2 * j], s->round_ev[2 * j + 1]) != hipSuccess)
      return vc::set_error(VC_EHIP, "reading a verify timing event (has the round completed?)");
  }
  return VC_OK;
}
