// Cross-resource staggering: streaming the full cache of the verifying
// requests from pinned host memory while other requests draft from HBM.
//
// "Riepilogo Tecnico: VeriCache", "Innovazioni Chiave del Sistema", P1: draft
// is bound by GPU HBM bandwidth, verify by the interconnect that brings the
// full cache from CPU memory; the runtime staggers requests so that both
// resources stay busy.  "Supporto Architetturale": for long-context decoding
// the full cache lives in CPU memory and verification loads it over PCIe.
//
// The object below is the runtime half of that schedule: a host-to-device
// copy stream feeding a ring of device staging slots layer by layer, a
// write-back stream for committed rows, and the events that order them
// against the compute streams (verify waits for its layer's copy; a slot is
// refilled only after the verify that read it has finished).  Which kernels
// run on which compute stream is the caller's choice; the draft work of the
// other cohort goes on a stream that never waits for a copy.
#include <hip/hip_runtime.h>

#include <string>
#include <vector>

#include "stagger_impl.h"

namespace {

vc_status hipfail(hipError_t e, const char *what) {
  return vc::set_error(VC_EHIP, (std::string(what) + ": " + hipGetErrorString(e)).c_str());
}

#define HIPCHK(x)                            \
  do {                                       \
    hipError_t e_ = (x);                     \
    if (e_ != hipSuccess) return hipfail(e_, #x); \
  } while (0)

// Streams and events of a new object; on failure the caller destroys the
// partly built object (handles not yet created are null).
vc_status stagger_init(vc_stagger *s, void *const *slots, int32_t nslots, size_t slot_bytes, int32_t max_layers) {
  s->slots.assign(slots, slots + nslots);
  s->slot_bytes = slot_bytes;
  s->slot_free.assign(nslots, nullptr);
  s->holder.assign(nslots, -1);
  s->released.assign(nslots, 1);
  s->copy_start.assign(max_layers, nullptr);
  s->copied.assign(max_layers, nullptr);
  s->copy_recorded.assign(max_layers, 0);
  s->copy_timed.assign(max_layers, 0);
  HIPCHK(hipStreamCreateWithFlags(&s->h2d, hipStreamNonBlocking));
  HIPCHK(hipStreamCreateWithFlags(&s->d2h, hipStreamNonBlocking));
  for (auto &e : s->slot_free) HIPCHK(hipEventCreateWithFlags(&e, hipEventDisableTiming));
  for (int l = 0; l < max_layers; ++l) {
    HIPCHK(hipEventCreate(&s->copy_start[l]));
    HIPCHK(hipEventCreate(&s->copied[l]));
  }
  return VC_OK;
}

// `waiter` runs its later work only after what `producer` holds now (a
// one-off event, destroyed again on every path).
vc_status stream_waits_for(hipStream_t waiter, hipStream_t producer) {
  hipEvent_t ev;
  HIPCHK(hipEventCreateWithFlags(&ev, hipEventDisableTiming));
  hipError_t e = hipEventRecord(ev, producer);
  if (e == hipSuccess) e = hipStreamWaitEvent(waiter, ev, 0);
  (void)hipEventDestroy(ev);
  if (e != hipSuccess) return hipfail(e, "ordering a copy stream after the caller's stream");
  return VC_OK;
}

}  // namespace

extern "C" {

vc_status vc_stagger_create(vc_stagger **out, void *const *slots, int32_t nslots, size_t slot_bytes,
                            int32_t max_layers) {
  if (!out || !slots || nslots < 1 || max_layers < 1) return vc::set_error(VC_EINVAL, "bad stagger arguments");
  for (int i = 0; i < nslots; ++i)
    if (!slots[i]) return vc::set_error(VC_EINVAL, "null staging slot");
  vc_stagger *s = new vc_stagger;
  const vc_status st = stagger_init(s, slots, nslots, slot_bytes, max_layers);
  if (st != VC_OK) {
    vc_stagger_destroy(s);   // frees what was created; the error message stays the init failure's
    return st;
  }
  *out = s;
  return VC_OK;
}

vc_status vc_stagger_stream_layer(vc_stagger *s, int32_t layer, const void *host_src, size_t bytes) {
  if (!s || layer < 0 || layer >= (int)s->copied.size() || !host_src || bytes > s->slot_bytes)
    return vc::set_error(VC_EINVAL, "bad stream_layer arguments");
  const int slot = layer % (int)s->slots.size();
  // the slot's previous layer must have been released, or the copy would
  // overwrite a slot that verify may still read
  if (!s->released[slot]) {
    std::string m = "stream_layer(" + std::to_string(layer) + "): slot " + std::to_string(slot) +
                    " still holds layer " + std::to_string(s->holder[slot]) + ", which was not released";
    return vc::set_error(VC_EINVAL, m.c_str());
  }
  HIPCHK(hipStreamWaitEvent(s->h2d, s->slot_free[slot], 0));
  HIPCHK(hipEventRecord(s->copy_start[layer], s->h2d));
  HIPCHK(hipMemcpyAsync(s->slots[slot], host_src, bytes, hipMemcpyHostToDevice, s->h2d));
  HIPCHK(hipEventRecord(s->copied[layer], s->h2d));
  s->copy_recorded[layer] = 1;
  s->copy_timed[layer] = 1;
  s->holder[slot] = layer;
  s->released[slot] = 0;
  return VC_OK;
}

vc_status vc_stagger_acquire(vc_stagger *s, int32_t layer, void *stream, void **slot) {
  if (!s || layer < 0 || layer >= (int)s->copied.size() || !slot)
    return vc::set_error(VC_EINVAL, "bad acquire arguments");
  const int sl = layer % (int)s->slots.size();
  if (!s->copy_recorded[layer] || s->holder[sl] != layer)
    return vc::set_error(VC_EINVAL, "acquire of a layer that is not streamed into its slot (not streamed, or "
                                    "already released)");
  HIPCHK(hipStreamWaitEvent((hipStream_t)stream, s->copied[layer], 0));
  *slot = s->slots[sl];
  return VC_OK;
}

vc_status vc_stagger_release(vc_stagger *s, int32_t layer, void *stream) {
  if (!s || layer < 0 || layer >= (int)s->copied.size()) return vc::set_error(VC_EINVAL, "bad release");
  const int sl = layer % (int)s->slots.size();
  if (s->holder[sl] != layer || s->released[sl])
    return vc::set_error(VC_EINVAL, "release of a layer that does not hold its slot");
  HIPCHK(hipEventRecord(s->slot_free[sl], (hipStream_t)stream));
  s->released[sl] = 1;
  s->copy_recorded[layer] = 0;   // the slot may be refilled: a later acquire needs a new copy
  return VC_OK;
}

vc_status vc_stagger_writeback(vc_stagger *s, void *host_dst, const void *dev_src, size_t bytes, void *after) {
  if (!s || !host_dst || !dev_src) return vc::set_error(VC_EINVAL, "bad writeback arguments");
  const vc_status st = stream_waits_for(s->d2h, (hipStream_t)after);
  if (st != VC_OK) return st;
  HIPCHK(hipMemcpyAsync(host_dst, dev_src, bytes, hipMemcpyDeviceToHost, s->d2h));
  return VC_OK;
}

vc_status vc_stagger_after(vc_stagger *s, void *stream) {
  if (!s) return vc::set_error(VC_EINVAL, "null stagger");
  return stream_waits_for(s->h2d, (hipStream_t)stream);
}

vc_status vc_stagger_sync(vc_stagger *s) {
  if (!s) return vc::set_error(VC_EINVAL, "null stagger");
  HIPCHK(hipStreamSynchronize(s->h2d));
  HIPCHK(hipStreamSynchronize(s->d2h));
  return VC_OK;
}

vc_status vc_stagger_copy_ms(vc_stagger *s, int32_t layer, float *ms) {
  if (!s || layer < 0 || layer >= (int)s->copied.size() || !ms || !s->copy_timed[layer])
    return vc::set_error(VC_EINVAL, "no copy recorded for this layer");
  HIPCHK(hipEventElapsedTime(ms, s->copy_start[layer], s->copied[layer]));
  return VC_OK;
}

vc_status vc_stagger_destroy(vc_stagger *s) {
  if (!s) return VC_OK;
  // only handles that exist are passed on, so no HIP error is left behind
  // for a later call to pick up
  if (s->h2d) (void)hipStreamSynchronize(s->h2d);
  if (s->d2h) (void)hipStreamSynchronize(s->d2h);
  for (auto *v : {&s->slot_free, &s->copy_start, &s->copied, &s->round_ev, &s->fetch_ev})
    for (auto e : *v)
      if (e) (void)hipEventDestroy(e);
  if (s->h2d) (void)hipStreamDestroy(s->h2d);
  if (s->d2h) (void)hipStreamDestroy(s->d2h);
  delete s;
  return VC_OK;
}

}  // extern "C"
