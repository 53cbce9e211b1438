// The streaming runtime object (internal): its streams, the slot ring and
// the events that order copies against the compute streams.
#pragma once

#include <hip/hip_runtime.h>

#include <vector>

#include "../../include/vc.h"

struct vc_stagger {
  std::vector<void *> slots;
  size_t slot_bytes = 0;
  hipStream_t h2d = nullptr, d2h = nullptr;
  std::vector<hipEvent_t> slot_free;             // per slot: recorded at the release of its layer
  std::vector<int> holder;                       // per slot: the layer last streamed into it (-1: none)
  std::vector<char> released;                    // per slot: that layer was released
  std::vector<hipEvent_t> copy_start, copied;    // per layer
  std::vector<char> copy_recorded;               // per layer: streamed and not yet released
  std::vector<char> copy_timed;                  // per layer: a copy was timed (vc_stagger_copy_ms)
  // kernel timing of the last round (vc_stagger_round with time_every > 0):
  // event pairs around the timed draft calls, then around every verify call
  std::vector<hipEvent_t> round_ev;
  int timed_drafts = 0, timed_verifies = 0;
  // completion of a round's fetches (vc_round_desc::fetch), one event each
  std::vector<hipEvent_t> fetch_ev;
};

namespace vc {
vc_status set_error(vc_status s, const char *msg);
}
