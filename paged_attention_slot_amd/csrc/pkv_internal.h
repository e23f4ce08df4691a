// Internal helpers shared by the host-side translation units of libpkv.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records the message returned by pkv_last_error() on this host thread and
// returns ``code`` so call sites can write ``return fail(PKV_ERR_..., "...")``.
pkv_status fail(pkv_status code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
void clear_error();

// Tuning knobs (the names and ranges are documented with pkv_set_tuning in
// pkv.h).  Each takes the environment variable of its name, read once in the
// process at the first use of any knob; pkv_set_tuning changes it later.
// 0 = the library's heuristic.
enum Knob : int {
  kKnobHeadsPerWave = 0,
  kKnobPrefetch,
  kKnobMode,
  kKnobAppend,
  kKnobWavesPerBlock,
  kKnobPartsPerWg,
  kKnobCount
};
int tuning(Knob k);

}  // namespace pkv
