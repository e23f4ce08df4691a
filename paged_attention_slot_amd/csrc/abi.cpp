// Error reporting, version and tuning knobs of libpkv's C ABI.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "pkv_internal.h"

namespace {
thread_local std::string g_last_error;

struct KnobDef {
  const char* name;
  int lo, hi;
  bool pow2;
};
const KnobDef kKnobs[pkv::kKnobCount] = {
    {"PKV_ATTN_HEADS_PER_WAVE", 1, 4, false}, {"PKV_ATTN_PREFETCH", 2, 4, false},
    {"PKV_ATTN_MODE", 1, 4, false},           {"PKV_ATTN_APPEND", 1, 2, false},
    {"PKV_ATTN_WAVES_PER_BLOCK", 1, 8, true}, {"PKV_ATTN_PARTS_PER_WG", 1, 65535, false},
};
std::atomic<int> g_knob[pkv::kKnobCount];
std::once_flag g_knob_once;

bool knob_valid(const KnobDef& d, int x) {
  return x >= d.lo && x <= d.hi && (!d.pow2 || (x & (x - 1)) == 0);
}

// The environment's values, once per process (invalid or unset: 0).
void load_knobs() {
  for (int i = 0; i < pkv::kKnobCount; ++i) {
    const char* v = std::getenv(kKnobs[i].name);
    const int x = (v && *v) ? std::atoi(v) : 0;
    g_knob[i].store(knob_valid(kKnobs[i], x) ? x : 0, std::memory_order_relaxed);
  }
}

int knob_index(const char* name) {
  if (!name) return -1;
  for (int i = 0; i < pkv::kKnobCount; ++i)
    if (std::strcmp(name, kKnobs[i].name) == 0) return i;
  return -1;
}
}  // namespace

namespace pkv {

pkv_status fail(pkv_status code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

void clear_error() { g_last_error.clear(); }

int tuning(Knob k) {
  std::call_once(g_knob_once, load_knobs);
  return g_knob[k].load(std::memory_order_relaxed);
}

}  // namespace pkv

extern "C" {

int32_t pkv_version(void) { return 100; }  // 0.1.0

const char* pkv_last_error(void) { return g_last_error.c_str(); }

pkv_status pkv_set_tuning(const char* name, int32_t value) {
  std::call_once(g_knob_once, load_knobs);
  const int i = knob_index(name);
  if (i < 0) return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_set_tuning: unknown knob %s", name ? name : "(null)");
  if (value != 0 && !knob_valid(kKnobs[i], value))
    return pkv::fail(PKV_ERR_INVALID_ARG, "pkv_set_tuning: %s = %d is out of range", kKnobs[i].name,
                     value);
  g_knob[i].store(value, std::memory_order_relaxed);
  return PKV_OK;
}

int32_t pkv_get_tuning(const char* name) {
  std::call_once(g_knob_once, load_knobs);
  const int i = knob_index(name);
  return i < 0 ? -1 : g_knob[i].load(std::memory_order_relaxed);
}

}  // extern "C"
