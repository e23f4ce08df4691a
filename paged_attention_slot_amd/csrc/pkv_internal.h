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

}  // namespace pkv
