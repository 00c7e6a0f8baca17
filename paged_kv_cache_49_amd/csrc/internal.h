// Host-side helpers shared by the library's translation units.
#pragma once

#include "libpagedattn.h"

namespace pa {

// Record a formatted message for pa_last_error() and return `status`.
pa_status fail(pa_status status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the thread's last-error message (called at the start of each entry point).
void clear_error();
// True when PA_DEBUG=1: device entry points validate device-side inputs on the host.
bool debug_enabled();
// Host-side check of a pool descriptor (shape, dtype, alignment, scales).
pa_status validate_cache(const pa_kv_cache* cache);

}  // namespace pa
