// Status strings, the thread-local last-error message and the PA_DEBUG switch.
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.h"

namespace {
thread_local char g_last_error[512] = "";
}

namespace pa {

pa_status fail(pa_status status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_last_error[0] = '\0'; }

// read at every call, so a process can switch it (the cost is one
// environment lookup per device entry point)
bool debug_enabled() {
  const char* v = std::getenv("PA_DEBUG");
  return v != nullptr && std::strcmp(v, "1") == 0;
}

}  // namespace pa

extern "C" {

const char* pa_status_string(pa_status status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_OUT_OF_BLOCKS: return "PA_ERR_OUT_OF_BLOCKS";
    case PA_ERR_UNKNOWN_SEQ: return "PA_ERR_UNKNOWN_SEQ";
    case PA_ERR_SEQ_EXISTS: return "PA_ERR_SEQ_EXISTS";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE";
    case PA_ERR_OUT_OF_HOST_MEMORY: return "PA_ERR_OUT_OF_HOST_MEMORY";
  }
  return "PA_ERR_UNKNOWN_STATUS";
}

const char* pa_last_error(void) { return g_last_error; }

int32_t pa_abi_version(void) { return PA_ABI_VERSION; }

}  // extern "C"
