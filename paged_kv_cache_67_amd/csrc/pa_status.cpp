// Status strings and the thread-local error detail of libpa.
#include <stdarg.h>
#include <stdio.h>

#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pa {

static thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

void clear_error() { g_err[0] = '\0'; }

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PA_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PA_OK;
}

}  // namespace pa

extern "C" {

int pa_version(void) { return 100; }  // 0.1.0

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_SHAPE: return "bad shape";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_ALIGN: return "misaligned pointer or stride";
    case PA_ERR_WORKSPACE: return "workspace too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_CAPACITY: return "not enough free blocks";
    case PA_ERR_CONTRACT: return "device-side metadata breaks the contract";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return pa::g_err; }

}  // extern "C"
