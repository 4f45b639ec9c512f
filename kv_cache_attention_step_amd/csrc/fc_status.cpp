// Status strings, per-thread last-error message and launch checks.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "fc_common.hpp"

static thread_local char g_last_error[512] = "";

fc_status_t fc_fail(fc_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

void fc_clear_error() { g_last_error[0] = 0; }

fc_status_t fc_check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fc_fail(FC_ERR_HIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return FC_OK;
}

extern "C" const char* fc_status_string(fc_status_t st) {
  // a C caller may pass any int; read it as one (an enum load outside the
  // enumerators' range is undefined in C++)
  int v;
  memcpy(&v, &st, sizeof v);
  switch (v) {
    case FC_OK: return "FC_OK";
    case FC_ERR_INVALID_VALUE: return "FC_ERR_INVALID_VALUE: invalid argument";
    case FC_ERR_UNSUPPORTED: return "FC_ERR_UNSUPPORTED: shape or dtype not supported";
    case FC_ERR_WORKSPACE: return "FC_ERR_WORKSPACE: workspace missing or too small";
    case FC_ERR_HIP: return "FC_ERR_HIP: HIP runtime error";
  }
  return "unknown fc_status_t";
}

extern "C" const char* fc_last_error(void) { return g_last_error; }

extern "C" const char* fc_version(void) { return "flashcache-gfx950 0.1"; }
