// Library-wide entry points and host helpers (version, errors, validation).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "host.h"

namespace svg {

static thread_local char g_err[512] = "";

svgear_status fail(svgear_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

bool fault_injected(const char* call) {
  const char* f = getenv("SVGEAR_FAULT");
  return f != nullptr && strcmp(f, call) == 0;
}

svgear_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SVGEAR_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return SVGEAR_OK;
}

svgear_status check_common(const char* call, svgear_dtype dt, int B, int H, int N, int D) {
  if (fault_injected(call)) return fail(SVGEAR_ERR_INJECTED, "%s: fault injected by SVGEAR_FAULT", call);
  if (dt != SVGEAR_BF16 && dt != SVGEAR_F32) return fail(SVGEAR_ERR_INVALID_ARG, "%s: unknown dtype %d", call, (int)dt);
  if (B < 1 || H < 1) return fail(SVGEAR_ERR_INVALID_ARG, "%s: B=%d H=%d must be >= 1", call, B, H);
  if ((long long)B * H > 65535) return fail(SVGEAR_ERR_INVALID_ARG, "%s: B*H=%lld exceeds 65535", call, (long long)B * H);
  if (N < 1 || N >= (1 << 24)) return fail(SVGEAR_ERR_INVALID_ARG, "%s: N=%d must be in [1, 2^24)", call, N);
  if (D != 64 && D != 128) return fail(SVGEAR_ERR_INVALID_ARG, "%s: D=%d must be 64 or 128", call, D);
  return SVGEAR_OK;
}

svgear_status check_ws(const char* call, void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return SVGEAR_OK;
  if (ws == nullptr) return fail(SVGEAR_ERR_WORKSPACE, "%s: workspace is null (%zu bytes needed)", call, need);
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SVGEAR_ERR_WORKSPACE, "%s: workspace must be 256-byte aligned", call);
  if (ws_bytes < need) return fail(SVGEAR_ERR_WORKSPACE, "%s: workspace has %zu bytes, %zu needed", call, ws_bytes, need);
  return SVGEAR_OK;
}

}  // namespace svg

extern "C" const char* svgear_version(void) { return "svgear 0.1.0 gfx950"; }
extern "C" const char* svgear_last_error(void) { return svg::g_err; }
