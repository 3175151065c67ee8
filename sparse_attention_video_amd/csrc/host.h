// Host-side helpers: status reporting, argument checks, workspace carving.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/svgear.h"

namespace svg {

// Records a message for svgear_last_error() and returns the status.
svgear_status fail(svgear_status st, const char* fmt, ...);

// Returns SVGEAR_ERR_INJECTED (with a message) if SVGEAR_FAULT names `call`.
bool fault_injected(const char* call);

// Maps the last HIP launch error to a status.
svgear_status check_launch(const char* what);

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }
inline int round_up(int v, int m) { return (v + m - 1) / m * m; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
inline int bit_length(unsigned v) { int n = 0; while (v) { ++n; v >>= 1; } return n; }

// Sequential carving of the caller's workspace into 256-byte aligned pieces.
struct Carver {
  char* base;
  size_t used = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename T>
  T* take(size_t count) {
    T* p = reinterpret_cast<T*>(base ? base + used : nullptr);
    used += align256(count * sizeof(T));
    return p;
  }
};

inline size_t elem_size(svgear_dtype dt) { return dt == SVGEAR_BF16 ? 2 : 4; }

svgear_status check_common(const char* call, svgear_dtype dt, int B, int H, int N, int D);
svgear_status check_ws(const char* call, void* ws, size_t ws_bytes, size_t need);

}  // namespace svg
