// Bounds assertions of the debug build.  With QMOE_DEBUG_BOUNDS defined, QMOE_BOUNDS(c) checks
// c in host code and, on failure, prints the condition and its place and aborts; without it,
// and always in device code, it compiles to nothing.  The index math that host and device
// share (the store's chunk map, the bucket table entries, the workspace and LDS layouts) is
// written as __host__ __device__ functions, so the debug build runs it on the CPU with these
// checks and the sanitizers.
#pragma once

#if defined(QMOE_DEBUG_BOUNDS) && !defined(__HIP_DEVICE_COMPILE__)
#include <cstdio>
#include <cstdlib>
namespace qmoe {
[[noreturn]] inline void bounds_failed(const char *cond, const char *file, int line) {
  std::fprintf(stderr, "qmoe bounds check failed: %s (%s:%d)\n", cond, file, line);
  std::abort();
}
}  // namespace qmoe
#define QMOE_BOUNDS(c) ((c) ? (void)0 : ::qmoe::bounds_failed(#c, __FILE__, __LINE__))
#else
#define QMOE_BOUNDS(c) ((void)0)
#endif
