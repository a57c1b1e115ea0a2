// Internal helpers shared by the library's translation units (not installed).
#pragma once
#include <cstddef>
#include <cstdint>

#include "lowbit.h"

namespace ll {
// Records `msg` as the calling thread's last error and returns `st`.
ll_status fail(ll_status st, const char* msg);
// Same, with printf-style formatting.
ll_status failf(ll_status st, const char* fmt, ...);
}  // namespace ll
