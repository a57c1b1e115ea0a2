// Status strings and the per-thread last-error text.
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "internal.h"

namespace {
thread_local char g_last[512] = "";
}

namespace ll {
ll_status fail(ll_status st, const char* msg) {
    std::snprintf(g_last, sizeof g_last, "%s", msg);
    return st;
}
ll_status failf(ll_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last, sizeof g_last, fmt, ap);
    va_end(ap);
    return st;
}
}  // namespace ll

extern "C" {
int ll_abi_version(void) { return LL_ABI_VERSION; }

const char* ll_last_error(void) { return g_last; }

const char* ll_strerror(int status) {
    switch (status) {
    case LL_OK: return "ok";
    case LL_EINVAL: return "invalid argument";
    case LL_ESHAPE: return "unsupported shape";
    case LL_EALIGN: return "device pointer not 16-byte aligned";
    case LL_ECODE: return "invalid weight value or packed code";
    case LL_EWORKSPACE: return "workspace missing or too small";
    case LL_EHIP: return "HIP runtime error";
    case LL_ERANGE: return "size out of range";
    default: return "unknown status";
    }
}
}
