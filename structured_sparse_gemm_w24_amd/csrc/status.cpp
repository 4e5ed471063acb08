// Thread-local status message and version string.
#include <cstdarg>
#include <cstdio>

#include "status.h"

namespace ssg {

static thread_local char g_msg[512] = "";

int fail(int code, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_msg[0] = '\0'; }

}  // namespace ssg

SSG_API const char *ssg_last_error(void) { return ssg::g_msg; }

SSG_API const char *ssg_version(void) { return "ssg 0.1.0 gfx950"; }
