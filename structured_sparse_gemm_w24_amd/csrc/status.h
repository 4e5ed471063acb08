// Internal helpers shared by the host files of libssg: export macro and the
// thread-local error message behind ssg_last_error().
#pragma once

#include <cstdint>

#include "../../include/ssg.h"

#define SSG_API extern "C" __attribute__((visibility("default")))

namespace ssg {

// Formats a message into the thread-local error buffer and returns `code`.
int fail(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the thread-local error message.
void clear_error();

inline bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace ssg
