// Error reporting shared by the C entry points: every non-OK status carries a
// thread-local message readable through astr_last_error().
#pragma once

#include "astr.h"

namespace astr {

// Record a printf-style message for the calling thread and return `status`.
int fail(int status, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace astr
