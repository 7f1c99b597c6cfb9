// Internal helpers shared by the library's translation units: status
// reporting through a thread-local message.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "pa.h"

namespace pa {

// Records a message for pa_last_error() and returns `code`.
pa_status_t fail(pa_status_t code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
