// Internal helpers shared by the library's translation units (not installed).
#pragma once

#include <cstdarg>
#include <cstdint>

#include "../../include/pa.h"

namespace pa {

// Record a message for pa_last_error() on this thread and return `code`.
pa_status fail(pa_status code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

// Clear the thread's message (called at the start of every entry point).
void clear_error();

// Maps the most recent HIP error (if any) after a launch to PA_EHIP.
pa_status check_launch(const char *what);

}  // namespace pa
