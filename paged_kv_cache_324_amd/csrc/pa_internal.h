// Error reporting shared by the library's host sources (not exported).
#pragma once

namespace pa {

// Record a thread-local message for pa_last_error() and return `code`.
__attribute__((visibility("hidden"))) int fail(int code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
// Clear the message and return PA_OK.
__attribute__((visibility("hidden"))) int ok();

}  // namespace pa
