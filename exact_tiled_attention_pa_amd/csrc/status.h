// Thread-local error text shared by the host-side parts of the library.
#pragma once

namespace pa {

// Records printf-style detail for pa_last_error() and returns status.
int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// Clears the detail and returns PA_OK.
int ok();

}  // namespace pa
