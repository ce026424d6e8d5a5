// Thread-local error message shared by every entry point of libpa.so.
#pragma once

#include "pa.h"

namespace pa {

// Record msg as the calling thread's last error and return code.
pa_status fail(pa_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace pa
