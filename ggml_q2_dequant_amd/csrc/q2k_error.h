// Internal: the thread-local message behind q2k_last_error_message()
// (defined in q2k_api.cpp). Plain C++, no HIP, so host-only parts of the
// library can be built and checked without the GPU toolchain.
#pragma once

#include <stdarg.h>

#include "q2k.h"

namespace q2k {

q2k_status set_error_v(q2k_status s, const char *fmt, va_list ap);
void clear_error();

}  // namespace q2k
