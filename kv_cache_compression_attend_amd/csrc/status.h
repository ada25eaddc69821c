// Error text and status helpers shared by the host translation units.
#pragma once

#include <cstdarg>

namespace hk {

// Records printf-style text as this thread's last error and returns `code`.
int fail(int code, const char* fmt, ...);

}  // namespace hk
