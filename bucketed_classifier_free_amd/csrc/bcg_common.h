// Internal helpers shared by the host and device translation units of libbcg.
#pragma once

#include <cstdarg>
#include <cstdio>

#include "bcg.h"

namespace bcg {

// Records a formatted message as the thread's last error and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the thread's last error.
void clear_error();

}  // namespace bcg
