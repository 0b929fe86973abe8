// Internal helpers shared by the library's translation units.
#pragma once

#include "rimuru.h"

// Record a thread-local error message and return code.
rimuru_status rimuru_fail(rimuru_status code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
