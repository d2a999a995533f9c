// Host-side helpers shared by the C ABI's source files (not part of the ABI).
#pragma once
#include "moe.h"

namespace moe {

// Record the thread-local text moe_last_error() returns, and return s.
moe_status set_error(moe_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace moe
