// Internal helpers shared by the C-ABI source files (not exported).
#pragma once

#include "../../include/hstu.h"

namespace hstu {

// Records a printf-style detail for hstu_last_error() on the calling thread
// and returns `st`.
hstu_status_t api_fail(hstu_status_t st, const char* fmt, ...);

}  // namespace hstu
