// Internal declarations shared by the library's translation units.
#pragma once

#include <cstdarg>
#include <cstdint>

#include "pa.h"

namespace pa {

// Records a printf-style message for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...);

}  // namespace pa
