// Internal helpers shared by the library's host translation units.
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pa.h"

namespace pa {

// Records a formatted message for pa_last_error() and returns `st`.
pa_status fail(pa_status st, const char* fmt, ...);
// Clears the message and returns PA_OK.
pa_status ok();

}  // namespace pa
