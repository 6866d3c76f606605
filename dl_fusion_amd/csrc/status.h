// Status reporting shared by the C-ABI translation units: a failed check stores its reason in
// the thread-local string that dlf_last_error() returns.
#pragma once

#include "../../include/dlfusion.h"

namespace dlf {

// Formats the reason (printf-style) and returns s.
dlf_status fail(dlf_status s, const char* fmt, ...);
// Clears the reason and returns DLF_OK.
dlf_status ok();

}  // namespace dlf
