// Thread-local error reporting shared by the host and device entry points.
#pragma once

#include <string>

#include "pa.h"

namespace pa {
// Record msg as the calling thread's last error and return st.
pa_status fail(pa_status st, const std::string& msg);
// Clear the last error and return PA_OK.
pa_status ok();
}  // namespace pa
