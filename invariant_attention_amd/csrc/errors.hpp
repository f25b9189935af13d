// errors.hpp -- thread-local error message shared by the C ABI entry points.
#pragma once

#include "../../include/invattn.h"

namespace ia {
// Records a printf-style message for ia_last_error() and returns st.
ia_status fail(ia_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the message and returns IA_OK.
ia_status ok();
}  // namespace ia
