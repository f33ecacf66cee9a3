// Host-side helpers shared by the library's translation units.
#pragma once

#include "../../include/jepa_mi355x.h"

namespace jepa {

// Record a printf-style message for jepa_last_error (this thread) and
// return st.
jepa_status fail(jepa_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace jepa
