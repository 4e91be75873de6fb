// Error reporting shared by the host sources of libgdnreplay: the message of
// the last failed call is kept per thread and returned by gdn_last_error().
#pragma once

#include "../../include/gdnreplay.h"

namespace gdn {

// Records a printf-style message for gdn_last_error() and returns st.
gdn_status host_fail(gdn_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace gdn
