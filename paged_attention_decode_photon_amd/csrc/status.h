// Status helpers shared by the C ABI translation units: a non-OK status
// carries a message for photon_last_error_detail() on the calling thread.
#pragma once

#include "photon_decode.h"

namespace photon {

// Set the calling thread's detail message (printf format) and return st.
photon_status fail(photon_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the detail message and return PHOTON_OK.
photon_status ok();
const char *last_detail();
// Number of the next kernel call (never 0), the epoch of its arrival counters.
uint32_t next_epoch();

}  // namespace photon
