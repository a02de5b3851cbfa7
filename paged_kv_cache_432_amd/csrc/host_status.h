// Status reporting shared by the host-side parts of libpa.so: the message is
// the one pa_last_error_message() returns on the calling thread.
#pragma once

#include "pa.h"

namespace pa {

pa_status report(pa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_status report_ok();

}  // namespace pa
