// Status reporting shared by every C entry point of libpa: a failing call
// stores its message in a thread-local string (read back by pa_last_error)
// and returns its pa_status; a succeeding call clears the message.  Plain
// C++, no device code, so the host pool half of the library builds and runs
// without the HIP runtime (and under the host sanitizers).
#pragma once

#include <string>

#include "pa.h"

namespace pa {

pa_status fail(pa_status st, const std::string& msg);
pa_status ok();

}  // namespace pa
