// pa_error.h — the thread-local last-error record shared by every C ABI
// entry point (pa_last_error), usable from host-only translation units.
#pragma once

#include <stdint.h>

namespace pa {

// Stores msg as the calling thread's last error (cleared for PA_OK) and
// returns code.
int32_t record_error(int32_t code, const char* msg);

}  // namespace pa
