// Host-side helpers shared by the library's C-ABI translation units.
#pragma once

#include <cstdint>

#include "../../include/wkv7.h"

namespace wkv7 {

// Record a printf-style message as the calling thread's last error and
// return `code`.
wkv7_status host_fail(wkv7_status code, const char* fmt, ...)
    __attribute__((format(printf, 2, 3)));
// Clear the calling thread's last error (every entry point starts so).
void host_clear_error();
// Device of a pool and its slot image size in bytes.
int pool_device(const wkv7_pool* p);

}  // namespace wkv7
