// Host-side helpers shared by the library's C-ABI translation units.
#pragma once

#include <cstddef>
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

// Scratch of the allocation-free forward: a static device array of this many
// bytes on every GPU the library runs on (noalloc.hip). The work description
// takes at most kStaticMetaBytes of it (also the size of each pinned staging
// buffer a pool preallocates); segment buffers take the rest.
constexpr size_t kStaticScratchBytes = size_t(32) << 20;
constexpr size_t kStaticMetaBytes = size_t(64) << 10;
// Device address of that array on the current device (looked up once per
// device; call with the device current).
wkv7_status static_scratch_setup(void** out);

}  // namespace wkv7
