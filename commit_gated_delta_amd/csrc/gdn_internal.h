// gdn_internal.h -- helpers shared by the library's translation units (not
// part of the C ABI).
#pragma once

namespace gdn {

// Records the detail string returned by gdn_last_error() on this thread.
__attribute__((visibility("hidden"))) void set_error(const char* msg);

}  // namespace gdn
