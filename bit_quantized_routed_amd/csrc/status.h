// Per-thread error text of the C ABI (moe_last_error), shared by the host
// sources of the library.
#pragma once

namespace moe {

// stores the formatted detail for the calling thread and returns `code`
int set_error(int code, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

}  // namespace moe
