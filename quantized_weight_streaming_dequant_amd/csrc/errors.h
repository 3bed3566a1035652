// Error reporting shared by the C-ABI source files.
#pragma once

namespace nt {
// Record msg as the calling thread's nt_last_error() message and return code.
int set_error(int code, const char* msg);
}  // namespace nt
