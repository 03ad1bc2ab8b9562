// errors.h -- status text shared by the C-ABI entry points of libpagedkv.so
// (pagedkv_last_error): host code only, no HIP.
#pragma once

namespace pkv {

// Set the calling thread's error text (printf format) and return `code`.
int fail(int code, const char* fmt, ...);

}  // namespace pkv
