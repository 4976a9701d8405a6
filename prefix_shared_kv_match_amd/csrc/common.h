// Shared helpers of libpkv: the per-thread error message behind pkv_last_error().
#pragma once

#include <cstdarg>
#include <cstdio>
#include <string>

#include "pkv.h"

namespace pkv {

// Records a message for pkv_last_error() and returns `code`, so call sites can write
// `return fail(PKV_ERR_INVAL, "...")`.
int fail(int code, const char* fmt, ...)
#if defined(__GNUC__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;

}  // namespace pkv
