// Status reporting shared by the C ABI entry points: the thread-local text of
// the last non-OK status and the helpers that set it. Host code only.
#pragma once

#include <cstdio>

#include <hip/hip_runtime.h>

#include "attn_block.h"
#include "validate.hpp"

#define ATTN_API extern "C" __attribute__((visibility("default")))

namespace attnblk {

inline char *last_error_buffer() {
    static thread_local char buf[512] = "";
    return buf;
}

inline attn_status_t set_error(int status, const char *msg) {
    std::snprintf(last_error_buffer(), 512, "%s", msg);
    return static_cast<attn_status_t>(status);
}

inline attn_status_t report(const Check &c) {
    if (c.status == kOk) return ATTN_OK;
    return set_error(c.status, c.msg);
}

inline attn_status_t hip_fail(const char *where, hipError_t e) {
    char buf[512];
    std::snprintf(buf, sizeof(buf), "%s: %s", where, hipGetErrorString(e));
    return set_error(kHip, buf);
}

}  // namespace attnblk

#define HIP_TRY(where, expr)                                       \
    do {                                                           \
        hipError_t e_ = (expr);                                    \
        if (e_ != hipSuccess) return ::attnblk::hip_fail(where, e_); \
    } while (0)
