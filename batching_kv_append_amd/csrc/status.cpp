// Status strings and per-thread error detail for the C ABI.
#include <cstdio>
#include <cstring>

#include "kvc.h"
#include "kvc_status.h"

namespace {
thread_local char g_last_error[512] = "";
}

int kvc_fail(int status, const char* detail) {
    std::snprintf(g_last_error, sizeof g_last_error, "%s", detail ? detail : "");
    return status;
}

extern "C" const char* kvc_status_string(int status) {
    switch (status) {
        case KVC_OK: return "ok";
        case KVC_ERR_INVALID_ARG: return "invalid argument";
        case KVC_ERR_OOM: return "out of blocks";
        case KVC_ERR_UNSUPPORTED: return "unsupported configuration";
        case KVC_ERR_WORKSPACE: return "workspace missing or too small";
        case KVC_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" const char* kvc_last_error(void) { return g_last_error; }
