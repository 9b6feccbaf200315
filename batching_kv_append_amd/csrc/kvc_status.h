// Status strings and the per-thread "last error" detail of the C ABI.
#pragma once
#include "kvc.h"

// Record `detail` as this thread's last error and return `status`.
int kvc_fail(int status, const char* detail);
