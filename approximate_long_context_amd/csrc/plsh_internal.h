// plsh_internal.h -- error reporting shared by the host and device halves of
// libplsh (thread-local message behind plsh_last_error()).
#pragma once

#include "../../include/plsh.h"

namespace plsh {

// Records a formatted message for plsh_last_error() and returns `st`.
plsh_status fail(plsh_status st, const char *fmt, ...)
#if defined(__GNUC__)
    __attribute__((format(printf, 2, 3)))
#endif
    ;

// Clears the thread-local message (called on entry of every ABI function).
void clear_error();

// Largest number of samples per head: the per-row multiplicity counters of
// the attention kernels are bytes.
constexpr int32_t kMaxSamples = 255;

}  // namespace plsh
