// Thread-local last-error message shared by every C entry point.
#pragma once

#include "../../include/pkv.h"

namespace pkv {

// Record a formatted message and return `st`.
pkv_status fail(pkv_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return PKV_OK.
pkv_status ok();

}  // namespace pkv

#define PKV_EXPORT extern "C" __attribute__((visibility("default")))
