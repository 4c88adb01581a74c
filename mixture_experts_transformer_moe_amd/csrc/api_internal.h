// Helpers the C-ABI translation units share (not part of the public ABI).
#pragma once

#include "moe.h"

namespace moe {
// Record msg as this thread's moe_last_error() detail and return st.
moe_status_t api_error(moe_status_t st, const char* msg);
}  // namespace moe

// Return the status of expr unless it is MOE_OK.
#define MOE_RETURN_IF_ERROR(expr)    \
  do {                               \
    const moe_status_t st_ = (expr); \
    if (st_ != MOE_OK) return st_;   \
  } while (0)
