// Error reporting shared by the C-ABI sources: fail() records the message
// that csa_last_error() returns (per calling thread) and passes the status on.
#pragma once

#include <hip/hip_runtime.h>

#include "csa.h"

namespace csa {

csa_status fail(csa_status s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
csa_status hip_status(hipError_t e, const char* where);
const char* last_error();

}  // namespace csa
