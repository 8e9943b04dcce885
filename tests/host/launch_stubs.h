// Shared state of the launcher stand-ins (see launch_stubs.cpp).
#pragma once
#include <stdint.h>

#include "launch.h"

namespace stub {
extern uintptr_t ws_lo, ws_hi;  // the workspace of the call under test
extern int calls, bad;          // launches seen; regions that straddle the workspace
}  // namespace stub
