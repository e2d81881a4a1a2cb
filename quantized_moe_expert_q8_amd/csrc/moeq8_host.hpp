// Host-side helpers shared by the libmoeq8 entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/moeq8.h"

namespace moeq8 {

// Status of the launch just enqueued: MOEQ8_EHIP (and the error cleared) when
// the runtime reports a failure.
inline int check_launch() {
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? MOEQ8_OK : MOEQ8_EHIP;
}

}  // namespace moeq8
