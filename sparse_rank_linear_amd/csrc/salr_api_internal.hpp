// Internal entry shared by the forward's C-ABI variants (salr_api.cpp,
// noalloc.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "salr.h"

namespace salr {

// Validates and runs one forward call on workspace `ws` of `ws_bytes`
// (zero-filled before its first use; every completed call leaves it ready
// for the next).  A bounded wait that times out sets *err_word.  Returns a
// salr_status_t; SALR_ERR_WORKSPACE when ws is null, misaligned or smaller
// than the call's layout needs.
int forward_impl(const salr_layer_t* L, const uint16_t* X, int64_t M, uint16_t* Y, void* ws, size_t ws_bytes,
                 uint32_t* err_word, hipStream_t s);

}  // namespace salr
