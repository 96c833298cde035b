// Pieces of the C ABI shared between its source files. Not installed; the
// public interface is include/kascade.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kascade.h"

namespace kascade {

// Argument checks of kascade_reuse_decode other than the workspace:
// KASCADE_OK or the status the call returns.
int reuse_decode_check(const kascade_problem* p, const void* q, const void* k, const void* v,
                       const int32_t* idx, const void* out);

// Enqueue the reuse-decode kernels on `s` with `ws` (at least
// kascade_workspace_bytes(p, KASCADE_OP_REUSE_DECODE) bytes, 256-byte aligned,
// arrival counters zero) as the workspace. Arguments already checked.
int reuse_decode_enqueue(const kascade_problem* p, const void* q, const void* k, const void* v,
                         const int32_t* idx, void* out, char* ws, hipStream_t s);

}  // namespace kascade
