// gdr2_internal.h -- declarations shared between the host API and the kernel
// translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "gdr2.h"

namespace gdr2 {

// Launchers: arguments are already validated; they only enqueue work.
hipError_t launch_decode(const gdr2_decode_args& a, hipStream_t stream);
hipError_t launch_forward_staged(const gdr2_fwd_args& a, hipStream_t stream);
hipError_t launch_state_copy(const float* src, float* dst, int64_t n_floats, hipStream_t stream);
hipError_t launch_backward(const gdr2_bwd_args& a, hipStream_t stream);

// Workspace of the staged forward, in bytes (0 if nothing to do).
size_t staged_workspace_bytes(const gdr2_fwd_args& a);

// Workspace of the chunked backward, in bytes (0 if nothing to do).
size_t backward_workspace_bytes(const gdr2_bwd_args& a);

}  // namespace gdr2
