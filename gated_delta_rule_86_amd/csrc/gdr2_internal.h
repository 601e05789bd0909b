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
hipError_t launch_forward_fused(const gdr2_fwd_args& a, hipStream_t stream);

// The fused forward has a kernel for these arguments (dtype, sizes).
bool fused_supported(const gdr2_fwd_args& a);
// The algorithm a forward call runs: GDR2_ALGO_FUSED, or STAGED (which
// may segment, per segment_plan).
int forward_algo(const gdr2_fwd_args& a);
hipError_t launch_state_copy(const float* src, float* dst, int64_t n_floats, hipStream_t stream);
hipError_t launch_backward(const gdr2_bwd_args& a, hipStream_t stream);

// Workspace of the staged forward, in bytes (0 if nothing to do).
size_t staged_workspace_bytes(const gdr2_fwd_args& a);

// Workspace of the chunked backward, in bytes (0 if nothing to do).
size_t backward_workspace_bytes(const gdr2_bwd_args& a);

// Every check of gdr2_forward_chunked except the workspace's (host only).
gdr2_status check_forward_args(const gdr2_fwd_args* a);

// Records a message for gdr2_last_error() in the calling thread; returns s.
gdr2_status set_error(gdr2_status s, const char* fmt, ...);

// Compute units of the current device (256 when it cannot be queried).
int device_cu_count();

// Segments of a two-level scan over NC chunks run by `wgs` workgroups per
// pass (gdr2_algo `algo`): *nseg segments of *len chunks (the last may be
// shorter); nseg == 1 is one pass.
void segment_plan(int algo, int64_t NC, int64_t wgs, int64_t* nseg, int64_t* len);

// The segment fold of a two-level scan over `span` (per (b,h), nseg - 1
// entries of two D x D fp32 matrices: a product Pi and a local part L):
// X = L of entry 0, then X <- Pi_e X + L_e for e = 1 .. nseg-2, each X
// written over L_e.  Launched only for nseg > 2.
hipError_t launch_span_fold(float* span, int64_t nbh, int64_t nseg, int D, hipStream_t stream);

}  // namespace gdr2
