// Host-side launchers of the delta-rule kernels.  Arguments are validated by
// the C ABI layer before these are called; they only enqueue work on `stream`
// and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

// Fused chunkwise forward (one workgroup per (b, h, value tile)).  g is the
// log forget gate [B,T,H] (fp32) of the gated rule, or nullptr.
hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v,
                            const void *beta, const float *g, const float *S0, void *o,
                            float *S_T, int64_t B, int64_t T, int64_t H, int Dk, int Dv,
                            int chunk, bool bf16, hipStream_t stream);

// Single-token decode step, state updated in place.  g is the log forget gate
// [B,H] (fp32) of the gated rule, or nullptr.
hipError_t launch_recurrent_step(const void *q, const void *k, const void *v,
                                 const void *beta, const float *g, float *S, void *o,
                                 int64_t BH, int Dk, int Dv, bool bf16, hipStream_t stream);

}  // namespace dr
