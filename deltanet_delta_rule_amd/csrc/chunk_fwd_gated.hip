// Chunked forward of the gated delta rule (scalar forget gate per token and
// head): the kernels of chunk_fwd.hpp with the in-chunk decays switched on.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd_gated(const void *q, const void *k, const void *v,
                                  const void *beta, const float *g, const float *S0, void *o,
                                  float *S_T, int64_t B, int64_t T, int64_t H, int Dk, int Dv,
                                  int chunk, bool bf16, hipStream_t stream) {
    return launch_rule<true>(q, k, v, beta, g, S0, o, S_T, B, T, H, Dk, Dv, chunk, bf16, stream);
}

}  // namespace dr
