// Chunked forward of the plain delta rule: the kernels of chunk_fwd.hpp
// without the forget gate, and the entry that routes gated calls to
// chunk_fwd_gated.hip.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v,
                            const void *beta, const float *g, const float *S0, void *o,
                            float *S_T, int64_t B, int64_t T, int64_t H, int Dk, int Dv,
                            int chunk, bool bf16, hipStream_t stream) {
    if (g)
        return launch_chunk_fwd_gated(q, k, v, beta, g, S0, o, S_T, B, T, H, Dk, Dv, chunk, bf16,
                                      stream);
    return launch_rule<false>(q, k, v, beta, nullptr, S0, o, S_T, B, T, H, Dk, Dv, chunk, bf16,
                              stream);
}

}  // namespace dr
