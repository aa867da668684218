// Chunked forward of the gated delta rule (scalar forget gate per token and
// head): the kernels of chunk_fwd.hpp with the in-chunk decays switched on.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd_gated(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    return launch_rule<true, false>(a, bf16, stream);
}

hipError_t launch_chunk_state_pair_gated(const ChunkFwdArgs &a, float *M, hipStream_t stream) {
    return launch_pair_rule<true>(a, M, stream);
}

}  // namespace dr
