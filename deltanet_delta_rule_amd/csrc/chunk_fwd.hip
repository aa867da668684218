// Chunked forward of the plain delta rule: the kernels of chunk_fwd.hpp
// without the forget gate, and the entry that routes gated calls to
// chunk_fwd_gated.hip.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    return a.g ? launch_chunk_fwd_gated(a, bf16, stream) : launch_rule<false>(a, bf16, stream);
}

}  // namespace dr
