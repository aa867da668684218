// Chunked forward of the gated delta rule with q and k L2-normalised inside
// the kernel.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd_gated_l2(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    return launch_rule<true, true>(a, bf16, stream);
}

}  // namespace dr
