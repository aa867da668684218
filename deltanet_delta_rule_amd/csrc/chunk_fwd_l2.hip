// Chunked forward of the plain delta rule with q and k L2-normalised inside
// the kernel: the kernels of chunk_fwd.hpp with the norm scalings on.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd_l2(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    return launch_rule<false, true>(a, bf16, stream);
}

}  // namespace dr
