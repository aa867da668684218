// The plain rule's bf16 chunked forward at d_k = 128 and 64-token chunks (the
// layer shape's launch, and the output pass of the segment-parallel schedule
// at that size).  Its own translation unit so that the build can compile it
// with the instruction scheduler that favours independent instructions
// (-amdgpu-sched-strategy=max-ilp): that interleaves more of the state and
// preparation waves' independent work and measured ~4 % faster for this
// kernel, while the other forward kernels measured the same or slower.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd_plain_d128_c64(const ChunkFwdArgs &a, hipStream_t stream) {
    return dispatch_nw<__bf16, 128, 64, false, false>(a, stream);
}

}  // namespace dr
