// Chunked forward of the plain delta rule: the kernels of chunk_fwd.hpp
// without the forget gate or in-kernel normalisation, and the entry that
// routes the other variants to their translation units.
#include "chunk_fwd.hpp"

namespace dr {

hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    if (a.gk && !a.h && kda_chunk_supported(a, bf16)) return launch_kda_chunk(a, stream);
    if (a.gk || a.recurrent)  // no checkpoints from the token-serial schedule
        return a.h ? hipErrorInvalidValue : launch_fused_recurrent(a, bf16, stream);
    if (a.l2)
        return a.g ? launch_chunk_fwd_gated_l2(a, bf16, stream) : launch_chunk_fwd_l2(a, bf16, stream);
    return a.g ? launch_chunk_fwd_gated(a, bf16, stream) : launch_rule<false, false>(a, bf16, stream);
}

bool chunk_state_pair_supported(const ChunkFwdArgs &a, bool bf16) {
    return bf16 && !a.gk && !a.l2 && !a.recurrent && (a.Dk == 64 || a.Dk == 128) &&
           a.Dv == a.Dk;
}

hipError_t launch_chunk_state_pair(const ChunkFwdArgs &a, float *M, bool bf16,
                                   hipStream_t stream) {
    if (!chunk_state_pair_supported(a, bf16) || a.h || a.o || a.S0) return hipErrorNotSupported;
    return a.g ? launch_chunk_state_pair_gated(a, M, stream) : launch_pair_rule<false>(a, M, stream);
}

}  // namespace dr
