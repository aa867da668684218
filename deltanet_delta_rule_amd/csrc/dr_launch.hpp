// Host-side launchers of the delta-rule kernels.  Arguments are validated by
// the C ABI layer before these are called; they only enqueue work on `stream`
// and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

// Arguments of the fused chunkwise forward (one workgroup per (sequence,
// head, value tile)).  g is the log forget gate [B,T,H] (fp32) of the gated
// rule, or nullptr.  cu, when set, holds B+1 sequence offsets into the single
// batch row of T tokens (packed variable-length input); scale multiplies the
// outputs; l2 normalises the rows of q and k inside the kernel.  o may be
// nullptr (no outputs written); h, when set, receives each chunk's incoming
// state, [B,H,N,Dv,Dk] in the input dtype with N = ceil(T / chunk) (no
// packed sequences).  gk, when set (with g unset), is the per-key-channel log
// decay [B,T,H,Dk] (KDA); recurrent selects the token-serial schedule.  Both
// run launch_fused_recurrent, which takes everything above except chunk and h.
struct ChunkFwdArgs {
    const void *q, *k, *v, *beta;
    const float *g, *S0;
    void *o;
    float *S_T;
    void *h;
    const int *cu;
    int64_t B, T, H;
    int Dk, Dv, chunk;
    float scale;
    bool l2;
    const float *gk = nullptr;
    bool recurrent = false;
    // segment view (cu unset, chunked kernels of the plain and gated rule):
    // sequence b is segment b % segP of batch row b / segP, tokens
    // (b % segP) segL .. + segL of that row (B counts segments, T the row)
    int segP = 0, segL = 0;
};

hipError_t launch_chunk_fwd(const ChunkFwdArgs &a, bool bf16, hipStream_t stream);
// a without outputs or initial state (value rows from zero states into
// a.S_T) and, in the same launch, the d_k x d_k transition map of each
// sequence (from the identity) into M; plain or gated rule, bf16, d_k = d_v
// in {64, 128} (chunks of 32, or 64 at d_k = 128), else hipErrorNotSupported
// (before any launch).  chunk_state_pair_supported tells whether a's rule,
// dtype and sizes allow it.
bool chunk_state_pair_supported(const ChunkFwdArgs &a, bool bf16);
hipError_t launch_chunk_state_pair(const ChunkFwdArgs &a, float *M, bool bf16,
                                   hipStream_t stream);
hipError_t launch_fused_recurrent(const ChunkFwdArgs &a, bool bf16, hipStream_t stream);
// Segment-parallel schedule of the chunked forward (plain or gated rule, no
// packed sequences): P segments of L tokens (a multiple of the chunk), and
// the workspace it needs; P = 0 when the plain schedule fills the GPU anyway.
// combined: the call runs the combined state-and-map pass, which allows
// shorter segments at d_k <= 64 (never a larger workspace without it).
struct SegPlan {
    int P, L;
    int64_t bytes;
};
SegPlan seg_plan(int64_t B, int64_t T, int64_t H, int Dk, int Dv, int chunk, bool combined);
hipError_t launch_chunk_fwd_segmented(const ChunkFwdArgs &a, const SegPlan &pl, void *ws,
                                      bool bf16, hipStream_t stream);
// Device address of the library's static scratch (DR_STATIC_SCRATCH_BYTES)
// on the current device, resolved on the first call per device.
hipError_t static_scratch(void **ptr);

// Chunked KDA (per-channel decay): bf16, d_k = 128, d_v a multiple of 64;
// other cases run the token-serial kernel.
bool kda_chunk_supported(const ChunkFwdArgs &a, bool bf16);
hipError_t launch_kda_chunk(const ChunkFwdArgs &a, hipStream_t stream);

// Arguments of the backward of the chunked forward.  h holds the
// checkpoints the forward kernel wrote with chunk = chunk_bwd_chunk(bf16);
// dS_T and dS0 may be nullptr.  g, when set, is the log forget gate [B,T,H]
// (fp32) of the gated rule, and dg [B,T,H] (fp32) receives its gradient.
// dsb (like h) and dsz ([B,T,H,Dv], input dtype), when both are set, are
// scratch for the two-pass schedule (the gradient of every chunk's state,
// and the solve's Z).
struct ChunkBwdArgs {
    const void *q, *k, *v, *beta, *dout;
    const float *dS_T;
    const void *h;
    void *dq, *dk, *dv, *dbeta;
    float *dS0;
    int64_t B, T, H;
    int Dk, Dv;
    const float *g = nullptr;
    float *dg = nullptr;
    void *dsb = nullptr, *dsz = nullptr;
    void *segws = nullptr;  // per-segment maps of the segmented recursion
};

hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, bool bf16, hipStream_t stream);
// Chain over P segments per (b, h): S <- S M_p + H_p in fp32, segments first
// to last (rev: last to first); Hs holds H_p on entry and each step's
// incoming S on exit; S0 (or zero) enters, S_T (if set) gets the result.
hipError_t launch_seg_chain(float *Hs, const float *M, const float *S0, float *S_T, int64_t B,
                            int P, int64_t H, int Dk, int Dv, bool rev, hipStream_t stream);
// Tokens per chunk of the backward (and of its forward checkpoints).
int chunk_bwd_chunk(bool bf16);
// Segments of the backward's state-gradient recursion for few (b, h): P
// segments of L chunks (P = 0: no segments), and the bytes of their maps.
struct BwdSegPlan {
    int P, L;
};
BwdSegPlan bwd_seg_plan(int64_t B, int64_t H, int64_t N);
int64_t bwd_seg_bytes(int64_t B, int64_t H, int64_t N, int64_t Dk, int64_t Dv);

// Arguments of the token-serial backward of the per-key-channel decay rule.
// Without cu the nseq = B sequences are T tokens each; with cu, nseq packed
// sequences share one row of T tokens.  ws holds kda_bwd_workspace_bytes.
struct KdaBwdArgs {
    const void *q, *k, *v, *beta;
    const float *gk, *S0;
    const void *dout;
    const float *dS_T;
    void *dq, *dk, *dv, *dbeta;
    float *dgk, *dS0;
    void *ws;
    const int *cu;
    int64_t nseq, T, H;
    int Dk, Dv;
    float scale;
};

hipError_t launch_kda_bwd(const KdaBwdArgs &a, bool bf16, hipStream_t stream);
// Workspace bytes for ntok tokens in total (B*T, or T when packed) in nseq
// sequences; -1 for an unsupported d_k.
int64_t kda_bwd_workspace_bytes(int64_t ntok, int64_t nseq, int64_t H, int Dk, int Dv);

// Arguments of the single-token decode step (state updated in place).  g is
// the log forget gate [B,H] (fp32) of the gated rule, or nullptr; scale
// multiplies the outputs; l2 normalises q and k in the kernel; gk, when set
// (with g unset), is the per-key-channel log decay [B,H,Dk] (KDA).
struct StepArgs {
    const void *q, *k, *v, *beta;
    const float *g;
    float *S;
    void *o;
    int64_t BH;
    int Dk, Dv;
    float scale;
    bool l2;
    const float *gk;
};

hipError_t launch_recurrent_step(const StepArgs &a, bool bf16, hipStream_t stream);

}  // namespace dr
