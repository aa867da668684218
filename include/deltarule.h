/*
 * libdeltarule -- the DeltaNet delta-rule operator on AMD Instinct MI355X
 * (gfx950), behind a plain C ABI.
 *
 * The operator.  For every batch row b and head h independently, with a state
 * S of d_v x d_k mapping key space to value space:
 *
 *     S_t = S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *         = S_{t-1} + beta_t (v_t - S_{t-1} k_t) k_t^T
 *     o_t = S_t q_t                               (read after the write)
 *
 *   - houmin.site "infra/delta-net", section "DeltaNet 引入 Delta Rule":
 *     both forms of the update and the read o_t = S_t q_t;
 *   - hada.io digest "Tour d'horizon des variantes d'attention lineaire de la
 *     famille DeltaNet", sections "DeltaNet : ecrire l'erreur de prediction
 *     plutot que la valeur" and "Transition d'etat structuree";
 *   - frankenstein-transformer docs, deltanet_attn.py, module docstring: the
 *     same update with beta in (0,1) and L2-normalised keys.
 *
 * The operator does not normalise q or k, does not scale q and does not
 * clamp beta: callers pass the features they want (the DeltaNet layer of fla,
 * fla/layers/delta_net.py, feeds SiLU + L2-normalised q/k and may double beta
 * into (0,2)).
 *
 * Common conventions
 *   Layout   Contiguous row-major.  q, k: [B,T,H,Dk]; v, o: [B,T,H,Dv];
 *            beta: [B,T,H] (one scalar per token and head);
 *            states S0, S_T, S: [B,H,Dv,Dk], always fp32.
 *            The decode entry point drops the T axis.
 *   Dtype    DR_F32: q, k, v, beta, o are float.  DR_BF16: they are bfloat16
 *            (raw 16-bit storage).  States are float in both cases.  All
 *            accumulation is fp32.
 *   Sizes    Dk and Dv in {16, 32, 64, 128}; chunk in {16, 32, 64};
 *            B, H, T >= 0 (B or H zero: the call does nothing).  T and H
 *            must fit in int32, and so must B*H*Dv/16.  For the chunked
 *            entry point, chunk * H * max(Dk, Dv) * element size must not
 *            exceed 2^30 bytes (one chunk of all heads is addressed with
 *            32-bit offsets).
 *   Pointers Device pointers (hipMalloc'd or equivalent).  q, k and every
 *            state pointer must be 16-byte aligned (they are read as 16-byte
 *            vectors), and so must o of the sequence entry points (the
 *            chunked kernels write it in 8- or 16-byte vectors); v, beta and
 *            the decode step's o need only their element alignment.
 *            They are borrowed: the library never allocates, frees or keeps
 *            them beyond the work queued on `stream`.
 *   Stream   `stream` is a hipStream_t passed as void*; NULL is the default
 *            stream.  Calls only enqueue work: they never synchronise the
 *            device and never block on the GPU.  The backward may run part
 *            of its work on a second stream of the library's (see
 *            delta_rule_chunk_bwd); that work starts after the work queued
 *            on `stream` before the call, and work queued on `stream` after
 *            the call starts after it.
 *   Errors   Every entry point returns a dr_status.  Arguments are validated
 *            on the host before any HIP call; on DR_ERR_INVALID_ARG or
 *            DR_ERR_UNSUPPORTED nothing was enqueued.  DR_ERR_HIP means a HIP
 *            launch reported an error; the hipError_t value is then available
 *            from delta_rule_last_hip_error() on the calling thread.
 *   Threads  Global state: that thread-local error code; per GPU, the
 *            array of delta_rule_chunk_fwd_noalloc and, from the first
 *            backward call that splits its reverse walk, a second stream
 *            and two events (default priority), held until the process
 *            ends.  A call's fork, launches and join on that stream are
 *            enqueued under a per-GPU mutex.  Concurrent calls on different
 *            streams are safe (the noalloc entry point excepted, see
 *            there); calls on one stream run in order.
 */
#ifndef DELTARULE_H
#define DELTARULE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum dr_status {
    DR_OK = 0,
    DR_ERR_INVALID_ARG = 1, /* null/misaligned pointer, negative size, bad enum */
    DR_ERR_UNSUPPORTED = 2, /* valid request outside the supported size set */
    DR_ERR_HIP = 3,         /* a HIP runtime call failed; see last_hip_error */
    DR_ERR_SCRATCH = 4      /* the call needs more than the static scratch holds */
} dr_status;

typedef enum dr_dtype {
    DR_F32 = 0,
    DR_BF16 = 1
} dr_dtype;

/*
 * delta_rule_chunk_fwd -- training / prefill forward over whole sequences.
 *
 * Computes o[b,t,h,:] = S_t q_t for every token and, when S_T is not NULL,
 * the final state S_T = S_T(b,h) after the last token.  The result is the
 * token recurrence above; it is evaluated in the chunkwise-parallel form
 * (paperlayer summary of arXiv:2406.06484, section 3 "Parallelizing DeltaNet
 * Across the Sequence Dimension" and App. B.2 "UT transform derivation";
 * hada.io digest, section "Chunkwise KDA : reorganiser la recurrence en
 * multiplications matricielles"): per chunk of `chunk` tokens, a unit
 * lower-triangular solve resolves the chunk's errors against its incoming
 * state, then one set of matrix products writes the chunk's outputs and
 * advances the state.
 *
 *   q, k    [B,T,H,Dk]  inputs, dtype `dtype`
 *   v       [B,T,H,Dv]  input,  dtype `dtype`
 *   beta    [B,T,H]     input,  dtype `dtype`; any finite value
 *   S0      [B,H,Dv,Dk] fp32 initial state, or NULL for the zero state
 *   o       [B,T,H,Dv]  output, dtype `dtype`; every element is written
 *   S_T     [B,H,Dv,Dk] fp32 final state, or NULL to skip it.  S_T may be the
 *                       same buffer as S0 (state carried in place); any other
 *                       overlap between outputs and inputs is not allowed.
 *   chunk   tokens per chunk (16, 32 or 64).  T need not be a multiple of it;
 *           the last chunk is shorter.  The result does not depend on chunk
 *           beyond rounding.
 *
 * T == 0 writes S_T = S0 (or zeros) and no o.
 */
dr_status delta_rule_chunk_fwd(const void *q, const void *k, const void *v,
                               const void *beta, const float *S0, void *o,
                               float *S_T, int64_t B, int64_t T, int64_t H,
                               int64_t Dk, int64_t Dv, int64_t chunk,
                               dr_dtype dtype, void *stream);

/* Flags of dr_chunk_opts. */
enum {
    /* L2-normalise every token row of q and k inside the kernel:
     * x / sqrt(sum x^2 + 1e-6) (the l2norm of the gated layer on houmin.site
     * "infra/delta-net"; fla's use_qk_l2norm_in_kernel).  q and k are read as
     * given and never written. */
    DR_QK_L2NORM = 1u,
    /* Run the token-serial ("fused recurrent") schedule: one pass over the
     * tokens of each sequence with the state held on chip (hada.io digest,
     * section "Kernel Triton recurrent fusionne pour le decodage").  Same
     * results as the chunked schedule up to rounding; the chunk argument is
     * validated but unused.  Suited to short sequences.  With the
     * per-channel decay (gk) it is the path for any gk (see gk below). */
    DR_FUSED_RECURRENT = 2u
};

/*
 * Options of delta_rule_chunk_fwd_ex (zero-initialise, then set scale = 1).
 *
 *   g           [B,T,H] fp32 log forget gate, or NULL.  Non-NULL selects the
 *               gated rule of gated_delta_rule_chunk_fwd.
 *   cu_seqlens  device int32 [num_seqs+1], or NULL.  Non-NULL packs num_seqs
 *               variable-length sequences into one batch row (B must be 1):
 *               sequence s is tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of
 *               the T tokens, chunked from its own first token, with its own
 *               initial and final state: S0 and S_T are then
 *               [num_seqs,H,Dv,Dk].  Offsets should be non-decreasing from 0
 *               to T; the kernels clamp them into [0, T] (an empty or
 *               inverted range is an empty sequence) so that no access leaves
 *               the buffers.  The array must not change while the call runs.
 *               Tokens covered by no sequence get no output.  This is the
 *               packed layout of fla's `cu_seqlens` (fla
 *               fla/layers/delta_net.py, forward).
 *   num_seqs    number of packed sequences (>= 0) when cu_seqlens != NULL.
 *   scale       finite output scale: o = scale * S_t q_t (the same as
 *               scaling q; the DeltaNet layer passes none, the gated layer
 *               of houmin.site "infra/delta-net" divides q by sqrt(d_k)).
 *   flags       0 or a combination of DR_QK_L2NORM and DR_FUSED_RECURRENT.
 *   gk          [B,T,H,Dk] fp32 (16-byte aligned) per-key-channel log decay,
 *               or NULL.  Non-NULL selects Kimi Delta Attention (hada.io
 *               digest, section "Kimi Delta Attention : attenuation par
 *               canal"): before token t, column j of the state (key channel
 *               j) is multiplied by exp(gk_t[j]), then the token is
 *               predicted, corrected, written and read as in the plain rule.
 *               Exclusive with g (both set: DR_ERR_INVALID_ARG).  bf16 inputs
 *               with Dk = 128 and Dv a multiple of 64, without
 *               DR_FUSED_RECURRENT, run the chunked kernel (32-token
 *               chunks, same digest, "Chunkwise KDA"; the chunk argument is
 *               validated but unused).  It forms every decay ratio between
 *               two tokens of a chunk as a product of per-token factors
 *               exp(gk) <= 1, so it is exact up to rounding for any gk <= 0,
 *               down to -inf (a channel erased in one token).  Positive gk
 *               is computed as given while those products stay finite.  All
 *               other cases run the token-serial schedule.
 *   workspace, workspace_bytes
 *               device scratch (16-byte aligned, not overlapping any argument;
 *               an overlap is DR_ERR_INVALID_ARG)
 *               for the segment-parallel schedule, or NULL.  When the
 *               sequences are too few to fill the GPU (say B = 1, H = 16,
 *               T = 32768), the plain and gated rules and the chunked KDA
 *               kernel (not the token-serial schedule), without cu_seqlens, cut
 *               each sequence into P segments of whole chunks, run them in
 *               parallel from zero states and (with v = 0) from S = I to get
 *               each segment's affine state map S_out = S_in M + H, chain the
 *               maps in fp32, and run the segments again from their true
 *               incoming states for the outputs (about three passes of work
 *               on P times as many workgroups; the first two are one launch
 *               for the plain and gated rules in bf16 with Dk = Dv in
 *               {64, 128}).  Used
 *               only when workspace_bytes >=
 *               delta_rule_chunk_fwd_workspace_bytes(...) > 0 (the call may
 *               plan fewer segments, and use less of it, for other rules);
 *               otherwise the plain schedule runs and the workspace is not
 *               touched.  Results agree with the plain schedule up to
 *               rounding.
 */
typedef struct dr_chunk_opts {
    const float *g;
    const int32_t *cu_seqlens;
    int64_t num_seqs;
    float scale;
    uint32_t flags;
    const float *gk;
    void *workspace;
    int64_t workspace_bytes;
} dr_chunk_opts;

/*
 * Bytes of workspace for the segment-parallel schedule of
 * delta_rule_chunk_fwd_ex on this shape (B sequences of T tokens; enough for
 * every rule and dtype), or 0 when the plain schedule already fills the GPU
 * (the schedule is then never used); -1 for an unsupported dtype, dimension
 * or chunk.  Pure host arithmetic.
 */
int64_t delta_rule_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                             int64_t Dv, int64_t chunk, dr_dtype dtype);

/*
 * delta_rule_chunk_fwd_ex -- delta_rule_chunk_fwd with the options above
 * (opts == NULL: none, i.e. exactly delta_rule_chunk_fwd).  Every other
 * argument, size, layout and error behaves as in delta_rule_chunk_fwd; in
 * addition DR_ERR_INVALID_ARG is returned for cu_seqlens with B != 1, a
 * negative num_seqs, a misaligned cu_seqlens, cu_seqlens overlapping an
 * output, a non-finite scale or unknown flag bits.
 */
dr_status delta_rule_chunk_fwd_ex(const void *q, const void *k, const void *v,
                                  const void *beta, const float *S0, void *o, float *S_T,
                                  int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                  int64_t chunk, const dr_chunk_opts *opts, dr_dtype dtype,
                                  void *stream);

/*
 * Size of the static device scratch of delta_rule_chunk_fwd_noalloc, per GPU:
 * 16 MiB + 64 KiB, enough for the segment-parallel schedule of every shape
 * with Dv = 128 (B = 1, H = 16, T = 32768, d = 128 needs 16 MiB + 256 B).
 */
#define DR_STATIC_SCRATCH_BYTES ((int64_t)16 * 1024 * 1024 + 64 * 1024)

/*
 * delta_rule_chunk_fwd_noalloc -- delta_rule_chunk_fwd_ex for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the segment-parallel schedule takes
 * its scratch from a static device array of DR_STATIC_SCRATCH_BYTES that the
 * library holds on each GPU it runs on until the process ends, instead of
 * from opts->workspace.  Nothing is allocated or freed.
 *
 *   Every argument, size, layout and result is that of delta_rule_chunk_fwd_ex
 *   with a workspace of DR_STATIC_SCRATCH_BYTES, except:
 *   - opts->workspace must be NULL and opts->workspace_bytes 0
 *     (DR_ERR_INVALID_ARG otherwise);
 *   - when the segment-parallel schedule applies to the shape and needs more
 *     than DR_STATIC_SCRATCH_BYTES (delta_rule_chunk_fwd_workspace_bytes says
 *     how much), the call returns DR_ERR_SCRATCH and enqueues nothing; use
 *     delta_rule_chunk_fwd_ex with a workspace for such shapes;
 *   - the scratch belongs to the current device, which must be the device
 *     of `stream`.  Every call on a GPU shares that GPU's array (it keeps the
 *     last call's contents; each call writes everything it reads there before
 *     reading it), so calls that overlap in time on one GPU -- on different
 *     streams or from different threads -- race and give wrong results:
 *     serialise them.
 *   The first call on a device resolves the array's device address
 *   (hipGetSymbolAddress); a failure there is DR_ERR_HIP.
 */
dr_status delta_rule_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                       const void *beta, const float *S0, void *o, float *S_T,
                                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                       int64_t chunk, const dr_chunk_opts *opts, dr_dtype dtype,
                                       void *stream);

/*
 * delta_rule_recurrent_step -- one decode token per sequence, state in place.
 *
 * For every (b,h): reads S, applies the delta-rule write for the token
 * (q,k,v,beta) and stores the new state back into S, then writes
 * o = S_new q.  This is the token-serial schedule of the same recurrence
 * (hada.io digest, section "Kernel Triton recurrent fusionne pour le
 * decodage"; fla fla/layers/delta_net.py routes short inputs to its fused
 * recurrent kernel); S is streamed through HBM once per call.
 *
 *   q, k    [B,H,Dk]     inputs, dtype `dtype`
 *   v       [B,H,Dv]     input,  dtype `dtype`
 *   beta    [B,H]        input,  dtype `dtype`
 *   S       [B,H,Dv,Dk]  fp32 state, read and overwritten in place
 *   o       [B,H,Dv]     output, dtype `dtype`; must not overlap S
 */
dr_status delta_rule_recurrent_step(const void *q, const void *k,
                                    const void *v, const void *beta, float *S,
                                    void *o, int64_t B, int64_t H, int64_t Dk,
                                    int64_t Dv, dr_dtype dtype, void *stream);

/*
 * gated_delta_rule_chunk_fwd -- the gated rule (scalar forget gate), chunked.
 *
 * Each token first multiplies the whole state by alpha_t = exp(g_t), then
 * predicts from the decayed state, corrects and writes:
 *
 *     S_t = alpha_t S_{t-1} (I - beta_t k_t k_t^T) + beta_t v_t k_t^T
 *     o_t = S_t q_t
 *
 * (houmin.site "infra/delta-net", section "Gated DeltaNet"; hada.io digest,
 * section "Gated DeltaNet : oublier d'abord l'etat entier", which fixes the
 * order forget, predict, correct, write).  Evaluated chunkwise with the decay
 * carried as in-chunk prefix sums of g (hada.io digest, sections "Chunkwise
 * KDA" with a scalar decay and "Pipeline Triton Chunkwise").
 *
 *   g       [B,T,H] fp32, the natural log of the forget gate, required when
 *           T > 0 (4-byte aligned; must not overlap any output).  Values are
 *           expected to be <= 0 (alpha in (0,1]); g = 0 everywhere gives
 *           delta_rule_chunk_fwd's result up to rounding.  Within a chunk the
 *           kernel forms exp of differences of prefix sums, so positive g
 *           large enough to overflow fp32 over one chunk is not supported.
 *   Every other argument, size, layout and error behaves as in
 *   delta_rule_chunk_fwd.
 */
dr_status gated_delta_rule_chunk_fwd(const void *q, const void *k, const void *v,
                                     const void *beta, const float *g, const float *S0,
                                     void *o, float *S_T, int64_t B, int64_t T, int64_t H,
                                     int64_t Dk, int64_t Dv, int64_t chunk, dr_dtype dtype,
                                     void *stream);

/*
 * gated_delta_rule_recurrent_step -- one decode token of the gated rule per
 * sequence, state in place: S <- exp(g) S, then the delta-rule write and
 * o = S_new q as in delta_rule_recurrent_step.
 *
 *   g       [B,H] fp32, log forget gate of this token (required, 4-byte
 *           aligned, not overlapping S or o).
 *   Every other argument behaves as in delta_rule_recurrent_step.
 */
dr_status gated_delta_rule_recurrent_step(const void *q, const void *k, const void *v,
                                          const void *beta, const float *g, float *S, void *o,
                                          int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                                          dr_dtype dtype, void *stream);

/*
 * Options of delta_rule_recurrent_step_ex (zero-initialise, then set
 * scale = 1): g ([B,H] fp32 log forget gate, or NULL for the plain rule),
 * scale (finite output scale) and flags (0 or DR_QK_L2NORM), with the
 * meanings they have in dr_chunk_opts; gk ([B,H,Dk] fp32, 16-byte aligned,
 * or NULL): the per-key-channel log decay of Kimi Delta Attention (hada.io
 * digest, section "Kimi Delta Attention : attenuation par canal"): before
 * the token, column j of S (key channel j) is multiplied by exp(gk[j]).
 * g and gk are exclusive (both set: DR_ERR_INVALID_ARG).
 */
typedef struct dr_step_opts {
    const float *g;
    float scale;
    uint32_t flags;
    const float *gk;
} dr_step_opts;

/*
 * delta_rule_recurrent_step_ex -- delta_rule_recurrent_step with the options
 * above (opts == NULL: none).  Every other argument and error behaves as in
 * delta_rule_recurrent_step (g as in gated_delta_rule_recurrent_step); in
 * addition DR_ERR_INVALID_ARG is returned for a non-finite scale or unknown
 * flag bits.
 */
dr_status delta_rule_recurrent_step_ex(const void *q, const void *k, const void *v,
                                       const void *beta, float *S, void *o, int64_t B,
                                       int64_t H, int64_t Dk, int64_t Dv,
                                       const dr_step_opts *opts, dr_dtype dtype, void *stream);

/*
 * delta_rule_chunk_bwd -- gradients of delta_rule_chunk_fwd (plain rule).
 *
 * For upstream gradients dout = dL/do ([B,T,H,Dv], dtype `dtype`) and
 * dS_T = dL/dS_T ([B,H,Dv,Dk] fp32, or NULL for none), writes
 * dq, dk [B,T,H,Dk], dv [B,T,H,Dv], dbeta [B,T,H] (dtype `dtype`) and, when
 * dS0 is not NULL, dS0 = dL/dS0 [B,H,Dv,Dk] fp32.  The gradients are those of
 * the token recurrence; they are computed chunkwise (the training strategy
 * of the paperlayer summary of arXiv:2406.06484, section 3: the forward
 * states of every chunk are kept and the chunk-internal quantities
 * recomputed).  The call first reruns the forward pass to store each chunk's
 * incoming state in `workspace` (in `dtype`, the precision the backward's
 * products use it in), then walks the chunks in reverse.  With B*H <= 64
 * the walk is a reverse pass over the state-gradient recursion alone, then
 * the gradients of the chunks formed in parallel from its results; with
 * B*H <= 32 and at least 16 chunks that recursion itself runs in segments:
 * each segment's linear map and its response to dout are formed at once,
 * chained from the last segment, and the segments then run side by side
 * from their incoming state gradients.  With
 * 64 < B*H <= 128 (one workgroup per (b, h) would leave half the GPU idle)
 * and at least 8 chunks it goes in two pieces: the last ~21/32 of the
 * chunks run from dS_T on the library's second stream while `stream` runs
 * the recursion alone over those chunks, then the first ~11/32 from the
 * state gradient that gives.
 *
 *   q, k, v, beta, S0   the forward inputs, as in delta_rule_chunk_fwd
 *   workspace           device memory of at least
 *                       delta_rule_chunk_bwd_workspace_bytes(B,T,H,Dk,Dv,dtype)
 *                       bytes (16-byte aligned; contents on return: the
 *                       forward checkpoints, [B,H,N,Dv,Dk] in the input
 *                       dtype at its start, then scratch of the two-pass
 *                       schedule or the split walk's state gradient, and
 *                       of the segments' maps);
 *                       may be NULL when T == 0
 *   Outputs must not overlap the inputs, the workspace or each other.
 * Sizes as delta_rule_chunk_fwd (Dk, Dv in {16,32,64,128}); the chunk length
 * is chosen by the library (32 tokens for bf16, 16 for fp32).  Errors as
 * delta_rule_chunk_fwd; a missing or too small workspace is
 * DR_ERR_INVALID_ARG.
 */
size_t delta_rule_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                            int64_t Dv, dr_dtype dtype);

dr_status delta_rule_chunk_bwd(const void *q, const void *k, const void *v, const void *beta,
                               const float *S0, const void *dout, const float *dS_T, void *dq,
                               void *dk, void *dv, void *dbeta, float *dS0, void *workspace,
                               size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                               int64_t Dk, int64_t Dv, dr_dtype dtype, void *stream);

/*
 * gated_delta_rule_chunk_bwd -- gradients of gated_delta_rule_chunk_fwd.
 *
 * As delta_rule_chunk_bwd, with the log forget gate g among the inputs and
 * its gradient among the outputs.  The forward is the gated rule of the
 * hada.io digest (section "Gated DeltaNet : oublier d'abord l'etat entier",
 * chunkwise as in "Chunkwise KDA" with a scalar decay), and the gradients are
 * those of its token recurrence.  Within a chunk the decays are exponentials
 * of differences of in-chunk prefix sums b of g, so dg is the reverse
 * in-chunk cumulative sum of dL/db.
 *
 *   g       [B,T,H] fp32 log forget gate (required when T > 0, 4-byte
 *           aligned; values <= 0 as in gated_delta_rule_chunk_fwd)
 *   dg      [B,T,H] fp32 output dL/dg (required when T > 0, 4-byte aligned)
 *   workspace  delta_rule_chunk_bwd_workspace_bytes(B,T,H,Dk,Dv,dtype) bytes
 *   Every other argument, size and error behaves as in delta_rule_chunk_bwd;
 *   dg must not overlap the inputs, the workspace or the other outputs.
 */
dr_status gated_delta_rule_chunk_bwd(const void *q, const void *k, const void *v,
                                     const void *beta, const float *g, const float *S0,
                                     const void *dout, const float *dS_T, void *dq, void *dk,
                                     void *dv, void *dbeta, float *dg, float *dS0,
                                     void *workspace, size_t workspace_bytes, int64_t B,
                                     int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                     dr_dtype dtype, void *stream);

/* Static, human-readable name of a status code (never NULL). */
const char *delta_rule_status_string(dr_status status);

/* Flags of delta_rule_chunk_bwd_ex. */
enum {
    /* The workspace already holds the forward checkpoints of these very
     * inputs (written by delta_rule_chunk_fwd_checkpointed into the same
     * workspace, and not changed since): the backward skips its
     * checkpointing forward pass.  Nothing checks that the inputs match. */
    DR_BWD_CHECKPOINTS_READY = 1u
};

/*
 * delta_rule_chunk_fwd_checkpointed -- the forward of the plain rule (g ==
 * NULL) or the gated rule (g: [B,T,H] fp32 log forget gate) that also keeps
 * what the backward needs: o and S_T as delta_rule_chunk_fwd /
 * gated_delta_rule_chunk_fwd with the backward's chunk length (32 tokens for
 * bf16, 16 for fp32; output scale 1, no in-kernel norm, no packed
 * sequences), and every chunk's incoming state written to the start of
 * `workspace` in the layout the backward keeps there.  A training step then
 * runs this forward and delta_rule_chunk_bwd_ex with
 * DR_BWD_CHECKPOINTS_READY on the same workspace, so the states are formed
 * once (the training strategy of the paperlayer summary of arXiv:2406.06484,
 * section 3: the forward keeps the chunk states for the backward).
 *
 *   workspace   at least delta_rule_chunk_bwd_workspace_bytes(B,T,H,Dk,Dv,
 *               dtype) bytes, 16-byte aligned, not overlapping any argument;
 *               may be NULL when T == 0
 * Other arguments, sizes, layouts and errors as delta_rule_chunk_fwd (S_T
 * may be NULL; S_T may equal S0).  Results equal delta_rule_chunk_fwd's with
 * chunk = that length.
 */
dr_status delta_rule_chunk_fwd_checkpointed(const void *q, const void *k, const void *v,
                                            const void *beta, const float *g, const float *S0,
                                            void *o, float *S_T, void *workspace,
                                            size_t workspace_bytes, int64_t B, int64_t T,
                                            int64_t H, int64_t Dk, int64_t Dv, dr_dtype dtype,
                                            void *stream);

/*
 * delta_rule_chunk_bwd_ex -- delta_rule_chunk_bwd (g == NULL, dg ignored) or
 * gated_delta_rule_chunk_bwd (g and dg set) with flags: 0 or
 * DR_BWD_CHECKPOINTS_READY.  Arguments, sizes and errors as those entry
 * points; unknown flag bits are DR_ERR_INVALID_ARG.
 */
dr_status delta_rule_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *beta,
                                  const float *g, const float *S0, const void *dout,
                                  const float *dS_T, void *dq, void *dk, void *dv, void *dbeta,
                                  float *dg, float *dS0, void *workspace, size_t workspace_bytes,
                                  int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                  uint32_t flags, dr_dtype dtype, void *stream);

/*
 * kda_bwd -- gradients of the per-key-channel decay rule (Kimi Delta
 * Attention; hada.io digest, section "Kimi Delta Attention : attenuation par
 * canal") for any log decay, erased channels (gk = -inf or very negative)
 * included: the forward it differentiates is delta_rule_chunk_fwd_ex with
 * opts.gk (either schedule; they agree up to rounding), optionally with
 * opts.cu_seqlens and opts.scale, without DR_QK_L2NORM.  With a_t[j] =
 * exp(gk_t[j]): P_t = S_{t-1} Diag(a_t), e_t = v_t - P_t k_t, S_t = P_t +
 * beta_t e_t k_t^T, o_t = scale S_t q_t; the gradients are those of the
 * loss L = sum_t <do_t, o_t> + <dS_T, S_T> through that recurrence (the
 * backward with recomputed states of the paper summary of "Parallelizing
 * Linear Transformers with the Delta Rule over Sequence Length", section 3).
 *
 * Token-serial: one workgroup per (sequence, head, tile of state rows) walks
 * the sequence forward, storing the state every 16 tokens in the workspace,
 * then walks it backward block by block, recomputing each block's states.
 *
 *   q, k, v, beta, S0, dout, dS_T  as delta_rule_chunk_bwd (S0, dS_T may be
 *               NULL: zero); gk [B,T,H,Dk] fp32, 16-byte aligned
 *   cu_seqlens, num_seqs  packed sequences as in dr_chunk_opts (B must be 1;
 *               S0, dS_T and dS0 are then [num_seqs,H,Dv,Dk]), or NULL
 *   scale       finite output scale of the forward
 *   dq, dk      [B,T,H,Dk] in the input dtype
 *   dv          [B,T,H,Dv] in the input dtype
 *   dbeta       [B,T,H] in the input dtype
 *   dgk         [B,T,H,Dk] fp32, 16-byte aligned
 *   dS0         [B,H,Dv,Dk] fp32 or NULL (not written)
 *   workspace   kda_bwd_workspace_bytes(B,T,H,Dk,Dv,num_seqs) bytes (num_seqs
 *               = B without packing), 16-byte aligned; may be NULL when
 *               T == 0.  Contents on return: scratch.
 *   Tokens covered by no packed sequence get no gradient (left untouched).
 *   Outputs must not overlap the inputs, the workspace or each other.
 * Sizes: Dk, Dv in {16,32,64,128}, else DR_ERR_UNSUPPORTED.  Other errors as
 * delta_rule_chunk_bwd; a missing or too small workspace, a non-finite
 * scale or cu_seqlens with B != 1 is DR_ERR_INVALID_ARG.  Asynchronous on
 * `stream`; allocates nothing.
 */
int64_t kda_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                int64_t num_seqs);

dr_status kda_bwd(const void *q, const void *k, const void *v, const void *beta,
                  const float *gk, const float *S0, const void *dout, const float *dS_T,
                  void *dq, void *dk, void *dv, void *dbeta, float *dgk, float *dS0,
                  const int32_t *cu_seqlens, int64_t num_seqs, float scale, void *workspace,
                  size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t Dk,
                  int64_t Dv, dr_dtype dtype, void *stream);

/* The hipError_t value of the last DR_ERR_HIP returned on this thread
 * (0 if none). */
int delta_rule_last_hip_error(void);

/* Library version as major*10000 + minor*100 + patch (2.0.0: the gated
 * entry points; 2.1.0: delta_rule_chunk_fwd_ex; 2.2.0: DR_QK_L2NORM; 2.3.0:
 * delta_rule_recurrent_step_ex; 2.4.0: delta_rule_chunk_bwd; 2.5.0: per-channel
 * decay (gk) in dr_step_opts; 2.6.0: DR_FUSED_RECURRENT and gk in
 * dr_chunk_opts; 2.7.0: the segment-parallel schedule's workspace in
 * dr_chunk_opts and delta_rule_chunk_fwd_workspace_bytes; 2.8.0:
 * delta_rule_chunk_fwd_noalloc and DR_ERR_SCRATCH; 2.9.0:
 * gated_delta_rule_chunk_bwd; 2.10.0: the backward's workspace also holds
 * the scratch of its two-pass schedule; 2.11.0: the backward's split
 * reverse walk on a second stream; 2.12.0: the segmented state-gradient
 * recursion for few heads, its maps in the workspace; 2.13.0:
 * delta_rule_chunk_fwd_checkpointed and delta_rule_chunk_bwd_ex; 2.14.0:
 * kda_bwd). */
int delta_rule_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DELTARULE_H */
