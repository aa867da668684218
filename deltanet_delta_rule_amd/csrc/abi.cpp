// C ABI of libdeltarule: argument validation and dispatch to the HIP
// launchers.  Every check happens on the host before any HIP call, so a
// rejected call has enqueued nothing.  See include/deltarule.h for the
// contract of each entry point.
#include "deltarule.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "dr_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// A C caller may pass any int where the header says dr_dtype or dr_status.
// Loading such a value as a C++ enum outside its enumerators' range is
// undefined, so the entry points read the raw integer and check it before the
// value is used as an enum.
template <typename E>
int raw_enum(const E &e) {
    static_assert(sizeof(E) == sizeof(int), "the ABI's enums are int-sized");
    int v;
    memcpy(&v, &e, sizeof v);
    return v;
}
bool valid_dtype(const dr_dtype &d) {
    const int v = raw_enum(d);
    return v == DR_F32 || v == DR_BF16;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned_to(const void *p, int64_t n) {
    return (reinterpret_cast<uintptr_t>(p) % static_cast<uintptr_t>(n)) == 0;
}
bool supported_dim(int64_t d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int64_t c) { return c == 16 || c == 32 || c == 64; }

struct Span {
    const void *p;
    int64_t bytes;
};

bool overlaps(Span a, Span b) {
    if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
    return a0 < b0 + (uintptr_t)b.bytes && b0 < a0 + (uintptr_t)a.bytes;
}

// Product of non-negative factors, or -1 when it exceeds 2^62.
int64_t mul_checked(std::initializer_list<int64_t> xs) {
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x != 0 && r > (int64_t(1) << 62) / x) return -1;
        r *= x;
    }
    return r;
}

dr_status hip_status(hipError_t e) {
    if (e == hipSuccess) return DR_OK;
    g_last_hip_error = static_cast<int>(e);
    return DR_ERR_HIP;
}

// Shared validation and dispatch of the chunked forward.  g (log forget
// gate, fp32 [B,T,H]) is nullptr for the plain rule and required for the
// gated one when T > 0; cu (int32 [nseq+1], nullable) packs nseq sequences
// into the single batch row; scale multiplies the outputs.
dr_status chunk_fwd(const void *q, const void *k, const void *v, const void *beta,
                    const float *g, bool gated, const float *S0, void *o, float *S_T,
                    int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, int64_t chunk,
                    const int32_t *cu, int64_t nseq, float scale, bool l2, dr_dtype dtype,
                    void *stream, const float *gk = nullptr, bool recurrent = false,
                    void *ws = nullptr, int64_t ws_bytes = 0, bool noalloc = false,
                    void *ckpt = nullptr, int64_t ckpt_bytes = 0) {
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0 || chunk < 0) return DR_ERR_INVALID_ARG;
    if (cu && (B != 1 || nseq < 0 || !aligned_to(cu, 4))) return DR_ERR_INVALID_ARG;
    if (!(scale == scale) || scale - scale != 0.f) return DR_ERR_INVALID_ARG;  // NaN or inf
    if (!supported_dim(Dk) || !supported_dim(Dv) || !supported_chunk(chunk))
        return DR_ERR_UNSUPPORTED;
    const int64_t ns_count = cu ? nseq : B;  // sequences (states)
    if (ns_count == 0 || H == 0) return DR_OK;  // nothing to do

    const int64_t esz = dtype == DR_BF16 ? 2 : 4;
    const int64_t nqk = mul_checked({B, T, H, Dk}), nv = mul_checked({B, T, H, Dv});
    const int64_t nb = mul_checked({B, T, H}), ns = mul_checked({ns_count, H, Dv, Dk});
    if (nqk < 0 || nv < 0 || nb < 0 || ns < 0) return DR_ERR_UNSUPPORTED;
    // grid = sequences*H*(Dv/16) at most; sequence length and heads index in 32 bits
    if (T > INT32_MAX || H > INT32_MAX || mul_checked({ns_count, H, Dv / 16}) > INT32_MAX)
        return DR_ERR_UNSUPPORTED;
    // one chunk of one head (chunk tokens x H rows) is addressed with 32-bit
    // byte offsets
    const int64_t span = mul_checked({chunk, H, Dk > Dv ? Dk : Dv, esz});
    if (span < 0 || span > INT32_MAX / 2) return DR_ERR_UNSUPPORTED;

    if (T > 0 && (!q || !k || !v || !beta || !o)) return DR_ERR_INVALID_ARG;
    if (gated && T > 0 && !g) return DR_ERR_INVALID_ARG;
    if (gk && gated) return DR_ERR_INVALID_ARG;  // one decay kind
    if (ws && (ws_bytes < 0 || !aligned16(ws))) return DR_ERR_INVALID_ARG;
    if (noalloc && (ws || ws_bytes != 0)) return DR_ERR_INVALID_ARG;  // scratch is the library's
    // checkpoints for the backward: its chunk, the forward it differentiates
    if (ckpt && (cu || gk || recurrent || l2 || scale != 1.f || ws || noalloc ||
                 chunk != dr::chunk_bwd_chunk(dtype == DR_BF16) || !aligned16(ckpt)))
        return DR_ERR_INVALID_ARG;
    // q, k, gk and the states are read in 16-byte vectors and o is written
    // in 8- or 16-byte vectors (the chunked kernels); v and beta are read
    // element-wise
    const void *vec_ptrs[] = {q, k, S0, S_T, gk, o};
    for (const void *p : vec_ptrs)
        if (p && !aligned16(p)) return DR_ERR_INVALID_ARG;
    const void *elem_ptrs[] = {v, beta};
    for (const void *p : elem_ptrs)
        if (p && !aligned_to(p, esz)) return DR_ERR_INVALID_ARG;
    if (g && !aligned_to(g, 4)) return DR_ERR_INVALID_ARG;

    const Span in[] = {{q, nqk * esz},        {k, nqk * esz},
                       {v, nv * esz},         {beta, nb * esz},
                       {S0, ns * 4},          {gated ? g : nullptr, nb * 4},
                       {cu, (nseq + 1) * 4},  {gk, nqk * 4}};
    // the workspace is written before the inputs are read: an output too
    const Span so{o, nv * esz}, sst{S_T, ns * 4}, sws{ws, ws ? ws_bytes : 0};
    const Span sck{ckpt, ckpt ? ckpt_bytes : 0};
    for (const Span &s : in) {
        if (T > 0 && overlaps(so, s)) return DR_ERR_INVALID_ARG;
        // S_T may be exactly S0 (in-place carry); any other overlap is rejected
        if (overlaps(sst, s) && !(s.p == S0 && S_T == S0)) return DR_ERR_INVALID_ARG;
        if (overlaps(sws, s) || overlaps(sck, s)) return DR_ERR_INVALID_ARG;
    }
    if (T > 0 && overlaps(so, sst)) return DR_ERR_INVALID_ARG;
    if (overlaps(so, sws) || overlaps(sst, sws)) return DR_ERR_INVALID_ARG;
    if ((T > 0 && overlaps(so, sck)) || overlaps(sst, sck)) return DR_ERR_INVALID_ARG;

    dr::ChunkFwdArgs a{q,       k,        v,       beta,       gated ? g : nullptr,
                       S0,      o,        S_T,     ckpt,       cu,
                       ns_count, T,       H,       (int)Dk,    (int)Dv,
                       (int)chunk, scale, l2,     gk,       recurrent};
    // one long sequence per head: the segment-parallel schedule, when the
    // caller gave it a large enough workspace (or, without allocation, when
    // the library's static scratch holds what it needs)
    if ((ws || noalloc) && !cu && !recurrent && !ckpt &&
        (!gk || dr::kda_chunk_supported(a, dtype == DR_BF16))) {
        const dr::SegPlan pl =
            dr::seg_plan(B, T, H, (int)Dk, (int)Dv, (int)chunk,
                         dr::chunk_state_pair_supported(a, dtype == DR_BF16));
        if (noalloc && pl.P > 0) {
            if (pl.bytes > DR_STATIC_SCRATCH_BYTES) return DR_ERR_SCRATCH;
            const hipError_t e = dr::static_scratch(&ws);
            if (e != hipSuccess) return hip_status(e);
            ws_bytes = DR_STATIC_SCRATCH_BYTES;
        }
        if (pl.P > 0 && ws_bytes >= pl.bytes)
            return hip_status(dr::launch_chunk_fwd_segmented(
                a, pl, ws, dtype == DR_BF16, static_cast<hipStream_t>(stream)));
    }
    return hip_status(dr::launch_chunk_fwd(a, dtype == DR_BF16, static_cast<hipStream_t>(stream)));
}

// Shared validation and dispatch of the decode step; g (fp32 [B,H]) as above.
dr_status recurrent_step(const void *q, const void *k, const void *v, const void *beta,
                         const float *g, bool gated, float *S, void *o, int64_t B, int64_t H,
                         int64_t Dk, int64_t Dv, float scale, bool l2, dr_dtype dtype,
                         void *stream, const float *gk = nullptr) {
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || Dk < 0 || Dv < 0) return DR_ERR_INVALID_ARG;
    if (!(scale == scale) || scale - scale != 0.f) return DR_ERR_INVALID_ARG;  // NaN or inf
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DR_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return DR_OK;

    const int64_t esz = dtype == DR_BF16 ? 2 : 4;
    const int64_t bh = mul_checked({B, H});
    const int64_t ns = mul_checked({B, H, Dv, Dk});
    if (bh < 0 || ns < 0 || mul_checked({bh, Dv}) > INT32_MAX) return DR_ERR_UNSUPPORTED;

    if (!q || !k || !v || !beta || !S || !o) return DR_ERR_INVALID_ARG;
    if (gated && !g) return DR_ERR_INVALID_ARG;
    if (gk && (gated || !aligned16(gk))) return DR_ERR_INVALID_ARG;  // one decay kind
    // q, k and S are read in 16-byte vectors; v, beta and o element-wise
    if (!aligned16(q) || !aligned16(k) || !aligned16(S)) return DR_ERR_INVALID_ARG;
    if (!aligned_to(v, esz) || !aligned_to(beta, esz) || !aligned_to(o, esz))
        return DR_ERR_INVALID_ARG;
    if (g && !aligned_to(g, 4)) return DR_ERR_INVALID_ARG;
    const Span so{o, bh * Dv * esz}, ss{S, ns * 4};
    const Span in[] = {{q, bh * Dk * esz}, {k, bh * Dk * esz}, {v, bh * Dv * esz},
                       {beta, bh * esz}, {gated ? g : nullptr, bh * 4},
                       {gk, bh * Dk * 4}};
    if (overlaps(so, ss)) return DR_ERR_INVALID_ARG;
    for (const Span &s : in)
        if (overlaps(so, s) || overlaps(ss, s)) return DR_ERR_INVALID_ARG;

    const dr::StepArgs a{q,  k,       v,       beta,  gated ? g : nullptr, S, o,
                         bh, (int)Dk, (int)Dv, scale, l2,                  gk};
    return hip_status(
        dr::launch_recurrent_step(a, dtype == DR_BF16, static_cast<hipStream_t>(stream)));
}

// Workspace of the backward: every chunk's incoming state (the forward
// checkpoints), then the gradient of every chunk's state and the solve's Z
// ([B,T,H,Dv]) for the two-pass schedule, then (few heads) the segments'
// maps of the state-gradient recursion; each part 256-byte aligned.
struct BwdWs {
    int64_t ckpt, dsz, seg, total;  // bytes of the checkpoints, of Z, of the maps; all parts
};
BwdWs bwd_workspace(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, bool bf16) {
    const int64_t cb = dr::chunk_bwd_chunk(bf16);
    const int64_t N = (T + cb - 1) / cb;
    const int64_t esz = bf16 ? 2 : 4;
    BwdWs w;
    w.ckpt = mul_checked({B, H, N, Dv, Dk, esz});
    w.dsz = mul_checked({B, T, H, Dv, esz});
    w.seg = w.ckpt < 0 ? -1 : dr::bwd_seg_bytes(B, H, N, Dk, Dv);
    const auto al = [](int64_t x) { return (x + 255) / 256 * 256; };
    w.total = w.ckpt < 0 || w.dsz < 0 || w.seg < 0 || w.ckpt > INT64_MAX / 4 ||
                      w.dsz > INT64_MAX / 4 || w.seg > INT64_MAX / 4
                  ? -1
                  : 2 * al(w.ckpt) + al(w.dsz) + w.seg;
    return w;
}
int64_t bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, bool bf16) {
    return bwd_workspace(B, T, H, Dk, Dv, bf16).total;
}

dr_status chunk_bwd(const void *q, const void *k, const void *v, const void *beta,
                    const float *g, const float *S0, const void *dout, const float *dS_T,
                    void *dq, void *dk, void *dv, void *dbeta, float *dg, float *dS0, void *ws,
                    size_t ws_bytes, int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                    bool gated, dr_dtype dtype, void *stream, bool ckpt_ready = false) {
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return DR_ERR_INVALID_ARG;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DR_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return DR_OK;
    const bool bf16 = dtype == DR_BF16;
    const int64_t esz = bf16 ? 2 : 4;
    const int64_t nqk = mul_checked({B, T, H, Dk}), nv = mul_checked({B, T, H, Dv});
    const int64_t nb = mul_checked({B, T, H}), ns = mul_checked({B, H, Dv, Dk});
    const int64_t need = bwd_workspace_bytes(B, T, H, Dk, Dv, bf16);
    if (nqk < 0 || nv < 0 || nb < 0 || ns < 0 || need < 0) return DR_ERR_UNSUPPORTED;
    if (T > INT32_MAX || H > INT32_MAX || mul_checked({B, H}) > INT32_MAX) return DR_ERR_UNSUPPORTED;
    const int64_t span = mul_checked({32, H, Dk > Dv ? Dk : Dv, esz});
    if (span < 0 || span > INT32_MAX / 2) return DR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !beta || !dout || !dq || !dk || !dv || !dbeta))
        return DR_ERR_INVALID_ARG;
    if (gated && T > 0 && (!g || !dg)) return DR_ERR_INVALID_ARG;
    if (!gated) g = dg = nullptr;
    if (T > 0 && (!ws || (int64_t)ws_bytes < need)) return DR_ERR_INVALID_ARG;
    const void *vec_ptrs[] = {q, k, S0, dS_T, dS0, ws};
    for (const void *p : vec_ptrs)
        if (p && !aligned16(p)) return DR_ERR_INVALID_ARG;
    const void *elem_ptrs[] = {v, beta, dout, dq, dk, dv, dbeta};
    for (const void *p : elem_ptrs)
        if (p && !aligned_to(p, esz)) return DR_ERR_INVALID_ARG;
    if ((g && !aligned_to(g, 4)) || (dg && !aligned_to(dg, 4))) return DR_ERR_INVALID_ARG;
    // outputs must not overlap any input or each other
    const Span in[] = {{q, nqk * esz},  {k, nqk * esz},   {v, nv * esz},
                       {beta, nb * esz}, {S0, ns * 4},    {dout, nv * esz},
                       {dS_T, ns * 4},   {g, nb * 4}};
    const Span out[] = {{dq, nqk * esz},   {dk, nqk * esz}, {dv, nv * esz},
                        {dbeta, nb * esz}, {dS0, ns * 4},   {ws, need},
                        {dg, nb * 4}};
    for (const Span &o : out) {
        for (const Span &s : in)
            if (overlaps(o, s)) return DR_ERR_INVALID_ARG;
        for (const Span &o2 : out)
            if (&o2 != &o && overlaps(o, o2)) return DR_ERR_INVALID_ARG;
    }
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void *h = ws;
    if (T > 0 && !ckpt_ready) {
        const dr::ChunkFwdArgs f{q,      k,       v,        beta,     g,       S0,
                                 nullptr, nullptr, h,        nullptr,  B,       T,
                                 H,      (int)Dk, (int)Dv,  dr::chunk_bwd_chunk(bf16),
                                 1.f,    false};
        const hipError_t e = dr::launch_chunk_fwd(f, bf16, st);
        if (e != hipSuccess) return hip_status(e);
    }
    dr::ChunkBwdArgs a{q,  k,     v,   beta, dout, dS_T, h,       dq,      dk,
                       dv, dbeta, dS0, B,    T,    H,    (int)Dk, (int)Dv, g, dg};
    if (T > 0) {
        const BwdWs wl = bwd_workspace(B, T, H, Dk, Dv, bf16);
        const int64_t ck = (wl.ckpt + 255) / 256 * 256;
        a.dsb = static_cast<char *>(ws) + ck;
        a.dsz = static_cast<char *>(ws) + 2 * ck;
        if (wl.seg > 0) a.segws = static_cast<char *>(ws) + 2 * ck + (wl.dsz + 255) / 256 * 256;
    }
    return hip_status(dr::launch_chunk_bwd(a, bf16, st));
}

// Validation and dispatch of the token-serial backward of the per-channel
// decay rule (packed sequences as in chunk_fwd).
dr_status kda_bwd_impl(const void *q, const void *k, const void *v, const void *beta,
                       const float *gk, const float *S0, const void *dout, const float *dS_T,
                       void *dq, void *dk, void *dv, void *dbeta, float *dgk, float *dS0,
                       const int32_t *cu, int64_t nseq, float scale, void *ws, size_t ws_bytes,
                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv, dr_dtype dtype,
                       void *stream) {
    if (dtype != DR_F32 && dtype != DR_BF16) return DR_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return DR_ERR_INVALID_ARG;
    if (cu && (B != 1 || nseq < 0 || !aligned_to(cu, 4))) return DR_ERR_INVALID_ARG;
    if (!(scale == scale) || scale - scale != 0.f) return DR_ERR_INVALID_ARG;  // NaN or inf
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DR_ERR_UNSUPPORTED;
    const int64_t ns_count = cu ? nseq : B;
    if (ns_count == 0 || H == 0) return DR_OK;
    const bool bf16 = dtype == DR_BF16;
    const int64_t esz = bf16 ? 2 : 4;
    const int64_t nqk = mul_checked({B, T, H, Dk}), nv = mul_checked({B, T, H, Dv});
    const int64_t nb = mul_checked({B, T, H}), ns = mul_checked({ns_count, H, Dv, Dk});
    const int64_t ntok = mul_checked({B, T});
    if (nqk < 0 || nv < 0 || nb < 0 || ns < 0 || ntok < 0) return DR_ERR_UNSUPPORTED;
    const int64_t need = dr::kda_bwd_workspace_bytes(ntok, ns_count, H, (int)Dk, (int)Dv);
    if (need < 0) return DR_ERR_UNSUPPORTED;
    // grid = sequences * H * row tiles (at most Dv / 16) and token offsets in 32 bits
    if (T > INT32_MAX || H > INT32_MAX || mul_checked({ns_count, H, Dv / 16}) > INT32_MAX ||
        mul_checked({ns_count, 2048}) > INT32_MAX)
        return DR_ERR_UNSUPPORTED;
    if (T > 0 && (!q || !k || !v || !beta || !gk || !dout || !dq || !dk || !dv || !dbeta ||
                  !dgk))
        return DR_ERR_INVALID_ARG;
    if (T > 0 && (!ws || (int64_t)ws_bytes < need)) return DR_ERR_INVALID_ARG;
    if (T == 0) ws = nullptr;
    const void *vec_ptrs[] = {q, k, gk, S0, dS_T, dS0, dgk, ws};
    for (const void *p : vec_ptrs)
        if (p && !aligned16(p)) return DR_ERR_INVALID_ARG;
    const void *elem_ptrs[] = {v, beta, dout, dq, dk, dv, dbeta};
    for (const void *p : elem_ptrs)
        if (p && !aligned_to(p, esz)) return DR_ERR_INVALID_ARG;
    const Span in[] = {{q, nqk * esz},    {k, nqk * esz},   {v, nv * esz},
                       {beta, nb * esz},  {gk, nqk * 4},    {S0, ns * 4},
                       {dout, nv * esz},  {dS_T, ns * 4},   {cu, cu ? (nseq + 1) * 4 : 0}};
    const Span out[] = {{dq, nqk * esz},   {dk, nqk * esz}, {dv, nv * esz},
                        {dbeta, nb * esz}, {dgk, nqk * 4},  {dS0, ns * 4},
                        {ws, ws ? need : 0}};
    for (const Span &o : out) {
        for (const Span &s : in)
            if (overlaps(o, s)) return DR_ERR_INVALID_ARG;
        for (const Span &o2 : out)
            if (&o2 != &o && overlaps(o, o2)) return DR_ERR_INVALID_ARG;
    }
    dr::KdaBwdArgs a{q,   k,    v,     beta, gk,       S0,      dout,    dS_T,
                     dq,  dk,   dv,    dbeta, dgk,     dS0,     ws,      cu,
                     ns_count, T, H,   (int)Dk, (int)Dv, scale};
    return hip_status(dr::launch_kda_bwd(a, bf16, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

dr_status delta_rule_chunk_fwd(const void *q, const void *k, const void *v,
                               const void *beta, const float *S0, void *o,
                               float *S_T, int64_t B, int64_t T, int64_t H,
                               int64_t Dk, int64_t Dv, int64_t chunk,
                               dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return chunk_fwd(q, k, v, beta, nullptr, false, S0, o, S_T, B, T, H, Dk, Dv, chunk, nullptr,
                     0, 1.f, false, dtype, stream);
}

int64_t delta_rule_chunk_fwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                             int64_t Dv, int64_t chunk, dr_dtype dtype) {
    if (!valid_dtype(dtype)) return -1;
    if (B < 0 || T < 0 || H < 0 || !supported_dim(Dk) || !supported_dim(Dv) ||
        !supported_chunk(chunk))
        return -1;
    // the largest plan any rule takes for these sizes (the combined pass
    // allows the most segments)
    return dr::seg_plan(B, T, H, (int)Dk, (int)Dv, (int)chunk, true).bytes;
}

dr_status delta_rule_chunk_fwd_ex(const void *q, const void *k, const void *v,
                                  const void *beta, const float *S0, void *o, float *S_T,
                                  int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                  int64_t chunk, const dr_chunk_opts *opts, dr_dtype dtype,
                                  void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    dr_chunk_opts d{};
    d.scale = 1.f;
    const dr_chunk_opts &x = opts ? *opts : d;
    if (x.flags & ~uint32_t(DR_QK_L2NORM | DR_FUSED_RECURRENT))
        return DR_ERR_INVALID_ARG;  // unknown flags
    return chunk_fwd(q, k, v, beta, x.g, x.g != nullptr, S0, o, S_T, B, T, H, Dk, Dv, chunk,
                     x.cu_seqlens, x.num_seqs, x.scale, (x.flags & DR_QK_L2NORM) != 0, dtype,
                     stream, x.gk, (x.flags & DR_FUSED_RECURRENT) != 0, x.workspace,
                     x.workspace_bytes);
}

dr_status delta_rule_chunk_fwd_noalloc(const void *q, const void *k, const void *v,
                                       const void *beta, const float *S0, void *o, float *S_T,
                                       int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                       int64_t chunk, const dr_chunk_opts *opts, dr_dtype dtype,
                                       void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    dr_chunk_opts d{};
    d.scale = 1.f;
    const dr_chunk_opts &x = opts ? *opts : d;
    if (x.flags & ~uint32_t(DR_QK_L2NORM | DR_FUSED_RECURRENT))
        return DR_ERR_INVALID_ARG;  // unknown flags
    return chunk_fwd(q, k, v, beta, x.g, x.g != nullptr, S0, o, S_T, B, T, H, Dk, Dv, chunk,
                     x.cu_seqlens, x.num_seqs, x.scale, (x.flags & DR_QK_L2NORM) != 0, dtype,
                     stream, x.gk, (x.flags & DR_FUSED_RECURRENT) != 0, x.workspace,
                     x.workspace_bytes, true);
}

dr_status delta_rule_recurrent_step(const void *q, const void *k,
                                    const void *v, const void *beta, float *S,
                                    void *o, int64_t B, int64_t H, int64_t Dk,
                                    int64_t Dv, dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return recurrent_step(q, k, v, beta, nullptr, false, S, o, B, H, Dk, Dv, 1.f, false, dtype,
                          stream);
}

dr_status gated_delta_rule_chunk_fwd(const void *q, const void *k, const void *v,
                                     const void *beta, const float *g, const float *S0,
                                     void *o, float *S_T, int64_t B, int64_t T, int64_t H,
                                     int64_t Dk, int64_t Dv, int64_t chunk, dr_dtype dtype,
                                     void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return chunk_fwd(q, k, v, beta, g, true, S0, o, S_T, B, T, H, Dk, Dv, chunk, nullptr, 0, 1.f,
                     false, dtype, stream);
}

dr_status gated_delta_rule_recurrent_step(const void *q, const void *k, const void *v,
                                          const void *beta, const float *g, float *S, void *o,
                                          int64_t B, int64_t H, int64_t Dk, int64_t Dv,
                                          dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return recurrent_step(q, k, v, beta, g, true, S, o, B, H, Dk, Dv, 1.f, false, dtype, stream);
}

dr_status delta_rule_recurrent_step_ex(const void *q, const void *k, const void *v,
                                       const void *beta, float *S, void *o, int64_t B,
                                       int64_t H, int64_t Dk, int64_t Dv,
                                       const dr_step_opts *opts, dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    dr_step_opts d{};
    d.scale = 1.f;
    const dr_step_opts &x = opts ? *opts : d;
    if (x.flags & ~uint32_t(DR_QK_L2NORM)) return DR_ERR_INVALID_ARG;  // unknown flags
    return recurrent_step(q, k, v, beta, x.g, x.g != nullptr, S, o, B, H, Dk, Dv, x.scale,
                          (x.flags & DR_QK_L2NORM) != 0, dtype, stream, x.gk);
}

size_t delta_rule_chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk,
                                            int64_t Dv, dr_dtype dtype) {
    if (!valid_dtype(dtype)) return 0;
    if (B < 0 || T < 0 || H < 0 || !supported_dim(Dk) || !supported_dim(Dv) ||
        (dtype != DR_F32 && dtype != DR_BF16))
        return 0;
    const int64_t n = bwd_workspace_bytes(B, T, H, Dk, Dv, dtype == DR_BF16);
    return n < 0 ? 0 : (size_t)n;
}

dr_status delta_rule_chunk_bwd(const void *q, const void *k, const void *v, const void *beta,
                               const float *S0, const void *dout, const float *dS_T, void *dq,
                               void *dk, void *dv, void *dbeta, float *dS0, void *workspace,
                               size_t workspace_bytes, int64_t B, int64_t T, int64_t H,
                               int64_t Dk, int64_t Dv, dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return chunk_bwd(q, k, v, beta, nullptr, S0, dout, dS_T, dq, dk, dv, dbeta, nullptr, dS0,
                     workspace, workspace_bytes, B, T, H, Dk, Dv, false, dtype, stream);
}

dr_status gated_delta_rule_chunk_bwd(const void *q, const void *k, const void *v,
                                     const void *beta, const float *g, const float *S0,
                                     const void *dout, const float *dS_T, void *dq, void *dk,
                                     void *dv, void *dbeta, float *dg, float *dS0,
                                     void *workspace, size_t workspace_bytes, int64_t B,
                                     int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                     dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return chunk_bwd(q, k, v, beta, g, S0, dout, dS_T, dq, dk, dv, dbeta, dg, dS0, workspace,
                     workspace_bytes, B, T, H, Dk, Dv, true, dtype, stream);
}

dr_status delta_rule_chunk_fwd_checkpointed(const void *q, const void *k, const void *v,
                                            const void *beta, const float *g, const float *S0,
                                            void *o, float *S_T, void *workspace,
                                            size_t workspace_bytes, int64_t B, int64_t T,
                                            int64_t H, int64_t Dk, int64_t Dv, dr_dtype dtype,
                                            void *stream) {
    if (!valid_dtype(dtype) || (dtype != DR_F32 && dtype != DR_BF16)) return DR_ERR_INVALID_ARG;
    if (B < 0 || T < 0 || H < 0 || Dk < 0 || Dv < 0) return DR_ERR_INVALID_ARG;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return DR_ERR_UNSUPPORTED;
    if (B == 0 || H == 0) return DR_OK;
    const bool bf16 = dtype == DR_BF16;
    const int64_t need = bwd_workspace_bytes(B, T, H, Dk, Dv, bf16);
    if (need < 0) return DR_ERR_UNSUPPORTED;
    if (T > 0 && (!workspace || (int64_t)workspace_bytes < need)) return DR_ERR_INVALID_ARG;
    return chunk_fwd(q, k, v, beta, g, g != nullptr, S0, o, S_T, B, T, H, Dk, Dv,
                     dr::chunk_bwd_chunk(bf16), nullptr, 0, 1.f, false, dtype, stream, nullptr,
                     false, nullptr, 0, false, T > 0 ? workspace : nullptr,
                     bwd_workspace(B, T, H, Dk, Dv, bf16).ckpt);
}

dr_status delta_rule_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *beta,
                                  const float *g, const float *S0, const void *dout,
                                  const float *dS_T, void *dq, void *dk, void *dv, void *dbeta,
                                  float *dg, float *dS0, void *workspace, size_t workspace_bytes,
                                  int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                  uint32_t flags, dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    if (flags & ~(uint32_t)DR_BWD_CHECKPOINTS_READY) return DR_ERR_INVALID_ARG;
    return chunk_bwd(q, k, v, beta, g, S0, dout, dS_T, dq, dk, dv, dbeta, g ? dg : nullptr, dS0,
                     workspace, workspace_bytes, B, T, H, Dk, Dv, g != nullptr, dtype, stream,
                     (flags & DR_BWD_CHECKPOINTS_READY) != 0);
}

int64_t kda_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int64_t Dk, int64_t Dv,
                                int64_t num_seqs) {
    if (B < 0 || T < 0 || H < 0 || num_seqs < 0) return -1;
    if (!supported_dim(Dk) || !supported_dim(Dv)) return -1;
    const int64_t ntok = mul_checked({B, T});
    if (ntok < 0 || mul_checked({ntok + num_seqs, H, Dv, Dk, 16}) < 0) return -1;
    return dr::kda_bwd_workspace_bytes(ntok, num_seqs, H, (int)Dk, (int)Dv);
}

dr_status kda_bwd(const void *q, const void *k, const void *v, const void *beta,
                  const float *gk, const float *S0, const void *dout, const float *dS_T,
                  void *dq, void *dk, void *dv, void *dbeta, float *dgk, float *dS0,
                  const int32_t *cu_seqlens, int64_t num_seqs, float scale, void *workspace,
                  size_t workspace_bytes, int64_t B, int64_t T, int64_t H, int64_t Dk,
                  int64_t Dv, dr_dtype dtype, void *stream) {
    if (!valid_dtype(dtype)) return DR_ERR_INVALID_ARG;
    return kda_bwd_impl(q, k, v, beta, gk, S0, dout, dS_T, dq, dk, dv, dbeta, dgk, dS0,
                        cu_seqlens, num_seqs, scale, workspace, workspace_bytes, B, T, H, Dk,
                        Dv, dtype, stream);
}

const char *delta_rule_status_string(dr_status status) {
    switch (raw_enum(status)) {
    case DR_OK: return "DR_OK";
    case DR_ERR_INVALID_ARG: return "DR_ERR_INVALID_ARG: invalid argument";
    case DR_ERR_UNSUPPORTED: return "DR_ERR_UNSUPPORTED: unsupported size or shape";
    case DR_ERR_HIP: return "DR_ERR_HIP: HIP runtime error (see delta_rule_last_hip_error)";
    case DR_ERR_SCRATCH:
        return "DR_ERR_SCRATCH: the segment-parallel schedule of this shape needs more than "
               "the static scratch (DR_STATIC_SCRATCH_BYTES); pass a workspace instead";
    default: return "unknown dr_status";
    }
}

int delta_rule_last_hip_error(void) { return g_last_hip_error; }

int delta_rule_version(void) { return 21400; }

}  // extern "C"
