// Token-serial forward over whole sequences, the state kept in registers.
//
// The "fused recurrent" schedule of the recurrence (hada.io digest, section
// "Kernel Triton recurrent fusionne pour le decodage": each program owns a
// tile of one head's state and walks the tokens in order -- decay, predict
// with the key, residual, rank-1 write, read with the query).  It suits short
// sequences, where the chunked kernel's per-chunk set-up does not pay off, and
// it is the sequence forward of the per-key-channel decay (Kimi Delta
// Attention, same digest, section "Kimi Delta Attention : attenuation par
// canal").  Like the decode step it is vector work (no MFMA): per token each
// state row takes two dot products over d_k and one axpy.
//
// Work split.  A workgroup of 256 lanes owns RW = 256 / (d_k / 8) rows of one
// (sequence, head) state; d_k / 8 lanes share a row, each holding 8
// consecutive columns in registers for the whole sequence.  The inputs of 16
// tokens at a time (k, q, the workgroup's v rows, beta and the decay factors
// exp(g)) are staged in LDS in fp32, converted and exponentiated once per
// element on the way in rather than once per row, and double-buffered:
// the global loads of the next 16 tokens are issued before the current ones
// are processed and land in the other buffer afterwards, so the token loop
// reads only LDS.  State rows are read from S0 once and written to S_T once.
#include "dr_common.hpp"
#include "dr_launch.hpp"

namespace dr {

namespace {

// DECAY: 0 none, 1 scalar forget gate per (token, head) (Gated DeltaNet),
// 2 one log decay per key channel (KDA).
template <typename DT, int DK, int DECAY>
struct FrCfg {
    static constexpr int ESZ = sizeof(DT);
    static constexpr int LPR = DK / 8;       // lanes per state row
    static constexpr int RW = 256 / LPR;     // state rows per workgroup
    static constexpr int TB = 16;            // tokens per staged block
    static constexpr int VPR = DK * ESZ / 16;            // 16-byte input vectors per k (q) row
    static constexpr int KV = TB * VPR;                  // ... per block
    static constexpr int GV = DECAY == 2 ? TB * DK / 4 : 0;  // float4 vectors of gk per block
    static constexpr int NK = (KV + 255) / 256;
    static constexpr int NG = (GV + 255) / 256;
    static constexpr int NV = (TB * RW + 255) / 256;     // v elements per lane per block
    // byte offsets inside one LDS buffer (all fp32)
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = TB * DK * 4;
    static constexpr int OFF_G = 2 * TB * DK * 4;
    static constexpr int OFF_V = OFF_G + GV * 16;
    static constexpr int OFF_B = OFF_V + TB * RW * 4;
    static constexpr int OFF_A = OFF_B + TB * 4;
    static constexpr int BUF = OFF_A + TB * 4;
};

template <typename DT, int DK, int DECAY>
struct FrStage {
    typedef FrCfg<DT, DK, DECAY> C;
    uint4 k[C::NK], q[C::NK];
    float4 g[C::NG > 0 ? C::NG : 1];
    DT v[C::NV];        // raw: converted when stored, so no load waits here
    DT b;
    float a;
};

// 16 bytes of input (4 fp32 or 8 bf16 values) widened to fp32 into LDS.
__device__ __forceinline__ void put_f32(float *dst, const uint4 &x, float) {
    *reinterpret_cast<uint4 *>(dst) = x;
}
__device__ __forceinline__ void put_f32(float *dst, const uint4 &x, __bf16) {
    const bf16x8 h = __builtin_bit_cast(bf16x8, x);
    reinterpret_cast<float4 *>(dst)[0] = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
    reinterpret_cast<float4 *>(dst)[1] = make_float4((float)h[4], (float)h[5], (float)h[6], (float)h[7]);
}

__device__ __forceinline__ void lds8(const char *p, float (&x)[8], float) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    return group_sum<LPR>(x);
}

// The token rows of one (sequence, head): token t of the sequence is row
// (base + t) * H + h of the [*, H, d] input arrays.
struct SeqRows {
    int64_t base;   // first token of the sequence in the flattened (batch, time) axis
    int64_t H, h;
    __device__ __forceinline__ int64_t row(int t) const { return (base + t) * H + h; }
};

template <typename DT, int DK, int DECAY>
__device__ __forceinline__ void stage_load(FrStage<DT, DK, DECAY> &st, const DT *__restrict__ q,
                                           const DT *__restrict__ k, const DT *__restrict__ v,
                                           const DT *__restrict__ beta,
                                           const float *__restrict__ g, const SeqRows &sr,
                                           int t0, int nt, int row0, int Dv) {
    typedef FrCfg<DT, DK, DECAY> C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int n = 0; n < C::NK; ++n) {
        const int u = tid + 256 * n;
        const int i = u / C::VPR, c = u % C::VPR;
        st.k[n] = st.q[n] = make_uint4(0, 0, 0, 0);
        if (u < C::KV && i < nt) {
            const int64_t off = sr.row(t0 + i) * DK + c * (16 / C::ESZ);
            st.k[n] = *reinterpret_cast<const uint4 *>(k + off);
            st.q[n] = *reinterpret_cast<const uint4 *>(q + off);
        }
    }
    if constexpr (DECAY == 2) {
#pragma unroll
        for (int n = 0; n < C::NG; ++n) {
            const int u = tid + 256 * n;
            const int i = u / (DK / 4), c = u % (DK / 4);
            st.g[n] = make_float4(0.f, 0.f, 0.f, 0.f);
            if (u < C::GV && i < nt)
                st.g[n] = *reinterpret_cast<const float4 *>(g + sr.row(t0 + i) * DK + 4 * c);
        }
    }
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
        const int u = tid + 256 * n;
        const int i = u / C::RW, r = row0 + u % C::RW;
        st.v[n] = DT(0.f);
        if (u < C::TB * C::RW && i < nt && r < Dv) st.v[n] = v[sr.row(t0 + i) * Dv + r];
    }
    st.b = DT(0.f);
    st.a = 0.f;
    if (tid < nt) {
        st.b = beta[sr.row(t0 + tid)];
        if constexpr (DECAY == 1) st.a = g[sr.row(t0 + tid)];
    }
}

template <typename DT, int DK, int DECAY>
__device__ __forceinline__ void stage_store(const FrStage<DT, DK, DECAY> &st, char *buf) {
    typedef FrCfg<DT, DK, DECAY> C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int n = 0; n < C::NK; ++n) {
        const int u = tid + 256 * n;
        if (u < C::KV) {
            put_f32(reinterpret_cast<float *>(buf + C::OFF_K) + u * (16 / C::ESZ), st.k[n], DT{});
            put_f32(reinterpret_cast<float *>(buf + C::OFF_Q) + u * (16 / C::ESZ), st.q[n], DT{});
        }
    }
    if constexpr (DECAY == 2) {
#pragma unroll
        for (int n = 0; n < C::NG; ++n) {
            const int u = tid + 256 * n;
            if (u < C::GV) {
                const float4 x = st.g[n];
                reinterpret_cast<float4 *>(buf + C::OFF_G)[u] =
                    make_float4(__expf(x.x), __expf(x.y), __expf(x.z), __expf(x.w));
            }
        }
    }
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
        const int u = tid + 256 * n;
        if (u < C::TB * C::RW) reinterpret_cast<float *>(buf + C::OFF_V)[u] = to_f32(st.v[n]);
    }
    if (tid < C::TB) {
        reinterpret_cast<float *>(buf + C::OFF_B)[tid] = to_f32(st.b);
        if constexpr (DECAY == 1) reinterpret_cast<float *>(buf + C::OFF_A)[tid] = __expf(st.a);
    }
}

// One token's operands for one lane: its 8 columns of k and q (and of the
// channel decay factors), its row's v, beta and the scalar decay factor.
template <int DECAY>
struct FrTok {
    float k[8], q[8], g[DECAY == 2 ? 8 : 1];
    float v, b, a;
};

template <typename DT, int DK, int DECAY>
__device__ __forceinline__ void tok_load(const char *buf, int i, int sub, int rloc,
                                         FrTok<DECAY> &t) {
    typedef FrCfg<DT, DK, DECAY> C;
    lds8(buf + C::OFF_K + (i * DK + 8 * sub) * 4, t.k, float{});
    lds8(buf + C::OFF_Q + (i * DK + 8 * sub) * 4, t.q, float{});
    if constexpr (DECAY == 2) lds8(buf + C::OFF_G + (i * DK + 8 * sub) * 4, t.g, float{});
    t.v = reinterpret_cast<const float *>(buf + C::OFF_V)[i * C::RW + rloc];
    t.b = reinterpret_cast<const float *>(buf + C::OFF_B)[i];
    t.a = DECAY == 1 ? reinterpret_cast<const float *>(buf + C::OFF_A)[i] : 1.f;
}

// One token on one lane's 8 columns of a state row: decay, predict, correct,
// write, read (o_row receives the row's output from the row's first lane).
template <int DK, int DECAY, bool L2, typename DT>
__device__ __forceinline__ void fr_token(FrTok<DECAY> &t, float (&s)[8], int sub, bool live,
                                         DT *o_row, float scale) {
    constexpr int LPR = DK / 8;
    if constexpr (L2) {
        float kk = 0.f, qq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            kk += t.k[e] * t.k[e];
            qq += t.q[e] * t.q[e];
        }
        const float nk = rsqrtf(row_sum<LPR>(kk) + 1e-6f);
        const float nq = rsqrtf(row_sum<LPR>(qq) + 1e-6f);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            t.k[e] *= nk;
            t.q[e] *= nq;
        }
    }
    if constexpr (DECAY == 1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] *= t.a;
    }
    if constexpr (DECAY == 2) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[e] *= t.g[e];
    }
    float pk = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) pk += s[e] * t.k[e];
    pk = row_sum<LPR>(pk);                 // prediction from the decayed row
    const float u = t.b * (t.v - pk);      // corrected error
    float oq = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        s[e] += u * t.k[e];                // rank-1 write
        oq += s[e] * t.q[e];
    }
    oq = row_sum<LPR>(oq);                 // read after the write
    if (live && sub == 0 && o_row) *o_row = from_f32<DT>(oq * scale);
}

// Grid: (sequence, head, row slab) flattened, slab fastest.  cu (packed
// sequences, one batch row of T tokens) or the batch index picks the token
// range; offsets are clamped into [0, T] so that no access leaves the buffers.
template <typename DT, int DK, int DECAY, bool L2>
__global__ __launch_bounds__(256) void fused_recurrent_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ g, const float *S0,
    DT *__restrict__ o, float *S_T, const int *__restrict__ cu, int T, int H, int Dv,
    int wg_per_head, float scale) {
    typedef FrCfg<DT, DK, DECAY> C;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];

    const int part = blockIdx.x % wg_per_head;
    const int64_t seqhead = blockIdx.x / wg_per_head;   // n * H + h
    const int64_t n = seqhead / H;
    const int h = (int)(seqhead % H);
    int lo = 0, hi = T;
    int64_t batch = n;
    if (cu) {
        lo = min(max(cu[n], 0), T);
        hi = min(max(cu[n + 1], lo), T);
        batch = 0;
    }
    const SeqRows sr{batch * T + lo, H, h};
    const int len = hi - lo;

    const int sub = threadIdx.x % C::LPR, rloc = threadIdx.x / C::LPR;
    const int row0 = part * C::RW;
    const int row = row0 + rloc;
    const bool live = row < Dv;
    const int64_t srow = (seqhead * Dv + row) * DK + 8 * sub;

    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    if (S0 && live) {
        const float4 a = reinterpret_cast<const float4 *>(S0 + srow)[0];
        const float4 b = reinterpret_cast<const float4 *>(S0 + srow)[1];
        s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
        s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
    }
    // Retire the state load here, on every path: otherwise the compiler sees
    // it possibly pending at the token loop (which reads s) and waits for all
    // memory operations before that loop -- including the next block's
    // staging loads that are meant to overlap it.  (s_waitcnt vmcnt(0); the
    // export and LDS counters left at their maximum.)
    __builtin_amdgcn_s_waitcnt(0x0F70);

    const int nblk = (len + C::TB - 1) / C::TB;
    FrStage<DT, DK, DECAY> st;
    if (nblk > 0) {
        stage_load<DT, DK, DECAY>(st, q, k, v, beta, g, sr, 0, min(C::TB, len), row0, Dv);
        stage_store<DT, DK, DECAY>(st, smem);
    }
    lds_barrier();
    for (int j = 0; j < nblk; ++j) {
        const int t0 = j * C::TB;
        const int nt = min(C::TB, len - t0);
        const bool more = j + 1 < nblk;
        if (more)
            stage_load<DT, DK, DECAY>(st, q, k, v, beta, g, sr, t0 + C::TB,
                                      min(C::TB, len - t0 - C::TB), row0, Dv);
        const char *buf = smem + (j & 1) * C::BUF;
        // the next token's operands are read from LDS while this one computes;
        // two operand sets alternate so that no registers are copied
        FrTok<DECAY> ta, tb;
        tok_load<DT, DK, DECAY>(buf, 0, sub, rloc, ta);
        for (int i = 0; i < nt; i += 2) {
            tok_load<DT, DK, DECAY>(buf, min(i + 1, C::TB - 1), sub, rloc, tb);
            fr_token<DK, DECAY, L2>(ta, s, sub, live, o ? o + sr.row(t0 + i) * Dv + row : nullptr, scale);
            if (i + 1 >= nt) break;
            tok_load<DT, DK, DECAY>(buf, min(i + 2, C::TB - 1), sub, rloc, ta);
            fr_token<DK, DECAY, L2>(tb, s, sub, live, o ? o + sr.row(t0 + i + 1) * Dv + row : nullptr, scale);
        }
        if (more) stage_store<DT, DK, DECAY>(st, smem + ((j + 1) & 1) * C::BUF);
        lds_barrier();
    }
    if (S_T && live) {
        float4 *dst = reinterpret_cast<float4 *>(S_T + srow);
        dst[0] = make_float4(s[0], s[1], s[2], s[3]);
        dst[1] = make_float4(s[4], s[5], s[6], s[7]);
    }
}

template <typename DT, int DK, int DECAY, bool L2>
hipError_t launch_fr(const ChunkFwdArgs &a, hipStream_t stream) {
    typedef FrCfg<DT, DK, DECAY> C;
    const int wg_per_head = (a.Dv + C::RW - 1) / C::RW;
    const int64_t grid = a.B * a.H * wg_per_head;
    const float *g = DECAY == 2 ? a.gk : a.g;
    hipLaunchKernelGGL((fused_recurrent_kernel<DT, DK, DECAY, L2>), dim3((unsigned)grid),
                       dim3(256), 0, stream, static_cast<const DT *>(a.q),
                       static_cast<const DT *>(a.k), static_cast<const DT *>(a.v),
                       static_cast<const DT *>(a.beta), g, a.S0, static_cast<DT *>(a.o), a.S_T,
                       a.cu, (int)a.T, (int)a.H, a.Dv, wg_per_head, a.scale);
    return hipGetLastError();
}

template <typename DT, int DK>
hipError_t fr_opts(const ChunkFwdArgs &a, hipStream_t stream) {
    if (a.gk) return a.l2 ? launch_fr<DT, DK, 2, true>(a, stream) : launch_fr<DT, DK, 2, false>(a, stream);
    if (a.g) return a.l2 ? launch_fr<DT, DK, 1, true>(a, stream) : launch_fr<DT, DK, 1, false>(a, stream);
    return a.l2 ? launch_fr<DT, DK, 0, true>(a, stream) : launch_fr<DT, DK, 0, false>(a, stream);
}

template <typename DT>
hipError_t fr_dk(const ChunkFwdArgs &a, hipStream_t stream) {
    switch (a.Dk) {
    case 16: return fr_opts<DT, 16>(a, stream);
    case 32: return fr_opts<DT, 32>(a, stream);
    case 64: return fr_opts<DT, 64>(a, stream);
    case 128: return fr_opts<DT, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_fused_recurrent(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    return bf16 ? fr_dk<__bf16>(a, stream) : fr_dk<float>(a, stream);
}

}  // namespace dr
