// Backward of the per-key-channel decay rule (Kimi Delta Attention), token
// by token, exact for any log decay gk <= 0 (a channel erased in one token
// included).
//
// The forward (hada.io digest, section "Kimi Delta Attention : attenuation
// par canal": decay the state's key columns, predict, correct, write, read),
// per (sequence, head) with a_t[j] = exp(gk_t[j]):
//
//   P_t = S_{t-1} Diag(a_t);  e_t = v_t - P_t k_t;  S_t = P_t + beta_t e_t k_t^T;
//   o_t = scale S_t q_t.
//
// Its gradients, token by token in reverse with D = dL/dS_t (dS_T at the end):
//
//   D += scale do_t q_t^T;     dq_t = scale S_t^T do_t;     w = D k_t;
//   dv_t = beta_t w;           dbeta_t = e_t . w;
//   dk_t = beta_t (D^T e_t - P_t^T w);
//   D -= beta_t w k_t^T;       dgk_t[j] = sum_i D_ij (P_t)_ij;    D <- D Diag(a_t)
//
// and dS0 = D.  The pages give the strategy of recomputing states in the
// backward (paper summary of "Parallelizing Linear Transformers with the Delta
// Rule over Sequence Length", section 3) and these equations follow from the
// chain rule through one token.
//
// Work split.  Row i of the state depends only on row i before it, in both
// directions, so a workgroup owns RW rows of one (sequence, head) state and
// needs no other workgroup: LPR = d_k / 8 lanes per row, each holding 8
// consecutive columns (as the token-serial forward), and at d_k >= 64 two
// rows per lane (RL rows apart), which fills the GPU in one round at the
// layer shape and halves the cross-row sums per row.  Only dq, dk, dgk and
// dbeta are sums over all rows: each lane first adds its own rows' terms,
// then each workgroup adds up its rows (a reduce-scatter on lane swaps
// inside a wave, then across its waves in LDS, two tokens per barrier) and
// writes one partial per row tile to the workspace; a second kernel adds the
// tiles' partials and converts them.
//
// Phases of the main kernel:
//   1. the forward over the sequence, storing the state at the start of every
//      16-token block to the workspace (each lane its own values, read back
//      by the same lane);
//   2. blocks last to first (with two rows per lane, in two halves of 8
//      tokens, the second half first): the block's starting state reloaded
//      and advanced to the sub-block, its tokens recomputed with every
//      decayed pre-token state P_t kept in registers, then walked in
//      reverse.
// The inputs of a block (k, q, exp(gk), the workgroup's rows of v and do,
// beta) are staged in LDS in fp32 and double-buffered: the next block's
// global loads are in flight while the current one is processed.
#include <algorithm>

#include "dr_common.hpp"
#include "dr_launch.hpp"

namespace dr {

namespace {

// Lanes per workgroup: 128 rows of d_k / 8 lanes, at most 512.
template <int DK>
struct KbLanes {
    static constexpr int value = DK / 8 * 128 < 512 ? DK / 8 * 128 : 512;
};

template <typename DT, int DK, int RPL_ = 1, int NTH_ = KbLanes<DK>::value>
struct KbCfg {
    static constexpr int ESZ = sizeof(DT);
    static constexpr int LPR = DK / 8;                          // lanes per state row
    static constexpr int NTH = NTH_;
    static constexpr int RPL = RPL_;                            // state rows per lane
    static constexpr int RL = NTH / LPR;                        // rows of one lane layer
    static constexpr int RW = RPL * RL;                         // state rows per workgroup
    static constexpr int NWV = NTH / 64;
    static constexpr int TB = 16;                               // tokens per block
    static constexpr int HB = TB / RPL;                         // tokens of a sub-block
    static constexpr int G = 2;                                 // tokens per cross-wave sum
    static constexpr int NRED = 3 * DK + 4;                     // dq, dk, dgk, dbeta (+ pad)
    static constexpr int VPR = DK * ESZ / 16;                   // 16-byte vectors per k row
    static constexpr int KV = TB * VPR;
    static constexpr int GV = TB * DK / 4;                      // float4 of gk per block
    static constexpr int NK = (KV + NTH - 1) / NTH;
    static constexpr int NG = (GV + NTH - 1) / NTH;
    static constexpr int NV = (TB * RW + NTH - 1) / NTH;
    // byte offsets in one staging buffer (all fp32)
    static constexpr int OFF_K = 0;
    static constexpr int OFF_Q = TB * DK * 4;
    static constexpr int OFF_A = 2 * TB * DK * 4;
    static constexpr int OFF_V = 3 * TB * DK * 4;
    static constexpr int OFF_D = OFF_V + TB * RW * 4;
    static constexpr int OFF_B = OFF_D + TB * RW * 4;
    static constexpr int BUF = OFF_B + TB * 4;
    static constexpr int RED = 2 * G * NWV * NRED;              // floats, two parities
};

template <typename DT, int DK, int RPL, int NTH>
struct KbStage {
    typedef KbCfg<DT, DK, RPL, NTH> C;
    uint4 k[C::NK], q[C::NK];
    float4 g[C::NG];
    DT v[C::NV], d[C::NV];
    DT b;
};

// Token row of one (sequence, head): token t is row (base + t) * H + h of the
// [*, H, d] arrays.
struct KbRows {
    int64_t base, H, h;
    __device__ __forceinline__ int64_t row(int t) const { return (base + t) * H + h; }
};

template <typename DT, int DK, int RPL, int NTH>
__device__ __forceinline__ void kb_load(KbStage<DT, DK, RPL, NTH> &st, const DT *__restrict__ q,
                                        const DT *__restrict__ k, const DT *__restrict__ v,
                                        const DT *__restrict__ beta, const float *__restrict__ gk,
                                        const DT *__restrict__ dout, const KbRows &sr, int t0,
                                        int nt, int row0, int Dv, bool want_qd) {
    typedef KbCfg<DT, DK, RPL, NTH> C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int n = 0; n < C::NK; ++n) {
        const int u = tid + C::NTH * n;
        const int i = u / C::VPR, c = u % C::VPR;
        st.k[n] = st.q[n] = make_uint4(0, 0, 0, 0);
        if (u < C::KV && i < nt) {
            const int64_t off = sr.row(t0 + i) * DK + c * (16 / C::ESZ);
            st.k[n] = *reinterpret_cast<const uint4 *>(k + off);
            if (want_qd) st.q[n] = *reinterpret_cast<const uint4 *>(q + off);
        }
    }
#pragma unroll
    for (int n = 0; n < C::NG; ++n) {
        const int u = tid + C::NTH * n;
        const int i = u / (DK / 4), c = u % (DK / 4);
        st.g[n] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (u < C::GV && i < nt)
            st.g[n] = *reinterpret_cast<const float4 *>(gk + sr.row(t0 + i) * DK + 4 * c);
    }
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
        const int u = tid + C::NTH * n;
        const int i = u / C::RW, r = row0 + u % C::RW;
        st.v[n] = st.d[n] = DT(0.f);
        if (u < C::TB * C::RW && i < nt && r < Dv) {
            st.v[n] = v[sr.row(t0 + i) * Dv + r];
            if (want_qd) st.d[n] = dout[sr.row(t0 + i) * Dv + r];
        }
    }
    st.b = DT(0.f);
    if (tid < nt) st.b = beta[sr.row(t0 + tid)];
}

__device__ __forceinline__ void kb_put(float *dst, const uint4 &x, float) {
    *reinterpret_cast<uint4 *>(dst) = x;
}
__device__ __forceinline__ void kb_put(float *dst, const uint4 &x, __bf16) {
    const bf16x8 h = __builtin_bit_cast(bf16x8, x);
    reinterpret_cast<float4 *>(dst)[0] = make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
    reinterpret_cast<float4 *>(dst)[1] = make_float4((float)h[4], (float)h[5], (float)h[6], (float)h[7]);
}

template <typename DT, int DK, int RPL, int NTH>
__device__ __forceinline__ void kb_store(const KbStage<DT, DK, RPL, NTH> &st, char *buf) {
    typedef KbCfg<DT, DK, RPL, NTH> C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int n = 0; n < C::NK; ++n) {
        const int u = tid + C::NTH * n;
        if (u < C::KV) {
            kb_put(reinterpret_cast<float *>(buf + C::OFF_K) + u * (16 / C::ESZ), st.k[n], DT{});
            kb_put(reinterpret_cast<float *>(buf + C::OFF_Q) + u * (16 / C::ESZ), st.q[n], DT{});
        }
    }
#pragma unroll
    for (int n = 0; n < C::NG; ++n) {
        const int u = tid + C::NTH * n;
        if (u < C::GV) {
            const float4 x = st.g[n];
            reinterpret_cast<float4 *>(buf + C::OFF_A)[u] =
                make_float4(__expf(x.x), __expf(x.y), __expf(x.z), __expf(x.w));
        }
    }
#pragma unroll
    for (int n = 0; n < C::NV; ++n) {
        const int u = tid + C::NTH * n;
        if (u < C::TB * C::RW) {
            reinterpret_cast<float *>(buf + C::OFF_V)[u] = to_f32(st.v[n]);
            reinterpret_cast<float *>(buf + C::OFF_D)[u] = to_f32(st.d[n]);
        }
    }
    if (tid < C::TB) reinterpret_cast<float *>(buf + C::OFF_B)[tid] = to_f32(st.b);
}

__device__ __forceinline__ void kb_lds8(const char *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Sum over the rows of the wave at the same column position: the rows sit
// LPR lanes apart, so rotations of the 16-lane DPP row by LPR, 2 LPR, ...
// keep every lane's column and leave it the sum over the rows in its DPP row.
template <int LPR>
__device__ __forceinline__ float kb_dpp_rows_sum(float x) {
    if constexpr (LPR <= 1) x += dpp_move<0x121>(x);  // row_ror:1
    if constexpr (LPR <= 2) x += dpp_move<0x122>(x);  // row_ror:2
    if constexpr (LPR <= 4) x += dpp_move<0x124>(x);  // row_ror:4
    if constexpr (LPR <= 8) x += dpp_move<0x128>(x);  // row_ror:8
    return x;
}

// a + b after swapping the upper 32 lanes of a with the lower 32 of b: the
// lower half then holds a's two halves added, the upper half b's.
__device__ __forceinline__ float kb_fold32(float a, float b) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// a + b after swapping the odd 16-lane rows of a with the even rows of b:
// rows 0 and 2 then hold a's row pairs added, rows 1 and 3 b's.
__device__ __forceinline__ float kb_fold16(float a, float b) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Reduce-scatter of 24 per-lane values over the 4 DPP rows of the wave
// (after kb_dpp_rows_sum): value x[e + 6 r] summed over the wave's rows ends
// in z[e] of the lanes of DPP row r (e < 6).  Two halvings of the values
// (upper with lower half of the wave, then odd with even rows), 18 lane
// swaps instead of 48 for a sum in every lane.
__device__ __forceinline__ void kb_scatter24(const float (&x)[24], float (&z)[6]) {
    float y[12];
#pragma unroll
    for (int e = 0; e < 12; ++e) y[e] = kb_fold32(x[e], x[e + 12]);
    // lower half: x[e] (rows 0,1), upper half: x[e + 12] (rows 2,3)
#pragma unroll
    for (int e = 0; e < 6; ++e) z[e] = kb_fold16(y[e], y[e + 6]);
    // row 0: x[e], row 1: x[e + 6], row 2: x[e + 12], row 3: x[e + 18]
}

// One token forward on a lane's rows: decay, predict, correct, write.
template <int LPR, int RPL>
__device__ __forceinline__ void kb_fwd_token(float (&s)[RPL][8], const float (&kk)[8],
                                             const float (&aa)[8], const float (&vv)[RPL],
                                             float bb) {
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
        float pk = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            s[u][e] *= aa[e];
            pk += s[u][e] * kk[e];
        }
        const float bu = bb * (vv[u] - group_sum<LPR>(pk));
#pragma unroll
        for (int e = 0; e < 8; ++e) s[u][e] += bu * kk[e];
    }
}

// Grid: (sequence, head, row tile) flattened, tile fastest.  cu (packed
// sequences in one batch row of T tokens) or the batch index picks the token
// range; offsets are clamped into [0, T].  Checkpoint slots of a sequence
// start at block base / 16 + n (disjoint between sequences, in bounds for
// any offsets).  A lane holds RPL rows, RL rows apart, and 8 columns of each.
template <typename DT, int DK, int RPL_, int NTH_>
__global__ __launch_bounds__(NTH_) void kda_bwd_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ gk, const float *__restrict__ S0,
    const DT *__restrict__ dout, const float *__restrict__ dS_T, DT *__restrict__ dv,
    float *__restrict__ dS0, float *__restrict__ ckpt, float *__restrict__ part,
    float *__restrict__ partb, const int *__restrict__ cu, int T, int H, int Dv, int R,
    int64_t rows_total, float scale) {
    typedef KbCfg<DT, DK, RPL_, NTH_> C;
    constexpr int LPR = C::LPR, TB = C::TB, G = C::G, RPL = C::RPL, RL = C::RL, HB = C::HB;
    static_assert(HB % (2 * G) == 0 && TB == RPL * HB, "whole flush-group pairs per sub-block");
    __shared__ __attribute__((aligned(16))) char smem[2 * C::BUF];
    __shared__ __attribute__((aligned(16))) float red[C::RED];

    const int tile = blockIdx.x % R;
    const int64_t seqhead = blockIdx.x / R;   // n * H + h
    const int64_t n = seqhead / H;
    const int h = (int)(seqhead % H);
    int lo = 0, hi = T;
    int64_t batch = n;
    if (cu) {
        lo = min(max(cu[n], 0), T);
        hi = min(max(cu[n + 1], lo), T);
        batch = 0;
    }
    const KbRows sr{batch * T + lo, H, h};
    const int len = hi - lo;
    const int nblk = (len + TB - 1) / TB;
    const int64_t blk0 = sr.base / TB + n;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int sub = tid % LPR, rloc = tid / LPR;
    const int row0 = tile * C::RW;
    int row[RPL];
    bool live[RPL];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
        row[u] = row0 + rloc + u * RL;
        live[u] = row[u] < Dv;
    }
    auto srow = [&](int u) { return (seqhead * Dv + row[u]) * DK + 8 * sub; };
    auto ck_at = [&](int j, int u) {
        return ckpt + (((blk0 + j) * H + h) * (int64_t)(R * C::RW) + row[u]) * DK + 8 * sub;
    };
    auto lds_v = [&](const char *buf, int off, int i, float (&x)[RPL]) {
#pragma unroll
        for (int u = 0; u < RPL; ++u)
            x[u] = reinterpret_cast<const float *>(buf + off)[i * C::RW + rloc + u * RL];
    };
    auto load8 = [&](const float *p, float (&x)[8]) {
        const float4 a0 = reinterpret_cast<const float4 *>(p)[0];
        const float4 a1 = reinterpret_cast<const float4 *>(p)[1];
        x[0] = a0.x; x[1] = a0.y; x[2] = a0.z; x[3] = a0.w;
        x[4] = a1.x; x[5] = a1.y; x[6] = a1.z; x[7] = a1.w;
    };

    // ---- phase 1: forward, the state at every block start to the workspace
    float s[RPL][8];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) s[u][e] = 0.f;
        if (S0 && live[u]) load8(S0 + srow(u), s[u]);
    }
    KbStage<DT, DK, RPL, NTH_> st;
    if (nblk > 0) {
        kb_load<DT, DK, RPL, NTH_>(st, q, k, v, beta, gk, dout, sr, 0, min(TB, len), row0, Dv, false);
        kb_store<DT, DK, RPL, NTH_>(st, smem);
    }
    lds_barrier();
    for (int j = 0; j < nblk; ++j) {
        const int t0 = j * TB, nt = min(TB, len - t0);
        const bool more = j + 1 < nblk;
        if (more)
            kb_load<DT, DK, RPL, NTH_>(st, q, k, v, beta, gk, dout, sr, t0 + TB, min(TB, len - t0 - TB),
                            row0, Dv, false);
#pragma unroll
        for (int u = 0; u < RPL; ++u) {
            float4 *cp = reinterpret_cast<float4 *>(ck_at(j, u));
            cp[0] = make_float4(s[u][0], s[u][1], s[u][2], s[u][3]);
            cp[1] = make_float4(s[u][4], s[u][5], s[u][6], s[u][7]);
        }
        const char *buf = smem + (j & 1) * C::BUF;
        for (int i = 0; i < nt; ++i) {
            float kk[8], aa[8], vv[RPL];
            kb_lds8(buf + C::OFF_K + (i * DK + 8 * sub) * 4, kk);
            kb_lds8(buf + C::OFF_A + (i * DK + 8 * sub) * 4, aa);
            lds_v(buf, C::OFF_V, i, vv);
            kb_fwd_token<LPR, RPL>(s, kk, aa, vv, reinterpret_cast<const float *>(buf + C::OFF_B)[i]);
        }
        if (more) kb_store<DT, DK, RPL, NTH_>(st, smem + ((j + 1) & 1) * C::BUF);
        lds_barrier();
    }
    // the checkpoint stores complete before phase 2 reads them back
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // ---- phase 2: blocks last to first, each in RPL sub-blocks of HB tokens
    // (the registers hold HB x RPL pre-token states)
    float D[RPL][8];
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
#pragma unroll
        for (int e = 0; e < 8; ++e) D[u][e] = 0.f;
        if (dS_T && live[u]) load8(dS_T + srow(u), D[u]);
    }
    if (nblk > 0) {
        const int t0 = (nblk - 1) * TB;
        kb_load<DT, DK, RPL, NTH_>(st, q, k, v, beta, gk, dout, sr, t0, len - t0, row0, Dv, true);
        kb_store<DT, DK, RPL, NTH_>(st, smem + ((nblk - 1) & 1) * C::BUF);
    }
    lds_barrier();
    for (int j = nblk - 1; j >= 0; --j) {
        const int t0 = j * TB, nt = min(TB, len - t0);
        // the block's state first, so that waiting for it does not wait for
        // the next block's loads
        float c0[RPL][8];
#pragma unroll
        for (int u = 0; u < RPL; ++u) load8(ck_at(j, u), c0[u]);
        if (j > 0)
            kb_load<DT, DK, RPL, NTH_>(st, q, k, v, beta, gk, dout, sr, t0 - TB, TB, row0, Dv, true);
        const char *buf = smem + (j & 1) * C::BUF;
#pragma unroll 1
        for (int hb = RPL - 1; hb >= 0; --hb) {
            const int i0 = hb * HB;   // first token of the sub-block
            if (i0 >= nt) continue;   // uniform; an even number of flush groups skipped
#pragma unroll
            for (int u = 0; u < RPL; ++u)
#pragma unroll
                for (int e = 0; e < 8; ++e) s[u][e] = c0[u][e];
            // a later sub-block starts from the state after the earlier ones
            for (int i = 0; i < i0 && i < nt; ++i) {
                float kk[8], aa[8], vv[RPL];
                kb_lds8(buf + C::OFF_K + (i * DK + 8 * sub) * 4, kk);
                kb_lds8(buf + C::OFF_A + (i * DK + 8 * sub) * 4, aa);
                lds_v(buf, C::OFF_V, i, vv);
                kb_fwd_token<LPR, RPL>(s, kk, aa, vv, reinterpret_cast<const float *>(buf + C::OFF_B)[i]);
            }
            // recompute: sp[i] = P of token i0 + i, the decayed state before
            // its write (read below only for tokens of the sequence)
            float sp[HB][RPL][8];
#pragma unroll
            for (int i = 0; i < HB; ++i) {
                if constexpr (RPL > 1) {
                    // defined on every path: with two rows per lane the
                    // partly defined states cost the allocator spills
#pragma unroll
                    for (int u = 0; u < RPL; ++u)
#pragma unroll
                        for (int e = 0; e < 8; ++e) sp[i][u][e] = 0.f;
                }
                if (i0 + i < nt) {
                    float kk[8], aa[8], vv[RPL];
                    kb_lds8(buf + C::OFF_K + ((i0 + i) * DK + 8 * sub) * 4, kk);
                    kb_lds8(buf + C::OFF_A + ((i0 + i) * DK + 8 * sub) * 4, aa);
                    lds_v(buf, C::OFF_V, i0 + i, vv);
                    const float bb = reinterpret_cast<const float *>(buf + C::OFF_B)[i0 + i];
#pragma unroll
                    for (int u = 0; u < RPL; ++u) {
                        float pk = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            s[u][e] *= aa[e];
                            sp[i][u][e] = s[u][e];
                            pk += s[u][e] * kk[e];
                        }
                        const float bu = bb * (vv[u] - group_sum<LPR>(pk));
#pragma unroll
                        for (int e = 0; e < 8; ++e) s[u][e] += bu * kk[e];
                    }
                }
            }
            // reverse
#pragma unroll
            for (int i = HB - 1; i >= 0; --i) {
                const int ti = i0 + i;
                const int par = (i / G) & 1;   // HB is a multiple of 2 G
                if (ti < nt) {
                    float kk[8], qq[8], aa[8], vv[RPL], sd[RPL];
                    kb_lds8(buf + C::OFF_K + (ti * DK + 8 * sub) * 4, kk);
                    kb_lds8(buf + C::OFF_Q + (ti * DK + 8 * sub) * 4, qq);
                    kb_lds8(buf + C::OFF_A + (ti * DK + 8 * sub) * 4, aa);
                    lds_v(buf, C::OFF_V, ti, vv);
                    lds_v(buf, C::OFF_D, ti, sd);
                    const float bb = reinterpret_cast<const float *>(buf + C::OFF_B)[ti];
                    // the lane's rows' terms, added over its rows in the lane
                    float xq[8], xk[8], xg[8], xb = 0.f;
#pragma unroll
                    for (int e = 0; e < 8; ++e) xq[e] = xk[e] = xg[e] = 0.f;
#pragma unroll
                    for (int u = 0; u < RPL; ++u) {
                        const float(&P)[8] = sp[i][u];
                        float pk = 0.f;
                        const float sdu = scale * sd[u];
#pragma unroll
                        for (int e = 0; e < 8; ++e) pk += P[e] * kk[e];
                        const float err = vv[u] - group_sum<LPR>(pk);   // e_t for this row
                        const float bu = bb * err;
                        float wk = 0.f;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            xq[e] += (P[e] + bu * kk[e]) * sdu;       // S_t^T do (this row's term)
                            D[u][e] += sdu * qq[e];
                            wk += D[u][e] * kk[e];
                        }
                        const float w = group_sum<LPR>(wk);
                        if (live[u] && sub == 0)
                            dv[sr.row(t0 + ti) * Dv + row[u]] = from_f32<DT>(bb * w);
                        const float bw = bb * w;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            // (the two forms round alike; the second
                            // keeps fewer values live with two rows a lane)
                            if constexpr (RPL == 1)
                                xk[e] += D[u][e] * bu - P[e] * bw;
                            else
                                xk[e] += bb * (D[u][e] * err - P[e] * w);
                            D[u][e] -= bw * kk[e];
                            xg[e] += D[u][e] * P[e];
                            D[u][e] *= aa[e];
                        }
                        xb += err * w;
                    }
                    // this wave's rows summed: lane (DPP row r, column group sub)
                    // ends with values 6r .. 6r+5 of (xq, xk, xg) for its columns
                    float x24[24], z[6];
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        x24[e] = kb_dpp_rows_sum<LPR>(xq[e]);
                        x24[8 + e] = kb_dpp_rows_sum<LPR>(xk[e]);
                        x24[16 + e] = kb_dpp_rows_sum<LPR>(xg[e]);
                    }
                    kb_scatter24(x24, z);
                    xb = xor32_sum(xor16_sum(kb_dpp_rows_sum<LPR>(xb)));
                    float *rw = red + ((par * G + i % G) * C::NWV + wave) * C::NRED;
                    if ((lane & 15) < LPR) {
                        const int r4 = lane >> 4;
#pragma unroll
                        for (int e = 0; e < 6; ++e) {
                            const int x = 6 * r4 + e;   // quantity x / 8, column 8 sub + x % 8
                            rw[(x >> 3) * DK + 8 * sub + (x & 7)] = z[e];
                        }
                        if (lane == 0) rw[3 * DK] = xb;
                    }
                }
                if (i % G == 0) {
                    // tokens ti .. ti+G-1 of the block: the waves' sums added
                    // up and written as this row tile's partials
                    lds_barrier();
                    constexpr int NV1 = 3 * DK + 1;
                    for (int u = tid; u < G * NV1; u += C::NTH) {
                        const int tk = u / NV1, e = u % NV1;
                        if (ti + tk < nt) {
                            const float *rr = red + (par * G + tk) * C::NWV * C::NRED + e;
                            float acc = 0.f;
#pragma unroll
                            for (int wv = 0; wv < C::NWV; ++wv) acc += rr[wv * C::NRED];
                            const int64_t grow = sr.row(t0 + ti + tk);
                            if (e < 3 * DK)
                                part[((int64_t)((e / DK) * R + tile) * rows_total + grow) * DK +
                                     e % DK] = acc;
                            else
                                partb[(int64_t)tile * rows_total + grow] = acc;
                        }
                    }
                }
            }
        }
        if (j > 0) kb_store<DT, DK, RPL, NTH_>(st, smem + ((j - 1) & 1) * C::BUF);
        lds_barrier();
    }
#pragma unroll
    for (int u = 0; u < RPL; ++u) {
        if (dS0 && live[u]) {
            float4 *dst = reinterpret_cast<float4 *>(dS0 + srow(u));
            dst[0] = make_float4(D[u][0], D[u][1], D[u][2], D[u][3]);
            dst[1] = make_float4(D[u][4], D[u][5], D[u][6], D[u][7]);
        }
    }
}

// dq, dk, dgk, dbeta of every covered token: the row tiles' partials added
// (tile order fixed, so results do not depend on scheduling) and converted.
// Grid: (sequence, split); split s takes tokens s, s + nsplit, ... of the
// sequence.
template <typename DT, int DK>
__global__ __launch_bounds__(256) void kda_bwd_reduce_kernel(
    const float *__restrict__ part, const float *__restrict__ partb, DT *__restrict__ dq,
    DT *__restrict__ dk, float *__restrict__ dgk, DT *__restrict__ dbeta,
    const int *__restrict__ cu, int T, int H, int R, int64_t rows_total, int nsplit) {
    const int64_t n = blockIdx.x / nsplit;
    const int sp = blockIdx.x % nsplit;
    int lo = 0, hi = T;
    int64_t batch = n;
    if (cu) {
        lo = min(max(cu[n], 0), T);
        hi = min(max(cu[n + 1], lo), T);
        batch = 0;
    }
    const int64_t base = batch * T + lo;
    const int len = hi - lo;
    const int nvec = H * (DK / 4);
    for (int t = sp; t < len; t += nsplit) {
        const int64_t r0 = (base + t) * H;
        for (int u = threadIdx.x; u < nvec; u += 256) {
            const int64_t grow = r0 + u / (DK / 4);
            const int c = 4 * (u % (DK / 4));
#pragma unroll
            for (int qty = 0; qty < 3; ++qty) {
                float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
                for (int tl = 0; tl < R; ++tl) {
                    const float4 x = *reinterpret_cast<const float4 *>(
                        part + ((int64_t)(qty * R + tl) * rows_total + grow) * DK + c);
                    acc.x += x.x; acc.y += x.y; acc.z += x.z; acc.w += x.w;
                }
                if (qty == 2) {
                    *reinterpret_cast<float4 *>(dgk + grow * DK + c) = acc;
                } else {
                    DT *dst = (qty == 0 ? dq : dk) + grow * DK + c;
                    dst[0] = from_f32<DT>(acc.x);
                    dst[1] = from_f32<DT>(acc.y);
                    dst[2] = from_f32<DT>(acc.z);
                    dst[3] = from_f32<DT>(acc.w);
                }
            }
        }
        for (int u = threadIdx.x; u < H; u += 256) {
            float acc = 0.f;
            for (int tl = 0; tl < R; ++tl) acc += partb[(int64_t)tl * rows_total + r0 + u];
            dbeta[r0 + u] = from_f32<DT>(acc);
        }
    }
}

// Workgroup shape from d_k = 64: two state rows per lane when one would need
// more workgroups than the GPU has CUs (the layer shape: one round instead
// of two, and half the cross-row sums per row); half the lanes (256) when
// even that would leave half the CUs idle (few heads: twice the workgroups,
// half the issue per SIMD); else one row per lane on 512 lanes.
constexpr int64_t KB_CUS = 256;

struct KbShape {
    int rpl, nth;
};

template <int DK>
KbShape kb_shape(int64_t nseq, int64_t H, int Dv) {
    constexpr int full = KbLanes<DK>::value;
    if constexpr (DK < 64) {
        return {1, full};
    } else {
        const int rl = KbCfg<float, DK, 1, full>::RL;
        const int64_t wg = nseq * H * ((Dv + rl - 1) / rl);
        if (wg > KB_CUS) return {2, full};
        if (2 * wg <= KB_CUS) return {1, full / 2};
        return {1, full};
    }
}

struct KbLayout {
    KbShape shape;
    int R;               // row tiles per (sequence, head)
    int64_t ckpt, part, partb, total;  // float offsets: checkpoints, partials; total bytes
};

template <int DK>
KbLayout kb_layout_dk(int64_t ntok, int64_t nseq, int64_t H, int Dv) {
    KbLayout l{{0, 0}, 0, 0, 0, 0, -1};
    if (ntok < 0 || nseq < 0 || H < 0) return l;
    l.shape = kb_shape<DK>(nseq, H, Dv);
    const int rw = l.shape.nth / (DK / 8) * l.shape.rpl;
    l.R = (Dv + rw - 1) / rw;
    const auto al = [](int64_t x) { return (x + 63) / 64 * 64; };  // 256-byte parts
    const int64_t nck = (ntok / KbCfg<float, DK>::TB + nseq) * H * l.R * rw * DK;
    const int64_t npart = 3 * (int64_t)l.R * ntok * H * DK;
    const int64_t npb = (int64_t)l.R * ntok * H;
    l.part = al(nck);
    l.partb = l.part + al(npart);
    l.total = (l.partb + al(npb)) * 4;
    return l;
}

KbLayout kb_layout(int64_t ntok, int64_t nseq, int64_t H, int Dk, int Dv) {
    switch (Dk) {
    case 16: return kb_layout_dk<16>(ntok, nseq, H, Dv);
    case 32: return kb_layout_dk<32>(ntok, nseq, H, Dv);
    case 64: return kb_layout_dk<64>(ntok, nseq, H, Dv);
    case 128: return kb_layout_dk<128>(ntok, nseq, H, Dv);
    default: return KbLayout{{0, 0}, 0, 0, 0, 0, -1};
    }
}

template <typename DT, int DK, int RPL, int NTH>
hipError_t launch_kb(const KdaBwdArgs &a, const KbLayout &l, hipStream_t stream) {
    float *ws = static_cast<float *>(a.ws);
    const int64_t ntok = a.cu ? a.T : a.nseq * a.T;
    const int64_t rows_total = ntok * a.H;
    const int64_t grid = a.nseq * a.H * l.R;
    if (grid > 0) {
        hipLaunchKernelGGL((kda_bwd_kernel<DT, DK, RPL, NTH>), dim3((unsigned)grid),
                           dim3(NTH), 0, stream, static_cast<const DT *>(a.q),
                           static_cast<const DT *>(a.k), static_cast<const DT *>(a.v),
                           static_cast<const DT *>(a.beta), a.gk, a.S0,
                           static_cast<const DT *>(a.dout), a.dS_T, static_cast<DT *>(a.dv),
                           a.dS0, ws + l.ckpt, ws + l.part, ws + l.partb, a.cu, (int)a.T,
                           (int)a.H, a.Dv, l.R, rows_total, a.scale);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // enough reduce workgroups to fill the GPU whatever the number of sequences
    const int64_t nsplit = std::max<int64_t>(1, std::min<int64_t>(std::max<int64_t>(a.T, 1),
                                                                  (2048 + a.nseq - 1) / std::max<int64_t>(a.nseq, 1)));
    const int64_t rgrid = a.nseq * nsplit;
    if (rgrid > 0 && a.T > 0) {
        hipLaunchKernelGGL((kda_bwd_reduce_kernel<DT, DK>), dim3((unsigned)rgrid), dim3(256), 0,
                           stream, ws + l.part, ws + l.partb, static_cast<DT *>(a.dq),
                           static_cast<DT *>(a.dk), a.dgk, static_cast<DT *>(a.dbeta), a.cu,
                           (int)a.T, (int)a.H, l.R, rows_total, (int)nsplit);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename DT, int DK>
hipError_t launch_kb_shape(const KdaBwdArgs &a, const KbLayout &l, hipStream_t stream) {
    constexpr int full = KbLanes<DK>::value;
    if constexpr (DK >= 64) {
        if (l.shape.rpl == 2) return launch_kb<DT, DK, 2, full>(a, l, stream);
        if (l.shape.nth == full / 2) return launch_kb<DT, DK, 1, full / 2>(a, l, stream);
    }
    return launch_kb<DT, DK, 1, full>(a, l, stream);
}

template <typename DT>
hipError_t kb_dk(const KdaBwdArgs &a, const KbLayout &l, hipStream_t stream) {
    switch (a.Dk) {
    case 16: return launch_kb_shape<DT, 16>(a, l, stream);
    case 32: return launch_kb_shape<DT, 32>(a, l, stream);
    case 64: return launch_kb_shape<DT, 64>(a, l, stream);
    case 128: return launch_kb_shape<DT, 128>(a, l, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t kda_bwd_workspace_bytes(int64_t ntok, int64_t nseq, int64_t H, int Dk, int Dv) {
    return kb_layout(ntok, nseq, H, Dk, Dv).total;
}

hipError_t launch_kda_bwd(const KdaBwdArgs &a, bool bf16, hipStream_t stream) {
    if (a.nseq == 0 || a.H == 0) return hipSuccess;
    const int64_t ntok = a.cu ? a.T : a.nseq * a.T;
    const KbLayout l = kb_layout(ntok, a.nseq, a.H, a.Dk, a.Dv);
    if (l.total < 0) return hipErrorInvalidValue;
    return bf16 ? kb_dk<__bf16>(a, l, stream) : kb_dk<float>(a, l, stream);
}

}  // namespace dr
