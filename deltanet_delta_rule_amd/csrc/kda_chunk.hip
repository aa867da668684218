// Chunked forward of Kimi Delta Attention (per-key-channel decay), bf16
// inputs, d_k = 128, chunks of 32 tokens (gfx950).
//
// hada.io digest, sections "Chunkwise KDA" and "Pipeline Triton Chunkwise".
// With b_t the in-chunk prefix sums of the log decays gk (a vector over the
// key channels), Gamma_t = exp(b_t) and chunk c entered with state S_c:
//   G_ij = k_i^T diag(exp(b_i - b_j)) k_j        (j < i; decayed couplings)
//   P_ij = q_i^T diag(exp(b_i - b_j)) k_j        (j <= i; read weights)
//   E    = (I + diag(beta) G)^{-1} diag(beta) (V - (K . Gamma) S_c^T)
//   O    = (Q . Gamma) S_c^T + P E
//   S_{c+1} = S_c diag(Gamma_last) + E^T (K . exp(b_last - b))
// which is the recurrence token by token (decay, predict, correct, write,
// read).  The same block substitution as the scalar-decay kernels resolves E:
// the diagonal 16-token blocks of (I + diag(beta) G) are inverted on the
// matrix cores, the block below them is a product.
//
// The decay ratio exp(b_i - b_j) lives inside the contraction over key
// channels, so it cannot be applied to a finished Gram tile, and a split into
// a row factor and a column factor around one reference token per block
// overflows on one side once a channel decays hard inside the block (an
// erased channel, gk -> -inf, is the case the digest's KDA section motivates).
// The pairs (i, j), j < i, of a 32-token chunk are therefore taken by levels:
// pair (i, j) belongs to level L = the highest bit in which i and j differ, so
// they sit in the two halves of one aligned segment of 2L tokens, and its
// reference is the last token of that segment's first half.  Row token i
// then carries exp(b_i - b_ref) (the decay over ref+1 .. i) and column token
// j carries exp(b_ref - b_j) (the decay over j+1 .. ref): both are products
// of per-token factors exp(gk) <= 1, so nothing overflows and the product of
// the two is exp(b_i - b_j) exactly up to rounding, for every gk <= 0.  Each
// level is one product over the channels (levels 8, 4, 2, 1 inside the
// 16-token diagonal blocks, masked to their own pairs; level 16 is the
// off-diagonal block), and the read weight of a token's own write is q_i . k_i.
// The state operands k Gamma, q Gamma and k exp(b_last - b) are products of
// the same factors and stay <= 1 as well.
//
// Work split: see kda_pipe_kernel.
#include "chunk_fwd.hpp"

#include <type_traits>

namespace dr {

namespace {

constexpr int KDA_DK = 128;      // key channels
constexpr int KDA_DVW = 64;      // value rows per workgroup
constexpr int KDA_LD = 136;      // row pitch (bf16) of the token x channel tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr int KDA_LV = 5;        // levels 16, 8, 4, 2, 1 of the pairs of a 32-token chunk

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ unsigned pk2(float a, float b) { return pk_bf16(a, b); }

__device__ __forceinline__ float2 fmul2(float2 a, float2 b) { return make_float2(a.x * b.x, a.y * b.y); }

// Factor of token s (0..7) of an 8-token quarter at level L <= 4 (its
// 2L-segment lies inside the quarter): the product of exp(gk) over ref+1 .. s
// for a row token (second half), over s+1 .. ref for a column token, ref the
// last token of the segment's first half.  s and L are constants after
// unrolling, so this folds to a few multiplies.
__device__ __forceinline__ float2 lvl_factor(const float2 (&e)[8], int s, int L) {
    const int ref = (s & ~(2 * L - 1)) + L - 1;
    float2 f = make_float2(1.f, 1.f);
#pragma unroll
    for (int u = 0; u < 8; ++u)
        if (s > ref ? (u > ref && u <= s) : (u > s && u <= ref)) f = fmul2(f, e[u]);
    return f;
}

// Eight sums over the 64 lanes at once: lane l receives the sum of v[l >> 3]
// (lanes 8s .. 8s + 7 hold token s's).  Each exchange step halves the values
// a lane keeps -- lane xor 32 (the wave halves swap by permlane32), xor 16
// (rows by permlane16), xor 8 (a DPP rotation by 8 within each row) -- and
// sums the half it keeps with its partner's copy of it; three DPP steps then
// sum the 8-lane groups.  Ten exchanges in a dependent chain six deep, where
// eight separate sums take 48 in eight chains of six.
__device__ __forceinline__ float batch_sum8(const float (&v)[8], int lane) {
    float u[4], w[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // lower half keeps token i, upper half token 4 + i
        const auto x = __builtin_amdgcn_permlane32_swap(__float_as_uint(v[i]),
                                                        __float_as_uint(v[4 + i]), false, false);
        u[i] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        // row r (16 lanes) keeps token 2 r + i
        const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(u[i]),
                                                        __float_as_uint(u[2 + i]), false, false);
        w[i] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
    }
    // lanes 0-7 of a row keep token 2 r, lanes 8-15 token 2 r + 1
    const bool upper = lane & 8;
    const float send = upper ? w[0] : w[1];
    const float keep = upper ? w[1] : w[0];
    return group_sum<8>(keep + dpp_move<0x128>(send));  // row_ror:8
}

__device__ __forceinline__ float lo_bf16(unsigned x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_bf16(unsigned x) { return __uint_as_float(x & 0xffff0000u); }

// Prefetched inputs of one chunk for one thread.
struct KdaRegs {
    unsigned k[8], q[8];     // bf16 pairs: channels 2p, 2p + 1 of token 8w + s
    u32x2 g[8];              // their log decays (fp32 pairs)
    unsigned short beta;
};

struct KdaSeq {
    const __bf16 *q, *k, *v, *beta;
    const float *gk;
    __bf16 *o;
    int64_t base;  // first token of the sequence in the flattened (batch, time) axis
    int H, h, Dv, vcol0, len;
    __device__ __forceinline__ int64_t row(int t) const { return (base + t) * H + h; }
};

// ---------------------------------------------------------------------------
// Work split.  One workgroup of eight waves owns one (sequence, head) and a
// slice of 64 value rows of S (wave 4 + i: rows 16i .. 16i + 15, fp32 in
// registers in the canonical k order of the matrix-core operands), walks the
// 32-token chunks in order, and is pipelined: waves 0-3 (preparation) build the
// operands and the G / P blocks of chunk c + 1 while waves 4-7 (state) run
// the state path of chunk c on 16 value rows each, so the exponentials and
// LDS writes of one overlap the matrix-core work of the other.  What the
// state waves read (K.Gamma, Q.Gamma, KE, the blocks, Gamma_last) is double
// buffered by chunk parity; at 32 tokens everything fits in LDS.  Each step
// has three segments separated by workgroup barriers:
//   1. preparation: per-token factors exp(gk) of its 8 tokens, their
//      products and the level operands inside its quarter and block;
//      state: X and (Q.Gamma) S^T
//   2. preparation: the operands that need the other quarters' products;
//      state: block substitution, P E, outputs
//   3. preparation: G and P blocks level by level, inverses;  state: state
//      update
// Step -1 prepares chunk 0 only; the last step only runs the state path.
// ---------------------------------------------------------------------------
constexpr int KP_C = 32;

struct alignas(16) KdaPipeBuf {
    __bf16 KT[KP_C * KDA_LD];        // k_t Gamma_t
    __bf16 QT[KP_C * KDA_LD];        // q_t Gamma_t
    __bf16 KE[KP_C * KDA_LD];        // k_t exp(b_last - b_t)
    __bf16 Gb[1 * FRAG_ELEMS];       // G_10
    __bf16 Gd[2 * FRAG_ELEMS];       // diag(beta_I) G_II (strictly lower)
    __bf16 Tb[2 * FRAG_ELEMS];       // -T_II diag(beta_I)
    __bf16 Pb[3 * FRAG_ELEMS];       // P_00, P_10, P_11
    float gamC[KDA_DK];              // Gamma_last
};

// Level lv (L = 16 >> lv): W holds k_t times its factor at that level (the
// row factor exp(b_t - b_ref) for a token in the second half of its
// 2L-segment, the column factor exp(b_ref - b_t) otherwise); QR holds q_t
// times the row factor (second-half tokens only; the other rows are never
// selected).
struct alignas(16) KdaPipeSmem {
    __bf16 W[KDA_LV][KP_C * KDA_LD];
    __bf16 QR[KDA_LV][KP_C * KDA_LD];
    KdaPipeBuf buf[2];
    float beta[KP_C];
    float pdiag[KP_C];               // q_t . k_t: read weight of the token's own write
    float hq[4][KDA_DK];             // decay over each 8-token quarter (product of exp(gk))
};
// Level lv operands of one token (offset o_t, channels 2p, 2p + 1): k times
// the factor, and q times it for a row token.
__device__ __forceinline__ void put_level(KdaPipeSmem &sm, int lv, int o_t, float2 kk,
                                          float2 qq, float2 f, bool row) {
    *reinterpret_cast<unsigned *>(sm.W[lv] + o_t) = pk2(kk.x * f.x, kk.y * f.y);
    if (row) *reinterpret_cast<unsigned *>(sm.QR[lv] + o_t) = pk2(qq.x * f.x, qq.y * f.y);
}

// Raw k, q, gk of tokens 8w .. 8w + 7 and beta of token tid (< 32) of the
// 32-token chunk at t0, zeros past the sequence's end.
__device__ __forceinline__ void kp_prefetch(KdaRegs &x, const KdaSeq &sq, int t0, int w, int p,
                                            int tid) {
    const int nv = min(KP_C, sq.len - t0);
    const int64_t r0 = sq.row(t0);
    const int sk = sq.H * KDA_DK * 2, sg = sq.H * KDA_DK * 4;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(sq.k + r0 * KDA_DK, nv * sk);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(sq.q + r0 * KDA_DK, nv * sk);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(sq.gk + r0 * KDA_DK, nv * sg);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(sq.beta + r0, nv * sq.H * 2);
    const int ws = __builtin_amdgcn_readfirstlane(w);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        const int tk = 8 * ws + s;
        x.k[s] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * p, tk * sk, 0);
        x.q[s] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * p, tk * sk, 0);
        x.g[s] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * p, tk * sg, 0));
    }
    x.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, min(tid, KP_C - 1) * sq.H * 2, 0, 0);
}

// v[t0 + 16 I + 4 g + e][vcol] for I < 2, e < 4 (the D layout of X); v ==
// nullptr loads zeros.  With 32-bit elements each value keeps a register of
// its own: packing two 16-bit loads into one register right after they are
// issued waits for every load in flight (16-bit elements save the registers
// where the kernel has none to spare).
template <typename VT>
__device__ __forceinline__ void kp_prefetch_v(VT (&vr)[8], const KdaSeq &sq, int t0,
                                              int g, int vcol) {
    const int nv = min(KP_C, sq.len - t0);
    const int sv = sq.H * sq.Dv * 2;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(sq.v + sq.row(t0) * sq.Dv, sq.v ? nv * sv : 0);
#pragma unroll
    for (int I = 0; I < 2; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vr[4 * I + e] = __builtin_amdgcn_raw_buffer_load_b16(
                rv, (4 * g) * sv + 2 * vcol, (16 * I + e) * sv, 0);
}

// L2: q and k rows are divided by sqrt(|x|^2 + 1e-6) first (the l2norm of the
// gated layer on houmin.site "infra/delta-net"); a preparation lane holds two
// channels of each of its tokens, so a token's norm is one wave-wide sum.
template <bool L2>
__global__ __launch_bounds__(512) void kda_pipe_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const __bf16 *__restrict__ beta, const float *__restrict__ gk, const float *S0,
    __bf16 *__restrict__ o, float *S_T, const int *__restrict__ cu, int T, int H, int Dv,
    float scale) {
    __shared__ KdaPipeSmem sm;
    int wg = blockIdx.x;
    const int nwg = gridDim.x;
    if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;  // value slices of a head on one XCD
    const int nvb = Dv / KDA_DVW;
    const int vb = wg % nvb;
    const int64_t seqhead = wg / nvb;
    const int64_t n = seqhead / H;
    const int h = (int)(seqhead % H);
    int lo = 0, hi = T;
    int64_t batch = n;
    if (cu) {
        lo = min(max(cu[n], 0), T);
        hi = min(max(cu[n + 1], lo), T);
        batch = 0;
    }
    const KdaSeq sq{q, k, v, beta, gk, o, batch * T + lo, H, h, Dv, vb * KDA_DVW, hi - lo};

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, r = lane & 15;
    const int p = lane;                       // channel pair of the operand step
    const bool prep = wave < 4;
    const int vt = wave & 3;                  // value tile of a state wave
    const int vcol = vb * KDA_DVW + 16 * vt + r;
    const int64_t srow = (seqhead * Dv + vcol) * KDA_DK;
    const int J = (wave & 3) >> 1, hf = wave & 1;  // token block and half (preparation)

    f32x4 S[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            S[s][hh] = zero4();
            if (S0 && !prep) {
                const float4 x = *reinterpret_cast<const float4 *>(S0 + srow + 32 * s + 16 * hh + 4 * g);
                S[s][hh] = f32x4{x.x, x.y, x.z, x.w};
            }
        }
    // The chunk loop must not see these loads as pending (it would wait for
    // every memory operation in flight at their first use, in every chunk).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    const int nchunk = (sq.len + KP_C - 1) / KP_C;
    KdaRegs x;
    typename std::conditional<L2, unsigned short, unsigned>::type vr[8];
    if (nchunk > 0) {
        if (prep) kp_prefetch(x, sq, 0, wave, p, tid);
        else kp_prefetch_v(vr, sq, 0, g, vcol);
    }

    // G_10 (G) or P_10 of a chunk from its level-16 operands into buffer b
    auto level16 = [&](bool G, KdaPipeBuf &b) {
        const __bf16 *rows = G ? sm.W[0] : sm.QR[0];
        f32x4 a16 = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 fc, fr;
            frag_rows(sm.W[0], KDA_LD, 0, 32 * s, lane, fc);
            frag_rows(rows, KDA_LD, 16, 32 * s, lane, fr);
            mma_k32(a16, fc, fr);
        }
        if (G) store_fragblk(b.Gb, 0, lane, a16);
        else store_fragblk(b.Pb, 1, lane, a16);
    };
    for (int it = -1; it < nchunk; ++it) {
        const bool pw = prep && it + 1 < nchunk;   // prepare chunk it + 1
        const bool sw = !prep && it >= 0;          // state path of chunk it
        const int tp = (it + 1) * KP_C, ts = it * KP_C;
        KdaPipeBuf &bp = sm.buf[(it + 1) & 1];
        KdaPipeBuf &bs = sm.buf[it & 1];

        // ---- segment 1
        float2 F[8], Bk[8];    // products of exp(gk) over tokens 0..s and s+1..7 of the quarter
        float nk[8], nq[8];    // inverse norms of k_t and q_t (1 without L2)
        bf16x8 fS[4];
        f32x4 Xs[2], O[2];
        if (pw) {
            float2 e[8];       // exp(gk) of the two channels
#pragma unroll
            for (int s = 0; s < 8; ++s)
                e[s] = make_float2(exp2_(__uint_as_float(x.g[s][0]) * LOG2E),
                                   exp2_(__uint_as_float(x.g[s][1]) * LOG2E));
            F[0] = e[0];
#pragma unroll
            for (int s = 1; s < 8; ++s) F[s] = fmul2(F[s - 1], e[s]);
            Bk[7] = make_float2(1.f, 1.f);
#pragma unroll
            for (int s = 6; s >= 0; --s) Bk[s] = fmul2(Bk[s + 1], e[s + 1]);
            *reinterpret_cast<float2 *>(&sm.hq[wave][2 * p]) = F[7];
            // q_t . k_t (and with L2 |k_t|^2, |q_t|^2) of the quarter's 8
            // tokens, each summed over the 64 lanes' channel pairs at once
            float qk[8];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                qk[s] = lo_bf16(x.q[s]) * lo_bf16(x.k[s]) + hi_bf16(x.q[s]) * hi_bf16(x.k[s]);
                nk[s] = nq[s] = 1.f;
            }
            float pd = batch_sum8(qk, lane);  // token lane >> 3
            if constexpr (L2) {
                float kk[8], qq[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    const float k0 = lo_bf16(x.k[s]), k1 = hi_bf16(x.k[s]);
                    const float q0 = lo_bf16(x.q[s]), q1 = hi_bf16(x.q[s]);
                    kk[s] = k0 * k0 + k1 * k1;
                    qq[s] = q0 * q0 + q1 * q1;
                }
                const float tk = batch_sum8(kk, lane), tq = batch_sum8(qq, lane);
#pragma unroll
                for (int s = 0; s < 8; ++s) {
                    nk[s] = rsqrtf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(tk), 8 * s)) + 1e-6f);
                    nq[s] = rsqrtf(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(tq), 8 * s)) + 1e-6f);
                }
                pd *= rsqrtf(tk + 1e-6f) * rsqrtf(tq + 1e-6f);
            }
            if ((lane & 7) == 0) sm.pdiag[8 * wave + (lane >> 3)] = pd;
            // levels 8, 4, 2, 1 lie inside the quarter's 16-token block;
            // level 16 here for the quarters on either side of the block
            // boundary (1: columns, 2: rows), the others need a neighbour's
            // product (segment 2)
            const int col = 2 * p;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int o_t = (8 * wave + s) * KDA_LD + col;
                const float2 kk = make_float2(lo_bf16(x.k[s]) * nk[s], hi_bf16(x.k[s]) * nk[s]);
                const float2 qq = make_float2(lo_bf16(x.q[s]) * nq[s], hi_bf16(x.q[s]) * nq[s]);
                put_level(sm, 1, o_t, kk, qq, hf ? F[s] : Bk[s], hf);
                put_level(sm, 2, o_t, kk, qq, lvl_factor(e, s, 4), s & 4);
                put_level(sm, 3, o_t, kk, qq, lvl_factor(e, s, 2), s & 2);
                put_level(sm, 4, o_t, kk, qq, lvl_factor(e, s, 1), s & 1);
                if (wave == 1 || wave == 2) put_level(sm, 0, o_t, kk, qq, hf ? Bk[s] : F[s], J);
            }
        }
        if (sw) {
            // waves 4, 5: the inverse of diagonal block vt of this chunk (its
            // G block was formed by the preparation waves one step earlier)
            if (vt < 2) {
                bf16x4 fg;
                load_fragblk(bs.Gd, vt, lane, fg);
                f32x4 a;
#pragma unroll
                for (int e = 0; e < 4; ++e) a[e] = (float)fg[e];
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sm.beta + 16 * vt + 4 * g);
                diag_inverse(a, b4, bs.Tb, vt, lane);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) cvt8(S[s][0], S[s][1], fS[s]);
#pragma unroll
            for (int I = 0; I < 2; ++I) Xs[I] = O[I] = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int I = 0; I < 2; ++I) {
                    bf16x8 fk, fq;
                    frag_rows(bs.KT, KDA_LD, 16 * I, 32 * s, lane, fk);
                    frag_rows(bs.QT, KDA_LD, 16 * I, 32 * s, lane, fq);
                    mma_k32(Xs[I], fk, fS[s]);
                    mma_k32(O[I], fS[s], fq);  // O transposed (see the stores)
                }
        }
        lds_barrier();

        // ---- segment 2
        bf16x4 fE[2];
        if (pw) {
            float2 Hq[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) Hq[w] = *reinterpret_cast<const float2 *>(&sm.hq[w][2 * p]);
            // decay over the quarters before and after this one
            float2 pre = wave > 0 ? Hq[0] : make_float2(1.f, 1.f);
            pre = wave > 1 ? fmul2(pre, Hq[1]) : pre;
            pre = wave > 2 ? fmul2(pre, Hq[2]) : pre;
            float2 post = wave < 3 ? Hq[3] : make_float2(1.f, 1.f);
            post = wave < 2 ? fmul2(Hq[2], post) : post;
            post = wave < 1 ? fmul2(Hq[1], post) : post;
            if (wave == 0)
                *reinterpret_cast<float2 *>(&bp.gamC[2 * p]) =
                    fmul2(fmul2(Hq[0], Hq[1]), fmul2(Hq[2], Hq[3]));
            const float2 h16 = wave == 0 ? Hq[1] : Hq[2];  // level 16 across the neighbour
            const int col = 2 * p;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int o_t = (8 * wave + s) * KDA_LD + col;
                const float2 kk = make_float2(lo_bf16(x.k[s]) * nk[s], hi_bf16(x.k[s]) * nk[s]);
                const float2 qq = make_float2(lo_bf16(x.q[s]) * nq[s], hi_bf16(x.q[s]) * nq[s]);
                const float2 gm = fmul2(pre, F[s]);     // Gamma_t
                const float2 ke = fmul2(Bk[s], post);   // exp(b_last - b_t)
                *reinterpret_cast<unsigned *>(bp.KT + o_t) = pk2(kk.x * gm.x, kk.y * gm.y);
                *reinterpret_cast<unsigned *>(bp.QT + o_t) = pk2(qq.x * gm.x, qq.y * gm.y);
                *reinterpret_cast<unsigned *>(bp.KE + o_t) = pk2(kk.x * ke.x, kk.y * ke.y);
                if (wave == 0 || wave == 3)
                    put_level(sm, 0, o_t, kk, qq, fmul2(hf ? F[s] : Bk[s], h16), J);
            }
            if (tid < KP_C) sm.beta[tid] = (float)__builtin_bit_cast(__bf16, x.beta);
            if (it + 2 < nchunk) kp_prefetch(x, sq, tp + KP_C, wave, p, tid);
        }
        if (sw) {
            f32x4 E[2];
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                f32x4 X = Xs[I];
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[e] -= (float)__builtin_bit_cast(__bf16, (unsigned short)vr[4 * I + e]);
                if (I == 1) {
                    bf16x4 fa;
                    load_fragblk(bs.Gb, 0, lane, fa);
                    mma_k16(X, fa, fE[0]);
                }
                bf16x4 ft, fy;
                load_fragblk(bs.Tb, I, lane, ft);
                frag_from_acc16(X, fy);
                E[I] = zero4();
                mma_k16(E[I], ft, fy);
                frag_from_acc16(E[I], fE[I]);
            }
            const int so = H * Dv * 2;
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(sq.o + sq.row(ts) * Dv, sq.o ? min(KP_C, sq.len - ts) * so : 0);
#pragma unroll
            for (int I = 0; I < 2; ++I) {
#pragma unroll
                for (int Jb = 0; Jb <= I; ++Jb) {
                    bf16x4 fa;
                    load_fragblk(bs.Pb, I * (I + 1) / 2 + Jb, lane, fa);
                    mma_k16(O[I], fE[Jb], fa);
                }
                // O is computed transposed (operands swapped): lane (g, r)
                // holds token 16 I + r, value columns vcol - r + 4g .. + 3,
                // written with one 8-byte store
                __builtin_amdgcn_raw_buffer_store_b64(pk4_bf16(scale * O[I]), ro,
                                                      (16 * I + r) * so + 2 * (vcol - r + 4 * g), 0, 0);
            }
            // after the output stores: the next chunk's wait for these loads
            // then covers no store issued just before it
            if (it + 1 < nchunk) kp_prefetch_v(vr, sq, ts + KP_C, g, vcol);
        }
        lds_barrier();

        // ---- segment 3
        if (pw) {
            // waves 0, 1: G of diagonal block I and its inverse; waves 2, 3:
            // P of diagonal block I, then the level-16 block of G (wave 2)
            // or P (wave 3).  Each level has its own accumulator; lane (g, r)
            // element e is pair (i, j) = (r, 4g + e) of the block, which
            // belongs to the level of the highest bit of i xor j.
            const int I = wave & 1;
            f32x4 acc[4];
#pragma unroll
            for (int l = 0; l < 4; ++l) acc[l] = zero4();
            if (wave < 2) {
#pragma unroll
                for (int l = 0; l < 4; ++l)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        bf16x8 f;
                        frag_rows(sm.W[l + 1], KDA_LD, 16 * I, 32 * s, lane, f);
                        mma_k32(acc[l], f, f);
                    }
            } else {
#pragma unroll
                for (int l = 0; l < 4; ++l)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        bf16x8 fc, fr;
                        frag_rows(sm.W[l + 1], KDA_LD, 16 * I, 32 * s, lane, fc);
                        frag_rows(sm.QR[l + 1], KDA_LD, 16 * I, 32 * s, lane, fr);
                        mma_k32(acc[l], fc, fr);
                    }
            }
            f32x4 m;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int j = 4 * g + e, d = r ^ j;
                const float lv = d >= 8 ? acc[0][e] : d >= 4 ? acc[1][e] : d >= 2 ? acc[2][e] : acc[3][e];
                m[e] = r > j ? lv : 0.f;
            }
            if (wave < 2) {
                // inverted by state waves 4, 5 in the next step's first segment
                store_fragblk(bp.Gd, I, lane, sm.beta[16 * I + r] * m);
            } else {
                const float pd = sm.pdiag[16 * I + r];
#pragma unroll
                for (int e = 0; e < 4; ++e) m[e] = r == 4 * g + e ? pd : m[e];
                store_fragblk(bp.Pb, 2 * I, lane, m);
                if (it < 0) level16(wave == 2, bp);  // chunk 0: no state path yet
            }
        }
        // the level-16 block of the next chunk's G (wave 6) and P (wave 7)
        if (!prep && it >= 0 && it + 1 < nchunk && vt >= 2) level16(vt == 2, bp);
        if (sw) {
            const bf16x8 fE32 = __builtin_shufflevector(fE[0], fE[1], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x4 d = zero4();
                    bf16x8 fa;
                    frag_cols32(bs.KE, KDA_LD, 0, 32 * s + 16 * hh, lane, fa);
                    mma_k32(d, fa, fE32);
                    const f32x4 gc = *reinterpret_cast<const f32x4 *>(bs.gamC + 32 * s + 16 * hh + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[s][hh][e] = S[s][hh][e] * gc[e] + d[e];
                }
        }
        lds_barrier();
    }
    if (S_T && !prep) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
                *reinterpret_cast<float4 *>(S_T + srow + 32 * s + 16 * hh + 4 * g) =
                    make_float4(S[s][hh][0], S[s][hh][1], S[s][hh][2], S[s][hh][3]);
    }
}

}  // namespace

bool kda_chunk_supported(const ChunkFwdArgs &a, bool bf16) {
    // one chunk of one head's rows of every input must be addressable with
    // 32-bit byte offsets
    const int64_t span = int64_t(KP_C) * a.H * (a.Dv > 2 * KDA_DK ? 2 * a.Dv : 4 * KDA_DK);
    return bf16 && a.gk && !a.g && !a.recurrent && a.Dk == KDA_DK &&
           a.Dv % KDA_DVW == 0 && span < INT32_MAX;
}

hipError_t launch_kda_chunk(const ChunkFwdArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    const int64_t grid = a.B * a.H * (a.Dv / KDA_DVW);
    auto kern = a.l2 ? kda_pipe_kernel<true> : kda_pipe_kernel<false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(512), 0, stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), static_cast<const __bf16 *>(a.beta),
                       a.gk, a.S0, static_cast<__bf16 *>(a.o), a.S_T, a.cu, (int)a.T, (int)a.H,
                       a.Dv, a.scale);
    return hipGetLastError();
}

}  // namespace dr
