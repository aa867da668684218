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
// channels, so it cannot be applied to a finished Gram tile.  It is split
// around a reference point m_I per 16-token row block I (the prefix sum at
// the block's 8th token): rows use k_i exp(b_i - m_I), columns k_j exp(m_I -
// b_j).  For j in an earlier block the column factor is at most 1; inside the
// block either factor grows by at most the decay of 8 tokens.  That bounds
// the domain: the log decay summed over any 8 consecutive tokens of a channel
// should stay above -40 (per-token gk >= -5 guarantees it); the growing
// exponents are clamped at 80 so that nothing overflows outside it.
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
constexpr float KDA_EXP2_MAX = 80.f * LOG2E;  // clamp of growing exponents (log2)

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Column operands of row block I start at row 8 I (I + 1) of KC: block I has
// the 16 (I + 1) tokens 0 .. 16 I + 15.
constexpr int kc_base(int I) { return 8 * I * (I + 1); }

// Block pair p = I (I + 1) / 2 + J of the pairs (I, J <= I).
__device__ __forceinline__ void pair_ij(int p, int &I, int &J) {
    I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    J = p - I * (I + 1) / 2;
}

__device__ __forceinline__ unsigned pk2(float a, float b) { return pk_bf16(a, b); }

// Sum over the 64 lanes of the wave, every lane receiving it.
__device__ __forceinline__ float wave_sum(float v) {
    v = group_sum<16>(v);
    v += __shfl_xor(v, 16, 64);
    v += __shfl_xor(v, 32, 64);
    return v;
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
//   1. preparation: prefix sums of its 8 tokens and the operands that need
//      only in-block differences;  state: X and (Q.Gamma) S^T
//   2. preparation: the operands that need the other waves' sums;  state:
//      block substitution, P E, outputs
//   3. preparation: G and P blocks, inverses;  state: state update
// Step -1 prepares chunk 0 only; the last step only runs the state path.
// ---------------------------------------------------------------------------
constexpr int KP_C = 32;

struct alignas(16) KdaPipeBuf {
    __bf16 KT[KP_C * KDA_LD];        // k_t Gamma_t
    __bf16 QT[KP_C * KDA_LD];        // q_t Gamma_t
    __bf16 KE[KP_C * KDA_LD];        // k_t exp(b_last - b_t)
    __bf16 Gb[1 * FRAG_ELEMS];       // G_10
    __bf16 Tb[2 * FRAG_ELEMS];       // -T_II diag(beta_I)
    __bf16 Pb[3 * FRAG_ELEMS];       // P_00, P_10, P_11
    float gamC[KDA_DK];              // Gamma_last
};

struct alignas(16) KdaPipeSmem {
    __bf16 KR[KP_C * KDA_LD];        // k_i exp(b_i - m_I)
    __bf16 QR[KP_C * KDA_LD];        // q_i exp(b_i - m_I)
    __bf16 KC[48 * KDA_LD];          // k_j exp(m_I - b_j): I = 0 rows 0..15, I = 1 rows 16..47
    KdaPipeBuf buf[2];
    float beta[KP_C];
    float htot[4][KDA_DK];           // sums of gk over each 8-token quarter (log2)
};

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

    for (int it = -1; it < nchunk; ++it) {
        const bool pw = prep && it + 1 < nchunk;   // prepare chunk it + 1
        const bool sw = !prep && it >= 0;          // state path of chunk it
        const int tp = (it + 1) * KP_C, ts = it * KP_C;
        KdaPipeBuf &bp = sm.buf[(it + 1) & 1];
        KdaPipeBuf &bs = sm.buf[it & 1];

        // ---- segment 1
        float2 bl[8];
        float2 ef[8], ifc[8];  // exp(b_t - m_J) and exp(m_J - b_t) of the two channels
        float nk[8], nq[8];    // inverse norms of k_t and q_t (1 without L2)
        bf16x8 fS[4];
        f32x4 Xs[2], O[2];
        if (pw) {
            float2 acc = make_float2(0.f, 0.f);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                acc.x += __uint_as_float(x.g[s][0]) * LOG2E;
                acc.y += __uint_as_float(x.g[s][1]) * LOG2E;
                bl[s] = acc;
            }
            *reinterpret_cast<float2 *>(&sm.htot[wave][2 * p]) = bl[7];
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                nk[s] = nq[s] = 1.f;
                if constexpr (L2) {
                    const float k0 = lo_bf16(x.k[s]), k1 = hi_bf16(x.k[s]);
                    const float q0 = lo_bf16(x.q[s]), q1 = hi_bf16(x.q[s]);
                    nk[s] = rsqrtf(wave_sum(k0 * k0 + k1 * k1) + 1e-6f);
                    nq[s] = rsqrtf(wave_sum(q0 * q0 + q1 * q1) + 1e-6f);
                }
            }
            // everything that needs only in-block differences: b_t - m_J is
            // the first half's own prefix difference (>= 0, rows grow) or
            // the second half's own prefix sum (<= 0, columns grow); only the
            // growing side is clamped.  Rows k e, q e and the block's own
            // columns k i go to LDS now.
            const int col = 2 * p;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int t = 16 * J + 8 * hf + s;
                if (hf == 0) {
                    const float d0 = bl[s].x - bl[7].x, d1 = bl[s].y - bl[7].y;
                    ef[s] = make_float2(exp2_(fminf(d0, KDA_EXP2_MAX)), exp2_(fminf(d1, KDA_EXP2_MAX)));
                    ifc[s] = make_float2(exp2_(-d0), exp2_(-d1));
                } else {
                    const float d0 = bl[s].x, d1 = bl[s].y;
                    ef[s] = make_float2(exp2_(d0), exp2_(d1));
                    ifc[s] = make_float2(exp2_(fminf(-d0, KDA_EXP2_MAX)), exp2_(fminf(-d1, KDA_EXP2_MAX)));
                }
                const float k0 = lo_bf16(x.k[s]) * nk[s], k1 = hi_bf16(x.k[s]) * nk[s];
                const float q0 = lo_bf16(x.q[s]) * nq[s], q1 = hi_bf16(x.q[s]) * nq[s];
                const int o_t = t * KDA_LD + col;
                *reinterpret_cast<unsigned *>(sm.KR + o_t) = pk2(k0 * ef[s].x, k1 * ef[s].y);
                *reinterpret_cast<unsigned *>(sm.QR + o_t) = pk2(q0 * ef[s].x, q1 * ef[s].y);
                *reinterpret_cast<unsigned *>(sm.KC + (kc_base(J) + t) * KDA_LD + col) =
                    pk2(k0 * ifc[s].x, k1 * ifc[s].y);
            }
        }
        if (sw) {
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
            float2 mI[2];
            float2 run = make_float2(0.f, 0.f);
#pragma unroll
            for (int I = 0; I < 2; ++I) {
                const float2 h0 = *reinterpret_cast<const float2 *>(&sm.htot[2 * I][2 * p]);
                const float2 h1 = *reinterpret_cast<const float2 *>(&sm.htot[2 * I + 1][2 * p]);
                mI[I] = make_float2(run.x + h0.x, run.y + h0.y);
                run.x += h0.x + h1.x;
                run.y += h0.y + h1.y;
            }
            if (wave == 0) {
                bp.gamC[2 * p] = exp2_(run.x);
                bp.gamC[2 * p + 1] = exp2_(run.y);
            }
            const float2 mJ = mI[J];
            const float2 GJ = make_float2(exp2_(mJ.x), exp2_(mJ.y));
            const float2 EJ = make_float2(exp2_(run.x - mJ.x), exp2_(run.y - mJ.y));
            const float2 F1 = make_float2(exp2_(fminf(mI[1].x - mJ.x, 0.f)), exp2_(fminf(mI[1].y - mJ.y, 0.f)));
            const int col = 2 * p;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int t = 16 * J + 8 * hf + s;
                const float k0 = lo_bf16(x.k[s]) * nk[s], k1 = hi_bf16(x.k[s]) * nk[s];
                const float q0 = lo_bf16(x.q[s]) * nq[s], q1 = hi_bf16(x.q[s]) * nq[s];
                const float g0 = ef[s].x * GJ.x, g1 = ef[s].y * GJ.y;   // Gamma_t
                const float c0 = k0 * ifc[s].x, c1 = k1 * ifc[s].y;     // column operand, block J
                const int o_t = t * KDA_LD + col;
                *reinterpret_cast<unsigned *>(bp.KT + o_t) = pk2(k0 * g0, k1 * g1);
                *reinterpret_cast<unsigned *>(bp.QT + o_t) = pk2(q0 * g0, q1 * g1);
                *reinterpret_cast<unsigned *>(bp.KE + o_t) = pk2(c0 * EJ.x, c1 * EJ.y);
                if (J == 0)
                    *reinterpret_cast<unsigned *>(sm.KC + (kc_base(1) + t) * KDA_LD + col) =
                        pk2(c0 * F1.x, c1 * F1.y);
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
        if (pw && wave < 3) {
            int I, Jb;
            pair_ij(wave, I, Jb);
            f32x4 aG = zero4(), aP = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 fc, fk, fq;
                frag_rows(sm.KC, KDA_LD, kc_base(I) + 16 * Jb, 32 * s, lane, fc);
                frag_rows(sm.KR, KDA_LD, 16 * I, 32 * s, lane, fk);
                frag_rows(sm.QR, KDA_LD, 16 * I, 32 * s, lane, fq);
                mma_k32(aG, fc, fk);
                mma_k32(aP, fc, fq);
            }
            if (I == Jb) {
                const float br = sm.beta[16 * I + r];
                f32x4 a, pm;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = r > 4 * g + e ? br * aG[e] : 0.f;
                    pm[e] = r >= 4 * g + e ? aP[e] : 0.f;
                }
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sm.beta + 16 * I + 4 * g);
                diag_inverse(a, b4, bp.Tb, I, lane);
                store_fragblk(bp.Pb, wave, lane, pm);
            } else {
                store_fragblk(bp.Gb, 0, lane, aG);
                store_fragblk(bp.Pb, wave, lane, aP);
            }
        }
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
