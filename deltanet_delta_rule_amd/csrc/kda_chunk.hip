// Chunked forward of Kimi Delta Attention (per-key-channel decay), bf16
// inputs, d_k = 128, chunks of 64 tokens (gfx950).
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
// matrix cores, the blocks below them are products.
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
// Work split.  One workgroup of eight waves owns one (sequence, head) and a
// slice of 64 value rows of S, and walks the chunks in order.  Per chunk:
//   1. wave w (tokens 8w .. 8w + 7) and lane p (key channels 2p, 2p + 1)
//      turn the prefetched k, q and gk of its tokens into the scaled
//      operands in LDS (prefix sums, with half-block sums exchanged through
//      LDS);
//   2. the ten 16-token block pairs (I, J <= I) of G and P are shared out over
//      the waves; diagonal blocks are inverted right away;
//   3. waves 0-3 (the solvers) each take 16 value rows: X = (K.Gamma) S^T and
//      the block substitution for E, which they hand to waves 4-7 through
//      LDS; waves 4-7 (the readers) meanwhile form (Q.Gamma) S^T for the same
//      rows, then add P E and store O.  Both keep the rows of S in registers
//      (fp32, the canonical k order of the matrix-core operands) and apply
//      the same state update from the same bf16 E, so their copies stay
//      identical.
// Two waves per SIMD let one wave's exponentials and LDS traffic overlap the
// other's matrix-core work.  The next chunk's inputs are loaded into
// registers while steps 2 and 3 run.
#include "chunk_fwd.hpp"

namespace dr {

namespace {

constexpr int KDA_C = 64;        // tokens per chunk
constexpr int KDA_DK = 128;      // key channels
constexpr int KDA_DVW = 64;      // value rows per workgroup
constexpr int KDA_LD = 136;      // row pitch (bf16) of the token x channel tiles
constexpr float LOG2E = 1.4426950408889634f;
constexpr float KDA_EXP2_MAX = 80.f * LOG2E;  // clamp of growing exponents (log2)

__device__ __forceinline__ float exp2_(float x) { return __builtin_amdgcn_exp2f(x); }

// Column operands of row block I start at row 8 I (I + 1) of KC: block I has
// the 16 (I + 1) tokens 0 .. 16 I + 15.
constexpr int kc_base(int I) { return 8 * I * (I + 1); }

struct alignas(16) KdaSmem {
    __bf16 KR[KDA_C * KDA_LD];        // k_i exp(b_i - m_I)        (Gram rows)
    __bf16 QR[KDA_C * KDA_LD];        // q_i exp(b_i - m_I)        (P rows)
    __bf16 KC[160 * KDA_LD];          // k_j exp(m_I - b_j), per row block I
    __bf16 KT[KDA_C * KDA_LD];        // k_t Gamma_t               (X)
    __bf16 QT[KDA_C * KDA_LD];        // q_t Gamma_t               (O)
    __bf16 KE[KDA_C * KDA_LD];        // k_t exp(b_last - b_t)     (state update)
    __bf16 Gb[6 * FRAG_ELEMS];        // G blocks below the diagonal
    __bf16 Tb[4 * FRAG_ELEMS];        // -T_II diag(beta_I), T_II = (I + diag(beta) G_II)^{-1}
    __bf16 Pb[10 * FRAG_ELEMS];       // P blocks on and below the diagonal
    float beta[KDA_C];
    float gamC[KDA_DK];               // Gamma_last per channel
    float htot[8][KDA_DK];            // sums of gk over each 8-token half block (log2)
    __bf16 Ex[4][4 * FRAG_ELEMS];     // E of each solver wave, as B-operand fragments
};

// Block pair p = I (I + 1) / 2 + J of the ten (I, J <= I).
__device__ __forceinline__ void pair_ij(int p, int &I, int &J) {
    I = p >= 6 ? 3 : p >= 3 ? 2 : p >= 1 ? 1 : 0;
    J = p - I * (I + 1) / 2;
}

__device__ __forceinline__ unsigned pk2(float a, float b) { return pk_bf16(a, b); }
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

// Loads of one chunk (tokens t0 .. t0 + 63 of the sequence) through buffer
// resources that span exactly its valid tokens: offsets are constants per
// lane and token, and tokens past the end of the sequence load as zeros
// (k = q = v = 0, gk = 0, beta = 0 leave the state unchanged).  The token part
// of each offset is wave-uniform and goes in the scalar offset.
__device__ __forceinline__ void kda_prefetch(KdaRegs &x, const KdaSeq &sq, int t0, int w,
                                             int p, int tid) {
    const int nv = min(KDA_C, sq.len - t0);
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
    x.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, min(tid, KDA_C - 1) * sq.H * 2, 0, 0);
}

// The value entries a solver lane needs, in the D layout of its X tiles:
// v[t0 + 16 I + 4 g + e][vcol] for I, e = 0..3.
__device__ __forceinline__ void kda_prefetch_v(unsigned short (&vr)[16], const KdaSeq &sq,
                                               int t0, int g, int vcol) {
    const int nv = min(KDA_C, sq.len - t0);
    const int sv = sq.H * sq.Dv * 2;
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(sq.v + sq.row(t0) * sq.Dv, nv * sv);
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            vr[4 * I + e] = __builtin_amdgcn_raw_buffer_load_b16(
                rv, (4 * g) * sv + 2 * vcol, (16 * I + e) * sv, 0);
}

__global__ __launch_bounds__(512) void kda_chunk_kernel(
    const __bf16 *__restrict__ q, const __bf16 *__restrict__ k, const __bf16 *__restrict__ v,
    const __bf16 *__restrict__ beta, const float *__restrict__ gk, const float *S0,
    __bf16 *__restrict__ o, float *S_T, const int *__restrict__ cu, int T, int H, int Dv,
    float scale) {
    __shared__ KdaSmem sm;
    // Consecutive workgroup ids go round-robin over the 8 XCDs (each with its
    // own L2); remap so that the value slices of one head, which read the same
    // k, q and gk and write the same o rows, run on the same XCD.
    int wg = blockIdx.x;
    const int nwg = gridDim.x;
    if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
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
    const int p = lane;                      // channel pair of the operand step
    const bool solver = wave < 4;
    const int vt = wave & 3;                 // value tile of the state step
    const int vcol = vb * KDA_DVW + 16 * vt + r;   // this lane's state row
    const int64_t srow = (seqhead * Dv + vcol) * KDA_DK;

    // state: slab s (channels 32 s ..), half 0: 32 s + 4 g + e, half 1: + 16
    f32x4 S[4][2];
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            S[s][hh] = zero4();
            if (S0) {
                const float4 x = *reinterpret_cast<const float4 *>(S0 + srow + 32 * s + 16 * hh + 4 * g);
                S[s][hh] = f32x4{x.x, x.y, x.z, x.w};
            }
        }

    const int nchunk = (sq.len + KDA_C - 1) / KDA_C;
    KdaRegs x;
    unsigned short vr[16];
    if (nchunk > 0) {
        kda_prefetch(x, sq, 0, wave, p, tid);
        if (solver) kda_prefetch_v(vr, sq, 0, g, vcol);
    }

    const int J = wave >> 1, hf = wave & 1;  // token block and half of the operand step
    for (int c = 0; c < nchunk; ++c) {
        const int t0 = c * KDA_C;
        // ---- 1. operands: prefix sums of the two channels over this wave's
        // 8 tokens, in log2 units (every exponential below is one exp2)
        float2 bl[8];
        {
            float2 acc = make_float2(0.f, 0.f);
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                acc.x += __uint_as_float(x.g[s][0]) * LOG2E;
                acc.y += __uint_as_float(x.g[s][1]) * LOG2E;
                bl[s] = acc;
            }
        }
        *reinterpret_cast<float2 *>(&sm.htot[wave][2 * p]) = bl[7];
        lds_barrier();
        {
            // m_I: prefix sum at the 8th token of block I = the end of its
            // first half; run: the prefix sum before block I, then b_last
            float2 mI[4];
            float2 run = make_float2(0.f, 0.f);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float2 h0 = *reinterpret_cast<const float2 *>(&sm.htot[2 * I][2 * p]);
                const float2 h1 = *reinterpret_cast<const float2 *>(&sm.htot[2 * I + 1][2 * p]);
                mI[I] = make_float2(run.x + h0.x, run.y + h0.y);
                run.x += h0.x + h1.x;
                run.y += h0.y + h1.y;
            }
            if (wave == 0) {
                sm.gamC[2 * p] = exp2_(run.x);
                sm.gamC[2 * p + 1] = exp2_(run.y);
            }
            const float2 mJ = mI[J];
            const float2 GJ = make_float2(exp2_(mJ.x), exp2_(mJ.y));            // Gamma at m_J
            const float2 EJ = make_float2(exp2_(run.x - mJ.x), exp2_(run.y - mJ.y));
            float2 F[4];  // exp(m_I - m_J) <= 1 for I > J
#pragma unroll
            for (int I = 0; I < 4; ++I)
                F[I] = make_float2(exp2_(fminf(mI[I].x - mJ.x, 0.f)), exp2_(fminf(mI[I].y - mJ.y, 0.f)));
            const int col = 2 * p;
#pragma unroll
            for (int s = 0; s < 8; ++s) {
                const int t = 16 * J + 8 * hf + s;
                // b_t - m_J: the first half's own prefix difference (>= 0,
                // rows grow), or the second half's own prefix sum (<= 0,
                // columns grow); only the growing side is clamped
                float e0, e1, i0, i1;
                if (hf == 0) {
                    const float d0 = bl[s].x - bl[7].x, d1 = bl[s].y - bl[7].y;
                    e0 = exp2_(fminf(d0, KDA_EXP2_MAX));
                    e1 = exp2_(fminf(d1, KDA_EXP2_MAX));
                    i0 = exp2_(-d0);
                    i1 = exp2_(-d1);
                } else {
                    const float d0 = bl[s].x, d1 = bl[s].y;
                    e0 = exp2_(d0);
                    e1 = exp2_(d1);
                    i0 = exp2_(fminf(-d0, KDA_EXP2_MAX));
                    i1 = exp2_(fminf(-d1, KDA_EXP2_MAX));
                }
                const float k0 = lo_bf16(x.k[s]), k1 = hi_bf16(x.k[s]);
                const float q0 = lo_bf16(x.q[s]), q1 = hi_bf16(x.q[s]);
                const float g0 = e0 * GJ.x, g1 = e1 * GJ.y;      // Gamma_t
                const float c0 = k0 * i0, c1 = k1 * i1;          // column operand, block J
                const int o_t = t * KDA_LD + col;
                *reinterpret_cast<unsigned *>(sm.KR + o_t) = pk2(k0 * e0, k1 * e1);
                *reinterpret_cast<unsigned *>(sm.QR + o_t) = pk2(q0 * e0, q1 * e1);
                *reinterpret_cast<unsigned *>(sm.KT + o_t) = pk2(k0 * g0, k1 * g1);
                *reinterpret_cast<unsigned *>(sm.QT + o_t) = pk2(q0 * g0, q1 * g1);
                *reinterpret_cast<unsigned *>(sm.KE + o_t) = pk2(c0 * EJ.x, c1 * EJ.y);
                *reinterpret_cast<unsigned *>(sm.KC + (kc_base(J) + t) * KDA_LD + col) = pk2(c0, c1);
#pragma unroll
                for (int I = 0; I < 4; ++I)
                    if (I > J)
                        *reinterpret_cast<unsigned *>(sm.KC + (kc_base(I) + t) * KDA_LD + col) =
                            pk2(c0 * F[I].x, c1 * F[I].y);
            }
        }
        if (tid < KDA_C) sm.beta[tid] = (float)__builtin_bit_cast(__bf16, x.beta);
        if (c + 1 < nchunk) kda_prefetch(x, sq, t0 + KDA_C, wave, p, tid);
        lds_barrier();

        // ---- 2. G and P blocks, diagonal inverses
        for (int pp = wave; pp < 10; pp += 8) {
            int I, Jb;
            pair_ij(pp, I, Jb);
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
            // lane (g, r) holds G[16 I + r][16 Jb + 4 g + e] (and P alike)
            if (I == Jb) {
                const float br = sm.beta[16 * I + r];
                f32x4 a, pm;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    a[e] = r > 4 * g + e ? br * aG[e] : 0.f;
                    pm[e] = r >= 4 * g + e ? aP[e] : 0.f;
                }
                const f32x4 b4 = *reinterpret_cast<const f32x4 *>(sm.beta + 16 * I + 4 * g);
                diag_inverse(a, b4, sm.Tb, I, lane);
                store_fragblk(sm.Pb, pp, lane, pm);
            } else {
                store_fragblk(sm.Gb, off_idx(I, Jb), lane, aG);
                store_fragblk(sm.Pb, pp, lane, aP);
            }
        }
        lds_barrier();

        // ---- 3. state path on 16 value rows
        {
            bf16x8 fS[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) cvt8(S[s][0], S[s][1], fS[s]);
            bf16x4 fE[4];  // E_I as B-operand fragments (lane (g, r): E_I[4g + e][r])
            if (solver) {
                // all four X tiles first (independent), then the serial solve
                f32x4 E[4], Xs[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) Xs[I] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        bf16x8 fk;
                        frag_rows(sm.KT, KDA_LD, 16 * I, 32 * s, lane, fk);
                        mma_k32(Xs[I], fk, fS[s]);
                    }
#pragma unroll
                for (int I = 0; I < 4; ++I) {
                    f32x4 X = Xs[I];
                    // Y = X - V + sum_{J<I} G_IJ E_J;  E_I = (-T_II diag(beta_I)) Y
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        X[e] -= (float)__builtin_bit_cast(__bf16, vr[4 * I + e]);
#pragma unroll
                    for (int Jb = 0; Jb < I; ++Jb) {
                        bf16x4 fa;
                        load_fragblk(sm.Gb, off_idx(I, Jb), lane, fa);
                        mma_k16(X, fa, fE[Jb]);
                    }
                    bf16x4 ft, fy;
                    load_fragblk(sm.Tb, I, lane, ft);
                    frag_from_acc16(X, fy);
                    E[I] = zero4();
                    mma_k16(E[I], ft, fy);
                    frag_from_acc16(E[I], fE[I]);
                    store_frag16(sm.Ex[vt] + I * FRAG_ELEMS + 4 * lane, fE[I]);
                }
                if (c + 1 < nchunk) kda_prefetch_v(vr, sq, t0 + KDA_C, g, vcol);
                lds_barrier();
            } else {
                f32x4 O[4];
#pragma unroll
                for (int I = 0; I < 4; ++I) O[I] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int I = 0; I < 4; ++I) {
                        bf16x8 fq;
                        frag_rows(sm.QT, KDA_LD, 16 * I, 32 * s, lane, fq);
                        mma_k32(O[I], fq, fS[s]);
                    }
                lds_barrier();
#pragma unroll
                for (int I = 0; I < 4; ++I) load_chunk(sm.Ex[vt] + I * FRAG_ELEMS + 4 * lane, fE[I]);
                // O_I += sum_{J<=I} P_IJ E_J, then out (stores past the
                // sequence's end fall outside the resource and are dropped)
                const int so = H * Dv * 2;
                const __amdgpu_buffer_rsrc_t ro =
                    make_rsrc(sq.o + sq.row(t0) * Dv, min(KDA_C, sq.len - t0) * so);
#pragma unroll
                for (int I = 0; I < 4; ++I) {
#pragma unroll
                    for (int Jb = 0; Jb <= I; ++Jb) {
                        bf16x4 fa;
                        load_fragblk(sm.Pb, I * (I + 1) / 2 + Jb, lane, fa);
                        mma_k16(O[I], fa, fE[Jb]);
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        buf_store_elem((__bf16)(scale * O[I][e]), ro,
                                       (16 * I + 4 * g + e) * so + 2 * vcol, 0);
                }
            }
            // S <- S diag(Gamma_last) + (E^T KE)^T, slab by slab (both copies)
            bf16x8 fE32[2];
            fE32[0] = __builtin_shufflevector(fE[0], fE[1], 0, 1, 2, 3, 4, 5, 6, 7);
            fE32[1] = __builtin_shufflevector(fE[2], fE[3], 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x4 d = zero4();
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        bf16x8 fa;
                        frag_cols32(sm.KE, KDA_LD, 32 * u, 32 * s + 16 * hh, lane, fa);
                        mma_k32(d, fa, fE32[u]);
                    }
                    const f32x4 gc = *reinterpret_cast<const f32x4 *>(sm.gamC + 32 * s + 16 * hh + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[s][hh][e] = S[s][hh][e] * gc[e] + d[e];
                }
        }
        // the next chunk's first LDS writes (half-block sums) touch only htot,
        // which nobody reads after the first barrier of this chunk
    }
    if (S_T && solver) {
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
    // v is read in 16-byte vectors here (the ABI only guarantees element
    // alignment), and one chunk of one head's rows of every input must be
    // addressable with 32-bit byte offsets
    const int64_t span = int64_t(KDA_C) * a.H * (a.Dv > 2 * KDA_DK ? 2 * a.Dv : 4 * KDA_DK);
    return bf16 && a.gk && !a.g && !a.l2 && !a.recurrent && a.Dk == KDA_DK &&
           a.Dv % KDA_DVW == 0 && (reinterpret_cast<uintptr_t>(a.v) & 15) == 0 &&
           span < INT32_MAX;
}

hipError_t launch_kda_chunk(const ChunkFwdArgs &a, hipStream_t stream) {
    if (a.B == 0 || a.H == 0) return hipSuccess;
    const int64_t grid = a.B * a.H * (a.Dv / KDA_DVW);
    hipLaunchKernelGGL(kda_chunk_kernel, dim3((unsigned)grid), dim3(512), 0, stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), static_cast<const __bf16 *>(a.beta),
                       a.gk, a.S0, static_cast<__bf16 *>(a.o), a.S_T, a.cu, (int)a.T, (int)a.H,
                       a.Dv, a.scale);
    return hipGetLastError();
}

}  // namespace dr
