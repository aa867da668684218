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
// Work split.  One workgroup of four waves owns one (sequence, head) and a
// slice of 64 value rows of S (wave w: rows 16w .. 16w + 15 of the slice, all
// d_k columns, fp32 in registers in the canonical k order of the matrix-core
// operands), and walks the chunks in order.  Per chunk:
//   1. wave J (token block J) and lane p (key channels 2p, 2p + 1) turn the
//      prefetched k, q and gk of its 16 tokens into the scaled operands in
//      LDS (prefix sums, with block totals exchanged through LDS);
//   2. the ten block pairs (I, J <= I) of G and P are shared out over the
//      waves; diagonal blocks are inverted right away;
//   3. each wave runs the state path on its 16 value rows: X = (K.Gamma)
//      S^T, the block substitution for E, O, and the state update.
// The next chunk's inputs are loaded into registers while steps 2 and 3 run.
#include "chunk_fwd.hpp"

namespace dr {

namespace {

constexpr int KDA_C = 64;        // tokens per chunk
constexpr int KDA_DK = 128;      // key channels
constexpr int KDA_DVW = 64;      // value rows per workgroup
constexpr int KDA_LD = 136;      // row pitch (bf16) of the token x channel tiles
constexpr int KDA_LDV = 72;      // row pitch (bf16) of the value tile
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
    __bf16 V[KDA_C * KDA_LDV];        // this workgroup's 64 value columns
    __bf16 Gb[6 * FRAG_ELEMS];        // G blocks below the diagonal
    __bf16 Tb[4 * FRAG_ELEMS];        // -T_II diag(beta_I), T_II = (I + diag(beta) G_II)^{-1}
    __bf16 Pb[10 * FRAG_ELEMS];       // P blocks on and below the diagonal
    float beta[KDA_C];
    float gamC[KDA_DK];               // Gamma_last per channel
    float tot[4][KDA_DK];             // block sums of gk
    float mid[4][KDA_DK];             // in-block prefix sum at the 8th token
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
    unsigned k[16], q[16];   // bf16 pairs: channels 2p, 2p + 1 of token 16J + s
    u32x2 g[16];             // their log decays (fp32 pairs)
    uint4 v[2];              // 8 bf16 value entries each
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
// (k = q = v = 0, gk = 0, beta = 0 leave the state unchanged).
__device__ __forceinline__ void kda_prefetch(KdaRegs &x, const KdaSeq &sq, int t0, int J,
                                             int p, int tid) {
    const int nv = min(KDA_C, sq.len - t0);
    const int64_t r0 = sq.row(t0);
    const int sk = sq.H * KDA_DK * 2, sg = sq.H * KDA_DK * 4, sv = sq.H * sq.Dv * 2;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(sq.k + r0 * KDA_DK, nv * sk);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(sq.q + r0 * KDA_DK, nv * sk);
    const __amdgpu_buffer_rsrc_t rg = make_rsrc(sq.gk + r0 * KDA_DK, nv * sg);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(sq.v + r0 * sq.Dv + sq.vcol0, nv * sv);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(sq.beta + r0, nv * sq.H * 2);
    // J is uniform over the wave: the token part of each offset goes in the
    // scalar offset, the lane part (the channel pair) in the vector offset
    const int Js = __builtin_amdgcn_readfirstlane(J);
#pragma unroll
    for (int s = 0; s < 16; ++s) {
        const int tk = 16 * Js + s;
        x.k[s] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * p, tk * sk, 0);
        x.q[s] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * p, tk * sk, 0);
        x.g[s] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, 8 * p, tk * sg, 0));
    }
#pragma unroll
    for (int n = 0; n < 2; ++n) {
        const int u = tid + 256 * n;
        x.v[n] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rv, (u / 8) * sv + 16 * (u % 8), 0, 0));
    }
    x.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, min(tid, KDA_C - 1) * sq.H * 2, 0, 0);
}

__global__ __launch_bounds__(256) void kda_chunk_kernel(
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
    const int p = lane;                       // channel pair of the operand step
    const int drow = vb * KDA_DVW + 16 * wave + r;  // this lane's state row
    const int64_t srow = (seqhead * Dv + drow) * KDA_DK;

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
    if (nchunk > 0) kda_prefetch(x, sq, 0, wave, p, tid);

    for (int c = 0; c < nchunk; ++c) {
        const int t0 = c * KDA_C;
        const int J = wave;
        // ---- 1. operands: in-block prefix sums of the two channels, in log2
        // units (every exponential below is one exp2)
        float2 bl[16];
        {
            float2 acc = make_float2(0.f, 0.f);
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                acc.x += __uint_as_float(x.g[s][0]) * LOG2E;
                acc.y += __uint_as_float(x.g[s][1]) * LOG2E;
                bl[s] = acc;
            }
        }
        *reinterpret_cast<float2 *>(&sm.tot[J][2 * p]) = bl[15];
        *reinterpret_cast<float2 *>(&sm.mid[J][2 * p]) = bl[7];
        lds_barrier();
        {
            float2 mI[4];
            float2 run = make_float2(0.f, 0.f);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                const float2 md = *reinterpret_cast<const float2 *>(&sm.mid[I][2 * p]);
                mI[I] = make_float2(run.x + md.x, run.y + md.y);
                const float2 tt = *reinterpret_cast<const float2 *>(&sm.tot[I][2 * p]);
                run.x += tt.x;
                run.y += tt.y;
            }
            // run = b_last (log2)
            if (J == 0) {
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
            for (int s = 0; s < 16; ++s) {
                const int t = 16 * J + s;
                // b_t - m_J is the in-block prefix difference: e grows for
                // s < 7 (rows), ei for s > 7 (columns); only those are clamped
                const float d0 = bl[s].x - bl[7].x, d1 = bl[s].y - bl[7].y;
                float e0 = 1.f, e1 = 1.f, i0 = 1.f, i1 = 1.f;
                if (s < 7) {
                    e0 = exp2_(fminf(d0, KDA_EXP2_MAX));
                    e1 = exp2_(fminf(d1, KDA_EXP2_MAX));
                    i0 = exp2_(-d0);
                    i1 = exp2_(-d1);
                } else if (s > 7) {
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
#pragma unroll
        for (int nn = 0; nn < 2; ++nn) {
            const int u = tid + 256 * nn;
            *reinterpret_cast<uint4 *>(sm.V + (u / 8) * KDA_LDV + 8 * (u % 8)) = x.v[nn];
        }
        if (tid < KDA_C) sm.beta[tid] = (float)__builtin_bit_cast(__bf16, x.beta);
        if (c + 1 < nchunk) kda_prefetch(x, sq, t0 + KDA_C, wave, p, tid);
        lds_barrier();

        // ---- 2. G and P blocks, diagonal inverses
        for (int pp = wave; pp < 10; pp += 4) {
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

        // ---- 3. state path on this wave's 16 value rows
        {
            bf16x8 fS[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) cvt8(S[s][0], S[s][1], fS[s]);
            f32x4 E[4], O[4];
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 X = zero4();
                O[I] = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    bf16x8 fk, fq;
                    frag_rows(sm.KT, KDA_LD, 16 * I, 32 * s, lane, fk);
                    frag_rows(sm.QT, KDA_LD, 16 * I, 32 * s, lane, fq);
                    mma_k32(X, fk, fS[s]);
                    mma_k32(O[I], fq, fS[s]);
                }
                // Y = X - V + sum_{J<I} G_IJ E_J;  E_I = (-T_II diag(beta_I)) Y
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    X[e] -= (float)sm.V[(16 * I + 4 * g + e) * KDA_LDV + 16 * wave + r];
#pragma unroll
                for (int Jb = 0; Jb < I; ++Jb) {
                    bf16x4 fa, fe;
                    load_fragblk(sm.Gb, off_idx(I, Jb), lane, fa);
                    frag_from_acc16(E[Jb], fe);
                    mma_k16(X, fa, fe);
                }
                bf16x4 ft, fy;
                load_fragblk(sm.Tb, I, lane, ft);
                frag_from_acc16(X, fy);
                E[I] = zero4();
                mma_k16(E[I], ft, fy);
            }
            // O_I += sum_{J<=I} P_IJ E_J, then out (stores past the sequence's
            // end fall outside the resource and are dropped)
            const int so = H * Dv * 2;
            const __amdgpu_buffer_rsrc_t ro =
                make_rsrc(sq.o + sq.row(t0) * Dv, min(KDA_C, sq.len - t0) * so);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
#pragma unroll
                for (int Jb = 0; Jb <= I; ++Jb) {
                    bf16x4 fa, fe;
                    load_fragblk(sm.Pb, I * (I + 1) / 2 + Jb, lane, fa);
                    frag_from_acc16(E[Jb], fe);
                    mma_k16(O[I], fa, fe);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    buf_store_elem((__bf16)(scale * O[I][e]), ro, (16 * I + 4 * g + e) * so + 2 * drow, 0);
            }
            // S <- S diag(Gamma_last) + (E^T KE)^T, slab by slab
            bf16x8 fE[2];
            cvt8(E[0], E[1], fE[0]);
            cvt8(E[2], E[3], fE[1]);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int hh = 0; hh < 2; ++hh) {
                    f32x4 d = zero4();
#pragma unroll
                    for (int u = 0; u < 2; ++u) {
                        bf16x8 fa;
                        frag_cols32(sm.KE, KDA_LD, 32 * u, 32 * s + 16 * hh, lane, fa);
                        mma_k32(d, fa, fE[u]);
                    }
                    const f32x4 gc = *reinterpret_cast<const f32x4 *>(sm.gamC + 32 * s + 16 * hh + 4 * g);
#pragma unroll
                    for (int e = 0; e < 4; ++e) S[s][hh][e] = S[s][hh][e] * gc[e] + d[e];
                }
        }
        // the next chunk's first LDS writes (block sums) touch only tot and
        // mid, which nobody reads after the barrier above
    }
    if (S_T) {
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
    hipLaunchKernelGGL(kda_chunk_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const __bf16 *>(a.q), static_cast<const __bf16 *>(a.k),
                       static_cast<const __bf16 *>(a.v), static_cast<const __bf16 *>(a.beta),
                       a.gk, a.S0, static_cast<__bf16 *>(a.o), a.S_T, a.cu, (int)a.T, (int)a.H,
                       a.Dv, a.scale);
    return hipGetLastError();
}

}  // namespace dr
