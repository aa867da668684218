// Fused chunkwise-parallel forward of the delta rule (gfx950).
//
// Math (per head; chunk c spans C tokens with incoming state S_c, d_v x d_k):
//   A   = tril(diag(beta) K K^T, -1)                     chunk key couplings
//   Ti  = (I + A)^{-1}                                    unit lower-triangular
//   E   = Ti diag(beta) (V - K S_c^T)                     resolved errors
//   O   = Q S_c^T + (Q K^T (.) M) E                       M incl. the diagonal
//   S_{c+1} = S_c + E^T K
// The pieces come from the paperlayer summary of arXiv:2406.06484 (section 3
// "Parallelizing DeltaNet Across the Sequence Dimension": chunking, the
// Householder/WY representation, forward substitution for the triangular
// inverse; App. B.2 "UT transform derivation": T = (I + A)^{-1} diag(beta))
// and the hada.io digest (section "Chunkwise KDA": provisional errors against
// the incoming state, the unit lower-triangular solve that restores the causal
// coupling, the end-of-chunk state as one product and the outputs with the
// diagonal included; section "Pipeline Triton Chunkwise": 16-token diagonal
// blocks solved first, then the off-diagonal blocks).  With D = I and no
// output scale this is plain DeltaNet.  E = U - W S_c^T of the UT form; the
// kernel applies Ti to the residual instead of forming W = T K and U = T V,
// which skips the C x C x d_k product for W.
//
// Work split.  One workgroup owns one (b, h) and a tile of BV = 16*NW value
// rows of S and walks the chunks in order, so the state never leaves the chip.
// Wave w owns 16 rows of S as fp32 MFMA accumulators (lane (g, r) holds
// S[row r][16*dt + 4g + i]).  Rows of S evolve independently, so waves never
// exchange state: every product on the state path (K S^T, Q S^T, Ti R, P E,
// K^T E) runs inside one wave from registers, using the D-layout-as-B-operand
// identity of dr_common.hpp; K^T fragments come from the token-major K tile
// through the LDS transpose read.  The per-chunk work that does not depend on
// the state -- the Gram tiles K K^T and Q K^T and the blocked triangular
// inverse -- is shared by the waves through LDS.
//
// Two kernels implement this:
//  * chunk_fwd_pipelined_kernel (used whenever its buffers fit in LDS) runs a
//    two-phase software pipeline with two barriers per chunk:
//      phase 1: state path of chunk c  +  Gram tiles of chunk c+1
//      phase 2: triangular inverse of chunk c+1  +  staging of chunk c+2
//    with K, Q, Ti, P double-buffered and chunk c+3 loading into registers.
//  * chunk_fwd_serial_kernel runs the same steps one after the other on single
//    buffers (fp32 inputs with large d_k * chunk, whose double buffers would
//    exceed the 160 KiB of LDS).
#include "dr_common.hpp"
#include "dr_launch.hpp"

namespace dr {

namespace {

template <typename DT> struct Vec16;  // 16 bytes of DT
template <> struct Vec16<__bf16> {
    typedef bf16x8 type;
    static constexpr int N = 8;
};
template <> struct Vec16<float> {
    typedef f32x4 type;
    static constexpr int N = 4;
};

template <typename DT, int DK, int C, int NW>
struct ChunkCfg {
    static constexpr int BV = 16 * NW;          // value rows per workgroup
    static constexpr int NT = C / 16;           // 16-token tiles per chunk
    static constexpr int ND = DK / 16;          // 16-wide key tiles
    static constexpr int KSD = (DK % 32 == 0) ? 32 : 16;  // slab over d_k
    static constexpr int KSC = (C % 32 == 0) ? 32 : 16;   // slab over tokens
    static constexpr int PADE = 16 / (int)sizeof(DT);     // 16 bytes per row
    static constexpr int LDK = DK + PADE;       // K, Q row stride
    static constexpr int LDC = C + PADE;        // Ti, P (and K^T) row stride
    static constexpr int LDA = C + 4;           // A row stride (fp32)
    static constexpr int LDD = 16 + PADE;       // diagonal-inverse scratch stride
    static constexpr int VEC = Vec16<DT>::N;    // elements per 16-byte load
    static constexpr int VPR = DK / VEC;        // 16-byte vectors per K row
    static constexpr int NTHR = 64 * NW;
    static constexpr int NPRE = (C * VPR + NTHR - 1) / NTHR;  // vectors/thread
    static constexpr int NTILE = NT * (NT + 1) / 2;          // lower 16x16 tiles
};

template <bool K32, typename DT> struct SlabFrag;
template <typename DT> struct SlabFrag<true, DT> { typedef typename Frag<DT>::k32 type; };
template <typename DT> struct SlabFrag<false, DT> { typedef typename Frag<DT>::k16 type; };

// acc += M[rows row0..row0+15, slab k0] * (B operand built from accumulator
// tiles bt[k0/16], bt[k0/16 + 1]).
template <typename DT, int KS>
__device__ __forceinline__ void mma_rows_acc(f32x4 &acc, const DT *M, int ld, int row0,
                                             int k0, int lane, const f32x4 *bt) {
    typename SlabFrag<KS == 32, DT>::type fa, fb;
    frag_rows(M, ld, row0, k0, lane, fa);
    if constexpr (KS == 32) {
        frag_from_acc32(bt[k0 / 16], bt[k0 / 16 + 1], fb);
        mma_k32(acc, fa, fb);
    } else {
        frag_from_acc16(bt[k0 / 16], fb);
        mma_k16(acc, fa, fb);
    }
}

// acc += M^T[rows col0..col0+15, slab k0] * (B from accumulator tiles), where
// M is row-major with k along its rows (the transpose is read from LDS).
template <typename DT, int KS>
__device__ __forceinline__ void mma_cols_acc(f32x4 &acc, const DT *M, int ld, int col0,
                                             int k0, int lane, const f32x4 *bt) {
    typename SlabFrag<KS == 32, DT>::type fa, fb;
    if constexpr (KS == 32) {
        frag_cols32(M, ld, k0, col0, lane, fa);
        frag_from_acc32(bt[k0 / 16], bt[k0 / 16 + 1], fb);
        mma_k32(acc, fa, fb);
    } else {
        frag_cols16(M, ld, k0, col0, lane, fa);
        frag_from_acc16(bt[k0 / 16], fb);
        mma_k16(acc, fa, fb);
    }
}

// acc += M1[rows ra..ra+15, slab k0] * M2[rows rb..rb+15, slab k0]^T
template <typename DT, int KS>
__device__ __forceinline__ void mma_rows_rows(f32x4 &acc, const DT *M1, const DT *M2,
                                              int ld, int ra, int rb, int k0, int lane) {
    typename SlabFrag<KS == 32, DT>::type fa, fb;
    frag_rows(M1, ld, ra, k0, lane, fa);
    frag_rows(M2, ld, rb, k0, lane, fb);
    if constexpr (KS == 32) mma_k32(acc, fa, fb);
    else mma_k16(acc, fa, fb);
}

// Row and column of the jj-th lower tile (row-major order over ti >= tj).
__device__ __forceinline__ void lower_tile(int jj, int &ti, int &tj) {
    ti = 0;
    while ((ti + 1) * (ti + 2) / 2 <= jj) ++ti;
    tj = jj - ti * (ti + 1) / 2;
}

// ---------------------------------------------------------------------------
// Per-chunk building blocks shared by both kernels.
// ---------------------------------------------------------------------------

// Gram tiles of one chunk, split over the waves (tile jobs w, w + NW, ...):
//   Af[i][j] = beta_i (K K^T)_ij for i > j, else 0      (fp32)
//   Ps[i][j] = (Q K^T)_ij for i >= j, else 0             (DT)
// Only lower tiles are written; upper tiles of Ps stay zero.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void gram_tiles(const DT *Ks, const DT *Qs, const float *betas,
                                           float *Af, DT *Ps, int wave, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    const int g = lane >> 4, r = lane & 15;
    constexpr int NJ = (2 * G::NTILE + NW - 1) / NW;
#pragma unroll
    for (int s = 0; s < NJ; ++s) {
        const int job = wave + s * NW;
        if (job < 2 * G::NTILE) {
            const bool isP = job >= G::NTILE;
            int ti, tj;
            lower_tile(isP ? job - G::NTILE : job, ti, tj);
            f32x4 acc = zero4();
#pragma unroll
            for (int k0 = 0; k0 < DK; k0 += G::KSD)
                mma_rows_rows<DT, G::KSD>(acc, isP ? Qs : Ks, Ks, G::LDK, 16 * ti, 16 * tj, k0,
                                          lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * ti + 4 * g + i, col = 16 * tj + r;
                if (isP)
                    Ps[row * G::LDC + col] = from_f32<DT>(row >= col ? acc[i] : 0.f);
                else
                    Af[row * G::LDA + col] = (row > col) ? betas[row] * acc[i] : 0.f;
            }
        }
    }
}

// Ti = (I + A)^{-1} by blocks of 16, written into Ts (DT, row-major).
//  1. Every wave inverts all NT diagonal blocks (lane = 16*d + column, fp32
//     forward substitution) into its private scratch Dw, stored transposed
//     (row 16d + c of Dw is column c of block d).
//  2. Wave w then fills the block columns j = w, w + NW, ...:
//       Ti_jj from step 1, and for i > j
//       Ti_ij = -Ti_ii * sum_{k=j}^{i-1} A_ik Ti_kj,
//     each block column needing only its own earlier blocks and the diagonal
//     inverses, so no wave waits for another.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void tri_inverse(const float *Af, DT *Ts, DT *Dw, int wave,
                                            int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, LDA = G::LDA, LDC = G::LDC, LDD = G::LDD;
    const int g = lane >> 4, r = lane & 15;
    const int d = lane >> 4, cc = lane & 15;
    float x[16];
    if (lane < C) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == cc) ? 1.f : 0.f;
            const float *arow = Af + (16 * d + i) * LDA + 16 * d;
#pragma unroll
            for (int j = 0; j < i; ++j) s -= arow[j] * x[j];
            x[i] = s;
        }
        DT *drow = Dw + (16 * d + cc) * LDD;
#pragma unroll
        for (int i = 0; i < 16; ++i) drow[i] = from_f32<DT>(x[i]);
    }
    wave_lds_fence();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if (j % NW != wave) continue;
        // diagonal block j: lanes of block j hold its columns
        if (d == j) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
                Ts[(16 * j + i) * LDC + 16 * j + cc] = from_f32<DT>(x[i]);
        }
        f32x4 Tcol[NT];
#pragma unroll
        for (int i = j + 1; i < NT; ++i) {
            f32x4 acc = zero4();
#pragma unroll
            for (int kb = j; kb < i; ++kb) {
                typename Frag<DT>::k16 fa, fb;
                float a4[4];
                load4(Af + (16 * i + r) * LDA + 16 * kb + 4 * g, a4);
#pragma unroll
                for (int e = 0; e < 4; ++e) frag_set(fa, e, a4[e]);
                if (kb == j) {
                    // B = Ti_jj: lane (g, r) takes Ti_jj[4g + e][r] = Dw row 16j + r
                    float b4[4];
                    load4(Dw + (16 * j + r) * LDD + 4 * g, b4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) frag_set(fb, e, b4[e]);
                } else {
                    frag_from_acc16(Tcol[kb], fb);
                }
                mma_k16(acc, fa, fb);
            }
            // A = Ti_ii: lane (g, r) takes Ti_ii[r][4g + e] = Dw[16i + 4g + e][r]
            typename Frag<DT>::k16 fa, fb;
            frag_cols16(Dw, LDD, 16 * i, 0, lane, fa);
            frag_from_acc16(acc, fb);
            f32x4 res = zero4();
            mma_k16(res, fa, fb);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Tcol[i][e] = -res[e];
                Ts[(16 * i + 4 * g + e) * LDC + 16 * j + r] = from_f32<DT>(-res[e]);
            }
        }
    }
}

// State path of one chunk for this wave's 16 rows of S:
//   X = K S^T, Y = Q S^T, R = diag(beta)(V - X), E = Ti R,
//   O = Y + P E (stored for tokens < len), S^T += K^T E.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void state_path(const DT *Ks, const DT *Qs, const DT *Ts,
                                           const DT *Ps, const float *betas,
                                           const float (&vcur)[C / 16][4], f32x4 *Sacc,
                                           DT *oh, int64_t tsv, int t0, int len, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    const int g = lane >> 4;
    f32x4 X[NT], Y[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) X[mt] = Y[mt] = zero4();
#pragma unroll
    for (int k0 = 0; k0 < DK; k0 += G::KSD)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            mma_rows_acc<DT, G::KSD>(X[mt], Ks, G::LDK, 16 * mt, k0, lane, Sacc);
            mma_rows_acc<DT, G::KSD>(Y[mt], Qs, G::LDK, 16 * mt, k0, lane, Sacc);
        }
    // R = diag(beta) (V - K S^T), in place in X
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            X[mt][i] = betas[16 * mt + 4 * g + i] * (vcur[mt][i] - X[mt][i]);
    // E = Ti R  (Ti lower-triangular: slabs past the diagonal are zero)
    f32x4 E[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        E[mt] = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16 * (mt + 1); k0 += G::KSC)
            mma_rows_acc<DT, G::KSC>(E[mt], Ts, G::LDC, 16 * mt, k0, lane, X);
    }
    // S^T += K^T E  (K^T read through the transpose path of the K tile)
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int k0 = 0; k0 < C; k0 += G::KSC)
            mma_cols_acc<DT, G::KSC>(Sacc[dt], Ks, G::LDK, 16 * dt, k0, lane, E);
    // O = Q S^T + P E.  P E gets its own accumulator: Y comes from slabs
    // over d_k and P E from slabs over tokens, which can be different MFMA
    // shapes, and an accumulation chain must never switch shape (the compiler
    // issues such a dependent pair back to back and the second one reads a
    // stale accumulator).
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        f32x4 PE = zero4();
#pragma unroll
        for (int k0 = 0; k0 < 16 * (mt + 1); k0 += G::KSC)
            mma_rows_acc<DT, G::KSC>(PE, Ps, G::LDC, 16 * mt, k0, lane, E);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = 16 * mt + 4 * g + i;
            if (t < len) oh[(t0 + t) * tsv] = from_f32<DT>(Y[mt][i] + PE[i]);
        }
    }
}

// Common per-workgroup addressing: (b, h, value tile) of this workgroup with
// an XCD-aware remap, and the base pointers of its head.
template <typename DT>
struct HeadPtrs {
    const DT *kh, *qh, *vh, *bh;
    DT *oh;
    int64_t tsk, tsv, sbase;
    int vcol;
};

template <typename DT, int DK, int NW>
__device__ __forceinline__ HeadPtrs<DT> head_ptrs(const DT *q, const DT *k, const DT *v,
                                                  const DT *beta, DT *o, int T, int H,
                                                  int Dv, int nvt, int wave, int r) {
    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs
    // (each with its own L2).  Remap so that the value tiles of one head,
    // which read the same K and Q, run on the same XCD.
    int wg = blockIdx.x;
    const int nwg = gridDim.x;
    if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
    const int head = wg / nvt, vt = wg % nvt;
    const int b = head / H, h = head % H;
    HeadPtrs<DT> p;
    p.vcol = vt * 16 * NW + wave * 16 + r;
    p.tsk = (int64_t)H * DK;
    p.tsv = (int64_t)H * Dv;
    p.kh = k + ((int64_t)b * T * H + h) * DK;
    p.qh = q + ((int64_t)b * T * H + h) * DK;
    p.vh = v + ((int64_t)b * T * H + h) * Dv + p.vcol;
    p.oh = o + ((int64_t)b * T * H + h) * Dv + p.vcol;
    p.bh = beta + (int64_t)b * T * H + h;
    p.sbase = ((int64_t)head * Dv + p.vcol) * DK;
    return p;
}

// Register staging of one chunk's K, Q and beta.  Loads are unconditional
// (addresses clamped into the sequence) so that none sits in a branch that
// would force an early wait; out-of-range tokens are zeroed when staged.
template <typename DT, int DK, int C, int NW>
struct KQRegs {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename Vec16<DT>::type vec_t;
    vec_t k[G::NPRE], q[G::NPRE];
    DT b;

    __device__ __forceinline__ void load(const HeadPtrs<DT> &p, int T, int H, int t0, int tid) {
        const int last = min(C, T - t0) - 1;  // >= 0: the chunk holds a token
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            const int idx = min(tid + j * G::NTHR, C * G::VPR - 1);
            const int t = min(idx / G::VPR, last), e0 = (idx % G::VPR) * G::VEC;
            k[j] = *reinterpret_cast<const vec_t *>(p.kh + (t0 + t) * p.tsk + e0);
            q[j] = *reinterpret_cast<const vec_t *>(p.qh + (t0 + t) * p.tsk + e0);
        }
        b = p.bh[(int64_t)(t0 + min(tid, last)) * H];
    }
    // Write into one LDS buffer set; tokens >= len become zeros.
    __device__ __forceinline__ void stage(DT *Ks, DT *Qs, float *betas, int len, int tid) const {
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            const int idx = tid + j * G::NTHR;
            if (idx < C * G::VPR) {
                const int t = idx / G::VPR, e0 = (idx % G::VPR) * G::VEC;
                *reinterpret_cast<vec_t *>(Ks + t * G::LDK + e0) = (t < len) ? k[j] : vec_t{};
                *reinterpret_cast<vec_t *>(Qs + t * G::LDK + e0) = (t < len) ? q[j] : vec_t{};
            }
        }
        if (tid < C) betas[tid] = (tid < len) ? to_f32(b) : 0.f;
    }
};

// This lane's values of V for one chunk in D layout (token 16mt + 4g + i).
template <typename DT, int C>
__device__ __forceinline__ void load_v(const HeadPtrs<DT> &p, int T, int t0, int g,
                                       DT (&dst)[C / 16][4]) {
    const int last = min(C, T - t0) - 1;
#pragma unroll
    for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[mt][i] = p.vh[(t0 + min(16 * mt + 4 * g + i, last)) * p.tsv];
}

template <typename DT, int C>
__device__ __forceinline__ void widen_v(const DT (&raw)[C / 16][4], int len, int g,
                                        float (&dst)[C / 16][4]) {
#pragma unroll
    for (int mt = 0; mt < C / 16; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[mt][i] = (16 * mt + 4 * g + i < len) ? to_f32(raw[mt][i]) : 0.f;
}

// ---------------------------------------------------------------------------
// Pipelined kernel
// ---------------------------------------------------------------------------
template <typename DT, int DK, int C, int NW>
struct PipeSmem {
    typedef ChunkCfg<DT, DK, C, NW> G;
    DT Ks[2][C * G::LDK];          // K, token-major (double-buffered)
    DT Qs[2][C * G::LDK];          // Q, token-major
    DT Ts[2][C * G::LDC];          // (I + A)^{-1}
    DT Ps[2][C * G::LDC];          // Q K^T (.) M
    float Af[C * G::LDA];          // A = beta (K K^T) strictly lower, fp32
    float betas[2][C];
    DT Dw[NW][C * G::LDD];         // per-wave diagonal inverses (transposed)
};

template <typename DT, int DK, int C, int NW>
constexpr bool pipelined_fits() {
    return sizeof(PipeSmem<DT, DK, C, NW>) <= 160 * 1024;
}

template <typename DT, int DK, int C, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_fwd_pipelined_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *S0, DT *__restrict__ o, float *S_T,
    int T, int H, int Dv, int nvt) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    __shared__ __attribute__((aligned(16))) PipeSmem<DT, DK, C, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const HeadPtrs<DT> p = head_ptrs<DT, DK, NW>(q, k, v, beta, o, T, H, Dv, nvt, wave, r);

    f32x4 Sacc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
        Sacc[dt] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + p.sbase + 16 * dt + 4 * g)
                      : zero4();

    const int N = (T + C - 1) / C;
    if (N > 0) {
        // Upper blocks of Ts and Ps stay zero for the whole sequence.
        for (int i = tid; i < 2 * C * G::LDC; i += G::NTHR) {
            (&sm.Ts[0][0])[i] = from_f32<DT>(0.f);
            (&sm.Ps[0][0])[i] = from_f32<DT>(0.f);
        }
        KQRegs<DT, DK, C, NW> kq;
        DT vraw[NT][4], vnext[NT][4];
        // prologue: chunks 0 and 1 staged, chunk 0 solved, chunk 2 in flight
        kq.load(p, T, H, 0, tid);
        load_v<DT, C>(p, T, 0, g, vraw);
        kq.stage(sm.Ks[0], sm.Qs[0], sm.betas[0], min(C, T), tid);
        const int c1 = min(1, N - 1);
        kq.load(p, T, H, c1 * C, tid);
        kq.stage(sm.Ks[1], sm.Qs[1], sm.betas[1], min(C, T - c1 * C), tid);
        kq.load(p, T, H, min(2, N - 1) * C, tid);
        lds_barrier();
        gram_tiles<DT, DK, C, NW>(sm.Ks[0], sm.Qs[0], sm.betas[0], sm.Af, sm.Ps[0], wave, lane);
        lds_barrier();
        tri_inverse<DT, DK, C, NW>(sm.Af, sm.Ts[0], sm.Dw[wave], wave, lane);
        lds_barrier();

        for (int c = 0; c < N; ++c) {
            const int b = c & 1, b1 = b ^ 1;
            const int t0 = c * C;
            const int len = min(C, T - t0);
            // ---- phase 1: state path of chunk c, Gram tiles of chunk c+1 ----
            load_v<DT, C>(p, T, min(c + 1, N - 1) * C, g, vnext);
            float vcur[NT][4];
            widen_v<DT, C>(vraw, len, g, vcur);
            state_path<DT, DK, C, NW>(sm.Ks[b], sm.Qs[b], sm.Ts[b], sm.Ps[b], sm.betas[b],
                                      vcur, Sacc, p.oh, p.tsv, t0, len, lane);
            // (past the last chunk this works on stale buffers; never read)
            gram_tiles<DT, DK, C, NW>(sm.Ks[b1], sm.Qs[b1], sm.betas[b1], sm.Af, sm.Ps[b1],
                                      wave, lane);
            lds_barrier();
            // ---- phase 2: inverse of chunk c+1, staging of chunk c+2 ----
            tri_inverse<DT, DK, C, NW>(sm.Af, sm.Ts[b1], sm.Dw[wave], wave, lane);
            const int c2 = min(c + 2, N - 1);
            kq.stage(sm.Ks[b], sm.Qs[b], sm.betas[b], min(C, T - c2 * C), tid);
            kq.load(p, T, H, min(c + 3, N - 1) * C, tid);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) vraw[mt][i] = vnext[mt][i];
            lds_barrier();
        }
    }
    if (S_T) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            *reinterpret_cast<f32x4 *>(S_T + p.sbase + 16 * dt + 4 * g) = Sacc[dt];
    }
}

// ---------------------------------------------------------------------------
// Serial kernel (single-buffered; for shapes whose double buffers do not fit)
// ---------------------------------------------------------------------------
template <typename DT, int DK, int C, int NW>
struct SerialSmem {
    typedef ChunkCfg<DT, DK, C, NW> G;
    DT Ks[C * G::LDK];
    DT Qs[C * G::LDK];
    DT Ts[C * G::LDC];
    DT Ps[C * G::LDC];
    float Af[C * G::LDA];
    float betas[C];
    DT Dw[NW][C * G::LDD];
};

template <typename DT, int DK, int C, int NW>
__global__ __launch_bounds__(64 * NW) void chunk_fwd_serial_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *S0, DT *__restrict__ o, float *S_T,
    int T, int H, int Dv, int nvt) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    __shared__ __attribute__((aligned(16))) SerialSmem<DT, DK, C, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, r = lane & 15;
    const HeadPtrs<DT> p = head_ptrs<DT, DK, NW>(q, k, v, beta, o, T, H, Dv, nvt, wave, r);

    f32x4 Sacc[ND];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
        Sacc[dt] = S0 ? *reinterpret_cast<const f32x4 *>(S0 + p.sbase + 16 * dt + 4 * g)
                      : zero4();

    const int N = (T + C - 1) / C;
    if (N > 0) {
        for (int i = tid; i < C * G::LDC; i += G::NTHR) {
            sm.Ts[i] = from_f32<DT>(0.f);
            sm.Ps[i] = from_f32<DT>(0.f);
        }
        KQRegs<DT, DK, C, NW> kq;
        DT vraw[NT][4];
        kq.load(p, T, H, 0, tid);
        load_v<DT, C>(p, T, 0, g, vraw);
        for (int c = 0; c < N; ++c) {
            const int t0 = c * C;
            const int len = min(C, T - t0);
            lds_barrier();
            kq.stage(sm.Ks, sm.Qs, sm.betas, len, tid);
            float vcur[NT][4];
            widen_v<DT, C>(vraw, len, g, vcur);
            lds_barrier();
            kq.load(p, T, H, min(c + 1, N - 1) * C, tid);
            load_v<DT, C>(p, T, min(c + 1, N - 1) * C, g, vraw);
            gram_tiles<DT, DK, C, NW>(sm.Ks, sm.Qs, sm.betas, sm.Af, sm.Ps, wave, lane);
            lds_barrier();
            tri_inverse<DT, DK, C, NW>(sm.Af, sm.Ts, sm.Dw[wave], wave, lane);
            lds_barrier();
            state_path<DT, DK, C, NW>(sm.Ks, sm.Qs, sm.Ts, sm.Ps, sm.betas, vcur, Sacc, p.oh,
                                      p.tsv, t0, len, lane);
        }
    }
    if (S_T) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            *reinterpret_cast<f32x4 *>(S_T + p.sbase + 16 * dt + 4 * g) = Sacc[dt];
    }
}

// ---------------------------------------------------------------------------
// Host dispatch
// ---------------------------------------------------------------------------
template <typename DT, int DK, int C, int NW>
hipError_t launch_cfg(const void *q, const void *k, const void *v, const void *beta,
                      const float *S0, void *o, float *S_T, int64_t B, int64_t T,
                      int64_t H, int Dv, hipStream_t stream) {
    const int nvt = Dv / (16 * NW);
    const int64_t grid = B * H * nvt;
    if constexpr (pipelined_fits<DT, DK, C, NW>()) {
        hipLaunchKernelGGL((chunk_fwd_pipelined_kernel<DT, DK, C, NW>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, stream, static_cast<const DT *>(q),
                           static_cast<const DT *>(k), static_cast<const DT *>(v),
                           static_cast<const DT *>(beta), S0, static_cast<DT *>(o), S_T,
                           (int)T, (int)H, Dv, nvt);
    } else {
        hipLaunchKernelGGL((chunk_fwd_serial_kernel<DT, DK, C, NW>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, stream, static_cast<const DT *>(q),
                           static_cast<const DT *>(k), static_cast<const DT *>(v),
                           static_cast<const DT *>(beta), S0, static_cast<DT *>(o), S_T,
                           (int)T, (int)H, Dv, nvt);
    }
    return hipGetLastError();
}

// Waves per workgroup.  The chunk walk is sequential, so the time per chunk
// sets the pace: four waves share a chunk's Gram tiles and triangular inverse
// four ways, which beats spreading value tiles over more, thinner workgroups
// even when that leaves CUs idle.  Fewer waves only when Dv is too small.
inline int pick_waves(int64_t /*BH*/, int Dv) {
    for (int nw = 4; nw >= 1; nw >>= 1)
        if (Dv % (16 * nw) == 0) return nw;
    return 1;
}

template <typename DT, int DK, int C>
hipError_t dispatch_nw(const void *q, const void *k, const void *v, const void *beta,
                       const float *S0, void *o, float *S_T, int64_t B, int64_t T,
                       int64_t H, int Dv, hipStream_t stream) {
    switch (pick_waves(B * H, Dv)) {
    case 4: return launch_cfg<DT, DK, C, 4>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    case 2: return launch_cfg<DT, DK, C, 2>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    default: return launch_cfg<DT, DK, C, 1>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    }
}

template <typename DT, int DK>
hipError_t dispatch_c(const void *q, const void *k, const void *v, const void *beta,
                      const float *S0, void *o, float *S_T, int64_t B, int64_t T,
                      int64_t H, int Dv, int chunk, hipStream_t stream) {
    switch (chunk) {
    case 16: return dispatch_nw<DT, DK, 16>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    case 32: return dispatch_nw<DT, DK, 32>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    case 64: return dispatch_nw<DT, DK, 64>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename DT>
hipError_t dispatch_dk(const void *q, const void *k, const void *v, const void *beta,
                       const float *S0, void *o, float *S_T, int64_t B, int64_t T,
                       int64_t H, int Dk, int Dv, int chunk, hipStream_t stream) {
    switch (Dk) {
    case 16: return dispatch_c<DT, 16>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, chunk, stream);
    case 32: return dispatch_c<DT, 32>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, chunk, stream);
    case 64: return dispatch_c<DT, 64>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, chunk, stream);
    case 128: return dispatch_c<DT, 128>(q, k, v, beta, S0, o, S_T, B, T, H, Dv, chunk, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_chunk_fwd(const void *q, const void *k, const void *v,
                            const void *beta, const float *S0, void *o, float *S_T,
                            int64_t B, int64_t T, int64_t H, int Dk, int Dv,
                            int chunk, bool bf16, hipStream_t stream) {
    if (bf16)
        return dispatch_dk<__bf16>(q, k, v, beta, S0, o, S_T, B, T, H, Dk, Dv, chunk, stream);
    return dispatch_dk<float>(q, k, v, beta, S0, o, S_T, B, T, H, Dk, Dv, chunk, stream);
}

}  // namespace dr
