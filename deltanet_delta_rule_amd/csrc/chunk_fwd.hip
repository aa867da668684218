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
    // LDS has 64 banks of 4 bytes.  A 16-byte read serves 16 lanes per pass
    // (lanes 0-7 with 24-31, 8-15 with 16-23, and likewise in the upper
    // half), an 8-byte read or transpose read 32 lanes per pass.  Strides of
    // 8*odd dwords make both the 16-byte row-fragment reads (lane r reads row
    // r) and the transpose reads (a 16-lane group reads 4 rows x 32 bytes)
    // conflict-free.  The bf16 K and Q tiles are unpadded and swizzled
    // instead (kq_off).
    static constexpr bool SWZ = sizeof(DT) == 2 && DK >= 32;
    static constexpr int LDK = SWZ ? DK : DK + PADE;   // K, Q
    static constexpr int LDP = C + 2 * PADE;    // P (row fragments)
    static constexpr int LDT = C + 2 * PADE;    // Ti^T (transpose reads)
    static constexpr int LDA = C + 8;           // A (fp32)
    static constexpr int VEC = Vec16<DT>::N;    // elements per 16-byte load
    static constexpr int VPR = DK / VEC;        // 16-byte vectors per K row
    static constexpr int NTHR = 64 * NW;
    static constexpr int NPRE = (C * VPR + NTHR - 1) / NTHR;  // vectors/thread
    static constexpr int NTILE = NT * (NT + 1) / 2;          // lower 16x16 tiles
    static constexpr int LDV = BV + 2 * PADE;   // V tile (transpose reads)
    static constexpr int VPRV = BV / VEC;       // 16-byte vectors per V tile row
    static constexpr int NPREV = (C * VPRV + NTHR - 1) / NTHR;  // V vectors/thread
};

// Row swizzle of the bf16 K and Q tiles: 16-byte chunk c of row t is stored
// at chunk c ^ kq_swz(t).  The masks make each pass of the three access
// patterns of these tiles -- chunk-order row fragments, the transpose reads of
// the state update (state_col order) and the 16-byte staging writes -- touch
// every bank once.
template <int NCH>
__device__ __forceinline__ int kq_swz(int t) {
    const int b0 = t & 1, b1 = (t >> 1) & 1, b2 = (t >> 2) & 1, b3 = (t >> 3) & 1;
    if constexpr (NCH == 16) return b0 | (b1 << 2) | (b2 << 3) | (b3 << 1);
    else if constexpr (NCH == 8) return b1 | (b2 << 2) | (b3 << 1);
    else if constexpr (NCH == 4) return b2 | (b3 << 1);
    else return 0;
}

// Element offset of K[t][e] (or Q[t][e]) in a chunk tile.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ int kq_off(int t, int e) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    if constexpr (G::SWZ) return t * G::LDK + (((e >> 3) ^ kq_swz<DK / 8>(t)) << 3) + (e & 7);
    else return t * G::LDK + e;
}

// Column of token u in the P tile.  P rows are read in the canonical k order
// over tokens (u = 32s + 4g + j and 32s + 16 + 4g + j for lane group g), so
// those eight columns are stored next to each other: one 16-byte read.
template <int KSC>
__device__ __forceinline__ int p_col(int u) {
    if constexpr (KSC == 32) return 32 * (u >> 5) + 8 * ((u >> 2) & 3) + 4 * ((u >> 4) & 1) + (u & 3);
    else return u;
}

template <bool K32, typename DT> struct SlabFrag;
template <typename DT> struct SlabFrag<true, DT> { typedef typename Frag<DT>::k32 type; };
template <typename DT> struct SlabFrag<false, DT> { typedef typename Frag<DT>::k16 type; };

// Row fragment of a K or Q tile over d_k in chunk order (16-byte reads).
template <typename DT, int DK, int C, int NW, typename F>
__device__ __forceinline__ void kq_rows(const DT *M, int row0, int k0, int lane, F &f) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    const int g = lane >> 4, r = lane & 15;
    load_chunk(M + kq_off<DT, DK, C, NW>(row0 + r, k0 + (G::KSD == 32 ? 8 : 4) * g), f);
}

// Row fragment of the P tile in canonical token order (see p_col).
template <typename DT, int DK, int C, int NW, typename F>
__device__ __forceinline__ void p_rows(const DT *Ps, int row0, int k0, int lane, F &f) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    const int g = lane >> 4, r = lane & 15;
    load_chunk(Ps + (row0 + r) * G::LDP + k0 + (G::KSC == 32 ? 8 : 4) * g, f);
}

// K^T fragment for state tile dt over the 16 tokens k0 .. k0 + 15: lane
// (g, r) takes K[k0 + 4g + j][state_col(dt, r / 4) + r % 4], j = 0..3.  For
// bf16 this is one transpose read: lane (g, r) fetches the 4 keys at
// state_col(dt, r % 4) of token k0 + 4g + r / 4, and the hardware hands lane
// r element r % 4 of lanes r / 4, 4 + r / 4, 8 + r / 4, 12 + r / 4.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void kt_frag16(const __bf16 *Ks, int k0, int dt, int lane, bf16x4 &f) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int g = lane >> 4, r = lane & 15;
    const __bf16 *p = Ks + kq_off<DT, DK, C, NW>(k0 + 4 * g + (r >> 2), state_col<G::KSD>(dt, r & 3));
    f = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void kt_frag16(const float *Ks, int k0, int dt, int lane, f32x4_arr &f) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    const int g = lane >> 4, r = lane & 15;
    const int col = state_col<G::KSD>(dt, r >> 2) + (r & 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[j] = Ks[kq_off<DT, DK, C, NW>(k0 + 4 * g + j, col)];
}
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void kt_frag32(const __bf16 *Ks, int k0, int dt, int lane, bf16x8 &f) {
    bf16x4 lo, hi;
    kt_frag16<DT, DK, C, NW>(Ks, k0, dt, lane, lo);
    kt_frag16<DT, DK, C, NW>(Ks, k0 + 16, dt, lane, hi);
    f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void kt_frag32(const float *Ks, int k0, int dt, int lane, f32x8_arr &f) {
    f32x4_arr lo, hi;
    kt_frag16<DT, DK, C, NW>(Ks, k0, dt, lane, lo);
    kt_frag16<DT, DK, C, NW>(Ks, k0 + 16, dt, lane, hi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.v[j] = lo.v[j];
        f.v[4 + j] = hi.v[j];
    }
}

// ---------------------------------------------------------------------------
// Per-chunk building blocks shared by both kernels.
// ---------------------------------------------------------------------------

// Gram tiles of one chunk:
//   Af[i][j] = beta_i (K K^T)_ij for i > j, else 0      (fp32)
//   Ps[i][j] = (Q K^T)_ij for i >= j, else 0             (DT)
// Each 16x16 tile (ti, tj) is computed transposed, D = K_tj X_ti^T (X = K or
// Q), so lane (g, r) ends up with row 16ti + r, columns 16tj + 4g .. + 3: one
// vector store per tile.  Work comes in row jobs: the A-row of tile row ti
// goes to wave ti % NW and the P-row to wave (NT-1-ti) % NW, so with NW = NT
// every wave computes NT+1 tiles.  A job loads all its operand fragments
// before its first MFMA.  Upper tiles of Ps stay zero.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void gram_tiles(const DT *Ks, const DT *Qs, const float *betas,
                                           float *Af, DT *Ps, int wave, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, KSD = G::KSD, NSD = DK / KSD;
    typedef typename SlabFrag<KSD == 32, DT>::type FD;
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int ti = 0; ti < NT; ++ti) {
#pragma unroll
        for (int isP = 0; isP < 2; ++isP) {
            const int owner = isP ? (NT - 1 - ti) % NW : ti % NW;
            if (owner != wave) continue;
            FD fx[NSD], fk[NT][NSD];
#pragma unroll
            for (int s = 0; s < NSD; ++s) kq_rows<DT, DK, C, NW>(isP ? Qs : Ks, 16 * ti, s * KSD, lane, fx[s]);
#pragma unroll
            for (int tj = 0; tj <= ti; ++tj)
#pragma unroll
                for (int s = 0; s < NSD; ++s)
                    kq_rows<DT, DK, C, NW>(Ks, 16 * tj, s * KSD, lane, fk[tj][s]);
            const int row = 16 * ti + r;
            const float brow = betas[row];
#pragma unroll
            for (int tj = 0; tj <= ti; ++tj) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < NSD; ++s) {
                    if constexpr (KSD == 32) mma_k32(acc, fk[tj][s], fx[s]);
                    else mma_k16(acc, fk[tj][s], fx[s]);
                }
                const int col = 16 * tj + 4 * g;  // columns col .. col+3 of row
                if (isP) {
                    typename Frag<DT>::k16 out;
                    f32x4 m;
#pragma unroll
                    for (int e = 0; e < 4; ++e) m[e] = row >= col + e ? acc[e] : 0.f;
                    cvt4(m, out);
                    store_frag16(Ps + row * G::LDP + p_col<G::KSC>(col), out);
                } else {
                    f32x4 out;
#pragma unroll
                    for (int e = 0; e < 4; ++e) out[e] = row > col + e ? brow * acc[e] : 0.f;
                    *reinterpret_cast<f32x4 *>(Af + row * G::LDA + col) = out;
                }
            }
        }
    }
}

// Ti = (I + A)^{-1}, stored transposed: TsT[col][row] = Ti[row][col] (Ti is
// unit lower-triangular, so TsT is upper-triangular; its lower blocks stay
// zero).  Blocked forward substitution by doubling: if T inverts the diagonal
// blocks of size h of (I + A) and A_h holds the entries of A in the blocks of
// size h just below them (rows in the upper half, columns in the lower half
// of each diagonal block of size 2h), then T - T A_h T inverts the diagonal
// blocks of size 2h, since (T A_h)^2 = 0.
//  1. diag_inverse: the 4x4 diagonal blocks by substitution (VALU), then
//     sizes 8 and 16 by doubling on the MFMA units.  A wave inverts the
//     diagonal 16-blocks of the Gram row jobs it owns, right after computing
//     them, so it reads back only its own A tiles.
//  2. offdiag_inverse: sizes 32 and 64 by doubling over 16-blocks, after a
//     barrier.  For a 64-token chunk the six new blocks are split into four
//     self-contained jobs, each recomputing the size-32 blocks it needs.

// A-operand rows of an Af tile (fp32 LDS) narrowed to DT: lane (g, r) takes
// Af[row0 + r][col0 + 4g .. + 3].
template <typename DT, int LDA>
__device__ __forceinline__ void af_rows(const float *Af, int row0, int col0, int lane,
                                        typename Frag<DT>::k16 &f) {
    const int g = lane >> 4, r = lane & 15;
    cvt4(*reinterpret_cast<const f32x4 *>(Af + (row0 + r) * LDA + col0 + 4 * g), f);
}

// Fresh 16x16 product A * B (16-wide k).
template <typename F>
__device__ __forceinline__ f32x4 mm16(const F &a, const F &b) {
    f32x4 acc = zero4();
    mma_k16(acc, a, b);
    return acc;
}

template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void diag_inverse(const float *Af, DT *TsT, int d, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename Frag<DT>::k16 F;
    constexpr int LDA = G::LDA, LDT = G::LDT;
    const int g = lane >> 4, r = lane & 15, c = r & 3;
    const int o = 16 * d;
    // Size 4: lane (g, r) with r / 4 == g takes 4x4 block g and solves for
    // column c of its inverse (x) and for column c of the inverse of its
    // transpose (y), i.e. row c of the inverse.  In D layout these are
    // T[4g + i][r] and T^T[4g + i][r]; every other lane holds zeros.
    float a1[4], a2[4], a3[4], ar[4];
    load4(Af + (o + 4 * g + 1) * LDA + o + 4 * g, a1);
    load4(Af + (o + 4 * g + 2) * LDA + o + 4 * g, a2);
    load4(Af + (o + 4 * g + 3) * LDA + o + 4 * g, a3);
    load4(Af + (o + r) * LDA + o + 4 * g, ar);  // A-operand row r, columns 4g..4g+3
    const float e0 = c == 0 ? 1.f : 0.f, e1 = c == 1 ? 1.f : 0.f;
    const float e2 = c == 2 ? 1.f : 0.f, e3 = c == 3 ? 1.f : 0.f;
    const float x0 = e0, x1 = e1 - a1[0] * x0, x2 = e2 - a2[0] * x0 - a2[1] * x1;
    const float x3 = e3 - a3[0] * x0 - a3[1] * x1 - a3[2] * x2;
    const float y3 = e3, y2 = e2 - a3[2] * y3, y1 = e1 - a2[1] * y2 - a3[1] * y3;
    const float y0 = e0 - a1[0] * y1 - a2[0] * y2 - a3[0] * y3;
    const bool act = (r >> 2) == g;
    f32x4 Tm = act ? f32x4{x0, x1, x2, x3} : zero4();
    f32x4 Tt = act ? f32x4{y0, y1, y2, y3} : zero4();
    // Sizes 8 and 16: M = A_h T, T <- T - T M and T^T <- T^T - M^T T^T.
    // Operands: rows of T are the D layout of T^T and rows of M^T the D
    // layout of M, so both products come straight from registers.
#pragma unroll
    for (int lv = 0; lv < 2; ++lv) {
        const int h = 4 << lv;
        const bool keep = (r / (2 * h) == (4 * g) / (2 * h)) && (r % (2 * h) >= h) &&
                          ((4 * g) % (2 * h) < h);
        F fa, fT, fTt, fM;
        cvt4(keep ? f32x4{ar[0], ar[1], ar[2], ar[3]} : zero4(), fa);
        frag_from_acc16(Tm, fT);
        frag_from_acc16(Tt, fTt);
        f32x4 M = zero4(), P = zero4(), Pt = zero4();
        mma_k16(M, fa, fT);
        frag_from_acc16(M, fM);
        mma_k16(P, fTt, fM);
        mma_k16(Pt, fM, fTt);
        Tm -= P;
        Tt -= Pt;
    }
    // lane (g, r) holds Ti[o + 4g + i][o + r] = TsT[o + r][o + 4g + i]
    F out;
    frag_from_acc16(Tm, out);
    store_frag16(TsT + (o + r) * LDT + o + 4 * g, out);
}

template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void offdiag_inverse(const float *Af, DT *TsT, int wave, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename Frag<DT>::k16 F;
    constexpr int NT = G::NT, LDA = G::LDA, LDT = G::LDT;
    const int g = lane >> 4, r = lane & 15;
    // T_lj as B operand (lane (g, r): T_lj[4g + e][r] = TsT[16j + r][16l + 4g + e])
    auto tB = [&](int l, int j, F &f) { load_chunk(TsT + (16 * j + r) * LDT + 16 * l + 4 * g, f); };
    // rows of T_ik as A operand (lane (g, r): T_ik[r][4g + e] = TsT[16k + 4g + e][16i + r])
    auto tA = [&](int i, int k, F &f) { frag_cols16(TsT, LDT, 16 * k, 16 * i, lane, f); };
    auto aA = [&](int k, int l, F &f) { af_rows<DT, LDA>(Af, 16 * k, 16 * l, lane, f); };
    auto store = [&](int i, int j, const f32x4 &D) {  // D = D layout of -T_ij
        F out;
        cvt4(-D, out);
        store_frag16(TsT + (16 * j + r) * LDT + 16 * i + 4 * g, out);
    };
    // Every job loads all of its operands before its first product (the
    // scheduling barrier keeps the loads from sinking to their uses), then
    // runs its chain of products.  X_ij denotes -T_ij.
    if constexpr (NT == 2) {
        if (wave != 0) return;
        F a10, t00, t11r;
        aA(1, 0, a10); tB(0, 0, t00); tA(1, 1, t11r);
        __builtin_amdgcn_sched_barrier(0);
        F n;
        cvt4(mm16(a10, t00), n);
        store(1, 0, mm16(t11r, n));                       // X10 = T11 A10 T00
    } else if constexpr (NT == 4) {
#pragma unroll
        for (int job = 0; job < 4; ++job) {
            if (job % NW != wave) continue;
            if (job == 0) {  // T10, T20
                F a10, a20, a21, t00, t11r, t22r;
                aA(1, 0, a10); aA(2, 0, a20); aA(2, 1, a21);
                tB(0, 0, t00); tA(1, 1, t11r); tA(2, 2, t22r);
                __builtin_amdgcn_sched_barrier(0);
                F n, t10, m2;
                cvt4(mm16(a10, t00), n);
                const f32x4 X10 = mm16(t11r, n);
                store(1, 0, X10);
                cvt4(-X10, t10);
                f32x4 M2 = mm16(a20, t00);                // A20 T00 + A21 T10
                mma_k16(M2, a21, t10);
                cvt4(M2, m2);
                store(2, 0, mm16(t22r, m2));              // X20 = T22 M2
            } else if (job == 1) {  // T21
                F a21, t11, t22r, m2;
                aA(2, 1, a21); tB(1, 1, t11); tA(2, 2, t22r);
                __builtin_amdgcn_sched_barrier(0);
                cvt4(mm16(a21, t11), m2);                  // A21 T11
                store(2, 1, mm16(t22r, m2));               // X21 = T22 M2
            } else if (job == 2) {  // T32, T31
                F a32, a21, a31, t22, t11, t33r;
                aA(3, 2, a32); aA(2, 1, a21); aA(3, 1, a31);
                tB(2, 2, t22); tB(1, 1, t11); tA(3, 3, t33r);
                __builtin_amdgcn_sched_barrier(0);
                F n, t32r, m2, m3;
                cvt4(mm16(a32, t22), n);
                store(3, 2, mm16(t33r, n));                // X32 = T33 A32 T22
                cvt4(-mm16(n, t33r), t32r);                // rows of T32 (D layout of T32^T)
                cvt4(mm16(a21, t11), m2);
                cvt4(mm16(a31, t11), m3);
                f32x4 Y = mm16(t32r, m2);                  // T32 M2 + T33 M3 = X31
                mma_k16(Y, t33r, m3);
                store(3, 1, Y);
            } else {  // T30, recomputing T10 and T32
                F a10, a32, a20, a21, a30, a31, t00, t22, t11r, t33r;
                aA(1, 0, a10); aA(3, 2, a32); aA(2, 0, a20);
                aA(2, 1, a21); aA(3, 0, a30); aA(3, 1, a31);
                tB(0, 0, t00); tB(2, 2, t22); tA(1, 1, t11r); tA(3, 3, t33r);
                __builtin_amdgcn_sched_barrier(0);
                F n1, n3, t10, t32r, m2, m3;
                cvt4(mm16(a10, t00), n1);
                cvt4(mm16(a32, t22), n3);
                cvt4(-mm16(t11r, n1), t10);               // T10
                cvt4(-mm16(n3, t33r), t32r);               // rows of T32
                f32x4 M2 = mm16(a20, t00), M3 = mm16(a30, t00);
                mma_k16(M2, a21, t10);
                mma_k16(M3, a31, t10);
                cvt4(M2, m2);
                cvt4(M3, m3);
                f32x4 Y = mm16(t32r, m2);                  // T32 M2 + T33 M3 = X30
                mma_k16(Y, t33r, m3);
                store(3, 0, Y);
            }
        }
    }
}

// State path of one chunk for this wave's 16 rows of S:
//   X = K S^T, Y = Q S^T, R = diag(beta)(V - X), E = Ti R,
//   S^T += K^T E, O = Y + P E (stored for tokens < len).
// Output rows of one chunk: a buffer resource over the chunk's valid tokens,
// this lane's byte offset (its value column, rows 4g..) and the token stride.
struct OutChunk {
    __amdgpu_buffer_rsrc_t rsrc;
    int voff, row_bytes;
};

// Operand fragments are loaded into registers ahead of their MFMAs: the Ti
// and P rows first (they do not depend on the state), the K and Q slabs of
// X and Y one slab ahead, the K^T fragments while X and Y run.
template <typename DT, int DK, int C, int NW>
__device__ __forceinline__ void state_path(const DT *Ks, const DT *Qs, const DT *Vs,
                                           const DT *TsT, const DT *Ps, const float *betas,
                                           f32x4 *Sacc, const OutChunk &out, int wave,
                                           int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND, KSD = G::KSD, KSC = G::KSC;
    constexpr int NSD = DK / KSD, NSC = C / KSC;
    typedef typename SlabFrag<KSD == 32, DT>::type FD;
    typedef typename SlabFrag<KSC == 32, DT>::type FC;
    const int g = lane >> 4;

    FC fT[NT][NSC], fP[NT][NSC];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int s = 0; s < NSC; ++s)
            if (s * KSC < 16 * (mt + 1)) {  // Ti and P are lower-triangular
                // Ti row fragment = column fragment of Ti^T
                if constexpr (KSC == 32) frag_cols32(TsT, G::LDT, s * KSC, 16 * mt, lane, fT[mt][s]);
                else frag_cols16(TsT, G::LDT, s * KSC, 16 * mt, lane, fT[mt][s]);
                p_rows<DT, DK, C, NW>(Ps, 16 * mt, s * KSC, lane, fP[mt][s]);
            }
    float bcur[NT][4];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) bcur[mt][i] = betas[16 * mt + 4 * g + i];
    // this wave's V columns in D layout: lane (g, r) takes V[16mt + 4g + j][16w + r]
    typename Frag<DT>::k16 fv[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) frag_cols16(Vs, G::LDV, 16 * mt, 16 * wave, lane, fv[mt]);

    // X = K S^T, Y = Q S^T
    f32x4 X[NT], Y[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) X[mt] = Y[mt] = zero4();
    FD fk[2][NT], fq[2][NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        kq_rows<DT, DK, C, NW>(Ks, 16 * mt, 0, lane, fk[0][mt]);
        kq_rows<DT, DK, C, NW>(Qs, 16 * mt, 0, lane, fq[0][mt]);
    }
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
        const int cur = s & 1;
        if (s + 1 < NSD) {
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                kq_rows<DT, DK, C, NW>(Ks, 16 * mt, (s + 1) * KSD, lane, fk[cur ^ 1][mt]);
                kq_rows<DT, DK, C, NW>(Qs, 16 * mt, (s + 1) * KSD, lane, fq[cur ^ 1][mt]);
            }
        }
        FD fb;
        if constexpr (KSD == 32) frag_from_state(Sacc[2 * s], Sacc[2 * s + 1], g, fb);
        else frag_from_acc16(Sacc[s], fb);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            if constexpr (KSD == 32) {
                mma_k32(X[mt], fk[cur][mt], fb);
                mma_k32(Y[mt], fq[cur][mt], fb);
            } else {
                mma_k16(X[mt], fk[cur][mt], fb);
                mma_k16(Y[mt], fq[cur][mt], fb);
            }
        }
    }
    // K^T fragments for the state update (read through the transpose path)
    FC fkt[ND][NSC];
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
            if constexpr (KSC == 32) kt_frag32<DT, DK, C, NW>(Ks, s * KSC, dt, lane, fkt[dt][s]);
            else kt_frag16<DT, DK, C, NW>(Ks, s * KSC, dt, lane, fkt[dt][s]);
        }
    // R = diag(beta) (V - K S^T), in place in X
#pragma unroll
    for (int mt = 0; mt < NT; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) X[mt][i] = bcur[mt][i] * (frag_get(fv[mt], i) - X[mt][i]);
    // E = Ti R  (slabs past the diagonal are zero and skipped)
    f32x4 E[NT];
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        E[mt] = zero4();
#pragma unroll
        for (int s = 0; s < NSC; ++s)
            if (s * KSC < 16 * (mt + 1)) {
                FC fb;
                if constexpr (KSC == 32) {
                    frag_from_acc32(X[2 * s], X[2 * s + 1], fb);
                    mma_k32(E[mt], fT[mt][s], fb);
                } else {
                    frag_from_acc16(X[s], fb);
                    mma_k16(E[mt], fT[mt][s], fb);
                }
            }
    }
    // B operands built from E, shared by the state update and the output
    FC fe[NSC];
#pragma unroll
    for (int s = 0; s < NSC; ++s) {
        if constexpr (KSC == 32) frag_from_acc32(E[2 * s], E[2 * s + 1], fe[s]);
        else frag_from_acc16(E[s], fe[s]);
    }
    // S^T += K^T E
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
            if constexpr (KSC == 32) mma_k32(Sacc[dt], fkt[dt][s], fe[s]);
            else mma_k16(Sacc[dt], fkt[dt][s], fe[s]);
        }
    // O = Q S^T + P E.  When the slabs over d_k and over tokens have the same
    // MFMA shape, P E accumulates onto Q S^T; otherwise it gets its own
    // accumulator, since an accumulation chain must never switch shape (the
    // compiler issues such a dependent pair back to back and the second one
    // reads a stale accumulator).
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        f32x4 PE = zero4();
        f32x4 &acc = (KSC == KSD) ? Y[mt] : PE;
#pragma unroll
        for (int s = 0; s < NSC; ++s)
            if (s * KSC < 16 * (mt + 1)) {
                if constexpr (KSC == 32) mma_k32(acc, fP[mt][s], fe[s]);
                else mma_k16(acc, fP[mt][s], fe[s]);
            }
        // token 16mt + 4g + i of the chunk; stores past the chunk's last
        // token fall outside the resource and are dropped
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float oi = (KSC == KSD) ? Y[mt][i] : Y[mt][i] + PE[i];
            buf_store_elem(from_f32<DT>(oi), out.rsrc, out.voff, (16 * mt + i) * out.row_bytes);
        }
    }
}

// Common per-workgroup addressing: (b, h, value tile) of this workgroup with
// an XCD-aware remap, and the base pointers of its head.
template <typename DT>
struct HeadPtrs {
    const DT *kh, *qh, *vh, *bh;  // token 0 of the head (vh: first value column of the tile)
    DT *oh;                       // token 0, column 0 of the head's output
    int tsk, tsv, tsb;            // token strides in elements: H*d_k, H*d_v, H
    int64_t sbase;
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
    p.tsk = H * DK;
    p.tsv = H * Dv;
    p.tsb = H;
    p.kh = k + ((int64_t)b * T * H + h) * DK;
    p.qh = q + ((int64_t)b * T * H + h) * DK;
    p.vh = v + ((int64_t)b * T * H + h) * Dv + vt * 16 * NW;
    p.oh = o + ((int64_t)b * T * H + h) * Dv;
    p.bh = beta + (int64_t)b * T * H + h;
    p.sbase = ((int64_t)head * Dv + p.vcol) * DK;
    return p;
}

// Register staging of one chunk's K, Q, V (this workgroup's value columns)
// and beta.  Each tensor is read through a buffer resource that spans exactly
// the chunk's valid tokens, so the tokens past the end of the sequence load as
// zeros (beta = 0 leaves the state unchanged) without any masking, and every
// lane's offsets within a chunk are constants computed once.
template <typename DT, int DK, int C, int NW>
struct ChunkRegs {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename Vec16<DT>::type vec_t;
    static constexpr int OUT = 0x7ffffff0;  // offset past any resource: loads 0
    vec_t k[G::NPRE], q[G::NPRE], v[G::NPREV];
    DT b;
    int offk[G::NPRE], offv[G::NPREV], offb;

    __device__ __forceinline__ void init(const HeadPtrs<DT> &p, int tid) {
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            const int idx = tid + j * G::NTHR;
            const int t = idx / G::VPR, e0 = (idx % G::VPR) * G::VEC;
            offk[j] = idx < C * G::VPR ? (t * p.tsk + e0) * (int)sizeof(DT) : OUT;
        }
#pragma unroll
        for (int j = 0; j < G::NPREV; ++j) {
            const int idx = tid + j * G::NTHR;
            const int t = idx / G::VPRV, e0 = (idx % G::VPRV) * G::VEC;
            offv[j] = idx < C * G::VPRV ? (t * p.tsv + e0) * (int)sizeof(DT) : OUT;
        }
        offb = tid < C ? tid * p.tsb * (int)sizeof(DT) : OUT;
    }
    __device__ __forceinline__ void load(const HeadPtrs<DT> &p, int T, int t0) {
        const int len = min(C, T - t0);
        const int esz = (int)sizeof(DT);
        const auto rk = make_rsrc(p.kh + (int64_t)t0 * p.tsk, len * p.tsk * esz);
        const auto rq = make_rsrc(p.qh + (int64_t)t0 * p.tsk, len * p.tsk * esz);
        const auto rv = make_rsrc(p.vh + (int64_t)t0 * p.tsv, len * p.tsv * esz);
        const auto rb = make_rsrc(p.bh + (int64_t)t0 * p.tsb, len * p.tsb * esz);
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            k[j] = buf_load16<vec_t>(rk, offk[j]);
            q[j] = buf_load16<vec_t>(rq, offk[j]);
        }
#pragma unroll
        for (int j = 0; j < G::NPREV; ++j) v[j] = buf_load16<vec_t>(rv, offv[j]);
        b = buf_load_elem<DT>(rb, offb);
    }
    // Write into one LDS buffer set.
    __device__ __forceinline__ void stage(DT *Ks, DT *Qs, DT *Vs, float *betas, int tid) const {
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            const int idx = tid + j * G::NTHR;
            if (idx < C * G::VPR) {
                const int t = idx / G::VPR, e0 = (idx % G::VPR) * G::VEC;
                const int off = kq_off<DT, DK, C, NW>(t, e0);
                *reinterpret_cast<vec_t *>(Ks + off) = k[j];
                *reinterpret_cast<vec_t *>(Qs + off) = q[j];
            }
        }
#pragma unroll
        for (int j = 0; j < G::NPREV; ++j) {
            const int idx = tid + j * G::NTHR;
            if (idx < C * G::VPRV) {
                const int t = idx / G::VPRV, e0 = (idx % G::VPRV) * G::VEC;
                *reinterpret_cast<vec_t *>(Vs + t * G::LDV + e0) = v[j];
            }
        }
        if (tid < C) betas[tid] = to_f32(b);
    }
};

// ---------------------------------------------------------------------------
// Pipelined kernel
// ---------------------------------------------------------------------------
template <typename DT, int DK, int C, int NW>
struct PipeSmem {
    typedef ChunkCfg<DT, DK, C, NW> G;
    DT Ks[2][C * G::LDK];          // K, token-major (double-buffered)
    DT Qs[2][C * G::LDK];          // Q, token-major
    DT Vs[2][C * G::LDV];          // V, this workgroup's value columns
    DT TsT[2][C * G::LDT];         // ((I + A)^{-1})^T
    DT Ps[2][C * G::LDP];          // Q K^T (.) M
    float Af[C * G::LDA];          // A = beta (K K^T) strictly lower, fp32
    float betas[2][C];
};

template <typename DT, int DK, int C, int NW>
constexpr bool pipelined_fits() {
    return sizeof(PipeSmem<DT, DK, C, NW>) <= 160 * 1024;
}

template <typename DT, int DK, int C, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_fwd_pipelined_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *S0, DT *__restrict__ o, float *S_T,
    int T, int H, int Dv, int nvt) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    __shared__ __attribute__((aligned(16))) PipeSmem<DT, DK, C, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int g = lane >> 4, r = lane & 15;
    const HeadPtrs<DT> p = head_ptrs<DT, DK, NW>(q, k, v, beta, o, T, H, Dv, nvt, wave, r);

    f32x4 Sacc[ND];
    if (S0) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            Sacc[dt] = *reinterpret_cast<const f32x4 *>(S0 + p.sbase + state_col<G::KSD>(dt, g));
    } else {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) Sacc[dt] = zero4();
    }

    const int N = (T + C - 1) / C;
    if (N > 0) {
        // Lower blocks of TsT and upper blocks of Ps stay zero for the whole
        // sequence.
        for (int i = tid; i < 2 * C * G::LDT; i += G::NTHR) (&sm.TsT[0][0])[i] = from_f32<DT>(0.f);
        for (int i = tid; i < 2 * C * G::LDP; i += G::NTHR) (&sm.Ps[0][0])[i] = from_f32<DT>(0.f);
        ChunkRegs<DT, DK, C, NW> rg;
        rg.init(p, tid);
        OutChunk out;
        out.voff = (4 * g * p.tsv + p.vcol) * (int)sizeof(DT);
        out.row_bytes = p.tsv * (int)sizeof(DT);
        // prologue: chunks 0 and 1 staged, chunk 0 solved, chunk 2 in flight
        rg.load(p, T, 0);
        rg.stage(sm.Ks[0], sm.Qs[0], sm.Vs[0], sm.betas[0], tid);
        rg.load(p, T, min(1, N - 1) * C);
        rg.stage(sm.Ks[1], sm.Qs[1], sm.Vs[1], sm.betas[1], tid);
        rg.load(p, T, min(2, N - 1) * C);
        lds_barrier();
        gram_tiles<DT, DK, C, NW>(sm.Ks[0], sm.Qs[0], sm.betas[0], sm.Af, sm.Ps[0], wave, lane);
        wave_lds_fence();
        for (int d = wave; d < NT; d += NW) diag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT[0], d, lane);
        lds_barrier();
        offdiag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT[0], wave, lane);
        lds_barrier();

        for (int c = 0; c < N; ++c) {
            const int b = c & 1, b1 = b ^ 1;
            const int t0 = c * C;
            const int len = min(C, T - t0);
            // ---- phase 1: state path of chunk c, Gram tiles of chunk c+1 ----
            out.rsrc = make_rsrc(p.oh + (int64_t)t0 * p.tsv, len * out.row_bytes);
            state_path<DT, DK, C, NW>(sm.Ks[b], sm.Qs[b], sm.Vs[b], sm.TsT[b], sm.Ps[b],
                                      sm.betas[b], Sacc, out, wave, lane);
            // (past the last chunk this works on stale buffers; never read)
            gram_tiles<DT, DK, C, NW>(sm.Ks[b1], sm.Qs[b1], sm.betas[b1], sm.Af, sm.Ps[b1],
                                      wave, lane);
            wave_lds_fence();
            for (int d = wave; d < NT; d += NW)
                diag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT[b1], d, lane);
            lds_barrier();
            // ---- phase 2: rest of the inverse of chunk c+1, staging of chunk c+2 ----
            offdiag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT[b1], wave, lane);
            rg.stage(sm.Ks[b], sm.Qs[b], sm.Vs[b], sm.betas[b], tid);
            rg.load(p, T, min(c + 3, N - 1) * C);
            lds_barrier();
        }
    }
    if (S_T) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            *reinterpret_cast<f32x4 *>(S_T + p.sbase + state_col<G::KSD>(dt, g)) = Sacc[dt];
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
    DT Vs[C * G::LDV];
    DT TsT[C * G::LDT];
    DT Ps[C * G::LDP];
    float Af[C * G::LDA];
    float betas[C];
};

template <typename DT, int DK, int C, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_fwd_serial_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *S0, DT *__restrict__ o, float *S_T,
    int T, int H, int Dv, int nvt) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    __shared__ __attribute__((aligned(16))) SerialSmem<DT, DK, C, NW> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int g = lane >> 4, r = lane & 15;
    const HeadPtrs<DT> p = head_ptrs<DT, DK, NW>(q, k, v, beta, o, T, H, Dv, nvt, wave, r);

    f32x4 Sacc[ND];
    if (S0) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            Sacc[dt] = *reinterpret_cast<const f32x4 *>(S0 + p.sbase + state_col<G::KSD>(dt, g));
    } else {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) Sacc[dt] = zero4();
    }

    const int N = (T + C - 1) / C;
    if (N > 0) {
        for (int i = tid; i < C * G::LDT; i += G::NTHR) sm.TsT[i] = from_f32<DT>(0.f);
        for (int i = tid; i < C * G::LDP; i += G::NTHR) sm.Ps[i] = from_f32<DT>(0.f);
        ChunkRegs<DT, DK, C, NW> rg;
        rg.init(p, tid);
        OutChunk out;
        out.voff = (4 * g * p.tsv + p.vcol) * (int)sizeof(DT);
        out.row_bytes = p.tsv * (int)sizeof(DT);
        rg.load(p, T, 0);
        for (int c = 0; c < N; ++c) {
            const int t0 = c * C;
            const int len = min(C, T - t0);
            lds_barrier();
            rg.stage(sm.Ks, sm.Qs, sm.Vs, sm.betas, tid);
            lds_barrier();
            rg.load(p, T, min(c + 1, N - 1) * C);
            gram_tiles<DT, DK, C, NW>(sm.Ks, sm.Qs, sm.betas, sm.Af, sm.Ps, wave, lane);
            wave_lds_fence();
            for (int d = wave; d < NT; d += NW) diag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT, d, lane);
            lds_barrier();
            offdiag_inverse<DT, DK, C, NW>(sm.Af, sm.TsT, wave, lane);
            lds_barrier();
            out.rsrc = make_rsrc(p.oh + (int64_t)t0 * p.tsv, len * out.row_bytes);
            state_path<DT, DK, C, NW>(sm.Ks, sm.Qs, sm.Vs, sm.TsT, sm.Ps, sm.betas, Sacc, out,
                                      wave, lane);
        }
    }
    if (S_T) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            *reinterpret_cast<f32x4 *>(S_T + p.sbase + state_col<G::KSD>(dt, g)) = Sacc[dt];
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
