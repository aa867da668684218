// Fused chunkwise-parallel forward of the delta rule (gfx950).
//
// Math (per head; chunk c spans C tokens with incoming state S_c, d_v x d_k):
//   A   = tril(diag(beta) K K^T, -1)                     chunk key couplings
//   R   = diag(beta) (V - K S_c^T)                       provisional errors
//   E   = (I + A)^{-1} R                                 resolved errors
//   O   = Q S_c^T + (Q K^T (.) M) E                       M incl. the diagonal
//   S_{c+1} = S_c + E^T K
// The pieces come from the paperlayer summary of arXiv:2406.06484 (section 3
// "Parallelizing DeltaNet Across the Sequence Dimension": chunking, the
// Householder/WY representation, forward substitution with the unit
// lower-triangular matrix; App. B.2 "UT transform derivation": T = (I +
// A)^{-1} diag(beta)) and the hada.io digest (section "Chunkwise KDA":
// provisional errors against the incoming state, the unit lower-triangular
// solve that restores the causal coupling, the end-of-chunk state as one
// product and the outputs with the diagonal included; section "Pipeline
// Triton Chunkwise": 16-token diagonal blocks solved first, then the blocks
// below them).  With D = I and no output scale this is plain DeltaNet.  E is
// U - W S_c^T of the UT form; the kernel solves for it from the residual
// instead of forming W = T K and U = T V, which skips the C x C x d_k product
// for W, and it does the solve by 16-token blocks: the diagonal blocks of
// (I + A) are inverted once per chunk, and each block of E is one product
// with its inverse after the blocks above it are subtracted.
//
// Gated rule (houmin.site "infra/delta-net", section "Gated DeltaNet"; hada.io
// digest, section "Gated DeltaNet"): every token first scales the state by
// alpha_t = exp(g_t).  With b the in-chunk prefix sums of g, the same steps
// hold with the decays folded in (hada.io digest, sections "Chunkwise KDA"
// with a scalar decay and "Pipeline Triton Chunkwise"):
//   A_ij = beta_i (k_i . k_j) exp(b_i - b_j),  P_ij = (q_i . k_j) exp(b_i - b_j)
//   R    = diag(beta) (V - diag(exp(b)) K S_c^T),  O = diag(exp(b)) Q S_c^T + P E
//   S_{c+1} = exp(b_last) S_c + E^T diag(exp(b_last - b)) K
// The decays multiply the Gram tiles once, where they are made, so the state
// path only rescales X, Y, the state and E before the state update.
//
// Work split.  One workgroup owns one (b, h) and a tile of BV = 16*NW value
// rows of S and walks the chunks in order, so the state never leaves the chip.
// A state wave owns 16 rows of S as fp32 MFMA accumulators (lane (g, r) holds
// S[row r][state_col(dt, g) + i]).  Rows of S evolve independently, so waves
// never exchange state: every product on the state path (K S^T, S Q^T, the
// block substitution, E^T P^T, K^T E) runs inside one wave from registers,
// using the D-layout-as-operand identity of dr_common.hpp; K^T fragments come
// from the token-major K tile through the LDS transpose read.  The per-chunk
// work that does not depend on the state -- the Gram tiles K K^T and Q K^T
// and the inverses of the diagonal blocks of (I + A) -- is shared through LDS.
//
// Two kernels implement this:
//  * chunk_fwd_ws_kernel (used whenever its buffers fit in LDS) pairs each
//    state wave with a preparation wave on the same SIMD, with one barrier
//    per chunk;
//  * chunk_fwd_serial_kernel runs the same steps one after the other on single
//    buffers (fp32 inputs with large d_k * chunk, whose double buffers would
//    exceed the 160 KiB of LDS).
#pragma once

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
    static constexpr int VEC = Vec16<DT>::N;    // elements per 16-byte load
    static constexpr int VPR = DK / VEC;        // 16-byte vectors per K row
    static constexpr int NTHR = 64 * NW;
    static constexpr int NPRE = (C * VPR + NTHR - 1) / NTHR;  // vectors/thread
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
// Per-chunk building blocks
// ---------------------------------------------------------------------------

// Fragment blocks.  A 16x16 matrix that some wave uses as a 16-wide MFMA
// operand is kept in LDS "fragment-major": lane l's four elements at
// 4l .. 4l+3, so writing and reading a block are both one linear 8-byte (bf16)
// or 16-byte (fp32) access per lane.  Block (i, j) of the strictly lower
// couplings, i > j, is block number i(i-1)/2 + j.
constexpr int off_idx(int i, int j) { return i * (i - 1) / 2 + j; }
constexpr int FRAG_ELEMS = 256;  // 64 lanes x 4 elements

template <typename DT>
__device__ __forceinline__ void store_fragblk(DT *base, int blk, int lane, const f32x4 &x) {
    typename Frag<DT>::k16 f;
    cvt4(x, f);
    store_frag16(base + blk * FRAG_ELEMS + 4 * lane, f);
}
template <typename DT>
__device__ __forceinline__ void load_fragblk(const DT *base, int blk, int lane,
                                             typename Frag<DT>::k16 &f) {
    load_chunk(base + blk * FRAG_ELEMS + 4 * lane, f);
}

// Inverse T_dd = (I + A_dd)^{-1} of a diagonal 16x16 block of the couplings
// (unit lower-triangular), from the block in registers: lane (g, r) holds
// A_dd[r][4g + e] (strictly lower, zero elsewhere), the A-operand fragment.
// Blocked forward substitution by doubling: if T inverts the diagonal blocks
// of size h of (I + A) and A_h holds the entries of A in the blocks of size h
// just below them (rows in the lower half, columns in the upper half of each
// diagonal block of size 2h), then T - T A_h T inverts the diagonal blocks of
// size 2h, since (T A_h)^2 = 0.  Starting from T = I, four such steps (h = 1,
// 2, 4, 8) on the MFMA units give the 16x16 inverse.  T is kept in D layout
// both as T and as T^T: rows of T are the D layout of T^T and rows of M^T the
// D layout of M, so every product comes straight from registers.  The result
// goes to Tb as the fragment block of T_dd as an A operand.
template <typename F>
__device__ __forceinline__ f32x4 mm16(const F &a, const F &b) {
    f32x4 acc = zero4();
    mma_k16(acc, a, b);
    return acc;
}

template <typename DT>
__device__ __forceinline__ void diag_inverse(const f32x4 &a, const f32x4 &b4, DT *Tb, int d,
                                             int lane) {
    typedef typename Frag<DT>::k16 F;
    const int g = lane >> 4, r = lane & 15;
    f32x4 Tm, Tt;  // T[4g + i][r] and T^T[4g + i][r]
#pragma unroll
    for (int i = 0; i < 4; ++i) Tm[i] = Tt[i] = (4 * g + i == r) ? 1.f : 0.f;
#pragma unroll
    for (int lv = 0; lv < 4; ++lv) {
        const int h = 1 << lv;
        f32x4 ah;  // A_h: entry (r, 4g + e) of A
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int col = 4 * g + e;
            const bool keep = (r / (2 * h) == col / (2 * h)) && (r % (2 * h) >= h) &&
                              (col % (2 * h) < h);
            ah[e] = keep ? a[e] : 0.f;
        }
        F fa, fT, fTt, fM;
        cvt4(ah, fa);
        frag_from_acc16(Tm, fT);
        frag_from_acc16(Tt, fTt);
        const f32x4 M = mm16(fa, fT);  // A_h T
        frag_from_acc16(M, fM);
        Tm -= mm16(fTt, fM);           // T M
        Tt -= mm16(fM, fTt);           // M^T T^T
    }
    // lane (g, r) holds T^T[4g + i][r] = T[r][4g + i]: row r, columns 4g ..
    // 4g + 3, the A-operand fragment of T_dd.  Stored as -T_dd diag(beta_d)
    // (b4: beta of columns 4g .. 4g + 3), the form the block substitution
    // uses (state_rest).
    store_fragblk(Tb, d, lane, -(Tt * b4));
}

// Per-chunk decay of the gated rule (hada.io digest, "Pipeline Triton
// Chunkwise": differences of in-chunk prefix sums of the log gate stand for
// the decay between two tokens), kept in LDS next to the chunk's betas:
//   bc[t]  = b_t = g_0 + ... + g_t      (log decay from the chunk start)
//   gam[t] = exp(b_t)                    (decay of the incoming state at t)
//   rto[t] = exp(b_last - b_t)           (decay of token t's write to the end)
// Tokens past the end of the sequence load g = 0, so b stays at the last
// valid token's value and b_last is that token's.
template <int C>
struct alignas(16) GateLds {
    float bc[C], gam[C], rto[C];
};

// One wave (lane = token, lanes >= C idle) turns the chunk's log gates into
// GateLds: an inclusive prefix sum across the wave, then the two exponentials.
template <int C>
__device__ __forceinline__ void write_gate(GateLds<C> &gs, float g, int lane) {
    float x = lane < C ? g : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    const float bl = __shfl(x, C - 1, 64);
    if (lane < C) {
        gs.bc[lane] = x;
        gs.gam[lane] = __expf(x);
        gs.rto[lane] = __expf(bl - x);
    }
}

// NS gate buffers in LDS for the gated rule; nothing for the plain rule.
template <int C, int NS, bool GATED>
struct GateSets {
    GateLds<C> s[NS];
    __device__ __forceinline__ GateLds<C> *at(int i) { return &s[i]; }
};
template <int C, int NS>
struct GateSets<C, NS, false> {
    __device__ __forceinline__ GateLds<C> *at(int) { return nullptr; }
};

// In-kernel L2 normalisation of q and k (L2): per-token inverse norms
// 1/sqrt(|x|^2 + eps), the l2norm of the gated layer on houmin.site
// ("infra/delta-net", section "Gated DeltaNet", code).  |k_t|^2 is the
// diagonal of the chunk's K K^T tiles and |q_t|^2 that of a Q Q^T product
// per 16-token tile; the kernel never rewrites q or k but applies the norms
// as row scalings:
//   A      = diag(beta nk) G diag(nk) on the diagonal blocks (their inverses),
//            raw G = K K^T off the diagonal,
//   F_j    = diag(nk_j) E_j replaces E_j as the operand of every product,
//   X_i    <- diag(nk_i) (K_i S^T + sum_{j<i} G_ij F_j) - V_i before the
//            block product with -T_ii diag(beta_i),
//   O      = diag(nq) (Q S^T + P F),   S^T += K^T F,
// which is the chunk form on the normalised q and k.  Two buffers (chunk
// parity), like the Gram products that carry them.
constexpr float L2_EPS = 1e-6f;

template <int C>
struct alignas(16) NormLds {
    float nk[C], nq[C];  // 1/|k_t|, 1/|q_t|
};
template <int C, int NS, bool L2>
struct NormSets {
    NormLds<C> s[NS];
    __device__ __forceinline__ NormLds<C> *at(int i) { return &s[i]; }
};
template <int C, int NS>
struct NormSets<C, NS, false> {
    __device__ __forceinline__ NormLds<C> *at(int) { return nullptr; }
};

// Inverse norm of token 16 ti + r from a 16x16 Gram tile of a matrix with
// itself (lane (g, r) holds entries (r, 4g + e)): lanes with 4g <= r < 4g + 4
// hold the diagonal entry; the result is valid in those lanes only.
__device__ __forceinline__ float diag_inv_norm(const f32x4 &acc, int lane, bool &own) {
    const int g = lane >> 4, r = lane & 15, e0 = r - 4 * g;
    float d = acc[0];
    d = e0 == 1 ? acc[1] : d;
    d = e0 == 2 ? acc[2] : d;
    d = e0 == 3 ? acc[3] : d;
    own = e0 >= 0 && e0 < 4;
    return rsqrtf(d + L2_EPS);
}

// Gram tiles of one chunk, for the rows of the Gram jobs of wave W:
//   A-row job ti:  the K K^T tiles of row ti.  The diagonal tile, scaled
//                  to A = tril(diag(beta) K K^T, -1), is inverted right away
//                  from registers (diag_inverse, into Tb); the tiles left of
//                  it go unscaled to Ab as fragment blocks G_ij = (K K^T)_ij,
//                  the A operands of the block substitution.
//   P-row job ti:  P = (Q K^T)_ij for i >= j into Ps (DT, masked).
// Each 16x16 tile (ti, tj) is computed transposed, D = K_tj X_ti^T (X = K or
// Q), so lane (g, r) ends up with row 16ti + r, columns 16tj + 4g .. + 3:
// exactly the A-operand fragment of that tile.  The A-row of tile row ti goes
// to wave ti % NW and the P-row to wave (NT-1-ti) % NW (with NW = NT every
// wave computes NT+1 tiles).  The assignment is fixed at compile time per
// wave; a wave loads every K tile its jobs touch once, plus the Q tiles of its
// P rows, all before its first MFMA, and does its A rows first so that the
// chain of its diagonal inverse overlaps the products of its P rows.
template <int NT, int NW, int W, bool NOOUT = false>
struct GramJobs {
    static constexpr bool a_row(int ti) { return ti % NW == W; }
    // P = Q K^T is needed only for the outputs
    static constexpr bool p_row(int ti) { return !NOOUT && (NT - 1 - ti) % NW == W; }
    static constexpr int kmax() {
        int m = -1;
        for (int ti = 0; ti < NT; ++ti)
            if (a_row(ti) || p_row(ti)) m = ti;
        return m;
    }
};

template <int NT, int NW, int W, bool NOOUT = false>
constexpr int n_prows() {
    int n = 0;
    for (int ti = 0; ti < NT; ++ti) n += GramJobs<NT, NW, W, NOOUT>::p_row(ti) ? 1 : 0;
    return n;
}

// One Gram tile (ti, tj) from its operand fragments, written where its job
// needs it.
// Gated rule: every tile is multiplied elementwise by the decay between its
// row and column tokens, exp(b_row - b_col) (bc: the chunk's prefix sums),
// which turns K K^T into the decayed couplings and Q K^T into the decayed
// reads of the pages' chunked form.
template <typename DT, int DK, int C, int NW, bool GATED, bool L2, typename FD>
__device__ __forceinline__ void gram_tile(const FD *fkj, const FD *fx, bool isP, int ti, int tj,
                                          float brow, const float *betas, const float *bc,
                                          DT *Ab, DT *Tb, DT *Ps, NormLds<C> *nl, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int KSD = G::KSD, NSD = DK / KSD;
    const int g = lane >> 4, r = lane & 15;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
        if constexpr (KSD == 32) mma_k32(acc, fkj[s], fx[s]);
        else mma_k16(acc, fkj[s], fx[s]);
    }
    const int row = 16 * ti + r;
    const int col = 16 * tj + 4 * g;  // columns col .. col+3 of row
    if constexpr (GATED) {
        const float brw = bc[row];
        const f32x4 bcl = *reinterpret_cast<const f32x4 *>(bc + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= __expf(brw - bcl[e]);
    }
    // (above the diagonal the ratio may overflow; those entries are selected
    // away below, never used)
    if (isP) {
        typename Frag<DT>::k16 out;
        f32x4 m;
#pragma unroll
        for (int e = 0; e < 4; ++e) m[e] = row >= col + e ? acc[e] : 0.f;
        cvt4(m, out);
        store_frag16(Ps + row * G::LDP + p_col<G::KSC>(col), out);
    } else if (tj == ti) {
        f32x4 a;
        const f32x4 b4 = *reinterpret_cast<const f32x4 *>(betas + col);
        if constexpr (L2) {
            // the diagonal of G gives |k|^2 of the tile's tokens (its decay
            // factor is exactly 1); normalise the block on both sides
            bool own;
            const float nk = diag_inv_norm(acc, lane, own);
            const float nr = __shfl(nk, 16 * (r >> 2) + r, 64);  // token row
            f32x4 nc;                                              // tokens col + e
#pragma unroll
            for (int e = 0; e < 4; ++e) nc[e] = __shfl(nk, 20 * g + e, 64);
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = row > col + e ? brow * nr * nc[e] * acc[e] : 0.f;
            if (own) nl->nk[row] = nk;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) a[e] = row > col + e ? brow * acc[e] : 0.f;
        }
        diag_inverse(a, b4, Tb, ti, lane);
    } else {
        store_fragblk(Ab, off_idx(ti, tj), lane, acc);
    }
}

// 1/|q| of the 16 tokens of tile ti from the diagonal of Q_ti Q_ti^T (L2).
template <typename DT, int DK, int C, int NW, typename FD>
__device__ __forceinline__ void q_norms(const FD *fq, int ti, NormLds<C> *nl, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int KSD = G::KSD, NSD = DK / KSD;
    f32x4 acc = zero4();
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
        if constexpr (KSD == 32) mma_k32(acc, fq[s], fq[s]);
        else mma_k16(acc, fq[s], fq[s]);
    }
    bool own;
    const float nq = diag_inv_norm(acc, lane, own);
    if (own) nl->nq[16 * ti + (lane & 15)] = nq;
}

// When the fragments of all the wave's jobs fit in 96 VGPRs they are loaded
// once, before the first MFMA; otherwise each job loads its own.
template <typename DT, int DK, int C, int NW, int W, bool GATED, bool L2, bool NOOUT = false>
__device__ __forceinline__ void gram_tiles_w(const DT *Ks, const DT *Qs, const float *betas,
                                             const float *bc, DT *Ab, DT *Tb, DT *Ps,
                                             NormLds<C> *nl, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef GramJobs<G::NT, NW, W, NOOUT> J;
    constexpr int NT = G::NT, KSD = G::KSD, NSD = DK / KSD, KM = J::kmax();
    typedef typename SlabFrag<KSD == 32, DT>::type FD;
    constexpr bool ALL = (KM + 1 + n_prows<NT, NW, W, NOOUT>()) * NSD * sizeof(FD) <= 384;
    const int r = lane & 15;
    float brow[NT];
#pragma unroll
    for (int ti = 0; ti < NT; ++ti)
        if (J::a_row(ti)) brow[ti] = betas[16 * ti + r];
    if constexpr (ALL) {
        FD fk[NT][NSD], fq[NT][NSD];
#pragma unroll
        for (int tj = 0; tj < NT; ++tj)
            if (tj <= KM)
#pragma unroll
                for (int s = 0; s < NSD; ++s) kq_rows<DT, DK, C, NW>(Ks, 16 * tj, s * KSD, lane, fk[tj][s]);
#pragma unroll
        for (int ti = 0; ti < NT; ++ti)
            if (J::p_row(ti))
#pragma unroll
                for (int s = 0; s < NSD; ++s) kq_rows<DT, DK, C, NW>(Qs, 16 * ti, s * KSD, lane, fq[ti][s]);
#pragma unroll
        for (int isP = 0; isP < 2; ++isP)
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                if (!(isP ? J::p_row(ti) : J::a_row(ti))) continue;
                if constexpr (L2)
                    if (isP) q_norms<DT, DK, C, NW>(fq[ti], ti, nl, lane);
#pragma unroll
                for (int tj = 0; tj <= ti; ++tj)
                    gram_tile<DT, DK, C, NW, GATED, L2>(fk[tj], isP ? fq[ti] : fk[ti], isP, ti, tj,
                                                        isP ? 0.f : brow[ti], betas, bc, Ab, Tb,
                                                        Ps, nl, lane);
            }
    } else {
#pragma unroll
        for (int isP = 0; isP < 2; ++isP)
#pragma unroll
            for (int ti = 0; ti < NT; ++ti) {
                if (!(isP ? J::p_row(ti) : J::a_row(ti))) continue;
                FD fx[NSD];
#pragma unroll
                for (int s = 0; s < NSD; ++s) kq_rows<DT, DK, C, NW>(isP ? Qs : Ks, 16 * ti, s * KSD, lane, fx[s]);
                if constexpr (L2)
                    if (isP) q_norms<DT, DK, C, NW>(fx, ti, nl, lane);
#pragma unroll
                for (int tj = 0; tj <= ti; ++tj) {
                    FD fk[NSD];
#pragma unroll
                    for (int s = 0; s < NSD; ++s) kq_rows<DT, DK, C, NW>(Ks, 16 * tj, s * KSD, lane, fk[s]);
                    gram_tile<DT, DK, C, NW, GATED, L2>(fk, fx, isP, ti, tj, isP ? 0.f : brow[ti],
                                                        betas, bc, Ab, Tb, Ps, nl, lane);
                }
            }
    }
}

template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
__device__ __forceinline__ void gram_tiles(const DT *Ks, const DT *Qs, const float *betas,
                                           const float *bc, DT *Ab, DT *Tb, DT *Ps,
                                           NormLds<C> *nl, int wave, int lane) {
    switch (wave) {
    case 0: gram_tiles_w<DT, DK, C, NW, 0, GATED, L2>(Ks, Qs, betas, bc, Ab, Tb, Ps, nl, lane); break;
    case 1: if constexpr (NW > 1) gram_tiles_w<DT, DK, C, NW, 1, GATED, L2>(Ks, Qs, betas, bc, Ab, Tb, Ps, nl, lane); break;
    case 2: if constexpr (NW > 2) gram_tiles_w<DT, DK, C, NW, 2, GATED, L2>(Ks, Qs, betas, bc, Ab, Tb, Ps, nl, lane); break;
    default: if constexpr (NW > 3) gram_tiles_w<DT, DK, C, NW, 3, GATED, L2>(Ks, Qs, betas, bc, Ab, Tb, Ps, nl, lane); break;
    }
}

// Output rows of one chunk: a buffer resource over the chunk's valid tokens,
// this lane's byte offset (its token row r and value columns 4g ..) and the
// token stride.
struct OutChunk {
    __amdgpu_buffer_rsrc_t rsrc;
    int voff, row_bytes;
    float scale;  // output scale (1: none)
};

// Four consecutive output elements of one token row (8 bytes for bf16, 16 for
// fp32), times the output scale; stores outside the resource are dropped by
// its range check.
__device__ __forceinline__ void store_out4(const f32x4 &x, const OutChunk &out, int soff) {
    bf16x4 f;
    cvt4(x * out.scale, f);
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned, f),
                                          out.rsrc, out.voff, soff, 0);
}
// A buffer store of more than 8 bytes still reads its data registers in the
// cycle after issue, so the next instruction must not overwrite them.  The
// compiler inserts that wait state only for stores whose scalar offset field
// is zero (it assumes none is needed with a register there), and the fp32
// parity grid caught an output register rewritten right after such a store.
// The whole offset therefore goes into the per-lane offset.
__device__ __forceinline__ void store_out4_f32(const f32x4 &x, const OutChunk &out, int soff) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) unsigned,
                                                              x * out.scale),
                                           out.rsrc, out.voff + soff, 0, 0);
}

// The state path of one chunk for this wave's 16 rows of S, in two halves so
// that a pipeline can put the products over d_k of the next chunk right after
// the state update of this one:
//   state_xy:   X = K S^T - V (tokens x rows), Y = S Q^T (rows x tokens)
//   state_rest: E by block forward substitution, S^T += K^T E,
//               O^T = Y + E^T P^T (stored for valid tokens)
// Y and the output are computed transposed so that a lane holds four
// consecutive value columns of one token, which it stores with one access.
// Gated rule: X starts at zero, and gate_xy applies the decays and -V after
// the products (V is then loaded after them, which keeps its fragments out of
// the products' live range).
// NOOUT (no outputs wanted): Y is left at zero and Q is not read.
template <typename DT, int DK, int C, int NW, bool GATED, bool L2, bool NOOUT = false>
__device__ __forceinline__ void state_xy(const DT *Ks, const DT *Qs, const f32x4 *Sacc,
                                         const typename Frag<DT>::k16 *fv, f32x4 *X, f32x4 *Y,
                                         int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, KSD = G::KSD;
    constexpr int NSD = DK / KSD;
    typedef typename SlabFrag<KSD == 32, DT>::type FD;
    const int g = lane >> 4;
    // X accumulates onto -V: X = K S^T - V (gated: onto zero, see below)
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        Y[mt] = zero4();
#pragma unroll
        for (int i = 0; i < 4; ++i) X[mt][i] = (GATED || L2) ? 0.f : -frag_get(fv[mt], i);
    }
    // All operand fragments are loaded before the first MFMA when they fit in
    // 128 VGPRs; otherwise they are double-buffered one slab ahead.
    constexpr bool ALL = (NOOUT ? 1 : 2) * NSD * NT * sizeof(FD) <= 512;
    constexpr int NB = ALL ? NSD : 2;
    FD fk[NB][NT], fq[NOOUT ? 1 : NB][NT];
#pragma unroll
    for (int s = 0; s < (ALL ? NSD : 1); ++s)
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            kq_rows<DT, DK, C, NW>(Ks, 16 * mt, s * KSD, lane, fk[s][mt]);
            if constexpr (!NOOUT) kq_rows<DT, DK, C, NW>(Qs, 16 * mt, s * KSD, lane, fq[s][mt]);
        }
#pragma unroll
    for (int s = 0; s < NSD; ++s) {
        const int cur = ALL ? s : (s & 1);
        if (!ALL && s + 1 < NSD) {
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                kq_rows<DT, DK, C, NW>(Ks, 16 * mt, (s + 1) * KSD, lane, fk[cur ^ 1][mt]);
                if constexpr (!NOOUT)
                    kq_rows<DT, DK, C, NW>(Qs, 16 * mt, (s + 1) * KSD, lane, fq[cur ^ 1][mt]);
            }
        }
        FD fb;  // rows of S: B operand of X, A operand of Y
        if constexpr (KSD == 32) frag_from_state(Sacc[2 * s], Sacc[2 * s + 1], g, fb);
        else frag_from_acc16(Sacc[s], fb);
#pragma unroll
        for (int mt = 0; mt < NT; ++mt) {
            if constexpr (KSD == 32) {
                mma_k32(X[mt], fk[cur][mt], fb);
                if constexpr (!NOOUT) mma_k32(Y[mt], fb, fq[NOOUT ? 0 : cur][mt]);
            } else {
                mma_k16(X[mt], fk[cur][mt], fb);
                if constexpr (!NOOUT) mma_k16(Y[mt], fb, fq[NOOUT ? 0 : cur][mt]);
            }
        }
    }
}

// Gated rule (gam: the chunk's decay from its start): the incoming state is
// read through the decay, X = diag(gam) K S^T - V and Y = S Q^T diag(gam).
// With SUBV false (L2) the V term is left to the block substitution.
template <typename DT, int C, int NT, bool SUBV>
__device__ __forceinline__ void gate_xy(const typename Frag<DT>::k16 *fv, const float *gam,
                                        f32x4 *X, f32x4 *Y, int lane) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        // X rows are tokens 16mt + 4g + i, Y columns token 16mt + r
        const f32x4 gx = *reinterpret_cast<const f32x4 *>(gam + 16 * mt + 4 * g);
        const float gy = gam[16 * mt + r];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            X[mt][i] = SUBV ? gx[i] * X[mt][i] - frag_get(fv[mt], i) : gx[i] * X[mt][i];
            Y[mt][i] *= gy;
        }
    }
}

// Operands that come from the chunk's K and V tiles: the K^T fragments of the
// state update and this wave's V columns in D layout.  Loading them ahead
// frees those tiles early.
template <typename DT, int DK, int C, int NW>
struct ChunkOperands {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename SlabFrag<G::KSC == 32, DT>::type FC;
    FC fkt[G::ND][C / G::KSC];
    typename Frag<DT>::k16 fv[G::NT];

    // lane (g, r) takes V[16mt + 4g + j][16 vtile + r]
    __device__ __forceinline__ void load_v(const DT *Vs, int vtile, int lane) {
#pragma unroll
        for (int mt = 0; mt < G::NT; ++mt) frag_cols16(Vs, G::LDV, 16 * mt, 16 * vtile, lane, fv[mt]);
    }
    __device__ __forceinline__ void load_kt(const DT *Ks, int lane) {
        constexpr int ND = G::ND, KSC = G::KSC, NSC = C / KSC;
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
#pragma unroll
            for (int s = 0; s < NSC; ++s) {
                if constexpr (KSC == 32) kt_frag32<DT, DK, C, NW>(Ks, s * KSC, dt, lane, fkt[dt][s]);
                else kt_frag16<DT, DK, C, NW>(Ks, s * KSC, dt, lane, fkt[dt][s]);
            }
    }
};

// Two 16-wide fragments as one 32-wide fragment (k order of the 32-wide slab).
__device__ __forceinline__ void cat16(const bf16x4 &a, const bf16x4 &b, bf16x8 &f) {
    f = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void cat16(const f32x4_arr &a, const f32x4_arr &b, f32x8_arr &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = a.v[i];
        f.v[4 + i] = b.v[i];
    }
}

// E solves (I + A) E = R, R = diag(beta)(V - K S^T), block by block
// (16-token blocks i).  With A_ij = diag(beta_i) G_ij, G = K K^T and
// T_ii = (I + A_ii)^{-1}:
//   E_i = T_ii diag(beta_i) (V_i - X_i - sum_{j<i} G_ij E_j)
//       = (-T_ii diag(beta_i)) (X'_i + sum_{j<i} G_ij E_j),   X' = K S^T - V
// so the products G_ij E_j accumulate onto X' in place and each block costs
// one more product with the stored -T_ii diag(beta_i) (Tb); G_ij comes from
// Ab.  X'_i and E_j enter as B operands straight from their D layout (tokens
// along k).  No beta and no residual arithmetic remain on the state path.
// Gated rule (ga: the chunk's GateLds): A, T and P already carry the in-chunk
// decay and X, Y the decay from the chunk start, so the substitution and the
// outputs are unchanged; the state update becomes
//   S^T <- gam_last S^T + K^T diag(rto) E
// with its own copy of the E fragments (the outputs need the unscaled E).
// NOOUT: the outputs (and the reads of P) are skipped.
template <typename DT, int DK, int C, int NW, bool GATED, bool L2, bool NOOUT = false>
__device__ __forceinline__ void state_rest(const ChunkOperands<DT, DK, C, NW> &op,
                                           const DT *Ab, const DT *Tb, const DT *Ps,
                                           const GateLds<C> *ga, const NormLds<C> *nl,
                                           f32x4 *Sacc, f32x4 *X, f32x4 *Y, const OutChunk &out,
                                           int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND, KSD = G::KSD, KSC = G::KSC;
    constexpr int NSC = C / KSC, NOFF = NT * (NT - 1) / 2;
    typedef typename SlabFrag<KSC == 32, DT>::type FC;
    typedef typename Frag<DT>::k16 F16;

    F16 ft[NT], fa[NOFF > 0 ? NOFF : 1];
#pragma unroll
    for (int i = 0; i < NT; ++i) load_fragblk(Tb, i, lane, ft[i]);
#pragma unroll
    for (int i = 0; i < NOFF; ++i) load_fragblk(Ab, i, lane, fa[i]);
    FC fP[NOOUT ? 1 : NT][NSC];
    if constexpr (!NOOUT) {
#pragma unroll
        for (int mt = 0; mt < NT; ++mt)
#pragma unroll
            for (int s = 0; s < NSC; ++s)
                if (s * KSC < 16 * (mt + 1))  // P is lower-triangular
                    p_rows<DT, DK, C, NW>(Ps, 16 * mt, s * KSC, lane, fP[mt][s]);
    }
    // block forward substitution
    f32x4 E[NT];
    F16 fe16[NT], fs16[GATED ? NT : 1];
#pragma unroll
    for (int i = 0; i < NT; ++i) {
#pragma unroll
        for (int j = 0; j < i; ++j) mma_k16(X[i], fa[off_idx(i, j)], fe16[j]);
        // rows of X[i] and E[i] are tokens 16i + 4g .. 16i + 4g + 3
        f32x4 nk4;
        if constexpr (L2) {
            nk4 = *reinterpret_cast<const f32x4 *>(nl->nk + 16 * i + 4 * (lane >> 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) X[i][e] = nk4[e] * X[i][e] - frag_get(op.fv[i], e);
        }
        F16 fr;
        frag_from_acc16(X[i], fr);
        E[i] = mm16(ft[i], fr);
        if constexpr (L2) E[i] *= nk4;  // F_i, the operand form of E_i
        frag_from_acc16(E[i], fe16[i]);
        if constexpr (GATED) {
            const f32x4 rt = *reinterpret_cast<const f32x4 *>(ga->rto + 16 * i + 4 * (lane >> 4));
            frag_from_acc16(E[i] * rt, fs16[i]);
        }
    }
    // B operands over 32-token slabs, shared by the state update and the output
    // (gated: first the decayed fs16 for the update, then fe16)
    FC fe[NSC];
    auto slabs = [&](const F16 *f16) {
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
            if constexpr (KSC == 32) cat16(f16[2 * s], f16[2 * s + 1], fe[s]);
            else fe[s] = f16[s];
        }
    };
    slabs(GATED ? fs16 : fe16);
    if constexpr (GATED) {
        const float gl = ga->gam[C - 1];
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) Sacc[dt] *= gl;
    }
    // S^T += K^T E
#pragma unroll
    for (int dt = 0; dt < ND; ++dt)
#pragma unroll
        for (int s = 0; s < NSC; ++s) {
            if constexpr (KSC == 32) mma_k32(Sacc[dt], op.fkt[dt][s], fe[s]);
            else mma_k16(Sacc[dt], op.fkt[dt][s], fe[s]);
        }
    if constexpr (NOOUT) return;
    if constexpr (GATED) slabs(fe16);
    // O^T = S Q^T + E^T P^T.  When the slabs over d_k and over tokens have the
    // same MFMA shape, E^T P^T accumulates onto S Q^T; otherwise it gets its
    // own accumulator, since an accumulation chain must never switch shape
    // (the compiler issues such a dependent pair back to back and the second
    // one reads a stale accumulator).
#pragma unroll
    for (int mt = 0; mt < NT; ++mt) {
        f32x4 PE = zero4();
        f32x4 &acc = (KSC == KSD) ? Y[mt] : PE;
#pragma unroll
        for (int s = 0; s < NSC; ++s)
            if (s * KSC < 16 * (mt + 1)) {
                if constexpr (KSC == 32) mma_k32(acc, fe[s], fP[NOOUT ? 0 : mt][s]);
                else mma_k16(acc, fe[s], fP[NOOUT ? 0 : mt][s]);
            }
        // lane (g, r): token 16mt + r, value columns 4g .. 4g + 3
        f32x4 o4 = (KSC == KSD) ? Y[mt] : Y[mt] + PE;
        if constexpr (L2) o4 *= nl->nq[16 * mt + (lane & 15)];
        if constexpr (sizeof(DT) == 2) store_out4(o4, out, 16 * mt * out.row_bytes);
        else store_out4_f32(o4, out, 16 * mt * out.row_bytes);
    }
}

// Both halves back to back (single-buffered kernel).
template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
__device__ __forceinline__ void state_path(const DT *Ks, const DT *Qs, const DT *Vs,
                                           const DT *Ab, const DT *Tb, const DT *Ps,
                                           const GateLds<C> *ga, const NormLds<C> *nl,
                                           f32x4 *Sacc, const OutChunk &out, int wave, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    f32x4 X[G::NT], Y[G::NT];
    ChunkOperands<DT, DK, C, NW> op;
    if constexpr (!GATED && !L2) op.load_v(Vs, wave, lane);
    state_xy<DT, DK, C, NW, GATED, L2>(Ks, Qs, Sacc, op.fv, X, Y, lane);
    if constexpr (GATED || L2) op.load_v(Vs, wave, lane);
    if constexpr (GATED) gate_xy<DT, C, G::NT, !L2>(op.fv, ga->gam, X, Y, lane);
    op.load_kt(Ks, lane);
    state_rest<DT, DK, C, NW, GATED, L2>(op, Ab, Tb, Ps, ga, nl, Sacc, X, Y, out, lane);
}

// A state tile row (this lane's row r, keys in state_col order) to row-major
// memory at `row` (the row's first element), in DT (the checkpoints of the
// backward, which uses them only as DT product operands).
template <int KSD, int ND, typename DT>
__device__ __forceinline__ void store_state_row(DT *row, const f32x4 *Sacc, int g) {
    if constexpr (sizeof(DT) == 2 && KSD == 32) {
        // tiles 2m, 2m + 1 hold keys 32m + 8g .. 32m + 8g + 7 between them:
        // one 16-byte store per pair
#pragma unroll
        for (int m = 0; m < ND / 2; ++m) {
            bf16x8 f;
            frag_from_state(Sacc[2 * m], Sacc[2 * m + 1], g, f);
            *reinterpret_cast<bf16x8 *>(row + 32 * m + 8 * g) = f;
        }
        return;
    }
#pragma unroll
    for (int dt = 0; dt < ND; ++dt) {
        if constexpr (sizeof(DT) == 4) {
            *reinterpret_cast<f32x4 *>(row + state_col<KSD>(dt, g)) = Sacc[dt];
        } else {
            *reinterpret_cast<u32x2 *>(row + state_col<KSD>(dt, g)) = pk4_bf16(Sacc[dt]);
        }
    }
}

// Common per-workgroup addressing: (b, h, value tile) of this workgroup with
// an XCD-aware remap, and the base pointers of its head.
template <typename DT>
struct HeadPtrs {
    const DT *kh, *qh, *vh, *bh;  // token 0 of the head (vh: first value column of the tile)
    const float *gh;              // token 0 of the head's log forget gate (gated rule)
    DT *oh;                       // token 0, column 0 of the head's output
    int tsk, tsv, tsb;            // token strides in elements: H*d_k, H*d_v, H
    int T;                        // tokens of this sequence
    int64_t head;                 // sequence * H + head
    int64_t sbase;
    int vcol;
    bool vz;                      // v == nullptr: every value loads as zero
};

// Packed variable-length input (cu != nullptr): sequence b spans tokens
// cu[b] .. cu[b+1] of the single batch row of T tokens; the bounds are
// clamped into [0, T] so that no access leaves the buffers whatever cu holds.
// Sequence b of the launch: batch row b (tokens b T ..), packed sequence b
// (cu), or, with segL > 0, segment b % segP of batch row b / segP (tokens
// (b % segP) segL .. of that row, at most segL of them).
template <typename DT, int DK, int NW>
__device__ __forceinline__ HeadPtrs<DT> head_ptrs(const DT *q, const DT *k, const DT *v,
                                                  const DT *beta, const float *gl, DT *o,
                                                  const int *cu, int T, int H, int Dv, int nvt,
                                                  int wave, int r, int segP = 0, int segL = 0) {
    // Consecutive workgroup ids are dispatched round-robin over the 8 XCDs
    // (each with its own L2).  Remap so that the value tiles of one head,
    // which read the same K and Q, run on the same XCD.
    int wg = blockIdx.x;
    const int nwg = gridDim.x;
    if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
    const int head = wg / nvt, vt = wg % nvt;
    const int b = head / H, h = head % H;
    HeadPtrs<DT> p;
    int64_t t0 = (int64_t)b * T;  // first token of the sequence in the token axis
    p.T = T;
    if (cu) {
        const int lo = min(max(cu[b], 0), T);
        const int hi = min(max(cu[b + 1], lo), T);
        t0 = lo;
        p.T = hi - lo;
    } else if (segL > 0) {
        const int lo = min((b % segP) * segL, T), hi = min(lo + segL, T);
        t0 = (int64_t)(b / segP) * T + lo;
        p.T = hi - lo;
    }
    p.vcol = vt * 16 * NW + wave * 16 + r;
    p.tsk = H * DK;
    p.tsv = H * Dv;
    p.tsb = H;
    p.kh = k + (t0 * H + h) * DK;
    p.qh = q + (t0 * H + h) * DK;
    p.vh = v + (t0 * H + h) * Dv + vt * 16 * NW;
    p.oh = o + (t0 * H + h) * Dv;
    p.bh = beta + t0 * H + h;
    p.gh = gl ? gl + t0 * H + h : nullptr;
    p.head = head;
    p.sbase = ((int64_t)head * Dv + p.vcol) * DK;
    p.vz = v == nullptr;
    return p;
}

// Register staging of one chunk's K, Q, V (this workgroup's value columns)
// and beta.  Each tensor is read through a buffer resource that spans exactly
// the chunk's valid tokens, so the tokens past the end of the sequence load as
// zeros (beta = 0 leaves the state unchanged) without any masking, and every
// lane's offsets within a chunk are constants computed once.
template <typename DT, int DK, int C, int NW, bool GATED>
struct ChunkRegs {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef typename Vec16<DT>::type vec_t;
    static constexpr int OUT = 0x7ffffff0;  // offset past any resource: loads 0
    vec_t k[G::NPRE], q[G::NPRE], v[G::NPREV];
    DT b;
    float gv;  // log gate of token tid (gated rule; 0 past the end)
    int offk[G::NPRE], offv[G::NPREV], offb, offg;

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
        offg = tid < C ? tid * p.tsb * (int)sizeof(float) : OUT;
    }
    // A chunk that starts at or past the end of the sequence gets empty
    // resources: its loads return zeros and touch no memory.
    __device__ __forceinline__ void load(const HeadPtrs<DT> &p, int T, int t0) {
        const int len = max(0, min(C, T - t0));
        const int esz = (int)sizeof(DT);
        const auto rk = make_rsrc(p.kh + (int64_t)t0 * p.tsk, len * p.tsk * esz);
        const auto rq = make_rsrc(p.qh + (int64_t)t0 * p.tsk, len * p.tsk * esz);
        const auto rv = make_rsrc(p.vh + (int64_t)t0 * p.tsv, p.vz ? 0 : len * p.tsv * esz);
        const auto rb = make_rsrc(p.bh + (int64_t)t0 * p.tsb, len * p.tsb * esz);
#pragma unroll
        for (int j = 0; j < G::NPRE; ++j) {
            k[j] = buf_load16<vec_t>(rk, offk[j]);
            q[j] = buf_load16<vec_t>(rq, offk[j]);
        }
#pragma unroll
        for (int j = 0; j < G::NPREV; ++j) v[j] = buf_load16<vec_t>(rv, offv[j]);
        b = buf_load_elem<DT>(rb, offb);
        if constexpr (GATED) {
            const auto rg = make_rsrc(p.gh + (int64_t)t0 * p.tsb, len * p.tsb * (int)sizeof(float));
            gv = buf_load_elem<float>(rg, offg);
        }
    }
    // Write into one LDS buffer set (wave 0 also turns the gates into ga).
    __device__ __forceinline__ void stage(DT *Ks, DT *Qs, DT *Vs, float *betas, GateLds<C> *ga,
                                          int tid) const {
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
        if constexpr (GATED)
            if (tid < 64) write_gate(*ga, gv, tid);
    }
};

// Direct global-to-LDS staging of one chunk's K, Q and V tiles (the LDS
// form of a buffer load: 64 lanes x 16 bytes land at an LDS base + 16 lane,
// for every lane, whatever the execution mask).  Instruction j of a tile
// fills 16-byte units 64j .. 64j + 63 of the tile as it is laid out in LDS
// (rows of LD elements, K and Q rows swizzled), so each lane's global offset
// encodes the layout.  Tile buffers are rounded up to whole KiB; units in a
// row's padding or past the tile load from past the resource (zeros), and a
// chunk that ends early loads zeros for its missing tokens.  The K, Q, V
// instructions of a chunk are dealt round-robin to the NW preparation waves;
// wave W's share is fixed at compile time, so the number of loads it has in
// flight is a constant.  Without outputs (NOQ) no product reads Q, so its
// tiles are not loaded.
// Per-token scalars of one chunk in flight to LDS (wave 0 loads them).
template <typename DT>
struct TokScalars {
    DT b;     // beta of token lane
    float g;  // log gate of token lane (gated rule)
};

template <typename DT, int DK, int C, int NW, int W, bool GATED = false, bool NOQ = false>
struct DmaStage {
    typedef ChunkCfg<DT, DK, C, NW> G;
    static constexpr int ESZ = (int)sizeof(DT);
    static constexpr int OUT = 0x7ffffff0;  // offset past any resource: loads 0
    static constexpr int UPR_K = G::LDK * ESZ / 16, NU_K = C * UPR_K, NI_K = (NU_K + 63) / 64;
    static constexpr int UPR_V = G::LDV * ESZ / 16, NU_V = C * UPR_V, NI_V = (NU_V + 63) / 64;
    static constexpr int KTILE = NI_K * 1024 / ESZ, VTILE = NI_V * 1024 / ESZ;  // buffer sizes
    static constexpr int NI_Q = NOQ ? 0 : NI_K;               // Q instructions
    static constexpr int NI = NI_K + NI_Q + NI_V;             // instructions per chunk: K, Q, V
    static constexpr int NMINE = (NI - W + NW - 1) / NW;      // this wave's: j = W, W + NW, ...
    static constexpr int NVMEM = NMINE + (W == 0 ? 1 + GATED : 0);  // + beta, g (wave 0)
    static_assert(G::LDK * ESZ % 16 == 0 && G::LDV * ESZ % 16 == 0, "16-byte units");
    int off[NMINE > 0 ? NMINE : 1];
    int offb, offg;

    __device__ __forceinline__ void init(const HeadPtrs<DT> &p, int lane) {
#pragma unroll
        for (int i = 0; i < NMINE; ++i) {
            const int j = W + i * NW;
            const bool isv = j >= NI_K + NI_Q;
            const int jj = isv ? j - NI_K - NI_Q : (j < NI_K ? j : j - NI_K);
            const int upr = isv ? UPR_V : UPR_K;
            const int u = 64 * jj + lane;
            const int t = u / upr, cu = u % upr;
            const int ec = cu * (16 / ESZ);
            const int data = isv ? G::BV : DK;
            int e = ec;
            if (!isv && G::SWZ) e = (cu ^ kq_swz<DK / 8>(t)) * 8;
            off[i] = (t < C && ec < data) ? (t * (isv ? p.tsv : p.tsk) + e) * ESZ : OUT;
        }
        offb = lane < C ? lane * p.tsb * ESZ : OUT;
        offg = lane < C ? lane * p.tsb * (int)sizeof(float) : OUT;
    }
    // Issue the loads of chunk m (tokens mC ..) into one K, Q, V buffer set;
    // beta (and g) of that chunk go to registers.
    __device__ __forceinline__ void issue(const HeadPtrs<DT> &p, int T, int m, DT *Ks, DT *Qs,
                                          DT *Vs, TokScalars<DT> &ts, int lane) const {
        typedef __attribute__((address_space(3))) void lds_void;
        const int t0 = m * C;
        const int len = max(0, min(C, T - t0));
        const auto rk = make_rsrc(p.kh + (int64_t)t0 * p.tsk, len * p.tsk * ESZ);
        const auto rq = make_rsrc(p.qh + (int64_t)t0 * p.tsk, len * p.tsk * ESZ);
        const auto rv = make_rsrc(p.vh + (int64_t)t0 * p.tsv, p.vz ? 0 : len * p.tsv * ESZ);
#pragma unroll
        for (int i = 0; i < NMINE; ++i) {
            const int j = W + i * NW;
            const bool isv = j >= NI_K + NI_Q, isq = !isv && j >= NI_K;
            const int jj = isv ? j - NI_K - NI_Q : (isq ? j - NI_K : j);
            DT *dst = (isv ? Vs : isq ? Qs : Ks) + jj * (1024 / ESZ);
            const auto &rs = isv ? rv : isq ? rq : rk;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void *)dst, 16, off[i], 0, 0, 0);
        }
        if (W == 0) {
            const auto rb = make_rsrc(p.bh + (int64_t)t0 * p.tsb, len * p.tsb * ESZ);
            ts.b = buf_load_elem<DT>(rb, offb);
            if constexpr (GATED) {
                const auto rg = make_rsrc(p.gh + (int64_t)t0 * p.tsb,
                                          len * p.tsb * (int)sizeof(float));
                ts.g = buf_load_elem<float>(rg, offg);
            }
        }
    }
};

// Wait until at most N of this wave's vector-memory operations are in flight
// (the counter holds at most 63; a smaller count only waits longer).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N < 63 ? N : 63) : "memory");
}

// Buffer index of a chunk period as a type, for unrolled loops.
template <int B>
struct Parity {
    static constexpr int value = B;
};

// Byte offset of this lane's first output element within a chunk: token row
// r, value columns 4g .. 4g + 3 of this wave's 16 columns.
template <typename DT>
__device__ __forceinline__ OutChunk out_chunk(const HeadPtrs<DT> &p, float scale, int g, int r) {
    OutChunk out;
    out.scale = scale;
    out.voff = (r * p.tsv + (p.vcol - r) + 4 * g) * (int)sizeof(DT);
    out.row_bytes = p.tsv * (int)sizeof(DT);
    return out;
}

// ---------------------------------------------------------------------------
// Warp-specialised kernel
// ---------------------------------------------------------------------------
// LDS of one workgroup: K, Q, V (this workgroup's value columns) and beta of
// three chunks (one being consumed, two landing), and the per-chunk products
// the preparation waves hand to the state waves for two chunks.
template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
struct PipeSmem {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef DmaStage<DT, DK, C, NW, 0> D;
    static constexpr int NOFF = G::NT * (G::NT - 1) / 2;
    DT Ks[3][D::KTILE];                      // K, token-major (whole KiB)
    DT Qs[3][D::KTILE];                      // Q, token-major
    DT Vs[3][D::VTILE];                      // V, this workgroup's value columns
    DT Ps[2][C * G::LDP];                    // Q K^T (.) M
    DT Ab[2][(NOFF > 0 ? NOFF : 1) * FRAG_ELEMS];  // G_ij = (K K^T)_ij, i > j (fragment blocks)
    DT Tb[2][G::NT * FRAG_ELEMS];            // -T_ii diag(beta_i) (fragment blocks)
    float betas[3][C];
    GateSets<C, 3, GATED> gate;              // decays of the chunk in each K, Q, V set
    NormSets<C, 2, L2> norm;                 // 1/|k|, 1/|q| (L2), buffers like Ab, Tb, Ps
};

template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
constexpr bool ws_fits() {
    return sizeof(PipeSmem<DT, DK, C, NW, GATED, L2>) <= 160 * 1024;
}

// Preparation wave W.  Chunk m's K, Q, V go to buffer set m % 3 by DMA issued
// two periods before the period that reads them; its Gram tiles and diagonal
// inverses go to buffers m & 1.  In the period of chunk c the wave issues the
// loads of chunk c+3 (into the set chunk c has just vacated), computes the
// Gram tiles and diagonal inverses of chunk c+1, waits for the loads of chunk
// c+2 and publishes them at the barrier.
template <typename DT, int DK, int C, int NW, int W, bool GATED, bool L2, bool NOOUT = false>
__device__ __forceinline__ void prep_role(PipeSmem<DT, DK, C, NW, GATED, L2> &sm,
                                          const HeadPtrs<DT> &p, int T, int N, int lane) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    typedef DmaStage<DT, DK, C, NW, W, GATED, NOOUT> D;
    D dma;
    dma.init(p, lane);
    const int ptid = 64 * W + lane;
    // upper blocks of Ps stay zero for the whole sequence
    for (int i = ptid; i < 2 * C * G::LDP; i += G::NTHR) (&sm.Ps[0][0])[i] = from_f32<DT>(0.f);
    // per-token scalars of chunks in flight (tq[m & 1] holds chunk m + 2)
    TokScalars<DT> t0s, t1s, tq[2];
    // wave 0 publishes a landed chunk's betas (and decays) into set s
    auto publish = [&](int s, const TokScalars<DT> &ts) {
        if (W == 0) {
            if (lane < C) sm.betas[s][lane] = to_f32(ts.b);
            if constexpr (GATED) write_gate(*sm.gate.at(s), ts.g, lane);
        }
    };
    auto bc_of = [&](int s) -> const float * {
        if constexpr (GATED) return sm.gate.at(s)->bc;
        else return nullptr;
    };
    dma.issue(p, T, 0, sm.Ks[0], sm.Qs[0], sm.Vs[0], t0s, lane);
    dma.issue(p, T, 1, sm.Ks[1], sm.Qs[1], sm.Vs[1], t1s, lane);
    dma.issue(p, T, 2, sm.Ks[2], sm.Qs[2], sm.Vs[2], tq[0], lane);
    wait_vmcnt<2 * D::NVMEM>();  // chunk 0 landed
    publish(0, t0s);
    lds_barrier();  // chunk 0 staged
    if (N > 0)
        gram_tiles_w<DT, DK, C, NW, W, GATED, L2, NOOUT>(sm.Ks[0], sm.Qs[0], sm.betas[0], bc_of(0),
                                                  sm.Ab[0], sm.Tb[0], sm.Ps[0], sm.norm.at(0),
                                                  lane);
    wait_vmcnt<D::NVMEM>();  // chunk 1 landed
    publish(1, t1s);
    lds_barrier();  // Gram tiles of chunk 0 done, chunk 1 staged
    auto period = [&](int c, auto parity, TokScalars<DT> &tcur, TokScalars<DT> &tnext) {
        constexpr int b1p = decltype(parity)::value ^ 1;
        const int s0 = c % 3, s1 = (c + 1) % 3, s2 = (c + 2) % 3;
        dma.issue(p, T, c + 3, sm.Ks[s0], sm.Qs[s0], sm.Vs[s0], tnext, lane);
        if (c + 1 < N)
            gram_tiles_w<DT, DK, C, NW, W, GATED, L2, NOOUT>(sm.Ks[s1], sm.Qs[s1], sm.betas[s1],
                                                      bc_of(s1), sm.Ab[b1p], sm.Tb[b1p],
                                                      sm.Ps[b1p], sm.norm.at(b1p), lane);
        wait_vmcnt<D::NVMEM>();  // chunk c+2 landed
        publish(s2, tcur);
        lds_barrier();
    };
    for (int c = 0; c < N; c += 2) {
        period(c, Parity<0>(), tq[0], tq[1]);
        if (c + 1 < N) period(c + 1, Parity<1>(), tq[1], tq[0]);
    }
    // the loads of the last chunks (past the sequence: nothing) drain here
    wait_vmcnt<0>();
}

// 2*NW waves: waves 0 .. NW-1 are state waves (wave w owns value rows
// 16w .. 16w+15 of the workgroup's tile and keeps them in registers), waves
// NW .. 2NW-1 are preparation waves (input staging by DMA, Gram tiles,
// diagonal inverses).  Each SIMD runs one wave of each role, so the latency
// of one role's LDS reads and MFMA chains hides behind the other's issue
// (with NW <= 2 the waves spread over distinct SIMDs and may use all their
// registers).  One barrier per chunk; in the period of chunk c:
//
//   state: the block substitution, S^T += K^T E and the outputs of chunk c
//          (X, Y and the K^T operands already in registers; A, T and P
//          blocks from buffers c & 1); then V, X = K S^T - V, Y = S Q^T and
//          the K^T operands of chunk c+1 (K, Q, V set (c+1) % 3)
//   prep:  loads of chunk c+3 into set c % 3; Gram tiles and diagonal
//          inverses of chunk c+1 (set (c+1) % 3 -> buffers (c+1) & 1); wait
//          for chunk c+2 (set (c+2) % 3)
//
// Within a period the state waves read only A, T, P buffers c & 1 and K, Q, V
// set (c+1) % 3, and the preparation waves write only the others.
//
// Gated rule (GATED, gl = log gates [B,T,H]): wave 0 of the preparation waves
// also loads each chunk's gates and publishes their decays with its betas.
//
// NOOUT: a launch without outputs (o == nullptr: the checkpoint pass of the
// backward, the state passes of the segment-parallel schedule) skips every
// product that only the outputs need (P = Q K^T, Y = S Q^T, E^T P^T).
//
// PAIR (with NOOUT, plain or gated rule, d_v = d_k): a second group of NW
// state waves carries d_k rows of the chunk walk's transition map beside the
// workgroup's value rows, on the same loaded K, gates, Gram tiles and
// inverses: the map's rows run the same recurrence with v = 0 from the
// identity and are written to Mst (3 NW waves, three per SIMD).
template <typename DT, int DK, int C, int NW, bool GATED, bool L2, bool NOOUT = false,
          bool PAIR = false>
__global__ __launch_bounds__((PAIR ? 192 : 128) * NW) __attribute__((amdgpu_waves_per_eu(PAIR ? 3 : NW / 4 + 1, PAIR ? 3 : NW / 4 + 1))) void chunk_fwd_ws_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ gl, const float *S0,
    DT *__restrict__ o, float *S_T, DT *__restrict__ hs, const int *__restrict__ cu, int T,
    int H, int Dv, int nvt, float scale, float *Mst, int segP, int segL) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int NT = G::NT, ND = G::ND;
    constexpr int NSW = (PAIR ? 2 : 1) * NW;  // state waves
    static_assert(!PAIR || (NOOUT && !L2), "map rows: no outputs, no in-kernel norm");
    __shared__ __attribute__((aligned(16))) PipeSmem<DT, DK, C, NW, GATED, L2> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int g = lane >> 4, r = lane & 15;

    if (wave < NSW) {
        // ------------------------------ state waves ------------------------------
        const bool mrow = PAIR && wave >= NW;  // rows of the transition map
        const int sw = mrow ? wave - NW : wave;
        if (mrow) {
            v = nullptr;
            S0 = nullptr;
            S_T = Mst;
            Dv = DK;
        }
        const HeadPtrs<DT> p =
            head_ptrs<DT, DK, NW>(q, k, v, beta, gl, o, cu, T, H, Dv, nvt, sw, r, segP, segL);
        const int N = (p.T + C - 1) / C;
        f32x4 Sacc[ND], X[NT], Y[NT];
        ChunkOperands<DT, DK, C, NW> op;
        if (mrow) {
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) op.fv[mt] = typename Frag<DT>::k16{};
            // the map starts as the identity: row vcol of this lane
            const int row = p.vcol;
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    Sacc[dt][i] = state_col<G::KSD>(dt, g) + i == row ? 1.f : 0.f;
        } else if (S0) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
                Sacc[dt] = *reinterpret_cast<const f32x4 *>(S0 + p.sbase + state_col<G::KSD>(dt, g));
        } else {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt) Sacc[dt] = zero4();
        }
        OutChunk out = out_chunk(p, scale, g, r);
        lds_barrier();  // chunk 0 staged
        // X, Y and the K^T operands of the chunk in set s
        // (L2: V stays in op.fv for the block substitution of that chunk)
        auto xy = [&](int s) {
            if constexpr (!GATED && !L2)
                if (!mrow) op.load_v(sm.Vs[s], sw, lane);
            state_xy<DT, DK, C, NW, GATED, L2, NOOUT>(sm.Ks[s], sm.Qs[s], Sacc, op.fv, X, Y, lane);
            if constexpr (GATED || L2)
                if (!mrow) op.load_v(sm.Vs[s], sw, lane);
            if constexpr (GATED) gate_xy<DT, C, NT, !L2>(op.fv, sm.gate.at(s)->gam, X, Y, lane);
            op.load_kt(sm.Ks[s], lane);
        };
        if (N > 0) xy(0);
        lds_barrier();  // Gram tiles of chunk 0 done, chunk 1 staged
        // the loop is unrolled by three so that the K, Q, V set index is a
        // constant (these tiles take most of the state waves' LDS reads)
        auto period = [&](int c, auto set) {
            constexpr int s0 = decltype(set)::value, s1 = (s0 + 1) % 3;  // sets of chunks c, c+1
            const int b = c & 1;
            const int t0 = c * C;
            const int len = o ? min(C, p.T - t0) : 0;
            out.rsrc = make_rsrc(p.oh + (int64_t)t0 * p.tsv, len * out.row_bytes);
            if (hs) store_state_row<G::KSD, ND>(hs + ((p.head * N + c) * Dv + p.vcol) * DK, Sacc, g);
            state_rest<DT, DK, C, NW, GATED, L2, NOOUT>(op, sm.Ab[b], sm.Tb[b], sm.Ps[b],
                                                        sm.gate.at(s0), sm.norm.at(b), Sacc, X, Y,
                                                        out, lane);
            // V first (X starts at -V); the K^T fragments of the next state
            // update only after X and Y have used their operands
            if (c + 1 < N) xy(s1);
            lds_barrier();
        };
        for (int c = 0; c < N; c += 3) {
            period(c, Parity<0>());
            if (c + 1 < N) period(c + 1, Parity<1>());
            if (c + 2 < N) period(c + 2, Parity<2>());
        }
        if (S_T) {
#pragma unroll
            for (int dt = 0; dt < ND; ++dt)
                *reinterpret_cast<f32x4 *>(S_T + p.sbase + state_col<G::KSD>(dt, g)) = Sacc[dt];
        }
    } else {
        // --------------------------- preparation waves ---------------------------
        __builtin_amdgcn_s_setprio(3);
        const HeadPtrs<DT> p =
            head_ptrs<DT, DK, NW>(q, k, v, beta, gl, o, cu, T, H, Dv, nvt, 0, r, segP, segL);
        const int N = (p.T + C - 1) / C;
        switch (wave - NSW) {
        case 0: prep_role<DT, DK, C, NW, 0, GATED, L2, NOOUT>(sm, p, p.T, N, lane); break;
        case 1: if constexpr (NW > 1) prep_role<DT, DK, C, NW, 1, GATED, L2, NOOUT>(sm, p, p.T, N, lane); break;
        case 2: if constexpr (NW > 2) prep_role<DT, DK, C, NW, 2, GATED, L2, NOOUT>(sm, p, p.T, N, lane); break;
        default: if constexpr (NW > 3) prep_role<DT, DK, C, NW, 3, GATED, L2, NOOUT>(sm, p, p.T, N, lane); break;
        }
    }
}

// ---------------------------------------------------------------------------
// Serial kernel (single-buffered; for shapes whose double buffers do not fit)
// ---------------------------------------------------------------------------
template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
struct SerialSmem {
    typedef ChunkCfg<DT, DK, C, NW> G;
    static constexpr int NOFF = G::NT * (G::NT - 1) / 2;
    DT Ks[C * G::LDK];
    DT Qs[C * G::LDK];
    DT Vs[C * G::LDV];
    DT Ps[C * G::LDP];
    DT Ab[(NOFF > 0 ? NOFF : 1) * FRAG_ELEMS];
    DT Tb[G::NT * FRAG_ELEMS];
    float betas[C];
    GateSets<C, 1, GATED> gate;
    NormSets<C, 1, L2> norm;
};

template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1))) void chunk_fwd_serial_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ gl, const float *S0,
    DT *__restrict__ o, float *S_T, DT *__restrict__ hs, const int *__restrict__ cu, int T,
    int H, int Dv, int nvt, float scale, int segP, int segL) {
    typedef ChunkCfg<DT, DK, C, NW> G;
    constexpr int ND = G::ND;
    __shared__ __attribute__((aligned(16))) SerialSmem<DT, DK, C, NW, GATED, L2> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int g = lane >> 4, r = lane & 15;
    const HeadPtrs<DT> p =
        head_ptrs<DT, DK, NW>(q, k, v, beta, gl, o, cu, T, H, Dv, nvt, wave, r, segP, segL);

    f32x4 Sacc[ND];
    if (S0) {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt)
            Sacc[dt] = *reinterpret_cast<const f32x4 *>(S0 + p.sbase + state_col<G::KSD>(dt, g));
    } else {
#pragma unroll
        for (int dt = 0; dt < ND; ++dt) Sacc[dt] = zero4();
    }

    const int N = (p.T + C - 1) / C;
    if (N > 0) {
        for (int i = tid; i < C * G::LDP; i += G::NTHR) sm.Ps[i] = from_f32<DT>(0.f);
        ChunkRegs<DT, DK, C, NW, GATED> rg;
        rg.init(p, tid);
        OutChunk out = out_chunk(p, scale, g, r);
        rg.load(p, p.T, 0);
        for (int c = 0; c < N; ++c) {
            const int t0 = c * C;
            const int len = o ? min(C, p.T - t0) : 0;
            if (hs) store_state_row<G::KSD, ND>(hs + ((p.head * N + c) * Dv + p.vcol) * DK, Sacc, g);
            lds_barrier();
            rg.stage(sm.Ks, sm.Qs, sm.Vs, sm.betas, sm.gate.at(0), tid);
            lds_barrier();
            rg.load(p, p.T, min(c + 1, N - 1) * C);
            const float *bc = nullptr;
            if constexpr (GATED) bc = sm.gate.at(0)->bc;
            gram_tiles<DT, DK, C, NW, GATED, L2>(sm.Ks, sm.Qs, sm.betas, bc, sm.Ab, sm.Tb, sm.Ps,
                                                 sm.norm.at(0), wave, lane);
            lds_barrier();
            out.rsrc = make_rsrc(p.oh + (int64_t)t0 * p.tsv, len * out.row_bytes);
            state_path<DT, DK, C, NW, GATED, L2>(sm.Ks, sm.Qs, sm.Vs, sm.Ab, sm.Tb, sm.Ps,
                                                 sm.gate.at(0), sm.norm.at(0), Sacc, out, wave,
                                                 lane);
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
// B in ChunkFwdArgs counts sequences (batch rows, or packed sequences when
// cu is set); T is the token axis of each batch row.
template <typename DT, int DK, int C, int NW, bool GATED, bool L2>
hipError_t launch_cfg(const ChunkFwdArgs &a, hipStream_t stream) {
    const int nvt = a.Dv / (16 * NW);
    const int64_t grid = a.B * a.H * nvt;
    const DT *q = static_cast<const DT *>(a.q), *k = static_cast<const DT *>(a.k);
    const DT *v = static_cast<const DT *>(a.v), *beta = static_cast<const DT *>(a.beta);
    DT *o = static_cast<DT *>(a.o);
    // without outputs, the specialisation that skips their products (bf16,
    // the larger head and chunk sizes: the backward's checkpoints and the
    // segment passes; other shapes compute the outputs and drop them)
    constexpr bool HAS_NOOUT = sizeof(DT) == 2 && DK >= 64 && C >= 32 && !L2;
    if constexpr (HAS_NOOUT && ws_fits<DT, DK, C, NW, GATED, L2>()) {
        if (!o) {
            hipLaunchKernelGGL((chunk_fwd_ws_kernel<DT, DK, C, NW, GATED, L2, true>),
                               dim3((unsigned)grid), dim3(128 * NW), 0, stream, q, k, v, beta, a.g,
                               a.S0, o, a.S_T, static_cast<DT *>(a.h), a.cu, (int)a.T, (int)a.H,
                               a.Dv, nvt, a.scale, nullptr, a.segP, a.segL);
            return hipGetLastError();
        }
    }
    if constexpr (ws_fits<DT, DK, C, NW, GATED, L2>()) {
        hipLaunchKernelGGL((chunk_fwd_ws_kernel<DT, DK, C, NW, GATED, L2>), dim3((unsigned)grid),
                           dim3(128 * NW), 0, stream, q, k, v, beta, a.g, a.S0, o, a.S_T,
                           static_cast<DT *>(a.h), a.cu,
                           (int)a.T, (int)a.H, a.Dv, nvt, a.scale, nullptr, a.segP, a.segL);
    } else {
        hipLaunchKernelGGL((chunk_fwd_serial_kernel<DT, DK, C, NW, GATED, L2>), dim3((unsigned)grid),
                           dim3(64 * NW), 0, stream, q, k, v, beta, a.g, a.S0, o, a.S_T,
                           static_cast<DT *>(a.h), a.cu,
                           (int)a.T, (int)a.H, a.Dv, nvt, a.scale, a.segP, a.segL);
    }
    return hipGetLastError();
}

// The zero-state pass and the transition-map pass of the segment-parallel
// schedule in one launch (PAIR): value rows from zero states into a.S_T and
// the d_k rows of each segment's map (from the identity) into M.
template <typename DT, int DK, int C, bool GATED>
hipError_t launch_pair_cfg(const ChunkFwdArgs &a, float *M, hipStream_t stream) {
    constexpr int NW = 4;
    const int nvt = DK / (16 * NW);
    const int64_t grid = a.B * a.H * nvt;
    hipLaunchKernelGGL((chunk_fwd_ws_kernel<DT, DK, C, NW, GATED, false, true, true>),
                       dim3((unsigned)grid), dim3(192 * NW), 0, stream,
                       static_cast<const DT *>(a.q), static_cast<const DT *>(a.k),
                       static_cast<const DT *>(a.v), static_cast<const DT *>(a.beta), a.g,
                       nullptr, nullptr, a.S_T, nullptr, a.cu, (int)a.T, (int)a.H, a.Dv, nvt,
                       a.scale, M, a.segP, a.segL);
    return hipGetLastError();
}

// The combined pass for one rule: d_k = d_v = 64 at chunks of 32, 128 at 32
// or 64.
template <bool GATED>
hipError_t launch_pair_rule(const ChunkFwdArgs &a, float *M, hipStream_t stream) {
    if (a.Dk == 64)
        return a.chunk == 32 ? launch_pair_cfg<__bf16, 64, 32, GATED>(a, M, stream)
                             : hipErrorNotSupported;
    switch (a.chunk) {
    case 32: return launch_pair_cfg<__bf16, 128, 32, GATED>(a, M, stream);
    case 64: return launch_pair_cfg<__bf16, 128, 64, GATED>(a, M, stream);
    default: return hipErrorNotSupported;
    }
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

template <typename DT, int DK, int C, bool GATED, bool L2>
hipError_t dispatch_nw(const ChunkFwdArgs &a, hipStream_t stream) {
    switch (pick_waves(a.B * a.H, a.Dv)) {
    case 4: return launch_cfg<DT, DK, C, 4, GATED, L2>(a, stream);
    case 2: return launch_cfg<DT, DK, C, 2, GATED, L2>(a, stream);
    default: return launch_cfg<DT, DK, C, 1, GATED, L2>(a, stream);
    }
}

}  // namespace

// The plain rule's bf16 kernels at d_k = 128 and 64-token chunks (the layer
// shape's launch) live in a translation unit of their own, built with another
// instruction-scheduling strategy.
hipError_t launch_chunk_fwd_plain_d128_c64(const ChunkFwdArgs &a, hipStream_t stream);

namespace {

template <typename DT, int DK, bool GATED, bool L2>
hipError_t dispatch_c(const ChunkFwdArgs &a, hipStream_t stream) {
    switch (a.chunk) {
    case 16: return dispatch_nw<DT, DK, 16, GATED, L2>(a, stream);
    case 32: return dispatch_nw<DT, DK, 32, GATED, L2>(a, stream);
    case 64:
        if constexpr (sizeof(DT) == 2 && DK == 128 && !GATED && !L2)
            return launch_chunk_fwd_plain_d128_c64(a, stream);
        else
            return dispatch_nw<DT, DK, 64, GATED, L2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename DT, bool GATED, bool L2>
hipError_t dispatch_dk(const ChunkFwdArgs &a, hipStream_t stream) {
    switch (a.Dk) {
    case 16: return dispatch_c<DT, 16, GATED, L2>(a, stream);
    case 32: return dispatch_c<DT, 32, GATED, L2>(a, stream);
    case 64: return dispatch_c<DT, 64, GATED, L2>(a, stream);
    case 128: return dispatch_c<DT, 128, GATED, L2>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

// Every kernel of one rule (plain or gated), both dtypes.
template <bool GATED, bool L2>
hipError_t launch_rule(const ChunkFwdArgs &a, bool bf16, hipStream_t stream) {
    return bf16 ? dispatch_dk<__bf16, GATED, L2>(a, stream) : dispatch_dk<float, GATED, L2>(a, stream);
}

}  // namespace

// The gated and the L2-normalising instantiations live in translation units
// of their own.
hipError_t launch_chunk_fwd_gated(const ChunkFwdArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_chunk_state_pair_gated(const ChunkFwdArgs &a, float *M, hipStream_t stream);
hipError_t launch_chunk_fwd_l2(const ChunkFwdArgs &a, bool bf16, hipStream_t stream);
hipError_t launch_chunk_fwd_gated_l2(const ChunkFwdArgs &a, bool bf16, hipStream_t stream);

}  // namespace dr
