// Backward of the chunked delta rule (plain and gated rule, gfx950).
//
// The forward pass is S_{c+1} = S_c + E^T K and O = Q S_c^T + P E per chunk c
// (C tokens), with P = Q K^T (.) M, A = diag(beta) tril(K K^T, -1),
// Tm = (I + A)^{-1} and the resolved errors E = Tm diag(beta) R,
// R = V - K S_c^T (paperlayer summary of arXiv:2406.06484, section 3; hada.io
// digest, section "Chunkwise KDA").  The pages state the training strategy --
// keep only the chunk states and recompute the rest in the backward -- but not
// its equations; by the chain rule through those products, with dS the
// gradient of the loss with respect to S_{c+1} and dO that of O:
//
//   dE   = P^T dO + K dS^T                      gradient reaching E
//   Z    = Tm^T dE,   dV = diag(beta) Z         through the triangular solve
//   Y    = R - tril(K K^T, -1) E                (the solve's right-hand side)
//   dbeta_t = sum_v Z[t][v] Y[t][v]
//   dG   = -tril(dV E^T, -1)                    G = K K^T inside A
//   dQ   = dO S_c + (dO E^T (.) M) K
//   dK   = -dV S_c + E dS + (dG + dG^T) K + (dO E^T (.) M)^T Q
//   dS  <- dS + dO^T Q - dV^T K                 gradient with respect to S_c
//
// and dS0 is dS after the first chunk.  The fp64 oracle (reverse token order)
// pins all of it.
//
// Gated rule (hada.io digest, "Gated DeltaNet" and "Chunkwise KDA" with a
// scalar decay).  With b the in-chunk prefix sums of the log gate,
// gamma_t = exp(b_t), rho_t = exp(b_last - b_t) and D_ij = exp(b_i - b_j),
// the forward uses G (.) D and P (.) D, R = V - diag(gamma) K S_c^T,
// O = diag(gamma) Q S_c^T + P E and S_{c+1} = gamma_last S_c +
// E^T diag(rho) K.  The same chain rule gives
//
//   dE   = P^T dO + diag(rho) K dS^T
//   dQ   = diag(gamma) dO S_c + ((dO E^T) (.) M (.) D) K
//   dK   = -diag(gamma) dV S_c + diag(rho) E dS + (dG' + dG'^T) K
//          + ((dO E^T) (.) M (.) D)^T Q,            dG' = dG (.) D
//   dS  <- gamma_last dS + (diag(gamma) dO)^T Q - (diag(gamma) dV)^T K
//
// and for b: dL/dgamma_t = sum_k (Q (.) dO S_c - K (.) dV S_c)_tk,
// dL/drho_t = sum_k (K (.) E dS)_tk, dL/dgamma_last = <dS, S_c>, and
// W = dG (.) (G (.) D) + (dO E^T) (.) (P (.) D) off the diagonal (dL/dD_ij
// times D_ij), so that
//
//   dL/db_t = gamma_t dL/dgamma_t - rho_t dL/drho_t + sum_j W_tj - sum_i W_it
//             (+ gamma_last dL/dgamma_last + sum_s rho_s dL/drho_s at the last token)
//
// and dg_t is the sum of dL/db_s over s >= t within the chunk.  The sums
// over k come from the transposed dQ and dK tiles before their decays, so
// the per-wave phase keeps no extra products.
//
// Work split.  One workgroup per (b, h) walks the chunks in reverse.  Wave w
// owns value columns 16w .. 16w+15: its slices of R, E, dE, Z, dV and the
// rows of dS (kept transposed, d_k x 16, as fp32 MFMA accumulators for the
// whole sequence).  The state S_c of each chunk comes from checkpoints the
// forward kernel writes.  Products that sum over all value columns (dO E^T,
// dV E^T, dQ, dK) run after the waves have published their slices in LDS:
// the C x C tiles dealt round-robin to the waves, dQ and dK by key tile.
// Chunks are 32 tokens for bf16 and 16 for fp32 (LDS capacity), which the
// forward checkpoints follow.
//
// Memory traffic.  The next chunk's inputs travel in registers, loaded in
// three parts at three phases of the current chunk (S_c, then K and Q, then
// V, dO and beta), and the outputs are written at the start of the last
// phase (dV from its LDS copy and dQ, dK of the previous chunk from
// registers, all as vectors): the last phase is bound by LDS reads and leaves
// the vector memory path free, while a burst of loads just before a barrier
// had every wave waiting for the slowest one to issue its share.
#include "dr_common.hpp"
#include "dr_launch.hpp"

#include <algorithm>
#include <climits>
#include <mutex>
#include <type_traits>

namespace dr {

namespace {

template <typename DT, int DK, int DV, int C>
struct BwdCfg {
    static constexpr int NW = DV / 16;            // waves
    static constexpr int NT = C / 16;             // token tiles
    static constexpr int KT = DK / 16;            // key tiles
    static constexpr int VT = DV / 16;            // value tiles
    static constexpr int PAD = 16 / (int)sizeof(DT);
    static constexpr int LDK = DK + PAD;          // K, Q rows (tokens x d_k)
    static constexpr int LDV = DV + PAD;          // V, dO, E, dV rows (tokens x d_v)
    static constexpr int LDS_ = DK + PAD;         // dS_{c+1} rows (d_v x d_k, like S_c)
    static constexpr int LDSK = DK + PAD;         // S_c rows (d_v x d_k)
    static constexpr int LDC = C + PAD;           // C x C matrices
    // dS_{c+1}^T gets its own LDS buffer unless that overflows LDS (fp32 with
    // d_k = d_v = 128); then it reuses the S_c^T buffer in a second pass.
    static constexpr int BASE = (int)sizeof(DT) * (4 * C * LDK + 4 * C * LDV + DV * LDSK + 6 * C * LDC) +
                                4 * C * (2 + NW);
    static constexpr bool DBUF = BASE + (int)sizeof(DT) * DV * LDS_ + 256 <= 160 * 1024;
};

// Gated rule: the chunk's decays and the parts of dL/db, b the in-chunk
// prefix sums of the log gate (nothing for the plain rule).  The parts are
// summed into dg at the start of the next chunk (after the loop for the
// first), so they are only read behind a barrier.
template <int C, int NW, int NJ, int KT, bool GATED>
struct BwdGate {
    float gb[2][C], gam[2][C], rto[2][C];  // b, exp(b), exp(b_last - b), by chunk parity
    float pdb[KT][C];                 // gamma_t dL/dgamma_t - rho_t dL/drho_t, per key tile
    float prd[KT][C];                 // rho_t dL/drho_t, per key tile
    float dgc[NW];                    // gamma_last dL/dgamma_last, per wave
    float wrow[2 * NJ][16], wcol[2 * NJ][16];  // row / column sums of W per C x C tile job
};
template <int C, int NW, int NJ, int KT>
struct BwdGate<C, NW, NJ, KT, false> {};

template <typename DT, int DK, int DV, int C, bool GATED>
struct BwdSmem {
    typedef BwdCfg<DT, DK, DV, C> G;
    DT Ks[2][C * G::LDK], Qs[2][C * G::LDK];     // by chunk parity (the next chunk's
                                                  // Gram tiles overlap this chunk's dQ, dK)
    DT Vs[C * G::LDV], Os[C * G::LDV];            // V, dO
    DT Es[C * G::LDV], Rb[C * G::LDV];            // E, dV
    DT Sb[DV * G::LDSK];                          // S_c (rows: value index); second
                                                  // pass without DBUF: dS_{c+1}
    DT Db[G::DBUF ? DV * G::LDS_ : 8];            // dS_{c+1} (DBUF; rows: value index)
    DT Pm[C * G::LDC];                            // Q K^T (.) M
    DT Gl[2][C * G::LDC];                         // tril(K K^T, -1), by chunk parity
    DT Tm[C * G::LDC];                            // (I + A)^{-1}
    DT Dm[C * G::LDC];                            // dO E^T (.) M
    DT Gs[C * G::LDC];                            // dG + dG^T
    float betas[2][C];
    float dbp[G::NW][C];                          // per-wave parts of dbeta
    BwdGate<C, G::NW, G::NT * (G::NT + 1) / 2, G::KT, GATED> gt;
};

template <typename DT, int DK, int DV, int C, bool GATED>
constexpr bool bwd_fits() {
    return sizeof(BwdSmem<DT, DK, DV, C, GATED>) <= 160 * 1024;
}

// Four consecutive elements of DT to global memory through a buffer resource
// (dropped past its range).
__device__ __forceinline__ void store4(const bf16x4 &f, __amdgpu_buffer_rsrc_t r, int voff) {
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, f), r, voff, 0, 0);
}
__device__ __forceinline__ void store4(const f32x4_arr &f, __amdgpu_buffer_rsrc_t r, int voff) {
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f), r, voff, 0, 0);
}

// One 16x16x16 product step on 16-wide fragments of DT.
template <typename DT>
__device__ __forceinline__ void mk(f32x4 &acc, const typename Frag<DT>::k16 &a,
                                   const typename Frag<DT>::k16 &b) {
    mma_k16(acc, a, b);
}

// acc += sum_i A_i B_i over N 16-wide slabs (fragments fa[i], fb[i]).  For
// bf16 two consecutive slabs go through one 16x16x32 product: a 32-wide
// fragment is two 16-wide ones side by side, and A and B take the same k
// order.  An odd last slab is paired with zeros, so that every product of an
// accumulation chain has the same shape (a dependent 16x16x16 product right
// after a 16x16x32 one on the same accumulator would read a stale value).
template <typename DT, int N>
__device__ __forceinline__ void mk_n(f32x4 &acc, const typename Frag<DT>::k16 *fa,
                                     const typename Frag<DT>::k16 *fb) {
    if constexpr (std::is_same<DT, __bf16>::value) {
#pragma unroll
        for (int i = 0; i < N; i += 2) {
            const bf16x4 z = {};
            const bf16x4 a1 = i + 1 < N ? fa[i + 1] : z, b1 = i + 1 < N ? fb[i + 1] : z;
            mma_k32(acc, __builtin_shufflevector(fa[i], a1, 0, 1, 2, 3, 4, 5, 6, 7),
                    __builtin_shufflevector(fb[i], b1, 0, 1, 2, 3, 4, 5, 6, 7));
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) mk<DT>(acc, fa[i], fb[i]);
    }
}

// 16x16 tile of A B with A row-major (rows m0.., k along the row) and B given
// as B^T row-major (rows n0..): sum over k in [k0, k1).  D layout:
// lane (g, r) holds (A B)[m0 + 4g + i][n0 + r].
// NK 16-wide steps from k0; every fragment is read before the first product
// so that the LDS latency is paid once per tile.
template <typename DT, int NK>
__device__ __forceinline__ void tile_rr(f32x4 &acc, const DT *A, int lda, int m0, const DT *Bt,
                                        int ldb, int n0, int k0, int lane) {
    typename Frag<DT>::k16 fa[NK], fb[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        frag_rows(A, lda, m0, k0 + 16 * i, lane, fa[i]);
        frag_rows(Bt, ldb, n0, k0 + 16 * i, lane, fb[i]);
    }
    mk_n<DT, NK>(acc, fa, fb);
}
// Same with B row-major (k along the rows of B: B[k][n]).
template <typename DT, int NK>
__device__ __forceinline__ void tile_rc(f32x4 &acc, const DT *A, int lda, int m0, const DT *B,
                                        int ldb, int n0, int k0, int lane) {
    typename Frag<DT>::k16 fa[NK], fb[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        frag_rows(A, lda, m0, k0 + 16 * i, lane, fa[i]);
        frag_cols16(B, ldb, k0 + 16 * i, n0, lane, fb[i]);
    }
    mk_n<DT, NK>(acc, fa, fb);
}
// Same with A given transposed (A^T row-major: A[m][k] = At[k][m]) and B
// row-major.
template <typename DT, int NK>
__device__ __forceinline__ void tile_cc(f32x4 &acc, const DT *At, int lda, int m0, const DT *B,
                                        int ldb, int n0, int k0, int lane) {
    typename Frag<DT>::k16 fa[NK], fb[NK];
#pragma unroll
    for (int i = 0; i < NK; ++i) {
        frag_cols16(At, lda, k0 + 16 * i, m0, lane, fa[i]);
        frag_cols16(B, ldb, k0 + 16 * i, n0, lane, fb[i]);
    }
    mk_n<DT, NK>(acc, fa, fb);
}

// x from the lane N places further in its row of 16 lanes (DPP row shift;
// zero past the row's end).
template <int N>
__device__ __forceinline__ float row_shl(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}

// Store a D-layout tile (lane (g, r): rows 4g + i, column r) into a
// row-major matrix at (m0, n0), keeping entry (row, col) only where
// keep(row, col); other entries are written as zero.
template <typename DT, typename Keep>
__device__ __forceinline__ void put_tile(DT *M, int ld, int m0, int n0, const f32x4 &x, int lane,
                                         Keep keep) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int row = m0 + 4 * g + i, col = n0 + r;
        M[row * ld + col] = from_f32<DT>(keep(row, col) ? x[i] : 0.f);
    }
}

// Product X Y of two 16x16 matrices held in D layout, given X^T in D layout
// (the A operand) and Y (the B operand).
template <typename DT>
__device__ __forceinline__ f32x4 dmul(const f32x4 &xt, const f32x4 &y) {
    typename Frag<DT>::k16 fa, fb;
    cvt4(xt, fa);
    cvt4(y, fb);
    f32x4 acc = zero4();
    mk<DT>(acc, fa, fb);
    return acc;
}

// (I + A)^{-1} for a strictly lower-triangular 16x16 A (A^16 = 0):
// (I - A)(I + A^2)(I + A^4)(I + A^8).  Matrices are carried with their
// transposes so that every product takes its A operand from a D-layout
// tile.  a, at: A and A^T in D layout.  Returns T (D layout).
template <typename DT>
__device__ __forceinline__ f32x4 inv_unit_lower(const f32x4 &a, const f32x4 &at, int lane) {
    const int g = lane >> 4, r = lane & 15;
    f32x4 I;
#pragma unroll
    for (int i = 0; i < 4; ++i) I[i] = (4 * g + i == r) ? 1.f : 0.f;
    const f32x4 a2 = dmul<DT>(at, a), a2t = dmul<DT>(a, at);
    const f32x4 a4 = dmul<DT>(a2t, a2), a4t = dmul<DT>(a2, a2t);
    const f32x4 a8 = dmul<DT>(a4t, a4);
    const f32x4 lt = I - at;                                  // (I - A)^T
    const f32x4 t1t = dmul<DT>(I + a2, lt);                   // ((I - A)(I + A^2))^T
    const f32x4 t2t = dmul<DT>(I + a4, t1t);                  // (... (I + A^4))^T
    return dmul<DT>(t2t, I + a8);                             // ... (I + A^8)
}

// 16 bytes of DT.
template <typename DT> struct V16;
template <> struct V16<__bf16> { typedef bf16x8 type; };
template <> struct V16<float> { typedef f32x4 type; };

// Register prefetch of one chunk's rows of a [tokens, cols] tile (row stride
// gs elements in global memory, ld in LDS): 16-byte vectors dealt to the
// threads; rows at or past the chunk's valid length load as zeros (buffer
// resource range check).
template <typename DT, int ROWS, int COLS, int NTHR>
struct RowPrefetch {
    typedef typename V16<DT>::type vec_t;
    static constexpr int VPR = COLS * (int)sizeof(DT) / 16;   // vectors per row
    static constexpr int NV = ROWS * VPR;
    static constexpr int PER = (NV + NTHR - 1) / NTHR;
    vec_t x[PER];
    __device__ __forceinline__ void load(const DT *src, int64_t gs, int nvalid, int tid) {
        const auto rs = make_rsrc(src, nvalid > 0 ? (int)((nvalid - 1) * gs + COLS) * (int)sizeof(DT) : 0);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTHR;
            const int t = i / VPR, e = (i % VPR) * (16 / (int)sizeof(DT));
            const int off = (i < NV && t < nvalid) ? (int)((t * gs + e) * (int)sizeof(DT)) : 0x7ffffff0;
            x[j] = buf_load16<vec_t>(rs, off);
        }
    }
    // Unguarded where the vectors divide evenly over the threads: a store
    // skipped on some path leaves its registers' loads pending there, and the
    // next load into them would then wait for every load in flight.
    __device__ __forceinline__ void store(DT *dst, int ld, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTHR;
            if (NV % NTHR == 0 || i < NV) {
                const int t = i / VPR, e = (i % VPR) * (16 / (int)sizeof(DT));
                *reinterpret_cast<vec_t *>(dst + t * ld + e) = x[j];
            }
        }
    }
};

// All per-chunk inputs of the backward, one chunk ahead: K, Q, V, dO, beta
// and the chunk's incoming state S_c (row-major [d_v][d_k] checkpoint).
template <typename DT, int DK, int DV, int C>
struct ChunkPrefetch {
    static constexpr int NTHR = 4 * DV;
    RowPrefetch<DT, C, DK, NTHR> k, q;
    RowPrefetch<DT, C, DV, NTHR> v, o;
    RowPrefetch<DT, DV, DK, NTHR> s;
    RowPrefetch<DT, DV, DK, NTHR> ds;  // dS_{c+1} checkpoint (products-only mode)
    RowPrefetch<DT, C, DV, NTHR> z;    // Z (products-only mode)
    DT b;      // beta of token tid (zero past the chunk's valid length)
    float gv;  // log gate of token tid (gated rule; zero past the valid length)
    // Part 0: S_c; part 1: K, Q, beta (and the log gates); part 2: V and dO
    // (issued at three points of a chunk, so that no single point floods the
    // vector memory path).  MODE 1 (recursion only) loads no S_c and no V;
    // MODE 2 (products only) also loads the dS_{c+1} checkpoint (part 0) and
    // Z (part 2).
    template <int P, int MODE>
    __device__ __forceinline__ void load_part(const DT *kk, const DT *qq, const DT *vv,
                                              const DT *oo, const DT *bb, const float *gg,
                                              const DT *sc, const DT *dsc, const DT *zz,
                                              int64_t tok0, int h, int H, int len, int tid) {
        const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
        if constexpr (P == 0 && MODE != 1) s.load(sc, DK, DV, tid);
        if constexpr (P == 0 && MODE == 2) ds.load(dsc, DK, DV, tid);
        if constexpr (P == 1) {
            k.load(kk + (tok0 * H + h) * DK, rk, len, tid);
            q.load(qq + (tok0 * H + h) * DK, rk, len, tid);
            // through a range-checked resource like the tiles, so that nothing
            // waits for this load before the chunk's LDS stores
            const auto rb = make_rsrc(bb + tok0 * H + h, len > 0 ? ((len - 1) * H + 1) * (int)sizeof(DT) : 0);
            b = buf_load_elem<DT>(rb, tid < len ? tid * H * (int)sizeof(DT) : 0x7ffffff0);
            if (gg && tid < 64) {
                const auto rg = make_rsrc(gg + tok0 * H + h, len > 0 ? ((len - 1) * H + 1) * 4 : 0);
                gv = buf_load_elem<float>(rg, tid < len ? tid * H * 4 : 0x7ffffff0);
            }
        }
        if constexpr (P == 2) {
            if constexpr (MODE != 1) v.load(vv + (tok0 * H + h) * DV, rv, len, tid);
            o.load(oo ? oo + (tok0 * H + h) * DV : oo, rv, oo ? len : 0, tid);  // null: dO = 0
            if constexpr (MODE == 2) z.load(zz + (tok0 * H + h) * DV, rv, len, tid);
        }
    }
};

// Rows [0, nvalid) of a [ROWS, COLS] LDS tile (row stride ld) to global rows
// of stride gs elements, 16 bytes per store; rows past nvalid are dropped by
// the buffer resource's range check.
template <typename DT, int ROWS, int COLS, int NTHR>
__device__ __forceinline__ void store_rows(DT *dst, int64_t gs, int nvalid, const DT *src, int ld,
                                           int tid) {
    typedef typename V16<DT>::type vec_t;
    typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
    constexpr int VPR = COLS * (int)sizeof(DT) / 16;
    constexpr int NV = ROWS * VPR;
    const auto rs = make_rsrc(dst, (int)((nvalid - 1) * gs + COLS) * (int)sizeof(DT));
#pragma unroll
    for (int j = 0; j < (NV + NTHR - 1) / NTHR; ++j) {
        const int i = tid + j * NTHR;
        if (NV % NTHR == 0 || i < NV) {
            const int t = i / VPR, e = (i % VPR) * (16 / (int)sizeof(DT));
            const vec_t x = *reinterpret_cast<const vec_t *>(src + t * ld + e);
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs,
                                                   (int)((t * gs + e) * (int)sizeof(DT)), 0, 0);
        }
    }
}

// MODE 0: the whole backward in one reverse walk per (b, h), over chunks
// [c_beg, c_end) from dS = dST at the end of c_end - 1 (dS0 gets dS at the
// start of c_beg).  MODE 1 (recursion only): dE, Z, dV and the dS recursion,
// one workgroup per (b, h); it writes dV, dS0, Z (dsz, [B,T,H,d_v]) and every
// chunk's dS_{c+1} (dsb, [B,H,N,d_v,d_k], like the forward checkpoints).
// MODE 2 (products only): R, E, dbeta, dQ, dK (and dg) from those, with
// nsplit workgroups per (b, h), each over its own run of chunks, so that the
// chunks of a head run in parallel.  MODE 3: the recursion of MODE 1 over
// chunks [c_beg, c_end), writing nothing but dS at the start of c_beg (into
// dS0): the incoming dS of a MODE 0 walk over the chunks before c_beg.
// Segmented launches of MODES 1 and 3 (segP > 1): segP workgroups per (b, h),
// workgroup part p over chunks [p segL, (p + 1) segL); their dS_T and (MODE
// 3) dS0 arrays are per segment, [(b segP + p) H + h][d_v][d_k], and MODE 1
// writes dS0 from segment 0 only.  ident starts dS from the identity (d_v =
// d_k), and a null dout reads dO as zero: with both, MODE 3 gives the
// segment's linear map of dS.
template <typename DT, int DK, int DV, int C, bool GATED, int MODE>
__global__ __launch_bounds__(DV * 4) void chunk_bwd_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ gl, const DT *__restrict__ dout,
    const float *__restrict__ dST, const DT *__restrict__ hs, DT *__restrict__ dq,
    DT *__restrict__ dk, DT *__restrict__ dv, DT *__restrict__ dbeta, float *__restrict__ dg,
    float *__restrict__ dS0, DT *__restrict__ dsb, DT *__restrict__ dsz, int T, int H,
    int nsplit, int c_beg, int c_end, int segP, int segL, int ident) {
    typedef BwdCfg<DT, DK, DV, C> G;
    constexpr int NW = G::NW, NT = G::NT, KT = G::KT, VT = G::VT;
    constexpr int LDK = G::LDK, LDV = G::LDV, LDS_ = G::LDS_, LDSK = G::LDSK, LDC = G::LDC;
    constexpr bool RONLY = MODE == 1 || MODE == 3;  // the recursion alone
    constexpr bool PROD = !RONLY;      // R, E, dbeta and the products over all value columns
    constexpr bool RECUR = MODE != 2;  // dE, Z and the dS recursion
    static_assert(MODE == 0 || G::DBUF, "split modes keep dS_{c+1} in its own LDS buffer");
    __shared__ __attribute__((aligned(16))) BwdSmem<DT, DK, DV, C, GATED> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int v0 = 16 * w;
    const bool segd = (MODE == 1 || MODE == 3) && segP > 1;  // segmented launch
    const int nper = MODE == 2 ? nsplit : segd ? segP : 1;      // workgroups per (b, h)
    const int64_t head = blockIdx.x / nper;
    const int part = (int)(blockIdx.x % nper);
    const int b = (int)(head / H), h = (int)(head % H);
    const int N = (T + C - 1) / C;
    const int nthr = 64 * NW;
    // chunks [c_lo, c_hi) of this workgroup, walked in reverse
    int c_lo = 0, c_hi = N;
    if constexpr (MODE == 0 || MODE == 1 || MODE == 3) {
        c_lo = max(0, c_beg);
        c_hi = min(N, c_end);
    }
    if (segd) {
        c_lo = min(N, part * segL);
        c_hi = min(N, c_lo + segL);
    }
    if constexpr (MODE == 2) {
        const int per = (N + nsplit - 1) / nsplit;
        c_lo = min(N, part * per);
        c_hi = min(N, c_lo + per);
    }
    // row of the per-segment state arrays of a segmented launch
    const int64_t sidx = segd ? ((int64_t)b * segP + part) * H + h : head;

    // upper tiles of the C x C matrices stay zero
    for (int i = tid; i < C * LDC; i += nthr) {
        sm.Pm[i] = sm.Gl[0][i] = sm.Gl[1][i] = sm.Tm[i] = sm.Dm[i] = sm.Gs[i] = from_f32<DT>(0.f);
    }
    // Tm, Pm and dO by chunk parity: mode 1 keeps two of each (the second in
    // the LDS its unused products would take: Dm, Gs, Vs), so that the next
    // chunk's Gram tiles and inverses form while this chunk's are read
    auto tm_buf = [&](int bb) -> DT * { return RONLY && bb ? sm.Dm : sm.Tm; };
    auto pm_buf = [&](int bb) -> DT * { return RONLY && bb ? sm.Gs : sm.Pm; };
    auto os_buf = [&](int bb) -> DT * { return RONLY && bb ? sm.Vs : sm.Os; };
    // dS^T of this wave's value columns: tile s holds dS^T[16s + 4g + i][v0 + r]
    f32x4 Dt[RECUR ? KT : 1];
#pragma unroll
    for (int s = 0; s < (RECUR ? KT : 0); ++s) {
        if (ident) {
#pragma unroll
            for (int i = 0; i < 4; ++i) Dt[s][i] = 16 * s + 4 * g + i == v0 + r ? 1.f : 0.f;
        } else {
            Dt[s] = dST ? *reinterpret_cast<const f32x4 *>(dST + (sidx * DV + v0 + r) * DK + 16 * s + 4 * g)
                        : zero4();
        }
    }
    // The in-loop code must not see these loads as pending (it would wait for
    // every memory operation in flight at their first use, in every chunk).
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)

    // Output tiles (mt, j) of dQ and dK: token tile mt, key tile j.  With
    // NW <= KT wave w takes key tiles j = w, w + NW, ... for every token tile;
    // with more waves than key tiles, key tile w % KT and token tiles w / KT,
    // w / KT + NW / KT, ...
    constexpr int NJW = NW <= KT ? KT / NW : 1;   // key tiles per wave
    constexpr int MS = NW <= KT ? 1 : NW / KT;    // token tile stride
    constexpr int NMU = (NT + MS - 1) / MS;       // token tiles per wave (at most)
    const int mt0 = NW <= KT ? 0 : w / KT;
    // dQ and dK tiles are computed transposed (operands swapped), so that a
    // lane holds four consecutive keys of one token and stores them at once.
    // Where a wave has at most two tiles of each, they are held in registers
    // and stored in the next chunk, after the loads of the chunk after it
    // have been issued: a store issued just before the wait for those loads
    // at the top of a chunk would be waited for with them (the wait covers
    // every memory operation issued before the last load).
    constexpr bool DEFER = NJW * NMU <= 2;
    typedef typename Frag<DT>::k16 out4;
    out4 pq[DEFER ? NJW * NMU : 1], pk[DEFER ? NJW * NMU : 1];
    const int64_t rowq = (int64_t)H * DK;
    auto chunk_rsrc = [&](DT *base, int cc, int64_t row, int cols) {
        const int ft0 = cc * C, flen = min(C, T - ft0);
        return make_rsrc(base + (((int64_t)b * T + ft0) * H + h) * cols,
                         (int)((flen - 1) * row + cols) * (int)sizeof(DT));
    };
    auto flush = [&](int cc) {
        if constexpr (DEFER) {
            const auto rq = chunk_rsrc(dq, cc, rowq, DK), rk = chunk_rsrc(dk, cc, rowq, DK);
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj)
#pragma unroll
                for (int u = 0; u < NMU; ++u) {
                    const int mt = mt0 + u * MS, j = NW <= KT ? w + jj * NW : w % KT;
                    if (mt < NT) {
                        const int voff = ((16 * mt + r) * (int)rowq + 16 * j + 4 * g) * (int)sizeof(DT);
                        store4(pq[jj * NMU + u], rq, voff);
                        store4(pk[jj * NMU + u], rk, voff);
                    }
                }
        }
    };

    // dg of chunk cc from the parts of dL/db (wave 0, lane t = token t):
    // dL/db_t = gamma_t dL/dgamma_t - rho_t dL/drho_t + (row sums - column
    // sums of W)_t, plus, at the last token, the terms of b_last (in
    // gamma_last and every rho_t); then dg_t = sum over s >= t of dL/db_s.
    auto finalize_dg = [&](int cc) {
        if constexpr (GATED) {
            constexpr int NJ = NT * (NT + 1) / 2;
            float db = 0.f, rd = 0.f;
            if (lane < C) {
#pragma unroll
                for (int j = 0; j < KT; ++j) {
                    db += sm.gt.pdb[j][lane];
                    rd += sm.gt.prd[j][lane];
                }
                const int tt = lane >> 4, tl = lane & 15;
#pragma unroll
                for (int jb = 0; jb < 2 * NJ; ++jb) {
                    int jj = jb < NJ ? jb : jb - NJ, ti = 0;
                    while (jj > ti) { jj -= ti + 1; ++ti; }
                    if (ti == tt) db += sm.gt.wrow[jb][tl];
                    if (jj == tt) db -= sm.gt.wcol[jb][tl];
                }
            }
            float gc = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) gc += sm.gt.dgc[ww];
            const float srd = wave_sum(rd);
            if (lane == C - 1) db += gc + srd;
            // reverse inclusive scan over the chunk's tokens: within each row
            // of 16 lanes by row shifts (lanes past a row's end add zero),
            // then rows 0 .. add the totals of the rows after them
            db += row_shl<1>(db);
            db += row_shl<2>(db);
            db += row_shl<4>(db);
            db += row_shl<8>(db);
            if constexpr (C > 16) {
                const float tail = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(db), 16));
                if (lane < 16) db += tail;
            }
            const int flen = min(C, T - cc * C);
            if (lane < flen) dg[(((int64_t)b * T + cc * C) + lane) * H + h] = db;
        }
    };
    // Token 16 mt + r's part of dL/db from the transposed dQ / dK tiles of
    // key tile j (lane (g, r): keys 16 j + 4 g + i):
    //   dL/dgamma_t = sum_k Q (.) dO S_c - K (.) dV S_c   (= sum_v dO (.) Q S_c^T - dV (.) K S_c^T)
    //   dL/drho_t   = sum_k K (.) E dS_{c+1}              (= sum_v E (.) K dS_{c+1}^T)
    // from aq = (dO S_c)^T, an = (dV S_c)^T and ed = (E dS_{c+1})^T before
    // their decays.  add: accumulate onto the part written by the first pass.
    auto gate_part = [&](int cb, int j, int mt, const f32x4 &aq, const f32x4 &an, const f32x4 *ed,
                         bool add) {
        if constexpr (GATED) {
            const int t = 16 * mt + r;
            const typename Frag<DT>::k16 qv =
                *reinterpret_cast<const typename Frag<DT>::k16 *>(sm.Qs[cb] + t * LDK + 16 * j + 4 * g);
            const typename Frag<DT>::k16 kv =
                *reinterpret_cast<const typename Frag<DT>::k16 *>(sm.Ks[cb] + t * LDK + 16 * j + 4 * g);
            float sg = 0.f, sr = 0.f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sg += frag_get(qv, i) * aq[i] - frag_get(kv, i) * an[i];
                if (ed) sr += frag_get(kv, i) * (*ed)[i];
            }
            sg = xor32_sum(xor16_sum(sg));
            sr = xor32_sum(xor16_sum(sr));
            if (g == 0) {
                const float pr = sm.gt.rto[cb][t] * sr;
                float pd = sm.gt.gam[cb][t] * sg - pr;
                if (add) pd += sm.gt.pdb[j][t];
                sm.gt.pdb[j][t] = pd;
                sm.gt.prd[j][t] = pr;
            }
        }
    };

    // inputs of the next chunk to process travel in registers one chunk ahead
    ChunkPrefetch<DT, DK, DV, C> pf;
    auto prefetch = [&](auto part, int cn) {
        const int tp = cn * C;
        pf.template load_part<decltype(part)::value, RONLY ? 1 : MODE>(
            k, q, v, dout, beta, GATED ? gl : nullptr, hs + (head * N + cn) * DV * DK,
            dsb + (head * N + cn) * DV * DK, dsz, (int64_t)b * T + tp, h, H, min(C, T - tp), tid);
    };
    // K, Q and beta of chunk cc (and its decays) from the prefetch registers
    // into buffer set bb; every lane converts beta (see RowPrefetch::store).
    auto stage_kqb = [&](int bb) {
        pf.k.store(sm.Ks[bb], LDK, tid);
        pf.q.store(sm.Qs[bb], LDK, tid);
        const float bt = to_f32(pf.b);
        if (tid < C) sm.betas[bb][tid] = bt;
        if constexpr (GATED) {
            // in-chunk prefix sums b of the log gate and the two decays; tokens
            // past the valid length have g = 0, so b_last is the last valid
            // token's
            if (w == 0) {
                float x = lane < C ? pf.gv : 0.f;
#pragma unroll
                for (int d = 1; d < C; d <<= 1) {
                    const float y = __shfl_up(x, d, 64);
                    if (lane >= d) x += y;
                }
                const float bl = __shfl(x, C - 1, 64);
                if (lane < C) {
                    sm.gt.gb[bb][lane] = x;
                    sm.gt.gam[bb][lane] = __expf(x);
                    sm.gt.rto[bb][lane] = __expf(bl - x);
                }
            }
        }
    };
    // off-diagonal block of the inverse (one wave): T_10 = -T_11 (A_10 T_00),
    // A_10 = diag(beta_1) G_10
    auto t10 = [&](int bb) {
        typename Frag<DT>::k16 fa, fb;
        f32x4 m1 = zero4();
        frag_rows(sm.Gl[bb], LDC, 16, 0, lane, fa);
        {
            f32x4 tmp;
#pragma unroll
            for (int i = 0; i < 4; ++i) tmp[i] = frag_get(fa, i) * sm.betas[bb][16 + r];
            cvt4(tmp, fa);
        }
        frag_cols16(tm_buf(bb), LDC, 0, 0, lane, fb);
        mk<DT>(m1, fa, fb);
        f32x4 t10v = zero4();
        frag_rows(tm_buf(bb), LDC, 16, 16, lane, fa);
        cvt4(m1, fb);
        mk<DT>(t10v, fa, fb);
        put_tile(tm_buf(bb), LDC, 16, 0, -t10v, lane, [](int, int) { return true; });
    };

    // Gram tiles of the chunk in buffer set bb (K K^T and Q K^T, lower tiles),
    // into Gl[bb], Tm and Pm.  One tile, decayed for the gated rule:
    auto gram_tile = [&](int bb, bool isP, int ti, int tj) {
        f32x4 acc = zero4();
        tile_rr<DT, KT>(acc, isP ? sm.Qs[bb] : sm.Ks[bb], LDK, 16 * ti, sm.Ks[bb], LDK, 16 * tj, 0, lane);
        if constexpr (GATED) {
            // decay exp(b_hi - b_lo) between the later and the earlier token
            // (symmetric, as the diagonal blocks use both triangles)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int x = 16 * ti + 4 * g + i, y = 16 * tj + r;
                acc[i] *= __expf(sm.gt.gb[bb][max(x, y)] - sm.gt.gb[bb][min(x, y)]);
            }
        }
        return acc;
    };
    // diagonal block ti of G and its inverse T_ii = (I + A_ii)^{-1}
    auto diag_job = [&](int bb, int ti) {
        const f32x4 acc = gram_tile(bb, false, ti, ti);
        put_tile(sm.Gl[bb], LDC, 16 * ti, 16 * ti, acc, lane, [](int x, int y) { return x > y; });
        // A and A^T of the diagonal block: A[x][y] = beta_x G[x][y], x > y
        f32x4 a, at;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int x = 4 * g + i;
            a[i] = x > r ? sm.betas[bb][16 * ti + x] * acc[i] : 0.f;
            at[i] = r > x ? sm.betas[bb][16 * ti + r] * acc[i] : 0.f;  // G symmetric
        }
        const f32x4 tinv = inv_unit_lower<DT>(a, at, lane);
        put_tile(tm_buf(bb), LDC, 16 * ti, 16 * ti, tinv, lane, [](int x, int y) { return x >= y; });
    };
    // the diagonal blocks on the last waves (idle in the C x C phase)
    auto diag_jobs = [&](int bb) {
        for (int ti = NW - 1 - w; ti >= 0 && ti < NT; ti += NW) diag_job(bb, ti);
    };
    // the other tiles (G below the diagonal, all of P) dealt to waves
    // 0 .. nwj-1; then T_10 = -T_11 (A_10 T_00), A_10 = diag(beta_1) G_10, on
    // the wave that formed G_10 (the diagonal inverses are done by then)
    constexpr int NOFF = NT * (NT - 1) / 2;  // tiles of G below the diagonal
    constexpr int NJ = NT * (NT + 1) / 2;    // lower tiles of a C x C matrix
    auto other_jobs = [&](int bb, int nwj, bool with_t10 = true) {
        for (int j = w; j < NOFF + NJ; j += nwj) {
            const bool isP = j >= NOFF;
            int jj = isP ? j - NOFF : j, ti = isP ? 0 : 1;
            if (isP) {
                while (jj > ti) { jj -= ti + 1; ++ti; }
            } else {
                while (jj >= ti) { jj -= ti; ++ti; }
            }
            const int tj = jj;
            const f32x4 acc = gram_tile(bb, isP, ti, tj);
            if (isP) put_tile(pm_buf(bb), LDC, 16 * ti, 16 * tj, acc, lane, [](int x, int y) { return x >= y; });
            else put_tile(sm.Gl[bb], LDC, 16 * ti, 16 * tj, acc, lane, [](int x, int y) { return x > y; });
        }
        if constexpr (NT == 2) {
            if (with_t10 && w == 0) t10(bb);
        }
    };
    // The last chunk's inputs, its K, Q, beta staged and its Gram tiles;
    // inside the loop the next chunk's are staged at the end of the per-wave
    // phase, its diagonal Gram blocks and their inverses formed by the last
    // waves during the C x C phase (where they have no tile), and its other
    // tiles and T_10 by the waves that finish their dQ, dK tiles first (waves
    // 0 .. 3: the second wave on each SIMD runs behind).
    if (c_hi > c_lo) {
        prefetch(std::integral_constant<int, 0>(), c_hi - 1);
        prefetch(std::integral_constant<int, 1>(), c_hi - 1);
        prefetch(std::integral_constant<int, 2>(), c_hi - 1);
        stage_kqb((c_hi - 1) & 1);
        __syncthreads();
        diag_jobs((c_hi - 1) & 1);
        __syncthreads();
        other_jobs((c_hi - 1) & 1, NW);
    }
    // The column work of chunk (parity cb) for this wave's 16 value columns:
    // R and E (products modes), dE, Z, dV and the dS update (recursion
    // modes), publishing E, dV (or Z), dS_{c+1} and the dbeta parts in LDS.
    f32x4 Dold[G::DBUF ? 1 : KT];  // dS_{c+1} kept for the second dK pass (no DBUF)
    auto per_wave = [&](int cb) {
        f32x4 R[NT], E[NT], Z[NT];
        {
            // R = V - K S_c^T (S_c rows of this wave's columns as B^T) and
            // dE = P^T dO + K dS^T share the K row fragments
            typename Frag<DT>::k16 fs[KT], fd[KT];
#pragma unroll
            for (int s = 0; s < KT; ++s) {
                if constexpr (PROD) frag_rows(sm.Sb, LDSK, v0, 16 * s, lane, fs[s]);
                if constexpr (RECUR) cvt4(Dt[s], fd[s]);
            }
            if constexpr (GATED && PROD) {
                // dL/dgamma_last = sum dS_{c+1} (.) S_c over this wave's rows
                float a = 0.f;
#pragma unroll
                for (int s = 0; s < KT; ++s) {
                    if constexpr (RECUR) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) a += Dt[s][i] * frag_get(fs[s], i);
                    } else {
                        typename Frag<DT>::k16 fdd;
                        frag_rows(sm.Db, LDS_, v0, 16 * s, lane, fdd);
#pragma unroll
                        for (int i = 0; i < 4; ++i) a += frag_get(fdd, i) * frag_get(fs[s], i);
                    }
                }
                a = wave_sum(a);
                if (lane == 0) sm.gt.dgc[w] = a * sm.gt.gam[cb][C - 1];
            }
            f32x4 dE[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                typename Frag<DT>::k16 fk[KT];
#pragma unroll
                for (int s = 0; s < KT; ++s) frag_rows(sm.Ks[cb], LDK, 16 * mt, 16 * s, lane, fk[s]);
                if constexpr (PROD) {
                    f32x4 x = zero4();
                    mk_n<DT, KT>(x, fk, fs);
                    typename Frag<DT>::k16 fvv;
                    frag_cols16(sm.Vs, LDV, 16 * mt, v0, lane, fvv);
                    if constexpr (GATED) {
                        // R = V - diag(gamma) K S_c^T
#pragma unroll
                        for (int i = 0; i < 4; ++i) x[i] *= sm.gt.gam[cb][16 * mt + 4 * g + i];
                    }
#pragma unroll
                    for (int i = 0; i < 4; ++i) R[mt][i] = frag_get(fvv, i) - x[i];
                }
                if constexpr (RECUR) {
                    dE[mt] = zero4();
                    // P^T is zero above the diagonal: slabs kt < mt are zeros
                    typename Frag<DT>::k16 fa[NT], fo[NT];
#pragma unroll
                    for (int kt = 0; kt < NT; ++kt) {
                        if (kt >= mt) {
                            frag_cols16(pm_buf(cb), LDC, 16 * kt, 16 * mt, lane, fa[kt]);
                            frag_cols16(os_buf(cb), LDV, 16 * kt, v0, lane, fo[kt]);
                        } else {
                            fa[kt] = fo[kt] = typename Frag<DT>::k16{};
                        }
                    }
                    mk_n<DT, NT>(dE[mt], fa, fo);
                    if constexpr (GATED) {
                        // dE = P^T dO + diag(rho) K dS^T
                        f32x4 kd = zero4();
                        mk_n<DT, KT>(kd, fk, fd);
#pragma unroll
                        for (int i = 0; i < 4; ++i) dE[mt][i] += sm.gt.rto[cb][16 * mt + 4 * g + i] * kd[i];
                    } else {
                        mk_n<DT, KT>(dE[mt], fk, fd);
                    }
                }
            }
            // E = Tm diag(beta) R
            if constexpr (PROD) {
                typename Frag<DT>::k16 frb[NT];
#pragma unroll
                for (int mt = 0; mt < NT; ++mt) {
                    f32x4 rb;
#pragma unroll
                    for (int i = 0; i < 4; ++i) rb[i] = sm.betas[cb][16 * mt + 4 * g + i] * R[mt][i];
                    cvt4(rb, frb[mt]);
                }
#pragma unroll
                for (int mt = 0; mt < NT; ++mt) {
                    E[mt] = zero4();
                    typename Frag<DT>::k16 ft;
#pragma unroll
                    for (int kt = 0; kt <= mt; ++kt) {
                        frag_rows(tm_buf(cb), LDC, 16 * mt, 16 * kt, lane, ft);
                        mk<DT>(E[mt], ft, frb[kt]);
                    }
                }
            }
            if constexpr (RECUR) {
                // Z = Tm^T dE
                typename Frag<DT>::k16 fde[NT];
#pragma unroll
                for (int mt = 0; mt < NT; ++mt) cvt4(dE[mt], fde[mt]);
#pragma unroll
                for (int mt = 0; mt < NT; ++mt) {
                    Z[mt] = zero4();
                    typename Frag<DT>::k16 fa;
#pragma unroll
                    for (int kt = mt; kt < NT; ++kt) {
                        frag_cols16(tm_buf(cb), LDC, 16 * kt, 16 * mt, lane, fa);
                        mk<DT>(Z[mt], fa, fde[kt]);
                    }
                }
            } else {
                // Z of this wave's columns, from the recursion pass
#pragma unroll
                for (int mt = 0; mt < NT; ++mt) {
                    typename Frag<DT>::k16 fz;
                    frag_cols16(sm.Rb, LDV, 16 * mt, v0, lane, fz);
#pragma unroll
                    for (int i = 0; i < 4; ++i) Z[mt][i] = to_f32(frag_get(fz, i));
                }
            }
        }
        // recursion only: dV = diag(beta) Z and Z itself, published for the
        // stores of this chunk
        if constexpr (!PROD) {
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 dvv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * mt + 4 * g + i;
                    dvv[i] = sm.betas[cb][t] * Z[mt][i];
                    sm.Es[t * LDV + v0 + r] = from_f32<DT>(Z[mt][i]);
                    sm.Rb[t * LDV + v0 + r] = from_f32<DT>(dvv[i]);
                }
                Z[mt] = dvv;
            }
        }
        // Y = R - tril(G, -1) E; dbeta parts; dV; publish E and dV
        if constexpr (PROD) {
            typename Frag<DT>::k16 fe[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) cvt4(E[mt], fe[mt]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 ge = zero4();
                typename Frag<DT>::k16 fa;
#pragma unroll
                for (int kt = 0; kt <= mt; ++kt) {
                    frag_rows(sm.Gl[cb], LDC, 16 * mt, 16 * kt, lane, fa);
                    mk<DT>(ge, fa, fe[kt]);
                }
                f32x4 zy;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float y = R[mt][i] - ge[i];
                    // sum over the 16 value columns of this wave (lanes r)
                    zy[i] = group_sum<16>(Z[mt][i] * y);
                }
                if (r == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.dbp[w][16 * mt + 4 * g + i] = zy[i];
                }
                f32x4 dvv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * mt + 4 * g + i;
                    dvv[i] = sm.betas[cb][t] * Z[mt][i];
                    sm.Es[t * LDV + v0 + r] = from_f32<DT>(E[mt][i]);
                    sm.Rb[t * LDV + v0 + r] = from_f32<DT>(dvv[i]);
                }
                Z[mt] = dvv;  // keep dV
            }
        }
        // publish S_c^T and dS_{c+1}^T (this wave's columns) for dQ, dK; then
        // the dS update
        if constexpr (!G::DBUF) {
#pragma unroll
            for (int s2 = 0; s2 < KT; ++s2) Dold[s2] = Dt[s2];
        }
        if constexpr (RECUR) {
            // lane (g, r) holds dS[v0 + r][16 s + 4 g .. + 3]: one vector per tile
            if constexpr (G::DBUF) {
#pragma unroll
                for (int s = 0; s < KT; ++s) {
                    typename Frag<DT>::k16 x;
                    cvt4(Dt[s], x);
                    *reinterpret_cast<typename Frag<DT>::k16 *>(sm.Db + (v0 + r) * LDS_ + 16 * s + 4 * g) = x;
                }
            }
            typename Frag<DT>::k16 fdv[NT], fo[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 nz = -Z[mt];
                frag_cols16(os_buf(cb), LDV, 16 * mt, v0, lane, fo[mt]);
                if constexpr (GATED) {
                    // dS <- gamma_last dS + (diag(gamma) dO)^T Q - (diag(gamma) dV)^T K
                    f32x4 od;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float gm = sm.gt.gam[cb][16 * mt + 4 * g + i];
                        nz[i] *= gm;
                        od[i] = frag_get(fo[mt], i) * gm;
                    }
                    cvt4(od, fo[mt]);
                }
                cvt4(nz, fdv[mt]);
            }
            if constexpr (GATED) {
                const float gc = sm.gt.gam[cb][C - 1];
#pragma unroll
                for (int s = 0; s < KT; ++s) Dt[s] = Dt[s] * gc;
            }
#pragma unroll
            for (int s = 0; s < KT; ++s) {
                typename Frag<DT>::k16 fa[NT], fb[NT];
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    frag_cols16(sm.Qs[cb], LDK, 16 * kt, 16 * s, lane, fa[kt]);
                    frag_cols16(sm.Ks[cb], LDK, 16 * kt, 16 * s, lane, fb[kt]);
                }
                mk_n<DT, NT>(Dt[s], fa, fo);
                mk_n<DT, NT>(Dt[s], fb, fdv);
            }
        }
    };

    constexpr int NWJ = NW < 4 ? NW : 4;  // waves that form the next chunk's Gram tiles
    if constexpr (RONLY) {
        // Recursion only, two barriers per chunk.  Chunk c's K, Q, beta, dO,
        // Tm and Pm sit in the buffers of parity c & 1.  With its column work
        // the waves form chunk c-1's Gram tiles and diagonal inverses (its
        // inputs were staged one chunk earlier); after the barrier, T_10 of
        // chunk c-1, the stores of chunk c (dV, Z, dS_{c+1}; MODE 1 only) and
        // the staging of chunk c-2 (loaded during the column work).
        if (c_hi > c_lo) pf.o.store(os_buf((c_hi - 1) & 1), LDV, tid);
        if (c_hi - c_lo > 1) {
            prefetch(std::integral_constant<int, 1>(), c_hi - 2);
            prefetch(std::integral_constant<int, 2>(), c_hi - 2);
            stage_kqb((c_hi - 2) & 1);
            pf.o.store(os_buf((c_hi - 2) & 1), LDV, tid);
        }
        __syncthreads();
        for (int c = c_hi - 1; c >= c_lo; --c) {
            const int len = min(C, T - c * C);
            const int64_t tok0 = (int64_t)b * T + c * C;
            const int cb = c & 1;
            if (c > c_lo + 1) {
                prefetch(std::integral_constant<int, 1>(), c - 2);
                prefetch(std::integral_constant<int, 2>(), c - 2);
            }
            per_wave(cb);
            if (c > c_lo) {
                diag_jobs(cb ^ 1);
                if (w < NWJ) other_jobs(cb ^ 1, NWJ, false);
            }
            __syncthreads();
            if constexpr (NT == 2)
                if (c > c_lo && w == 0) t10(cb ^ 1);
            if constexpr (MODE == 1) {
                store_rows<DT, C, DV, 64 * NW>(dv + (tok0 * H + h) * DV, (int64_t)H * DV, len,
                                               sm.Rb, LDV, tid);
                store_rows<DT, C, DV, 64 * NW>(dsz + (tok0 * H + h) * DV, (int64_t)H * DV, len,
                                               sm.Es, LDV, tid);
                store_rows<DT, DV, DK, 64 * NW>(dsb + (head * N + c) * DV * DK, DK, DV, sm.Db,
                                                LDS_, tid);
            }
            if (c > c_lo + 1) {
                stage_kqb(cb);
                pf.o.store(os_buf(cb), LDV, tid);
            }
            __syncthreads();
        }
    } else {
        for (int c = c_hi - 1; c >= c_lo; --c) {
            const int len = min(C, T - c * C);
            const int64_t tok0 = (int64_t)b * T + c * C;
            const int cb = c & 1;  // buffer set of this chunk's K, Q, beta, decays
            __syncthreads();
            // ---------------------------------------------------------------- load
            if constexpr (PROD) pf.v.store(sm.Vs, LDV, tid);
            pf.o.store(sm.Os, LDV, tid);
            if constexpr (PROD) pf.s.store(sm.Sb, LDSK, tid);
            if constexpr (MODE == 2) {
                pf.ds.store(sm.Db, LDS_, tid);
                pf.z.store(sm.Rb, LDV, tid);  // Z; each wave turns its columns into dV
            }
            if (c > c_lo) prefetch(std::integral_constant<int, 0>(), c - 1);
            if (GATED && w == 0 && c + 1 < c_hi) finalize_dg(c + 1);
            __syncthreads();

            // ------------------------------------------- per-wave value columns
            if (c > c_lo) prefetch(std::integral_constant<int, 1>(), c - 1);
            per_wave(cb);
            // the next chunk's K, Q, beta (loaded since the start of this phase)
            if (c > c_lo) stage_kqb(cb ^ 1);
            __syncthreads();

            // ---------------------- C x C products over all value columns, dbeta
            // (and the next chunk's diagonal Gram blocks and their inverses)
            if (c > c_lo) diag_jobs(cb ^ 1);
            for (int j = w; PROD && j < 2 * NJ; j += NW) {
                const bool isD = j < NJ;  // dO E^T, else dV E^T
                int jj = isD ? j : j - NJ, ti = 0;
                while (jj > ti) { jj -= ti + 1; ++ti; }
                const int tj = jj;
                f32x4 acc = zero4();
                tile_rr<DT, VT>(acc, isD ? sm.Os : sm.Rb, LDV, 16 * ti, sm.Es, LDV, 16 * tj, 0, lane);
                if constexpr (GATED) {
                    // W = dG (.) tril(K K^T (.) D, -1) + Dm (.) (Q K^T (.) D) off
                    // the diagonal (dL/dD_xy D_xy, D_xy = exp(b_x - b_y)): its row
                    // sums add to dL/db_x, its column sums subtract from dL/db_y.
                    // Dm and dG are stored times D for dQ and dK.
                    f32x4 wv;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int x = 16 * ti + 4 * g + i, y = 16 * tj + r;
                        const float a = isD ? acc[i] : -acc[i];
                        wv[i] = x > y ? a * to_f32((isD ? sm.Pm : sm.Gl[cb])[x * LDC + y]) : 0.f;
                        acc[i] = x > y ? acc[i] * __expf(sm.gt.gb[cb][x] - sm.gt.gb[cb][y]) : acc[i];
                    }
                    float cs = wv[0] + wv[1] + wv[2] + wv[3];
                    cs = xor32_sum(xor16_sum(cs));
                    if (g == 0) sm.gt.wcol[j][r] = cs;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const float rs = group_sum<16>(wv[i]);
                        if (r == 0) sm.gt.wrow[j][4 * g + i] = rs;
                    }
                }
                if (isD) {
                    put_tile(sm.Dm, LDC, 16 * ti, 16 * tj, acc, lane, [](int x, int y) { return x >= y; });
                } else {
                    // dG = -tril(dV E^T, -1), stored with its transpose
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int x = 16 * ti + 4 * g + i, y = 16 * tj + r;
                        const DT val = from_f32<DT>(x > y ? -acc[i] : 0.f);
                        if (x >= y) {
                            sm.Gs[x * LDC + y] = val;
                            sm.Gs[y * LDC + x] = val;
                        }
                    }
                }
            }
            for (int t = tid; PROD && t < len; t += nthr) {
                float sb = 0.f;
#pragma unroll
                for (int ww = 0; ww < NW; ++ww) sb += sm.dbp[ww][t];
                dbeta[(tok0 + t) * H + h] = from_f32<DT>(sb);
            }
            __syncthreads();

            // ------------------------------------------------------- dQ and dK
            if (c > c_lo) prefetch(std::integral_constant<int, 2>(), c - 1);
            if (c + 1 < c_hi) flush(c + 1);
            // dV of all value columns, from its LDS copy, 16 bytes per store
            store_rows<DT, C, DV, 64 * NW>(dv + (tok0 * H + h) * DV, (int64_t)H * DV, len, sm.Rb, LDV, tid);
            // The operands along d_k (columns of S_c, K and Q, rows of
            // dS_{c+1}^T) are read once per key tile and serve all of the wave's
            // token tiles.
            f32x4 dKa[G::DBUF ? 1 : NJW * NMU];
#pragma unroll
            for (int jj = 0; jj < NJW; ++jj) {
                const int j = NW <= KT ? w + jj * NW : w % KT;
                typename Frag<DT>::k16 fs[VT], fkc[NT], fqc[NT], fdb[G::DBUF ? VT : 1];
#pragma unroll
                for (int i = 0; i < VT; ++i) frag_cols16(sm.Sb, LDSK, 16 * i, 16 * j, lane, fs[i]);
#pragma unroll
                for (int i = 0; i < NT; ++i) {
                    frag_cols16(sm.Ks[cb], LDK, 16 * i, 16 * j, lane, fkc[i]);
                    frag_cols16(sm.Qs[cb], LDK, 16 * i, 16 * j, lane, fqc[i]);
                }
                if constexpr (G::DBUF) {
#pragma unroll
                    for (int i = 0; i < VT; ++i) frag_cols16(sm.Db, LDS_, 16 * i, 16 * j, lane, fdb[i]);
                }
#pragma unroll
                for (int u = 0; u < NMU; ++u) {
                    const int mt = mt0 + u * MS;
                    if (mt < NT) {
                        typename Frag<DT>::k16 fa[VT], fb[VT], fm[NT];
                        // dQ = dO S_c + Dm K   (Dm is zero above the diagonal)
                        f32x4 aq = zero4();
#pragma unroll
                        for (int i = 0; i < VT; ++i) frag_rows(sm.Os, LDV, 16 * mt, 16 * i, lane, fa[i]);
#pragma unroll
                        for (int i = 0; i < NT; ++i) frag_rows(sm.Dm, LDC, 16 * mt, 16 * i, lane, fm[i]);
                        mk_n<DT, VT>(aq, fs, fa);
                        const f32x4 aq0 = aq;
                        if constexpr (GATED) aq = aq * sm.gt.gam[cb][16 * mt + r];  // token 16 mt + r
                        mk_n<DT, NT>(aq, fkc, fm);
                        // dK = -dV S_c + E dS_{c+1} + Gs K + Dm^T Q
                        f32x4 an = zero4(), ak = zero4();
#pragma unroll
                        for (int i = 0; i < VT; ++i) frag_rows(sm.Rb, LDV, 16 * mt, 16 * i, lane, fb[i]);
                        mk_n<DT, VT>(an, fs, fb);
                        if constexpr (G::DBUF) {
#pragma unroll
                            for (int i = 0; i < VT; ++i) frag_rows(sm.Es, LDV, 16 * mt, 16 * i, lane, fa[i]);
                            mk_n<DT, VT>(ak, fdb, fa);
                            gate_part(cb, j, mt, aq0, an, &ak, false);
                            if constexpr (GATED) ak = ak * sm.gt.rto[cb][16 * mt + r];
                        } else {
                            gate_part(cb, j, mt, aq0, an, nullptr, false);
                        }
                        if constexpr (GATED) an = an * sm.gt.gam[cb][16 * mt + r];
#pragma unroll
                        for (int i = 0; i < NT; ++i) frag_rows(sm.Gs, LDC, 16 * mt, 16 * i, lane, fm[i]);
                        mk_n<DT, NT>(ak, fkc, fm);
#pragma unroll
                        for (int i = 0; i < NT; ++i) frag_cols16(sm.Dm, LDC, 16 * i, 16 * mt, lane, fm[i]);
                        mk_n<DT, NT>(ak, fqc, fm);
                        ak = ak - an;
                        if constexpr (DEFER) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                frag_set(pq[jj * NMU + u], i, aq[i]);
                                if constexpr (G::DBUF) frag_set(pk[jj * NMU + u], i, ak[i]);
                            }
                        } else {
                            const auto rq = chunk_rsrc(dq, c, rowq, DK), rk = chunk_rsrc(dk, c, rowq, DK);
                            const int voff = ((16 * mt + r) * (int)rowq + 16 * j + 4 * g) * (int)sizeof(DT);
                            out4 x;
#pragma unroll
                            for (int i = 0; i < 4; ++i) frag_set(x, i, aq[i]);
                            store4(x, rq, voff);
                            if constexpr (G::DBUF) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) frag_set(x, i, ak[i]);
                                store4(x, rk, voff);
                            }
                        }
                        if constexpr (!G::DBUF) dKa[jj * NMU + u] = ak;
                    }
                }
            }
            if constexpr (!G::DBUF) {
                // second pass: dS_{c+1} replaces S_c, then dK += E dS_{c+1}
                __syncthreads();
#pragma unroll
                for (int s2 = 0; s2 < KT; ++s2)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        sm.Sb[(v0 + r) * LDSK + 16 * s2 + 4 * g + i] = from_f32<DT>(Dold[s2][i]);
                __syncthreads();
#pragma unroll
                for (int jj = 0; jj < NJW; ++jj) {
                    const int j = NW <= KT ? w + jj * NW : w % KT;
                    typename Frag<DT>::k16 fs[VT];
#pragma unroll
                    for (int i = 0; i < VT; ++i) frag_cols16(sm.Sb, LDSK, 16 * i, 16 * j, lane, fs[i]);
#pragma unroll
                    for (int u = 0; u < NMU; ++u) {
                        const int mt = mt0 + u * MS;
                        if (mt < NT) {
                            typename Frag<DT>::k16 fa[VT];
                            f32x4 ak = dKa[jj * NMU + u];
#pragma unroll
                            for (int i = 0; i < VT; ++i) frag_rows(sm.Es, LDV, 16 * mt, 16 * i, lane, fa[i]);
                            if constexpr (GATED) {
                                f32x4 ed = zero4();
                                mk_n<DT, VT>(ed, fs, fa);
                                gate_part(cb, j, mt, zero4(), zero4(), &ed, true);
                                ak += ed * sm.gt.rto[cb][16 * mt + r];
                            } else {
                                mk_n<DT, VT>(ak, fs, fa);
                            }
                            if constexpr (DEFER) {
#pragma unroll
                                for (int i = 0; i < 4; ++i) frag_set(pk[jj * NMU + u], i, ak[i]);
                            } else {
                                const auto rk = chunk_rsrc(dk, c, rowq, DK);
                                out4 x;
#pragma unroll
                                for (int i = 0; i < 4; ++i) frag_set(x, i, ak[i]);
                                store4(x, rk, ((16 * mt + r) * (int)rowq + 16 * j + 4 * g) * (int)sizeof(DT));
                            }
                        }
                    }
                }
            }
            // the next chunk's other Gram tiles and T_10
            if (c > c_lo && w < NWJ) other_jobs(cb ^ 1, NWJ);
        }
    }
    if (PROD && c_hi > c_lo) flush(c_lo);
    if (PROD && GATED && c_hi > c_lo) {
        __syncthreads();
        if (w == 0) finalize_dg(c_lo);
    }
    if (RECUR && dS0 && (MODE == 3 || !segd || part == 0)) {
        const int64_t oidx = MODE == 3 ? sidx : head;
#pragma unroll
        for (int s = 0; s < KT; ++s)
            *reinterpret_cast<f32x4 *>(dS0 + (oidx * DV + v0 + r) * DK + 16 * s + 4 * g) = Dt[s];
    }
}

// Workgroups per (b, h) of the products-only pass: as many as fill the
// compute units once.  Fewer than 4 means the single-pass kernel: per chunk
// the recursion pass takes about half the single pass's time and the
// products pass about as long as the single pass (the clock drops with
// every compute unit busy), so two workgroups per (b, h) lose.
inline int bwd_nsplit(int64_t BH, int N) {
    const int64_t n = 256 / (BH > 0 ? BH : 1);
    const int ns = (int)(n < N ? n : N);
    return ns >= 4 ? ns : 1;
}

// nsplit: workgroups per (b, h) of MODE 2; segP, segL: segments per (b, h)
// and chunks per segment of a segmented MODE 1 / MODE 3 launch.
template <typename DT, int DK, int DV, bool GATED, int MODE>
hipError_t launch_bwd_mode(const ChunkBwdArgs &a, int nsplit, hipStream_t stream, int c_beg = 0,
                           int c_end = INT_MAX, int segP = 1, int segL = 0, bool ident = false) {
    const int nper = MODE == 2 ? nsplit : (MODE == 1 || MODE == 3) && segP > 1 ? segP : 1;
    hipLaunchKernelGGL((chunk_bwd_kernel<DT, DK, DV, sizeof(DT) == 2 ? 32 : 16, GATED, MODE>),
                       dim3((unsigned)(a.B * a.H * nper)), dim3(DV * 4), 0,
                       stream, static_cast<const DT *>(a.q), static_cast<const DT *>(a.k),
                       static_cast<const DT *>(a.v), static_cast<const DT *>(a.beta), a.g,
                       static_cast<const DT *>(a.dout), a.dS_T, static_cast<const DT *>(a.h),
                       static_cast<DT *>(a.dq), static_cast<DT *>(a.dk), static_cast<DT *>(a.dv),
                       static_cast<DT *>(a.dbeta), a.dg, a.dS0, static_cast<DT *>(a.dsb),
                       static_cast<DT *>(a.dsz), (int)a.T, (int)a.H, nsplit, c_beg, c_end,
                       segP, segL, ident ? 1 : 0);
    return hipGetLastError();
}

// A second stream per device, with a fork and a join event, for the split
// reverse walk below.  Created on first use with the device current (default
// priority); a mutex per device keeps each call's record / wait / launch
// sequence whole, so calls from several host threads stay ordered.
struct SideStream {
    hipStream_t s = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    hipError_t err = hipSuccess;
    std::mutex mu;
};
constexpr int BWD_MAX_DEVICES = 64;
std::once_flag g_side_once[BWD_MAX_DEVICES];
SideStream g_side[BWD_MAX_DEVICES];

hipError_t side_stream(SideStream **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= BWD_MAX_DEVICES) return hipErrorInvalidDevice;
    SideStream &ss = g_side[dev];
    std::call_once(g_side_once[dev], [&ss] {
        ss.err = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
        if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
        if (ss.err == hipSuccess) ss.err = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    });
    if (ss.err != hipSuccess) return ss.err;
    *out = &ss;
    return hipSuccess;
}

// Reverse walk in two pieces for B*H <= 128 (one workgroup per (b, h)
// leaves half the compute units idle): on the caller's stream the recursion
// alone (MODE 3, about half a single-pass chunk step) walks chunks [m, N)
// from dS_T to give dS at chunk m, and then the single pass over chunks
// [0, m) starts from it; meanwhile, on the side stream, the single pass over
// chunks [m, N) runs from dS_T.  The caller's stream, which holds the
// critical path, waits for nothing but the join at the end (a stream that
// waits on an event starts its next kernel several microseconds late).  The
// two sides take about as long when m is ~11/32 of the chunks (measured:
// 8/32, 13/32 and 15/32 were slower).  dS at chunk m (fp32, [B,H,Dv,Dk])
// goes to the workspace's scratch region (dsb).
constexpr int BWD_SPLIT_NUM = 11, BWD_SPLIT_DEN = 32;
constexpr int BWD_SPLIT_MIN_CHUNKS = 8;

template <typename DT, int DK, int DV, bool GATED>
hipError_t launch_bwd_split(const ChunkBwdArgs &a, int N, hipStream_t stream) {
    SideStream *ss = nullptr;
    hipError_t e = side_stream(&ss);
    if (e != hipSuccess) return e;
    const int m = N * BWD_SPLIT_NUM / BWD_SPLIT_DEN;
    float *mid = static_cast<float *>(a.dsb);
    ChunkBwdArgs tail = a, rec = a, head = a;
    tail.dS0 = nullptr;                 // [m, N) from dS_T; dS0 comes from the head piece
    rec.dS0 = mid;                      // dS at chunk m
    rec.dsb = rec.dsz = nullptr;
    head.dS_T = mid;                    // [0, m) from dS at chunk m
    std::lock_guard<std::mutex> lock(ss->mu);
    if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
    if ((e = launch_bwd_mode<DT, DK, DV, GATED, 0>(tail, 1, ss->s, m, N)) != hipSuccess) return e;
    if ((e = launch_bwd_mode<DT, DK, DV, GATED, 3>(rec, 1, stream, m, N)) != hipSuccess) return e;
    if ((e = launch_bwd_mode<DT, DK, DV, GATED, 0>(head, 1, stream, 0, m)) != hipSuccess) return e;
    if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
    return hipStreamWaitEvent(stream, ss->join, 0);
}

// Segmented recursion for few (b, h) (B*H <= 32, at least 4 segments of at
// least 4 chunks).  The dS recursion over a segment is affine in the dS that
// enters it (every chunk maps dS -> dS A_c + B_c, rows independently), so
//   dS_start(p) = dS_end(p) A_p + B_p,  dS_end(p) = dS_start(p + 1),
// with A_p the segment's map (the recursion from the identity with dO = 0:
// MODE 3, ident, null dout, d_v := d_k) and B_p its response to dO from zero
// (MODE 3).  Both run over all segments at once, the map on the side stream;
// the chain (segment.hip, last segment first) then turns them into every
// segment's entering dS, the recursion pass (MODE 1) runs over all segments
// at once from those, and the products pass follows as before.
constexpr int BWD_SEG_MAX_HEADS = 32, BWD_SEG_MIN = 4, BWD_SEG_MAX = 16;
constexpr int BWD_SEG_MIN_CHUNKS = 4;

int64_t al256(int64_t x) { return (x + 255) / 256 * 256; }

template <typename DT, int DK, int DV, bool GATED>
hipError_t launch_bwd_segmented(const ChunkBwdArgs &a, const BwdSegPlan &sp, int ns,
                                hipStream_t stream) {
    SideStream *ss = nullptr;
    hipError_t e = side_stream(&ss);
    if (e != hipSuccess) return e;
    float *Bs = static_cast<float *>(a.segws);  // B_p, then each segment's entering dS
    float *As = reinterpret_cast<float *>(static_cast<char *>(a.segws) +
                                          al256(a.B * sp.P * a.H * (int64_t)DV * DK * 4));
    ChunkBwdArgs aff = a, map = a, rec = a;
    aff.dS_T = nullptr;
    aff.dS0 = Bs;
    aff.dsb = aff.dsz = nullptr;
    map.Dv = DK;
    map.v = map.dout = nullptr;
    map.dv = nullptr;
    map.dS_T = nullptr;
    map.dS0 = As;
    map.dsb = map.dsz = nullptr;
    rec.dS_T = Bs;
    {
        std::lock_guard<std::mutex> lock(ss->mu);
        if ((e = hipEventRecord(ss->fork, stream)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(ss->s, ss->fork, 0)) != hipSuccess) return e;
        if ((e = launch_bwd_mode<DT, DK, DK, GATED, 3>(map, 1, ss->s, 0, INT_MAX, sp.P, sp.L,
                                                       true)) != hipSuccess)
            return e;
        if ((e = launch_bwd_mode<DT, DK, DV, GATED, 3>(aff, 1, stream, 0, INT_MAX, sp.P, sp.L,
                                                       false)) != hipSuccess)
            return e;
        if ((e = hipEventRecord(ss->join, ss->s)) != hipSuccess) return e;
        if ((e = hipStreamWaitEvent(stream, ss->join, 0)) != hipSuccess) return e;
    }
    if ((e = launch_seg_chain(Bs, As, a.dS_T, nullptr, a.B, sp.P, a.H, DK, DV, true, stream)) !=
        hipSuccess)
        return e;
    if ((e = launch_bwd_mode<DT, DK, DV, GATED, 1>(rec, 1, stream, 0, INT_MAX, sp.P, sp.L)) !=
        hipSuccess)
        return e;
    return launch_bwd_mode<DT, DK, DV, GATED, 2>(a, ns, stream);
}

// One reverse pass per (b, h); where that leaves compute units idle and the
// caller gave the scratch (dsb, dsz), either the recursion pass (segmented
// for few heads, above) then the products pass over nsplit runs of chunks
// per (b, h) (up to 64 heads), or the reverse walk in two pieces on two
// streams (up to 128 heads).
template <typename DT, int DK, int DV, bool GATED>
hipError_t launch_bwd_gate(const ChunkBwdArgs &a, hipStream_t stream) {
    constexpr int C = sizeof(DT) == 2 ? 32 : 16;
    if constexpr (!bwd_fits<DT, DK, DV, C, GATED>()) {
        return hipErrorInvalidValue;
    } else {
        if constexpr (BwdCfg<DT, DK, DV, C>::DBUF) {
            const int N = (int)((a.T + C - 1) / C);
            const int ns = bwd_nsplit(a.B * a.H, N);
            if (a.dsb && a.dsz && ns >= 2) {
                if constexpr (bwd_fits<DT, DK, DK, C, GATED>() && BwdCfg<DT, DK, DK, C>::DBUF) {
                    const BwdSegPlan sp = bwd_seg_plan(a.B, a.H, N);
                    if (a.segws && sp.P > 0)
                        return launch_bwd_segmented<DT, DK, DV, GATED>(a, sp, ns, stream);
                }
                const hipError_t e = launch_bwd_mode<DT, DK, DV, GATED, 1>(a, 1, stream);
                if (e != hipSuccess) return e;
                return launch_bwd_mode<DT, DK, DV, GATED, 2>(a, ns, stream);
            }
            if (a.dsb && a.B * a.H <= 128 && N >= BWD_SPLIT_MIN_CHUNKS)
                return launch_bwd_split<DT, DK, DV, GATED>(a, N, stream);
        }
        return launch_bwd_mode<DT, DK, DV, GATED, 0>(a, 1, stream);
    }
}

template <typename DT, int DK, int DV>
hipError_t launch_bwd_cfg(const ChunkBwdArgs &a, hipStream_t stream) {
    return a.g ? launch_bwd_gate<DT, DK, DV, true>(a, stream)
               : launch_bwd_gate<DT, DK, DV, false>(a, stream);
}

template <typename DT, int DK>
hipError_t bwd_dv(const ChunkBwdArgs &a, hipStream_t stream) {
    switch (a.Dv) {
    case 16: return launch_bwd_cfg<DT, DK, 16>(a, stream);
    case 32: return launch_bwd_cfg<DT, DK, 32>(a, stream);
    case 64: return launch_bwd_cfg<DT, DK, 64>(a, stream);
    case 128: return launch_bwd_cfg<DT, DK, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

template <typename DT>
hipError_t bwd_dk(const ChunkBwdArgs &a, hipStream_t stream) {
    switch (a.Dk) {
    case 16: return bwd_dv<DT, 16>(a, stream);
    case 32: return bwd_dv<DT, 32>(a, stream);
    case 64: return bwd_dv<DT, 64>(a, stream);
    case 128: return bwd_dv<DT, 128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

int chunk_bwd_chunk(bool bf16) { return bf16 ? 32 : 16; }

BwdSegPlan bwd_seg_plan(int64_t B, int64_t H, int64_t N) {
    BwdSegPlan pl{0, 0};
    const int64_t BH = B * H;
    if (BH <= 0 || BH > BWD_SEG_MAX_HEADS || N <= 0) return pl;
    int64_t P = std::min<int64_t>(std::min<int64_t>(128 / BH, N / BWD_SEG_MIN_CHUNKS), BWD_SEG_MAX);
    if (P < BWD_SEG_MIN) return pl;
    const int64_t L = (N + P - 1) / P;
    P = (N + L - 1) / L;
    if (P < BWD_SEG_MIN) return pl;
    pl.P = (int)P;
    pl.L = (int)L;
    return pl;
}

int64_t bwd_seg_bytes(int64_t B, int64_t H, int64_t N, int64_t Dk, int64_t Dv) {
    const BwdSegPlan pl = bwd_seg_plan(B, H, N);
    if (pl.P == 0) return 0;
    return al256(B * pl.P * H * Dv * Dk * 4) + al256(B * pl.P * H * Dk * Dk * 4);
}

hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, bool bf16, hipStream_t stream) {
    return bf16 ? bwd_dk<__bf16>(a, stream) : bwd_dk<float>(a, stream);
}

}  // namespace dr
