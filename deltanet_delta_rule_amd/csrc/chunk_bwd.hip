// Backward of the chunked delta rule (plain rule, gfx950).
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
// Work split.  One workgroup per (b, h) walks the chunks in reverse.  Wave w
// owns value columns 16w .. 16w+15: its slices of R, E, dE, Z, dV and the
// rows of dS (kept transposed, d_k x 16, as fp32 MFMA accumulators for the
// whole sequence).  The state S_c of each chunk comes from checkpoints the
// forward kernel writes.  Products that sum over all value columns (dO E^T,
// dV E^T, dQ, dK) run after the waves have published their slices in LDS,
// with output tiles dealt round-robin to the waves.  Chunks are 32 tokens for
// bf16 and 16 for fp32 (LDS capacity), which the forward checkpoints follow.
#include "dr_common.hpp"
#include "dr_launch.hpp"

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
    static constexpr int LDS_ = DV + PAD;         // dS^T rows (d_k x d_v)
    static constexpr int LDSK = DK + PAD;         // S_c rows (d_v x d_k)
    static constexpr int LDC = C + PAD;           // C x C matrices
    // dS_{c+1}^T gets its own LDS buffer unless that overflows LDS (fp32 with
    // d_k = d_v = 128); then it reuses the S_c^T buffer in a second pass.
    static constexpr int BASE = (int)sizeof(DT) * (2 * C * LDK + 4 * C * LDV + DV * LDSK + 5 * C * LDC) +
                                4 * C * (1 + NW);
    static constexpr bool DBUF = BASE + (int)sizeof(DT) * DK * LDS_ + 256 <= 160 * 1024;
};

template <typename DT, int DK, int DV, int C>
struct BwdSmem {
    typedef BwdCfg<DT, DK, DV, C> G;
    DT Ks[C * G::LDK], Qs[C * G::LDK];
    DT Vs[C * G::LDV], Os[C * G::LDV];            // V, dO
    DT Es[C * G::LDV], Rb[C * G::LDV];            // E, dV
    DT Sb[DV * G::LDSK];                          // S_c (rows: value index); second
                                                  // pass without DBUF: dS_{c+1}
    DT Db[G::DBUF ? DK * G::LDS_ : 8];            // dS_{c+1}^T (DBUF)
    DT Pm[C * G::LDC];                            // Q K^T (.) M
    DT Gl[C * G::LDC];                            // tril(K K^T, -1)
    DT Tm[C * G::LDC];                            // (I + A)^{-1}
    DT Dm[C * G::LDC];                            // dO E^T (.) M
    DT Gs[C * G::LDC];                            // dG + dG^T
    float betas[C];
    float dbp[G::NW][C];                          // per-wave parts of dbeta
};

template <typename DT, int DK, int DV, int C>
constexpr bool bwd_fits() {
    return sizeof(BwdSmem<DT, DK, DV, C>) <= 160 * 1024;
}

// One 16x16x16 product step on 16-wide fragments of DT.
template <typename DT>
__device__ __forceinline__ void mk(f32x4 &acc, const typename Frag<DT>::k16 &a,
                                   const typename Frag<DT>::k16 &b) {
    mma_k16(acc, a, b);
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
#pragma unroll
    for (int i = 0; i < NK; ++i) mk<DT>(acc, fa[i], fb[i]);
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
#pragma unroll
    for (int i = 0; i < NK; ++i) mk<DT>(acc, fa[i], fb[i]);
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
#pragma unroll
    for (int i = 0; i < NK; ++i) mk<DT>(acc, fa[i], fb[i]);
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
    __device__ __forceinline__ void store(DT *dst, int ld, int tid) const {
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int i = tid + j * NTHR;
            if (i < NV) {
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
    float b;
    __device__ __forceinline__ void load(const DT *kk, const DT *qq, const DT *vv, const DT *oo,
                                         const DT *bb, const DT *sc, int64_t tok0, int h, int H,
                                         int len, int tid) {
        const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;
        k.load(kk + (tok0 * H + h) * DK, rk, len, tid);
        q.load(qq + (tok0 * H + h) * DK, rk, len, tid);
        v.load(vv + (tok0 * H + h) * DV, rv, len, tid);
        o.load(oo + (tok0 * H + h) * DV, rv, len, tid);
        s.load(sc, DK, DV, tid);
        b = tid < len ? to_f32(bb[(tok0 + tid) * H + h]) : 0.f;
    }
};

template <typename DT, int DK, int DV, int C>
__global__ __launch_bounds__(DV * 4) void chunk_bwd_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const DT *__restrict__ dout, const float *__restrict__ dST,
    const DT *__restrict__ hs, DT *__restrict__ dq, DT *__restrict__ dk, DT *__restrict__ dv,
    DT *__restrict__ dbeta, float *__restrict__ dS0, int T, int H) {
    typedef BwdCfg<DT, DK, DV, C> G;
    constexpr int NW = G::NW, NT = G::NT, KT = G::KT, VT = G::VT;
    constexpr int LDK = G::LDK, LDV = G::LDV, LDS_ = G::LDS_, LDSK = G::LDSK, LDC = G::LDC;
    __shared__ __attribute__((aligned(16))) BwdSmem<DT, DK, DV, C> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int v0 = 16 * w;
    const int64_t head = blockIdx.x;
    const int b = (int)(head / H), h = (int)(head % H);
    const int N = (T + C - 1) / C;
    const int nthr = 64 * NW;

    // upper tiles of the C x C matrices stay zero
    for (int i = tid; i < C * LDC; i += nthr) {
        sm.Pm[i] = sm.Gl[i] = sm.Tm[i] = sm.Dm[i] = sm.Gs[i] = from_f32<DT>(0.f);
    }
    // dS^T of this wave's value columns: tile s holds dS^T[16s + 4g + i][v0 + r]
    f32x4 Dt[KT];
#pragma unroll
    for (int s = 0; s < KT; ++s) {
        Dt[s] = dST ? *reinterpret_cast<const f32x4 *>(dST + (head * DV + v0 + r) * DK + 16 * s + 4 * g)
                    : zero4();
    }

    // inputs of the next chunk to process travel in registers one chunk ahead
    ChunkPrefetch<DT, DK, DV, C> pf;
    if (N > 0) {
        const int t0 = (N - 1) * C;
        pf.load(k, q, v, dout, beta, hs + (head * N + N - 1) * DV * DK, (int64_t)b * T + t0, h, H,
                min(C, T - t0), tid);
    }
    for (int c = N - 1; c >= 0; --c) {
        const int t0 = c * C, len = min(C, T - t0);
        const int64_t tok0 = (int64_t)b * T + t0;
        __syncthreads();
        // ---------------------------------------------------------------- load
        pf.k.store(sm.Ks, LDK, tid);
        pf.q.store(sm.Qs, LDK, tid);
        pf.v.store(sm.Vs, LDV, tid);
        pf.o.store(sm.Os, LDV, tid);
        pf.s.store(sm.Sb, LDSK, tid);
        if (tid < C) sm.betas[tid] = pf.b;
        if (c > 0) {
            const int tp = (c - 1) * C;
            pf.load(k, q, v, dout, beta, hs + (head * N + c - 1) * DV * DK, (int64_t)b * T + tp, h,
                    H, min(C, T - tp), tid);
        }
        __syncthreads();

        // ---------------------------------------------------- Gram and inverse
        // jobs: lower tiles (ti >= tj) of G = K K^T and P = Q K^T
        constexpr int NJ = NT * (NT + 1) / 2;
        for (int j = w; j < 2 * NJ; j += NW) {
            const bool isP = j >= NJ;
            int jj = isP ? j - NJ : j, ti = 0;
            while (jj > ti) { jj -= ti + 1; ++ti; }
            const int tj = jj;
            f32x4 acc = zero4();
            tile_rr<DT, KT>(acc, isP ? sm.Qs : sm.Ks, LDK, 16 * ti, sm.Ks, LDK, 16 * tj, 0, lane);
            if (isP) {
                put_tile(sm.Pm, LDC, 16 * ti, 16 * tj, acc, lane, [](int x, int y) { return x >= y; });
            } else {
                put_tile(sm.Gl, LDC, 16 * ti, 16 * tj, acc, lane, [](int x, int y) { return x > y; });
                if (ti == tj) {
                    // A and A^T of the diagonal block: A[x][y] = beta_x G[x][y], x > y
                    f32x4 a, at;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int x = 4 * g + i;
                        a[i] = x > r ? sm.betas[16 * ti + x] * acc[i] : 0.f;
                        at[i] = r > x ? sm.betas[16 * ti + r] * acc[i] : 0.f;  // G symmetric
                    }
                    const f32x4 tinv = inv_unit_lower<DT>(a, at, lane);
                    put_tile(sm.Tm, LDC, 16 * ti, 16 * ti, tinv, lane, [](int x, int y) { return x >= y; });
                }
            }
        }
        __syncthreads();
        if constexpr (NT == 2) {
            // off-diagonal block: T_10 = -T_11 (A_10 T_00), A_10 = diag(beta_1) G_10
            if (w == 0) {
                typename Frag<DT>::k16 fa, fb;
                f32x4 m1 = zero4();
                frag_rows(sm.Gl, LDC, 16, 0, lane, fa);
                {
                    f32x4 tmp;
#pragma unroll
                    for (int i = 0; i < 4; ++i) tmp[i] = frag_get(fa, i) * sm.betas[16 + r];
                    cvt4(tmp, fa);
                }
                frag_cols16(sm.Tm, LDC, 0, 0, lane, fb);
                mk<DT>(m1, fa, fb);
                f32x4 t10 = zero4();
                frag_rows(sm.Tm, LDC, 16, 16, lane, fa);
                cvt4(m1, fb);
                mk<DT>(t10, fa, fb);
                put_tile(sm.Tm, LDC, 16, 0, -t10, lane, [](int, int) { return true; });
            }
            __syncthreads();
        }

        // ------------------------------------------- per-wave value columns
        f32x4 R[NT], E[NT], Z[NT];
        {
            // R = V - K S_c^T (S_c rows of this wave's columns as B^T)
            typename Frag<DT>::k16 fs[KT];
#pragma unroll
            for (int s = 0; s < KT; ++s) frag_rows(sm.Sb, LDSK, v0, 16 * s, lane, fs[s]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 x = zero4();
                typename Frag<DT>::k16 fk[KT];
#pragma unroll
                for (int s = 0; s < KT; ++s) frag_rows(sm.Ks, LDK, 16 * mt, 16 * s, lane, fk[s]);
#pragma unroll
                for (int s = 0; s < KT; ++s) mk<DT>(x, fk[s], fs[s]);
                typename Frag<DT>::k16 fvv;
                frag_cols16(sm.Vs, LDV, 16 * mt, v0, lane, fvv);
#pragma unroll
                for (int i = 0; i < 4; ++i) R[mt][i] = frag_get(fvv, i) - x[i];
            }
            // E = Tm diag(beta) R
            typename Frag<DT>::k16 frb[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 rb;
#pragma unroll
                for (int i = 0; i < 4; ++i) rb[i] = sm.betas[16 * mt + 4 * g + i] * R[mt][i];
                cvt4(rb, frb[mt]);
            }
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                E[mt] = zero4();
                typename Frag<DT>::k16 ft;
#pragma unroll
                for (int kt = 0; kt <= mt; ++kt) {
                    frag_rows(sm.Tm, LDC, 16 * mt, 16 * kt, lane, ft);
                    mk<DT>(E[mt], ft, frb[kt]);
                }
            }
            // dE = P^T dO + K dS^T, then Z = Tm^T dE
            typename Frag<DT>::k16 fd[KT];
#pragma unroll
            for (int s = 0; s < KT; ++s) cvt4(Dt[s], fd[s]);
            f32x4 dE[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                dE[mt] = zero4();
                typename Frag<DT>::k16 fa, fo;
#pragma unroll
                for (int kt = mt; kt < NT; ++kt) {
                    frag_cols16(sm.Pm, LDC, 16 * kt, 16 * mt, lane, fa);
                    frag_cols16(sm.Os, LDV, 16 * kt, v0, lane, fo);
                    mk<DT>(dE[mt], fa, fo);
                }
                typename Frag<DT>::k16 fks[KT];
#pragma unroll
                for (int s = 0; s < KT; ++s) frag_rows(sm.Ks, LDK, 16 * mt, 16 * s, lane, fks[s]);
#pragma unroll
                for (int s = 0; s < KT; ++s) mk<DT>(dE[mt], fks[s], fd[s]);
            }
            typename Frag<DT>::k16 fde[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) cvt4(dE[mt], fde[mt]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                Z[mt] = zero4();
                typename Frag<DT>::k16 fa;
#pragma unroll
                for (int kt = mt; kt < NT; ++kt) {
                    frag_cols16(sm.Tm, LDC, 16 * kt, 16 * mt, lane, fa);
                    mk<DT>(Z[mt], fa, fde[kt]);
                }
            }
        }
        // Y = R - tril(G, -1) E; dbeta parts; dV; publish E and dV
        {
            typename Frag<DT>::k16 fe[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) cvt4(E[mt], fe[mt]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 ge = zero4();
                typename Frag<DT>::k16 fa;
#pragma unroll
                for (int kt = 0; kt <= mt; ++kt) {
                    frag_rows(sm.Gl, LDC, 16 * mt, 16 * kt, lane, fa);
                    mk<DT>(ge, fa, fe[kt]);
                }
                f32x4 zy;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float y = R[mt][i] - ge[i];
                    float p = Z[mt][i] * y;
                    // sum over the 16 value columns of this wave (lanes r)
#pragma unroll
                    for (int m = 8; m >= 1; m >>= 1) p += __shfl_xor(p, m, 16);
                    zy[i] = p;
                }
                if (r == 0) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) sm.dbp[w][16 * mt + 4 * g + i] = zy[i];
                }
                f32x4 dvv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * mt + 4 * g + i;
                    dvv[i] = sm.betas[t] * Z[mt][i];
                    sm.Es[t * LDV + v0 + r] = from_f32<DT>(E[mt][i]);
                    sm.Rb[t * LDV + v0 + r] = from_f32<DT>(dvv[i]);
                    if (t < len) dv[((tok0 + t) * H + h) * DV + v0 + r] = from_f32<DT>(dvv[i]);
                }
                Z[mt] = dvv;  // keep dV
            }
        }
        // publish S_c^T and dS_{c+1}^T (this wave's columns) for dQ, dK; then
        // the dS update
        f32x4 Dold[G::DBUF ? 1 : KT];
        if constexpr (!G::DBUF) {
#pragma unroll
            for (int s2 = 0; s2 < KT; ++s2) Dold[s2] = Dt[s2];
        }
        {
#pragma unroll
            for (int s = 0; s < KT; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    if constexpr (G::DBUF)
                        sm.Db[(16 * s + 4 * g + i) * LDS_ + v0 + r] = from_f32<DT>(Dt[s][i]);
                }
            typename Frag<DT>::k16 fdv[NT], fo[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 nz = -Z[mt];
                cvt4(nz, fdv[mt]);
                frag_cols16(sm.Os, LDV, 16 * mt, v0, lane, fo[mt]);
            }
#pragma unroll
            for (int s = 0; s < KT; ++s) {
                typename Frag<DT>::k16 fa[NT], fb[NT];
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    frag_cols16(sm.Qs, LDK, 16 * kt, 16 * s, lane, fa[kt]);
                    frag_cols16(sm.Ks, LDK, 16 * kt, 16 * s, lane, fb[kt]);
                }
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    mk<DT>(Dt[s], fa[kt], fo[kt]);
                    mk<DT>(Dt[s], fb[kt], fdv[kt]);
                }
            }
        }
        __syncthreads();

        // ---------------------- C x C products over all value columns, dbeta
        for (int j = w; j < 2 * NJ; j += NW) {
            const bool isD = j < NJ;  // dO E^T, else dV E^T
            int jj = isD ? j : j - NJ, ti = 0;
            while (jj > ti) { jj -= ti + 1; ++ti; }
            const int tj = jj;
            f32x4 acc = zero4();
            tile_rr<DT, VT>(acc, isD ? sm.Os : sm.Rb, LDV, 16 * ti, sm.Es, LDV, 16 * tj, 0, lane);
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
        for (int t = tid; t < len; t += nthr) {
            float s = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) s += sm.dbp[ww][t];
            dbeta[(tok0 + t) * H + h] = from_f32<DT>(s);
        }
        __syncthreads();

        // ------------------------------------------------------- dQ and dK
        constexpr int NO = NT * KT;  // output tiles of each
        constexpr int NU = (NO + NW - 1) / NW;
        f32x4 dKa[G::DBUF ? 1 : NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int o = w + u * NW;
            if (o < NO) {
                const int mt = o / KT, j = o % KT;
                // dQ = dO S_c + Dm K   (Dm is zero above the diagonal)
                f32x4 aq = zero4();
                tile_rc<DT, VT>(aq, sm.Os, LDV, 16 * mt, sm.Sb, LDSK, 16 * j, 0, lane);
                tile_rc<DT, NT>(aq, sm.Dm, LDC, 16 * mt, sm.Ks, LDK, 16 * j, 0, lane);
                // dK = -dV S_c + E dS_{c+1} + Gs K + Dm^T Q
                f32x4 ak = zero4();
                tile_rc<DT, VT>(ak, sm.Rb, LDV, 16 * mt, sm.Sb, LDSK, 16 * j, 0, lane);
                ak = -ak;
                if constexpr (G::DBUF)
                    tile_rr<DT, VT>(ak, sm.Es, LDV, 16 * mt, sm.Db, LDS_, 16 * j, 0, lane);
                tile_rc<DT, NT>(ak, sm.Gs, LDC, 16 * mt, sm.Ks, LDK, 16 * j, 0, lane);
                tile_cc<DT, NT>(ak, sm.Dm, LDC, 16 * mt, sm.Qs, LDK, 16 * j, 0, lane);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int t = 16 * mt + 4 * g + i;
                    if (t < len) dq[((tok0 + t) * H + h) * DK + 16 * j + r] = from_f32<DT>(aq[i]);
                }
                if constexpr (G::DBUF) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * mt + 4 * g + i;
                        if (t < len) dk[((tok0 + t) * H + h) * DK + 16 * j + r] = from_f32<DT>(ak[i]);
                    }
                } else {
                    dKa[u] = ak;
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
            for (int u = 0; u < NU; ++u) {
                const int o = w + u * NW;
                if (o < NO) {
                    const int mt = o / KT, j = o % KT;
                    f32x4 ak = dKa[u];
                    tile_rc<DT, VT>(ak, sm.Es, LDV, 16 * mt, sm.Sb, LDSK, 16 * j, 0, lane);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = 16 * mt + 4 * g + i;
                        if (t < len) dk[((tok0 + t) * H + h) * DK + 16 * j + r] = from_f32<DT>(ak[i]);
                    }
                }
            }
        }
    }
    if (dS0) {
#pragma unroll
        for (int s = 0; s < KT; ++s)
            *reinterpret_cast<f32x4 *>(dS0 + (head * DV + v0 + r) * DK + 16 * s + 4 * g) = Dt[s];
    }
}

template <typename DT, int DK, int DV>
hipError_t launch_bwd_cfg(const ChunkBwdArgs &a, hipStream_t stream) {
    constexpr int C = sizeof(DT) == 2 ? 32 : 16;
    if constexpr (!bwd_fits<DT, DK, DV, C>()) {
        return hipErrorInvalidValue;
    } else {
        hipLaunchKernelGGL((chunk_bwd_kernel<DT, DK, DV, C>), dim3((unsigned)(a.B * a.H)),
                           dim3(DV * 4), 0, stream, static_cast<const DT *>(a.q),
                           static_cast<const DT *>(a.k), static_cast<const DT *>(a.v),
                           static_cast<const DT *>(a.beta), static_cast<const DT *>(a.dout),
                           a.dS_T, static_cast<const DT *>(a.h), static_cast<DT *>(a.dq), static_cast<DT *>(a.dk),
                           static_cast<DT *>(a.dv), static_cast<DT *>(a.dbeta), a.dS0,
                           (int)a.T, (int)a.H);
        return hipGetLastError();
    }
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

hipError_t launch_chunk_bwd(const ChunkBwdArgs &a, bool bf16, hipStream_t stream) {
    return bf16 ? bwd_dk<__bf16>(a, stream) : bwd_dk<float>(a, stream);
}

}  // namespace dr
