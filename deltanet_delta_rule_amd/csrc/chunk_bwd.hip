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
    static constexpr int LDS_ = DV + PAD;         // S_c^T / dS^T rows (d_k x d_v)
    static constexpr int LDC = C + PAD;           // C x C matrices
};

template <typename DT, int DK, int DV, int C>
struct BwdSmem {
    typedef BwdCfg<DT, DK, DV, C> G;
    DT Ks[C * G::LDK], Qs[C * G::LDK];
    DT Vs[C * G::LDV], Os[C * G::LDV];            // V, dO
    DT Es[C * G::LDV], Rb[C * G::LDV];            // E, dV
    DT Sb[DK * G::LDS_];                          // S_c^T, later dS_{c+1}^T
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
template <typename DT>
__device__ __forceinline__ void tile_rr(f32x4 &acc, const DT *A, int lda, int m0, const DT *Bt,
                                        int ldb, int n0, int k0, int k1, int lane) {
    typename Frag<DT>::k16 fa, fb;
    for (int k = k0; k < k1; k += 16) {
        frag_rows(A, lda, m0, k, lane, fa);
        frag_rows(Bt, ldb, n0, k, lane, fb);
        mk<DT>(acc, fa, fb);
    }
}
// Same with B row-major (k along the rows of B: B[k][n]).
template <typename DT>
__device__ __forceinline__ void tile_rc(f32x4 &acc, const DT *A, int lda, int m0, const DT *B,
                                        int ldb, int n0, int k0, int k1, int lane) {
    typename Frag<DT>::k16 fa, fb;
    for (int k = k0; k < k1; k += 16) {
        frag_rows(A, lda, m0, k, lane, fa);
        frag_cols16(B, ldb, k, n0, lane, fb);
        mk<DT>(acc, fa, fb);
    }
}
// Same with A given transposed (A^T row-major: A[m][k] = At[k][m]) and B
// row-major.
template <typename DT>
__device__ __forceinline__ void tile_cc(f32x4 &acc, const DT *At, int lda, int m0, const DT *B,
                                        int ldb, int n0, int k0, int k1, int lane) {
    typename Frag<DT>::k16 fa, fb;
    for (int k = k0; k < k1; k += 16) {
        frag_cols16(At, lda, k, m0, lane, fa);
        frag_cols16(B, ldb, k, n0, lane, fb);
        mk<DT>(acc, fa, fb);
    }
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

// Cooperative copy of `rows` rows (valid < nvalid; the rest zero) of `cols`
// elements from global (row stride gs elements) into LDS (row stride ld).
template <typename DT>
__device__ __forceinline__ void stage_rows(DT *dst, int ld, const DT *src, int64_t gs, int rows,
                                           int nvalid, int cols, int tid, int nthr) {
    const int per = cols / 4;  // groups of 4 elements
    for (int i = tid; i < rows * per; i += nthr) {
        const int t = i / per, e = (i % per) * 4;
        DT x[4];
        if (t < nvalid) {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = src[t * gs + e + j];
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) x[j] = from_f32<DT>(0.f);
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) dst[t * ld + e + j] = x[j];
    }
}

template <typename DT, int DK, int DV, int C>
__global__ __launch_bounds__(DV * 4) void chunk_bwd_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const DT *__restrict__ dout, const float *__restrict__ dST,
    const float *__restrict__ hs, DT *__restrict__ dq, DT *__restrict__ dk, DT *__restrict__ dv,
    DT *__restrict__ dbeta, float *__restrict__ dS0, int T, int H) {
    typedef BwdCfg<DT, DK, DV, C> G;
    constexpr int NW = G::NW, NT = G::NT, KT = G::KT;
    constexpr int LDK = G::LDK, LDV = G::LDV, LDS_ = G::LDS_, LDC = G::LDC;
    __shared__ __attribute__((aligned(16))) BwdSmem<DT, DK, DV, C> sm;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, r = lane & 15;
    const int v0 = 16 * w;
    const int64_t head = blockIdx.x;
    const int b = (int)(head / H), h = (int)(head % H);
    const int N = (T + C - 1) / C;
    const int nthr = 64 * NW;
    const int64_t rk = (int64_t)H * DK, rv = (int64_t)H * DV;  // token strides

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

    for (int c = N - 1; c >= 0; --c) {
        const int t0 = c * C, len = min(C, T - t0);
        const int64_t tok0 = (int64_t)b * T + t0;
        __syncthreads();
        // ---------------------------------------------------------------- load
        stage_rows(sm.Ks, LDK, k + (tok0 * H + h) * DK, rk, C, len, DK, tid, nthr);
        stage_rows(sm.Qs, LDK, q + (tok0 * H + h) * DK, rk, C, len, DK, tid, nthr);
        stage_rows(sm.Vs, LDV, v + (tok0 * H + h) * DV, rv, C, len, DV, tid, nthr);
        stage_rows(sm.Os, LDV, dout + (tok0 * H + h) * DV, rv, C, len, DV, tid, nthr);
        for (int t = tid; t < C; t += nthr) sm.betas[t] = t < len ? to_f32(beta[(tok0 + t) * H + h]) : 0.f;
        // S_c^T of this wave's columns (tile s: S^T[16s + 4g + i][v0 + r])
        f32x4 St[KT];
        const float *hc = hs + ((head * N + c) * DV + v0 + r) * DK;
#pragma unroll
        for (int s = 0; s < KT; ++s) St[s] = *reinterpret_cast<const f32x4 *>(hc + 16 * s + 4 * g);
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
            tile_rr(acc, isP ? sm.Qs : sm.Ks, LDK, 16 * ti, sm.Ks, LDK, 16 * tj, 0, DK, lane);
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
            // R = V - K S_c^T
            typename Frag<DT>::k16 fs[KT];
#pragma unroll
            for (int s = 0; s < KT; ++s) cvt4(St[s], fs[s]);
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 x = zero4();
                typename Frag<DT>::k16 fk;
#pragma unroll
                for (int s = 0; s < KT; ++s) {
                    frag_rows(sm.Ks, LDK, 16 * mt, 16 * s, lane, fk);
                    mk<DT>(x, fk, fs[s]);
                }
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
#pragma unroll
                for (int s = 0; s < KT; ++s) {
                    frag_rows(sm.Ks, LDK, 16 * mt, 16 * s, lane, fa);
                    mk<DT>(dE[mt], fa, fd[s]);
                }
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
        // dS update (keep dS_{c+1} for dK), and publish S_c^T for dQ, dK
        f32x4 Dold[KT];
        {
            typename Frag<DT>::k16 fdv[NT];
#pragma unroll
            for (int mt = 0; mt < NT; ++mt) {
                f32x4 nz = -Z[mt];
                cvt4(nz, fdv[mt]);
            }
#pragma unroll
            for (int s = 0; s < KT; ++s) {
                Dold[s] = Dt[s];
                typename Frag<DT>::k16 fa, fo;
#pragma unroll
                for (int kt = 0; kt < NT; ++kt) {
                    frag_cols16(sm.Qs, LDK, 16 * kt, 16 * s, lane, fa);
                    frag_cols16(sm.Os, LDV, 16 * kt, v0, lane, fo);
                    mk<DT>(Dt[s], fa, fo);
                    frag_cols16(sm.Ks, LDK, 16 * kt, 16 * s, lane, fa);
                    mk<DT>(Dt[s], fa, fdv[kt]);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    sm.Sb[(16 * s + 4 * g + i) * LDS_ + v0 + r] = from_f32<DT>(St[s][i]);
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
            tile_rr(acc, isD ? sm.Os : sm.Rb, LDV, 16 * ti, sm.Es, LDV, 16 * tj, 0, DV, lane);
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
        f32x4 dKa[(NO + NW - 1) / NW];
#pragma unroll
        for (int u = 0; u < (NO + NW - 1) / NW; ++u) {
            const int o = w + u * NW;
            if (o >= NO) break;
            const int mt = o / KT, j = o % KT;
            // dQ = dO S_c + Dm K
            f32x4 aq = zero4();
            tile_rr(aq, sm.Os, LDV, 16 * mt, sm.Sb, LDS_, 16 * j, 0, DV, lane);
            tile_rc(aq, sm.Dm, LDC, 16 * mt, sm.Ks, LDK, 16 * j, 0, 16 * (mt + 1), lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                if (t < len) dq[((tok0 + t) * H + h) * DK + 16 * j + r] = from_f32<DT>(aq[i]);
            }
            // dK (first part) = -dV S_c + Gs K + Dm^T Q
            f32x4 ak = zero4();
            tile_rr(ak, sm.Rb, LDV, 16 * mt, sm.Sb, LDS_, 16 * j, 0, DV, lane);
            ak = -ak;
            tile_rc(ak, sm.Gs, LDC, 16 * mt, sm.Ks, LDK, 16 * j, 0, C, lane);
            tile_cc(ak, sm.Dm, LDC, 16 * mt, sm.Qs, LDK, 16 * j, 16 * mt, C, lane);
            dKa[u] = ak;
        }
        __syncthreads();
        // dS_{c+1}^T into Sb, then dK += E dS_{c+1}
#pragma unroll
        for (int s = 0; s < KT; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.Sb[(16 * s + 4 * g + i) * LDS_ + v0 + r] = from_f32<DT>(Dold[s][i]);
        __syncthreads();
#pragma unroll
        for (int u = 0; u < (NO + NW - 1) / NW; ++u) {
            const int o = w + u * NW;
            if (o >= NO) break;
            const int mt = o / KT, j = o % KT;
            f32x4 ak = dKa[u];
            tile_rr(ak, sm.Es, LDV, 16 * mt, sm.Sb, LDS_, 16 * j, 0, DV, lane);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = 16 * mt + 4 * g + i;
                if (t < len) dk[((tok0 + t) * H + h) * DK + 16 * j + r] = from_f32<DT>(ak[i]);
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
                           a.dS_T, a.h, static_cast<DT *>(a.dq), static_cast<DT *>(a.dk),
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
