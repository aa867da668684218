// Decode: one delta-rule token per (b, h), state streamed through HBM once.
//
// The token-serial schedule of the recurrence (hada.io digest, section
// "Kernel Triton recurrent fusionne pour le decodage": read the prediction
// with the key, form the residual, write the outer product, read with the
// query).  Those are vector operations, not matrix products, so this kernel
// uses no MFMA: it is bound by the bytes of S it moves (read once, written
// once per call).
//
// Work split.  Row i of S (d_k floats) evolves on its own given k, q, v_i and
// beta:  p_i = S_i.k,  u_i = beta (v_i - p_i),  S_i += u_i k,  o_i = S_i.q.
// DK/8 lanes share a row, each holding 8 consecutive floats (two 16-byte
// loads, fully coalesced: a wave reads 64*32 contiguous bytes of one head's
// state).  A workgroup of 256 lanes covers PASSES*(256/(DK/8)) rows of one
// head; all its loads are issued before any reduction so that many bytes are
// in flight per CU.  The two dot products per row are reduced across the row's
// lanes with butterfly shuffles.
#include "dr_common.hpp"
#include "dr_launch.hpp"

namespace dr {

namespace {

__device__ __forceinline__ void load8(const float *p, float (&x)[8]) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0];
    const float4 b = reinterpret_cast<const float4 *>(p)[1];
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const __bf16 *p, float (&x)[8]) {
    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = (float)a[i];
}

// Sum over the LPR consecutive lanes that share a row (LPR a power of two).
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
    return group_sum<LPR>(x);
}

// GATED: the whole row first decays by alpha = exp(g) of its (b, h), then the
// token is predicted from the decayed row (forget before predict).
// L2: q and k are divided by sqrt(|x|^2 + 1e-6) first (the l2norm of the
// gated layer on houmin.site "infra/delta-net"); the row's lanes together
// hold all of q and k, so the norms are two more lane reductions.
// scale multiplies the output.
// KDA (Kimi Delta Attention, hada.io digest section "Kimi Delta Attention :
// attenuation par canal"): g is the per-key-channel log decay [B,H,Dk] and
// column j of the state decays by exp(g[j]); each lane holds 8 columns of a
// row, so it applies its 8 factors.
template <typename DT, int DK, int PASSES, bool GATED, bool L2, bool KDA = false>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ g, float *__restrict__ S,
    DT *__restrict__ o, int Dv, int wg_per_head, float scale) {
    constexpr int LPR = DK / 8;        // lanes per state row
    constexpr int RPP = 256 / LPR;     // rows per pass
    const int64_t head = blockIdx.x / wg_per_head;  // flattened b*H + h
    const int part = blockIdx.x % wg_per_head;
    const int sub = threadIdx.x % LPR;
    const int rloc = threadIdx.x / LPR;

    float kf[8], qf[8];
    load8(k + head * DK + 8 * sub, kf);
    load8(q + head * DK + 8 * sub, qf);
    if constexpr (L2) {
        float kk = 0.f, qq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kk += kf[i] * kf[i];
            qq += qf[i] * qf[i];
        }
        const float nk = rsqrtf(row_sum<LPR>(kk) + 1e-6f), nq = rsqrtf(row_sum<LPR>(qq) + 1e-6f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            kf[i] *= nk;
            qf[i] *= nq;
        }
    }
    const float b = to_f32(beta[head]);
    const float a = GATED ? __expf(g[head]) : 1.f;
    float ak[8];
    if constexpr (KDA) {
        load8(g + head * DK + 8 * sub, ak);
#pragma unroll
        for (int i = 0; i < 8; ++i) ak[i] = __expf(ak[i]);
    }

    float s[PASSES][8];
    float vr[PASSES];
    int row[PASSES];
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        row[p] = (part * PASSES + p) * RPP + rloc;
        if (row[p] < Dv) {
            load8(S + (head * Dv + row[p]) * DK + 8 * sub, s[p]);
            if (GATED) {
#pragma unroll
                for (int i = 0; i < 8; ++i) s[p][i] *= a;
            }
            if constexpr (KDA) {
#pragma unroll
                for (int i = 0; i < 8; ++i) s[p][i] *= ak[i];
            }
            vr[p] = to_f32(v[head * Dv + row[p]]);
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) s[p][i] = 0.f;
            vr[p] = 0.f;
        }
    }
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
        float pk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) pk += s[p][i] * kf[i];
        pk = row_sum<LPR>(pk);                 // prediction S_i . k
        const float u = b * (vr[p] - pk);      // scaled error
        float oq = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            s[p][i] += u * kf[i];              // rank-1 write
            oq += s[p][i] * qf[i];
        }
        oq = row_sum<LPR>(oq);                 // read after write: S_i . q
        if (row[p] < Dv) {
            float4 *dst = reinterpret_cast<float4 *>(S + (head * Dv + row[p]) * DK + 8 * sub);
            dst[0] = make_float4(s[p][0], s[p][1], s[p][2], s[p][3]);
            dst[1] = make_float4(s[p][4], s[p][5], s[p][6], s[p][7]);
            if (sub == 0) o[head * Dv + row[p]] = from_f32<DT>(oq * scale);
        }
    }
}

template <typename DT, int DK, bool GATED, bool L2, bool KDA = false>
hipError_t launch_step(const StepArgs &x, hipStream_t stream) {
    constexpr int LPR = DK / 8;
    constexpr int RPP = 256 / LPR;
    constexpr int PASSES = 2;
    const int rows_per_wg = RPP * PASSES;
    const int wg_per_head = (x.Dv + rows_per_wg - 1) / rows_per_wg;
    const int64_t grid = x.BH * wg_per_head;
    hipLaunchKernelGGL((recurrent_step_kernel<DT, DK, PASSES, GATED, L2, KDA>),
                       dim3((unsigned)grid), dim3(256), 0, stream, static_cast<const DT *>(x.q),
                       static_cast<const DT *>(x.k), static_cast<const DT *>(x.v),
                       static_cast<const DT *>(x.beta), KDA ? x.gk : x.g, x.S,
                       static_cast<DT *>(x.o), x.Dv, wg_per_head, x.scale);
    return hipGetLastError();
}

template <typename DT, int DK>
hipError_t dispatch_opts(const StepArgs &x, hipStream_t stream) {
    if (x.gk)
        return x.l2 ? launch_step<DT, DK, false, true, true>(x, stream)
                    : launch_step<DT, DK, false, false, true>(x, stream);
    if (x.g)
        return x.l2 ? launch_step<DT, DK, true, true>(x, stream)
                    : launch_step<DT, DK, true, false>(x, stream);
    return x.l2 ? launch_step<DT, DK, false, true>(x, stream)
                : launch_step<DT, DK, false, false>(x, stream);
}

template <typename DT>
hipError_t dispatch_dk(const StepArgs &x, hipStream_t stream) {
    switch (x.Dk) {
    case 16: return dispatch_opts<DT, 16>(x, stream);
    case 32: return dispatch_opts<DT, 32>(x, stream);
    case 64: return dispatch_opts<DT, 64>(x, stream);
    case 128: return dispatch_opts<DT, 128>(x, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent_step(const StepArgs &x, bool bf16, hipStream_t stream) {
    return bf16 ? dispatch_dk<__bf16>(x, stream) : dispatch_dk<float>(x, stream);
}

}  // namespace dr
