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
#pragma unroll
    for (int m = LPR / 2; m >= 1; m >>= 1) x += __shfl_xor(x, m, LPR);
    return x;
}

// GATED: the whole row first decays by alpha = exp(g) of its (b, h), then the
// token is predicted from the decayed row (forget before predict).
template <typename DT, int DK, int PASSES, bool GATED>
__global__ __launch_bounds__(256) void recurrent_step_kernel(
    const DT *__restrict__ q, const DT *__restrict__ k, const DT *__restrict__ v,
    const DT *__restrict__ beta, const float *__restrict__ g, float *__restrict__ S,
    DT *__restrict__ o, int Dv, int wg_per_head) {
    constexpr int LPR = DK / 8;        // lanes per state row
    constexpr int RPP = 256 / LPR;     // rows per pass
    const int64_t head = blockIdx.x / wg_per_head;  // flattened b*H + h
    const int part = blockIdx.x % wg_per_head;
    const int sub = threadIdx.x % LPR;
    const int rloc = threadIdx.x / LPR;

    float kf[8], qf[8];
    load8(k + head * DK + 8 * sub, kf);
    load8(q + head * DK + 8 * sub, qf);
    const float b = to_f32(beta[head]);
    const float a = GATED ? __expf(g[head]) : 1.f;

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
            if (sub == 0) o[head * Dv + row[p]] = from_f32<DT>(oq);
        }
    }
}

template <typename DT, int DK>
hipError_t launch_step(const void *q, const void *k, const void *v, const void *beta,
                       const float *g, float *S, void *o, int64_t BH, int Dv,
                       hipStream_t stream) {
    constexpr int LPR = DK / 8;
    constexpr int RPP = 256 / LPR;
    constexpr int PASSES = 2;
    const int rows_per_wg = RPP * PASSES;
    const int wg_per_head = (Dv + rows_per_wg - 1) / rows_per_wg;
    const int64_t grid = BH * wg_per_head;
    if (g)
        hipLaunchKernelGGL((recurrent_step_kernel<DT, DK, PASSES, true>), dim3((unsigned)grid),
                           dim3(256), 0, stream, static_cast<const DT *>(q),
                           static_cast<const DT *>(k), static_cast<const DT *>(v),
                           static_cast<const DT *>(beta), g, S, static_cast<DT *>(o), Dv,
                           wg_per_head);
    else
        hipLaunchKernelGGL((recurrent_step_kernel<DT, DK, PASSES, false>), dim3((unsigned)grid),
                           dim3(256), 0, stream, static_cast<const DT *>(q),
                           static_cast<const DT *>(k), static_cast<const DT *>(v),
                           static_cast<const DT *>(beta), g, S, static_cast<DT *>(o), Dv,
                           wg_per_head);
    return hipGetLastError();
}

template <typename DT>
hipError_t dispatch_dk(const void *q, const void *k, const void *v, const void *beta,
                       const float *g, float *S, void *o, int64_t BH, int Dk, int Dv,
                       hipStream_t stream) {
    switch (Dk) {
    case 16: return launch_step<DT, 16>(q, k, v, beta, g, S, o, BH, Dv, stream);
    case 32: return launch_step<DT, 32>(q, k, v, beta, g, S, o, BH, Dv, stream);
    case 64: return launch_step<DT, 64>(q, k, v, beta, g, S, o, BH, Dv, stream);
    case 128: return launch_step<DT, 128>(q, k, v, beta, g, S, o, BH, Dv, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_recurrent_step(const void *q, const void *k, const void *v,
                                 const void *beta, const float *g, float *S, void *o,
                                 int64_t BH, int Dk, int Dv, bool bf16, hipStream_t stream) {
    if (bf16) return dispatch_dk<__bf16>(q, k, v, beta, g, S, o, BH, Dk, Dv, stream);
    return dispatch_dk<float>(q, k, v, beta, g, S, o, BH, Dk, Dv, stream);
}

}  // namespace dr
