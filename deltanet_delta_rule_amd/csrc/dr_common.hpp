// Device-side building blocks shared by the delta-rule kernels (gfx950).
//
// Element types: `float` (fp32 inputs) or `__bf16` (bfloat16 inputs).  All
// arithmetic accumulates in fp32; fp32 -> bf16 narrowing rounds to nearest
// even (the hardware conversion).
//
// Matrix-core tiles.  Every product is built from 16x16 output tiles on the
// MFMA units.  The lane layout of an output tile (the "D layout") is the one
// all 16x16 MFMA shapes share on CDNA: lane l = 16*g + r (g = l/16, r = l%16)
// holds D[4g + i][r] for i = 0..3.
//
// Operands are fed in one canonical k order.  For a contraction slab starting
// at k0, lane (g, r) supplies the four k indices k0 + 4g + {0,1,2,3} of its
// row r (A) or column r (B); a 32-wide slab adds k0 + 16 + 4g + {0,1,2,3}.
// The hardware contracts lane (g, r)'s j-th A element with lane (g, n)'s j-th
// B element, so any k permutation applied identically to A and B gives the
// same sum -- and with this one, a D-layout tile stack whose rows run along k
// is already a B operand (lane (g, r) holds rows 4g..4g+3 of each 16-row
// tile).  Results computed with tokens along M can therefore feed the next
// product over tokens straight from registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dr {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;

// Two fp32 values narrowed to a packed bf16 pair (one v_cvt_pk_bf16_f32).
// Narrowing whole 4-vectors at once lets the compiler scalarise into four
// half-empty conversions and two permutes; pairs keep it to two instructions.
__device__ __forceinline__ unsigned pk_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ u32x2 pk4_bf16(const f32x4 &x) {
    return u32x2{pk_bf16(x[0], x[1]), pk_bf16(x[2], x[3])};
}

// x moved between lanes by one DPP pattern (a compile-time dpp_ctrl value).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of N consecutive lanes (N = 2, 4, 8 or 16), every
// lane of a group receiving the group's sum, on DPP row operations instead of
// LDS permutes: quad permutes for lane xor 1 and xor 2, then the half-row
// mirror (lane i and 7 - i of each 8) and the row mirror (i and 15 - i of
// each 16).  Each step adds partial sums over two disjoint lane sets, so the
// lanes of a group all end with the same value (additions commute).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16, "group of 1..16 lanes");
    if constexpr (N >= 2) x += dpp_move<0xB1>(x);   // quad_perm [1,0,3,2]
    if constexpr (N >= 4) x += dpp_move<0x4E>(x);   // quad_perm [2,3,0,1]
    if constexpr (N >= 8) x += dpp_move<0x141>(x);  // row_half_mirror
    if constexpr (N >= 16) x += dpp_move<0x140>(x); // row_mirror
    return x;
}

// x plus its value in lane i xor 16 (xor 32), on the cross-row lane swaps of
// gfx950: two register-to-register swaps instead of an LDS permute.  Every
// lane of the wave must be active.
__device__ __forceinline__ float xor16_sum(float x) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

// Sum over the 64 lanes of the wave, every lane receiving it (all lanes
// active).
__device__ __forceinline__ float wave_sum(float x) { return xor32_sum(xor16_sum(group_sum<16>(x))); }

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(__bf16 x) { return (float)x; }

template <typename DT>
__device__ __forceinline__ DT from_f32(float x);
template <>
__device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <>
__device__ __forceinline__ __bf16 from_f32<__bf16>(float x) { return (__bf16)x; }

// Operand fragments: 8 elements (32-wide slab) or 4 (16-wide slab) per lane.
template <typename DT> struct Frag;
template <> struct Frag<__bf16> {
    typedef bf16x8 k32;
    typedef bf16x4 k16;
};
struct f32x8_arr { float v[8]; };
struct f32x4_arr { float v[4]; };
template <> struct Frag<float> {
    typedef f32x8_arr k32;
    typedef f32x4_arr k16;
};

__device__ __forceinline__ void frag_set(bf16x8 &f, int i, float x) { f[i] = (__bf16)x; }
__device__ __forceinline__ void frag_set(bf16x4 &f, int i, float x) { f[i] = (__bf16)x; }
__device__ __forceinline__ void frag_set(f32x8_arr &f, int i, float x) { f.v[i] = x; }
__device__ __forceinline__ void frag_set(f32x4_arr &f, int i, float x) { f.v[i] = x; }
__device__ __forceinline__ float frag_get(const bf16x4 &f, int i) { return (float)f[i]; }
__device__ __forceinline__ float frag_get(const f32x4_arr &f, int i) { return f.v[i]; }

// acc += A * B over one 32-wide k slab.
__device__ __forceinline__ void mma_k32(f32x4 &acc, const bf16x8 &a, const bf16x8 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k32(f32x4 &acc, const f32x8_arr &a, const f32x8_arr &b) {
    // 16x16x4 fp32 MFMA: lane group g supplies hardware k = g.  Instruction j
    // (j < 4) covers k0 + 4g + j, instruction 4 + j covers k0 + 16 + 4g + j.
#pragma unroll
    for (int j = 0; j < 8; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}
// acc += A * B over one 16-wide k slab.
__device__ __forceinline__ void mma_k16(f32x4 &acc, const bf16x4 &a, const bf16x4 &b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                    __builtin_bit_cast(i16x4, b),
                                                    acc, 0, 0, 0);
}
__device__ __forceinline__ void mma_k16(f32x4 &acc, const f32x4_arr &a, const f32x4_arr &b) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.v[j], b.v[j], acc, 0, 0, 0);
}

// Load 4 consecutive elements (an aligned quad) as floats.
__device__ __forceinline__ void load4(const float *p, float (&x)[4]) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    x[0] = t.x; x[1] = t.y; x[2] = t.z; x[3] = t.w;
}
__device__ __forceinline__ void load4(const __bf16 *p, float (&x)[4]) {
    const bf16x4 t = *reinterpret_cast<const bf16x4 *>(p);
    x[0] = (float)t[0]; x[1] = (float)t[1]; x[2] = (float)t[2]; x[3] = (float)t[3];
}

// Operand fragment of a row-major matrix M (leading dimension ld, elements of
// type DT): lane (g, r) takes M[row0 + r][k0 + 4g + 0..3] (+ k0 + 16 + ...).
// Serves as A (rows = m) or as B when B[k][n] = M[n][k] (rows = n).
__device__ __forceinline__ void frag_rows(const __bf16 *M, int ld, int row0, int k0,
                                          int lane, bf16x8 &f) {
    const int g = lane >> 4, r = lane & 15;
    const __bf16 *p = M + (row0 + r) * ld + k0 + 4 * g;
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(p);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(p + 16);
    f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_rows(const __bf16 *M, int ld, int row0, int k0,
                                          int lane, bf16x4 &f) {
    const int g = lane >> 4, r = lane & 15;
    f = *reinterpret_cast<const bf16x4 *>(M + (row0 + r) * ld + k0 + 4 * g);
}
__device__ __forceinline__ void frag_rows(const float *M, int ld, int row0, int k0,
                                          int lane, f32x8_arr &f) {
    const int g = lane >> 4, r = lane & 15;
    const float *p = M + (row0 + r) * ld + k0 + 4 * g;
    const float4 lo = *reinterpret_cast<const float4 *>(p);
    const float4 hi = *reinterpret_cast<const float4 *>(p + 16);
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
}
__device__ __forceinline__ void frag_rows(const float *M, int ld, int row0, int k0,
                                          int lane, f32x4_arr &f) {
    const int g = lane >> 4, r = lane & 15;
    const float4 t = *reinterpret_cast<const float4 *>(M + (row0 + r) * ld + k0 + 4 * g);
    f.v[0] = t.x; f.v[1] = t.y; f.v[2] = t.z; f.v[3] = t.w;
}

// Fragment of the transpose of a row-major matrix M over one 16-wide slab:
// lane (g, r) takes M[k0 + 4g + j][col0 + r] for j = 0..3, i.e. column
// col0 + r of M with k running down the rows.  For bf16 this is one LDS
// transpose read (ds_read_b64_tr_b16): the 16 lanes of group g each address
// one 8-byte piece of the 4 x 16 block M[k0+4g .. k0+4g+3][col0 .. col0+15]
// (lane r: row r/4, columns 4(r%4)..4(r%4)+3) and the hardware hands lane r
// column r of that block.  fp32 has no transpose read and gathers instead.
__device__ __forceinline__ void frag_cols16(const __bf16 *M, int ld, int k0, int col0,
                                            int lane, bf16x4 &f) {
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const int g = lane >> 4, r = lane & 15;
    const __bf16 *p = M + (k0 + 4 * g + (r >> 2)) * ld + col0 + 4 * (r & 3);
    f = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)p));
}
__device__ __forceinline__ void frag_cols16(const float *M, int ld, int k0, int col0,
                                            int lane, f32x4_arr &f) {
    const int g = lane >> 4, r = lane & 15;
#pragma unroll
    for (int j = 0; j < 4; ++j) f.v[j] = M[(k0 + 4 * g + j) * ld + col0 + r];
}
__device__ __forceinline__ void frag_cols32(const __bf16 *M, int ld, int k0, int col0,
                                            int lane, bf16x8 &f) {
    bf16x4 lo, hi;
    frag_cols16(M, ld, k0, col0, lane, lo);
    frag_cols16(M, ld, k0 + 16, col0, lane, hi);
    f = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ void frag_cols32(const float *M, int ld, int k0, int col0,
                                            int lane, f32x8_arr &f) {
    f32x4_arr lo, hi;
    frag_cols16(M, ld, k0, col0, lane, lo);
    frag_cols16(M, ld, k0 + 16, col0, lane, hi);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f.v[j] = lo.v[j];
        f.v[4 + j] = hi.v[j];
    }
}

// Fragments in chunk order: lane (g, r) supplies the eight consecutive k
// indices k0 + 8g .. k0 + 8g + 7 (one 16-byte read for bf16).  Both operands
// of a product must use the same order; a D-layout stack is turned into a
// chunk-order operand by frag_from_state below.
__device__ __forceinline__ void load_chunk(const __bf16 *p, bf16x8 &f) {
    f = *reinterpret_cast<const bf16x8 *>(p);
}
__device__ __forceinline__ void load_chunk(const float *p, f32x8_arr &f) {
    const float4 lo = *reinterpret_cast<const float4 *>(p);
    const float4 hi = *reinterpret_cast<const float4 *>(p + 4);
    f.v[0] = lo.x; f.v[1] = lo.y; f.v[2] = lo.z; f.v[3] = lo.w;
    f.v[4] = hi.x; f.v[5] = hi.y; f.v[6] = hi.z; f.v[7] = hi.w;
}
__device__ __forceinline__ void load_chunk(const __bf16 *p, bf16x4 &f) {
    f = *reinterpret_cast<const bf16x4 *>(p);
}
__device__ __forceinline__ void load_chunk(const float *p, f32x4_arr &f) {
    const float4 t = *reinterpret_cast<const float4 *>(p);
    f.v[0] = t.x; f.v[1] = t.y; f.v[2] = t.z; f.v[3] = t.w;
}

// Key order of the state tiles.  With 32-wide slabs over d_k, row 4g + i of
// accumulator tile dt holds key index state_col<32>(dt, g) + i: tiles 2s and
// 2s + 1 split the 8-key chunk 4s + g of slab s into halves, the lower half
// going to tile 2s for even g and to tile 2s + 1 for odd g.  A product over
// d_k then reads its other operand in chunk order (16 bytes per lane), and
// the transpose read that feeds the state update fetches, per 16-lane row,
// quads from alternating halves of four chunks -- which, with the row
// swizzle of the key tile, spreads a read over all 64 LDS banks.  With
// 16-wide slabs (d_k = 16) the order is the plain one.
template <int KSD>
__device__ __forceinline__ int state_col(int dt, int g) {
    if constexpr (KSD == 32) return 8 * (4 * (dt >> 1) + g) + 4 * ((g & 1) ^ (dt & 1));
    else return 16 * dt + 4 * g;
}
// B operand in chunk order from state tiles 2s, 2s + 1 (32-wide slab): lane
// (g, r) needs keys 32s + 8g + 0..7, i.e. the tile holding the lower half
// first (see state_col).
__device__ __forceinline__ void frag_from_state(const f32x4 &t0, const f32x4 &t1, int g,
                                                bf16x8 &f) {
    // narrow first, then swap the packed halves (4 selects instead of 8)
    const u32x2 a = pk4_bf16(t0);
    const u32x2 b = pk4_bf16(t1);
    const bool odd = g & 1;
    const u32x2 lo = odd ? b : a, hi = odd ? a : b;
    f = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3));
}
__device__ __forceinline__ void frag_from_state(const f32x4 &t0, const f32x4 &t1, int g,
                                                f32x8_arr &f) {
    const bool odd = g & 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = odd ? t1[i] : t0[i];
        f.v[4 + i] = odd ? t0[i] : t1[i];
    }
}

// Store a 4-element fragment to 4 consecutive elements (8 or 16 bytes).
__device__ __forceinline__ void store_frag16(__bf16 *p, const bf16x4 &f) {
    *reinterpret_cast<bf16x4 *>(p) = f;
}
__device__ __forceinline__ void store_frag16(float *p, const f32x4_arr &f) {
    *reinterpret_cast<float4 *>(p) = make_float4(f.v[0], f.v[1], f.v[2], f.v[3]);
}

// Narrow four fp32 values to a 4-element fragment (bf16: two packed
// conversions).
__device__ __forceinline__ void cvt4(const f32x4 &x, bf16x4 &f) {
    f = __builtin_bit_cast(bf16x4, pk4_bf16(x));
}
__device__ __forceinline__ void cvt4(const f32x4 &x, f32x4_arr &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f.v[i] = x[i];
}
__device__ __forceinline__ void cvt8(const f32x4 &lo, const f32x4 &hi, bf16x8 &f) {
    const u32x2 a = pk4_bf16(lo), b = pk4_bf16(hi);
    f = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3));
}
__device__ __forceinline__ void cvt8(const f32x4 &lo, const f32x4 &hi, f32x8_arr &f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        f.v[i] = lo[i];
        f.v[4 + i] = hi[i];
    }
}
// Sign flip of a fragment.
__device__ __forceinline__ bf16x4 neg(const bf16x4 &f) {
    return __builtin_bit_cast(bf16x4, __builtin_bit_cast(u32x2, f) ^ 0x80008000u);
}
__device__ __forceinline__ f32x4_arr neg(const f32x4_arr &f) {
    f32x4_arr r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r.v[i] = -f.v[i];
    return r;
}

// B operand from a stack of D-layout accumulator tiles whose rows run along
// k: tile k0/16 (and k0/16 + 1 for a 32-wide slab), narrowed to DT.
template <typename F>
__device__ __forceinline__ void frag_from_acc32(const f32x4 &t0, const f32x4 &t1, F &f) {
    cvt8(t0, t1, f);
}
template <typename F>
__device__ __forceinline__ void frag_from_acc16(const f32x4 &t0, F &f) {
    cvt4(t0, f);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Raw buffer resource over `bytes` bytes from `base` (the 32-bit data format
// word of gfx9 resources).  Accesses are range-checked against `bytes`: loads
// past the end return zeros and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                             0x00020000);
}
template <typename V>
__device__ __forceinline__ V buf_load16(__amdgpu_buffer_rsrc_t r, int voff) {
    static_assert(sizeof(V) == 16, "16-byte vector");
    return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}
template <typename DT>
__device__ __forceinline__ DT buf_load_elem(__amdgpu_buffer_rsrc_t r, int voff);
template <>
__device__ __forceinline__ __bf16 buf_load_elem<__bf16>(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(__bf16, __builtin_amdgcn_raw_buffer_load_b16(r, voff, 0, 0));
}
template <>
__device__ __forceinline__ float buf_load_elem<float>(__amdgpu_buffer_rsrc_t r, int voff) {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, 0, 0));
}
// Element store at voff (per lane) + soff (uniform).
__device__ __forceinline__ void buf_store_elem(__bf16 x, __amdgpu_buffer_rsrc_t r, int voff,
                                               int soff) {
    __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, x), r, voff, soff, 0);
}
__device__ __forceinline__ void buf_store_elem(float x, __amdgpu_buffer_rsrc_t r, int voff,
                                               int soff) {
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, x), r, voff, soff, 0);
}

// Workgroup barrier for hand-offs through LDS: waits for this wave's LDS
// operations, then meets the other waves.  Unlike __syncthreads() it carries
// no fence over global memory, so register prefetches and output stores stay
// in flight across it.  The "memory" clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Value of x in lane N of this lane's 16-lane row (DPP row_newbcast).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x150 + N, 0xf, 0xf, true));
}
// Same with N known only after unrolling.
__device__ __forceinline__ float row_bcast_at(float x, int n) {
    switch (n) {
    case 0: return row_bcast<0>(x);
    case 1: return row_bcast<1>(x);
    case 2: return row_bcast<2>(x);
    case 3: return row_bcast<3>(x);
    case 4: return row_bcast<4>(x);
    case 5: return row_bcast<5>(x);
    case 6: return row_bcast<6>(x);
    case 7: return row_bcast<7>(x);
    case 8: return row_bcast<8>(x);
    case 9: return row_bcast<9>(x);
    case 10: return row_bcast<10>(x);
    case 11: return row_bcast<11>(x);
    case 12: return row_bcast<12>(x);
    case 13: return row_bcast<13>(x);
    case 14: return row_bcast<14>(x);
    default: return row_bcast<15>(x);
    }
}

// Orders this wave's LDS writes before its later LDS reads of data written by
// other lanes of the same wave (no other wave involved, so no barrier).
__device__ __forceinline__ void wave_lds_fence() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

}  // namespace dr
