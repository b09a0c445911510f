// Device-side building blocks shared by the gfx950 kernels of this library.
//
// MFMA tile convention (v_mfma_f32_16x16x32_bf16 / v_mfma_f32_16x16x4_f32,
// wave64): lane l = 16*g + i (g = l / 16 in 0..3, i = l % 16).
//   A operand  lane (g, i) supplies row i, 8 contraction values;
//   B operand  lane (g, i) supplies column i, the same 8 contraction values;
//   C/D        lane (g, i) holds rows 4g..4g+3 of column i.
// Which 8 contraction indices a lane group supplies is free as long as the A
// and B operands agree; every "Frag" below holds 8 consecutive contraction
// values of one row/column, the lane group g supplying indices 8g..8g+7 of a
// 32-wide contraction step.  For bf16 one instruction covers the step; for
// fp32 eight 16x16x4 instructions do (instruction t takes element t of each
// lane), which sums the same 32 products.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace avq {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <typename T> struct Frag;
template <> struct Frag<bf16> {
    bf16x8 v;
};
template <> struct Frag<float> {
    f32x4 lo, hi;
};

__device__ __forceinline__ f32x4 mma(const Frag<bf16> &a, const Frag<bf16> &b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma(const Frag<float> &a, const Frag<float> &b, f32x4 c)
{
#pragma unroll
    for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[t], b.lo[t], c, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < 4; ++t) c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[t], b.hi[t], c, 0, 0, 0);
    return c;
}

// 8 consecutive elements at p (16-byte aligned for bf16, 16-byte aligned
// halves for fp32)
__device__ __forceinline__ Frag<bf16> load_frag(const bf16 *p)
{
    Frag<bf16> f;
    f.v = *reinterpret_cast<const bf16x8 *>(p);
    return f;
}
__device__ __forceinline__ Frag<float> load_frag(const float *p)
{
    Frag<float> f;
    f.lo = *reinterpret_cast<const f32x4 *>(p);
    f.hi = *reinterpret_cast<const f32x4 *>(p + 4);
    return f;
}
template <typename T> __device__ __forceinline__ Frag<T> zero_frag();
template <> __device__ __forceinline__ Frag<bf16> zero_frag<bf16>()
{
    Frag<bf16> f;
    f.v = bf16x8{};
    return f;
}
template <> __device__ __forceinline__ Frag<float> zero_frag<float>()
{
    Frag<float> f;
    f.lo = f32x4{0.f, 0.f, 0.f, 0.f};
    f.hi = f.lo;
    return f;
}

__device__ __forceinline__ void store_frag(bf16 *dst, const Frag<bf16> &f)
{
    *reinterpret_cast<bf16x8 *>(dst) = f.v;
}
__device__ __forceinline__ void store_frag(float *dst, const Frag<float> &f)
{
    *reinterpret_cast<f32x4 *>(dst) = f.lo;
    *reinterpret_cast<f32x4 *>(dst + 4) = f.hi;
}
// store s * f (used with s = -2, exact in both types)
__device__ __forceinline__ void store_scaled_frag(bf16 *dst, const Frag<bf16> &f, float s)
{
    Frag<bf16> o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o.v[k] = (bf16)((float)f.v[k] * s);
    store_frag(dst, o);
}
__device__ __forceinline__ void store_scaled_frag(float *dst, const Frag<float> &f, float s)
{
    Frag<float> o;
    o.lo = f.lo * s;
    o.hi = f.hi * s;
    store_frag(dst, o);
}
__device__ __forceinline__ float frag_elem(const Frag<bf16> &f, int k) { return (float)f.v[k]; }
__device__ __forceinline__ float frag_elem(const Frag<float> &f, int k)
{
    return k < 4 ? f.lo[k] : f.hi[k - 4];
}

__host__ __device__ __forceinline__ int round16(int x) { return (x + 15) & ~15; }
__host__ __device__ __forceinline__ int round32(int x) { return (x + 31) & ~31; }

// Build a B-operand fragment from two 16x16 accumulator tiles of the same
// column (rows 4g..4g+3 of each): element k < 4 is row 4g+k of tile a,
// element k >= 4 is row 4g+k-4 of tile b.  The matching A operand must
// present its contraction index in the same order (see perm32 below).
__device__ __forceinline__ Frag<bf16> pack_frag_bf16(f32x4 a, f32x4 b)
{
    Frag<bf16> f;
    f.v[0] = (bf16)a[0];
    f.v[1] = (bf16)a[1];
    f.v[2] = (bf16)a[2];
    f.v[3] = (bf16)a[3];
    f.v[4] = (bf16)b[0];
    f.v[5] = (bf16)b[1];
    f.v[6] = (bf16)b[2];
    f.v[7] = (bf16)b[3];
    return f;
}
template <typename T> __device__ __forceinline__ Frag<T> pack_frag(f32x4 a, f32x4 b);
template <> __device__ __forceinline__ Frag<bf16> pack_frag<bf16>(f32x4 a, f32x4 b)
{
    return pack_frag_bf16(a, b);
}
template <> __device__ __forceinline__ Frag<float> pack_frag<float>(f32x4 a, f32x4 b)
{
    Frag<float> f;
    f.lo = a;
    f.hi = b;
    return f;
}

// Position, inside a 32-wide contraction step, at which row rho (0..31) of
// the two stacked accumulator tiles sits in the packed fragments above:
// lane group g supplies positions 8g..8g+7 = rows 4g..4g+3 then 16+4g..16+4g+3.
__host__ __device__ __forceinline__ int perm32(int rho)
{
    return 8 * ((rho & 15) >> 2) + 4 * (rho >> 4) + (rho & 3);
}

// ---------------------------------------------------------------- conversions
template <typename T> __device__ __forceinline__ T from_float(float x);
template <> __device__ __forceinline__ float from_float<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_float<bf16>(float x) { return (bf16)x; }
__device__ __forceinline__ float to_float(float x) { return x; }
__device__ __forceinline__ float to_float(bf16 x) { return (float)x; }

// nearest bf16 to a double (ties to even), as its bit pattern; the operand
// is assumed to lie in bf16's normal range or be zero
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x)
{
    unsigned long long b = (unsigned long long)__double_as_longlong(x);
    unsigned long long lsb = (b >> 45) & 1ull;
    b = (b + ((1ull << 44) - 1ull) + lsb) & ~((1ull << 45) - 1ull);
    float f = (float)__longlong_as_double((long long)b);   // exact
    return (uint16_t)(__float_as_uint(f) >> 16);
}

// ---------------------------------------------------------------- wave reductions
// DPP row controls (within rows of 16 lanes)
#define AVQ_DPP_QUAD_XOR1 0xB1    // quad_perm [1,0,3,2]
#define AVQ_DPP_QUAD_XOR2 0x4E    // quad_perm [2,3,0,1]
#define AVQ_DPP_ROW_HALF_MIRROR 0x141
#define AVQ_DPP_ROW_MIRROR 0x140

template <int CTRL> __device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// sum over the 16 lanes of each row (result in every lane of the row)
__device__ __forceinline__ float row16_sum(float x)
{
    x += dpp<AVQ_DPP_QUAD_XOR1>(x);
    x += dpp<AVQ_DPP_QUAD_XOR2>(x);
    x += dpp<AVQ_DPP_ROW_HALF_MIRROR>(x);
    x += dpp<AVQ_DPP_ROW_MIRROR>(x);
    return x;
}

#define AVQ_DPP_ROW_ROR8 0x128       // rotate by 8 inside a row: lane i <-> i ^ 8

// One halving step of a 16-lane reduce-scatter: lanes with `up` set keep the
// upper half of the N blocks, the others the lower half; each adds the half
// its DPP partner gives away (the partner differs from it in the split bit).
template <int N, int CTRL>
__device__ __forceinline__ void halve_blocks(f32x4 *t, bool up)
{
#pragma unroll
    for (int j = 0; j < N / 2; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float keep = up ? t[j + N / 2][r] : t[j][r];
            const float give = up ? t[j][r] : t[j + N / 2][r];
            t[j][r] = keep + dpp<CTRL>(give);
        }
    }
}

// Reduce-scatter over the 16 lanes of each row: on entry every lane holds
// NRB blocks of 4 values; on exit t[0] holds, summed over the row's 16 lanes,
// block (i16 >> (4 - log2 NRB)).  The partner masks 8, 7, 2, 1 (row_ror:8,
// row_half_mirror, quad_perm xor 2, quad_perm xor 1) span all 16 lanes, so
// every sum covers each lane exactly once; lanes left after log2 NRB halving
// steps finish with an all-reduce on the remaining masks.
template <int NRB>
__device__ __forceinline__ f32x4 row16_reduce_scatter(f32x4 *t, int i16)
{
    static_assert(NRB == 2 || NRB == 4 || NRB == 8 || NRB == 16, "NRB");
    halve_blocks<NRB, AVQ_DPP_ROW_ROR8>(t, (i16 & 8) != 0);
    if constexpr (NRB >= 4) halve_blocks<NRB / 2, AVQ_DPP_ROW_HALF_MIRROR>(t, (i16 & 4) != 0);
    if constexpr (NRB >= 8) halve_blocks<NRB / 4, AVQ_DPP_QUAD_XOR2>(t, (i16 & 2) != 0);
    if constexpr (NRB >= 16) halve_blocks<NRB / 8, AVQ_DPP_QUAD_XOR1>(t, (i16 & 1) != 0);
    f32x4 v = t[0];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        if constexpr (NRB <= 2) v[r] += dpp<AVQ_DPP_ROW_HALF_MIRROR>(v[r]);
        if constexpr (NRB <= 4) v[r] += dpp<AVQ_DPP_QUAD_XOR2>(v[r]);
        if constexpr (NRB <= 8) v[r] += dpp<AVQ_DPP_QUAD_XOR1>(v[r]);
    }
    return v;
}

// Across the four lane groups g (lanes i, i+16, i+32, i+48), with gfx950's
// v_permlane16_swap / v_permlane32_swap (VALU lane exchanges, no LDS round
// trip).  Called with the same register as both operands, the 16-lane swap
// returns {rows 0,0,2,2} and {rows 1,1,3,3} of it and the 32-lane swap
// {rows 0-1,0-1} and {rows 2-3,2-3}, so combining the two halves of each
// result is symmetric: every lane of a pair gets the same value without a
// lane-dependent select.
__device__ __forceinline__ void xswap16(float x, float &a, float &b)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void xswap32(float x, float &a, float &b)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    a = __uint_as_float(p[0]);
    b = __uint_as_float(p[1]);
}
__device__ __forceinline__ void xswap16(int x, int &a, int &b)
{
    const auto p = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
    a = (int)p[0];
    b = (int)p[1];
}
__device__ __forceinline__ void xswap32(int x, int &a, int &b)
{
    const auto p = __builtin_amdgcn_permlane32_swap((unsigned)x, (unsigned)x, false, false);
    a = (int)p[0];
    b = (int)p[1];
}

// sum over rows r and r^1 (lanes i and i^16) of a 16-lane row pair
__device__ __forceinline__ float pair16_sum(float x)
{
    float a, b;
    xswap16(x, a, b);
    return a + b;
}
__device__ __forceinline__ float xgroup_sum(float x)
{
    float a, b;
    xswap16(x, a, b);
    xswap32(a + b, a, b);
    return a + b;
}
__device__ __forceinline__ float xgroup_max(float x)
{
    float a, b;
    xswap16(x, a, b);
    xswap32(fmaxf(a, b), a, b);
    return fmaxf(a, b);
}
__device__ __forceinline__ float xgroup_min(float x)
{
    float a, b;
    xswap16(x, a, b);
    xswap32(fminf(a, b), a, b);
    return fminf(a, b);
}

// (value, index) minimum across the lane groups; ties -> smaller index
__device__ __forceinline__ void xgroup_argmin(float &v, int &idx)
{
#pragma unroll
    for (int m = 16; m <= 32; m <<= 1) {
        float v0, v1;
        int i0, i1;
        if (m == 16) {
            xswap16(v, v0, v1);
            xswap16(idx, i0, i1);
        } else {
            xswap32(v, v0, v1);
            xswap32(idx, i0, i1);
        }
        // bitwise, not short-circuit, so that no branch is emitted
        const bool take = (v1 < v0) | ((v1 == v0) & (i1 < i0));
        v = take ? v1 : v0;
        idx = take ? i1 : i0;
    }
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// max / min of three floats.  Written with the compiler builtins (not inline
// asm) so that the compiler's hazard recognizer sees the reads: an inline-asm
// VALU reading an MFMA result gets no wait states and can read the
// register's previous contents.  The sources that call these are compiled
// with -fno-honor-nans, so they lower to single v_max3 / v_min3 without
// NaN canonicalisation.
// (Left-nested, so that a chain min3f(min3f(a, b, c), d, e) folds into two
// instructions.)
__device__ __forceinline__ float max3f(float a, float b, float c)
{
    return __builtin_fmaxf(__builtin_fmaxf(a, b), c);
}
__device__ __forceinline__ float min3f(float a, float b, float c)
{
    return __builtin_fminf(__builtin_fminf(a, b), c);
}

// flip the sign of every element of a fragment
__device__ __forceinline__ Frag<bf16> negate(const Frag<bf16> &f)
{
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u = __builtin_bit_cast(u32x4, f.v) ^ 0x80008000u;
    Frag<bf16> o;
    o.v = __builtin_bit_cast(bf16x8, u);
    return o;
}
__device__ __forceinline__ Frag<float> negate(const Frag<float> &f)
{
    Frag<float> o;
    o.lo = -f.lo;
    o.hi = -f.hi;
    return o;
}

__device__ __forceinline__ int mbcnt(unsigned long long mask)
{
    return (int)__builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                          __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

// ---------------------------------------------------------------- distance frame
// Squared distances are compared as ||c||^2 - 2 k.c, whose fp32 rounding
// error grows with ||k||^2 and ||c||^2 rather than with the distance itself:
// a codebook far from the origin (every coordinate near +32, say) would make
// near-tied keys undecidable.  Translating keys and codewords by a common
// point r changes no distance, so the assignment kernels compare in the
// frame of a per-head reference point r that avq_build_tree derives from the
// codebook (r = 0 for a centred codebook; otherwise coordinates of 3
// significant bits for which every c_t - r_t is exact in the storage type).
// Codewords are staged as -2(c - r), keys shifted in registers, u = k - r,
// rounded to the storage type: exact for any key on the same side of zero
// as an offset coordinate of the codebook.

// round to 3 significant bits (representable in bf16)
__device__ __forceinline__ float coarse3(float x)
{
    return __uint_as_float((__float_as_uint(x) + (1u << 20)) & 0xFFE00000u);
}

template <typename T> __device__ __forceinline__ bool exact_in(float x);
template <> __device__ __forceinline__ bool exact_in<bf16>(float x) { return (float)(bf16)x == x; }
template <> __device__ __forceinline__ bool exact_in<float>(float) { return true; }

// -2 (f - r) for the 8 dimensions of fragment f (r0, r1: r of those
// dimensions); exact in bf16 for the codebook the frame was built from
__device__ __forceinline__ Frag<bf16> frame_m2(const Frag<bf16> &f, f32x4 r0, f32x4 r1)
{
    Frag<bf16> o;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o.v[k] = (bf16)(-2.f * ((float)f.v[k] - r0[k]));
        o.v[4 + k] = (bf16)(-2.f * ((float)f.v[4 + k] - r1[k]));
    }
    return o;
}
__device__ __forceinline__ Frag<float> frame_m2(const Frag<float> &f, f32x4 r0, f32x4 r1)
{
    Frag<float> o;
    o.lo = -2.f * (f.lo - r0);
    o.hi = -2.f * (f.hi - r1);
    return o;
}

// key fragment of dimensions dim0..dim0+7 moved into the frame: k - r
__device__ __forceinline__ Frag<bf16> shift_frag(const Frag<bf16> &f, const float *rv, int dim0)
{
    const f32x4 r0 = *reinterpret_cast<const f32x4 *>(rv + dim0);
    const f32x4 r1 = *reinterpret_cast<const f32x4 *>(rv + dim0 + 4);
    Frag<bf16> o;   // (rounded to nearest: exact for keys the frame covers)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o.v[k] = (bf16)((float)f.v[k] - r0[k]);
        o.v[4 + k] = (bf16)((float)f.v[4 + k] - r1[k]);
    }
    return o;
}
__device__ __forceinline__ Frag<float> shift_frag(const Frag<float> &f, const float *rv, int dim0)
{
    Frag<float> o;
    o.lo = f.lo - *reinterpret_cast<const f32x4 *>(rv + dim0);
    o.hi = f.hi - *reinterpret_cast<const f32x4 *>(rv + dim0 + 4);
    return o;
}

}  // namespace avq
