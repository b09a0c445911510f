// Stage 2 input preparation: the caller's fp32 value sums and int32 counts
// ("AVQ-Attention", Sec. 4.3: the numerator sums Vbar and the denominator
// counts n of every codeword) rearranged as the attention kernel's
// matrix-core operands (PackLayout in avq_kernels.h), in the call's
// workspace.  Pure data movement plus one rounding of each value sum to the
// input dtype; it runs at the start of every avq_attention_fwd call, so
// stage 2 reads only what the caller hands it.
//
// One item per thread, so that every thread issues its loads at once and
// the kernel costs a single memory round trip.  Items of one (b, h), in
// order:
//   pvt  item (t, q8): 8 consecutive operand columns 8*q8.. of dimension t;
//        column 32*b + perm32(rho) holds parent 32*b + rho (zero past M0).
//        Threads with consecutive t read consecutive sums (coalesced);
//   cvt  item (p, t, group of 8 children): the children's sums of dimension
//        t, children innermost; entry M0 is all zero;
//   pn   parent counts as fp32 (zero past M0);
//   cn   child counts as fp32; entry M0 is all zero;
//   pz, cz  (16-bit operands, two-level trees) the parent and child counts
//        split into three bf16 parts each (count_part), laid out like pvt
//        and cvt, for the kernel's denominators on the matrix cores;
//   and for a three-level tree the same two sections for the children as
//   parents of the leaves (gvt, gn).
// The grid is 1-D, with the (b, h) units spread over the XCDs in contiguous
// ranges the way the attention kernel spreads them, so that a head's operands
// are written from the XCD whose L2 then reads them.
#include "avq_kernels.h"

namespace avq {

constexpr int kPackThreads = 256;

template <typename T> __device__ __forceinline__ void store8(T *dst, const float (&v)[8]);
template <> __device__ __forceinline__ void store8<bf16>(bf16 *dst, const float (&v)[8])
{
    bf16x8 o;
#pragma unroll
    for (int k = 0; k < 8; ++k) o[k] = (bf16)v[k];
    *reinterpret_cast<bf16x8 *>(dst) = o;
}
template <> __device__ __forceinline__ void store8<float>(float *dst, const float (&v)[8])
{
    *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
}

template <int D, int CC, bool L3, bool ZB> __host__ __device__ inline int pack_items(int M0)
{
    const int NG = CC >= 8 ? CC / 8 : 1;
    const int n1 = M0 * CC;
    return D * (padded_parents(M0) / 8) + (CC > 0 ? (M0 + 1) * D * NG : 0) + padded_parents(M0) +
           (M0 + 1) * CC + (ZB ? 4 * (padded_parents(M0) / 8) + (M0 + 1) * 3 * CC : 0) +
           (L3 ? (n1 + 1) * D * NG + (n1 + 1) * CC : 0);
}

// part r (0, 1, 2) of the split of a count n (an integer below 2^21) into
// three bf16 values that sum to it exactly: hi = n rounded to bf16, mid = the
// rest rounded, lo = what is left (a small integer, exact in bf16)
__device__ __forceinline__ float count_part(float n, int r)
{
    const float hi = (float)(bf16)n;
    const float mid = (float)(bf16)(n - hi);
    return r == 0 ? hi : r == 1 ? mid : n - hi - mid;
}

// child sums of one level: item (p, t, group of 8 children) of `np1` parents
// (entry np1 - 1 all zero), children of parent p at slots c0 + p*CC + k
template <typename T, int D, int CC>
__device__ __forceinline__ void pack_child_item(int a, const float *vs, int c0, int np, T *cvt)
{
    constexpr int CG = CC >= 8 ? 8 : CC;   // children per item
    constexpr int NG = CC / CG;
    const int t = a % D, r = a / D, cg = r % NG, p = r / NG;
    T *dst = cvt + ((size_t)p * D + t) * CC + CG * cg;
    if constexpr (CG == 8) {
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = p < np ? vs[((size_t)c0 + (size_t)p * CC + 8 * cg + k) * D + t] : 0.f;
        store8<T>(dst, v);
    } else {
#pragma unroll
        for (int k = 0; k < CG; ++k) dst[k] = from_float<T>(p < np ? vs[((size_t)c0 + (size_t)p * CC + k) * D + t] : 0.f);
    }
}

template <typename T, int D, int CC, bool L3, bool ZB>
__global__ __launch_bounds__(kPackThreads) void pack_aggregates_kernel(
    const float *__restrict__ vsum, const int32_t *__restrict__ count, int M0, int nbh, int parts,
    unsigned char *__restrict__ pack)
{
    const int G8 = gridDim.x >> 3;
    const int unit = (blockIdx.x & 7) * G8 + (blockIdx.x >> 3);
    const int bh = unit / parts, part = unit - bh * parts;
    if (bh >= nbh) return;
    const int M0p = padded_parents(M0);
    const int n1 = M0 * CC;
    const int S = M0 + n1 + (L3 ? n1 * CC : 0);
    const PackLayout PL = pack_layout(M0, CC, D, (int)sizeof(T), L3);
    unsigned char *pk = pack + (size_t)bh * PL.bytes;
    const float *vs = vsum + (size_t)bh * S * D;
    const int32_t *cs = count + (size_t)bh * S;
    int a = part * kPackThreads + threadIdx.x;

    // parent value sums, transposed, columns permuted within 32-blocks
    const int n_pvt = D * (M0p / 8);
    if (a < n_pvt) {
        const int t = a % D, q8 = a / D;
        const int base = 32 * (q8 >> 2), q = q8 & 3;
        float v[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int j = base + (k < 4 ? 4 * q + k : 16 + 4 * q + (k - 4));
            v[k] = j < M0 ? vs[(size_t)j * D + t] : 0.f;
        }
        store8<T>(reinterpret_cast<T *>(pk + PL.pvt) + (size_t)t * M0p + 8 * q8, v);
        return;
    }
    a -= n_pvt;
    constexpr int NG = CC >= 8 ? CC / 8 : 1;
    if constexpr (CC > 0) {
        const int n_cvt = (M0 + 1) * D * NG;
        if (a < n_cvt) {
            pack_child_item<T, D, CC>(a, vs, M0, M0, reinterpret_cast<T *>(pk + PL.cvt));
            return;
        }
        a -= n_cvt;
    }
    if (a < M0p) {
        reinterpret_cast<float *>(pk + PL.pn)[a] = a < M0 ? (float)cs[a] : 0.f;
        return;
    }
    a -= M0p;
    if (a < (M0 + 1) * CC) {
        reinterpret_cast<float *>(pk + PL.cn)[a] = a < M0 * CC ? (float)cs[M0 + a] : 0.f;
        return;
    }
    a -= (M0 + 1) * CC;
    if constexpr (ZB) {   // the counts as exact sums of three bf16 parts
        const int n_pz = 4 * (M0p / 8);
        if (a < n_pz) {   // parents: rows hi, mid, lo, zero; columns as in pvt
            const int r = a / (M0p / 8), q8 = a % (M0p / 8);
            const int base = 32 * (q8 >> 2), q = q8 & 3;
            float v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int j = base + (k < 4 ? 4 * q + k : 16 + 4 * q + (k - 4));
                v[k] = r < 3 && j < M0 ? count_part((float)cs[j], r) : 0.f;
            }
            store8<bf16>(reinterpret_cast<bf16 *>(pk + PL.pz) + (size_t)r * M0p + 8 * q8, v);
            return;
        }
        a -= n_pz;
        if (a < (M0 + 1) * 3 * CC) {   // children [M0+1][3][CC], entry M0 zero
            const int p = a / (3 * CC), r = (a / CC) % 3, c = a % CC;
            reinterpret_cast<bf16 *>(pk + PL.cz)[a] = (bf16)(p < M0 ? count_part((float)cs[M0 + p * CC + c], r) : 0.f);
            return;
        }
        a -= (M0 + 1) * 3 * CC;
    }
    if constexpr (L3) {   // the leaves' sums and counts, the children as parents
        const int n_gvt = (n1 + 1) * D * NG;
        if (a < n_gvt) {
            pack_child_item<T, D, CC>(a, vs, M0 + n1, n1, reinterpret_cast<T *>(pk + PL.gvt));
            return;
        }
        a -= n_gvt;
        if (a < (n1 + 1) * CC)
            reinterpret_cast<float *>(pk + PL.gn)[a] = a < n1 * CC ? (float)cs[M0 + n1 + a] : 0.f;
    }
}

template <typename T, int D, int CC, bool L3>
static hipError_t launch_pack_k(const float *vsum, const int32_t *count, int BH, int M0, void *pack,
                                hipStream_t stream)
{
    constexpr bool ZB = sizeof(T) == 2 && !L3;
    const int parts = (pack_items<D, CC, L3, ZB>(M0) + kPackThreads - 1) / kPackThreads;
    const int grid = (BH * parts + 7) & ~7;
    hipLaunchKernelGGL((pack_aggregates_kernel<T, D, CC, L3, ZB>), dim3(grid), dim3(kPackThreads), 0, stream, vsum,
                       count, M0, BH, parts, (unsigned char *)pack);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_pack_t(const float *vsum, const int32_t *count, int BH, int M0, int C, void *pack,
                                hipStream_t stream, bool l3)
{
    if (l3) {
        switch (C) {
        case 2: return launch_pack_k<T, D, 2, true>(vsum, count, BH, M0, pack, stream);
        case 4: return launch_pack_k<T, D, 4, true>(vsum, count, BH, M0, pack, stream);
        case 8: return launch_pack_k<T, D, 8, true>(vsum, count, BH, M0, pack, stream);
        default: return launch_pack_k<T, D, 16, true>(vsum, count, BH, M0, pack, stream);
        }
    }
    switch (C) {
    case 0: return launch_pack_k<T, D, 0, false>(vsum, count, BH, M0, pack, stream);
    case 2: return launch_pack_k<T, D, 2, false>(vsum, count, BH, M0, pack, stream);
    case 4: return launch_pack_k<T, D, 4, false>(vsum, count, BH, M0, pack, stream);
    case 8: return launch_pack_k<T, D, 8, false>(vsum, count, BH, M0, pack, stream);
    default: return launch_pack_k<T, D, 16, false>(vsum, count, BH, M0, pack, stream);
    }
}

hipError_t launch_pack_aggregates(const float *vsum, const int32_t *count, int B, int H, int d, int M0, int C,
                                  int dtype, void *pack, hipStream_t stream, bool three_level)
{
    if (dtype == 1)
        return d == 64 ? launch_pack_t<bf16, 64>(vsum, count, B * H, M0, C, pack, stream, three_level)
                       : launch_pack_t<bf16, 128>(vsum, count, B * H, M0, C, pack, stream, three_level);
    return d == 64 ? launch_pack_t<float, 64>(vsum, count, B * H, M0, C, pack, stream, three_level)
                   : launch_pack_t<float, 128>(vsum, count, B * H, M0, C, pack, stream, three_level);
}

}  // namespace avq
