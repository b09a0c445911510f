// Exact softmax attention ("AVQ-Attention", Sec. 3.1), non-causal, computed
// flash-attention style (Sec. 3.3: per key block J, X_I(J) = A_IJ V_J and
// Z_I(J) = sum_j A_Ij, accumulated with an online maximum).  It serves as the
// timing context next to the AVQ kernels and as the GPU-side check of the
// one-key-per-leaf limit, where AVQ must reproduce exact attention.
//
// Same transposed layout as the AVQ attention kernel: S^T = K_J . Q^T with
// one query per lane, so P^T feeds X^T += V_J^T . P^T directly.
#include "avq_kernels.h"

namespace avq {

constexpr float kLog2eExact = 1.4426950408889634f;
constexpr int kExactKeys = 64;   // keys per LDS block
constexpr int kExactWaves = 4;   // 16 queries per wave

template <typename T, int D>
__global__ __launch_bounds__(64 * kExactWaves) void exact_attention_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const T *__restrict__ V, int N, float sl2,
    T *__restrict__ Y)
{
    constexpr int KB = kExactKeys;
    constexpr int NT = 64 * kExactWaves;
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int LDP = D + 8;
    constexpr int LDV = KB + 8;
    __shared__ __align__(16) T Ks[KB * LDP];
    __shared__ __align__(16) T Vt[D * LDV];

    const int bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int64_t base = (int64_t)bh * N * D;
    const int q = blockIdx.x * (16 * kExactWaves) + 16 * w + i16;
    const bool qv = q < N;
    Frag<T> qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = qv ? load_frag(Q + base + (int64_t)q * D + 32 * ks + 8 * g) : zero_frag<T>();

    float m = -INFINITY, lsum = 0.f;
    f32x4 X[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) X[db] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int k0 = 0; k0 < N; k0 += KB) {
        __syncthreads();
        for (int e = tid * 8; e < KB * D; e += NT * 8) {
            const int r = e / D, c = e % D;
            Frag<T> f = (k0 + r) < N ? load_frag(K + base + (int64_t)(k0 + r) * D + c) : zero_frag<T>();
            store_frag(Ks + r * LDP + c, f);
        }
        for (int e = tid; e < KB * (D / 8); e += NT) {
            const int r = e / (D / 8), c8 = e % (D / 8);
            Frag<T> f = (k0 + r) < N ? load_frag(V + base + (int64_t)(k0 + r) * D + 8 * c8) : zero_frag<T>();
            const int pos = (r & ~31) + perm32(r & 31);
#pragma unroll
            for (int k = 0; k < 8; ++k) Vt[(8 * c8 + k) * LDV + pos] = from_float<T>(frag_elem(f, k));
        }
        __syncthreads();
        f32x4 Sb[KB / 16];
        float mb = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < KB / 16; ++rb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a = mma(load_frag(Ks + (16 * rb + i16) * LDP + 32 * ks + 8 * g), qf[ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (k0 + 16 * rb + 4 * g + r) < N ? a[r] * sl2 : -INFINITY;
                a[r] = x;
                mb = fmaxf(mb, x);
            }
            Sb[rb] = a;
        }
        mb = xgroup_max(mb);
        const float mn = fmaxf(m, mb);
        const float alpha = exp2f(m - mn);
        m = mn;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) X[db] *= alpha;
#pragma unroll
        for (int rb = 0; rb < KB / 16; ++rb) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = exp2f(Sb[rb][r] - m);
                Sb[rb][r] = e;
                lsum += e;
            }
        }
#pragma unroll
        for (int s = 0; s < KB / 32; ++s) {
            const Frag<T> bf = pack_frag<T>(Sb[2 * s], Sb[2 * s + 1]);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                X[db] = mma(load_frag(Vt + (16 * db + i16) * LDV + 32 * s + 8 * g), bf, X[db]);
        }
    }
    const float L = xgroup_sum(lsum);
    if (qv) {
        const float rl = 1.0f / L;
        T *yr = Y + base + (int64_t)q * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) yr[16 * db + 4 * g + r] = from_float<T>(X[db][r] * rl);
    }
}

// Capture ("AVQ-Attention", Sec. 5.2 and Table 6): for every query, the
// fraction of its exact softmax weight that falls on keys whose parent is
// among the P parents its query tile selected.  Same logits and online
// maximum as above, without the values: per key block, the unnormalised
// weights are summed twice, over all keys and over the keys flagged for the
// wave's tile.  A wave's 16 queries always lie in one tile (tiles are
// multiples of 32 queries).
template <typename T, int D>
__global__ __launch_bounds__(64 * kExactWaves) void exact_capture_kernel(
    const T *__restrict__ Q, const T *__restrict__ K, const int32_t *__restrict__ leaf,
    const int32_t *__restrict__ sel, int N, int M0, int C, int P, int ltile, int ntiles, float sl2,
    float *__restrict__ capture)
{
    constexpr int KB = kExactKeys;
    constexpr int KS = D / 32;
    constexpr int LDP = D + 8;
    constexpr int NT = 64 * kExactWaves;
    __shared__ __align__(16) T Ks[KB * LDP];
    __shared__ int pk[KB];                                  // parent of each staged key
    __shared__ __align__(16) float flg[kExactWaves][KB];    // 1 if that parent is selected
    __shared__ unsigned msk[kExactWaves][8];                // the wave's tile selection, 256 bits

    const int bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int64_t base = (int64_t)bh * N * D;
    const int q0w = blockIdx.x * (16 * kExactWaves) + 16 * w;
    const int q = q0w + i16;
    const bool qv = q < N;
    const int tile = min(q0w >> ltile, ntiles - 1);

    if (lane < 8) msk[w][lane] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    for (int k = lane; k < P; k += 64) {
        const int p = sel[((int64_t)bh * ntiles + tile) * P + k];
        atomicOr(&msk[w][p >> 5], 1u << (p & 31));
    }

    Frag<T> qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = qv ? load_frag(Q + base + (int64_t)q * D + 32 * ks + 8 * g) : zero_frag<T>();

    float m = -INFINITY, lsum = 0.f, lsel = 0.f;
    for (int k0 = 0; k0 < N; k0 += KB) {
        __syncthreads();
        for (int e = tid * 8; e < KB * D; e += NT * 8) {
            const int r = e / D, c = e % D;
            Frag<T> f = (k0 + r) < N ? load_frag(K + base + (int64_t)(k0 + r) * D + c) : zero_frag<T>();
            store_frag(Ks + r * LDP + c, f);
        }
        if (tid < KB) {
            const int l = (k0 + tid) < N ? leaf[(int64_t)bh * N + k0 + tid] : 0;
            pk[tid] = (l < M0 || C == 0) ? l : (l - M0) / C;
        }
        __syncthreads();
        {   // this wave's flags for the staged keys
            const int p = pk[lane];
            flg[w][lane] = (msk[w][p >> 5] >> (p & 31)) & 1u ? 1.f : 0.f;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 Sb[KB / 16];
        float mb = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < KB / 16; ++rb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a = mma(load_frag(Ks + (16 * rb + i16) * LDP + 32 * ks + 8 * g), qf[ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (k0 + 16 * rb + 4 * g + r) < N ? a[r] * sl2 : -INFINITY;
                a[r] = x;
                mb = fmaxf(mb, x);
            }
            Sb[rb] = a;
        }
        mb = xgroup_max(mb);
        const float mn = fmaxf(m, mb);
        const float alpha = exp2f(m - mn);
        m = mn;
        lsum *= alpha;
        lsel *= alpha;
#pragma unroll
        for (int rb = 0; rb < KB / 16; ++rb) {
            const f32x4 f = *reinterpret_cast<const f32x4 *>(&flg[w][16 * rb + 4 * g]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = exp2f(Sb[rb][r] - m);
                lsum += e;
                lsel = fmaf(e, f[r], lsel);
            }
        }
    }
    const float L = xgroup_sum(lsum), Ls = xgroup_sum(lsel);
    if (qv && g == 0) capture[(int64_t)bh * N + q] = Ls / L;
}

template <typename T, int D>
static hipError_t launch_capture_t(const void *Q, const void *K, const int32_t *leaf, const int32_t *sel, int B,
                                   int H, int N, int M0, int C, int P, int tile, float scale, float *capture,
                                   hipStream_t stream)
{
    const int qpb = 16 * kExactWaves;
    int ltile = 0;
    while ((1 << (ltile + 1)) <= tile) ++ltile;
    hipLaunchKernelGGL((exact_capture_kernel<T, D>), dim3((N + qpb - 1) / qpb, B * H), dim3(64 * kExactWaves), 0,
                       stream, (const T *)Q, (const T *)K, leaf, sel, N, M0, C, P, ltile, (N + tile - 1) / tile,
                       scale * kLog2eExact, capture);
    return hipGetLastError();
}

hipError_t launch_capture(const void *Q, const void *K, const int32_t *leaf, const int32_t *sel, int B, int H,
                          int N, int d, int M0, int C, int P, int tile, float scale, int dtype, float *capture,
                          hipStream_t stream)
{
    if (dtype == 1)
        return d == 64 ? launch_capture_t<bf16, 64>(Q, K, leaf, sel, B, H, N, M0, C, P, tile, scale, capture, stream)
                       : launch_capture_t<bf16, 128>(Q, K, leaf, sel, B, H, N, M0, C, P, tile, scale, capture, stream);
    return d == 64 ? launch_capture_t<float, 64>(Q, K, leaf, sel, B, H, N, M0, C, P, tile, scale, capture, stream)
                   : launch_capture_t<float, 128>(Q, K, leaf, sel, B, H, N, M0, C, P, tile, scale, capture, stream);
}

template <typename T, int D>
static hipError_t launch_exact_t(const void *Q, const void *K, const void *V, int B, int H, int N,
                                 float scale, void *Y, hipStream_t stream)
{
    const int qpb = 16 * kExactWaves;
    hipLaunchKernelGGL((exact_attention_kernel<T, D>), dim3((N + qpb - 1) / qpb, B * H),
                       dim3(64 * kExactWaves), 0, stream, (const T *)Q, (const T *)K, (const T *)V, N,
                       scale * kLog2eExact, (T *)Y);
    return hipGetLastError();
}

hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int B, int H, int N,
                                  int d, float scale, int dtype, void *Y, hipStream_t stream)
{
    if (dtype == 1) {
        if (d == 64) return launch_exact_t<bf16, 64>(Q, K, V, B, H, N, scale, Y, stream);
        return launch_exact_t<bf16, 128>(Q, K, V, B, H, N, scale, Y, stream);
    }
    if (d == 64) return launch_exact_t<float, 64>(Q, K, V, B, H, N, scale, Y, stream);
    return launch_exact_t<float, 128>(Q, K, V, B, H, N, scale, Y, stream);
}

}  // namespace avq
