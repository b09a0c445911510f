// Unfused stage 1 of a flat codebook (C = 0), the comparison the pages make
// between fused and unfused VQ precomputation ("AVQ-Attention", Sec. 4.2 last
// paragraph; Table 2, the "unfused VQ" rows): the nearest codeword of every
// key is first written to memory, then a separate pass scatters each key's
// value and a count of one into its codeword's slot with global atomics.
// K, V and the leaf ids each make one trip through HBM, and the fp32 sums
// accumulate in whatever order the atomics land.
#include "avq_kernels.h"

namespace avq {

constexpr int kScatterThreads = 256;

// clear the sums and counts (a fill kernel rather than a memset, so that the
// call can be recorded into a graph)
__global__ __launch_bounds__(256) void zero_aggregates_kernel(float *__restrict__ vsum, int32_t *__restrict__ count,
                                                              int64_t nv, int64_t nc)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nv; i += stride) vsum[i] = 0.f;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nc; i += stride) count[i] = 0;
}

// one thread per (key, 4 consecutive dimensions); the first thread of a key
// also adds its count
template <typename T, int D>
__global__ __launch_bounds__(kScatterThreads) void scatter_aggregate_kernel(
    const T *__restrict__ V, const int32_t *__restrict__ leaf, int64_t nkeys_total, int N, int S,
    float *__restrict__ vsum, int32_t *__restrict__ count)
{
    constexpr int Q = D / 4;
    const int64_t i = (int64_t)blockIdx.x * kScatterThreads + threadIdx.x;
    if (i >= nkeys_total * Q) return;
    const int64_t kg = i / Q;             // global key index (bh * N + key)
    const int q = (int)(i % Q);
    const int64_t bh = kg / N;
    const int slot = leaf[kg];
    const T *v = V + kg * D + 4 * q;
    float *dst = vsum + (bh * S + slot) * D + 4 * q;
#pragma unroll
    for (int k = 0; k < 4; ++k) unsafeAtomicAdd(dst + k, to_float(v[k]));
    if (q == 0) atomicAdd(count + bh * S + slot, 1);
}

template <typename T, int D>
static hipError_t launch_scatter(const void *V, const int32_t *leaf, int B, int H, int N, int M0, float *vsum,
                                 int32_t *count, hipStream_t stream)
{
    const int64_t keys = (int64_t)B * H * N;
    const int64_t threads = keys * (D / 4);
    hipLaunchKernelGGL((scatter_aggregate_kernel<T, D>), dim3((unsigned)((threads + kScatterThreads - 1) / kScatterThreads)),
                       dim3(kScatterThreads), 0, stream, (const T *)V, leaf, keys, N, M0, vsum, count);
    return hipGetLastError();
}

hipError_t launch_assign_aggregate_unfused(const void *K, const void *V, const void *parents, const float *sqnorm,
                                           const float *frame, int B, int H, int N, int d, int M0, int dtype,
                                           float *vsum, int32_t *count, int32_t *leaf, const AssignWorkspace &ws,
                                           hipStream_t stream)
{
    // the leaf ids go to the caller's buffer if given, else to the workspace
    // area that the fused path uses for its bucketed lists (the same size)
    int32_t *ids = leaf ? leaf : ws.sorted;
    const int64_t nv = (int64_t)B * H * M0 * d, nc = (int64_t)B * H * M0;
    hipLaunchKernelGGL(zero_aggregates_kernel, dim3((unsigned)((nv + 255) / 256 < 2048 ? (nv + 255) / 256 : 2048)), dim3(256),
                       0, stream, vsum, count, nv, nc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    err = launch_assign_parent(K, parents, sqnorm, frame, B, H, N, d, M0, 0, dtype, ws, ids, stream);
    if (err != hipSuccess) return err;
    if (dtype == 1)
        return d == 64 ? launch_scatter<bf16, 64>(V, ids, B, H, N, M0, vsum, count, stream)
                       : launch_scatter<bf16, 128>(V, ids, B, H, N, M0, vsum, count, stream);
    return d == 64 ? launch_scatter<float, 64>(V, ids, B, H, N, M0, vsum, count, stream)
                   : launch_scatter<float, 128>(V, ids, B, H, N, M0, vsum, count, stream);
}

}  // namespace avq
