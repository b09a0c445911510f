// Codebook diagnostics the pages report next to the method ("AVQ-Attention",
// appendix "Per-layer codebook analysis", Table 7, and "Codebook
// utilization", Table 9):
//   commitment loss  E ||k - k_hat||^2, the mean over a head's keys of the
//                    squared distance to the leaf codeword the key was
//                    assigned to (from stage 1's leaf ids);
//   active ratio     the fraction of a head's M0 (1 + C) codewords whose
//                    count exceeds 1 % of the fair share N / M_total.
// Off the hot path: one extra read of K and the leaf ids when asked for.
// Sums run in a fixed order (per-chunk partials, then one ordered pass), so
// repeated calls give the same bits.
#include "avq_kernels.h"

namespace avq {

constexpr int kDiagThreads = 256;
constexpr int kDiagChunk = 1024;   // keys per work-group of the commitment pass

// sum over the work-group, every thread gets the result (fixed order: lanes
// by DPP/shuffles in a fixed pattern, then the waves in index order)
__device__ float block_sum(float x, float *red)
{
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    if (lane == 0) red[w] = x;
    __syncthreads();
    float s = 0.f;
    for (int i = 0; i < (int)(blockDim.x >> 6); ++i) s += red[i];
    __syncthreads();
    return s;
}

// per (b, h) and chunk of keys: sum of ||k - code(leaf)||^2; one key per
// thread at a time, 8 dimensions per load; differences of stored values are
// taken in fp32 (exact for bf16), squares summed in fp32
template <typename T, int D>
__global__ __launch_bounds__(kDiagThreads) void commitment_partial_kernel(
    const T *__restrict__ K, const T *__restrict__ parents, const T *__restrict__ children,
    const int32_t *__restrict__ leaf, int H, int N, int M0, int C, float *__restrict__ partial)
{
    __shared__ float red[kDiagThreads / 64];
    const int chunk = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int64_t head = (int64_t)bh * N;
    float acc = 0.f;
    for (int x = threadIdx.x; x < kDiagChunk; x += kDiagThreads) {
        const int key = chunk * kDiagChunk + x;
        if (key >= N) break;
        const int l = leaf[head + key];
        const T *cw = l < M0 ? parents + ((int64_t)h * M0 + l) * D
                             : children + ((int64_t)h * M0 * C + (l - M0)) * D;
        const T *kr = K + (head + key) * D;
        float s = 0.f;
#pragma unroll
        for (int t = 0; t < D; t += 8) {
            const Frag<T> a = load_frag(kr + t), b = load_frag(cw + t);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float u = frag_elem(a, k) - frag_elem(b, k);
                s = fmaf(u, u, s);
            }
        }
        acc += s;
    }
    const float tot = block_sum(acc, red);
    if (threadIdx.x == 0) partial[(int64_t)bh * gridDim.x + chunk] = tot;
}

// per (b, h): ordered sum of the chunk partials / N, and the active ratio
__global__ __launch_bounds__(kDiagThreads) void diagnostics_finish_kernel(
    const float *__restrict__ partial, int nchunks, const int32_t *__restrict__ count, int N, int S,
    float *__restrict__ commit_out, float *__restrict__ active_out)
{
    __shared__ float red[kDiagThreads / 64];
    const int bh = blockIdx.x;
    if (commit_out) {
        float s = 0.f;
        for (int c = threadIdx.x; c < nchunks; c += kDiagThreads) s += partial[(int64_t)bh * nchunks + c];
        const float tot = block_sum(s, red);
        if (threadIdx.x == 0) commit_out[bh] = tot / (float)N;
    }
    if (active_out) {
        const double thresh = 0.01 * (double)N / (double)S;
        float n = 0.f;
        for (int j = threadIdx.x; j < S; j += kDiagThreads) n += (double)count[(int64_t)bh * S + j] > thresh ? 1.f : 0.f;
        const float tot = block_sum(n, red);
        if (threadIdx.x == 0) active_out[bh] = tot / (float)S;
    }
}

size_t diagnostics_workspace_bytes(int B, int H, int N)
{
    return (size_t)B * H * ((N + kDiagChunk - 1) / kDiagChunk) * sizeof(float);
}

template <typename T, int D>
static hipError_t launch_commit(const void *K, const void *parents, const void *children, const int32_t *leaf,
                                int B, int H, int N, int M0, int C, float *partial, hipStream_t stream)
{
    const int nchunks = (N + kDiagChunk - 1) / kDiagChunk;
    hipLaunchKernelGGL((commitment_partial_kernel<T, D>), dim3(nchunks, B * H), dim3(kDiagThreads), 0, stream,
                       (const T *)K, (const T *)parents, (const T *)children, leaf, H, N, M0, C, partial);
    return hipGetLastError();
}

hipError_t launch_codebook_diagnostics(const void *K, const void *parents, const void *children,
                                       const int32_t *leaf, const int32_t *count, int B, int H, int N, int d,
                                       int M0, int C, int dtype, float *commit_out, float *active_out,
                                       void *workspace, hipStream_t stream)
{
    float *partial = (float *)workspace;
    if (commit_out) {
        hipError_t e = dtype == 1 ? (d == 64 ? launch_commit<bf16, 64>(K, parents, children, leaf, B, H, N, M0, C, partial, stream)
                                             : launch_commit<bf16, 128>(K, parents, children, leaf, B, H, N, M0, C, partial, stream))
                                  : (d == 64 ? launch_commit<float, 64>(K, parents, children, leaf, B, H, N, M0, C, partial, stream)
                                             : launch_commit<float, 128>(K, parents, children, leaf, B, H, N, M0, C, partial, stream));
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(diagnostics_finish_kernel, dim3(B * H), dim3(kDiagThreads), 0, stream, partial,
                       (N + kDiagChunk - 1) / kDiagChunk, count, N, M0 * (1 + C), commit_out, active_out);
    return hipGetLastError();
}

}  // namespace avq
