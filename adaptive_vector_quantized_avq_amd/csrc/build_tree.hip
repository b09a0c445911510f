// Frozen-tree preparation ("AVQ-Attention", Sec. 4.1 parent-child
// constraint): every parent is the mean of its C children (a flat codebook,
// C = 0, is copied: its codewords are the parents; a three-level tree, the
// deeper hierarchy of Sec. 6, gets the constraint at both upper levels);
// every head gets the reference point r of its distance frame (see codebook
// frame below), and every stored codeword its squared norm in that frame
// for the expansion ||k - c||^2 = ||u||^2 + ||c - r||^2 - 2 u.(c - r), u = k - r,
// used by the assignment kernels.
//
// Runs once per codebook; it is not on the per-forward path, so it favours
// exactness over speed: sums are taken in fp64 in index order and rounded
// once.
#include "avq_kernels.h"

namespace avq {

template <typename T>
__global__ void tree_parents_kernel(const T *__restrict__ children, int H, int M0, int C, int d,
                                    T *__restrict__ parents)
{
    const int64_t total = (int64_t)H * M0 * d;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    if (C == 0) {   // a flat codebook ([H][M0][d]) is its own parent level
        parents[i] = children[i];
        return;
    }
    const int t = (int)(i % d);
    const int64_t hp = i / d;                       // h * M0 + p
    const T *src = children + hp * C * d + t;
    double s = 0.0;
    for (int c = 0; c < C; ++c) s += (double)to_float(src[(int64_t)c * d]);
    const double mean = s / (double)C;
    if constexpr (sizeof(T) == 2) {
        uint16_t bits = f64_to_bf16_bits(mean);
        reinterpret_cast<uint16_t *>(parents)[i] = bits;
    } else {
        parents[i] = (float)mean;
    }
}

// Stored codeword row j of head h in slot order: parents [0, M0), children
// [M0, M0 + M0*C), and for a three-level tree (leaves != nullptr) its leaves
// [M0 + M0*C, M0 + M0*C + M0*C*C).
template <typename T>
__device__ __forceinline__ const T *tree_row(const T *parents, const T *children, const T *leaves, int h,
                                             int M0, int C, int d, int j)
{
    const int n1 = M0 * C;
    if (j < M0) return parents + ((int64_t)h * M0 + j) * d;
    if (j < M0 + n1 || leaves == nullptr) return children + ((int64_t)h * n1 + (j - M0)) * d;
    return leaves + ((int64_t)h * n1 * C + (j - M0 - n1)) * d;
}

// Codebook frame of each head: r_t = 0 unless coordinate t of the head's
// stored codewords (every level) is offset from zero by more than twice its
// spread, max |c_t - mean_t|; then r_t is the mean rounded to 3 significant
// bits, kept only if c_t - r_t is exact in the storage type for every
// codeword (else r_t = 0).  Comparing distances as
// ||c - r||^2 - 2 (k - r).(c - r) changes no distance but makes the fp32
// rounding scale with the codebook's spread rather than its offset from the
// origin.  One 256-thread work-group per (head, coordinate); the fp64 sum is
// taken in a fixed order (per-thread strided partials, then a tree), so the
// frame is the same on every run.
constexpr int kFrameThreads = 256;
template <typename T>
__global__ __launch_bounds__(kFrameThreads) void tree_frame_kernel(const T *__restrict__ parents,
                                                                   const T *__restrict__ children,
                                                                   const T *__restrict__ leaves, int H, int M0,
                                                                   int C, int d, float *__restrict__ frame)
{
    __shared__ double rs[kFrameThreads];
    __shared__ float rlo[kFrameThreads], rhi[kFrameThreads];
    __shared__ int rok[kFrameThreads];
    const int h = blockIdx.x / d, t = blockIdx.x % d, tid = threadIdx.x;
    const int S = M0 * (1 + C + (leaves ? C * C : 0));
    auto coord = [&](int j) -> float { return to_float(tree_row(parents, children, leaves, h, M0, C, d, j)[t]); };
    double s = 0.0;
    float lo = INFINITY, hi = -INFINITY;
    for (int j = tid; j < S; j += kFrameThreads) {
        const float c = coord(j);
        s += (double)c;
        lo = fminf(lo, c);
        hi = fmaxf(hi, c);
    }
    rs[tid] = s;
    rlo[tid] = lo;
    rhi[tid] = hi;
    __syncthreads();
    for (int w = kFrameThreads / 2; w >= 1; w >>= 1) {
        if (tid < w) {
            rs[tid] += rs[tid + w];
            rlo[tid] = fminf(rlo[tid], rlo[tid + w]);
            rhi[tid] = fmaxf(rhi[tid], rhi[tid + w]);
        }
        __syncthreads();
    }
    const float mu = (float)(rs[0] / (double)S);
    const float spread = fmaxf(rhi[0] - mu, mu - rlo[0]);
    const float r = fabsf(mu) > 2.f * spread ? coarse3(mu) : 0.f;
    int ok = 1;
    if (r != 0.f) {   // c - r must be exact in the storage type for every codeword
        for (int j = tid; j < S; j += kFrameThreads) {
            const double dl = (double)coord(j) - (double)r;   // exact in fp64
            const float df = (float)dl;
            ok &= ((double)df == dl && exact_in<T>(df)) ? 1 : 0;
        }
    }
    rok[tid] = ok;
    __syncthreads();
    for (int w = kFrameThreads / 2; w >= 1; w >>= 1) {
        if (tid < w) rok[tid] &= rok[tid + w];
        __syncthreads();
    }
    if (tid == 0) frame[blockIdx.x] = rok[0] ? r : 0.f;
}

// one thread per stored codeword row, in slot order (tree_row); norms are
// taken in the head's frame, ||c - r||^2, in fp64 and rounded once
template <typename T>
__global__ void tree_sqnorm_kernel(const T *__restrict__ parents, const T *__restrict__ children,
                                   const T *__restrict__ leaves, const float *__restrict__ frame, int H,
                                   int M0, int C, int d, float *__restrict__ sqnorm)
{
    const int S = M0 * (1 + C + (leaves ? C * C : 0));
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)H * S) return;
    const int h = (int)(i / S);
    const int j = (int)(i % S);
    const T *row = tree_row(parents, children, leaves, h, M0, C, d, j);
    const float *r = frame + (int64_t)h * d;
    double s = 0.0;
    for (int t = 0; t < d; ++t) {
        const double x = (double)to_float(row[t]) - (double)r[t];
        s += x * x;
    }
    sqnorm[i] = (float)s;
}

template <typename T>
static hipError_t launch_tree_t(const void *children, int H, int M0, int C, int d, void *parents,
                                float *sqnorm, float *frame, hipStream_t stream)
{
    const int64_t np = (int64_t)H * M0 * d;
    const int threads = 256;
    hipLaunchKernelGGL(tree_parents_kernel<T>, dim3((unsigned)((np + threads - 1) / threads)),
                       dim3(threads), 0, stream, (const T *)children, H, M0, C, d, (T *)parents);
    const int64_t nf = (int64_t)H * d;
    hipLaunchKernelGGL(tree_frame_kernel<T>, dim3((unsigned)nf), dim3(kFrameThreads), 0, stream,
                       (const T *)parents, (const T *)children, (const T *)nullptr, H, M0, C, d, frame);
    const int64_t nr = (int64_t)H * M0 * (1 + C);
    hipLaunchKernelGGL(tree_sqnorm_kernel<T>, dim3((unsigned)((nr + threads - 1) / threads)),
                       dim3(threads), 0, stream, (const T *)parents, (const T *)children, (const T *)nullptr,
                       (const float *)frame, H, M0, C, d, sqnorm);
    return hipGetLastError();
}

hipError_t launch_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                             void *parents, float *sqnorm, float *frame, hipStream_t stream)
{
    if (dtype == 1) return launch_tree_t<bf16>(children, H, M0, C, d, parents, sqnorm, frame, stream);
    return launch_tree_t<float>(children, H, M0, C, d, parents, sqnorm, frame, stream);
}

// Three-level tree from its leaves [H][M0][C][C][d]: a child is the mean of
// its C leaves and a root the mean of its C*C leaves (each an fp64 sum in
// index order, rounded once); frame and norms over all three levels.
template <typename T>
static hipError_t launch_tree3_t(const void *leaves, int H, int M0, int C, int d, void *level0, void *level1,
                                 float *sqnorm, float *frame, hipStream_t stream)
{
    const int threads = 256;
    const int64_t n1 = (int64_t)H * M0 * C * d, n0 = (int64_t)H * M0 * d;
    hipLaunchKernelGGL(tree_parents_kernel<T>, dim3((unsigned)((n1 + threads - 1) / threads)), dim3(threads), 0,
                       stream, (const T *)leaves, H, M0 * C, C, d, (T *)level1);
    hipLaunchKernelGGL(tree_parents_kernel<T>, dim3((unsigned)((n0 + threads - 1) / threads)), dim3(threads), 0,
                       stream, (const T *)leaves, H, M0, C * C, d, (T *)level0);
    const int64_t nf = (int64_t)H * d;
    hipLaunchKernelGGL(tree_frame_kernel<T>, dim3((unsigned)nf), dim3(kFrameThreads), 0, stream,
                       (const T *)level0, (const T *)level1, (const T *)leaves, H, M0, C, d, frame);
    const int64_t nr = (int64_t)H * M0 * (1 + C + C * C);
    hipLaunchKernelGGL(tree_sqnorm_kernel<T>, dim3((unsigned)((nr + threads - 1) / threads)), dim3(threads), 0,
                       stream, (const T *)level0, (const T *)level1, (const T *)leaves, (const float *)frame, H,
                       M0, C, d, sqnorm);
    return hipGetLastError();
}

hipError_t launch_build_tree3(const void *leaves, int H, int M0, int C, int d, int dtype, void *level0,
                              void *level1, float *sqnorm, float *frame, hipStream_t stream)
{
    if (dtype == 1) return launch_tree3_t<bf16>(leaves, H, M0, C, d, level0, level1, sqnorm, frame, stream);
    return launch_tree3_t<float>(leaves, H, M0, C, d, level0, level1, sqnorm, frame, stream);
}

}  // namespace avq
