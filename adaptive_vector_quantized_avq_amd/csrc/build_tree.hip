// Frozen-tree preparation ("AVQ-Attention", Sec. 4.1 parent-child
// constraint): every parent is the mean of its C children, and every stored
// codeword gets its squared norm for the distance expansion
// ||k - c||^2 = ||k||^2 + ||c||^2 - 2 k.c used by the assignment kernels.
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

// one thread per stored codeword row; rows [0, M0) of a head are parents,
// rows [M0, S_tot) children in slot order
template <typename T>
__global__ void tree_sqnorm_kernel(const T *__restrict__ parents, const T *__restrict__ children,
                                   int H, int M0, int C, int d, float *__restrict__ sqnorm)
{
    const int S = M0 * (1 + C);
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)H * S) return;
    const int h = (int)(i / S);
    const int j = (int)(i % S);
    const T *row = j < M0 ? parents + ((int64_t)h * M0 + j) * d
                          : children + ((int64_t)h * M0 * C + (j - M0)) * d;
    double s = 0.0;
    for (int t = 0; t < d; ++t) {
        const double x = (double)to_float(row[t]);
        s += x * x;
    }
    sqnorm[i] = (float)s;
}

template <typename T>
static hipError_t launch_tree_t(const void *children, int H, int M0, int C, int d, void *parents,
                                float *sqnorm, hipStream_t stream)
{
    const int64_t np = (int64_t)H * M0 * d;
    const int threads = 256;
    hipLaunchKernelGGL(tree_parents_kernel<T>, dim3((unsigned)((np + threads - 1) / threads)),
                       dim3(threads), 0, stream, (const T *)children, H, M0, C, d, (T *)parents);
    const int64_t nr = (int64_t)H * M0 * (1 + C);
    hipLaunchKernelGGL(tree_sqnorm_kernel<T>, dim3((unsigned)((nr + threads - 1) / threads)),
                       dim3(threads), 0, stream, (const T *)parents, (const T *)children, H, M0, C,
                       d, sqnorm);
    return hipGetLastError();
}

hipError_t launch_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                             void *parents, float *sqnorm, hipStream_t stream)
{
    if (dtype == 1) return launch_tree_t<bf16>(children, H, M0, C, d, parents, sqnorm, stream);
    return launch_tree_t<float>(children, H, M0, C, d, parents, sqnorm, stream);
}

}  // namespace avq
