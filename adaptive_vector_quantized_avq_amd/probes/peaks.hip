// Throughput probes for the roofline denominators (not part of the AVQ
// library): each kernel keeps 8 independent dependency chains per lane of one
// instruction kind in flight for `iters` iterations and writes one value per
// lane so that nothing is optimised away.  bench.py --peaks times them with
// HIP events and divides the work by the time.
//   mfma  v_mfma_f32_16x16x32_bf16: 16*16*32*2 flops per wave instruction
//   fma   v_fma_f32: 2 flops per lane
//   exp   v_exp_f32 (exp2): one exponential per lane
// Every launch writes exactly blocks * threads floats to `out`.
#include <hip/hip_runtime.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_mfma_kernel(int iters, float *out)
{
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    bf16x8 a, b;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        a[k] = (__bf16)(1e-3f * (float)((threadIdx.x + k) & 7));
        b[k] = (__bf16)(1e-3f * (float)((threadIdx.x * 3 + k) & 7));
    }
    f32x4 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, (float)j};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
    out[tid] = s;
}

__global__ __launch_bounds__(256) void probe_fma_kernel(int iters, float *out)
{
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    float x[8];
    const float m = 0.999f, a = 1e-3f * (float)(threadIdx.x & 15);
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = (float)j;
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = fmaf(x[j], m, a);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    out[tid] = s;
}

__global__ __launch_bounds__(256) void probe_exp_kernel(int iters, float *out)
{
    const int tid = blockIdx.x * blockDim.x + threadIdx.x;
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) x[j] = -1.0f - 0.125f * (float)j - 1e-3f * (float)(threadIdx.x & 7);
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __builtin_amdgcn_exp2f(x[j]);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) s += x[j];
    out[tid] = s;
}

// plain device copy of n 16-byte words (the profiler-counter calibration:
// it reads and writes exactly 16 n bytes)
__global__ __launch_bounds__(256) void probe_copy_kernel(const float4 *__restrict__ src, float4 *__restrict__ dst,
                                                         long long n)
{
    for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (long long)gridDim.x * blockDim.x)
        dst[i] = src[i];
}

extern "C" {

// copy `bytes` (a multiple of 16) from src to dst on the device
int avq_probe_copy(const void *src, void *dst, long long bytes, void *stream)
{
    if (!src || !dst || bytes <= 0 || (bytes & 15)) return -1;
    hipLaunchKernelGGL(probe_copy_kernel, dim3(4096), dim3(256), 0, (hipStream_t)stream,
                       (const float4 *)src, (float4 *)dst, bytes / 16);
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

// kind: 0 = mfma, 1 = fma, 2 = exp.  256 threads per block.
int avq_probe_launch(int kind, int blocks, int iters, float *out, void *stream)
{
    if (blocks < 1 || iters < 1 || !out) return -1;
    hipStream_t s = (hipStream_t)stream;
    switch (kind) {
    case 0: hipLaunchKernelGGL(probe_mfma_kernel, dim3(blocks), dim3(256), 0, s, iters, out); break;
    case 1: hipLaunchKernelGGL(probe_fma_kernel, dim3(blocks), dim3(256), 0, s, iters, out); break;
    case 2: hipLaunchKernelGGL(probe_exp_kernel, dim3(blocks), dim3(256), 0, s, iters, out); break;
    default: return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
