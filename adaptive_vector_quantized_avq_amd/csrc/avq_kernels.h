// Host-side launchers of the gfx950 kernels (internal to the library; the
// public boundary is include/avq.h).  Shapes are validated by the ABI layer
// before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "avq_device.h"

namespace avq {

// Raises kernel KERNEL's dynamic-LDS limit to a CU's 160 KB, once per device
// (the attribute belongs to the function on the current device).
template <auto KERNEL> inline void allow_full_lds()
{
    static std::atomic<unsigned long long> done{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    const unsigned long long bit = 1ull << dev;
    if (!(done.load(std::memory_order_relaxed) & bit)) {
        (void)hipFuncSetAttribute((const void *)KERNEL, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  160 * 1024);
        done.fetch_or(bit, std::memory_order_relaxed);
    }
}

// keys per chunk of the parent-assignment kernel; a chunk's keys are
// bucketed by parent in the workspace
constexpr int kAssignChunk = 1024;
// parents per work-group of the child-refinement / aggregation kernel: 4,
// or 2 for C = 16 at d = 128 (four such parents make 68 slots, whose fp32
// accumulators would hold the kernel to one wave per SIMD)
__host__ __device__ constexpr int refine_group(int C, int D)
{
    return C == 16 && D == 128 ? 2 : 4;
}

struct AssignWorkspace {
    int32_t *sorted;      // [B*H][N]  key index | parent << 24, bucketed per chunk
    int2 *seg;            // [B*H][ceil(M0/refine_group)][nchunks] {start, length} of
                          // each refinement group's keys inside each chunk's list
    size_t bytes;
};

// Aggregates rearranged as stage-2 MFMA operands (written by stage 1 next to
// the fp32 value sums).  Per (b, h), byte offsets into one block of
// `bytes` bytes, element type T (the input dtype):
//   pvt [D][M0p]  T      parent value sums, transposed; column of parent j
//                        at (j & ~31) + perm32(j & 31), zero for j >= M0
//   pn  [M0p]     float  parent counts (zero for j >= M0)
//   cvt [M0+1][D][C] T   child value sums, children innermost; entry M0 is
//                        all zero (read for the padding children of a
//                        partly filled chunk)
//   cn  [M0+1][C] float  child counts; entry M0 is all zero
// with M0p = padded_parents(M0).
struct PackLayout {
    size_t pvt, pn, cvt, cn, bytes;
};
// parents padded to a power of two >= 32, so that the stage-2 kernel can be
// specialised on the number of 16-row MFMA blocks
__host__ __device__ inline int padded_parents(int M0)
{
    return M0 <= 32 ? 32 : M0 <= 64 ? 64 : M0 <= 128 ? 128 : 256;
}
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline PackLayout pack_layout(int M0, int C, int D, int esize)
{
    const int M0p = padded_parents(M0);
    PackLayout L;
    size_t o = 0;
    L.pvt = o; o = align256(o + (size_t)D * M0p * esize);
    L.pn = o;  o = align256(o + (size_t)M0p * 4);
    L.cvt = o; o = align256(o + (size_t)(M0 + 1) * D * C * esize);
    L.cn = o;  o = align256(o + (size_t)(M0 + 1) * C * 4);
    L.bytes = o;
    return L;
}

size_t assign_workspace_bytes(int B, int H, int N, int M0, int C, int D);
AssignWorkspace carve_assign_workspace(void *base, int B, int H, int N, int M0, int C, int D);

hipError_t launch_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                             void *parents, float *sqnorm, hipStream_t stream);

// first stage-1 kernel alone (nearest parent + per-chunk bucketing)
hipError_t launch_assign_parent(const void *K, const void *parents, const float *sqnorm, int B, int H,
                                int N, int d, int M0, int C, int dtype, const AssignWorkspace &ws,
                                hipStream_t stream);

hipError_t launch_assign_aggregate(const void *K, const void *V, const void *parents,
                                   const void *children, const float *sqnorm, int B, int H, int N,
                                   int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                   int32_t *count, int32_t *leaf, void *pack,
                                   const AssignWorkspace &ws, hipStream_t stream);

// returns hipErrorInvalidConfiguration when the shape does not fit the
// kernel's on-chip budget
hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int d, int M0, int C, int P,
                                int tile, float scale, int dtype, void *Y, int32_t *sel,
                                float *importance, hipStream_t stream);
// rows of children staged per tile and per step by the attention kernel, or
// 0 if the shape does not fit its LDS budget
int attention_child_chunk(int d, int M0, int C, int P, int tile, int dtype);

hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int B, int H, int N,
                                  int d, float scale, int dtype, void *Y, hipStream_t stream);

}  // namespace avq
