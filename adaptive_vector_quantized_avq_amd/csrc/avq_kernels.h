// Host-side launchers of the gfx950 kernels (internal to the library; the
// public boundary is include/avq.h).  Shapes are validated by the ABI layer
// before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "avq_device.h"

namespace avq {

// keys per chunk of the parent-assignment kernel; a chunk's keys are
// bucketed by parent in the workspace
constexpr int kAssignChunk = 1024;
// parents per work-group of the child-refinement / aggregation kernel
constexpr int kRefineGroup = 4;

struct AssignWorkspace {
    int32_t *sorted;      // [B*H][N]            key index | parent << 24, bucketed per chunk
    int32_t *chunk_off;   // [B*H][nchunks][M0+1] bucket starts inside each chunk
    size_t bytes;
};

size_t assign_workspace_bytes(int B, int H, int N, int M0);
AssignWorkspace carve_assign_workspace(void *base, int B, int H, int N, int M0);

hipError_t launch_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                             void *parents, float *sqnorm, hipStream_t stream);

hipError_t launch_assign_aggregate(const void *K, const void *V, const void *parents,
                                   const void *children, const float *sqnorm, int B, int H, int N,
                                   int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                   int32_t *count, int32_t *leaf, const AssignWorkspace &ws,
                                   hipStream_t stream);

// returns hipErrorInvalidConfiguration when the shape does not fit the
// kernel's on-chip budget
hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const float *vsum, const int32_t *count, int B, int H, int N, int d,
                                int M0, int C, int P, int tile, float scale, int dtype, void *Y,
                                int32_t *sel, float *importance, hipStream_t stream);
size_t attention_lds_bytes(int d, int M0, int tile, int dtype);

hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int B, int H, int N,
                                  int d, float scale, int dtype, void *Y, hipStream_t stream);

}  // namespace avq
