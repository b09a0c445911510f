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

// How the refinement kernel splits its groups' key lists.  A (b, h) whose
// per-chunk largest group counts sum to at most `quiet` (three times the
// mean group length, at least 1024) cannot hold a group that long: no group
// is split.  Otherwise a group longer than `target` keys (twice the mean,
// at least 1024) becomes ceil(n / target) equal slices, one work-group
// each; then at most max_items items and max_partials stored partial sums
// per (b, h).
struct RefinePlan {
    int target, quiet, max_items, max_partials;
};
inline RefinePlan refine_plan(int N, int M0, int C, int D)
{
    const int ngroups = (M0 + refine_group(C, D) - 1) / refine_group(C, D);
    const int mean = (N + ngroups - 1) / ngroups;
    RefinePlan p;
    p.target = 2 * mean < 1024 ? 1024 : 2 * mean;
    p.quiet = 3 * mean < 1024 ? 1024 : 3 * mean;
    p.max_partials = (N + p.target - 1) / p.target;
    p.max_items = ngroups + p.max_partials;
    return p;
}
// fp32 words of one stored partial: the slot rows of a group (padded to 16)
// times (D value sums + 1 count)
inline size_t refine_partial_words(int C, int D)
{
    const int rows = (refine_group(C, D) * (C + 1) + 15) / 16 * 16;
    return (size_t)rows * (D + 1);
}
// a tag distinct for every refinement launch of the process (never 0): a
// slice's "partial stored" flag is the tag of its launch, so flags left in
// a workspace by earlier calls never match
unsigned next_call_tag();

struct AssignWorkspace {
    int32_t *sorted;      // [B*H][N]  key index | parent << 24, bucketed per chunk
    int2 *seg;            // [B*H][ceil(M0/refine_group)][nchunks] {start, length} of
                          // each refinement group's keys inside each chunk's list
    int32_t *cmax;        // [B*H][nchunks][2] largest group's key count in each chunk (two
                          // halves of the groups; a bound on every group's total)
    float *partial;       // [B*H][max_partials][refine_partial_words] sums of split groups' slices
    unsigned *pflag;      // [B*H][max_partials] launch tag once a slice's partial is stored
    size_t bytes;
};


// Aggregates rearranged as stage-2 MFMA operands (written into the stage-2
// workspace from the caller's fp32 value sums and int32 counts by
// pack_aggregates.hip).  Per (b, h), byte offsets into one block of `bytes`
// bytes, element type T (the input dtype):
//   pvt [D][M0p]  T      parent value sums, transposed; column of parent j
//                        at (j & ~31) + perm32(j & 31), zero for j >= M0
//   pn  [M0p]     float  parent counts (zero for j >= M0)
//   cvt [M0+1][D][C] T   child value sums, children innermost; entry M0 is
//                        all zero (read for the padding children of a
//                        partly filled chunk)
//   cn  [M0+1][C] float  child counts; entry M0 is all zero
// and, for a two-level tree with 16-bit operands, the counts as matrix-core
// operands (each count n split exactly into three bf16 parts n = hi + mid +
// lo, so that a product with a bf16 weight is exact), from which the kernel
// forms the softmax denominators with the same rounded weights as the value
// sums:
//   pz  [4][M0p] bf16    rows hi, mid, lo of the parent counts, columns
//                        permuted like pvt; row 3 all zero
//   cz  [M0+1][3][C] bf16  hi, mid, lo of the child counts; entry M0 zero
// and, for a three-level tree, the same two value/count sections one level
// down (the M0*C children as parents of their C leaves):
//   gvt [M0*C+1][D][C] T, gn [M0*C+1][C] float (entry M0*C all zero)
// with M0p = padded_parents(M0).
struct PackLayout {
    size_t pvt, pn, cvt, cn, pz, cz, gvt, gn, bytes;
};
// parents padded to a power of two >= 32, so that the stage-2 kernel can be
// specialised on the number of 16-row MFMA blocks
__host__ __device__ inline int padded_parents(int M0)
{
    return M0 <= 32 ? 32 : M0 <= 64 ? 64 : M0 <= 128 ? 128 : 256;
}
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
__host__ __device__ inline PackLayout pack_layout(int M0, int C, int D, int esize, bool three_level = false)
{
    const int M0p = padded_parents(M0);
    PackLayout L;
    size_t o = 0;
    L.pvt = o; o = align256(o + (size_t)D * M0p * esize);
    L.pn = o;  o = align256(o + (size_t)M0p * 4);
    L.cvt = o; o = align256(o + (size_t)(M0 + 1) * D * C * esize);
    L.cn = o;  o = align256(o + (size_t)(M0 + 1) * C * 4);
    const bool zb = esize == 2 && !three_level;
    L.pz = o;  o = align256(o + (zb ? (size_t)4 * M0p * 2 : 0));
    L.cz = o;  o = align256(o + (zb ? (size_t)(M0 + 1) * 3 * C * 2 : 0));
    L.gvt = o; L.gn = o;
    if (three_level) {
        const size_t n1 = (size_t)M0 * C;
        L.gvt = o; o = align256(o + (n1 + 1) * D * C * esize);
        L.gn = o;  o = align256(o + (n1 + 1) * C * 4);
    }
    L.bytes = o;
    return L;
}

size_t assign_workspace_bytes(int B, int H, int N, int M0, int C, int D);
AssignWorkspace carve_assign_workspace(void *base, int B, int H, int N, int M0, int C, int D);

hipError_t launch_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                             void *parents, float *sqnorm, float *frame, hipStream_t stream);

// first stage-1 kernel alone (nearest parent + per-chunk bucketing)
// (leaf_direct != nullptr: write each key's parent there instead of the
// bucketed lists -- the unfused stage 1 of a flat codebook)
hipError_t launch_assign_parent(const void *K, const void *parents, const float *sqnorm, const float *frame,
                                int B, int H, int N, int d, int M0, int C, int dtype,
                                const AssignWorkspace &ws, int32_t *leaf_direct, hipStream_t stream);

// Unfused stage 1 of a flat codebook (C = 0): nearest codeword of every key
// written to memory, then a separate scatter of values and counts with
// global atomics (fp32 sums in a nondeterministic order)
hipError_t launch_assign_aggregate_unfused(const void *K, const void *V, const void *parents, const float *sqnorm,
                                           const float *frame, int B, int H, int N, int d, int M0, int dtype,
                                           float *vsum, int32_t *count, int32_t *leaf, const AssignWorkspace &ws,
                                           hipStream_t stream);

hipError_t launch_assign_aggregate(const void *K, const void *V, const void *parents,
                                   const void *children, const float *sqnorm, const float *frame, int B,
                                   int H, int N,
                                   int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                   int32_t *count, int32_t *leaf, const AssignWorkspace &ws,
                                   hipStream_t stream);

// second stage-1 kernel alone on caller-built lists: slot_stride = slots
// (and norms) per head, leaf_base added to every leaf id written
hipError_t launch_refine_slots(const void *K, const void *V, const void *parents, const void *children,
                               const float *sqnorm, const float *frame, int B, int H, int N, int d, int M0,
                               int C, int dtype, unsigned flags, float *vsum, int32_t *count, int32_t *leaf,
                               const AssignWorkspace &ws, int slot_stride, int leaf_base, hipStream_t stream);

// three-level tree (roots -> children -> leaves): the two upper levels from
// the leaves, frame and norms over all three (slot order)
hipError_t launch_build_tree3(const void *leaves, int H, int M0, int C, int d, int dtype, void *level0,
                              void *level1, float *sqnorm, float *frame, hipStream_t stream);
size_t assign3_workspace_bytes(int B, int H, int N, int M0, int C, int D);
// stage 1 of a three-level tree; leaf may be null (the workspace then holds
// the leaf ids the second descent needs)
hipError_t launch_assign_aggregate3(const void *K, const void *V, const void *level0, const void *level1,
                                    const void *leaves, const float *sqnorm, const float *frame, int B, int H,
                                    int N, int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                    int32_t *count, int32_t *leaf, void *workspace, hipStream_t stream);

// stage-2 operand pack (PackLayout, B*H blocks) from fp32 sums and int32 counts
// (three_level: slots in the three-level layout, grandchild sections filled)
hipError_t launch_pack_aggregates(const float *vsum, const int32_t *count, int B, int H, int d, int M0, int C,
                                  int dtype, void *pack, hipStream_t stream, bool three_level = false);

// returns hipErrorInvalidConfiguration when the shape does not fit the
// kernel's on-chip budget.  leaves != nullptr: three-level tree (children
// are the middle level), sel1 receives the selected children
hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int d, int M0, int C, int P,
                                int tile, float scale, int dtype, void *Y, int32_t *sel,
                                float *importance, hipStream_t stream, const void *leaves = nullptr,
                                int32_t *sel1 = nullptr);
// rows of children staged per tile and per step by the attention kernel, or
// 0 if the shape does not fit its LDS budget
int attention_child_chunk(int d, int M0, int C, int P, int tile, int dtype, bool three_level = false);

// codebook diagnostics: commitment loss (needs K, the tree and leaf ids) and
// active ratio (needs counts); workspace of diagnostics_workspace_bytes
size_t diagnostics_workspace_bytes(int B, int H, int N);
hipError_t launch_codebook_diagnostics(const void *K, const void *parents, const void *children,
                                       const int32_t *leaf, const int32_t *count, int B, int H, int N, int d,
                                       int M0, int C, int dtype, float *commit_out, float *active_out,
                                       void *workspace, hipStream_t stream);
// per-query capture of the exact softmax weight by the tiles' selections
hipError_t launch_capture(const void *Q, const void *K, const int32_t *leaf, const int32_t *sel, int B, int H,
                          int N, int d, int M0, int C, int P, int tile, float scale, int dtype, float *capture,
                          hipStream_t stream);

// Gilbert-curve order of a W x H grid's cells (host), and row gather /
// scatter of [rows][row_bytes] tensors by a permutation of N rows per (b, h)
void gilbert_cells(int W, int H, int32_t *out);
hipError_t launch_permute_rows(const void *src, const int32_t *order, int64_t rows, int N, int row_bytes,
                               int inverse, void *dst, hipStream_t stream);

hipError_t launch_exact_attention(const void *Q, const void *K, const void *V, int B, int H, int N,
                                  int d, float scale, int dtype, void *Y, hipStream_t stream);

}  // namespace avq
