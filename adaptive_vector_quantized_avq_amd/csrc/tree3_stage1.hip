// Stage 1 for a three-level tree (roots -> children -> leaves), the deeper
// hierarchy "AVQ-Attention" proposes as its next step (Sec. 6): each key
// descends one level at a time, as the two-level rule of Sec. 4.2 does once
// -- nearest root, then that root's C children (taken only if strictly
// closer than the root), then that child's C leaves (taken only if strictly
// closer than the child) -- and every slot accumulates its whole cell.
//
// The two descents are the two-level kernels run twice:
//   1. assign_parent + refine_aggregate over (roots, children): every key's
//      root and child-or-root, the roots' whole cells and the children's
//      (every key that reached a child lies in that child's cell);
//   2. bucket_children_kernel lists, per chunk of keys, the keys that
//      reached a child by groups of children (stable, in key order), and
//      refine_aggregate runs again with the children as parents and the
//      leaves as their children, on the slot arrays offset to the children:
//      it writes the children's cells again (the same keys) and the leaves'.
// Slot layout per (b, h): [0, M0) roots, [M0, M0 + M0*C) children p*C + a,
// then leaves (p*C + a)*C + b.
#include "avq_kernels.h"

namespace avq {

// Stable counting sort of one chunk's keys by group of children.  Four
// waves per (chunk, b*h), each over a quarter of the chunk's keys in key
// order; keys that stayed at their root are left out.  A list entry is
// key | (child mod 256) << 24, the form the refinement kernel reads (it
// needs the child only relative to its group's first child).  A key's
// position: its group's start, plus that group's keys in earlier waves,
// plus those earlier in its own wave (same-group lanes matched with one
// ballot per bit of the group index).
constexpr int kBucketWaves = 4;
__global__ __launch_bounds__(64 * kBucketWaves) void bucket_children_kernel(
    const int32_t *__restrict__ leaf, int N, int M0, int C, int group, int ngroups, int nbits, int nchunks,
    int32_t *__restrict__ sorted, int2 *__restrict__ seg, int32_t *__restrict__ cmax)
{
    extern __shared__ int wcnt[];   // [kBucketWaves][ngroups] counts, then running positions; [ngroups] starts
    int *start = wcnt + kBucketWaves * ngroups;
    const int chunk = blockIdx.x, bh = blockIdx.y;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t head = (int64_t)bh * N;
    const int key0 = chunk * kAssignChunk, nk = min(kAssignChunk, N - key0);
    const int n1 = M0 * C;
    constexpr int KPW = kAssignChunk / kBucketWaves;   // keys per wave
    for (int g = tid; g < kBucketWaves * ngroups; g += 64 * kBucketWaves) wcnt[g] = 0;
    __syncthreads();

    // child reached by key x of the chunk, -1 for a key that stayed at its root
    auto child_of = [&](int x) -> int {
        if (x >= nk) return -1;
        const int l = leaf[head + key0 + x];
        return l < M0 ? -1 : l < M0 + n1 ? l - M0 : (l - M0 - n1) / C;
    };
    // lanes holding a listed key of the same group (one ballot per bit)
    auto same_group = [&](bool v, int gi) {
        unsigned long long m = __ballot(v);
        for (int bit = 0; bit < nbits; ++bit) {
            const bool set = (gi >> bit) & 1;
            const unsigned long long b = __ballot(set);
            m &= set ? b : ~b;
        }
        return m;
    };
    int *mine = wcnt + wave * ngroups;
    for (int r = 0; r < KPW / 64; ++r) {   // this wave's counts per group
        const int c = child_of(wave * KPW + 64 * r + lane);
        const bool v = c >= 0;
        const int gi = v ? c / group : 0;
        const unsigned long long m = same_group(v, gi);
        if (v && mbcnt(m) == 0) mine[gi] += __popcll(m);   // one lane per group
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    __syncthreads();
    for (int g = tid; g < ngroups; g += 64 * kBucketWaves) {   // earlier waves' counts, and totals
        int run = 0;
#pragma unroll
        for (int w = 0; w < kBucketWaves; ++w) {
            const int c = wcnt[w * ngroups + g];
            wcnt[w * ngroups + g] = run;
            run += c;
        }
        start[g] = run;
    }
    __syncthreads();
    if (wave == 0) {   // exclusive scan over the groups -> the chunk's segment table
        int carry = 0, most = 0;
        for (int base = 0; base < ngroups; base += 64) {
            const int g = base + lane;
            const int v = g < ngroups ? start[g] : 0;
            most = max(most, v);
            int inc = v;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(inc, off);
                if (lane >= off) inc += t;
            }
            if (g < ngroups) {
                const int st = carry + inc - v;
                seg[((int64_t)bh * ngroups + g) * nchunks + chunk] = make_int2(st, v);
                start[g] = st;
            }
            carry += __shfl(inc, 63);
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) most = max(most, __shfl_xor(most, off));
        if (lane < 2) cmax[((int64_t)bh * nchunks + chunk) * 2 + lane] = lane == 0 ? most : 0;
    }
    __syncthreads();
    for (int r = 0; r < KPW / 64; ++r) {   // stable scatter, this wave's keys in key order
        const int x = wave * KPW + 64 * r + lane;
        const int c = child_of(x);
        const bool v = c >= 0;
        const int gi = v ? c / group : 0;
        const unsigned long long m = same_group(v, gi);
        const int before = mbcnt(m);
        if (v) sorted[head + key0 + start[gi] + mine[gi] + before] = (key0 + x) | (int)(((unsigned)c & 0xFFu) << 24);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (v && before == 0) mine[gi] += __popcll(m);
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// the lists, the segment table of the larger (second) descent and, when the
// caller keeps no leaf ids, room for them
size_t assign3_workspace_bytes(int B, int H, int N, int M0, int C, int D)
{
    return assign_workspace_bytes(B, H, N, M0 * C, C, D) + align256((size_t)B * H * N * sizeof(int32_t));
}

hipError_t launch_assign_aggregate3(const void *K, const void *V, const void *level0, const void *level1,
                                    const void *leaves, const float *sqnorm, const float *frame, int B, int H,
                                    int N, int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                    int32_t *count, int32_t *leaf, void *workspace, hipStream_t stream)
{
    const AssignWorkspace ws = carve_assign_workspace(workspace, B, H, N, M0 * C, C, d);
    int32_t *lf = leaf ? leaf : (int32_t *)((char *)workspace + assign_workspace_bytes(B, H, N, M0 * C, C, d));
    const int S3 = M0 * (1 + C + C * C);
    // 1. roots -> children
    hipError_t err = launch_assign_parent(K, level0, sqnorm, frame, B, H, N, d, M0, C, dtype, ws, nullptr, stream);
    if (err != hipSuccess) return err;
    err = launch_refine_slots(K, V, level0, level1, sqnorm, frame, B, H, N, d, M0, C, dtype, flags, vsum, count, lf,
                              ws, S3, 0, stream);
    if (err != hipSuccess) return err;
    // 2. children -> leaves, for the keys that reached a child
    const int group = refine_group(C, d);
    const int n1 = M0 * C;
    const int ngroups = (n1 + group - 1) / group;
    int nbits = 1;
    while ((1 << nbits) < ngroups) ++nbits;
    const int nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    hipLaunchKernelGGL(bucket_children_kernel, dim3(nchunks, B * H), dim3(64 * kBucketWaves),
                       (size_t)(kBucketWaves + 1) * ngroups * sizeof(int), stream,
                       (const int32_t *)lf, N, M0, C, group, ngroups, nbits, nchunks, ws.sorted, ws.seg, ws.cmax);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_refine_slots(K, V, level1, leaves, sqnorm + M0, frame, B, H, N, d, n1, C, dtype, flags,
                               vsum + (size_t)M0 * d, count + M0, lf, ws, S3, M0, stream);
}

}  // namespace avq
