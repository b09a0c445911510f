// Stage 1, first kernel: nearest parent of every key ("AVQ-Attention",
// Sec. 4.2; the argmin of Sec. 3.2), and a counting sort of each chunk's keys
// by parent so that the second kernel (refine_aggregate.hip) can visit the
// keys of a group of parents; each group's segment of every chunk's list is
// recorded group-major, so that the second kernel reads its table in one
// contiguous piece.
//
// Distances use ||c||^2 - 2 k.c (the ||k||^2 term is common to all
// candidates): the MFMA accumulator starts at ||c||^2 and the LDS copy of the
// parents holds -2c (exact in bf16 and fp32).  Keys and parents are first
// moved into the frame of the head's reference point r (avq_build_tree; r =
// 0 for a centred codebook, see avq_device.h), so that the rounding error
// scales with the codebook's spread, not its offset; the norms passed in are
// ||c - r||^2.  Candidates are compared on 22
// of fp32's 24 significand bits; ties go to the lowest row block, and inside
// a lane's group of four rows to the lower row when the compared value is
// non-negative and to the higher one when it is negative (it is ||c||^2 -
// 2 k.c, not the full distance).  Such ties lie far below the comparison
// protocol's near-tie bound, under which either parent is accepted.
#include <float.h>

#include "avq_kernels.h"

namespace avq {

// workspace regions: key lists, segment tables, split groups' partial sums
// and their flags (each 256-byte aligned)
static void assign_regions(int B, int H, int N, int M0, int C, int D, size_t (&sz)[5])
{
    const int64_t nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    const int group = refine_group(C, D);
    const int64_t ngroups = (M0 + group - 1) / group;
    const size_t bh = (size_t)B * H;
    const RefinePlan pl = refine_plan(N, M0, C, D);
    sz[0] = align256(bh * N * sizeof(int32_t));
    sz[1] = align256(bh * ngroups * nchunks * sizeof(int2));
    sz[2] = align256(bh * nchunks * 2 * sizeof(int32_t));
    sz[3] = align256(bh * pl.max_partials * refine_partial_words(C, D) * sizeof(float));
    sz[4] = align256(bh * pl.max_partials * sizeof(unsigned));
}

size_t assign_workspace_bytes(int B, int H, int N, int M0, int C, int D)
{
    size_t sz[5];
    assign_regions(B, H, N, M0, C, D, sz);
    return sz[0] + sz[1] + sz[2] + sz[3] + sz[4];
}

AssignWorkspace carve_assign_workspace(void *base, int B, int H, int N, int M0, int C, int D)
{
    size_t sz[5];
    assign_regions(B, H, N, M0, C, D, sz);
    AssignWorkspace ws;
    char *p = (char *)base;
    ws.sorted = (int32_t *)p;
    p += sz[0];
    ws.seg = (int2 *)p;
    p += sz[1];
    ws.cmax = (int32_t *)p;
    p += sz[2];
    ws.partial = (float *)p;
    p += sz[3];
    ws.pflag = (unsigned *)p;
    ws.bytes = sz[0] + sz[1] + sz[2] + sz[3] + sz[4];
    return ws;
}

unsigned next_call_tag()
{
    static std::atomic<unsigned> counter{0x9E3779B9u};
    unsigned t;
    do t = counter.fetch_add(1u, std::memory_order_relaxed) + 1u;
    while (t == 0u);
    return t;
}

// ---------------------------------------------------------------------------
// kernel 1: nearest parent of every key + per-chunk bucketing by parent
// grid (nchunks, B*H), kAssignThreads threads (8 waves, two work-groups per
// CU, four waves per SIMD).  Each wave takes 16*KB keys per step; the next
// step's keys are loaded as soon as the last distance MFMAs have read the
// current ones.  NRB = parents padded to a
// power of two >= 16, in 16-row MFMA blocks (padding rows never win: their
// norm is FLT_MAX).
//
// The row-block loop is software pipelined: the MFMAs of block rb+1 are
// issued before the argmin update of block rb, whose operands were loaded
// from LDS one block earlier still, so the matrix cores, the VALU and LDS
// work on three different blocks at a time.
// ---------------------------------------------------------------------------
constexpr int kAssignThreads = 512;

template <typename T, int D> constexpr int assign_key_blocks()
{
    return (sizeof(T) == 2 && D == 64) ? 4 : 2;   // bounded by the key registers
}
// waves per SIMD the register budget is sized for (fp32 with d = 128 needs
// more than 128 registers for its key and codeword fragments)
template <typename T, int D> constexpr int assign_waves_per_simd()
{
    return (sizeof(T) == 4 && D == 128) ? 2 : 4;
}

template <typename T, int D, int NRB>
__global__ __launch_bounds__(kAssignThreads) __attribute__((amdgpu_waves_per_eu(assign_waves_per_simd<T, D>()))) void assign_parent_kernel(
    const T *__restrict__ K, const T *__restrict__ parents, const float *__restrict__ sqnorm,
    const float *__restrict__ frame, int H, int N, int M0, int C, int nchunks, int32_t *__restrict__ sorted,
    int2 *__restrict__ seg, int32_t *__restrict__ leaf_direct, int32_t *__restrict__ cmax)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int NT = kAssignThreads;
    constexpr int NWV = NT / 64;
    constexpr int LDP = D + 8;
    constexpr int KS = D / 32;
    constexpr int KB = assign_key_blocks<T, D>();
    constexpr int KEYS = 16 * KB;                        // keys per wave per step
    constexpr int M0p = 16 * NRB;
    constexpr int kIters = kAssignChunk / (NWV * KEYS);
    static_assert(kAssignChunk % (NWV * KEYS) == 0, "chunk must be a whole number of steps");
    T *Pm2 = reinterpret_cast<T *>(smem);
    float *pn = reinterpret_cast<float *>(smem + (size_t)M0p * LDP * sizeof(T));
    float *rv = pn + M0p;                                              // [D] frame reference (16-B aligned)
    unsigned char *pst = reinterpret_cast<unsigned char *>(rv + D);    // [kAssignChunk]
    int *hist = reinterpret_cast<int *>(pst + kAssignChunk);           // [257]
    int *wcnt = hist + 257;                                            // [NWV][256]

    const int chunk = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int64_t head = (int64_t)bh * N;
    const int key0 = chunk * kAssignChunk;
    const int S = M0 * (1 + C);

    auto load_keys = [&](int it, Frag<T> (&b)[KB][KS]) {
        const int kw = key0 + (it * NWV + wave) * KEYS;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            // keys past the end read the last key (their result is never stored);
            // the loads stay unconditional so that they can be left in flight
            const int key = min(kw + 16 * kb + i16, N - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) b[kb][ks] = load_frag(K + (head + key) * D + 32 * ks + 8 * g);
        }
    };
    Frag<T> b[KB][KS];
    load_keys(0, b);   // in flight while the parents are staged

    // stage -2 (parent - r) and the parent norms in the frame (all loads
    // issued before the first store; rows past M0 read the last parent and
    // store zeros)
    const T *Ph = parents + (int64_t)h * M0 * D;
    const float *fr = frame + (int64_t)h * D;
    constexpr int kStage = (M0p * D + NT * 8 - 1) / (NT * 8);
    Frag<T> sf[kStage];
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
        const int e = (tid + NT * k) * 8, r = min(e / D, M0 - 1), c = e % D;
        sf[k] = load_frag(Ph + (int64_t)r * D + c);
    }
    float snorm = sqnorm[(int64_t)h * S + min(tid, M0 - 1)];
    // the frame is all zero for a centred codebook: keys are then used as
    // they are (the same value in every wave)
    const float rl = fr[lane % D], rh = fr[(lane + 64) % D];
    const bool shift = __ballot(rl != 0.f || rh != 0.f) != 0ull;
    if (tid < D) rv[tid] = fr[tid];
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
        const int e = (tid + NT * k) * 8, r = e / D, c = e % D;
        if (e < M0p * D) {
            const f32x4 r0 = *reinterpret_cast<const f32x4 *>(fr + c);
            const f32x4 r1 = *reinterpret_cast<const f32x4 *>(fr + c + 4);
            store_frag(Pm2 + r * LDP + c, r < M0 ? frame_m2(sf[k], r0, r1) : zero_frag<T>());
        }
    }
    if (tid < M0p) pn[tid] = tid < M0 ? snorm : FLT_MAX;   // padding rows never win
    for (int r = tid; r < 257; r += NT) hist[r] = 0;
    for (int r = tid; r < NWV * 256; r += NT) wcnt[r] = 0;
    __syncthreads();

    // codeword fragments and norms of row block rb
    auto load_rows = [&](int rb, Frag<T> (&a)[KS], f32x4 &c0) {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) a[ks] = load_frag(Pm2 + (16 * rb + i16) * LDP + 32 * ks + 8 * g);
        c0 = *reinterpret_cast<const f32x4 *>(pn + 16 * rb + 4 * g);
    };

#pragma unroll 1
    for (int it = 0; it < kIters; ++it) {
        const int kw = key0 + (it * NWV + wave) * KEYS;
        if (kw >= N) break;
        // Running minimum per key column.  The row inside the lane's group of
        // four travels in the two lowest mantissa bits of the compared value
        // (the comparison keeps 22 of fp32's 24 significand bits), so the
        // four rows of an MFMA tile reduce with two v_min3 and the block
        // index is the only thing tracked by a select.
        float best[KB];
        int brb[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            best[kb] = FLT_MAX;
            brb[kb] = 0;
        }
        Frag<T> a[2][KS];
        f32x4 c0[2], acc[2][KB];
        // distances of row block s into acc[s & 1] (operands in buffer s & 1)
        auto issue = [&](int buf) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4 t = c0[buf];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) t = mma(a[buf][ks], b[kb][ks], t);
                acc[buf][kb] = t;
            }
        };
        auto consume = [&](int rb, int buf) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const f32x4 v = acc[buf][kb];
                float q[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) q[r] = __uint_as_float((__float_as_uint(v[r]) & ~3u) | (unsigned)r);
                const float m = min3f(min3f(q[0], q[1], q[2]), q[3], best[kb]);
                brb[kb] = m < best[kb] ? rb : brb[kb];
                best[kb] = m;
            }
        };
        const bool more = it + 1 < kIters;
        if (shift) {   // keys into the distance frame
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) b[kb][ks] = shift_frag(b[kb][ks], rv, 32 * ks + 8 * g);
        }
        load_rows(0, a[0], c0[0]);
        if constexpr (NRB == 1) {
            issue(0);
            // the distance MFMAs have read the keys: load the next step's keys
            // into the same registers while the last blocks are reduced
            if (more) load_keys(it + 1, b);
            consume(0, 0);
        } else {
            load_rows(1, a[1], c0[1]);
            issue(0);
            // pairs of row blocks (even block in buffer 0, odd in buffer 1);
            // at block rb the MFMAs of rb+1 are issued and the operands of
            // rb+2 are read before rb is reduced
#pragma unroll 1
            for (int rp = 0; rp < NRB - 2; rp += 2) {
                issue(1);
                load_rows(rp + 2, a[0], c0[0]);
                consume(rp, 0);
                issue(0);
                load_rows(rp + 3, a[1], c0[1]);
                consume(rp + 1, 1);
            }
            issue(1);
            if (more) load_keys(it + 1, b);   // (see above)
            consume(NRB - 2, 0);
            consume(NRB - 1, 1);
        }
        int bidx[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            bidx[kb] = 16 * brb[kb] + 4 * g + (int)(__float_as_uint(best[kb]) & 3u);
            xgroup_argmin(best[kb], bidx[kb]);
        }
        if (g == 0) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                const int key = kw + 16 * kb + i16;
                if (key < N) pst[key - key0] = (unsigned char)bidx[kb];
            }
        }
    }
    __syncthreads();
    const int nk = min(kAssignChunk, N - key0);
    if (leaf_direct) {   // unfused stage 1: each key's parent, no bucketing
        for (int x = tid; x < nk; x += NT) leaf_direct[head + key0 + x] = pst[x];
        return;
    }

    // Stable counting sort of the chunk's keys by parent, so that a bucket
    // lists its keys in key order and the sums the second kernel forms over
    // it come out the same in every run.  Wave w owns keys [w*KPW, (w+1)*KPW);
    // a key's position is its parent's bucket start, plus that parent's keys
    // in earlier waves, plus those earlier in its own wave (same-parent lanes
    // are matched with one ballot per bit of the parent index).
    constexpr int KPW = kAssignChunk / NWV;
    static_assert(KPW % 64 == 0, "a wave's keys must be whole rounds of 64");
    auto same_parent = [&](bool v, int p) {   // lanes holding a key of parent p
        unsigned long long m = __ballot(v);
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool set = (p >> bit) & 1;
            const unsigned long long b = __ballot(set);
            m &= set ? b : ~b;
        }
        return m;
    };
    constexpr int NRD = KPW / 64;
    int *mycnt = wcnt + wave * 256;
    int kp[NRD];
    unsigned long long km[NRD];
#pragma unroll
    for (int r = 0; r < NRD; ++r) {   // this wave's count of every parent
        const int x = wave * KPW + 64 * r + lane;
        const bool v = x < nk;
        kp[r] = v ? pst[x] : 0;
        km[r] = same_parent(v, kp[r]);
        if (v && mbcnt(km[r]) == 0) mycnt[kp[r]] += __popcll(km[r]);   // one lane per parent
    }
    __syncthreads();
    for (int p = tid; p < 256; p += NT) {   // earlier waves' counts, and totals
        int run = 0;
#pragma unroll
        for (int w = 0; w < NWV; ++w) {
            const int c = wcnt[w * 256 + p];
            wcnt[w * 256 + p] = run;
            run += c;
        }
        hist[p] = run;
    }
    __syncthreads();
    if (wave == 0) {
        int v[4], s = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v[k] = hist[4 * lane + k];
            s += v[k];
        }
        int inc = s;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const int t = __shfl_up(inc, off);
            if (lane >= off) inc += t;
        }
        int run = inc - s;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            hist[4 * lane + k] = run;
            run += v[k];
        }
        if (lane == 63) hist[256] = nk;
    }
    __syncthreads();
    // each refinement group's segment of this chunk's list (hist[p] for
    // p >= M0 equals nk: those parents have no keys)
    const int group = refine_group(C, D);
    const int ngroups = (M0 + group - 1) / group;
    int most = 0;   // the largest group of this chunk (groups < 128: waves 0 and 1)
    for (int gr = tid; gr < ngroups; gr += NT) {
        const int a = hist[gr * group], b = hist[min((gr + 1) * group, M0)];
        seg[((int64_t)bh * ngroups + gr) * nchunks + chunk] = int2{a, b - a};
        most = max(most, b - a);
    }
    if (wave < 2) {
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) most = max(most, __shfl_xor(most, off));
        if (lane == 0) cmax[((int64_t)bh * nchunks + chunk) * 2 + wave] = most;
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < NRD; ++r) {
        const int x = wave * KPW + 64 * r + lane;
        const int p = kp[r];
        const int before = mbcnt(km[r]);
        const int pos = hist[p] + mycnt[p] + before;
        // (every lane has read mycnt[p] before one lane per parent advances it:
        // a wave's LDS accesses complete in order)
        if (x < nk) {
            if (before == 0) mycnt[p] += __popcll(km[r]);
            sorted[head + key0 + pos] = (int32_t)((unsigned)(key0 + x) | ((unsigned)p << 24));
        }
    }
}

template <typename T, int D, int NRB>
static hipError_t launch_assign(const void *K, const void *parents, const float *sqnorm, const float *frame,
                                int B, int H, int N, int M0, int C, const AssignWorkspace &ws, int32_t *leaf_direct,
                                hipStream_t stream)
{
    const int nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    const size_t lds = (size_t)16 * NRB * (D + 8) * sizeof(T) + (size_t)16 * NRB * 4 +
                       kAssignChunk + 257 * 4 + (kAssignThreads / 64) * 256 * 4 + D * 4;
    allow_full_lds<assign_parent_kernel<T, D, NRB>>();
    hipLaunchKernelGGL((assign_parent_kernel<T, D, NRB>), dim3(nchunks, B * H), dim3(kAssignThreads), lds, stream,
                       (const T *)K, (const T *)parents, sqnorm, frame, H, N, M0, C, nchunks, ws.sorted,
                       ws.seg, leaf_direct, ws.cmax);
    return hipGetLastError();
}


template <typename T, int D>
static hipError_t launch_parent_t(const void *K, const void *parents, const float *sqnorm, const float *frame,
                                  int B, int H, int N, int M0, int C, const AssignWorkspace &ws,
                                  int32_t *leaf_direct, hipStream_t stream)
{
    const int m = round16(M0);
    if (m <= 16) return launch_assign<T, D, 1>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    if (m <= 32) return launch_assign<T, D, 2>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    if (m <= 64) return launch_assign<T, D, 4>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    if (m <= 128) return launch_assign<T, D, 8>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    return launch_assign<T, D, 16>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
}

hipError_t launch_assign_parent(const void *K, const void *parents, const float *sqnorm, const float *frame,
                                int B, int H, int N, int d, int M0, int C, int dtype,
                                const AssignWorkspace &ws, int32_t *leaf_direct, hipStream_t stream)
{
    if (dtype == 1) {
        if (d == 64) return launch_parent_t<bf16, 64>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
        return launch_parent_t<bf16, 128>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    }
    if (d == 64) return launch_parent_t<float, 64>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
    return launch_parent_t<float, 128>(K, parents, sqnorm, frame, B, H, N, M0, C, ws, leaf_direct, stream);
}

}  // namespace avq
