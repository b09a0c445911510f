// Stage 1 of the AVQ-Attention forward pass: full-tree assignment and
// aggregation ("AVQ-Attention", Sec. 4.2).
//
// Every key goes to its nearest parent (Sec. 3.2 argmin), then is compared
// with that parent's C children only and moves to the nearest child if it is
// strictly closer than the parent.  Value sums and counts are accumulated at
// both levels: a parent slot covers its whole cell, a child slot the keys that
// moved to it.
//
// gfx950 design (differs from the single fused pass on the pages, see the
// design notes): the C children of every parent do not fit in LDS for the
// large trees (M0*C*d bf16 = 256 KiB at M0=256, C=8, d=64), and gathering a
// key's 8 children from L2 costs 8x the key's own bytes.  So the work is split
// in two kernels that each keep their codewords on chip:
//   1. assign_parent_kernel: K . parents^T on MFMA with the parents in LDS,
//      argmin per key, then a counting sort of the chunk's keys by parent
//      (workspace: bucketed key list + per-chunk bucket offsets).
//   2. refine_aggregate_kernel: one work-group per group of kRefineGroup
//      parents; their children and the parents sit in LDS, the group's keys
//      are gathered through the bucket lists, child distances come from MFMA,
//      and values are summed into LDS slot accumulators that are written out
//      once (every output slot is written by exactly one work-group, so no
//      global atomics and no pre-zeroing).
// Distances use ||c||^2 - 2 k.c (the ||k||^2 term is common to all
// candidates): the MFMA accumulator starts at ||c||^2 and the LDS copy of the
// codewords holds -2c (exact in bf16 and fp32).
#include "avq_kernels.h"

namespace avq {


size_t assign_workspace_bytes(int B, int H, int N, int M0)
{
    const int64_t nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    size_t a = (size_t)B * H * N * sizeof(int32_t);
    a = (a + 255) & ~(size_t)255;
    size_t b = (size_t)B * H * nchunks * (M0 + 1) * sizeof(int32_t);
    return a + ((b + 255) & ~(size_t)255);
}

AssignWorkspace carve_assign_workspace(void *base, int B, int H, int N, int M0)
{
    AssignWorkspace ws;
    size_t a = (size_t)B * H * N * sizeof(int32_t);
    a = (a + 255) & ~(size_t)255;
    ws.sorted = (int32_t *)base;
    ws.chunk_off = (int32_t *)((char *)base + a);
    ws.bytes = assign_workspace_bytes(B, H, N, M0);
    return ws;
}

// ---------------------------------------------------------------------------
// kernel 1: nearest parent of every key + per-chunk bucketing by parent
// grid (nchunks, B*H), 256 threads; each wave takes 64 keys per step.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void assign_parent_kernel(
    const T *__restrict__ K, const T *__restrict__ parents, const float *__restrict__ sqnorm,
    int H, int N, int M0, int C, int nchunks, int32_t *__restrict__ sorted,
    int32_t *__restrict__ chunk_off)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int LDP = D + 8;
    constexpr int KS = D / 32;
    const int M0p = round16(M0);
    T *Pm2 = reinterpret_cast<T *>(smem);
    float *pn = reinterpret_cast<float *>(smem + (size_t)M0p * LDP * sizeof(T));
    int *pst = reinterpret_cast<int *>(pn + M0p);      // [kAssignChunk]
    int *hist = pst + kAssignChunk;                      // [257]

    const int chunk = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int64_t head = (int64_t)bh * N;
    const int key0 = chunk * kAssignChunk;
    const int S = M0 * (1 + C);

    // stage -2 * parents and the parent norms
    const T *Ph = parents + (int64_t)h * M0 * D;
    for (int e = tid * 8; e < M0p * D; e += 256 * 8) {
        const int r = e / D, c = e % D;
        Frag<T> f = r < M0 ? load_frag(Ph + (int64_t)r * D + c) : zero_frag<T>();
        T *dst = Pm2 + r * LDP + c;
        store_scaled_frag(dst, f, -2.0f);
    }
    for (int r = tid; r < M0p; r += 256) pn[r] = r < M0 ? sqnorm[(int64_t)h * S + r] : INFINITY;
    for (int r = tid; r < 257; r += 256) hist[r] = 0;
    __syncthreads();

    const int nrb = M0p / 16;
    for (int it = 0; it < kAssignChunk / 256; ++it) {
        const int kw = key0 + it * 256 + wave * 64;
        if (kw >= N) break;
        Frag<T> b[4][KS];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            const int key = kw + 16 * kb + i16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                b[kb][ks] = key < N ? load_frag(K + (head + key) * D + 32 * ks + 8 * g) : zero_frag<T>();
        }
        float best[4];
        int bidx[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
            best[kb] = INFINITY;
            bidx[kb] = 0;
        }
        for (int rb = 0; rb < nrb; ++rb) {
            Frag<T> a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a[ks] = load_frag(Pm2 + (16 * rb + i16) * LDP + 32 * ks + 8 * g);
            const f32x4 c0 = *reinterpret_cast<const f32x4 *>(pn + 16 * rb + 4 * g);
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                f32x4 acc = c0;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) acc = mma(a[ks], b[kb][ks], acc);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool lt = acc[r] < best[kb];
                    best[kb] = lt ? acc[r] : best[kb];
                    bidx[kb] = lt ? 16 * rb + 4 * g + r : bidx[kb];
                }
            }
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) xgroup_argmin(best[kb], bidx[kb]);
        if (g == 0) {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
                const int key = kw + 16 * kb + i16;
                if (key < N) pst[key - key0] = bidx[kb];
            }
        }
    }
    __syncthreads();

    // counting sort of the chunk's keys by parent
    const int nk = min(kAssignChunk, N - key0);
    for (int x = tid; x < nk; x += 256) atomicAdd(&hist[pst[x]], 1);
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
    int32_t *co = chunk_off + ((int64_t)bh * nchunks + chunk) * (M0 + 1);
    for (int p = tid; p <= M0; p += 256) co[p] = hist[p];
    __syncthreads();
    for (int x = tid; x < nk; x += 256) {
        const int p = pst[x];
        const int pos = atomicAdd(&hist[p], 1);
        sorted[head + key0 + pos] = (int32_t)((unsigned)(key0 + x) | ((unsigned)p << 24));
    }
}

// ---------------------------------------------------------------------------
// kernel 2: child refinement and aggregation for a group of parents
// grid (ngroups, B*H), 256 threads.
// LDS rows: child (lp, c) at row lp*C + c, parent lp at row G*C + lp; the
// slot accumulators use the same numbering (row G*C + lp = keys that stayed
// at parent lp).
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void refine_aggregate_kernel(
    const T *__restrict__ K, const T *__restrict__ V, const T *__restrict__ parents,
    const T *__restrict__ children, const float *__restrict__ sqnorm, int H, int N, int M0, int C,
    int nchunks, int force_child, const int32_t *__restrict__ sorted,
    const int32_t *__restrict__ chunk_off, float *__restrict__ vsum, int32_t *__restrict__ count,
    int32_t *__restrict__ leaf, unsigned char *__restrict__ pack)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int G = kRefineGroup;
    constexpr int LDP = D + 8;
    constexpr int LDA = D + 1;
    constexpr int KS = D / 32;
    const int NR = G * (C + 1);            // codeword rows == slots
    const int RP = round16(NR);
    T *Cw = reinterpret_cast<T *>(smem);
    float *rn = reinterpret_cast<float *>(smem + (size_t)RP * LDP * sizeof(T));
    float *acc = rn + RP;                  // [NR][LDA]
    int *cnt = reinterpret_cast<int *>(acc + (size_t)NR * LDA);   // [NR]
    int *pre = cnt + NR;                   // [nchunks + 1]
    int *segs = pre + nchunks + 1;         // [nchunks]

    const int p0 = blockIdx.x * G, bh = blockIdx.y, h = bh % H;
    const int Gv = min(G, M0 - p0);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int S = M0 * (1 + C);
    const int64_t head = (int64_t)bh * N;

    // stage -2 * codewords, their norms, zero accumulators
    for (int e = tid * 8; e < RP * D; e += 256 * 8) {
        const int r = e / D, c = e % D;
        const T *src = nullptr;
        if (r < G * C) {
            const int lp = r / C;
            if (lp < Gv) src = children + (((int64_t)h * M0 + p0 + lp) * C + (r % C)) * D + c;
        } else if (r < NR) {
            const int lp = r - G * C;
            if (lp < Gv) src = parents + ((int64_t)h * M0 + p0 + lp) * D + c;
        }
        Frag<T> f = src ? load_frag(src) : zero_frag<T>();
        store_scaled_frag(Cw + r * LDP + c, f, -2.0f);
    }
    for (int r = tid; r < RP; r += 256) {
        float v = INFINITY;
        if (r < G * C) {
            const int lp = r / C;
            if (lp < Gv) v = sqnorm[(int64_t)h * S + M0 + (p0 + lp) * C + (r % C)];
        } else if (r < NR) {
            const int lp = r - G * C;
            if (lp < Gv) v = sqnorm[(int64_t)h * S + p0 + lp];
        }
        rn[r] = v;
    }
    for (int e = tid; e < NR * LDA; e += 256) acc[e] = 0.f;
    for (int e = tid; e < NR; e += 256) cnt[e] = 0;
    // this group's bucket in every chunk
    for (int c = tid; c < nchunks; c += 256) {
        const int32_t *co = chunk_off + ((int64_t)bh * nchunks + c) * (M0 + 1);
        const int a = co[p0], b = co[p0 + Gv];
        pre[c] = b - a;
        segs[c] = c * kAssignChunk + a;
    }
    __syncthreads();
    if (tid == 0) {
        int run = 0;
        for (int c = 0; c < nchunks; ++c) {
            const int l = pre[c];
            pre[c] = run;
            run += l;
        }
        pre[nchunks] = run;
    }
    __syncthreads();
    const int total = pre[nchunks];
    const int nrb = RP / 16;

    for (int blk = wave; blk * 16 < total; blk += 4) {
        const int x = blk * 16 + i16;
        const bool valid = x < total;
        int key = 0, lp = 0;
        if (valid) {
            int lo = 0, hi = nchunks;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (pre[mid] <= x) lo = mid;
                else hi = mid;
            }
            const unsigned e = (unsigned)sorted[head + segs[lo] + (x - pre[lo])];
            key = (int)(e & 0xFFFFFFu);
            lp = (int)(e >> 24) - p0;
        }
        Frag<T> b[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            b[ks] = valid ? load_frag(K + (head + key) * D + 32 * ks + 8 * g) : zero_frag<T>();

        float cbest = INFINITY, pe = INFINITY;
        int crow = lp * C;
        for (int rb = 0; rb < nrb; ++rb) {
            f32x4 a = *reinterpret_cast<const f32x4 *>(rn + 16 * rb + 4 * g);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a = mma(load_frag(Cw + (16 * rb + i16) * LDP + 32 * ks + 8 * g), b[ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * rb + 4 * g + r;
                const bool mine = row >= lp * C && row < lp * C + C;
                const bool lt = mine && a[r] < cbest;
                cbest = lt ? a[r] : cbest;
                crow = lt ? row : crow;
                pe = row == G * C + lp ? a[r] : pe;
            }
        }
        xgroup_argmin(cbest, crow);
        pe = xgroup_min(pe);
        const bool to_child = force_child || cbest < pe;
        const int slot = to_child ? crow : G * C + lp;
        if (valid) {
            if (leaf && g == 0)
                leaf[head + key] = to_child ? M0 + (p0 + lp) * C + (crow - lp * C) : p0 + lp;
            const T *vr = V + (head + key) * D + g * (D / 4);
            float *ar = acc + slot * LDA + g * (D / 4);
#pragma unroll
            for (int t = 0; t < D / 4; t += 8) {
                const Frag<T> f = load_frag(vr + t);
#pragma unroll
                for (int k = 0; k < 8; ++k) atomicAdd(ar + t + k, frag_elem(f, k));
            }
            if (g == 0) atomicAdd(&cnt[slot], 1);
        }
    }
    __syncthreads();

    // children slots as accumulated; parent slot = stayed + all children
    float *vs = vsum + (int64_t)bh * S * D;
    int32_t *cs = count + (int64_t)bh * S;
    for (int e = tid; e < Gv * C * D; e += 256) {
        const int lp = e / (C * D), rem = e % (C * D), c = rem / D, t = rem % D;
        vs[((int64_t)M0 + (p0 + lp) * C + c) * D + t] = acc[(lp * C + c) * LDA + t];
    }
    for (int e = tid; e < Gv * D; e += 256) {
        const int lp = e / D, t = e % D;
        float s = acc[(G * C + lp) * LDA + t];
        for (int c = 0; c < C; ++c) s += acc[(lp * C + c) * LDA + t];
        vs[(int64_t)(p0 + lp) * D + t] = s;
    }
    for (int e = tid; e < Gv * C; e += 256) cs[M0 + (p0 + e / C) * C + e % C] = cnt[e];
    for (int lp = tid; lp < Gv; lp += 256) {
        int s = cnt[G * C + lp];
        for (int c = 0; c < C; ++c) s += cnt[lp * C + c];
        cs[p0 + lp] = s;
    }

    // the same aggregates as stage-2 operands (layout in PackLayout)
    const PackLayout PL = pack_layout(M0, C, D, (int)sizeof(T));
    const int M0p = padded_parents(M0);
    unsigned char *pk = pack + (size_t)bh * PL.bytes;
    T *pvt = reinterpret_cast<T *>(pk + PL.pvt);
    float *pnp = reinterpret_cast<float *>(pk + PL.pn);
    T *cvt = reinterpret_cast<T *>(pk + PL.cvt);
    float *cnp = reinterpret_cast<float *>(pk + PL.cn);
    for (int e = tid; e < Gv * D; e += 256) {
        const int lp = e / D, t = e % D, j = p0 + lp;
        float s = acc[(G * C + lp) * LDA + t];
        for (int c = 0; c < C; ++c) s += acc[(lp * C + c) * LDA + t];
        pvt[(size_t)t * M0p + (j & ~31) + perm32(j & 31)] = from_float<T>(s);
    }
    for (int lp = tid; lp < Gv; lp += 256) {
        int s = cnt[G * C + lp];
        for (int c = 0; c < C; ++c) s += cnt[lp * C + c];
        pnp[p0 + lp] = (float)s;
    }
    for (int e = tid; e < Gv * D * C; e += 256) {
        const int lp = e / (D * C), rem = e % (D * C), t = rem / C, c = rem % C;
        cvt[((size_t)(p0 + lp) * D + t) * C + c] = from_float<T>(acc[(lp * C + c) * LDA + t]);
    }
    for (int e = tid; e < Gv * C; e += 256) cnp[(size_t)p0 * C + e] = (float)cnt[e];
    if (p0 + Gv == M0) {   // padding columns of the parent operands
        for (int e = tid; e < (M0p - M0) * D; e += 256) {
            const int j = M0 + e / D, t = e % D;
            pvt[(size_t)t * M0p + (j & ~31) + perm32(j & 31)] = from_float<T>(0.f);
        }
        for (int j = M0 + tid; j < M0p; j += 256) pnp[j] = 0.f;
    }
}

// ---------------------------------------------------------------------------

template <typename T, int D>
static hipError_t launch_t(const void *K, const void *V, const void *parents, const void *children,
                           const float *sqnorm, int B, int H, int N, int M0, int C, unsigned flags,
                           float *vsum, int32_t *count, int32_t *leaf, void *pack,
                           const AssignWorkspace &ws, hipStream_t stream)
{
    const int nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    const int M0p = round16(M0);
    const size_t lds1 = (size_t)M0p * (D + 8) * sizeof(T) + (size_t)M0p * 4 + kAssignChunk * 4 + 257 * 4;
    static bool attr1 = false;
    if (!attr1) {
        (void)hipFuncSetAttribute((const void *)assign_parent_kernel<T, D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr1 = true;
    }
    hipLaunchKernelGGL((assign_parent_kernel<T, D>), dim3(nchunks, B * H), dim3(256), lds1, stream,
                       (const T *)K, (const T *)parents, sqnorm, H, N, M0, C, nchunks, ws.sorted,
                       ws.chunk_off);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;

    const int G = kRefineGroup;
    const int NR = G * (C + 1), RP = round16(NR);
    const size_t lds2 = (size_t)RP * (D + 8) * sizeof(T) + (size_t)RP * 4 + (size_t)NR * (D + 1) * 4 +
                        (size_t)NR * 4 + (size_t)(2 * nchunks + 1) * 4;
    static bool attr2 = false;
    if (!attr2) {
        (void)hipFuncSetAttribute((const void *)refine_aggregate_kernel<T, D>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr2 = true;
    }
    const int ngroups = (M0 + G - 1) / G;
    hipLaunchKernelGGL((refine_aggregate_kernel<T, D>), dim3(ngroups, B * H), dim3(256), lds2, stream,
                       (const T *)K, (const T *)V, (const T *)parents, (const T *)children, sqnorm, H,
                       N, M0, C, nchunks, (flags & 1u) ? 1 : 0, ws.sorted, ws.chunk_off, vsum, count,
                       leaf, (unsigned char *)pack);
    return hipGetLastError();
}

hipError_t launch_assign_aggregate(const void *K, const void *V, const void *parents,
                                   const void *children, const float *sqnorm, int B, int H, int N,
                                   int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                   int32_t *count, int32_t *leaf, void *pack,
                                   const AssignWorkspace &ws, hipStream_t stream)
{
    if (dtype == 1) {
        if (d == 64)
            return launch_t<bf16, 64>(K, V, parents, children, sqnorm, B, H, N, M0, C, flags, vsum, count, leaf, pack, ws, stream);
        return launch_t<bf16, 128>(K, V, parents, children, sqnorm, B, H, N, M0, C, flags, vsum, count, leaf, pack, ws, stream);
    }
    if (d == 64)
        return launch_t<float, 64>(K, V, parents, children, sqnorm, B, H, N, M0, C, flags, vsum, count, leaf, pack, ws, stream);
    return launch_t<float, 128>(K, V, parents, children, sqnorm, B, H, N, M0, C, flags, vsum, count, leaf, pack, ws, stream);
}

}  // namespace avq
