// Stage 1, second kernel: child refinement and aggregation ("AVQ-Attention",
// Sec. 4.2).  Each key, already assigned to its nearest parent by
// assign_parent.hip, is compared with that parent's C children only and moves
// to the nearest child (ties -> lowest index) if that child is strictly closer
// than the parent.  Value sums and counts are accumulated at both levels: a
// parent slot covers its whole cell, a child slot the keys that moved to it.
// Work is split by group of parents: a group whose key list is longer than a
// target (twice the mean, at least 1024 keys) is cut into equal slices of
// its list, one work-group each, so that a skewed key distribution (a few
// parents holding most keys) does not leave one work-group with most of the
// work.  A group of one slice writes its output slots itself; for a split
// group, every slice but the last stores its partial sums and the last one
// adds them in slice order to its own and writes the slots, so the result
// does not depend on timing (no float atomics, no pre-zeroing).
#include "avq_kernels.h"

namespace avq {

// ---------------------------------------------------------------------------
// child refinement and aggregation for a group of G parents
// grid (ngroups, B*H), kRefineThreads threads.
//
// Distances: the codeword rows of parent lp occupy a block of BR = 16 or 32
// rows (row j < CC: child j, row CC: the parent itself, the rest padding with
// norm +inf); one MFMA pass covers the G blocks and each key keeps only the
// rows of its own parent's block.  Keys and codewords are compared in the
// frame of the head's reference point r (avq_build_tree; r = 0 for a
// centred codebook, see avq_device.h); the norms passed in are ||c - r||^2.
//
// Aggregation is a product on the matrix cores: for a chunk of 32 keys,
//   sums[slot][dim] += onehot[slot][key] * V[key][dim],  counts likewise with
// a column of ones, accumulated in fp32 registers per wave (slot = lp*(CC+1)
// + j with j = child index, or CC for a key that stayed at its parent).  The
// one-hot matrix and V are exact in the input type, so every product is exact
// and only the fp32 summation order differs from a sequential sum.  V rows
// arrive as 16-byte fragments (8 consecutive dims of one key per lane) and
// are transposed through a per-wave LDS tile into the operand layout (8
// consecutive keys of one dim per lane).  (LDS float atomics are avoided:
// measured on gfx950, a 64-lane ds_add_f32 costs ~80 ns per CU, about 70x a
// plain LDS read-modify-write.)
//
// A wave takes KEYS = 16*KB consecutive list positions per step; list entries
// are looked up two steps ahead, and the next step's K and V fragments are
// loaded into the registers of the current ones as soon as these are consumed.
// ---------------------------------------------------------------------------
constexpr int kRefineThreads = 256;

template <typename T, int D, int CC> struct RefineCfg {
    static constexpr int G = refine_group(CC, D);
    static constexpr int NW = kRefineThreads / 64;
    static constexpr int BR = CC + 1 <= 16 ? 16 : 32;          // rows per parent block
    static constexpr int BRB = BR / 16;
    static constexpr int NRB = G * BRB;                        // distance row blocks
    static constexpr int NR = G * (CC + 1);                    // slots
    static constexpr int NSB = (NR + 15) / 16;                 // slot blocks
    static constexpr int NDB = D / 16;                         // dim blocks
    static constexpr int KS = D / 32;
    static constexpr int KB = (sizeof(T) == 2 && D == 64) ? 4 : 2;
    static constexpr int KEYS = 16 * KB;
    static constexpr int NCH = KEYS / 32;
    static constexpr int LDP = D + 8;                          // codeword row stride
    static constexpr int LDK = KEYS + 16 / (int)sizeof(T) * 2; // transposed-V row stride
    static constexpr int LDA = D + 1;                          // accumulator row stride
    static constexpr size_t cw_bytes = (size_t)G * BR * LDP * sizeof(T);
    static constexpr size_t rn_bytes = (size_t)G * BR * 4 + (size_t)D * 4;   // norms, frame reference
    static constexpr size_t vt_bytes = (size_t)NW * (D * LDK * sizeof(T) + KEYS);
    static constexpr size_t acc1_bytes = (size_t)NSB * 16 * (LDA + 1) * 4;
    // partial-sum slices in LDS (they share the region of the V tiles): one
    // per wave, summed in parallel, when that costs no LDS beyond the V tiles
    // or still leaves room for two work-groups per CU; else two (pairs of
    // waves take turns); else one (the waves take turns)
    static constexpr bool slices_fit(int n)
    {
        return (size_t)n * acc1_bytes <= vt_bytes ||
               cw_bytes + rn_bytes + (size_t)n * acc1_bytes <= 76 * 1024;
    }
    static constexpr int NSL = slices_fit(NW) ? NW : slices_fit(2) ? 2 : 1;
    static constexpr size_t acc_bytes = NSL * acc1_bytes;
    static constexpr size_t union_bytes = vt_bytes > acc_bytes ? vt_bytes : acc_bytes;
    static size_t lds(int nchunks)
    {
        return cw_bytes + rn_bytes + ((union_bytes + 15) & ~(size_t)15) + (size_t)(2 * nchunks + 1) * 4;
    }
};

// one-hot MFMA operand: element k is 1 if slot byte k of `sl` equals `target`
template <typename T> __device__ __forceinline__ Frag<T> onehot_frag(unsigned long long sl, int target);
template <> __device__ __forceinline__ Frag<bf16> onehot_frag<bf16>(unsigned long long sl, int target)
{
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    u32x4 u;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const unsigned b0 = (unsigned)(sl >> (16 * w)) & 0xFFu, b1 = (unsigned)(sl >> (16 * w + 8)) & 0xFFu;
        u[w] = ((unsigned)(b0 == (unsigned)target) * 0x3F80u) | ((unsigned)(b1 == (unsigned)target) * 0x3F800000u);
    }
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, u);
    return f;
}
template <> __device__ __forceinline__ Frag<float> onehot_frag<float>(unsigned long long sl, int target)
{
    Frag<float> f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        f.lo[k] = ((unsigned)(sl >> (8 * k)) & 0xFFu) == (unsigned)target ? 1.f : 0.f;
        f.hi[k] = ((unsigned)(sl >> (8 * k + 32)) & 0xFFu) == (unsigned)target ? 1.f : 0.f;
    }
    return f;
}
template <typename T> __device__ __forceinline__ Frag<T> ones_frag();
template <> __device__ __forceinline__ Frag<bf16> ones_frag<bf16>()
{
    Frag<bf16> f;
#pragma unroll
    for (int k = 0; k < 8; ++k) f.v[k] = (bf16)1.0f;
    return f;
}
template <> __device__ __forceinline__ Frag<float> ones_frag<float>()
{
    Frag<float> f;
    f.lo = f32x4{1.f, 1.f, 1.f, 1.f};
    f.hi = f.lo;
    return f;
}
__device__ __forceinline__ void store_elem(bf16 *p, float x) { *p = (bf16)x; }
__device__ __forceinline__ void store_elem(float *p, float x) { *p = x; }

// waves per SIMD the register allocation is held to (1: no limit beyond the
// hardware's).  bf16 at d = 128 with C >= 8 lands a few registers past two
// waves without it.
template <typename T, int D, int CC> constexpr int refine_waves_per_simd()
{
    return sizeof(T) == 2 && D == 128 && CC >= 8 ? 2 : 1;
}

template <typename T, int D, int CC>
__global__ __launch_bounds__(kRefineThreads) __attribute__((amdgpu_waves_per_eu(refine_waves_per_simd<T, D, CC>())))
void refine_aggregate_kernel(
    const T *__restrict__ K, const T *__restrict__ V, const T *__restrict__ parents,
    const T *__restrict__ children, const float *__restrict__ sqnorm, const float *__restrict__ frame,
    int H, int N, int M0,
    int nchunks, int force_child, const int32_t *__restrict__ sorted,
    const int2 *__restrict__ seg, float *__restrict__ vsum, int32_t *__restrict__ count,
    int32_t *__restrict__ leaf, int slot_stride, int leaf_base, int ngroups, int target, int quiet, int npmax,
    unsigned tag, const int32_t *__restrict__ cmax, float *__restrict__ partial,
    unsigned *__restrict__ pflag)
{
    using Cfg = RefineCfg<T, D, CC>;
    constexpr int G = Cfg::G, NW = Cfg::NW, BR = Cfg::BR, BRB = Cfg::BRB, NRB = Cfg::NRB;
    constexpr int NSB = Cfg::NSB, NDB = Cfg::NDB, KS = Cfg::KS, KB = Cfg::KB;
    constexpr int KEYS = Cfg::KEYS, NCH = Cfg::NCH, LDP = Cfg::LDP, LDK = Cfg::LDK, LDA = Cfg::LDA;
    constexpr int NT = kRefineThreads;
    extern __shared__ __align__(16) unsigned char smem[];
    T *Cw = reinterpret_cast<T *>(smem);                                   // [G*BR][LDP]
    float *rn = reinterpret_cast<float *>(smem + Cfg::cw_bytes);           // [G*BR]
    float *rv = rn + G * BR;                                               // [D] frame reference
    unsigned char *un = smem + Cfg::cw_bytes + Cfg::rn_bytes;              // union region
    int *pre = reinterpret_cast<int *>(un + ((Cfg::union_bytes + 15) & ~(size_t)15));   // [nchunks+1]
    int *segs = pre + nchunks + 1;                                         // [nchunks]

    const int bh = blockIdx.x, item = blockIdx.y, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;

    // ---- this work-group's item.  The per-chunk largest group counts bound
    // every group's total: when their sum stays within `quiet`, no group is
    // split and item g is simply group g (one load per lane).  Otherwise
    // the groups' totals are summed from the chunks' segment tables, the
    // slices per group scanned, and the item's group and slice looked up.
    // (The plan arrays live in the union region, before its use.)
    int *gsz = reinterpret_cast<int *>(un);      // [ngroups]
    int *ist = gsz + ngroups;                    // [ngroups + 1] first item of each group (in `ord` order)
    int *pst = ist + ngroups + 1;                // [ngroups + 1] first partial slot of each group
    int *ord = pst + ngroups + 1;                // [ngroups] groups by decreasing length
    int bound = 0;
    for (int c = lane; c < nchunks; c += 64) {
        const int2 m = *reinterpret_cast<const int2 *>(cmax + ((int64_t)bh * nchunks + c) * 2);
        bound += max(m.x, m.y);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) bound += __shfl_xor(bound, off);
    int gq, slice, nslices, gsize = -1, pslot = 0;
    if (bound <= quiet) {
        if (item >= ngroups) return;
        gq = item;
        slice = 0;
        nslices = 1;
    } else {
        for (int gi = tid; gi < ngroups; gi += NT) gsz[gi] = 0;
        __syncthreads();
        // every (group, chunk) entry once, loads independent of each other
        for (int e = tid; e < ngroups * nchunks; e += NT)
            atomicAdd(gsz + e / nchunks, seg[(int64_t)bh * ngroups * nchunks + e].y);
        __syncthreads();
        // Items go to the groups longest first (ties to the lower index): the
        // grid dispatches item-major over the heads, so every head's longest
        // work is dispatched first and the short items fill in at the end.
        for (int gi = tid; gi < ngroups; gi += NT) {
            const int sz = gsz[gi];
            int rank = 0;
            for (int o = 0; o < ngroups; ++o) {
                const int so = gsz[o];
                rank += (so > sz) | ((so == sz) & (o < gi));
            }
            ord[rank] = gi;
        }
        __syncthreads();
        if (wave == 0) {   // exclusive scans of the slice and partial-slot counts, in `ord` order
            int c1 = 0, c2 = 0;
            for (int base = 0; base < ngroups; base += 64) {
                const int gi = base + lane < ngroups ? ord[base + lane] : 0;
                const int ns = base + lane < ngroups ? max(1, (gsz[gi] + target - 1) / target) : 0;
                const int np = ns > 1 ? ns - 1 : 0;
                int i1 = ns, i2 = np;
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    const int t1 = __shfl_up(i1, off), t2 = __shfl_up(i2, off);
                    if (lane >= off) {
                        i1 += t1;
                        i2 += t2;
                    }
                }
                if (base + lane < ngroups) {
                    ist[base + lane] = c1 + i1 - ns;
                    pst[base + lane] = c2 + i2 - np;
                }
                c1 += __shfl(i1, 63);
                c2 += __shfl(i2, 63);
            }
            if (lane == 0) {
                ist[ngroups] = c1;
                pst[ngroups] = c2;
            }
        }
        __syncthreads();
        if (item >= ist[ngroups]) return;    // past this (b, h)'s items (the same for the whole group)
        int lo = 0, hi = ngroups;            // the group's place: last one whose first item is <= item
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            const bool right = ist[mid] <= item;
            lo = right ? mid : lo;
            hi = right ? hi : mid;
        }
        gq = ord[lo];
        slice = item - ist[lo];
        nslices = ist[lo + 1] - ist[lo];
        gsize = gsz[gq];
        pslot = pst[lo];
        __syncthreads();                     // the plan arrays are dead from here
    }

    const int p0 = gq * G;
    const int Gv = min(G, M0 - p0);
    // slots (and norms) per head: M0 * (1 + CC) for a two-level tree; the
    // second descent of a three-level tree passes the whole tree's stride
    // with the arrays offset to its children
    const int S = slot_stride;
    const int64_t head = (int64_t)bh * N;
    // this wave's transposed-V tile and slot bytes
    T *VT = reinterpret_cast<T *>(un + (size_t)wave * (D * LDK * sizeof(T) + KEYS));
    unsigned char *SL = reinterpret_cast<unsigned char *>(VT + D * LDK);

    // ---- stage -2 * codewords (block layout) and norms; bucket sizes
    constexpr int kRows = G * BR;
    constexpr int kStage = (kRows * D / 8 + NT - 1) / NT;
    const T *any_row = children + ((int64_t)h * M0 + p0) * CC * D;
    Frag<T> sf[kStage];
    // (a flat codebook, CC = 0, has no child level: nothing to stage, the
    // keys' distances are never needed)
#pragma unroll
    for (int k = 0; k < (CC > 0 ? kStage : 0); ++k) {
        const int e = (tid + NT * k) * 8, r = e / D, c = e % D, lp = r / BR, j = r % BR;
        const T *src = any_row;
        if (e < kRows * D && lp < Gv) {
            if (j < CC) src = children + (((int64_t)h * M0 + p0 + lp) * CC + j) * D + c;
            else if (j == CC) src = parents + ((int64_t)h * M0 + p0 + lp) * D + c;
        }
        sf[k] = load_frag(src);
    }
    float nrm = INFINITY;
    if (tid < kRows) {
        const int lp = tid / BR, j = tid % BR;
        if (lp < Gv) {
            if (j < CC) nrm = sqnorm[(int64_t)h * S + M0 + (p0 + lp) * CC + j];
            else if (j == CC) nrm = sqnorm[(int64_t)h * S + p0 + lp];
        }
    }
    for (int c = tid; c < nchunks; c += NT) {
        const int2 sg = seg[((int64_t)bh * ngroups + gq) * nchunks + c];
        pre[c] = sg.y;
        segs[c] = c * kAssignChunk + sg.x;
    }
    // the frame is all zero for a centred codebook: keys are then used as
    // they are (the same value in every wave)
    const float *fr = frame + (int64_t)h * D;
    const float rl = fr[lane % D], rh = fr[(lane + 64) % D];
    const bool shift = __ballot(rl != 0.f || rh != 0.f) != 0ull;
    if (tid < D) rv[tid] = fr[tid];
#pragma unroll
    for (int k = 0; k < (CC > 0 ? kStage : 0); ++k) {
        const int e = (tid + NT * k) * 8, r = e / D, c = e % D, lp = r / BR, j = r % BR;
        if (e < kRows * D) {
            const f32x4 r0 = *reinterpret_cast<const f32x4 *>(fr + c);
            const f32x4 r1 = *reinterpret_cast<const f32x4 *>(fr + c + 4);
            store_frag(Cw + r * LDP + c, (lp < Gv && j <= CC) ? frame_m2(sf[k], r0, r1) : zero_frag<T>());
        }
    }
    if (tid < kRows) rn[tid] = nrm;
    __syncthreads();
    if (wave == 0) {   // exclusive scan of the bucket sizes
        int carry = 0;
        for (int base = 0; base < nchunks; base += 64) {
            const int c = base + lane;
            const int v = c < nchunks ? pre[c] : 0;
            int inc = v;
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                const int t = __shfl_up(inc, off);
                if (lane >= off) inc += t;
            }
            if (c < nchunks) pre[c] = carry + inc - v;
            carry += __shfl(inc, 63);
        }
        if (lane == 0) pre[nchunks] = carry;
    }
    __syncthreads();
    const int total = pre[nchunks];
    // this work-group's list positions [xs, xe): the whole group, or its
    // slice of equal parts
    const int xs = gsize < 0 ? 0 : (int)((int64_t)gsize * slice / nslices);
    const int xe = gsize < 0 ? total : (int)((int64_t)gsize * (slice + 1) / nslices);

    // raw list entry (key | parent << 24) at position x of the group's list;
    // positions past the end read the last entry (never used)
    auto entry = [&](int x) -> unsigned {
        x = min(x, total - 1);
        int lo = 0, hi = nchunks;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            const bool right = pre[mid] <= x;
            lo = right ? mid : lo;
            hi = right ? hi : mid;
        }
        return (unsigned)sorted[head + segs[lo] + (x - pre[lo])];
    };
    auto xpos = [&](int s) { return xs + (s * NW + wave) * KEYS; };
    auto load_kv = [&](unsigned e, Frag<T> (&kf)[KB][KS], Frag<T> (&vf)[KB][KS]) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const int key = (int)((unsigned)__shfl((int)e, 16 * kb + i16) & 0xFFFFFFu);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                if constexpr (CC > 0) kf[kb][ks] = load_frag(K + (head + key) * D + 32 * ks + 8 * g);
                vf[kb][ks] = load_frag(V + (head + key) * D + 32 * ks + 8 * g);
            }
        }
    };

    f32x4 sums[NSB][NDB], cnts[NSB];
#pragma unroll
    for (int sb = 0; sb < NSB; ++sb) {
        cnts[sb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int db = 0; db < NDB; ++db) sums[sb][db] = cnts[sb];
    }
    const Frag<T> ones = ones_frag<T>();

    // One step: distances from kf, transposed values from vf, aggregation.
    // kf is reloaded with the keys of entry `en` as soon as the distance
    // MFMAs have consumed it, vf as soon as it has been transposed, so the
    // next step's rows are in flight during the rest of this one.
    auto compute = [&](int s, unsigned e, bool more, unsigned en, Frag<T> (&kf)[KB][KS],
                       Frag<T> (&vf)[KB][KS]) {
        const int x0 = xpos(s);
        if (CC > 0 && shift) {   // keys into the distance frame
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) kf[kb][ks] = shift_frag(kf[kb][ks], rv, 32 * ks + 8 * g);
        }
        int key[KB], lp[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            const unsigned ek = (unsigned)__shfl((int)e, 16 * kb + i16);
            key[kb] = (int)(ek & 0xFFFFFFu);
            lp[kb] = (int)(((ek >> 24) - (unsigned)p0) & 0xFFu);   // (entries carry parent mod 256)
        }
        // distances to every codeword row; keep the key's own parent block
        f32x4 own[KB][BRB];
#pragma unroll
        for (int rb = 0; rb < (CC > 0 ? NRB : 0); ++rb) {
            Frag<T> a[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) a[ks] = load_frag(Cw + (16 * rb + i16) * LDP + 32 * ks + 8 * g);
            const f32x4 seed = *reinterpret_cast<const f32x4 *>(rn + 16 * rb + 4 * g);
#pragma unroll
            for (int kb = 0; kb < KB; ++kb) {
                f32x4 d = seed;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) d = mma(a[ks], kf[kb][ks], d);
                const bool mine = rb / BRB == lp[kb];
                own[kb][rb % BRB] = mine ? d : (rb < BRB ? d : own[kb][rb % BRB]);
            }
        }
        int nkey[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) nkey[kb] = (int)((unsigned)__shfl((int)en, 16 * kb + i16) & 0xFFFFFFu);
        if (CC > 0 && more) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    kf[kb][ks] = load_frag(K + (head + nkey[kb]) * D + 32 * ks + 8 * g);
        }
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) {
            float cbest = INFINITY, pe = INFINITY;
            int crow = 0;
            if constexpr (CC > 0) {
#pragma unroll
                for (int q = 0; q < BRB; ++q)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int j = 16 * q + 4 * g + r;   // row inside the parent block
                        const float v = own[kb][q][r];
                        const bool lt = j < CC && v < cbest;
                        cbest = lt ? v : cbest;
                        crow = lt ? j : crow;
                        pe = j == CC ? v : pe;
                    }
                xgroup_argmin(cbest, crow);
                pe = xgroup_min(pe);
            }
            const bool to_child = CC > 0 && (force_child || cbest < pe);
            const int j = to_child ? crow : CC;
            const bool valid = x0 + 16 * kb + i16 < xe;
            if (g == 0) {
                SL[16 * kb + i16] = valid ? (unsigned char)(lp[kb] * (CC + 1) + j) : (unsigned char)0xFF;
                if (valid && leaf)
                    leaf[head + key[kb]] = leaf_base + (to_child ? M0 + (p0 + lp[kb]) * CC + crow : p0 + lp[kb]);
            }
            // transpose this column block's values into VT[dim][key]
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int t = 0; t < 8; ++t)
                    VT[(32 * ks + 8 * g + t) * LDK + 16 * kb + i16] = from_float<T>(frag_elem(vf[kb][ks], t));
        }
        if (more) {
#pragma unroll
            for (int kb = 0; kb < KB; ++kb)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    vf[kb][ks] = load_frag(V + (head + nkey[kb]) * D + 32 * ks + 8 * g);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const unsigned long long sl = *reinterpret_cast<const unsigned long long *>(SL + 32 * c + 8 * g);
            Frag<T> b[NDB];
#pragma unroll
            for (int db = 0; db < NDB; ++db) b[db] = load_frag(VT + (16 * db + i16) * LDK + 32 * c + 8 * g);
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb) {
                const Frag<T> oh = onehot_frag<T>(sl, 16 * sb + i16);
#pragma unroll
                for (int db = 0; db < NDB; ++db) sums[sb][db] = mma(oh, b[db], sums[sb][db]);
                cnts[sb] = mma(oh, ones, cnts[sb]);
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    const int span = xe - xs;   // this slice's list positions [xs, xe)
    const int nsteps = span > wave * KEYS ? (span - wave * KEYS + NW * KEYS - 1) / (NW * KEYS) : 0;
    if (nsteps > 0) {
        Frag<T> kf[KB][KS], vf[KB][KS];
        unsigned e0 = entry(xpos(0) + lane), e1 = entry(xpos(1) + lane);
        load_kv(e0, kf, vf);
        for (int s = 0; s < nsteps; ++s) {
            const unsigned e2 = entry(xpos(s + 2) + lane);   // two steps ahead
            compute(s, e0, s + 1 < nsteps, e1, kf, vf);
            e0 = e1;
            e1 = e2;
        }
    }
    __syncthreads();

    // ---- sum the waves' partial results into LDS (the V tiles are dead now):
    // every wave writes its own slice and the slices are summed in parallel
    // when they fit, else the waves add theirs in turn
    float *acc = reinterpret_cast<float *>(un);     // [NSL][NSB*16][LDA], slice 0 = total
    constexpr int NSL = Cfg::NSL;
    float *cntf = acc + NSL * NSB * 16 * LDA;       // [NSL][NSB*16]
    // round r: waves r*NSL .. r*NSL+NSL-1 write (r = 0) or add (r > 0) their
    // sums into slices 0..NSL-1; then the slices are summed into slice 0
    static_assert(NW % NSL == 0, "slices must divide the waves");
    for (int rnd = 0; rnd < NW / NSL; ++rnd) {
        if (wave / NSL == rnd) {
            const int sl = wave % NSL;
#pragma unroll
            for (int sb = 0; sb < NSB; ++sb)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int row = 16 * sb + 4 * g + r;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) {
                        float *pa = acc + (sl * NSB * 16 + row) * LDA + 16 * db + i16;
                        *pa = (rnd == 0 ? 0.f : *pa) + sums[sb][db][r];
                    }
                    if (i16 == 0) {
                        float *pc = cntf + sl * NSB * 16 + row;
                        *pc = (rnd == 0 ? 0.f : *pc) + cnts[sb][r];
                    }
                }
        }
        __syncthreads();
    }
    if constexpr (NSL > 1) {
        for (int e = tid; e < NSB * 16 * D; e += NT) {
            const int row = e / D, t = e % D;
            float s = acc[row * LDA + t];
#pragma unroll
            for (int w = 1; w < NSL; ++w) s += acc[(w * NSB * 16 + row) * LDA + t];
            acc[row * LDA + t] = s;
        }
        for (int e = tid; e < NSB * 16; e += NT) {
            float s = cntf[e];
#pragma unroll
            for (int w = 1; w < NSL; ++w) s += cntf[w * NSB * 16 + e];
            cntf[e] = s;
        }
        __syncthreads();
    }

    // ---- a split group: slices before the last store their sums for the
    // last one, which adds them in slice order.  The stores and loads are
    // agent-scope atomics (coherent across the XCDs' L2s); a slice's flag,
    // the call's tag, is stored once all its sums have landed.
    constexpr int PROWS = NSB * 16;
    if (nslices > 1) {
        const int64_t pbase = (int64_t)bh * npmax;
        if (slice < nslices - 1) {
            float *pp = partial + (pbase + pslot + slice) * (PROWS * (D + 1));
            for (int e = tid; e < PROWS * D; e += NT)
                __hip_atomic_store(pp + e, acc[(e / D) * LDA + e % D], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int e = tid; e < PROWS; e += NT)
                __hip_atomic_store(pp + PROWS * D + e, cntf[e], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            if (tid == 0) __hip_atomic_store(pflag + pbase + pslot + slice, tag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        // the last slice: every earlier slice of the group has a lower item
        // index, so it was dispatched earlier and finishes without waiting
        for (int q = tid; q < nslices - 1; q += NT) {
            const unsigned *f = pflag + pbase + pslot + q;
            while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != tag) __builtin_amdgcn_s_sleep(2);
        }
        __syncthreads();
        asm volatile("" ::: "memory");
        for (int e = tid; e < PROWS * (D + 1); e += NT) {
            float sum = 0.f;
            for (int q = 0; q < nslices - 1; ++q)
                sum += __hip_atomic_load(partial + (pbase + pslot + q) * (PROWS * (D + 1)) + e, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            if (e < PROWS * D) acc[(e / D) * LDA + e % D] += sum;
            else cntf[e - PROWS * D] += sum;
        }
        __syncthreads();
    }

    // ---- outputs: child slots as accumulated; parent = stayed + children
    float *vs = vsum + (int64_t)bh * S * D;
    int32_t *cs = count + (int64_t)bh * S;
    if constexpr (CC > 0) {
        for (int e = tid; e < Gv * CC * D; e += NT) {
            const int lp = e / (CC * D), c = (e / D) % CC, t = e % D;
            vs[((int64_t)M0 + p0 * CC) * D + e] = acc[(lp * (CC + 1) + c) * LDA + t];
        }
        for (int e = tid; e < Gv * CC; e += NT) cs[M0 + p0 * CC + e] = (int)cntf[(e / CC) * (CC + 1) + e % CC];
    }
    for (int e = tid; e < Gv * D; e += NT) {
        const int lp = e / D, t = e % D;
        float s = acc[(lp * (CC + 1) + CC) * LDA + t];
#pragma unroll
        for (int c = 0; c < CC; ++c) s += acc[(lp * (CC + 1) + c) * LDA + t];
        vs[(int64_t)(p0 + lp) * D + t] = s;
    }
    for (int lp = tid; lp < Gv; lp += NT) {
        float s = 0.f;
#pragma unroll
        for (int c = 0; c <= CC; ++c) s += cntf[lp * (CC + 1) + c];
        cs[p0 + lp] = (int)s;
    }
}

template <typename T, int D, int CC>
static hipError_t launch_refine(const void *K, const void *V, const void *parents,
                                const void *children, const float *sqnorm, const float *frame, int B, int H,
                                int N, int M0, unsigned flags, float *vsum, int32_t *count, int32_t *leaf,
                                const AssignWorkspace &ws, int slot_stride, int leaf_base, hipStream_t stream)
{
    using Cfg = RefineCfg<T, D, CC>;
    const int nchunks = (N + kAssignChunk - 1) / kAssignChunk;
    const int ngroups = (M0 + Cfg::G - 1) / Cfg::G;
    const RefinePlan pl = refine_plan(N, M0, CC, D);
    // the plan arrays share the union region when they fit in it
    const size_t plan_bytes = (size_t)(4 * ngroups + 2) * 4;
    const size_t lds = Cfg::lds(nchunks) + (plan_bytes > Cfg::union_bytes ? plan_bytes - Cfg::union_bytes + 16 : 0);
    allow_full_lds<refine_aggregate_kernel<T, D, CC>>();
    // grid (b*h, items): consecutive work-groups take the same item of
    // consecutive heads, so every head's real items come before any head's
    // unused ones
    hipLaunchKernelGGL((refine_aggregate_kernel<T, D, CC>), dim3(B * H, pl.max_items), dim3(kRefineThreads),
                       lds, stream, (const T *)K, (const T *)V, (const T *)parents,
                       (const T *)children, sqnorm, frame, H, N, M0, nchunks, (flags & 1u) ? 1 : 0,
                       ws.sorted, ws.seg, vsum, count, leaf, slot_stride, leaf_base, ngroups, pl.target,
                       pl.quiet, pl.max_partials, next_call_tag(), ws.cmax, ws.partial, ws.pflag);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_refine_t(const void *K, const void *V, const void *parents, const void *children,
                                  const float *sqnorm, const float *frame, int B, int H, int N, int M0, int C,
                                  unsigned flags,
                                  float *vsum, int32_t *count, int32_t *leaf,
                                  const AssignWorkspace &ws, int slot_stride, int leaf_base, hipStream_t stream)
{
#define AVQ_REFINE(CCV)                                                                                     \
    launch_refine<T, D, CCV>(K, V, parents, children, sqnorm, frame, B, H, N, M0, flags, vsum, count, leaf, ws, \
                             slot_stride, leaf_base, stream)
    switch (C) {
    case 0: return AVQ_REFINE(0);
    case 2: return AVQ_REFINE(2);
    case 4: return AVQ_REFINE(4);
    case 8: return AVQ_REFINE(8);
    default: return AVQ_REFINE(16);
    }
#undef AVQ_REFINE
}

hipError_t launch_refine_slots(const void *K, const void *V, const void *parents, const void *children,
                                    const float *sqnorm, const float *frame, int B, int H, int N, int d, int M0,
                                    int C, int dtype, unsigned flags, float *vsum, int32_t *count,
                                    int32_t *leaf, const AssignWorkspace &ws, int slot_stride, int leaf_base,
                                    hipStream_t stream)
{
#define AVQ_REFINE_ARGS K, V, parents, children, sqnorm, frame, B, H, N, M0, C, flags, vsum, count, leaf, ws, \
                        slot_stride, leaf_base, stream
    if (dtype == 1)
        return d == 64 ? launch_refine_t<bf16, 64>(AVQ_REFINE_ARGS) : launch_refine_t<bf16, 128>(AVQ_REFINE_ARGS);
    return d == 64 ? launch_refine_t<float, 64>(AVQ_REFINE_ARGS) : launch_refine_t<float, 128>(AVQ_REFINE_ARGS);
#undef AVQ_REFINE_ARGS
}

hipError_t launch_assign_aggregate(const void *K, const void *V, const void *parents,
                                   const void *children, const float *sqnorm, const float *frame, int B,
                                   int H, int N,
                                   int d, int M0, int C, int dtype, unsigned flags, float *vsum,
                                   int32_t *count, int32_t *leaf, const AssignWorkspace &ws,
                                   hipStream_t stream)
{
    hipError_t err = launch_assign_parent(K, parents, sqnorm, frame, B, H, N, d, M0, C, dtype, ws, nullptr, stream);
    if (err != hipSuccess) return err;
    return launch_refine_slots(K, V, parents, children, sqnorm, frame, B, H, N, d, M0, C, dtype, flags, vsum, count,
                               leaf, ws, M0 * (1 + C), 0, stream);
}

}  // namespace avq
