// Stage 2 of the AVQ-Attention forward pass: query-tile adaptive attention
// ("AVQ-Attention", Sec. 4.3).
//
// Work decomposition (gfx950): persistent work-groups of NWV waves (4; 8 for
// 256-query tiles and for bf16 at d = 128); each wave owns 32 queries as two
// 16-query MFMA column blocks (each codeword fragment read feeds two MFMAs;
// one block per wave, at twice the operand traffic per MFMA, measured ~1.6x
// slower), a work-group step covers NWV*32 queries (whole tiles).  One
// barrier per step, after the importance partials: every wave then selects
// its tile's parents itself (a three-level tree: the tile's first wave, and
// a second barrier after the selection).  A
// work-group stages its head's parents, their value sums (transposed) and
// counts in LDS once; LDS holds nothing else but the per-wave importance
// partials, so two work-groups share a CU and hide each other's barrier and
// load stalls (at d = 128 the value sums no longer fit beside a second
// work-group's parents: bf16 keeps them in LDS with one 8-wave work-group
// per CU, fp32 reads them from L2).  Work-groups are assigned to (head,
// query slice) so that consecutive work-group ids, which the dispatcher
// spreads over the 8 XCDs, give every XCD a contiguous range of heads: a
// head's children and value sums then live in one XCD's L2.
//
// Logits are computed transposed, S^T = C . Q^T (codewords as MFMA rows,
// queries as columns): each lane owns one query of each block, so the row
// max and the denominators are in-lane sums plus a reduction over the four
// lane groups, and the exponentiated tile is already laid out as the B
// operand of X^T += Vbar^T . E^T (Vbar^T comes from stage 1 with its
// contraction index permuted to match, see perm32).
//
// Per step:
//   parent pass  s = C_j . q over the M0 parents, shift m = max_j scale*s
//                over the parents that hold keys (n_j > 0),
//                E = exp2(scale*log2(e)*s - m'), Z = sum_j E n_j,
//                X^T = Vbar^T E^T ("Tiled VQ-attention");
//   importance   w_j = n_j sum_i E_ij / Z_i: reduced over the 16 queries of
//                each block with DPP, written per wave to LDS (alternating
//                between two buffers from step to step), summed over the
//                tile's waves ("Codeword importance");
//   top-P        every wave selects its tile's P parents into its own LDS
//                slots: exact bisection on the fp32 bit patterns of w
//                (w >= 0), ties to the lower index ("Child spawning");
//   correction   the selected parents' children are read straight from
//                global memory into MFMA operands, 32 children at a time
//                (the next 32 in flight).  Codeword rows are permuted so that lane group g holds
//                8 consecutive children, i.e. whole parents for C >= 8, and
//                the recovered parent logit (mean of the C child logits,
//                "Child attention") is an in-lane sum (plus one exchange for
//                C = 16).  The shift is raised if a child logit exceeds it
//                by more than 2^32 (X, Z rescaled) and X^T += Vbar_c^T . dA^T,
//                Z += sum dA n_c with
//                dA = exp(S_c - m) - exp(S_p - m);
//   Y = X / Z.
#include <type_traits>

#include "avq_kernels.h"

namespace avq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kQPW = 32;   // queries per wave

struct AttnLds {
    size_t ps, vt, np, wp, sel, wp2, sel2, total;
    bool wp2_shared;   // level-1 importance partials in the idle half of wp
};

// level-1 candidates of a three-level tree (the children of the P selected
// roots), rounded up to whole chunks of 32
__host__ __device__ inline int attn_cands(int P, int C) { return (P * C + 31) & ~31; }

// (nwave waves of kQPW queries per work-group step cover nwave * kQPW / tile
// tiles; each tile keeps one selection, or each wave its own copy of its
// tile's with wave_sel)
template <typename T, int D, bool VT_LDS>
__host__ __device__ inline AttnLds attn_lds(int M0, int P, int nwave, int tile, int C = 0, bool three_level = false,
                                            bool wave_sel = false)
{
    const int M0p = padded_parents(M0);
    const int ntile = nwave * kQPW > tile ? nwave * kQPW / tile : 1;
    AttnLds L;
    size_t o = 0;
    L.ps = o;  o += (size_t)M0p * (D + 8) * sizeof(T);
    L.vt = o;  if (VT_LDS) o += (size_t)D * (M0p + 8) * sizeof(T);
    L.np = o;  o += (size_t)M0p * 4;
    L.wp = o;  o += (size_t)2 * nwave * M0p * 4;
    // (one selection per wave when every wave of a tile selects for itself,
    // else one per tile)
    L.sel = o; o += (size_t)(wave_sel ? nwave : ntile) * ((P + 3) & ~3) * 4;
    L.wp2 = L.wp;
    L.sel2 = o;
    L.wp2_shared = true;
    if (three_level) {
        o += (size_t)ntile * ((P + 3) & ~3) * 4;
        L.wp2_shared = attn_cands(P, C) <= M0p;
        if (!L.wp2_shared) {
            L.wp2 = o;
            o += (size_t)nwave * attn_cands(P, C) * 4;
        }
    }
    L.total = o;
    return L;
}

// Exact top-P of w (w >= 0, M0 <= 256 values, lane l holds w[l + 64 i] in
// wv[i]) by one wave; ties go to the lower index.  Writes the selected
// indices in ascending order to selL (and sel_out if not null).
// The threshold is found by bisection on the bit patterns (monotone in w for
// w >= 0), from the top bit down; it stops early once exactly P values lie at
// or above the candidate, which for distinct values happens after a few bits
// past the first one that separates the P-th and (P+1)-th largest.
__device__ void select_top_p_regs(const float (&wv)[4], int M0, int P, int *selL, int32_t *sel_out)
{
    const int lane = lane_id();
    // entries past M0 count as 0; every bisection candidate is >= 1, so they
    // never pass a ">= cand" test (and equality with tau is masked below)
    unsigned u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = lane + 64 * i < M0 ? __float_as_uint(wv[i]) : 0u;
    unsigned tau = 0u;
    bool exact = false;   // exactly P values lie above tau
    if (P < M0) {
        for (int bit = 30; bit >= 0; --bit) {   // w >= 0: the sign bit is clear
            const unsigned cand = tau | (1u << bit);
            // (the four ballots are formed before any is counted, so that
            // they occupy separate scalar registers and issue back to back)
            const unsigned long long b0 = __builtin_amdgcn_ballot_w64(u[0] >= cand);
            const unsigned long long b1 = __builtin_amdgcn_ballot_w64(u[1] >= cand);
            const unsigned long long b2 = __builtin_amdgcn_ballot_w64(u[2] >= cand);
            const unsigned long long b3 = __builtin_amdgcn_ballot_w64(u[3] >= cand);
            const int cnt = (__popcll(b0) + __popcll(b1)) + (__popcll(b2) + __popcll(b3));
            if (cnt == P) {        // exactly P values >= cand: they are the top P
                tau = cand - 1u;
                exact = true;
                break;
            }
            tau = cnt > P ? cand : tau;
        }
    }
    int pos_base = 0;
    if (exact) {   // the selection is the values above tau, no tie to break
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool s = u[i] > tau;
            const unsigned long long sm = __ballot(s);
            if (s) {
                const int pos = pos_base + mbcnt(sm);
                selL[pos] = lane + 64 * i;
                if (sel_out) sel_out[pos] = lane + 64 * i;
            }
            pos_base += __popcll(sm);
        }
    } else {       // values above tau, then the lowest indices equal to tau
        int gt = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) gt += __popcll(__ballot(u[i] > tau));
        const int need = P - gt;
        int eq_before = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool in = lane + 64 * i < M0;
            const unsigned long long eqm = __ballot(in & (u[i] == tau));
            const bool s = (u[i] > tau) | (in & (u[i] == tau) & (eq_before + mbcnt(eqm) < need));
            eq_before += __popcll(eqm);
            const unsigned long long sm = __ballot(s);
            if (s) {
                const int pos = pos_base + mbcnt(sm);
                selL[pos] = lane + 64 * i;
                if (sel_out) sel_out[pos] = lane + 64 * i;
            }
            pos_base += __popcll(sm);
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename T> __device__ __forceinline__ Frag<T> frag_from8(const float (&v)[8]);
template <> __device__ __forceinline__ Frag<bf16> frag_from8<bf16>(const float (&v)[8])
{
    Frag<bf16> f;
#pragma unroll
    for (int k = 0; k < 8; ++k) f.v[k] = (bf16)v[k];
    return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from8<float>(const float (&v)[8])
{
    Frag<float> f;
    f.lo = f32x4{v[0], v[1], v[2], v[3]};
    f.hi = f32x4{v[4], v[5], v[6], v[7]};
    return f;
}

// y[16*db + r] = x[db][r] * s for r < 4, as one 8-byte (bf16) or 16-byte
// (fp32) store per db
template <typename T, int DB> __device__ __forceinline__ void store_row4(T *y, const f32x4 *x, float s);
template <> __device__ __forceinline__ void store_row4<bf16, 4>(bf16 *y, const f32x4 *x, float s)
{
#pragma unroll
    for (int db = 0; db < 4; ++db) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(x[db][r] * s);
        *reinterpret_cast<bf16x4 *>(y + 16 * db) = v;
    }
}
template <> __device__ __forceinline__ void store_row4<bf16, 8>(bf16 *y, const f32x4 *x, float s)
{
#pragma unroll
    for (int db = 0; db < 8; ++db) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (bf16)(x[db][r] * s);
        *reinterpret_cast<bf16x4 *>(y + 16 * db) = v;
    }
}
template <> __device__ __forceinline__ void store_row4<float, 4>(float *y, const f32x4 *x, float s)
{
#pragma unroll
    for (int db = 0; db < 4; ++db) *reinterpret_cast<f32x4 *>(y + 16 * db) = x[db] * s;
}
template <> __device__ __forceinline__ void store_row4<float, 8>(float *y, const f32x4 *x, float s)
{
#pragma unroll
    for (int db = 0; db < 8; ++db) *reinterpret_cast<f32x4 *>(y + 16 * db) = x[db] * s;
}

// chunks of 32 children processed together: one (two held the double-buffered
// codeword fragments in registers the rest of the step needs)
template <typename T, int D> constexpr int attn_super_chunks()
{
    return 1;
}

// NRB = number of 16-row parent blocks (padded_parents(M0) / 16).
// sl2 = |scale| * log2(e); neg != 0 flips the sign of Q (scale < 0), so the
// softmax shift is always a maximum.
// L3: three-level tree -- `children` is the middle level and `leaves` the
// C leaves of every child; after the children's correction the tile's
// level-1 importance picks P children, whose leaves correct them in turn.
template <typename T, int D, bool VT_LDS, int NRB, int CC, int NWV, bool L3, bool RANGES>
__global__ __launch_bounds__(64 * NWV, 2) void attention_kernel(
    const T *__restrict__ Q, const T *__restrict__ parents, const T *__restrict__ children,
    const unsigned char *__restrict__ pack, int H, int N, int M0, int P, int ltile, float sl2,
    int neg, int wsel, int ntiles, int nsteps, int per_bh, int nbh, T *__restrict__ Y,
    int32_t *__restrict__ sel_out, float *__restrict__ imp_out, const T *__restrict__ leaves,
    int32_t *__restrict__ sel1_out, int wsplit)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int LDP = D + 8;
    constexpr int M0p = 16 * NRB;
    constexpr int LDV = M0p + 8;
    constexpr int STEP = NWV * kQPW;
    constexpr int LC = CC == 2 ? 1 : CC == 4 ? 2 : CC == 8 ? 3 : 4;
    constexpr int SCH = attn_super_chunks<T, D>();
    const int selStride = (P + 3) & ~3;
    // wsel: every wave selects its tile's parents itself (two-level trees,
    // when the per-wave selections fit in LDS)
    const bool rsel = !L3 && wsel;
    const AttnLds L = attn_lds<T, D, VT_LDS>(M0, P, NWV, 1 << ltile, CC, L3, rsel);
    T *Ps = reinterpret_cast<T *>(smem + L.ps);
    T *Vt = reinterpret_cast<T *>(smem + L.vt);
    float *nP = reinterpret_cast<float *>(smem + L.np);
    float *Wp = reinterpret_cast<float *>(smem + L.wp);
    int *selS = reinterpret_cast<int *>(smem + L.sel);

    // The work-group's share of the (head, step) list, in one of two ways:
    //  - (head, slice) pairs (!RANGES): slice s of a head takes its steps
    //    s, s + per_bh, ... (see the step schedule below);
    //  - contiguous ranges of the list (RANGES), one per work-group,
    //    when the heads do not divide the CU slots evenly (e.g. 20 heads on
    //    256 one-work-group CUs): a range that crosses into the next head
    //    stages that head's codebook in LDS and goes on.
    // XCD x = blockIdx.x % 8 gets pairs (ranges) [x * G/8, (x+1) * G/8) of
    // the G = gridDim.x, so that every XCD holds a contiguous run of heads.
    const int G8 = gridDim.x >> 3;
    const int pair = (blockIdx.x & 7) * G8 + (blockIdx.x >> 3);
    const int TS = nbh * nsteps;
    const int gs0 = RANGES ? (int)((long long)pair * TS / gridDim.x) : 0;
    const int gs1 = RANGES ? (int)((long long)(pair + 1) * TS / gridDim.x) : 0;
    int bh = RANGES ? gs0 / nsteps : pair / per_bh;
    const int slice = RANGES ? 0 : pair - bh * per_bh;
    if (RANGES ? gs0 >= gs1 : bh >= nbh) return;
    int h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const PackLayout PL = pack_layout(M0, CC, D, (int)sizeof(T), L3);
    // Two-level trees with 16-bit operands form the output's denominators on
    // the matrix cores, from the counts split into three exact bf16 parts
    // (pack rows hi, mid, lo) and the same bf16 weights as the value sums, so
    // that the weights' rounding cancels in Y = X / Z; X gains a block whose
    // rows 0-2 collect them.  (The parent-level Z of the importance stays the
    // fp32 sum.)
    constexpr bool ZB = sizeof(T) == 2 && !L3;
    constexpr int DX = DB + (ZB ? 1 : 0);
    // the head's operands
    const unsigned char *pk;
    const T *pvt, *cvt, *Qh, *Ch, *Lh, *gvt, *pzp, *czp;
    const float *pnp, *cnp, *gnp;
    T *Yh;
    auto set_head = [&](int nb) {
        bh = nb;
        h = bh % H;
        pk = pack + (size_t)bh * PL.bytes;
        pvt = reinterpret_cast<const T *>(pk + PL.pvt);
        pnp = reinterpret_cast<const float *>(pk + PL.pn);
        cvt = reinterpret_cast<const T *>(pk + PL.cvt);
        cnp = reinterpret_cast<const float *>(pk + PL.cn);
        Qh = Q + (size_t)bh * N * D;
        Yh = Y + (size_t)bh * N * D;
        Ch = children + (size_t)h * M0 * CC * D;
        Lh = L3 ? leaves + (size_t)h * M0 * CC * CC * D : nullptr;
        gvt = reinterpret_cast<const T *>(pk + PL.gvt);
        gnp = reinterpret_cast<const float *>(pk + PL.gn);
        pzp = reinterpret_cast<const T *>(pk + PL.pz);
        czp = reinterpret_cast<const T *>(pk + PL.cz);
    };
    set_head(bh);
    const int zrow = i16 < 3 ? i16 : 3;   // count operand row of this lane (row 3: zero)

    // ---- stage the head's parents, parent value sums and counts (once per
    // head the work-group visits).
    // A row whose parent holds no key -- an empty parent, or a padding row
    // (M0 <= j < M0p) -- is staged as a copy of the first parent that does,
    // with its own count and value sum, which are zero: its logit is one of
    // the real ones, so the shift is the largest logit over the parents that
    // hold keys (an empty codeword far above them cannot push every weight
    // to zero), and it adds nothing to Z, X or the importance.
    auto stage_head = [&]() {
        int j0 = 0;   // first parent with keys (N >= 1: there is one)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = lane + 64 * i;
            const unsigned long long m = __ballot(j < M0 && pnp[j < M0 ? j : 0] > 0.f);
            if (m) {
                j0 = 64 * i + __ffsll((long long)m) - 1;
                break;
            }
        }
        for (int e = tid * 8; e < M0p * D; e += 64 * NWV * 8) {
            const int r = e / D, c = e % D;
            const int src = r < M0 && pnp[r] > 0.f ? r : j0;
            store_frag(Ps + r * LDP + c, load_frag(parents + ((size_t)h * M0 + src) * D + c));
        }
        if (VT_LDS) {
            for (int e = tid * 8; e < D * M0p; e += 64 * NWV * 8)
                store_frag(Vt + (e / M0p) * LDV + (e % M0p), load_frag(pvt + e));
        }
        for (int j = tid; j < M0p; j += 64 * NWV) nP[j] = pnp[j];
        __syncthreads();
    };
    stage_head();

    const int wpt = (1 << ltile) / kQPW;         // waves per tile
    const int tw0 = (w / wpt) * wpt;             // first wave of this wave's tile
    // With rsel every wave sums its tile's importance partials and selects
    // the tile's parents itself (the same values in the same order give every
    // wave of the tile the same selection), so no wave waits for another's
    // selection.  Otherwise the tile's first wave selects for the tile.
    int *mysel = selS + (rsel ? w : w / wpt) * selStride;   // this wave's copy of the tile's selection
    int *mysel2 = reinterpret_cast<int *>(smem + L.sel2) + (w / wpt) * selStride;   // its children's (L3)
    const int PC = P * CC;
    const int PCr = attn_cands(P, CC);

    // Rounds of per_bh steps: every slice takes one step per round.  With
    // two work-groups on every CU (wsplit), the last round goes to the
    // head's slices whose work-group was dispatched first to its CU (the
    // first half of the grid): the SIMDs favour the older waves, and the
    // first work-group runs ~1.2x faster than the second, which otherwise
    // ends ~15 us later, alone on its CU at a fraction of the CU's rate.
    const int G2 = G8 >> 1;
    auto early_before = [&](int p) { return (p / G8) * G2 + min(p % G8, G2); };
    const int p0 = bh * per_bh;
    const int nF = early_before(p0 + per_bh) - early_before(p0);   // early slices of the head
    const bool early = (pair % G8) < G2;
    const int eRank = early_before(pair) - early_before(p0);
    const int R = (nsteps + per_bh - 1) / per_bh;
    const bool split = wsplit && R >= 2 && nF > 0;
    const int lastR = (R - 1) * per_bh;   // first step of the last round
    int buf = 0;
    int st = RANGES ? gs0 - bh * nsteps : slice;
    for (int gs = gs0; RANGES ? gs < gs1 : st < nsteps; buf ^= 1) {
        const int q0 = st * STEP + kQPW * w + i16, q1 = q0 + 16;
        const bool v0 = q0 < N, v1 = q1 < N;
        // query fragments (queries past N read the last query; never stored)
        Frag<T> qa[KS], qb[KS];
        auto load_q = [&]() {
            const T *qra = Qh + (size_t)min(q0, N - 1) * D + 8 * g, *qrb = Qh + (size_t)min(q1, N - 1) * D + 8 * g;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                qa[ks] = load_frag(qra + 32 * ks);
                qb[ks] = load_frag(qrb + 32 * ks);
                if (neg) {
                    qa[ks] = negate(qa[ks]);
                    qb[ks] = negate(qb[ks]);
                }
            }
        };
        load_q();

        // ---- parent logits (raw dot products, sign of the scale folded in)
        // (codeword fragments of the next row block are read from LDS while
        // the current block's MFMAs run)
        f32x4 S0[NRB], S1[NRB];
        if constexpr (KS == 2) {
            // fragments two row blocks ahead (ring of three).  The scheduling
            // barriers pin the LDS reads of block rb+2 before the MFMAs of
            // block rb: left to itself the compiler reuses one pair of
            // fragment registers, and every block then waits for its own
            // LDS reads.
            Frag<T> pa[3][KS];
#pragma unroll
            for (int b = 0; b < 2 && b < NRB; ++b)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) pa[b][ks] = load_frag(Ps + (16 * b + i16) * LDP + 32 * ks + 8 * g);
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                if (rb + 2 < NRB) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks)
                        pa[(rb + 2) % 3][ks] = load_frag(Ps + (16 * (rb + 2) + i16) * LDP + 32 * ks + 8 * g);
                    __builtin_amdgcn_sched_barrier(0);
                }
                f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    a0 = mma(pa[rb % 3][ks], qa[ks], a0);
                    a1 = mma(pa[rb % 3][ks], qb[ks], a1);
                }
                __builtin_amdgcn_sched_barrier(0);
                S0[rb] = a0;
                S1[rb] = a1;
            }
        } else {
#pragma unroll
            for (int rb = 0; rb < NRB; ++rb) {
                f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const Frag<T> a = load_frag(Ps + (16 * rb + i16) * LDP + 32 * ks + 8 * g);
                    a0 = mma(a, qa[ks], a0);
                    a1 = mma(a, qb[ks], a1);
                }
                S0[rb] = a0;
                S1[rb] = a1;
            }
        }
        // ---- shift: largest logit of each query
        float e0 = -INFINITY, e1 = -INFINITY;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            e0 = max3f(e0, S0[rb][0], S0[rb][1]);
            e0 = max3f(e0, S0[rb][2], S0[rb][3]);
            e1 = max3f(e1, S1[rb][0], S1[rb][1]);
            e1 = max3f(e1, S1[rb][2], S1[rb][3]);
        }
        float m0 = sl2 * xgroup_max(e0), m1 = sl2 * xgroup_max(e1);

        // ---- E = exp(scale*s - m), denominators
        float z0 = 0.f, z1 = 0.f;
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            const f32x4 nv = *reinterpret_cast<const f32x4 *>(nP + 16 * rb + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x0 = __builtin_amdgcn_exp2f(fmaf(S0[rb][r], sl2, -m0));
                const float x1 = __builtin_amdgcn_exp2f(fmaf(S1[rb][r], sl2, -m1));
                S0[rb][r] = x0;
                S1[rb][r] = x1;
                z0 = fmaf(x0, nv[r], z0);
                z1 = fmaf(x1, nv[r], z1);
            }
        }
        float Zf0 = xgroup_sum(z0), Zf1 = xgroup_sum(z1);
        const float r0 = v0 ? __builtin_amdgcn_rcpf(Zf0) : 0.f, r1 = v1 ? __builtin_amdgcn_rcpf(Zf1) : 0.f;

        // ---- E as MFMA operands; the fp32 copy becomes the importance terms
        // t = E0 / Z0 + E1 / Z1 (this wave's two queries of every lane)
        Frag<T> E0[NRB / 2], E1[NRB / 2];
#pragma unroll
        for (int s = 0; s < NRB / 2; ++s) {
            E0[s] = pack_frag<T>(S0[2 * s], S0[2 * s + 1]);
            E1[s] = pack_frag<T>(S1[2 * s], S1[2 * s + 1]);
#pragma unroll
            for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S0[2 * s + hh][r] = fmaf(S0[2 * s + hh][r], r0, S1[2 * s + hh][r] * r1);
        }
        // sum over the 16 queries of each row and write this wave's partials
        {
            constexpr int LG = NRB == 16 ? 4 : NRB == 8 ? 3 : NRB == 4 ? 2 : 1;
            const f32x4 part = row16_reduce_scatter<NRB>(S0, i16);
            *reinterpret_cast<f32x4 *>(Wp + (buf * NWV + w) * M0p + 16 * (i16 >> (4 - LG)) + 4 * g) = part;
        }
        __syncthreads();       // every wave's importance partials are in Wp[buf]
        // X^T = Vbar^T E^T over the parents (issued after the barrier, so
        // that these MFMAs run beside the selection's chain of dependent
        // compare-and-count rounds below)
        f32x4 X0[DX], X1[DX];
#pragma unroll
        for (int db = 0; db < DX; ++db) {
            X0[db] = f32x4{0.f, 0.f, 0.f, 0.f};
            X1[db] = X0[db];
        }
        auto pz_frag = [&](int s_) -> Frag<T> { return load_frag(pzp + zrow * M0p + 32 * s_ + 8 * g); };
        // (value-sum fragments of the next 32 parents are read while the
        // current ones' MFMAs run)
        // From global memory the fragments are the same in every step; the
        // base is made opaque per step so that the compiler does not hoist
        // all D*M0p of them out of the loop (into scratch).
        const T *pvs = pvt;
        if constexpr (!VT_LDS) asm volatile("" : "+s"(pvs));
        auto vt_frag = [&](int s_, int db) -> Frag<T> {
            return VT_LDS ? load_frag(Vt + (16 * db + i16) * LDV + 32 * s_ + 8 * g)
                          : load_frag(pvs + (unsigned)((16 * db + i16) * M0p + 32 * s_ + 8 * g));
        };
        if constexpr (VT_LDS && D == 64) {
            Frag<T> va[2][DB];
#pragma unroll
            for (int db = 0; db < DB; ++db) va[0][db] = vt_frag(0, db);
#pragma unroll
            for (int s = 0; s < NRB / 2; ++s) {
                if (s + 1 < NRB / 2) {
#pragma unroll
                    for (int db = 0; db < DB; ++db) va[(s + 1) & 1][db] = vt_frag(s + 1, db);
                }
                if constexpr (ZB) {
                    const Frag<T> z = pz_frag(s);
                    X0[DB] = mma(z, E0[s], X0[DB]);
                    X1[DB] = mma(z, E1[s], X1[DB]);
                }
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    X0[db] = mma(va[s & 1][db], E0[s], X0[db]);
                    X1[db] = mma(va[s & 1][db], E1[s], X1[db]);
                }
            }
        } else {
#pragma unroll
            for (int s = 0; s < NRB / 2; ++s) {
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const Frag<T> a = vt_frag(s, db);
                    X0[db] = mma(a, E0[s], X0[db]);
                    X1[db] = mma(a, E1[s], X1[db]);
                }
                if constexpr (ZB) {
                    const Frag<T> a = pz_frag(s);
                    X0[DB] = mma(a, E0[s], X0[DB]);
                    X1[DB] = mma(a, E1[s], X1[DB]);
                }
            }
        }

        // ---- tile importance and top-P: by every wave (rsel), or by the
        // first wave of each tile while the tile's other waves wait at the
        // barrier below
        // (Wp[buf] is rewritten two steps later, after the next step's
        // barrier, which every wave reaches only once it has read Wp[buf])
        const int tg = ((st * STEP) >> ltile) + (w / wpt);   // global tile index
        if ((P > 0 || imp_out) && (rsel || w == tw0)) {
            // sum of the tile's wave partials (all NWV slots are read, those of
            // other tiles are masked out, so the loop has no branches)
            const float *wb = Wp + buf * NWV * M0p;
            float wv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = lane + 64 * i, jc = j < M0p ? j : 0;
                float a = 0.f;
#pragma unroll
                for (int ww = 0; ww < NWV; ++ww) {
                    const float x = wb[((tw0 + ww) & (NWV - 1)) * M0p + jc];
                    a += ww < wpt ? x : 0.f;
                }
                wv[i] = j < M0 ? a * nP[jc] : 0.f;
            }
            if (imp_out && tg < ntiles && w == tw0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = lane + 64 * i;
                    if (j < M0) imp_out[((size_t)bh * ntiles + tg) * M0 + j] = wv[i];
                }
            }
            if (P > 0)
                select_top_p_regs(wv, M0, P, mysel,
                                  (sel_out && tg < ntiles && w == tw0) ? sel_out + ((size_t)bh * ntiles + tg) * P
                                                                       : nullptr);
        }
        if (!rsel && P > 0 && wpt > 1) __syncthreads();   // the tile's selection is in LDS

        // ---- child correction, SCH chunks of 32 children at a time.
        // A position ph >= P*C (padding of the last chunks) takes the
        // codeword of child 0 of the first selected parent, whose logit is
        // already among the real ones (so the shift is unchanged), and the
        // all-zero count and value-sum entry of the level (so it adds
        // nothing); every chunk is therefore processed the same way, without
        // guards.  A level is described by the selected parents' indices,
        // the children's codewords, and their value sums and counts in the
        // pack; a three-level tree runs it once more one level down.
        // (at d = 128 the query fragments are read again here rather than
        // held through the weights, value sums and selection, which keeps
        // the parent pass out of scratch)
        float dz0 = 0.f, dz1 = 0.f;
        if constexpr (CC > 0) {   // (a flat codebook, CC = 0, has no child level)
        if constexpr (D == 128) {
            asm volatile("" ::: "memory");
            load_q();
        }
        const float sl2c = sl2 * (1.0f / (float)CC);   // mean over CC children, scaled
        constexpr int SC = 32 * SCH;                    // children per super-chunk

        struct Level {
            const int *sel;     // selected parents of the level (LDS)
            const T *cw;        // children's codewords, parent-major
            const T *vt;        // children's value sums [np + 1][D][CC]
            const float *cn;    // children's counts [np + 1][CC]
            int zero;           // the all-zero entry (np)
        };
        // codeword fragments of the super-chunk starting at c0: output row
        // 4g+r of tile A is child 8g+r of a chunk, of tile B child 8g+4+r
        struct CwBuf {
            Frag<T> a[SCH][KS], b[SCH][KS];
        };
        auto load_cw = [&](const Level &lv, int c0, CwBuf &cw) {
#pragma unroll
            for (int q = 0; q < SCH; ++q) {
                const int phA = c0 + 32 * q + 8 * (i16 >> 2) + (i16 & 3), phB = phA + 4;
                // (indices clamped so that the LDS reads are unconditional)
                const int sa = lv.sel[phA < PC ? phA >> LC : 0], sb = lv.sel[phB < PC ? phB >> LC : 0];
                const int ia = sa * CC + (phA < PC ? (phA & (CC - 1)) : 0);
                const int ib = sb * CC + (phB < PC ? (phB & (CC - 1)) : 0);
                const T *ra = lv.cw + (size_t)ia * D + 8 * g;
                const T *rb_ = lv.cw + (size_t)ib * D + 8 * g;
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    cw.a[q][ks] = load_frag(ra + 32 * ks);
                    cw.b[q][ks] = load_frag(rb_ + 32 * ks);
                }
            }
        };
        // child logits of a super-chunk (rows as in load_cw)
        auto child_logits = [&](const CwBuf &cw, int q, f32x4 &a0, f32x4 &b0, f32x4 &a1, f32x4 &b1) {
            a0 = f32x4{0.f, 0.f, 0.f, 0.f};
            b0 = a0; a1 = a0; b1 = a0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                a0 = mma(cw.a[q][ks], qa[ks], a0);
                b0 = mma(cw.b[q][ks], qa[ks], b0);
                a1 = mma(cw.a[q][ks], qb[ks], a1);
                b1 = mma(cw.b[q][ks], qb[ks], b1);
            }
        };
        // one super-chunk: its counts and value sums are loaded first (they
        // are needed last), the next super-chunk's codewords are loaded into
        // `nxt` while this one computes
        auto super_chunk = [&](const Level &lv, int c0, const CwBuf &cw, CwBuf &nxt, bool more) {
            f32x4 nA[SCH], nB[SCH];
            Frag<T> vc[SCH][DX];
#pragma unroll
            for (int q = 0; q < SCH; ++q) {
                const int ph0 = c0 + 32 * q + 8 * g;
                if constexpr (CC >= 8) {   // the 8 children share one parent
                    const int ps = lv.sel[ph0 < PC ? ph0 >> LC : 0];
                    const int pp = ph0 < PC ? ps : lv.zero;
                    const float *cp = lv.cn + (size_t)pp * CC + (ph0 & (CC - 1));
                    nA[q] = *reinterpret_cast<const f32x4 *>(cp);
                    nB[q] = *reinterpret_cast<const f32x4 *>(cp + 4);
                    const T *vp = lv.vt + ((size_t)pp * D + i16) * CC + (ph0 & (CC - 1));
#pragma unroll
                    for (int db = 0; db < DB; ++db) vc[q][db] = load_frag(vp + (size_t)16 * db * CC);
                    if constexpr (ZB)   // count parts of the 8 children (lanes past row 2: the zero entry)
                        vc[q][DB] = load_frag(czp + ((size_t)(i16 < 3 ? pp : lv.zero) * 3 + (i16 < 3 ? i16 : 0)) * CC +
                                              (ph0 & (CC - 1)));
                } else {
                    int pk8[8];   // slot (parent index, or the zero entry) of children ph0..ph0+7
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int ph = ph0 + k;
                        const int ps = lv.sel[ph < PC ? ph >> LC : 0];
                        pk8[k] = ph < PC ? ps : lv.zero;
                    }
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        nA[q][r] = lv.cn[(size_t)pk8[r] * CC + ((ph0 + r) & (CC - 1))];
                        nB[q][r] = lv.cn[(size_t)pk8[4 + r] * CC + ((ph0 + 4 + r) & (CC - 1))];
                    }
#pragma unroll
                    for (int db = 0; db < DB; ++db) {
                        float v[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            v[k] = to_float(lv.vt[((size_t)pk8[k] * D + 16 * db + i16) * CC + ((ph0 + k) & (CC - 1))]);
                        vc[q][db] = frag_from8<T>(v);
                    }
                    if constexpr (ZB) {
                        float v[8];
#pragma unroll
                        for (int k = 0; k < 8; ++k)
                            v[k] = to_float(czp[((size_t)(i16 < 3 ? pk8[k] : lv.zero) * 3 + (i16 < 3 ? i16 : 0)) * CC +
                                                ((ph0 + k) & (CC - 1))]);
                        vc[q][DB] = frag_from8<T>(v);
                    }
                }
            }
            if (more) load_cw(lv, c0 + SC, nxt);
            // child logits and their maximum
            f32x4 SA0[SCH], SB0[SCH], SA1[SCH], SB1[SCH];
            float c0m = -INFINITY, c1m = -INFINITY;
#pragma unroll
            for (int q = 0; q < SCH; ++q) {
                f32x4 a0, b0, a1, b1;
                child_logits(cw, q, a0, b0, a1, b1);
                SA0[q] = a0; SB0[q] = b0; SA1[q] = a1; SB1[q] = b1;
                c0m = max3f(c0m, max3f(a0[0], a0[1], a0[2]), max3f(a0[3], b0[0], b0[1]));
                c0m = max3f(c0m, b0[2], b0[3]);
                c1m = max3f(c1m, max3f(a1[0], a1[1], a1[2]), max3f(a1[3], b1[0], b1[1]));
                c1m = max3f(c1m, b1[2], b1[3]);
            }
            // raise the shift to cover the child logits, rescale X and Z
            // The shift only has to keep the weights in range: child weights
            // up to 2^32 above it are harmless in fp32 and bf16, so it is
            // raised (and X, Z rescaled) only when a child logit exceeds it
            // by more than that, which takes extreme logit ranges.
            // (any lane over the limit <=> some query's maximum is: the shift
            // is the same in a query's four lanes; the cross-lane maximum is
            // formed only then)
            if (__ballot((fmaf(c0m, sl2, -m0) > 32.f) | (fmaf(c1m, sl2, -m1) > 32.f))) {
                const float n0 = fmaxf(m0, sl2 * xgroup_max(c0m));
                const float n1 = fmaxf(m1, sl2 * xgroup_max(c1m));
                {
                    const float a0 = __builtin_amdgcn_exp2f(m0 - n0), a1 = __builtin_amdgcn_exp2f(m1 - n1);
                    m0 = n0; m1 = n1;
                    Zf0 *= a0; dz0 *= a0; Zf1 *= a1; dz1 *= a1;
#pragma unroll
                    for (int db = 0; db < DX; ++db) { X0[db] *= a0; X1[db] *= a1; }
                }
            }
#pragma unroll
            for (int q = 0; q < SCH; ++q) {
                // exp of the recovered parent logit of each child's parent
                float eA0[2], eB0[2], eA1[2], eB1[2];   // [r >> 1]
                if constexpr (CC >= 8) {
                    float u0 = (SA0[q][0] + SA0[q][1]) + (SA0[q][2] + SA0[q][3]) +
                               ((SB0[q][0] + SB0[q][1]) + (SB0[q][2] + SB0[q][3]));
                    float u1 = (SA1[q][0] + SA1[q][1]) + (SA1[q][2] + SA1[q][3]) +
                               ((SB1[q][0] + SB1[q][1]) + (SB1[q][2] + SB1[q][3]));
                    if constexpr (CC == 16) {
                        u0 = pair16_sum(u0);
                        u1 = pair16_sum(u1);
                    }
                    const float f0 = __builtin_amdgcn_exp2f(fmaf(u0, sl2c, -m0));
                    const float f1 = __builtin_amdgcn_exp2f(fmaf(u1, sl2c, -m1));
                    eA0[0] = eA0[1] = eB0[0] = eB0[1] = f0;
                    eA1[0] = eA1[1] = eB1[0] = eB1[1] = f1;
                } else if constexpr (CC == 4) {
                    eA0[0] = eA0[1] = __builtin_amdgcn_exp2f(fmaf((SA0[q][0] + SA0[q][1]) + (SA0[q][2] + SA0[q][3]), sl2c, -m0));
                    eB0[0] = eB0[1] = __builtin_amdgcn_exp2f(fmaf((SB0[q][0] + SB0[q][1]) + (SB0[q][2] + SB0[q][3]), sl2c, -m0));
                    eA1[0] = eA1[1] = __builtin_amdgcn_exp2f(fmaf((SA1[q][0] + SA1[q][1]) + (SA1[q][2] + SA1[q][3]), sl2c, -m1));
                    eB1[0] = eB1[1] = __builtin_amdgcn_exp2f(fmaf((SB1[q][0] + SB1[q][1]) + (SB1[q][2] + SB1[q][3]), sl2c, -m1));
                } else {   // CC == 2
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        eA0[k] = __builtin_amdgcn_exp2f(fmaf(SA0[q][2 * k] + SA0[q][2 * k + 1], sl2c, -m0));
                        eB0[k] = __builtin_amdgcn_exp2f(fmaf(SB0[q][2 * k] + SB0[q][2 * k + 1], sl2c, -m0));
                        eA1[k] = __builtin_amdgcn_exp2f(fmaf(SA1[q][2 * k] + SA1[q][2 * k + 1], sl2c, -m1));
                        eB1[k] = __builtin_amdgcn_exp2f(fmaf(SB1[q][2 * k] + SB1[q][2 * k + 1], sl2c, -m1));
                    }
                }
                f32x4 dA0, dB0, dA1, dB1;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dA0[r] = __builtin_amdgcn_exp2f(fmaf(SA0[q][r], sl2, -m0)) - eA0[r >> 1];
                    dB0[r] = __builtin_amdgcn_exp2f(fmaf(SB0[q][r], sl2, -m0)) - eB0[r >> 1];
                    dA1[r] = __builtin_amdgcn_exp2f(fmaf(SA1[q][r], sl2, -m1)) - eA1[r >> 1];
                    dB1[r] = __builtin_amdgcn_exp2f(fmaf(SB1[q][r], sl2, -m1)) - eB1[r >> 1];
                    if constexpr (!ZB) {
                        dz0 = fmaf(dA0[r], nA[q][r], fmaf(dB0[r], nB[q][r], dz0));
                        dz1 = fmaf(dA1[r], nA[q][r], fmaf(dB1[r], nB[q][r], dz1));
                    }
                }
                const Frag<T> b0 = pack_frag<T>(dA0, dB0), b1 = pack_frag<T>(dA1, dB1);
#pragma unroll
                for (int db = 0; db < DX; ++db) {
                    X0[db] = mma(vc[q][db], b0, X0[db]);
                    X1[db] = mma(vc[q][db], b1, X1[db]);
                }
            }
        };
        auto correct_level = [&](const Level &lv) {
            if (PC > 0) {
                CwBuf cwA, cwB;
                load_cw(lv, 0, cwA);
                for (int c0 = 0; c0 < PC; c0 += 2 * SC) {
                    super_chunk(lv, c0, cwA, cwB, c0 + SC < PC);
                    if (c0 + SC >= PC) break;
                    super_chunk(lv, c0 + SC, cwB, cwA, c0 + 2 * SC < PC);
                }
            }
        };
        correct_level(Level{mysel, Ch, cvt, cnp, M0});

        if constexpr (L3) {
            // ---- level 1 of a three-level tree: importance of the P*C
            // children just added, w_c = n_c sum_i exp(S_ic - m_i) / Z_i with
            // Z after their correction (the logits are formed again: a
            // second pass over the same codewords, from L2), top-P children,
            // then the same correction one level down
            const float Z10 = Zf0 + xgroup_sum(dz0), Z11 = Zf1 + xgroup_sum(dz1);
            const float u0 = v0 ? __builtin_amdgcn_rcpf(Z10) : 0.f, u1 = v1 ? __builtin_amdgcn_rcpf(Z11) : 0.f;
            float *W2 = L.wp2_shared ? Wp + (buf ^ 1) * NWV * M0p : reinterpret_cast<float *>(smem + L.wp2);
            const Level lv1{mysel, Ch, cvt, cnp, M0};
            for (int c0 = 0; c0 < PC; c0 += 32) {
                CwBuf cw;
                load_cw(lv1, c0, cw);
                f32x4 a0, b0, a1, b1;
                child_logits(cw, 0, a0, b0, a1, b1);
                f32x4 t[2];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    t[0][r] = __builtin_amdgcn_exp2f(fmaf(a0[r], sl2, -m0)) * u0 +
                              __builtin_amdgcn_exp2f(fmaf(a1[r], sl2, -m1)) * u1;
                    t[1][r] = __builtin_amdgcn_exp2f(fmaf(b0[r], sl2, -m0)) * u0 +
                              __builtin_amdgcn_exp2f(fmaf(b1[r], sl2, -m1)) * u1;
                }
                // summed over the 16 queries of each row: children
                // c0 + 8g + 4 (i16 >> 3) + r
                const f32x4 part = row16_reduce_scatter<2>(t, i16);
                if ((i16 & 7) == 0) *reinterpret_cast<f32x4 *>(W2 + w * PCr + c0 + 8 * g + 4 * (i16 >> 3)) = part;
            }
            __syncthreads();   // every wave's level-1 partials are in W2
            if (w == tw0) {
                float wv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int j = lane + 64 * i, jc = j < PC ? j : 0;
                    float a = 0.f;
#pragma unroll
                    for (int ww = 0; ww < NWV; ++ww) {
                        const float x = W2[((tw0 + ww) & (NWV - 1)) * PCr + jc];
                        a += ww < wpt ? x : 0.f;
                    }
                    const float nc = cnp[(size_t)mysel[jc >> LC] * CC + (jc & (CC - 1))];
                    wv[i] = j < PC ? a * nc : 0.f;
                }
                // positions among the candidates (ascending), then child ids
                select_top_p_regs(wv, PC, P, mysel2, nullptr);
                for (int k = lane; k < P; k += 64) {
                    const int pos = mysel2[k];
                    const int child = mysel[pos >> LC] * CC + (pos & (CC - 1));
                    mysel2[k] = child;
                    if (sel1_out && tg < ntiles) sel1_out[((size_t)bh * ntiles + tg) * P + k] = child;
                }
            }
            __syncthreads();   // the children's selection is in LDS
            correct_level(Level{mysel2, Lh, gvt, gnp, M0 * CC});
        }
        }   // CC > 0

        // ---- Y = X / Z: lane (g, i) holds dims 16*db + 4g .. +3 of its query
        // (with ZB the rows hi, mid and lo of the count block are in lane
        // group 0, and the other lane groups' rows of it are zero)
        const float Z0 = ZB ? xgroup_sum((X0[DX - 1][0] + X0[DX - 1][1]) + X0[DX - 1][2]) : Zf0 + xgroup_sum(dz0);
        const float Z1 = ZB ? xgroup_sum((X1[DX - 1][0] + X1[DX - 1][1]) + X1[DX - 1][2]) : Zf1 + xgroup_sum(dz1);
        if (v0) store_row4<T, DB>(Yh + (size_t)q0 * D + 4 * g, X0, __builtin_amdgcn_rcpf(Z0));
        if (v1) store_row4<T, DB>(Yh + (size_t)q1 * D + 4 * g, X1, __builtin_amdgcn_rcpf(Z1));
        // the next step
        if constexpr (RANGES) {
            ++gs;
            ++st;
            if (gs < gs1 && st == nsteps) {   // the range goes on in the next head
                __syncthreads();              // every wave is done with this head's LDS
                set_head(bh + 1);
                stage_head();
                st = 0;
            }
        } else if (!split) {
            st += per_bh;
        } else if (st < lastR) {
            st += per_bh;
            if (st >= lastR) st = early ? lastR + eRank : nsteps;   // entering the last round
        } else {
            st += nF;
        }
    }
}

// ---------------------------------------------------------------------------

// waves per work-group for a query tile: 4, or 8 for 256-query tiles and
// whenever the d = 128 value sums are held in LDS (the work-group then fills
// its CU alone)
template <int D, bool VT> static int attn_waves(int tile) { return tile >= 256 || (VT && D == 128) ? 8 : 4; }

int attention_child_chunk(int d, int M0, int C, int P, int tile, int dtype, bool three_level)
{
    if (tile != 32 && tile != 64 && tile != 128 && tile != 256) return 0;
    size_t lds;
    if (dtype == 1)
        lds = d == 64 ? attn_lds<bf16, 64, true>(M0, P, attn_waves<64, true>(tile), tile, C, three_level).total
                      : attn_lds<bf16, 128, true>(M0, P, attn_waves<128, true>(tile), tile, C, three_level).total;
    else
        lds = d == 64 ? attn_lds<float, 64, true>(M0, P, attn_waves<64, true>(tile), tile, C, three_level).total
                      : attn_lds<float, 128, false>(M0, P, attn_waves<128, false>(tile), tile, C, three_level).total;
    return lds <= 160 * 1024 ? 32 : 0;
}

static int ilog2(int x)
{
    int l = 0;
    while ((1 << (l + 1)) <= x) ++l;
    return l;
}

static int device_cus()
{
    static int cus[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

struct AttnArgs {
    const void *Q, *parents, *children, *pack, *leaves;
    int B, H, N, M0, C, P, tile;
    float scale;
    void *Y;
    int32_t *sel, *sel1;
    float *imp;
};

template <typename T, int D, bool VT, int NRB, int CC, int NWV, bool L3>
static hipError_t launch_attn_k(const AttnArgs &a, hipStream_t stream)
{
    allow_full_lds<attention_kernel<T, D, VT, NRB, CC, NWV, L3, false>>();
    // per-wave selections (two-level trees) when they fit in LDS without
    // costing a CU its second work-group
    const size_t lds_t = attn_lds<T, D, VT>(a.M0, a.P, NWV, a.tile, CC, L3, false).total;
    const size_t lds_w = attn_lds<T, D, VT>(a.M0, a.P, NWV, a.tile, CC, L3, true).total;
    auto cu_share = [](size_t b) { return NWV == 4 && b * 2 <= 160 * 1024 ? 2 : 1; };
    const bool wsel = !L3 && lds_w <= 160 * 1024 && cu_share(lds_w) == cu_share(lds_t);
    const size_t lds = wsel ? lds_w : lds_t;
    const int ntiles = (a.N + a.tile - 1) / a.tile;
    const int nsteps = (a.N + NWV * kQPW - 1) / (NWV * kQPW);
    const int BH = a.B * a.H;
    // two work-groups per CU when LDS and registers allow (an 8-wave
    // work-group takes both of a SIMD's two wave slots), each a slice of one
    // head's steps; rounded down, so that every work-group is resident from
    // the start (one more slice per head would leave work-groups waiting for
    // a second round)
    const int per_cu = cu_share(lds);
    const int slots = per_cu * device_cus();
    const int per_bh = max(1, min(nsteps, slots / BH));
    // contiguous ranges of the (head, step) list when they take fewer steps
    // per work-group than whole slices of a head (heads that do not divide
    // the slots), one work-group per slot
    const long long TS = (long long)BH * nsteps;
    const bool ranges = NWV == 8 && slots % 8 == 0 && TS < (1ll << 31) &&
                        (TS + slots - 1) / slots < (nsteps + per_bh - 1) / per_bh;
    const int grid = ranges ? slots : (BH * per_bh + 7) & ~7;
    // (the range form is built for the one-work-group-per-CU shapes only)
    if constexpr (NWV == 8) {
        if (ranges) {
            allow_full_lds<attention_kernel<T, D, VT, NRB, CC, NWV, L3, true>>();
            hipLaunchKernelGGL((attention_kernel<T, D, VT, NRB, CC, NWV, L3, true>), dim3(grid), dim3(64 * NWV), lds,
                               stream, (const T *)a.Q, (const T *)a.parents, (const T *)a.children,
                               (const unsigned char *)a.pack, a.H, a.N, a.M0, a.P, ilog2(a.tile),
                               fabsf(a.scale) * kLog2e, a.scale < 0.f ? 1 : 0, wsel ? 1 : 0, ntiles, nsteps, per_bh,
                               BH, (T *)a.Y, a.sel, a.imp, (const T *)a.leaves, a.sel1, 0);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((attention_kernel<T, D, VT, NRB, CC, NWV, L3, false>), dim3(grid), dim3(64 * NWV), lds, stream,
                       (const T *)a.Q, (const T *)a.parents, (const T *)a.children, (const unsigned char *)a.pack,
                       a.H, a.N, a.M0, a.P, ilog2(a.tile), fabsf(a.scale) * kLog2e, a.scale < 0.f ? 1 : 0,
                       wsel ? 1 : 0, ntiles,
                       nsteps, per_bh, BH, (T *)a.Y, a.sel, a.imp, (const T *)a.leaves, a.sel1,
                       per_cu == 2 && grid == 2 * device_cus() ? 1 : 0);   // wsplit
    return hipGetLastError();
}

template <typename T, int D, bool VT, int NRB, int CC, bool L3>
static hipError_t launch_attn_w(const AttnArgs &a, hipStream_t stream)
{
    if (attn_waves<D, VT>(a.tile) == 8) return launch_attn_k<T, D, VT, NRB, CC, 8, L3>(a, stream);
    if constexpr (!(VT && D == 128)) return launch_attn_k<T, D, VT, NRB, CC, 4, L3>(a, stream);
    return hipErrorInvalidConfiguration;
}

template <typename T, int D, bool VT, int NRB>
static hipError_t launch_attn_nrb(const AttnArgs &a, hipStream_t stream)
{
    if (a.leaves) {
        switch (a.C) {
        case 2: return launch_attn_w<T, D, VT, NRB, 2, true>(a, stream);
        case 4: return launch_attn_w<T, D, VT, NRB, 4, true>(a, stream);
        case 8: return launch_attn_w<T, D, VT, NRB, 8, true>(a, stream);
        default: return launch_attn_w<T, D, VT, NRB, 16, true>(a, stream);
        }
    }
    switch (a.C) {
    case 0: return launch_attn_w<T, D, VT, NRB, 0, false>(a, stream);
    case 2: return launch_attn_w<T, D, VT, NRB, 2, false>(a, stream);
    case 4: return launch_attn_w<T, D, VT, NRB, 4, false>(a, stream);
    case 8: return launch_attn_w<T, D, VT, NRB, 8, false>(a, stream);
    default: return launch_attn_w<T, D, VT, NRB, 16, false>(a, stream);
    }
}

template <typename T, int D, bool VT>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t stream)
{
    if (attn_lds<T, D, VT>(a.M0, a.P, attn_waves<D, VT>(a.tile), a.tile, a.C, a.leaves != nullptr).total > 160 * 1024)
        return hipErrorInvalidConfiguration;
    switch (padded_parents(a.M0)) {
    case 32: return launch_attn_nrb<T, D, VT, 2>(a, stream);
    case 64: return launch_attn_nrb<T, D, VT, 4>(a, stream);
    case 128: return launch_attn_nrb<T, D, VT, 8>(a, stream);
    default: return launch_attn_nrb<T, D, VT, 16>(a, stream);
    }
}

hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int d, int M0, int C, int P,
                                int tile, float scale, int dtype, void *Y, int32_t *sel,
                                float *importance, hipStream_t stream, const void *leaves, int32_t *sel1)
{
    const AttnArgs a{Q, parents, children, pack, leaves, B, H, N, M0, C, P, tile, scale, Y, sel, sel1, importance};
    if (dtype == 1) return d == 64 ? launch_attn_t<bf16, 64, true>(a, stream) : launch_attn_t<bf16, 128, true>(a, stream);
    return d == 64 ? launch_attn_t<float, 64, true>(a, stream) : launch_attn_t<float, 128, false>(a, stream);
}

}  // namespace avq
