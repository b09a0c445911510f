// Stage 2 of the AVQ-Attention forward pass: query-tile adaptive attention
// ("AVQ-Attention", Sec. 4.3).
//
// Work decomposition (gfx950): one persistent work-group of 8 waves per
// slice of a (batch, head); it stages the head's parents, their value sums
// and counts in LDS once and then walks its query steps of 256 queries.
// Every wave owns 32 queries as two 16-query MFMA column blocks, so each
// codeword fragment read from LDS feeds two MFMAs.
//
// Logits are computed transposed, S^T = C . Q^T (codewords as MFMA rows,
// queries as columns): each lane owns one query of each block, so the row
// max and the denominators are in-lane sums plus a reduction over the four
// lane groups, and the exponentiated tile is already laid out as the B
// operand of X^T += Vbar^T . E^T (Vbar^T comes from stage 1 with its
// contraction index permuted to match, see perm32).
//
// Per step, for every tile of the step (tile in {32, 64, 128, 256}):
//   parent pass  s = C_j . q over the M0 parents, shift m = max_j scale*s,
//                E = exp2(scale*log2(e)*s - m'), Z = sum_j E n_j,
//                X^T = Vbar^T E^T ("Tiled VQ-attention");
//   importance   w_j = n_j sum_i E_ij / Z_i, reduced over the 16 queries of
//                each block with DPP, then across the tile's waves in LDS
//                ("Codeword importance");
//   top-P        one wave per tile: exact selection by bisection on the fp32
//                bit patterns of w (w >= 0, so bit order is value order),
//                ties to the lower index ("Child spawning");
//   correction   the P*C children of the tile's parents are staged in LDS in
//                chunks.  Inside a 32-wide contraction step lane group g
//                holds 8 consecutive children, i.e. whole parents for C >= 8,
//                so the recovered parent logit (mean of the C child logits,
//                "Child attention") is an in-lane sum (plus one exchange for
//                C = 16).  The shift is raised to cover the child logits (X, Z
//                rescaled) and X^T += Vbar_c^T . dA^T, Z += sum dA n_c with
//                dA = exp(S_c - m) - exp(S_p - m);
//   Y = X / Z.
#include <type_traits>

#include "avq_kernels.h"

namespace avq {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kQPW = 32;                 // queries per wave
constexpr int kStep = kWaves * kQPW;     // queries per work-group step

struct AttnLds {
    size_t ps, vt, np, wimp, sel, child, cs, vc, nc, total;
};

// LDS regions (bytes).  The per-wave importance partials share the child
// area: they are consumed before the first child chunk is staged.  Children
// are staged for `tpg` tiles at a time, `chk` children per tile.
template <typename T, int D, bool VT_LDS>
__host__ __device__ inline AttnLds attn_lds(int M0, int P, int tile, int chk, int tpg)
{
    const int M0p = padded_parents(M0);
    const int ntl = kStep / tile;
    AttnLds L;
    size_t o = 0;
    L.ps = o;   o += (size_t)M0p * (D + 8) * sizeof(T);
    L.vt = o;   if (VT_LDS) o += (size_t)D * (M0p + 8) * sizeof(T);
    L.np = o;   o += (size_t)M0p * 4;
    L.wimp = o; o += (size_t)ntl * M0p * 4;
    L.sel = o;  o += (size_t)ntl * ((P + 3) & ~3) * 4;
    L.child = o;
    size_t c = 0;
    L.cs = o + c; c += (size_t)tpg * chk * (D + 8) * sizeof(T);
    L.vc = o + c; c += (size_t)tpg * D * (chk + 8) * sizeof(T);
    L.nc = o + c; c += (size_t)tpg * chk * 4;
    const size_t wp = (size_t)kWaves * M0p * 4;
    o += c > wp ? c : wp;
    L.total = o;
    return L;
}

// LDS row of child phi (within a staged chunk): the rows of a 32-wide
// contraction step are ordered so that MFMA lane group g sees children
// 8g..8g+3 in the first 16-row tile and 8g+4..8g+7 in the second.
__device__ __forceinline__ int child_row(int phi)
{
    return (phi & ~31) + ((phi & 4) << 2) + (((phi >> 3) & 3) << 2) + (phi & 3);
}

// Exact top-P of w[0..M0) (w >= 0) by one wave; ties go to the lower index.
// Writes the selected indices in ascending order.
__device__ void select_top_p(const float *wimp, int M0, int P, int *selL, int32_t *sel_out)
{
    const int lane = lane_id();
    unsigned u[4];
    bool ok[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = lane + 64 * i;
        ok[i] = j < M0;
        u[i] = ok[i] ? __float_as_uint(wimp[j]) : 0u;
    }
    unsigned tau = 0u;
    if (P < M0) {
        for (int bit = 31; bit >= 0; --bit) {
            const unsigned cand = tau | (1u << bit);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) cnt += __popcll(__ballot(ok[i] && u[i] >= cand));
            if (cnt >= P) tau = cand;
        }
    }
    int gt = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) gt += __popcll(__ballot(ok[i] && u[i] > tau));
    const int need = P - gt;
    int eq_before = 0, pos_base = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned long long eqm = __ballot(ok[i] && u[i] == tau);
        const bool s = ok[i] && (u[i] > tau || (u[i] == tau && eq_before + mbcnt(eqm) < need));
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

// NRB = number of 16-row parent blocks (padded_parents(M0) / 16).
// sl2 = |scale| * log2(e); neg != 0 flips the sign of Q (scale < 0), so the
// softmax shift is always a maximum.
template <typename T, int D, bool VT_LDS, int NRB, int CC>
__global__ __launch_bounds__(kThreads) void attention_kernel(
    const T *__restrict__ Q, const T *__restrict__ parents, const T *__restrict__ children,
    const unsigned char *__restrict__ pack, int H, int N, int M0, int C, int lc, int P, int tile,
    int chk, int lchk, int tpg, float sl2, int neg, int ntiles, int nsteps, T *__restrict__ Y,
    int32_t *__restrict__ sel_out, float *__restrict__ imp_out)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int LDP = D + 8;
    constexpr int M0p = 16 * NRB;
    constexpr int LDV = M0p + 8;
    const int LDC = chk + 8;
    const int ntl = kStep / tile;
    const int wpt = tile / kQPW;                 // waves per tile
    const int selStride = (P + 3) & ~3;
    const AttnLds L = attn_lds<T, D, VT_LDS>(M0, P, tile, chk, tpg);
    T *Ps = reinterpret_cast<T *>(smem + L.ps);
    T *Vt = reinterpret_cast<T *>(smem + L.vt);
    float *nP = reinterpret_cast<float *>(smem + L.np);
    float *wimp = reinterpret_cast<float *>(smem + L.wimp);
    int *selL = reinterpret_cast<int *>(smem + L.sel);
    float *Wp = reinterpret_cast<float *>(smem + L.child);
    T *Cs = reinterpret_cast<T *>(smem + L.cs);
    T *Vc = reinterpret_cast<T *>(smem + L.vc);
    float *nC = reinterpret_cast<float *>(smem + L.nc);

    const int bh = blockIdx.y, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const PackLayout PL = pack_layout(M0, C, D, (int)sizeof(T));
    const unsigned char *pk = pack + (size_t)bh * PL.bytes;
    const T *pvt = reinterpret_cast<const T *>(pk + PL.pvt);
    const float *pnp = reinterpret_cast<const float *>(pk + PL.pn);
    const T *cvt = reinterpret_cast<const T *>(pk + PL.cvt);
    const float *cnp = reinterpret_cast<const float *>(pk + PL.cn);
    const T *Qh = Q + (size_t)bh * N * D;
    T *Yh = Y + (size_t)bh * N * D;
    const T *Ch = children + (size_t)h * M0 * C * D;

    // ---- stage the head's parents, parent value sums and counts once
    for (int e = tid * 8; e < M0p * D; e += kThreads * 8) {
        const int r = e / D, c = e % D;
        const Frag<T> f = r < M0 ? load_frag(parents + ((size_t)h * M0 + r) * D + c) : zero_frag<T>();
        store_frag(Ps + r * LDP + c, f);
    }
    if (VT_LDS) {
        for (int e = tid * 8; e < D * M0p; e += kThreads * 8)
            store_frag(Vt + (e / M0p) * LDV + (e % M0p), load_frag(pvt + e));
    }
    for (int j = tid; j < M0p; j += kThreads) nP[j] = pnp[j];
    __syncthreads();

    const int full_rb = M0 / 16;                 // blocks without padding rows
    const int tw = (kQPW * w) / tile;            // this wave's tile inside the step
    const int PC = P * C;

    // query fragments of a step (prefetched one step ahead)
    Frag<T> nqa[KS], nqb[KS];
    auto load_q = [&](int st_) {
        const int q0_ = st_ * kStep + kQPW * w + i16, q1_ = q0_ + 16;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            nqa[ks] = (st_ < nsteps && q0_ < N) ? load_frag(Qh + (size_t)q0_ * D + 32 * ks + 8 * g) : zero_frag<T>();
            nqb[ks] = (st_ < nsteps && q1_ < N) ? load_frag(Qh + (size_t)q1_ * D + 32 * ks + 8 * g) : zero_frag<T>();
        }
    };
    load_q(blockIdx.x);

    for (int st = blockIdx.x; st < nsteps; st += gridDim.x) {
        const int q0 = st * kStep + kQPW * w + i16, q1 = q0 + 16;
        const bool v0 = q0 < N, v1 = q1 < N;
        Frag<T> qa[KS], qb[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            qa[ks] = neg ? negate(nqa[ks]) : nqa[ks];
            qb[ks] = neg ? negate(nqb[ks]) : nqb[ks];
        }

        // ---- parent logits (raw dot products, sign of the scale folded in)
        f32x4 S0[NRB], S1[NRB];
#pragma unroll
        for (int rb = 0; rb < NRB; ++rb) {
            f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = a0;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const Frag<T> a = load_frag(Ps + (16 * rb + i16) * LDP + 32 * ks + 8 * g);
                a0 = mma(a, qa[ks], a0);
                a1 = mma(a, qb[ks], a1);
            }
            if (rb >= full_rb) {   // padding parents never take part
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const bool ok = (16 * rb + 4 * g + r) < M0;
                    a0[r] = ok ? a0[r] : -INFINITY;
                    a1[r] = ok ? a1[r] : -INFINITY;
                }
            }
            S0[rb] = a0;
            S1[rb] = a1;
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
            __builtin_amdgcn_sched_barrier(0);   // keep the count loads block-local
        }
        float Zf0 = xgroup_sum(z0), Zf1 = xgroup_sum(z1);
        const float r0 = v0 ? 1.0f / Zf0 : 0.f, r1 = v1 ? 1.0f / Zf1 : 0.f;

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
            *reinterpret_cast<f32x4 *>(Wp + w * M0p + 16 * (i16 >> (4 - LG)) + 4 * g) = part;
        }
        // X^T = Vbar^T E^T over the parents
        f32x4 X0[DB], X1[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            X0[db] = f32x4{0.f, 0.f, 0.f, 0.f};
            X1[db] = X0[db];
        }
#pragma unroll
        for (int s = 0; s < NRB / 2; ++s) {
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const Frag<T> a = VT_LDS ? load_frag(Vt + (16 * db + i16) * LDV + 32 * s + 8 * g)
                                         : load_frag(pvt + (size_t)(16 * db + i16) * M0p + 32 * s + 8 * g);
                X0[db] = mma(a, E0[s], X0[db]);
                X1[db] = mma(a, E1[s], X1[db]);
            }
        }
        load_q(st + gridDim.x);   // next step's queries, in flight during the rest
        __syncthreads();

        // ---- tile importance
        const int tile0 = (st * kStep) / tile;
        for (int idx = tid; idx < ntl * M0p; idx += kThreads) {
            const int tl = idx / M0p, j = idx % M0p;
            float s = 0.f;
            for (int ww = tl * wpt; ww < (tl + 1) * wpt; ++ww) s += Wp[ww * M0p + j];
            s *= nP[j];
            wimp[idx] = s;
            if (imp_out && j < M0 && tile0 + tl < ntiles)
                imp_out[((size_t)bh * ntiles + tile0 + tl) * M0 + j] = s;
        }
        __syncthreads();

        // ---- top-P, one wave per tile
        if (P > 0 && w < ntl) {
            if (tile0 + w < ntiles) {
                select_top_p(wimp + w * M0p, M0, P, selL + w * selStride,
                             sel_out ? sel_out + ((size_t)bh * ntiles + tile0 + w) * P : nullptr);
            } else {
                for (int k = lane; k < P; k += 64) selL[w * selStride + k] = 0;
            }
        }

        // ---- child correction
        float dz0 = 0.f, dz1 = 0.f;
        for (int cg = 0; cg < ((PC + chk - 1) / chk) * (ntl / tpg); ++cg) {
            const int c0 = (cg / (ntl / tpg)) * chk;   // first child of the chunk
            const int tg0 = (cg % (ntl / tpg)) * tpg;  // first tile of the staged group
            __syncthreads();   // selections visible; previous chunk consumed
            // stage codewords (row-permuted), value sums (transposed) and
            // counts; every size here is a power of two
            constexpr int LD8 = D == 128 ? 4 : 3;           // log2(D / 8)
            const int lcw = lchk + LD8;                      // log2(children x 8-dim pieces)
            constexpr int cmask = CC - 1;
            for (int it = tid; it < (tpg << lcw); it += kThreads) {
                const int tl = it >> lcw, ph = (it >> LD8) & (chk - 1), dg = it & ((D / 8) - 1);
                const int phi = c0 + ph;
                const Frag<T> f = phi < PC
                    ? load_frag(Ch + ((size_t)selL[(tg0 + tl) * selStride + (phi >> lc)] * C + (phi & cmask)) * D + 8 * dg)
                    : zero_frag<T>();
                store_frag(Cs + ((size_t)tl * chk + child_row(ph)) * LDP + 8 * dg, f);
            }
            const int lvs = lchk - 3;                        // log2(chk / 8)
            for (int it = tid; it < (tpg * D) << lvs; it += kThreads) {
                const int tl = it >> (lvs + LD8 + 3), dim = (it >> lvs) & (D - 1), pg = it & ((chk >> 3) - 1);
                const int phi0 = c0 + 8 * pg;
                const int *sl = selL + (tg0 + tl) * selStride;
                Frag<T> f;
                if constexpr (CC >= 8) {
                    f = phi0 < PC ? load_frag(cvt + ((size_t)sl[phi0 >> lc] * D + dim) * C + (phi0 & cmask))
                                  : zero_frag<T>();
                } else {
                    float v[8];
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const int phi = phi0 + k;
                        v[k] = phi < PC ? to_float(cvt[((size_t)sl[phi >> lc] * D + dim) * C + (phi & cmask)]) : 0.f;
                    }
                    f = frag_from8<T>(v);
                }
                store_frag(Vc + ((size_t)tl * D + dim) * LDC + 8 * pg, f);
            }
            for (int it = tid; it < (tpg << lchk); it += kThreads) {
                const int tl = it >> lchk, phi = c0 + (it & (chk - 1));
                nC[it] = phi < PC ? cnp[(size_t)selL[(tg0 + tl) * selStride + (phi >> lc)] * C + (phi & cmask)] : 0.f;
            }
            __syncthreads();
            if (tw < tg0 || tw >= tg0 + tpg) continue;   // wave's tile not in this group
            const int lt = tw - tg0;                      // its slot in the staged group

            // child logits of this wave's tile
            const int nks = min(chk, PC - c0 + 31) / 32;   // contraction steps holding children
            const bool partial = c0 + chk > PC;
            f32x4 SA0[4], SB0[4], SA1[4], SB1[4];
            float c0m = -INFINITY, c1m = -INFINITY;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                if (s < nks) {
                    f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, b0 = a0, a1 = a0, b1 = a0;
                    const T *rowA = Cs + ((size_t)lt * chk + 32 * s + i16) * LDP + 8 * g;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const Frag<T> fa = load_frag(rowA + 32 * ks);
                        const Frag<T> fb = load_frag(rowA + 16 * LDP + 32 * ks);
                        a0 = mma(fa, qa[ks], a0);
                        b0 = mma(fb, qa[ks], b0);
                        a1 = mma(fa, qb[ks], a1);
                        b1 = mma(fb, qb[ks], b1);
                    }
                    SA0[s] = a0; SB0[s] = b0; SA1[s] = a1; SB1[s] = b1;
                    if (partial) {   // children past P*C of the last chunk
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            const int phA = c0 + 32 * s + 8 * g + r;
                            if (phA >= PC) { a0[r] = -INFINITY; a1[r] = -INFINITY; }
                            if (phA + 4 >= PC) { b0[r] = -INFINITY; b1[r] = -INFINITY; }
                        }
                    }
                    c0m = max3f(c0m, max3f(a0[0], a0[1], a0[2]), max3f(a0[3], b0[0], b0[1]));
                    c0m = max3f(c0m, b0[2], b0[3]);
                    c1m = max3f(c1m, max3f(a1[0], a1[1], a1[2]), max3f(a1[3], b1[0], b1[1]));
                    c1m = max3f(c1m, b1[2], b1[3]);
                }
            }
            // raise the shift to cover the child logits, rescale X and Z
            {
                const float n0 = fmaxf(m0, sl2 * xgroup_max(c0m));
                const float n1 = fmaxf(m1, sl2 * xgroup_max(c1m));
                const float a0 = __builtin_amdgcn_exp2f(m0 - n0), a1 = __builtin_amdgcn_exp2f(m1 - n1);
                m0 = n0; m1 = n1;
                Zf0 *= a0; dz0 *= a0; Zf1 *= a1; dz1 *= a1;
#pragma unroll
                for (int db = 0; db < DB; ++db) { X0[db] *= a0; X1[db] *= a1; }
            }
            const float sl2c = sl2 * (1.0f / (float)CC);   // mean over CC children, scaled
            auto correct = [&](auto masked) {
                constexpr bool MASK = decltype(masked)::value;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    if (s < nks) {
                        // exp of the recovered parent logit of each child's parent:
                        // lane group g holds children 8g..8g+7 of the step
                        float eA0[2], eB0[2], eA1[2], eB1[2];   // [r >> 1]
                        if constexpr (CC >= 8) {
                            float u0 = (SA0[s][0] + SA0[s][1]) + (SA0[s][2] + SA0[s][3]) +
                                       ((SB0[s][0] + SB0[s][1]) + (SB0[s][2] + SB0[s][3]));
                            float u1 = (SA1[s][0] + SA1[s][1]) + (SA1[s][2] + SA1[s][3]) +
                                       ((SB1[s][0] + SB1[s][1]) + (SB1[s][2] + SB1[s][3]));
                            if constexpr (CC == 16) {
                                u0 += __shfl_xor(u0, 16);
                                u1 += __shfl_xor(u1, 16);
                            }
                            const float e0 = __builtin_amdgcn_exp2f(fmaf(u0, sl2c, -m0));
                            const float e1 = __builtin_amdgcn_exp2f(fmaf(u1, sl2c, -m1));
                            eA0[0] = eA0[1] = eB0[0] = eB0[1] = e0;
                            eA1[0] = eA1[1] = eB1[0] = eB1[1] = e1;
                        } else if constexpr (CC == 4) {
                            eA0[0] = eA0[1] = __builtin_amdgcn_exp2f(fmaf((SA0[s][0] + SA0[s][1]) + (SA0[s][2] + SA0[s][3]), sl2c, -m0));
                            eB0[0] = eB0[1] = __builtin_amdgcn_exp2f(fmaf((SB0[s][0] + SB0[s][1]) + (SB0[s][2] + SB0[s][3]), sl2c, -m0));
                            eA1[0] = eA1[1] = __builtin_amdgcn_exp2f(fmaf((SA1[s][0] + SA1[s][1]) + (SA1[s][2] + SA1[s][3]), sl2c, -m1));
                            eB1[0] = eB1[1] = __builtin_amdgcn_exp2f(fmaf((SB1[s][0] + SB1[s][1]) + (SB1[s][2] + SB1[s][3]), sl2c, -m1));
                        } else {   // CC == 2
#pragma unroll
                            for (int k = 0; k < 2; ++k) {
                                eA0[k] = __builtin_amdgcn_exp2f(fmaf(SA0[s][2 * k] + SA0[s][2 * k + 1], sl2c, -m0));
                                eB0[k] = __builtin_amdgcn_exp2f(fmaf(SB0[s][2 * k] + SB0[s][2 * k + 1], sl2c, -m0));
                                eA1[k] = __builtin_amdgcn_exp2f(fmaf(SA1[s][2 * k] + SA1[s][2 * k + 1], sl2c, -m1));
                                eB1[k] = __builtin_amdgcn_exp2f(fmaf(SB1[s][2 * k] + SB1[s][2 * k + 1], sl2c, -m1));
                            }
                        }
                        const f32x4 nA = *reinterpret_cast<const f32x4 *>(nC + lt * chk + 32 * s + 8 * g);
                        const f32x4 nB = *reinterpret_cast<const f32x4 *>(nC + lt * chk + 32 * s + 8 * g + 4);
                        f32x4 dA0, dB0, dA1, dB1;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            dA0[r] = __builtin_amdgcn_exp2f(fmaf(SA0[s][r], sl2, -m0)) - eA0[r >> 1];
                            dB0[r] = __builtin_amdgcn_exp2f(fmaf(SB0[s][r], sl2, -m0)) - eB0[r >> 1];
                            dA1[r] = __builtin_amdgcn_exp2f(fmaf(SA1[s][r], sl2, -m1)) - eA1[r >> 1];
                            dB1[r] = __builtin_amdgcn_exp2f(fmaf(SB1[s][r], sl2, -m1)) - eB1[r >> 1];
                            if constexpr (MASK) {   // children past P*C of the last chunk
                                const int phA = c0 + 32 * s + 8 * g + r;
                                if (phA >= PC) { dA0[r] = 0.f; dA1[r] = 0.f; }
                                if (phA + 4 >= PC) { dB0[r] = 0.f; dB1[r] = 0.f; }
                            }
                            dz0 = fmaf(dA0[r], nA[r], fmaf(dB0[r], nB[r], dz0));
                            dz1 = fmaf(dA1[r], nA[r], fmaf(dB1[r], nB[r], dz1));
                        }
                        const Frag<T> b0 = pack_frag<T>(dA0, dB0), b1 = pack_frag<T>(dA1, dB1);
#pragma unroll
                        for (int db = 0; db < DB; ++db) {
                            const Frag<T> a = load_frag(Vc + ((size_t)lt * D + 16 * db + i16) * LDC + 32 * s + 8 * g);
                            X0[db] = mma(a, b0, X0[db]);
                            X1[db] = mma(a, b1, X1[db]);
                        }
                    }
                }
            };
            if (partial) correct(std::true_type{});
            else correct(std::false_type{});
        }

        // ---- Y = X / Z
        const float Z0 = Zf0 + xgroup_sum(dz0), Z1 = Zf1 + xgroup_sum(dz1);
        if (v0) {
            const float rz = 1.0f / Z0;
            T *yr = Yh + (size_t)q0 * D + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) yr[16 * db + r] = from_float<T>(X0[db][r] * rz);
        }
        if (v1) {
            const float rz = 1.0f / Z1;
            T *yr = Yh + (size_t)q1 * D + 4 * g;
#pragma unroll
            for (int db = 0; db < DB; ++db)
#pragma unroll
                for (int r = 0; r < 4; ++r) yr[16 * db + r] = from_float<T>(X1[db][r] * rz);
        }
        __syncthreads();   // child buffers / Wp free for the next step
    }
}

// ---------------------------------------------------------------------------

// (children per tile per chunk, tiles staged together): all tiles of a step
// with the largest chunk that fits, else fewer tiles at a time
template <typename T, int D, bool VT>
static bool choose_chunk_t(int M0, int C, int P, int tile, int *chk_out, int *tpg_out)
{
    const int PC = P * C;
    const int want = PC > 64 ? 128 : PC > 32 ? 64 : 32;
    for (int tpg = kStep / tile; tpg >= 1; tpg /= 2)
        for (int chk = want; chk >= 32; chk /= 2)
            if (attn_lds<T, D, VT>(M0, P, tile, chk, tpg).total <= 160 * 1024) {
                *chk_out = chk;
                *tpg_out = tpg;
                return true;
            }
    return false;
}

int attention_child_chunk(int d, int M0, int C, int P, int tile, int dtype)
{
    if (tile != 32 && tile != 64 && tile != 128 && tile != 256) return 0;
    int chk = 0, tpg = 0;
    bool ok;
    if (dtype == 1) ok = d == 64 ? choose_chunk_t<bf16, 64, true>(M0, C, P, tile, &chk, &tpg)
                                 : choose_chunk_t<bf16, 128, false>(M0, C, P, tile, &chk, &tpg);
    else ok = d == 64 ? choose_chunk_t<float, 64, true>(M0, C, P, tile, &chk, &tpg)
                      : choose_chunk_t<float, 128, false>(M0, C, P, tile, &chk, &tpg);
    return ok ? chk : 0;
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

template <typename T, int D, bool VT, int NRB, int CC>
static hipError_t launch_attn_k(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int M0, int P, int tile,
                                int chk, int tpg, size_t lds, float scale, void *Y, int32_t *sel,
                                float *imp, hipStream_t stream)
{
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void *)attention_kernel<T, D, VT, NRB, CC>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr = true;
    }
    const int ntiles = (N + tile - 1) / tile;
    const int nsteps = (N + kStep - 1) / kStep;
    const int BH = B * H;
    const int per_bh = max(1, min(nsteps, (device_cus() + BH - 1) / BH));
    hipLaunchKernelGGL((attention_kernel<T, D, VT, NRB, CC>), dim3(per_bh, BH), dim3(kThreads), lds,
                       stream, (const T *)Q, (const T *)parents, (const T *)children,
                       (const unsigned char *)pack, H, N, M0, CC, ilog2(CC), P, tile, chk, ilog2(chk),
                       tpg, fabsf(scale) * kLog2e, scale < 0.f ? 1 : 0, ntiles, nsteps, (T *)Y, sel, imp);
    return hipGetLastError();
}

template <typename T, int D, bool VT, int NRB>
static hipError_t launch_attn_nrb(const void *Q, const void *parents, const void *children,
                                  const void *pack, int B, int H, int N, int M0, int C, int P,
                                  int tile, int chk, int tpg, size_t lds, float scale, void *Y,
                                  int32_t *sel, float *imp, hipStream_t stream)
{
    switch (C) {
    case 2: return launch_attn_k<T, D, VT, NRB, 2>(Q, parents, children, pack, B, H, N, M0, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    case 4: return launch_attn_k<T, D, VT, NRB, 4>(Q, parents, children, pack, B, H, N, M0, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    case 8: return launch_attn_k<T, D, VT, NRB, 8>(Q, parents, children, pack, B, H, N, M0, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    default: return launch_attn_k<T, D, VT, NRB, 16>(Q, parents, children, pack, B, H, N, M0, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    }
}

template <typename T, int D, bool VT>
static hipError_t launch_attn_t(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int M0, int C, int P, int tile,
                                float scale, void *Y, int32_t *sel, float *imp, hipStream_t stream)
{
    int chk = 0, tpg = 0;
    if (!choose_chunk_t<T, D, VT>(M0, C, P, tile, &chk, &tpg)) return hipErrorInvalidConfiguration;
    const size_t lds = attn_lds<T, D, VT>(M0, P, tile, chk, tpg).total;
    switch (padded_parents(M0)) {
    case 32: return launch_attn_nrb<T, D, VT, 2>(Q, parents, children, pack, B, H, N, M0, C, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    case 64: return launch_attn_nrb<T, D, VT, 4>(Q, parents, children, pack, B, H, N, M0, C, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    case 128: return launch_attn_nrb<T, D, VT, 8>(Q, parents, children, pack, B, H, N, M0, C, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    default: return launch_attn_nrb<T, D, VT, 16>(Q, parents, children, pack, B, H, N, M0, C, P, tile, chk, tpg, lds, scale, Y, sel, imp, stream);
    }
}

hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const void *pack, int B, int H, int N, int d, int M0, int C, int P,
                                int tile, float scale, int dtype, void *Y, int32_t *sel,
                                float *importance, hipStream_t stream)
{
    if (dtype == 1) {
        if (d == 64)
            return launch_attn_t<bf16, 64, true>(Q, parents, children, pack, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
        return launch_attn_t<bf16, 128, false>(Q, parents, children, pack, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
    }
    if (d == 64)
        return launch_attn_t<float, 64, true>(Q, parents, children, pack, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
    return launch_attn_t<float, 128, false>(Q, parents, children, pack, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
}

}  // namespace avq
