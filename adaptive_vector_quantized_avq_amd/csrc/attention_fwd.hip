// Stage 2 of the AVQ-Attention forward pass: query-tile adaptive attention
// ("AVQ-Attention", Sec. 4.3).
//
// One work-group per (query tile, batch*head); one wave per 16 queries.
// Logits are computed transposed, S^T = C . Q^T (codewords as MFMA rows,
// queries as columns), so that each lane owns one query: the row max and the
// denominators are per-lane sums plus a reduction over the four lane groups,
// and the exponentiated tile E^T is already laid out as the B operand of the
// next contraction X^T += Vbar^T . E^T (the A operand Vbar^T is staged in LDS
// with its contraction index permuted to match, see perm32).
//
// Per tile:
//   parent pass  S^T over the M0 parents (parents in LDS), m = row max,
//                E = exp2((s - m) log2 e), Z = sum E n, X^T = Vbar^T E^T;
//   importance   w_j = n_j sum_i E_ij / Z_i: per-wave row sums over its 16
//                queries, then across waves through LDS;
//   top-P        exact selection by bisection on the fp32 bit patterns of w
//                (w >= 0, so bit order is value order), ties to the lowest
//                index;
//   correction   the P*C children of the selected parents, staged in chunks
//                with their value sums and counts; the recovered parent logit
//                is the mean of each parent's C child logits (Sec. 4.3
//                "Child attention"), the shift m is raised to cover the child
//                logits (X, Z rescaled), and
//                X^T += Vbar_c^T . (exp(S_c - m) - exp(S_p - m))^T,
//                Z += sum (exp(S_c - m) - exp(S_p - m)) n_c;
//   Y = X / Z.
#include "avq_kernels.h"

namespace avq {

constexpr float kLog2e = 1.4426950408889634f;

template <int D> struct ChildChunk {
    static constexpr int value = D == 128 ? 32 : 64;
};

struct AttnLayout {
    size_t ps, vt, np, wimp, sel, child, cs, vct, nc, wp, total;
};

// byte offsets of every LDS region
template <typename T, int D, int NW>
__host__ __device__ inline AttnLayout attn_layout(int M0)
{
    constexpr int CHK = ChildChunk<D>::value;
    const int M0p = round32(M0);
    AttnLayout L;
    size_t o = 0;
    L.ps = o;   o += (size_t)M0p * (D + 8) * sizeof(T);
    L.vt = o;   o += (size_t)D * (M0p + 8) * sizeof(T);
    L.np = o;   o += (size_t)M0p * 4;
    L.wimp = o; o += (size_t)M0p * 4;
    L.sel = o;  o += 256 * 4;
    L.child = o;
    // child staging area, also holding the per-wave importance partials
    // before the child pass starts
    size_t c = 0;
    L.cs = o + c;  c += (size_t)CHK * (D + 8) * sizeof(T);
    L.vct = o + c; c += (size_t)D * (CHK + 8) * sizeof(T);
    L.nc = o + c;  c += (size_t)CHK * 4;
    const size_t wpb = (size_t)NW * M0p * 4;
    L.wp = o;
    o += c > wpb ? c : wpb;
    L.total = o;
    return L;
}

// Exact top-P of w[0..M0) (w >= 0) by wave 0: ties broken toward the lower
// index.  Writes the selected indices in ascending order.
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

template <typename T, int D, int NW>
__global__ __launch_bounds__(64 * NW) void attention_kernel(
    const T *__restrict__ Q, const T *__restrict__ parents, const T *__restrict__ children,
    const float *__restrict__ vsum, const int32_t *__restrict__ count, int H, int N, int M0, int C,
    int P, float sl2, int ntiles, T *__restrict__ Y, int32_t *__restrict__ sel_out,
    float *__restrict__ imp_out)
{
    extern __shared__ __align__(16) unsigned char smem[];
    constexpr int TILE = 16 * NW;
    constexpr int NT = 64 * NW;
    constexpr int KS = D / 32;
    constexpr int DB = D / 16;
    constexpr int LDP = D + 8;
    constexpr int CHK = ChildChunk<D>::value;
    constexpr int LDVC = CHK + 8;
    const AttnLayout L = attn_layout<T, D, NW>(M0);
    const int M0p = round32(M0);
    const int LDV = M0p + 8;
    T *Ps = reinterpret_cast<T *>(smem + L.ps);
    T *Vt = reinterpret_cast<T *>(smem + L.vt);
    float *nP = reinterpret_cast<float *>(smem + L.np);
    float *wimp = reinterpret_cast<float *>(smem + L.wimp);
    int *selL = reinterpret_cast<int *>(smem + L.sel);
    float *Wp = reinterpret_cast<float *>(smem + L.wp);
    T *Cs = reinterpret_cast<T *>(smem + L.cs);
    T *Vct = reinterpret_cast<T *>(smem + L.vct);
    float *nC = reinterpret_cast<float *>(smem + L.nc);

    const int tile = blockIdx.x, bh = blockIdx.y, h = bh % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int g = lane >> 4, i16 = lane & 15;
    const int S = M0 * (1 + C);
    const float *vs = vsum + (int64_t)bh * S * D;
    const int32_t *cn = count + (int64_t)bh * S;

    // ---- stage parents, their value sums (transposed, permuted) and counts
    for (int e = tid * 8; e < M0p * D; e += NT * 8) {
        const int r = e / D, c = e % D;
        Frag<T> f = r < M0 ? load_frag(parents + ((int64_t)h * M0 + r) * D + c) : zero_frag<T>();
        store_frag(Ps + r * LDP + c, f);
    }
    for (int e = tid; e < M0p * (D / 4); e += NT) {
        const int j = e / (D / 4), q4 = e % (D / 4);
        f32x4 v = j < M0 ? *reinterpret_cast<const f32x4 *>(vs + (int64_t)j * D + 4 * q4)
                         : f32x4{0.f, 0.f, 0.f, 0.f};
        const int pos = (j & ~31) + perm32(j & 31);
#pragma unroll
        for (int k = 0; k < 4; ++k) Vt[(4 * q4 + k) * LDV + pos] = from_float<T>(v[k]);
    }
    for (int j = tid; j < M0p; j += NT) nP[j] = j < M0 ? (float)cn[j] : 0.f;
    __syncthreads();

    const int q = tile * TILE + 16 * w + i16;
    const bool qv = q < N;
    Frag<T> qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        qf[ks] = qv ? load_frag(Q + ((int64_t)bh * N + q) * D + 32 * ks + 8 * g) : zero_frag<T>();

    // ---- parent pass
    const int nrb = M0p / 16;
    f32x4 Sx[16];
    float m = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < 16; ++rb) {
        if (rb < nrb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                a = mma(load_frag(Ps + (16 * rb + i16) * LDP + 32 * ks + 8 * g), qf[ks], a);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float x = (16 * rb + 4 * g + r) < M0 ? a[r] * sl2 : -INFINITY;
                a[r] = x;
                m = fmaxf(m, x);
            }
            Sx[rb] = a;
        }
    }
    m = xgroup_max(m);
    float zp = 0.f;
#pragma unroll
    for (int rb = 0; rb < 16; ++rb) {
        if (rb < nrb) {
            const f32x4 nv = *reinterpret_cast<const f32x4 *>(nP + 16 * rb + 4 * g);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float e = exp2f(Sx[rb][r] - m);
                Sx[rb][r] = e;
                zp += e * nv[r];
            }
        }
    }
    float Zf = xgroup_sum(zp);
    const float rq = qv ? 1.0f / Zf : 0.0f;

    // ---- importance partials of this wave's 16 queries
#pragma unroll
    for (int rb = 0; rb < 16; ++rb) {
        if (rb < nrb) {
            f32x4 t;
#pragma unroll
            for (int r = 0; r < 4; ++r) t[r] = row16_sum(Sx[rb][r] * rq);
            if (i16 == rb) *reinterpret_cast<f32x4 *>(Wp + w * M0p + 16 * rb + 4 * g) = t;
        }
    }

    // ---- X^T = Vbar^T E^T over the parents
    f32x4 X[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) X[db] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 8; ++s) {
        if (2 * s < nrb) {
            const Frag<T> bf = pack_frag<T>(Sx[2 * s], Sx[2 * s + 1]);
#pragma unroll
            for (int db = 0; db < DB; ++db)
                X[db] = mma(load_frag(Vt + (16 * db + i16) * LDV + 32 * s + 8 * g), bf, X[db]);
        }
    }
    __syncthreads();

    // ---- tile importance and top-P
    const int64_t trow = (int64_t)bh * ntiles + tile;
    for (int j = tid; j < M0p; j += NT) {
        float s = 0.f;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) s += Wp[ww * M0p + j];
        s *= nP[j];
        wimp[j] = s;
        if (imp_out && j < M0) imp_out[trow * M0 + j] = s;
    }
    __syncthreads();
    if (P > 0) {
        if (w == 0) select_top_p(wimp, M0, P, selL, sel_out ? sel_out + trow * P : nullptr);
        __syncthreads();

        // ---- child pass
        const int nrows = P * C;
        float dz = 0.f;
        for (int c0 = 0; c0 < nrows; c0 += CHK) {
            for (int e = tid * 8; e < CHK * D; e += NT * 8) {
                const int rr = e / D, col = e % D, row = c0 + rr;
                Frag<T> f = row < nrows
                                ? load_frag(children + (((int64_t)h * M0 + selL[row / C]) * C + row % C) * D + col)
                                : zero_frag<T>();
                store_frag(Cs + rr * LDP + col, f);
            }
            for (int e = tid; e < CHK * (D / 4); e += NT) {
                const int rr = e / (D / 4), q4 = e % (D / 4), row = c0 + rr;
                f32x4 v = row < nrows
                              ? *reinterpret_cast<const f32x4 *>(
                                    vs + ((int64_t)M0 + selL[row / C] * C + row % C) * D + 4 * q4)
                              : f32x4{0.f, 0.f, 0.f, 0.f};
                const int pos = (rr & ~31) + perm32(rr & 31);
#pragma unroll
                for (int k = 0; k < 4; ++k) Vct[(4 * q4 + k) * LDVC + pos] = from_float<T>(v[k]);
            }
            for (int rr = tid; rr < CHK; rr += NT) {
                const int row = c0 + rr;
                nC[rr] = row < nrows ? (float)cn[M0 + selL[row / C] * C + row % C] : 0.f;
            }
            __syncthreads();

            f32x4 Sc[CHK / 16];
            float mc = -INFINITY;
#pragma unroll
            for (int rb = 0; rb < CHK / 16; ++rb) {
                f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    a = mma(load_frag(Cs + (16 * rb + i16) * LDP + 32 * ks + 8 * g), qf[ks], a);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float x = (c0 + 16 * rb + 4 * g + r) < nrows ? a[r] * sl2 : -INFINITY;
                    a[r] = x;
                    mc = fmaxf(mc, x);
                }
                Sc[rb] = a;
            }
            mc = xgroup_max(mc);
            // recovered parent logit of every row: mean of its parent's C
            // child logits (rows of one parent are contiguous, C | 16)
            float sp[CHK / 16][2];
#pragma unroll
            for (int rb = 0; rb < CHK / 16; ++rb) {
                if (C == 2) {
                    sp[rb][0] = 0.5f * (Sc[rb][0] + Sc[rb][1]);
                    sp[rb][1] = 0.5f * (Sc[rb][2] + Sc[rb][3]);
                } else {
                    float s4 = (Sc[rb][0] + Sc[rb][1]) + (Sc[rb][2] + Sc[rb][3]);
                    if (C >= 8) s4 += __shfl_xor(s4, 16);
                    if (C >= 16) s4 += __shfl_xor(s4, 32);
                    sp[rb][0] = sp[rb][1] = s4 / (float)C;
                }
            }
            const float mn = fmaxf(m, mc);
            const float alpha = exp2f(m - mn);
            m = mn;
            Zf *= alpha;
            dz *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) X[db] *= alpha;
#pragma unroll
            for (int rb = 0; rb < CHK / 16; ++rb) {
                const f32x4 nv = *reinterpret_cast<const f32x4 *>(nC + 16 * rb + 4 * g);
                const float e0 = exp2f(sp[rb][0] - m);
                const float e1 = C == 2 ? exp2f(sp[rb][1] - m) : e0;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float dA = exp2f(Sc[rb][r] - m) - (r < 2 ? e0 : e1);
                    Sc[rb][r] = dA;
                    dz += dA * nv[r];
                }
            }
#pragma unroll
            for (int s = 0; s < CHK / 32; ++s) {
                const Frag<T> bf = pack_frag<T>(Sc[2 * s], Sc[2 * s + 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    X[db] = mma(load_frag(Vct + (16 * db + i16) * LDVC + 32 * s + 8 * g), bf, X[db]);
            }
            __syncthreads();
        }
        Zf += xgroup_sum(dz);
    }

    // ---- Y = X / Z
    if (qv) {
        const float rz = 1.0f / Zf;
        T *yr = Y + ((int64_t)bh * N + q) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
#pragma unroll
            for (int r = 0; r < 4; ++r) yr[16 * db + 4 * g + r] = from_float<T>(X[db][r] * rz);
        }
    }
}

template <typename T, int D, int NW>
static hipError_t launch_attn_t(const void *Q, const void *parents, const void *children,
                                const float *vsum, const int32_t *count, int B, int H, int N, int M0,
                                int C, int P, float scale, void *Y, int32_t *sel, float *imp,
                                hipStream_t stream)
{
    const AttnLayout L = attn_layout<T, D, NW>(M0);
    if (L.total > 160 * 1024) return hipErrorInvalidConfiguration;
    static bool attr = false;
    if (!attr) {
        (void)hipFuncSetAttribute((const void *)attention_kernel<T, D, NW>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        attr = true;
    }
    const int TILE = 16 * NW;
    const int ntiles = (N + TILE - 1) / TILE;
    hipLaunchKernelGGL((attention_kernel<T, D, NW>), dim3(ntiles, B * H), dim3(64 * NW), L.total,
                       stream, (const T *)Q, (const T *)parents, (const T *)children, vsum, count, H,
                       N, M0, C, P, scale * kLog2e, ntiles, (T *)Y, sel, imp);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_attn_d(const void *Q, const void *parents, const void *children,
                                const float *vsum, const int32_t *count, int B, int H, int N, int M0,
                                int C, int P, int tile, float scale, void *Y, int32_t *sel,
                                float *imp, hipStream_t stream)
{
    switch (tile) {
    case 16: return launch_attn_t<T, D, 1>(Q, parents, children, vsum, count, B, H, N, M0, C, P, scale, Y, sel, imp, stream);
    case 32: return launch_attn_t<T, D, 2>(Q, parents, children, vsum, count, B, H, N, M0, C, P, scale, Y, sel, imp, stream);
    case 64: return launch_attn_t<T, D, 4>(Q, parents, children, vsum, count, B, H, N, M0, C, P, scale, Y, sel, imp, stream);
    case 128: return launch_attn_t<T, D, 8>(Q, parents, children, vsum, count, B, H, N, M0, C, P, scale, Y, sel, imp, stream);
    default: return hipErrorInvalidValue;
    }
}

size_t attention_lds_bytes(int d, int M0, int tile, int dtype)
{
    const int nw = tile / 16;
#define AVQ_L(T, D, NW) attn_layout<T, D, NW>(M0).total
    if (dtype == 1) {
        if (d == 64) return nw == 1 ? AVQ_L(bf16, 64, 1) : nw == 2 ? AVQ_L(bf16, 64, 2) : nw == 4 ? AVQ_L(bf16, 64, 4) : AVQ_L(bf16, 64, 8);
        return nw == 1 ? AVQ_L(bf16, 128, 1) : nw == 2 ? AVQ_L(bf16, 128, 2) : nw == 4 ? AVQ_L(bf16, 128, 4) : AVQ_L(bf16, 128, 8);
    }
    if (d == 64) return nw == 1 ? AVQ_L(float, 64, 1) : nw == 2 ? AVQ_L(float, 64, 2) : nw == 4 ? AVQ_L(float, 64, 4) : AVQ_L(float, 64, 8);
    return nw == 1 ? AVQ_L(float, 128, 1) : nw == 2 ? AVQ_L(float, 128, 2) : nw == 4 ? AVQ_L(float, 128, 4) : AVQ_L(float, 128, 8);
#undef AVQ_L
}

hipError_t launch_attention_fwd(const void *Q, const void *parents, const void *children,
                                const float *vsum, const int32_t *count, int B, int H, int N, int d,
                                int M0, int C, int P, int tile, float scale, int dtype, void *Y,
                                int32_t *sel, float *importance, hipStream_t stream)
{
    if (dtype == 1) {
        if (d == 64)
            return launch_attn_d<bf16, 64>(Q, parents, children, vsum, count, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
        return launch_attn_d<bf16, 128>(Q, parents, children, vsum, count, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
    }
    if (d == 64)
        return launch_attn_d<float, 64>(Q, parents, children, vsum, count, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
    return launch_attn_d<float, 128>(Q, parents, children, vsum, count, B, H, N, M0, C, P, tile, scale, Y, sel, importance, stream);
}

}  // namespace avq
