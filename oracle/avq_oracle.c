/*
 * CPU oracle for the AVQ-Attention forward pass ("AVQ-Attention: Adaptive
 * Vector-Quantized Attention", Sec. 3-4).
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this code.  The GPU library
 * never links it, includes it or shares any helper with it.
 *
 * Plain, slow and written to be checked by eye against the pages: every
 * quantity is computed in float64 straight from its definition, one (batch,
 * head) unit at a time, single-threaded.  Inputs are float64 arrays holding
 * the exact values of the stored bf16/fp32 tensors.
 *
 * Readings taken where the pages are silent (each also listed in the design doc):
 *  - argmin ties go to the lowest index; a child replaces the parent only if
 *    it is strictly closer;
 *  - top-P orders parents by importance descending, then index ascending;
 *  - query tiles are contiguous index ranges of T queries, the last may be
 *    shorter;
 *  - the importance uses the final parent-level denominator of each query;
 *  - the softmax scale is an explicit argument (the pages write exp(q.k)).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ */
/* storage rounding                                                    */
/* ------------------------------------------------------------------ */

/* Nearest bf16 value to x (8 significant bits, exponent range of fp32),
 * ties to even, returned as a double.  Written from the definition of
 * round-to-nearest-even on the significand. */
double avqo_round_bf16(double x)
{
    if (x == 0.0 || isnan(x) || isinf(x)) return x;
    int e;
    (void)frexp(x, &e);                 /* x = m * 2^e with 0.5 <= |m| < 1 */
    int q = e - 8;                      /* weight of the last kept bit   */
    if (q < -133) q = -133;             /* bf16 subnormal quantum 2^-133 */
    double scaled = ldexp(x, -q);       /* exact */
    double fl = floor(scaled);
    double diff = scaled - fl;
    double r;
    if (diff > 0.5) r = fl + 1.0;
    else if (diff < 0.5) r = fl;
    else r = (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
    double y = ldexp(r, q);
    if (fabs(y) >= 0x1p128) return copysign(INFINITY, x);
    return y;
}

/* dtype 0 = fp32, 1 = bf16 */
void avqo_round(const double *x, int64_t n, int dtype, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = dtype == 1 ? avqo_round_bf16(x[i]) : (double)(float)x[i];
}

/* ------------------------------------------------------------------ */
/* O1  tree: parent = mean of its children (Sec. 4.1, "Parent-child    */
/*     constraint"); one head.                                         */
/* ------------------------------------------------------------------ */
void avqo_build_tree(const double *children /*[M0][C][d]*/, int M0, int C, int d,
                     int dtype, double *parents /*[M0][d]*/)
{
    for (int p = 0; p < M0; ++p)
        for (int t = 0; t < d; ++t) {
            double s = 0.0;
            for (int c = 0; c < C; ++c) s += children[((int64_t)p * C + c) * d + t];
            double mean = s / C;
            parents[(int64_t)p * d + t] = dtype == 1 ? avqo_round_bf16(mean) : (double)(float)mean;
        }
}

/* squared norm of every row */
void avqo_sqnorm(const double *rows, int64_t nrows, int d, double *out)
{
    for (int64_t r = 0; r < nrows; ++r) {
        double s = 0.0;
        for (int t = 0; t < d; ++t) s += rows[r * d + t] * rows[r * d + t];
        out[r] = s;
    }
}

static double sqdist(const double *a, const double *b, int d)
{
    double s = 0.0;
    for (int t = 0; t < d; ++t) {
        double u = a[t] - b[t];
        s += u * u;
    }
    return s;
}

/* relative gap between the two smallest of n values (0 if fewer than 2) */
static double rel_gap(const double *v, int n)
{
    if (n < 2) return INFINITY;
    double a = INFINITY, b = INFINITY;
    for (int i = 0; i < n; ++i) {
        if (v[i] < a) { b = a; a = v[i]; }
        else if (v[i] < b) b = v[i];
    }
    if (b == 0.0) return 0.0;
    return (b - a) / b;
}

/* ------------------------------------------------------------------ */
/* O2  two-stage assignment (Sec. 3.2 assignment rule; Sec. 4.2: nearest */
/*     parent first, then only that parent's children, reassigned if a  */
/*     child is closer than the cached parent distance).                */
/*     leaf = p* (key stays at its parent) or M0 + p*C + c*.            */
/*     force_child != 0 treats the parent distance as +infinity.        */
/*     C == 0 is flat VQ (Sec. 3.2): the nearest codeword is the leaf.  */
/*     gap_parent: relative top-2 gap over the M0 parents;              */
/*     gap_leaf:   relative top-2 gap over {p*} U children(p*).         */
/* ------------------------------------------------------------------ */
void avqo_assign(const double *K /*[N][d]*/, int64_t N, int d,
                 const double *parents /*[M0][d]*/, const double *children /*[M0][C][d]*/,
                 int M0, int C, int force_child,
                 int32_t *pstar, int32_t *leaf, double *gap_parent, double *gap_leaf)
{
    double *Dp = (double *)malloc(sizeof(double) * (size_t)M0);
    double *Dl = (double *)malloc(sizeof(double) * (size_t)(C + 1));
    for (int64_t k = 0; k < N; ++k) {
        const double *key = K + k * d;
        int best = 0;
        for (int p = 0; p < M0; ++p) {
            Dp[p] = sqdist(key, parents + (int64_t)p * d, d);
            if (Dp[p] < Dp[best]) best = p;
        }
        pstar[k] = best;
        if (gap_parent) gap_parent[k] = rel_gap(Dp, M0);
        if (C == 0) {                   /* flat codebook: the parent is the leaf */
            leaf[k] = best;
            if (gap_leaf) gap_leaf[k] = INFINITY;
            continue;
        }
        int cbest = 0;
        for (int c = 0; c < C; ++c) {
            Dl[c] = sqdist(key, children + ((int64_t)best * C + c) * d, d);
            if (Dl[c] < Dl[cbest]) cbest = c;
        }
        int to_child = force_child || Dl[cbest] < Dp[best];
        leaf[k] = to_child ? M0 + best * C + cbest : best;
        if (gap_leaf) {
            Dl[C] = Dp[best];
            gap_leaf[k] = rel_gap(Dl, force_child ? C : C + 1);
        }
    }
    free(Dp);
    free(Dl);
}

/* ------------------------------------------------------------------ */
/* O3  aggregation (Sec. 4.2 "at each level"; Sec. 4.3 value sums and   */
/*     counts).  Slot p holds every key whose nearest parent is p; slot */
/*     M0 + p*C + c holds only the keys reassigned to that child.       */
/* ------------------------------------------------------------------ */
void avqo_aggregate(const double *V /*[N][d]*/, int64_t N, int d, const int32_t *leaf,
                    int M0, int C, double *vsum /*[M0(1+C)][d]*/, int64_t *count)
{
    int64_t S = (int64_t)M0 * (1 + C);
    memset(vsum, 0, sizeof(double) * (size_t)(S * d));
    memset(count, 0, sizeof(int64_t) * (size_t)S);
    for (int64_t k = 0; k < N; ++k) {
        int32_t l = leaf[k];
        int32_t p = l < M0 ? l : (l - M0) / C;
        for (int t = 0; t < d; ++t) vsum[(int64_t)p * d + t] += V[k * d + t];
        count[p] += 1;
        if (l >= M0) {
            for (int t = 0; t < d; ++t) vsum[(int64_t)l * d + t] += V[k * d + t];
            count[l] += 1;
        }
    }
}

/* ------------------------------------------------------------------ */
/* O4-O8  attention of every query over the tree, tile by tile          */
/*   O4 parent pass   (Sec. 4.3 "Tiled VQ-attention")                   */
/*   O5 importance    (Sec. 4.3 "Codeword importance")                  */
/*   O6 top-P         (Sec. 4.3 "Child spawning")                       */
/*   O7 correction    (Sec. 4.3 "Child attention": parent logit as the  */
/*                     mean of child logits; the parent weight of each  */
/*                     reassigned subset is replaced by the child       */
/*                     weight, exp(S_ic) - exp(S_ip), one shared shift) */
/*   O8 Y = X / Z                                                       */
/* Tiles [t_begin, t_end) only; Y rows of other tiles are untouched.    */
/* forced_sel (nullable, [ntiles][P]) replaces O6's choice.             */
/* Returns 0, or -1 on allocation failure.                              */
/* ------------------------------------------------------------------ */
typedef struct { double w; int idx; } wi_pair;
static int cmp_pair(const void *a, const void *b)
{
    const wi_pair *x = (const wi_pair *)a, *y = (const wi_pair *)b;
    if (x->w > y->w) return -1;
    if (x->w < y->w) return 1;
    return x->idx < y->idx ? -1 : (x->idx > y->idx ? 1 : 0);
}

int avqo_attention(const double *Q /*[N][d]*/, int64_t N, int d,
                   const double *parents /*[M0][d]*/, const double *children /*[M0][C][d]*/,
                   int M0, int C, const double *vsum /*[M0(1+C)][d]*/, const int64_t *count,
                   int P, int T, double scale, const int32_t *forced_sel,
                   int64_t t_begin, int64_t t_end,
                   double *Y /*[N][d]*/, double *importance /*[ntiles][M0]*/, int32_t *sel /*[ntiles][P]*/)
{
    double *E = (double *)malloc(sizeof(double) * (size_t)T * M0);
    double *m = (double *)malloc(sizeof(double) * (size_t)T);
    double *Z = (double *)malloc(sizeof(double) * (size_t)T);
    double *X = (double *)malloc(sizeof(double) * (size_t)T * d);
    double *s = (double *)malloc(sizeof(double) * (size_t)(M0 > C ? M0 : C));
    double *w = (double *)malloc(sizeof(double) * (size_t)M0);
    wi_pair *order = (wi_pair *)malloc(sizeof(wi_pair) * (size_t)M0);
    int32_t *chosen = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    if (!E || !m || !Z || !X || !s || !w || !order || !chosen) {
        free(E); free(m); free(Z); free(X); free(s); free(w); free(order); free(chosen);
        return -1;
    }

    for (int64_t t = t_begin; t < t_end; ++t) {
        int64_t i0 = t * T;
        int64_t i1 = i0 + T < N ? i0 + T : N;
        int nI = (int)(i1 - i0);

        /* O4 */
        for (int ii = 0; ii < nI; ++ii) {
            const double *q = Q + (i0 + ii) * d;
            double mx = -INFINITY;
            for (int j = 0; j < M0; ++j) {
                double dot = 0.0;
                for (int u = 0; u < d; ++u) dot += q[u] * parents[(int64_t)j * d + u];
                s[j] = scale * dot;
                if (s[j] > mx) mx = s[j];
            }
            m[ii] = mx;
            double z = 0.0;
            double *x = X + (int64_t)ii * d;
            for (int u = 0; u < d; ++u) x[u] = 0.0;
            for (int j = 0; j < M0; ++j) {
                double e = exp(s[j] - mx);
                E[(int64_t)ii * M0 + j] = e;
                z += e * (double)count[j];
                for (int u = 0; u < d; ++u) x[u] += e * vsum[(int64_t)j * d + u];
            }
            Z[ii] = z;
        }

        /* O5 */
        for (int j = 0; j < M0; ++j) {
            double acc = 0.0;
            for (int ii = 0; ii < nI; ++ii) acc += E[(int64_t)ii * M0 + j] * (double)count[j] / Z[ii];
            w[j] = acc;
            if (importance) importance[t * M0 + j] = acc;
        }

        /* O6 */
        if (forced_sel) {
            for (int k = 0; k < P; ++k) chosen[k] = forced_sel[t * P + k];
        } else {
            for (int j = 0; j < M0; ++j) { order[j].w = w[j]; order[j].idx = j; }
            qsort(order, (size_t)M0, sizeof(wi_pair), cmp_pair);
            for (int k = 0; k < P; ++k) chosen[k] = order[k].idx;
        }
        if (sel) for (int k = 0; k < P; ++k) sel[t * P + k] = chosen[k];

        /* O7 */
        for (int ii = 0; ii < nI; ++ii) {
            const double *q = Q + (i0 + ii) * d;
            double *x = X + (int64_t)ii * d;
            for (int k = 0; k < P; ++k) {
                int p = chosen[k];
                double mean = 0.0, smax = -INFINITY;
                for (int c = 0; c < C; ++c) {
                    const double *cw = children + ((int64_t)p * C + c) * d;
                    double dot = 0.0;
                    for (int u = 0; u < d; ++u) dot += q[u] * cw[u];
                    s[c] = scale * dot;
                    mean += s[c];
                    if (s[c] > smax) smax = s[c];
                }
                mean /= C;
                if (smax > m[ii]) {
                    double a = exp(m[ii] - smax);
                    for (int u = 0; u < d; ++u) x[u] *= a;
                    Z[ii] *= a;
                    m[ii] = smax;
                }
                double ep = exp(mean - m[ii]);
                for (int c = 0; c < C; ++c) {
                    int64_t slot = (int64_t)M0 + (int64_t)p * C + c;
                    double dA = exp(s[c] - m[ii]) - ep;
                    for (int u = 0; u < d; ++u) x[u] += dA * vsum[slot * d + u];
                    Z[ii] += dA * (double)count[slot];
                }
            }
            /* O8 */
            for (int u = 0; u < d; ++u) Y[(i0 + ii) * d + u] = x[u] / Z[ii];
        }
    }
    free(E); free(m); free(Z); free(X); free(s); free(w); free(order); free(chosen);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Diagnostics the pages report next to the method (Sec. 5.2, appendix  */
/* "Per-layer codebook analysis" and "Codebook utilization").           */
/* ------------------------------------------------------------------ */

/* Commitment loss E[||k - k_hat||^2]: the mean over the N keys of the
 * squared distance between each key and the codeword it is assigned to,
 * its leaf (child, or the parent itself; the codeword for a flat
 * codebook, C == 0).  Independent of P. */
double avqo_commitment(const double *K /*[N][d]*/, int64_t N, int d, const double *parents /*[M0][d]*/,
                       const double *children /*[M0][C][d]*/, int M0, int C, const int32_t *leaf)
{
    double s = 0.0;
    for (int64_t k = 0; k < N; ++k) {
        const int32_t l = leaf[k];
        const double *cw = l < M0 ? parents + (int64_t)l * d : children + (int64_t)(l - M0) * d;
        s += sqdist(K + k * d, cw, d);
    }
    return N > 0 ? s / (double)N : 0.0;
}

/* Active ratio: the fraction of the S codewords whose count exceeds
 * `share` times the fair-share count N / S (the pages use 1 %). */
double avqo_active_ratio(const int64_t *count, int S, int64_t N, double share)
{
    const double thresh = share * (double)N / (double)S;
    int active = 0;
    for (int j = 0; j < S; ++j) active += (double)count[j] > thresh;
    return (double)active / (double)S;
}

/* Capture of every query: the fraction of its exact softmax attention
 * weight (scale * q.k over all N keys) that falls on keys whose parent
 * (pstar) is among its tile's P selected parents (sel [ntiles][P], tiles
 * of T consecutive queries).  Returns 0, or -1 on allocation failure. */
int avqo_capture(const double *Q /*[N][d]*/, const double *K /*[N][d]*/, int64_t N, int d,
                 const int32_t *pstar, const int32_t *sel, int P, int T, double scale, int M0,
                 double *capture /*[N]*/)
{
    double *s = (double *)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    char *chosen = (char *)malloc((size_t)(M0 > 0 ? M0 : 1));
    if (!s || !chosen) { free(s); free(chosen); return -1; }
    for (int64_t i = 0; i < N; ++i) {
        const int64_t t = i / T;
        memset(chosen, 0, (size_t)M0);
        for (int k = 0; k < P; ++k) chosen[sel[t * P + k]] = 1;
        double mx = -INFINITY;
        for (int64_t k = 0; k < N; ++k) {
            double dot = 0.0;
            for (int u = 0; u < d; ++u) dot += Q[i * d + u] * K[k * d + u];
            s[k] = scale * dot;
            if (s[k] > mx) mx = s[k];
        }
        double all = 0.0, on_sel = 0.0;
        for (int64_t k = 0; k < N; ++k) {
            const double e = exp(s[k] - mx);
            all += e;
            if (chosen[pstar[k]]) on_sel += e;
        }
        capture[i] = on_sel / all;
    }
    free(s);
    free(chosen);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Token order along the generalized Hilbert ("Gilbert") curve of a W x H */
/* grid (Sec. 4.2: tokens are reordered so that contiguous query tiles   */
/* are compact 2D regions; ref. [4]).  The curve covers a rectangle      */
/* spanned by a major axis vector a and a minor axis vector b, starting  */
/* at its corner (x, y) and ending at the far end of a:                  */
/*  - a rectangle one cell thick is walked straight;                     */
/*  - a rectangle much longer than wide (2|a| > 3|b|) is cut across a     */
/*    into two halves (the first kept even), each walked the same way;   */
/*  - otherwise it is cut into three: a first piece along half of b      */
/*    (axes swapped), a middle piece over the rest of b with the full a, */
/*    and a last piece walked back along -b towards the end of a, so the */
/*    three join end to start.                                           */
/* order[i] receives y*W + x of the i-th cell.                            */
/* ------------------------------------------------------------------ */
static int sgn(int v) { return (v > 0) - (v < 0); }
static int fdiv2(int v) { return v >= 0 ? v / 2 : -((-v + 1) / 2); }   /* floor(v / 2) */

static void gilbert_walk(int x, int y, int ax, int ay, int bx, int by, int W, int32_t *order, int64_t *n)
{
    const int w = abs(ax + ay), h = abs(bx + by);
    const int dax = sgn(ax), day = sgn(ay), dbx = sgn(bx), dby = sgn(by);
    if (h == 1) {
        for (int i = 0; i < w; ++i) order[(*n)++] = (y + i * day) * W + (x + i * dax);
        return;
    }
    if (w == 1) {
        for (int i = 0; i < h; ++i) order[(*n)++] = (y + i * dby) * W + (x + i * dbx);
        return;
    }
    int ax2 = fdiv2(ax), ay2 = fdiv2(ay), bx2 = fdiv2(bx), by2 = fdiv2(by);
    const int w2 = abs(ax2 + ay2), h2 = abs(bx2 + by2);
    if (2 * w > 3 * h) {
        if ((w2 & 1) && w > 2) { ax2 += dax; ay2 += day; }
        gilbert_walk(x, y, ax2, ay2, bx, by, W, order, n);
        gilbert_walk(x + ax2, y + ay2, ax - ax2, ay - ay2, bx, by, W, order, n);
    } else {
        if ((h2 & 1) && h > 2) { bx2 += dbx; by2 += dby; }
        gilbert_walk(x, y, bx2, by2, ax2, ay2, W, order, n);
        gilbert_walk(x + bx2, y + by2, ax, ay, bx - bx2, by - by2, W, order, n);
        gilbert_walk(x + (ax - dax) + (bx2 - dbx), y + (ay - day) + (by2 - dby), -bx2, -by2,
                     -(ax - ax2), -(ay - ay2), W, order, n);
    }
}

void avqo_gilbert_order(int W, int H, int32_t *order /*[W*H]*/)
{
    int64_t n = 0;
    if (W >= H) gilbert_walk(0, 0, W, 0, 0, H, W, order, &n);
    else gilbert_walk(0, 0, 0, H, W, 0, W, order, &n);
}
