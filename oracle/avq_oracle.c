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
 * Readings taken where the pages are silent:
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

/* ------------------------------------------------------------------ */
/* Three-level tree (Sec. 6 "Discussion and Conclusion": a deeper       */
/* hierarchy adds P*C codes per extra level).  The pages propose it and */
/* give no algorithm; the readings taken here:                       */
/*  - leaves L[p][a][b] are given; level 1 c[p][a] is the mean of its C  */
/*    leaves and the root r[p] the mean of its C*C leaves (the mean      */
/*    constraint at every level), each rounded once to the storage type; */
/*  - assignment descends one level at a time: nearest root, then that   */
/*    root's children (taken if strictly closer than the root), then     */
/*    that child's leaves (taken if strictly closer than the child);     */
/*  - every slot holds its whole cell: root p all keys under p, child    */
/*    (p, a) all keys that reached it (including those that went on to a */
/*    leaf), leaf slots the keys assigned there;                         */
/*  - stage 2 repeats importance, top-P and correction once per level:   */
/*    level-1 importance w_c = n_c sum_i exp(S_ic)/Z1_i over the P*C      */
/*    children of the selected roots, Z1 the denominator after the       */
/*    level-1 correction; the top P children (ties to the lower child     */
/*    index) have their logits recovered as the mean of their leaves'   */
/*    logits and are replaced by their leaves as in O7.                  */
/* Slot layout per head: [0, M0) roots, [M0, M0 + M0*C) children         */
/* (p*C + a), [M0 + M0*C, M0 + M0*C + M0*C*C) leaves ((p*C + a)*C + b).   */
/* ------------------------------------------------------------------ */
void avqo_build_tree3(const double *leaves /*[M0][C][C][d]*/, int M0, int C, int d, int dtype,
                      double *level1 /*[M0][C][d]*/, double *level0 /*[M0][d]*/)
{
    for (int p = 0; p < M0; ++p)
        for (int t = 0; t < d; ++t) {
            double all = 0.0;
            for (int a = 0; a < C; ++a) {
                double s = 0.0;
                for (int b = 0; b < C; ++b) s += leaves[(((int64_t)p * C + a) * C + b) * d + t];
                all += s;
                double mean = s / C;
                level1[((int64_t)p * C + a) * d + t] = dtype == 1 ? avqo_round_bf16(mean) : (double)(float)mean;
            }
            double mean = all / ((double)C * C);
            level0[(int64_t)p * d + t] = dtype == 1 ? avqo_round_bf16(mean) : (double)(float)mean;
        }
}

/* gap0: relative top-2 gap over the roots; gap1: over {p*} U children(p*);
 * gap2: over {(p*, a*)} U leaves(p*, a*) when the key reached a child,
 * +infinity otherwise.  force_child != 0 treats the distance to the level
 * above as +infinity at both steps. */
void avqo_assign3(const double *K /*[N][d]*/, int64_t N, int d, const double *level0 /*[M0][d]*/,
                  const double *level1 /*[M0][C][d]*/, const double *leaves /*[M0][C][C][d]*/,
                  int M0, int C, int force_child, int32_t *pstar, int32_t *leaf,
                  double *gap0, double *gap1, double *gap2)
{
    double *Dp = (double *)malloc(sizeof(double) * (size_t)M0);
    double *Dl = (double *)malloc(sizeof(double) * (size_t)(C + 1));
    double *Dg = (double *)malloc(sizeof(double) * (size_t)(C + 1));
    for (int64_t k = 0; k < N; ++k) {
        const double *key = K + k * d;
        int best = 0;
        for (int p = 0; p < M0; ++p) {
            Dp[p] = sqdist(key, level0 + (int64_t)p * d, d);
            if (Dp[p] < Dp[best]) best = p;
        }
        pstar[k] = best;
        if (gap0) gap0[k] = rel_gap(Dp, M0);
        int a = 0;
        for (int c = 0; c < C; ++c) {
            Dl[c] = sqdist(key, level1 + ((int64_t)best * C + c) * d, d);
            if (Dl[c] < Dl[a]) a = c;
        }
        const int to_child = force_child || Dl[a] < Dp[best];
        if (gap1) {
            Dl[C] = Dp[best];
            gap1[k] = rel_gap(Dl, force_child ? C : C + 1);
        }
        if (!to_child) {
            leaf[k] = best;
            if (gap2) gap2[k] = INFINITY;
            continue;
        }
        const int64_t ci = (int64_t)best * C + a;   /* child index */
        int b = 0;
        for (int g = 0; g < C; ++g) {
            Dg[g] = sqdist(key, leaves + (ci * C + g) * d, d);
            if (Dg[g] < Dg[b]) b = g;
        }
        const int to_leaf = force_child || Dg[b] < Dl[a];
        leaf[k] = to_leaf ? (int32_t)(M0 + (int64_t)M0 * C + ci * C + b) : (int32_t)(M0 + ci);
        if (gap2) {
            Dg[C] = Dl[a];
            gap2[k] = rel_gap(Dg, force_child ? C : C + 1);
        }
    }
    free(Dp);
    free(Dl);
    free(Dg);
}

void avqo_aggregate3(const double *V /*[N][d]*/, int64_t N, int d, const int32_t *leaf, int M0, int C,
                     double *vsum /*[S3][d]*/, int64_t *count /*[S3]*/)
{
    const int64_t n1 = (int64_t)M0 * C, S = M0 + n1 + n1 * C;
    memset(vsum, 0, sizeof(double) * (size_t)(S * d));
    memset(count, 0, sizeof(int64_t) * (size_t)S);
    for (int64_t k = 0; k < N; ++k) {
        const int64_t l = leaf[k];
        int64_t slots[3];
        int ns = 0;
        if (l < M0) {
            slots[ns++] = l;
        } else if (l < M0 + n1) {
            slots[ns++] = (l - M0) / C;
            slots[ns++] = l;
        } else {
            const int64_t ci = (l - M0 - n1) / C;
            slots[ns++] = ci / C;
            slots[ns++] = M0 + ci;
            slots[ns++] = l;
        }
        for (int s = 0; s < ns; ++s) {
            for (int t = 0; t < d; ++t) vsum[slots[s] * d + t] += V[k * d + t];
            count[slots[s]] += 1;
        }
    }
}

/* one refinement level for query row q: the `nsel` codewords `sel` of the
 * level above (codeword j's C children at rows j*C .. j*C+C-1 of `kids`,
 * their slots at slot0 + j*C + c) are replaced by their children, the
 * parent logit recovered as the mean of the children's logits (O7).
 * Child logits are written to s_out[k*C + c] when s_out is not null. */
static void correct_level(const double *q, int d, double scale, const int32_t *sel, int nsel,
                          const double *kids, int C, int64_t slot0, const double *vsum,
                          const int64_t *count, double *x, double *Z, double *m, double *s,
                          double *s_out)
{
    for (int k = 0; k < nsel; ++k) {
        const int64_t j = sel[k];
        double mean = 0.0, smax = -INFINITY;
        for (int c = 0; c < C; ++c) {
            const double *cw = kids + (j * C + c) * d;
            double dot = 0.0;
            for (int u = 0; u < d; ++u) dot += q[u] * cw[u];
            s[c] = scale * dot;
            mean += s[c];
            if (s[c] > smax) smax = s[c];
        }
        mean /= C;
        if (smax > *m) {
            const double a = exp(*m - smax);
            for (int u = 0; u < d; ++u) x[u] *= a;
            *Z *= a;
            *m = smax;
        }
        const double ep = exp(mean - *m);
        for (int c = 0; c < C; ++c) {
            const int64_t slot = slot0 + j * C + c;
            const double dA = exp(s[c] - *m) - ep;
            for (int u = 0; u < d; ++u) x[u] += dA * vsum[slot * d + u];
            *Z += dA * (double)count[slot];
            if (s_out) s_out[(int64_t)k * C + c] = s[c];
        }
    }
}

static int cmp_int32(const void *a, const void *b)
{
    const int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Tiles [t_begin, t_end).  imp0 [ntiles][M0] and sel0 [ntiles][P] as in
 * avqo_attention (sel0 in importance order); imp1 [ntiles][P*C] is the
 * level-1 importance of the children of the selected roots listed by
 * ascending child index, sel1 [ntiles][P] the selected children's indices
 * (p*C + a) in ascending order.  forced_sel0 / forced_sel1 (nullable)
 * replace the two choices.  Returns 0, or -1 on allocation failure. */
int avqo_attention3(const double *Q /*[N][d]*/, int64_t N, int d, const double *level0 /*[M0][d]*/,
                    const double *level1 /*[M0][C][d]*/, const double *leaves /*[M0][C][C][d]*/,
                    int M0, int C, const double *vsum /*[S3][d]*/, const int64_t *count, int P, int T,
                    double scale, const int32_t *forced_sel0, const int32_t *forced_sel1,
                    int64_t t_begin, int64_t t_end, double *Y /*[N][d]*/, double *imp0, int32_t *sel0,
                    double *imp1, int32_t *sel1)
{
    const int PC = P * C;
    const int64_t n1 = (int64_t)M0 * C;
    double *E = (double *)malloc(sizeof(double) * (size_t)T * M0);
    double *m = (double *)malloc(sizeof(double) * (size_t)T);
    double *Z = (double *)malloc(sizeof(double) * (size_t)T);
    double *X = (double *)malloc(sizeof(double) * (size_t)T * d);
    double *s = (double *)malloc(sizeof(double) * (size_t)(M0 > C ? M0 : C));
    double *S1 = (double *)malloc(sizeof(double) * (size_t)T * (PC > 0 ? PC : 1));
    double *w = (double *)malloc(sizeof(double) * (size_t)(M0 > PC ? M0 : (PC > 0 ? PC : 1)));
    wi_pair *order = (wi_pair *)malloc(sizeof(wi_pair) * (size_t)(M0 > PC ? M0 : (PC > 0 ? PC : 1)));
    int32_t *ch0 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    int32_t *ch1 = (int32_t *)malloc(sizeof(int32_t) * (size_t)(P > 0 ? P : 1));
    if (!E || !m || !Z || !X || !s || !S1 || !w || !order || !ch0 || !ch1) {
        free(E); free(m); free(Z); free(X); free(s); free(S1); free(w); free(order); free(ch0); free(ch1);
        return -1;
    }
    for (int64_t t = t_begin; t < t_end; ++t) {
        const int64_t i0 = t * T, i1 = i0 + T < N ? i0 + T : N;
        const int nI = (int)(i1 - i0);

        /* O4: parent pass over the roots */
        for (int ii = 0; ii < nI; ++ii) {
            const double *q = Q + (i0 + ii) * d;
            double mx = -INFINITY;
            for (int j = 0; j < M0; ++j) {
                double dot = 0.0;
                for (int u = 0; u < d; ++u) dot += q[u] * level0[(int64_t)j * d + u];
                s[j] = scale * dot;
                if (s[j] > mx) mx = s[j];
            }
            m[ii] = mx;
            double z = 0.0, *x = X + (int64_t)ii * d;
            for (int u = 0; u < d; ++u) x[u] = 0.0;
            for (int j = 0; j < M0; ++j) {
                const double e = exp(s[j] - mx);
                E[(int64_t)ii * M0 + j] = e;
                z += e * (double)count[j];
                for (int u = 0; u < d; ++u) x[u] += e * vsum[(int64_t)j * d + u];
            }
            Z[ii] = z;
        }
        /* O5, O6 at the roots */
        for (int j = 0; j < M0; ++j) {
            double acc = 0.0;
            for (int ii = 0; ii < nI; ++ii) acc += E[(int64_t)ii * M0 + j] * (double)count[j] / Z[ii];
            w[j] = acc;
            if (imp0) imp0[t * M0 + j] = acc;
        }
        if (forced_sel0) {
            for (int k = 0; k < P; ++k) ch0[k] = forced_sel0[t * P + k];
        } else {
            for (int j = 0; j < M0; ++j) { order[j].w = w[j]; order[j].idx = j; }
            qsort(order, (size_t)M0, sizeof(wi_pair), cmp_pair);
            for (int k = 0; k < P; ++k) ch0[k] = order[k].idx;
        }
        if (sel0) for (int k = 0; k < P; ++k) sel0[t * P + k] = ch0[k];
        /* candidates of level 1: children of the selected roots by ascending index */
        qsort(ch0, (size_t)P, sizeof(int32_t), cmp_int32);

        /* O7 at level 1 (roots -> children), child logits kept */
        for (int ii = 0; ii < nI; ++ii)
            correct_level(Q + (i0 + ii) * d, d, scale, ch0, P, level1, C, M0, vsum, count,
                          X + (int64_t)ii * d, &Z[ii], &m[ii], s, S1 + (int64_t)ii * PC);

        /* level-1 importance over the P*C candidates, then top-P */
        for (int k = 0; k < PC; ++k) {
            const int64_t ci = (int64_t)ch0[k / C] * C + k % C;
            double acc = 0.0;
            for (int ii = 0; ii < nI; ++ii)
                acc += exp(S1[(int64_t)ii * PC + k] - m[ii]) * (double)count[M0 + ci] / Z[ii];
            w[k] = acc;
            if (imp1) imp1[t * PC + k] = acc;
        }
        if (forced_sel1) {
            for (int k = 0; k < P; ++k) ch1[k] = forced_sel1[t * P + k];
        } else {
            for (int k = 0; k < PC; ++k) { order[k].w = w[k]; order[k].idx = (int)((int64_t)ch0[k / C] * C + k % C); }
            qsort(order, (size_t)PC, sizeof(wi_pair), cmp_pair);
            for (int k = 0; k < P; ++k) ch1[k] = order[k].idx;
        }
        qsort(ch1, (size_t)P, sizeof(int32_t), cmp_int32);
        if (sel1) for (int k = 0; k < P; ++k) sel1[t * P + k] = ch1[k];

        /* O7 at level 2 (children -> leaves), then O8 */
        for (int ii = 0; ii < nI; ++ii) {
            double *x = X + (int64_t)ii * d;
            correct_level(Q + (i0 + ii) * d, d, scale, ch1, P, leaves, C, M0 + n1, vsum, count, x,
                          &Z[ii], &m[ii], s, NULL);
            for (int u = 0; u < d; ++u) Y[(i0 + ii) * d + u] = x[u] / Z[ii];
        }
    }
    free(E); free(m); free(Z); free(X); free(s); free(S1); free(w); free(order); free(ch0); free(ch1);
    return 0;
}
