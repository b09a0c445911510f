// Token reordering along the generalized Hilbert ("Gilbert") curve
// ("AVQ-Attention", Sec. 4.2 and the spatial reordering ablation, Table 8;
// ref. [4]): queries sharing a tile share a refinement decision, so tokens
// of an image grid are put in curve order, which makes every run of
// consecutive tokens a compact 2D region for any tile size.
//
// The order is a one-time layout computation per grid shape (host code);
// moving Q, K, V into it and Y back out is a gather / scatter of rows on the
// GPU, pure HBM traffic.
#include <stdlib.h>

#include <vector>

#include "avq_kernels.h"

namespace avq {

namespace {

int sign_of(int v) { return (v > 0) - (v < 0); }
int half_floor(int v) { return v >= 0 ? v / 2 : -((1 - v) / 2); }

// A rectangle of the curve: corner (x, y), major axis (ax, ay), minor axis
// (bx, by).  Its cells are emitted from the corner to the far end of the
// major axis.
struct Span {
    int x, y, ax, ay, bx, by;
};

}  // namespace

// Cells of a W x H grid (row-major index y*W + x) in curve order.  The
// curve over a span is: a straight walk when the span is one cell thick;
// two halves along the major axis when the span is long (2|a| > 3|b|, the
// first half kept even); otherwise three pieces -- along the first half of
// the minor axis with the axes swapped, across the rest of the minor axis
// with the full major axis, and back along the negated minor axis to the
// end of the major axis.  Pieces are processed depth first with an explicit
// stack (last pushed = next walked).
void gilbert_cells(int W, int H, int32_t *out)
{
    std::vector<Span> todo;
    todo.push_back(W >= H ? Span{0, 0, W, 0, 0, H} : Span{0, 0, 0, H, W, 0});
    int64_t n = 0;
    while (!todo.empty()) {
        const Span s = todo.back();
        todo.pop_back();
        const int len_a = abs(s.ax + s.ay), len_b = abs(s.bx + s.by);
        const int ua = sign_of(s.ax), va = sign_of(s.ay), ub = sign_of(s.bx), vb = sign_of(s.by);
        if (len_b == 1 || len_a == 1) {   // one cell thick: walk along the longer axis
            const int len = len_b == 1 ? len_a : len_b;
            const int ux = len_b == 1 ? ua : ub, vy = len_b == 1 ? va : vb;
            for (int i = 0; i < len; ++i) out[n++] = (s.y + i * vy) * W + (s.x + i * ux);
            continue;
        }
        int hax = half_floor(s.ax), hay = half_floor(s.ay), hbx = half_floor(s.bx), hby = half_floor(s.by);
        if (2 * len_a > 3 * len_b) {
            if ((abs(hax + hay) & 1) && len_a > 2) {
                hax += ua;
                hay += va;
            }
            // second half pushed first, so the first half is walked first
            todo.push_back(Span{s.x + hax, s.y + hay, s.ax - hax, s.ay - hay, s.bx, s.by});
            todo.push_back(Span{s.x, s.y, hax, hay, s.bx, s.by});
        } else {
            if ((abs(hbx + hby) & 1) && len_b > 2) {
                hbx += ub;
                hby += vb;
            }
            todo.push_back(Span{s.x + (s.ax - ua) + (hbx - ub), s.y + (s.ay - va) + (hby - vb), -hbx, -hby,
                                -(s.ax - hax), -(s.ay - hay)});
            todo.push_back(Span{s.x + hbx, s.y + hby, s.ax, s.ay, s.bx - hbx, s.by - hby});
            todo.push_back(Span{s.x, s.y, hbx, hby, hax, hay});
        }
    }
}

// row gather (dst row i = src row order[i]) or scatter (dst row order[i] =
// src row i) of 16-byte words; order entries outside [0, N) are skipped
__global__ __launch_bounds__(256) void permute_rows_kernel(const uint4 *__restrict__ src, const int32_t *__restrict__ order,
                                                           int64_t rows, int N, int words, int inverse,
                                                           uint4 *__restrict__ dst)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= rows * words) return;
    const int64_t r = i / words;
    const int w = (int)(i % words);
    const int64_t bh = r / N;
    const int t = (int)(r % N);
    const int j = order[t];
    if (j < 0 || j >= N) return;
    if (inverse)
        dst[(bh * N + j) * words + w] = src[r * words + w];
    else
        dst[r * words + w] = src[(bh * N + j) * words + w];
}

hipError_t launch_permute_rows(const void *src, const int32_t *order, int64_t rows, int N, int row_bytes,
                               int inverse, void *dst, hipStream_t stream)
{
    const int words = row_bytes / 16;
    const int64_t n = rows * words;
    hipLaunchKernelGGL(permute_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       (const uint4 *)src, order, rows, N, words, inverse, (uint4 *)dst);
    return hipGetLastError();
}

}  // namespace avq
