/*
 * avq.h -- C ABI of the MI355X (gfx950) AVQ-Attention forward pass.
 *
 * Operation: "AVQ-Attention: Adaptive Vector-Quantized Attention"
 * (van den Dool, Forre, Habibian, Asano, Welling), Sec. 4.  The forward pass
 * is two stages (Sec. 4.3 "Summary"):
 *   1. avq_assign_aggregate: assign every key to the frozen parent/child
 *      codebook tree and aggregate per-codeword value sums and counts
 *      (Sec. 4.2).
 *   2. avq_attention_fwd: count-weighted attention over the parents, tile
 *      importance, top-P parents per query tile, and replacement of those
 *      parents' contributions by their children's (Sec. 4.3).
 * avq_build_tree derives the parents from the children once per frozen
 * codebook (Sec. 4.1, parent-child constraint).
 *
 * Conventions for every entry point
 *  - All tensor pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), contiguous, row-major, owned by the caller.  The library keeps
 *    no reference to them after the call returns.
 *  - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *    enqueues work on that stream and returns; nothing synchronises.
 *  - dtype is AVQ_F32 or AVQ_BF16 and applies to every codebook / Q / K / V /
 *    Y tensor of the call.  Value sums are always fp32, counts int32,
 *    squared norms fp32.
 *  - Arguments are validated before anything is enqueued.  A bad argument
 *    returns AVQ_ERR_INVALID_ARG, a valid but unsupported shape returns
 *    AVQ_ERR_UNSUPPORTED; nothing is enqueued in either case.  A failure
 *    reported by the HIP runtime at launch returns AVQ_ERR_HIP.
 *    avq_last_error() gives a message for the last failure on the calling
 *    thread.
 *  - Supported shapes: head dim d in {64, 128}; C in {2, 4, 8, 16} children
 *    per parent, or C = 0 for a flat codebook (plain VQ-attention, Sec.
 *    3.2: no child level, P = 0); 1 <= M0 <= 256 parents; 1 <= N <= 1048576;
 *    query tile in {32, 64, 128, 256} (the pages use tiles of 32 to 128
 *    queries, Table 8).
 *  - Codeword slots: j in [0, M0) is parent j; j = M0 + p*C + c is child c
 *    of parent p.  S_tot = M0 * (1 + C).
 *  - With C = 0 the `children` argument of every call is the flat codebook
 *    [H][M0][d] itself; avq_build_tree copies it to parents_out.
 *  - Calls are stateless and thread-safe; no C++ exception crosses the ABI.
 */
#ifndef AVQ_H
#define AVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVQ_ABI_VERSION 3

enum avq_status {
    AVQ_OK = 0,
    AVQ_ERR_INVALID_ARG = -1,
    AVQ_ERR_UNSUPPORTED = -2,
    AVQ_ERR_HIP = -3
};

enum avq_dtype { AVQ_F32 = 0, AVQ_BF16 = 1 };

/* flags of avq_assign_aggregate */
enum {
    /* Treat the cached parent distance as +infinity in the child step, so
     * every key moves to its nearest child and the children of a parent
     * partition its cell (no residual keys).  Needs C > 0. */
    AVQ_FLAG_FORCE_CHILD = 1,
    /* Flat codebook (C = 0) only: the unfused precomputation the pages
     * compare the fused kernel with (Sec. 4.2, Table 2): the nearest
     * codeword of every key is written to memory (leaf_out if given, else
     * the workspace), then a separate pass adds values and counts with
     * global atomics.  Same results; the fp32 summation order then depends
     * on scheduling. */
    AVQ_FLAG_UNFUSED = 2
};

int avq_abi_version(void);
const char *avq_status_string(int status);
const char *avq_last_error(void);

/*
 * avq_build_tree -- parents, distance frame and squared codeword norms of a
 * frozen tree (once per codebook).
 *   Sec. 4.1 "Parent-child constraint": each parent is the mean of its C
 *   children.
 *   children   [H][M0][C][d]  dtype   input
 *   parents_out[H][M0][d]     dtype   output: mean of the C children,
 *                                     accumulated in fp64, rounded once to
 *                                     dtype (nearest, ties to even)
 *   frame_out  [H][d]         fp32    output: reference point r of each
 *                                     head's distance frame.  r_t = 0 unless
 *                                     coordinate t of the head's stored
 *                                     codewords lies further from zero than
 *                                     twice its spread (|mean| > 2 max|c_t -
 *                                     mean|); then r_t is the mean rounded to
 *                                     3 significant bits, provided c_t - r_t
 *                                     is exact in dtype for every codeword
 *                                     (else 0).  Stage 1 compares distances
 *                                     as ||c - r||^2 - 2 (k - r).(c - r):
 *                                     the same distances, with fp32 rounding
 *                                     that scales with the codebook's spread
 *                                     instead of its offset from the origin.
 *   sqnorm_out [H][S_tot]     fp32    output: ||c - r||^2 of every stored
 *                                     codeword (parents first, then
 *                                     children in slot order), accumulated
 *                                     in fp64 over the stored values,
 *                                     rounded once to fp32
 */
int avq_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                   void *parents_out, float *sqnorm_out, float *frame_out, void *stream);

/*
 * avq_assign_aggregate_workspace_size -- bytes of device workspace that
 * avq_assign_aggregate needs for this shape (0 if the shape is invalid or
 * unsupported).
 */
size_t avq_assign_aggregate_workspace_size(int B, int H, int N, int M0, int C, int d);

/*
 * avq_assign_aggregate -- stage 1, full-tree assignment and aggregation.
 *   Sec. 4.2: each key goes to its nearest parent among the M0 parents
 *   (Sec. 3.2 argmin of the squared distance; ties -> lowest index); it is
 *   then compared with that parent's C children only and moves to the
 *   nearest child (ties -> lowest index) if that child is strictly closer
 *   than the parent.  Its value and a count of one are added to the parent
 *   slot and, if it moved, to the child slot: a parent slot holds its whole
 *   cell, a child slot only the keys that moved to it.
 *   K, V       [B][H][N][d]   dtype   input keys and values
 *   parents    [H][M0][d]     dtype   from avq_build_tree
 *   children   [H][M0][C][d]  dtype
 *   sqnorm     [H][S_tot]     fp32    from avq_build_tree
 *   frame      [H][d]         fp32    from avq_build_tree
 *   flags      0, AVQ_FLAG_FORCE_CHILD (C > 0) or AVQ_FLAG_UNFUSED (C = 0)
 *   vsum_out   [B][H][S_tot][d] fp32  output value sums (every slot written)
 *   count_out  [B][H][S_tot]  int32   output key counts (every slot written)
 *   leaf_out   [B][H][N]      int32   optional (NULL = not written): slot of
 *                                     each key's leaf (p*, or M0+p*C+c*)
 *   workspace  device buffer of at least
 *              avq_assign_aggregate_workspace_size(...) bytes, 256-byte
 *              aligned, used only during this call's kernels (it must not
 *              be shared with a concurrent call).  The caller owns it.
 *   The fp32 value sums are accumulated in an order that depends only on
 *   the inputs: repeated calls give identical bits.
 *   Sums and counts are additive over keys: running this call on disjoint
 *   key subsets of the same heads and adding the outputs gives the
 *   aggregates of the union (up to fp32 summation order), which is what a
 *   sequence split over several devices would all-reduce.
 */
int avq_assign_aggregate(const void *K, const void *V, const void *parents,
                         const void *children, const float *sqnorm, const float *frame,
                         int B, int H, int N, int d, int M0, int C, int dtype,
                         unsigned flags, float *vsum_out, int32_t *count_out,
                         int32_t *leaf_out, void *workspace, size_t workspace_bytes,
                         void *stream);

/*
 * avq_assign_aggregate_noalloc -- avq_assign_aggregate for callers that
 *   cannot allocate device memory (code under stream capture, tight serving
 *   loops, harnesses that forbid hipMalloc).  Same arguments, results and
 *   errors, minus the workspace: the stage-1 scratch lives in a static
 *   device array of AVQ_NOALLOC_SCRATCH_BYTES bytes that the library holds
 *   on every device it runs on until the process ends.  The call allocates
 *   and frees nothing.
 *   Shapes whose scratch (avq_assign_aggregate_workspace_size) exceeds
 *   AVQ_NOALLOC_SCRATCH_BYTES return AVQ_ERR_UNSUPPORTED before anything is
 *   enqueued (16 MiB covers about 3.9 million keys over all (b, h), e.g.
 *   B*H*N = 524288 at N = 65536, H = 8).
 *   All calls on one device share that device's array: calls that overlap
 *   in time on one device (different streams, or different host threads)
 *   race and must be serialised by the caller.
 */
#define AVQ_NOALLOC_SCRATCH_BYTES (16u << 20)
int avq_assign_aggregate_noalloc(const void *K, const void *V, const void *parents,
                                 const void *children, const float *sqnorm, const float *frame,
                                 int B, int H, int N, int d, int M0, int C, int dtype,
                                 unsigned flags, float *vsum_out, int32_t *count_out,
                                 int32_t *leaf_out, void *stream);

/*
 * avq_attention_workspace_size -- bytes of device workspace that
 * avq_attention_fwd needs for this shape (0 if the shape is invalid or
 * unsupported).  The workspace receives the aggregates rearranged as the
 * attention kernel's matrix-core operands (value sums rounded to dtype,
 * counts as fp32 and, for bf16, as exact sums of three bf16 parts); its
 * layout is private to the library.
 */
size_t avq_attention_workspace_size(int B, int H, int M0, int C, int d, int dtype);

/*
 * avq_attention_fwd -- stage 2, query-tile adaptive attention.
 *   Sec. 4.3: for every query tile I (contiguous ranges of `tile` queries,
 *   the last one possibly shorter):
 *     parent pass   s_ij = scale * q_i.C_j over the M0 parents, row max m_i,
 *                   E_ij = exp(s_ij - m_i), Z_i = sum_j E_ij n_j,
 *                   X_i = sum_j E_ij Vbar_j ("Tiled VQ-attention");
 *     importance    w_j(I) = sum_{i in I} E_ij n_j / Z_i ("Codeword
 *                   importance");
 *     top-P         the P parents of largest w (ties -> lowest index)
 *                   ("Child spawning");
 *     correction    for each selected parent p and child c:
 *                   S_ic = scale * q_i.C_pc, S_ip = mean_c S_ic
 *                   ("Child attention"), and the child aggregate is added
 *                   with weight exp(S_ic - m) - exp(S_ip - m) to X and Z,
 *                   the shift m being raised (and X, Z rescaled) when a
 *                   child logit exceeds it;
 *     output        Y_i = X_i / Z_i, rounded to dtype.
 *   Q          [B][H][N][d]   dtype
 *   parents    [H][M0][d]     dtype   from avq_build_tree
 *   children   [H][M0][C][d]  dtype
 *   vsum       [B][H][S_tot][d] fp32  value sums Vbar (slot layout of
 *                                     avq_assign_aggregate)
 *   count      [B][H][S_tot]  int32   key counts n (every count row must sum
 *                                     to at least one key; a parent's count
 *                                     must include its children's)
 *   The aggregates may come from avq_assign_aggregate or from anywhere else
 *   (e.g. the sum of several partial runs); they are read, never written.
 *   The value sums enter the matrix-core products rounded to dtype.  For
 *   bf16 the weights enter them rounded to bf16 as well, and Z in the output
 *   step is summed from those same rounded weights (the counts split exactly
 *   into three bf16 parts), so that their rounding cancels in Y; the Z of
 *   the importance is the fp32 sum.
 *   P          0 <= P <= M0 parents refined per tile
 *   tile       queries per tile
 *   scale      finite softmax scale applied to every logit
 *   Y_out      [B][H][N][d]   dtype   output
 *   sel_out    [B][H][ceil(N/tile)][P] int32, optional: selected parents of
 *              every tile in ascending index order
 *   importance_out [B][H][ceil(N/tile)][M0] fp32, optional: w_j(I)
 *   workspace  device buffer of at least avq_attention_workspace_size(...)
 *              bytes, 256-byte aligned, used only during this call's
 *              kernels (not shared with a concurrent call); caller-owned.
 *   Every supported shape fits the kernel's 160 KB of LDS (a shape that did
 *   not would return AVQ_ERR_UNSUPPORTED).
 */
int avq_attention_fwd(const void *Q, const void *parents, const void *children,
                      const float *vsum, const int32_t *count, int B, int H, int N,
                      int d, int M0, int C, int P, int tile, float scale, int dtype,
                      void *Y_out, int32_t *sel_out, float *importance_out,
                      void *workspace, size_t workspace_bytes, void *stream);

/*
 * Three-level tree (roots -> children -> leaves): the deeper hierarchy the
 * pages propose as the next step (Sec. 6 "Discussion and Conclusion": each
 * extra level multiplies the codebook's resolution by C and adds P*C codes
 * per query).  The pages give no algorithm for it; these calls repeat the
 * two-level rules one level down:
 *  - tree: a child is the mean of its C leaves, a root the mean of its C*C
 *    leaves (the Sec. 4.1 constraint at every level);
 *  - stage 1: nearest root, then that root's C children (taken if strictly
 *    closer than the root), then that child's C leaves (taken if strictly
 *    closer than the child); every slot holds its whole cell;
 *  - stage 2: parent pass, importance and top-P over the roots, correction
 *    by their children (as avq_attention_fwd); then the level-1 importance
 *    w_c(I) = sum_{i in I} exp(S_ic - m_i) n_c / Z_i over the P*C children
 *    just added, with Z after their correction, top-P children (ties ->
 *    lower child index), and the same correction by their leaves, a child's
 *    logit recovered as the mean of its leaves' logits.
 * Slots per head: [0, M0) roots; M0 + p*C + a children; M0 + M0*C +
 * (p*C + a)*C + b leaves; S3 = M0 (1 + C + C*C).  C in {2, 4, 8, 16}.
 */

/*
 * avq_build_tree3 -- the two upper levels, frame and norms of a frozen
 * three-level tree (once per codebook).
 *   leaves     [H][M0][C][C][d] dtype  input
 *   level0_out [H][M0][d]       dtype  roots: mean of each root's C*C leaves
 *   level1_out [H][M0][C][d]    dtype  children: mean of each child's C leaves
 *              (both accumulated in fp64 and rounded once to dtype)
 *   sqnorm_out [H][S3]          fp32   ||c - r||^2 of every codeword, slot order
 *   frame_out  [H][d]           fp32   reference point r as in avq_build_tree,
 *                                      over the codewords of all three levels
 */
int avq_build_tree3(const void *leaves, int H, int M0, int C, int d, int dtype, void *level0_out,
                    void *level1_out, float *sqnorm_out, float *frame_out, void *stream);

/* bytes of device workspace avq_assign_aggregate3 needs (0 if invalid) */
size_t avq_assign_aggregate3_workspace_size(int B, int H, int N, int M0, int C, int d);

/*
 * avq_assign_aggregate3 -- stage 1 on a three-level tree (rule above).
 *   K, V       [B][H][N][d]       dtype
 *   level0, level1, sqnorm, frame from avq_build_tree3; leaves [H][M0][C][C][d]
 *   flags      0 or AVQ_FLAG_FORCE_CHILD (descend at both steps regardless
 *              of the distance to the level above)
 *   vsum_out   [B][H][S3][d] fp32, count_out [B][H][S3] int32: whole cells
 *              (every slot written)
 *   leaf_out   [B][H][N] int32 optional: each key's final slot
 *   workspace  at least avq_assign_aggregate3_workspace_size(...) bytes,
 *              256-byte aligned, caller-owned, not shared with a concurrent
 *              call.  Repeated calls give identical bits.
 */
int avq_assign_aggregate3(const void *K, const void *V, const void *level0, const void *level1,
                          const void *leaves, const float *sqnorm, const float *frame, int B, int H,
                          int N, int d, int M0, int C, int dtype, unsigned flags, float *vsum_out,
                          int32_t *count_out, int32_t *leaf_out, void *workspace,
                          size_t workspace_bytes, void *stream);

/* bytes of device workspace avq_attention3_fwd needs (0 if invalid) */
size_t avq_attention3_workspace_size(int B, int H, int M0, int C, int d, int dtype);

/*
 * avq_attention3_fwd -- stage 2 on a three-level tree (rule above).
 *   Q          [B][H][N][d] dtype
 *   level0, level1, leaves   the tree (avq_build_tree3)
 *   vsum, count [B][H][S3]   whole-cell aggregates (avq_assign_aggregate3 or
 *              any caller-built sums in that layout); read, never written
 *   P          0 <= P <= M0 and P*C <= 256: refinements per tile at each level
 *   tile, scale, Y_out, workspace as in avq_attention_fwd (workspace of
 *              avq_attention3_workspace_size bytes)
 *   sel0_out   [B][H][ceil(N/tile)][P] int32 optional: selected roots, ascending
 *   sel1_out   [B][H][ceil(N/tile)][P] int32 optional: selected children
 *              p*C + a, ascending
 */
int avq_attention3_fwd(const void *Q, const void *level0, const void *level1, const void *leaves,
                       const float *vsum, const int32_t *count, int B, int H, int N, int d, int M0,
                       int C, int P, int tile, float scale, int dtype, void *Y_out,
                       int32_t *sel0_out, int32_t *sel1_out, void *workspace,
                       size_t workspace_bytes, void *stream);

/*
 * avq_diagnostics_workspace_size -- bytes of device workspace that
 * avq_codebook_diagnostics needs for the commitment loss (0 if invalid).
 */
size_t avq_diagnostics_workspace_size(int B, int H, int N);

/*
 * avq_codebook_diagnostics -- the codebook measures the pages report next
 * to the method (appendix "Per-layer codebook analysis", Table 7, and
 * "Codebook utilization", Table 9).  Off the hot path; either output may
 * be NULL, not both.
 *   commit_out [B][H] fp32  commitment loss E ||k - k_hat||^2: the mean
 *              over the head's N keys of the squared distance between the
 *              key and its leaf codeword (leaf ids from avq_assign_aggregate's
 *              leaf_out); independent of P.  Needs K [B][H][N][d], parents,
 *              children (the flat codebook when C = 0), leaf [B][H][N] and a
 *              workspace of avq_diagnostics_workspace_size bytes (256-byte
 *              aligned).
 *   active_out [B][H] fp32  active ratio: the fraction of the head's
 *              M0 (1 + C) codewords whose count (avq_assign_aggregate's
 *              count_out [B][H][S_tot]) exceeds 1 % of the fair share
 *              N / (M0 (1 + C)).
 *   Sums run in a fixed order: repeated calls give identical bits.
 */
int avq_codebook_diagnostics(const void *K, const void *parents, const void *children,
                             const int32_t *leaf, const int32_t *count, int B, int H, int N,
                             int d, int M0, int C, int dtype, float *commit_out,
                             float *active_out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * avq_capture -- capture (Sec. 5.2, Table 6): for every query, the fraction
 * of its exact softmax attention weight (scale * q.k over all N keys) that
 * falls on keys whose parent is among the P parents its query tile
 * selected.  O(N^2 d) like exact attention; a diagnostic, off the hot path.
 *   Q, K       [B][H][N][d]   dtype
 *   leaf       [B][H][N]      int32  leaf ids from avq_assign_aggregate
 *   sel        [B][H][ceil(N/tile)][P] int32  selections from
 *              avq_attention_fwd's sel_out (NULL allowed when P = 0)
 *   capture_out [B][H][N]     fp32
 */
int avq_capture(const void *Q, const void *K, const int32_t *leaf, const int32_t *sel,
                int B, int H, int N, int d, int M0, int C, int P, int tile, float scale,
                int dtype, float *capture_out, void *stream);

/*
 * avq_gilbert_order -- the token order of the pages' spatial reordering
 *   (Sec. 4.2, Table 8; ref. [4]): the cells of a W x H token grid along the
 *   generalized Hilbert ("Gilbert") curve, which starts at cell (0, 0) and
 *   ends at the far corner of the longer side, so that consecutive tokens,
 *   and therefore query tiles of any size, form compact 2D regions.
 *   order_out  HOST buffer of W*H int32: order_out[i] = y*W + x of the i-th
 *              cell on the curve (a permutation of the row-major indices).
 *   Host code only, once per grid shape; 1 <= W*H <= 1048576.
 */
int avq_gilbert_order(int W, int H, int32_t *order_out);

/*
 * avq_permute_tokens -- move tokens into (inverse = 0: dst row i = src row
 *   order[i]) or out of (inverse != 0: dst row order[i] = src row i) an
 *   order, for every (b, h): Q, K and V before the forward pass, Y after it.
 *   src, dst   [B][H][N][d] dtype, device, must not alias
 *   order      [N] int32, device: a permutation of 0..N-1 (entries outside
 *              that range are skipped; with repeated entries the scatter's
 *              result is unspecified).  A grid with extra tokens (a class
 *              token, say) uses the Gilbert order offset past them.
 *   Rows must be a multiple of 16 bytes (d*sizeof(dtype)).
 */
int avq_permute_tokens(const void *src, const int32_t *order, int B, int H, int N, int d,
                       int dtype, int inverse, void *dst, void *stream);

/*
 * avq_exact_attention_fwd -- exact softmax attention, non-causal
 * (Sec. 3.1), computed flash-attention style (Sec. 3.3).  Used as the
 * timing context next to AVQ and to check the one-key-per-leaf limit.
 *   Q, K, V, Y_out [B][H][N][d] dtype;  scale finite.
 */
int avq_exact_attention_fwd(const void *Q, const void *K, const void *V,
                            int B, int H, int N, int d, float scale, int dtype,
                            void *Y_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* AVQ_H */
