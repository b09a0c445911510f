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
 *    per parent; 1 <= M0 <= 256 parents; 1 <= N <= 1048576; query tile in
 *    {32, 64, 128, 256} (the pages use tiles of 32 to 128 queries, Table 8).
 *  - Codeword slots: j in [0, M0) is parent j; j = M0 + p*C + c is child c
 *    of parent p.  S_tot = M0 * (1 + C).
 *  - Calls are stateless and thread-safe; no C++ exception crosses the ABI.
 */
#ifndef AVQ_H
#define AVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVQ_ABI_VERSION 1

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
     * partition its cell (no residual keys). */
    AVQ_FLAG_FORCE_CHILD = 1
};

int avq_abi_version(void);
const char *avq_status_string(int status);
const char *avq_last_error(void);

/*
 * avq_build_tree -- parents and squared codeword norms of a frozen tree.
 *   Sec. 4.1 "Parent-child constraint": each parent is the mean of its C
 *   children.
 *   children   [H][M0][C][d]  dtype   input
 *   parents_out[H][M0][d]     dtype   output: mean of the C children,
 *                                     accumulated in fp64, rounded once to
 *                                     dtype (nearest, ties to even)
 *   sqnorm_out [H][S_tot]     fp32    output: squared norm of every stored
 *                                     codeword (parents first, then
 *                                     children in slot order), accumulated
 *                                     in fp64 over the stored values,
 *                                     rounded once to fp32
 */
int avq_build_tree(const void *children, int H, int M0, int C, int d, int dtype,
                   void *parents_out, float *sqnorm_out, void *stream);

/*
 * avq_assign_aggregate_workspace_size -- bytes of device workspace that
 * avq_assign_aggregate needs for this shape (0 if the shape is invalid).
 */
size_t avq_assign_aggregate_workspace_size(int B, int H, int N, int M0, int C, int d);

/*
 * avq_operand_pack_size -- bytes of the operand pack written by
 * avq_assign_aggregate and read by avq_attention_fwd (0 if the shape is
 * invalid).
 */
size_t avq_operand_pack_size(int B, int H, int M0, int C, int d, int dtype);

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
 *   flags      0 or AVQ_FLAG_FORCE_CHILD
 *   vsum_out   [B][H][S_tot][d] fp32  output value sums (every slot written)
 *   count_out  [B][H][S_tot]  int32   output key counts (every slot written)
 *   leaf_out   [B][H][N]      int32   optional (NULL = not written): slot of
 *                                     each key's leaf (p*, or M0+p*C+c*)
 *   pack_out   avq_operand_pack_size(...) bytes, 256-byte aligned: the same
 *              value sums (rounded to dtype) and counts (as fp32) laid out
 *              as the MFMA operands of avq_attention_fwd; its layout is
 *              private to the library and only that call reads it.
 *   workspace  device buffer of at least
 *              avq_assign_aggregate_workspace_size(...) bytes, 256-byte
 *              aligned, used only during this call's kernels (it must not
 *              be shared with a concurrent call).
 *   The order in which fp32 value sums are accumulated is not specified.
 */
int avq_assign_aggregate(const void *K, const void *V, const void *parents,
                         const void *children, const float *sqnorm,
                         int B, int H, int N, int d, int M0, int C, int dtype,
                         unsigned flags, float *vsum_out, int32_t *count_out,
                         int32_t *leaf_out, void *pack_out, void *workspace,
                         size_t workspace_bytes, void *stream);

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
 *   pack       operand pack written by avq_assign_aggregate for these
 *              B, H, M0, C, d, dtype: the value sums Vbar and counts n
 *   P          0 <= P <= M0 parents refined per tile
 *   tile       queries per tile
 *   scale      finite softmax scale applied to every logit
 *   Y_out      [B][H][N][d]   dtype   output
 *   sel_out    [B][H][ceil(N/tile)][P] int32, optional: selected parents of
 *              every tile in ascending index order
 *   importance_out [B][H][ceil(N/tile)][M0] fp32, optional: w_j(I)
 *   Requires at least one key per (b, h) (every count row sums to N >= 1).
 *   Returns AVQ_ERR_UNSUPPORTED if the codebook and tile do not fit the
 *   kernel's 160 KB of LDS: only fp32 with M0 near 256, 256-query tiles and
 *   P above ~160 (d = 64) or ~224 (d = 128).
 */
int avq_attention_fwd(const void *Q, const void *parents, const void *children,
                      const void *pack, int B, int H, int N, int d, int M0, int C,
                      int P, int tile, float scale, int dtype, void *Y_out,
                      int32_t *sel_out, float *importance_out, void *stream);

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
