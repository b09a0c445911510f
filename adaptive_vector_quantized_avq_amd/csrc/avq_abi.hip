// C ABI of the library (declared in include/avq.h): argument validation,
// status codes and dispatch to the kernel launchers.  Nothing here touches
// tensor data; every launch is asynchronous on the caller's stream.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "avq.h"
#include "avq_kernels.h"

namespace {

thread_local char g_last_error[512] = "";

int fail(int status, const char *fmt, const char *what)
{
    snprintf(g_last_error, sizeof(g_last_error), fmt, what);
    return status;
}

#define AVQ_REQUIRE(cond, status, msg)                 \
    do {                                               \
        if (!(cond)) return fail((status), "%s", msg); \
    } while (0)

bool supported_d(int d) { return d == 64 || d == 128; }
bool supported_C(int C) { return C == 0 || C == 2 || C == 4 || C == 8 || C == 16; }
bool valid_dtype(int dt) { return dt == AVQ_F32 || dt == AVQ_BF16; }

// hard limits of the kernels
constexpr int kMaxM0 = 256;
constexpr int kMaxN = 1 << 20;   // key index packed in 24 bits; chunk table in LDS

int check_tree(int H, int M0, int C, int d, int dtype)
{
    AVQ_REQUIRE(H >= 1, AVQ_ERR_INVALID_ARG, "H must be >= 1");
    AVQ_REQUIRE(M0 >= 1, AVQ_ERR_INVALID_ARG, "M0 must be >= 1");
    AVQ_REQUIRE(C >= 0, AVQ_ERR_INVALID_ARG, "C must be >= 0");
    AVQ_REQUIRE(d >= 1, AVQ_ERR_INVALID_ARG, "d must be >= 1");
    AVQ_REQUIRE(valid_dtype(dtype), AVQ_ERR_INVALID_ARG, "dtype must be AVQ_F32 or AVQ_BF16");
    AVQ_REQUIRE(supported_d(d), AVQ_ERR_UNSUPPORTED, "d must be 64 or 128");
    AVQ_REQUIRE(supported_C(C), AVQ_ERR_UNSUPPORTED, "C must be 0, 2, 4, 8 or 16");
    AVQ_REQUIRE(M0 <= kMaxM0, AVQ_ERR_UNSUPPORTED, "M0 must be <= 256");
    return AVQ_OK;
}

// a three-level tree (roots -> children -> leaves) needs children
int check_tree3(int H, int M0, int C, int d, int dtype)
{
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(C > 0, AVQ_ERR_INVALID_ARG, "a three-level tree needs C > 0");
    return AVQ_OK;
}

int check_seq(int B, int N)
{
    AVQ_REQUIRE(B >= 1, AVQ_ERR_INVALID_ARG, "B must be >= 1");
    AVQ_REQUIRE(N >= 1, AVQ_ERR_INVALID_ARG, "N must be >= 1");
    AVQ_REQUIRE(N <= kMaxN, AVQ_ERR_UNSUPPORTED, "N must be <= 1048576");
    return AVQ_OK;
}

int check_assign_flags(unsigned flags, int C)
{
    AVQ_REQUIRE((flags & ~(unsigned)(AVQ_FLAG_FORCE_CHILD | AVQ_FLAG_UNFUSED)) == 0, AVQ_ERR_INVALID_ARG,
                "unknown flag bits");
    AVQ_REQUIRE(!(C == 0 && (flags & AVQ_FLAG_FORCE_CHILD)), AVQ_ERR_INVALID_ARG,
                "AVQ_FLAG_FORCE_CHILD needs children (C > 0)");
    AVQ_REQUIRE(!((flags & AVQ_FLAG_UNFUSED) && C != 0), AVQ_ERR_UNSUPPORTED,
                "AVQ_FLAG_UNFUSED is the flat-codebook (C = 0) comparison path");
    return AVQ_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return AVQ_OK;
    return fail(AVQ_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
}

}  // namespace

// Stage-1 scratch of the allocation-free entry point: one copy per device,
// held from the library's load until the process ends.  In host code
// `scratch` is only a handle; its device address comes from
// hipGetSymbolAddress, once per device.
static __device__ __align__(256) unsigned char scratch[AVQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};

// device address of `scratch` on the current device (resolved on the first
// call made with that device current)
int scratch_address(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_status(e);
    AVQ_REQUIRE(dev >= 0 && dev < kMaxDevices, AVQ_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_status(e);
        AVQ_REQUIRE(p != nullptr, AVQ_ERR_HIP, "hipGetSymbolAddress returned a null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return AVQ_OK;
}

}  // namespace

extern "C" {

int avq_abi_version(void) { return AVQ_ABI_VERSION; }

const char *avq_status_string(int status)
{
    switch (status) {
    case AVQ_OK: return "AVQ_OK";
    case AVQ_ERR_INVALID_ARG: return "AVQ_ERR_INVALID_ARG";
    case AVQ_ERR_UNSUPPORTED: return "AVQ_ERR_UNSUPPORTED";
    case AVQ_ERR_HIP: return "AVQ_ERR_HIP";
    default: return "unknown avq status";
    }
}

const char *avq_last_error(void) { return g_last_error; }

int avq_build_tree(const void *children, int H, int M0, int C, int d, int dtype, void *parents_out,
                   float *sqnorm_out, float *frame_out, void *stream)
{
    AVQ_REQUIRE(children && parents_out && sqnorm_out && frame_out, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    return hip_status(avq::launch_build_tree(children, H, M0, C, d, dtype, parents_out, sqnorm_out, frame_out,
                                             (hipStream_t)stream));
}

size_t avq_assign_aggregate_workspace_size(int B, int H, int N, int M0, int C, int d)
{
    if (check_tree(H, M0, C, d, AVQ_BF16) != AVQ_OK || check_seq(B, N) != AVQ_OK) return 0;
    return avq::assign_workspace_bytes(B, H, N, M0, C, d);
}

size_t avq_attention_workspace_size(int B, int H, int M0, int C, int d, int dtype)
{
    if (check_tree(H, M0, C, d, dtype) != AVQ_OK || B < 1) return 0;
    return (size_t)B * H * avq::pack_layout(M0, C, d, dtype == AVQ_BF16 ? 2 : 4).bytes;
}

int avq_assign_aggregate(const void *K, const void *V, const void *parents, const void *children,
                         const float *sqnorm, const float *frame, int B, int H, int N, int d, int M0, int C,
                         int dtype, unsigned flags, float *vsum_out, int32_t *count_out, int32_t *leaf_out,
                         void *workspace, size_t workspace_bytes, void *stream)
{
    AVQ_REQUIRE(K && V && parents && children && sqnorm && frame && vsum_out && count_out && workspace,
                AVQ_ERR_INVALID_ARG, "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    st = check_assign_flags(flags, C);
    if (st != AVQ_OK) return st;
    const size_t need = avq::assign_workspace_bytes(B, H, N, M0, C, d);
    AVQ_REQUIRE(workspace_bytes >= need, AVQ_ERR_INVALID_ARG, "workspace too small");
    AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const avq::AssignWorkspace ws = avq::carve_assign_workspace(workspace, B, H, N, M0, C, d);
    if (flags & AVQ_FLAG_UNFUSED)
        return hip_status(avq::launch_assign_aggregate_unfused(K, V, parents, sqnorm, frame, B, H, N, d, M0, dtype,
                                                               vsum_out, count_out, leaf_out, ws,
                                                               (hipStream_t)stream));
    return hip_status(avq::launch_assign_aggregate(K, V, parents, children, sqnorm, frame, B, H, N, d, M0, C,
                                                   dtype, flags, vsum_out, count_out, leaf_out, ws,
                                                   (hipStream_t)stream));
}

int avq_assign_aggregate_noalloc(const void *K, const void *V, const void *parents, const void *children,
                                 const float *sqnorm, const float *frame, int B, int H, int N, int d, int M0,
                                 int C, int dtype, unsigned flags, float *vsum_out, int32_t *count_out,
                                 int32_t *leaf_out, void *stream)
{
    AVQ_REQUIRE(K && V && parents && children && sqnorm && frame && vsum_out && count_out, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    st = check_assign_flags(flags, C);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(!(flags & AVQ_FLAG_UNFUSED), AVQ_ERR_UNSUPPORTED,
                "the allocation-free entry point runs the fused stage 1 only");
    const size_t need = avq::assign_workspace_bytes(B, H, N, M0, C, d);
    AVQ_REQUIRE(need <= (size_t)AVQ_NOALLOC_SCRATCH_BYTES, AVQ_ERR_UNSUPPORTED,
                "shape needs more stage-1 scratch than the allocation-free entry point holds "
                "(AVQ_NOALLOC_SCRATCH_BYTES); use avq_assign_aggregate with a workspace");
    void *base = nullptr;
    st = scratch_address(&base);
    if (st != AVQ_OK) return st;
    // every byte of the scratch that the kernels read is written earlier in
    // the same call, so nothing is cleared
    const avq::AssignWorkspace ws = avq::carve_assign_workspace(base, B, H, N, M0, C, d);
    return hip_status(avq::launch_assign_aggregate(K, V, parents, children, sqnorm, frame, B, H, N, d, M0, C,
                                                   dtype, flags, vsum_out, count_out, leaf_out, ws,
                                                   (hipStream_t)stream));
}

int avq_attention_fwd(const void *Q, const void *parents, const void *children, const float *vsum,
                      const int32_t *count, int B, int H, int N, int d, int M0, int C, int P, int tile,
                      float scale, int dtype, void *Y_out, int32_t *sel_out, float *importance_out,
                      void *workspace, size_t workspace_bytes, void *stream)
{
    AVQ_REQUIRE(Q && parents && children && vsum && count && Y_out && workspace, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(P >= 0 && P <= M0, AVQ_ERR_INVALID_ARG, "P must satisfy 0 <= P <= M0");
    AVQ_REQUIRE(C > 0 || P == 0, AVQ_ERR_INVALID_ARG, "a flat codebook (C = 0) has no children to refine: P must be 0");
    AVQ_REQUIRE(tile >= 1, AVQ_ERR_INVALID_ARG, "tile must be >= 1");
    AVQ_REQUIRE(isfinite(scale), AVQ_ERR_INVALID_ARG, "scale must be finite");
    AVQ_REQUIRE(tile == 32 || tile == 64 || tile == 128 || tile == 256, AVQ_ERR_UNSUPPORTED,
                "tile must be 32, 64, 128 or 256");
    AVQ_REQUIRE(avq::attention_child_chunk(d, M0, C, P, tile, dtype) > 0, AVQ_ERR_UNSUPPORTED,
                "codebook does not fit in LDS for this dtype/d/M0/P");
    const size_t need = (size_t)B * H * avq::pack_layout(M0, C, d, dtype == AVQ_BF16 ? 2 : 4).bytes;
    AVQ_REQUIRE(workspace_bytes >= need, AVQ_ERR_INVALID_ARG, "workspace too small");
    AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipError_t e = avq::launch_pack_aggregates(vsum, count, B, H, d, M0, C, dtype, workspace,
                                               (hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(avq::launch_attention_fwd(Q, parents, children, workspace, B, H, N, d, M0, C, P, tile,
                                                scale, dtype, Y_out, sel_out, importance_out,
                                                (hipStream_t)stream));
}

int avq_build_tree3(const void *leaves, int H, int M0, int C, int d, int dtype, void *level0_out, void *level1_out,
                    float *sqnorm_out, float *frame_out, void *stream)
{
    AVQ_REQUIRE(leaves && level0_out && level1_out && sqnorm_out && frame_out, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree3(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    return hip_status(avq::launch_build_tree3(leaves, H, M0, C, d, dtype, level0_out, level1_out, sqnorm_out,
                                              frame_out, (hipStream_t)stream));
}

size_t avq_assign_aggregate3_workspace_size(int B, int H, int N, int M0, int C, int d)
{
    if (check_tree3(H, M0, C, d, AVQ_BF16) != AVQ_OK || check_seq(B, N) != AVQ_OK) return 0;
    return avq::assign3_workspace_bytes(B, H, N, M0, C, d);
}

int avq_assign_aggregate3(const void *K, const void *V, const void *level0, const void *level1, const void *leaves,
                          const float *sqnorm, const float *frame, int B, int H, int N, int d, int M0, int C,
                          int dtype, unsigned flags, float *vsum_out, int32_t *count_out, int32_t *leaf_out,
                          void *workspace, size_t workspace_bytes, void *stream)
{
    AVQ_REQUIRE(K && V && level0 && level1 && leaves && sqnorm && frame && vsum_out && count_out && workspace,
                AVQ_ERR_INVALID_ARG, "null pointer argument");
    int st = check_tree3(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE((flags & ~(unsigned)AVQ_FLAG_FORCE_CHILD) == 0, AVQ_ERR_INVALID_ARG,
                "only AVQ_FLAG_FORCE_CHILD applies to a three-level tree");
    AVQ_REQUIRE(workspace_bytes >= avq::assign3_workspace_bytes(B, H, N, M0, C, d), AVQ_ERR_INVALID_ARG,
                "workspace too small");
    AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    return hip_status(avq::launch_assign_aggregate3(K, V, level0, level1, leaves, sqnorm, frame, B, H, N, d, M0, C,
                                                    dtype, flags, vsum_out, count_out, leaf_out, workspace,
                                                    (hipStream_t)stream));
}

size_t avq_attention3_workspace_size(int B, int H, int M0, int C, int d, int dtype)
{
    if (check_tree3(H, M0, C, d, dtype) != AVQ_OK || B < 1) return 0;
    return (size_t)B * H * avq::pack_layout(M0, C, d, dtype == AVQ_BF16 ? 2 : 4, true).bytes;
}

int avq_attention3_fwd(const void *Q, const void *level0, const void *level1, const void *leaves, const float *vsum,
                       const int32_t *count, int B, int H, int N, int d, int M0, int C, int P, int tile, float scale,
                       int dtype, void *Y_out, int32_t *sel0_out, int32_t *sel1_out, void *workspace,
                       size_t workspace_bytes, void *stream)
{
    AVQ_REQUIRE(Q && level0 && level1 && leaves && vsum && count && Y_out && workspace, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree3(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(P >= 0 && P <= M0, AVQ_ERR_INVALID_ARG, "P must satisfy 0 <= P <= M0");
    AVQ_REQUIRE(tile >= 1, AVQ_ERR_INVALID_ARG, "tile must be >= 1");
    AVQ_REQUIRE(isfinite(scale), AVQ_ERR_INVALID_ARG, "scale must be finite");
    AVQ_REQUIRE(tile == 32 || tile == 64 || tile == 128 || tile == 256, AVQ_ERR_UNSUPPORTED,
                "tile must be 32, 64, 128 or 256");
    AVQ_REQUIRE(P * C <= 256, AVQ_ERR_UNSUPPORTED, "P * C must be <= 256 (the level-1 candidates of a tile)");
    AVQ_REQUIRE(avq::attention_child_chunk(d, M0, C, P, tile, dtype, true) > 0, AVQ_ERR_UNSUPPORTED,
                "codebook does not fit in LDS for this dtype/d/M0/P");
    const size_t need = (size_t)B * H * avq::pack_layout(M0, C, d, dtype == AVQ_BF16 ? 2 : 4, true).bytes;
    AVQ_REQUIRE(workspace_bytes >= need, AVQ_ERR_INVALID_ARG, "workspace too small");
    AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    hipError_t e = avq::launch_pack_aggregates(vsum, count, B, H, d, M0, C, dtype, workspace, (hipStream_t)stream,
                                               true);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(avq::launch_attention_fwd(Q, level0, level1, workspace, B, H, N, d, M0, C, P, tile, scale,
                                                dtype, Y_out, sel0_out, nullptr, (hipStream_t)stream, leaves,
                                                sel1_out));
}

size_t avq_diagnostics_workspace_size(int B, int H, int N)
{
    if (B < 1 || H < 1 || check_seq(B, N) != AVQ_OK) return 0;
    return avq::diagnostics_workspace_bytes(B, H, N);
}

int avq_codebook_diagnostics(const void *K, const void *parents, const void *children, const int32_t *leaf,
                             const int32_t *count, int B, int H, int N, int d, int M0, int C, int dtype,
                             float *commit_out, float *active_out, void *workspace, size_t workspace_bytes,
                             void *stream)
{
    AVQ_REQUIRE(commit_out || active_out, AVQ_ERR_INVALID_ARG, "no output requested");
    AVQ_REQUIRE(!commit_out || (K && parents && children && leaf && workspace), AVQ_ERR_INVALID_ARG,
                "the commitment loss needs K, the tree, the leaf ids and a workspace");
    AVQ_REQUIRE(!active_out || count, AVQ_ERR_INVALID_ARG, "the active ratio needs the counts");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    if (commit_out) {
        AVQ_REQUIRE(workspace_bytes >= avq::diagnostics_workspace_bytes(B, H, N), AVQ_ERR_INVALID_ARG,
                    "workspace too small");
        AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    }
    return hip_status(avq::launch_codebook_diagnostics(K, parents, children, leaf, count, B, H, N, d, M0, C, dtype,
                                                       commit_out, active_out, workspace, (hipStream_t)stream));
}

int avq_capture(const void *Q, const void *K, const int32_t *leaf, const int32_t *sel, int B, int H, int N, int d,
                int M0, int C, int P, int tile, float scale, int dtype, float *capture_out, void *stream)
{
    AVQ_REQUIRE(Q && K && leaf && capture_out && (sel || P == 0), AVQ_ERR_INVALID_ARG, "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(P >= 0 && P <= M0, AVQ_ERR_INVALID_ARG, "P must satisfy 0 <= P <= M0");
    AVQ_REQUIRE(isfinite(scale), AVQ_ERR_INVALID_ARG, "scale must be finite");
    AVQ_REQUIRE(tile == 32 || tile == 64 || tile == 128 || tile == 256, AVQ_ERR_UNSUPPORTED,
                "tile must be 32, 64, 128 or 256");
    return hip_status(avq::launch_capture(Q, K, leaf, sel, B, H, N, d, M0, C, P, tile, scale, dtype, capture_out,
                                          (hipStream_t)stream));
}

int avq_gilbert_order(int W, int H, int32_t *order_out)
{
    AVQ_REQUIRE(order_out, AVQ_ERR_INVALID_ARG, "null pointer argument");
    AVQ_REQUIRE(W >= 1 && H >= 1, AVQ_ERR_INVALID_ARG, "W and H must be >= 1");
    AVQ_REQUIRE((int64_t)W * H <= kMaxN, AVQ_ERR_UNSUPPORTED, "W * H must be <= 1048576");
    avq::gilbert_cells(W, H, order_out);
    return AVQ_OK;
}

int avq_permute_tokens(const void *src, const int32_t *order, int B, int H, int N, int d, int dtype, int inverse,
                       void *dst, void *stream)
{
    AVQ_REQUIRE(src && order && dst, AVQ_ERR_INVALID_ARG, "null pointer argument");
    AVQ_REQUIRE(src != dst, AVQ_ERR_INVALID_ARG, "src and dst must not alias");
    AVQ_REQUIRE(H >= 1 && d >= 1, AVQ_ERR_INVALID_ARG, "H and d must be >= 1");
    AVQ_REQUIRE(valid_dtype(dtype), AVQ_ERR_INVALID_ARG, "dtype must be AVQ_F32 or AVQ_BF16");
    int st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    const int row_bytes = d * (dtype == AVQ_BF16 ? 2 : 4);
    AVQ_REQUIRE(row_bytes % 16 == 0, AVQ_ERR_UNSUPPORTED, "rows must be a multiple of 16 bytes");
    return hip_status(avq::launch_permute_rows(src, order, (int64_t)B * H * N, N, row_bytes, inverse ? 1 : 0, dst,
                                               (hipStream_t)stream));
}

int avq_exact_attention_fwd(const void *Q, const void *K, const void *V, int B, int H, int N, int d,
                            float scale, int dtype, void *Y_out, void *stream)
{
    AVQ_REQUIRE(Q && K && V && Y_out, AVQ_ERR_INVALID_ARG, "null pointer argument");
    AVQ_REQUIRE(H >= 1, AVQ_ERR_INVALID_ARG, "H must be >= 1");
    AVQ_REQUIRE(valid_dtype(dtype), AVQ_ERR_INVALID_ARG, "dtype must be AVQ_F32 or AVQ_BF16");
    int st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(isfinite(scale), AVQ_ERR_INVALID_ARG, "scale must be finite");
    AVQ_REQUIRE(supported_d(d), AVQ_ERR_UNSUPPORTED, "d must be 64 or 128");
    return hip_status(avq::launch_exact_attention(Q, K, V, B, H, N, d, scale, dtype, Y_out,
                                                  (hipStream_t)stream));
}

}  // extern "C"
