// C ABI of the library (declared in include/avq.h): argument validation,
// status codes and dispatch to the kernel launchers.  Nothing here touches
// tensor data; every launch is asynchronous on the caller's stream.
#include <math.h>
#include <stdio.h>
#include <string.h>

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
bool supported_C(int C) { return C == 2 || C == 4 || C == 8 || C == 16; }
bool valid_dtype(int dt) { return dt == AVQ_F32 || dt == AVQ_BF16; }

// hard limits of the kernels
constexpr int kMaxM0 = 256;
constexpr int kMaxN = 1 << 20;   // key index packed in 24 bits; chunk table in LDS

int check_tree(int H, int M0, int C, int d, int dtype)
{
    AVQ_REQUIRE(H >= 1, AVQ_ERR_INVALID_ARG, "H must be >= 1");
    AVQ_REQUIRE(M0 >= 1, AVQ_ERR_INVALID_ARG, "M0 must be >= 1");
    AVQ_REQUIRE(C >= 1, AVQ_ERR_INVALID_ARG, "C must be >= 1");
    AVQ_REQUIRE(d >= 1, AVQ_ERR_INVALID_ARG, "d must be >= 1");
    AVQ_REQUIRE(valid_dtype(dtype), AVQ_ERR_INVALID_ARG, "dtype must be AVQ_F32 or AVQ_BF16");
    AVQ_REQUIRE(supported_d(d), AVQ_ERR_UNSUPPORTED, "d must be 64 or 128");
    AVQ_REQUIRE(supported_C(C), AVQ_ERR_UNSUPPORTED, "C must be 2, 4, 8 or 16");
    AVQ_REQUIRE(M0 <= kMaxM0, AVQ_ERR_UNSUPPORTED, "M0 must be <= 256");
    return AVQ_OK;
}

int check_seq(int B, int N)
{
    AVQ_REQUIRE(B >= 1, AVQ_ERR_INVALID_ARG, "B must be >= 1");
    AVQ_REQUIRE(N >= 1, AVQ_ERR_INVALID_ARG, "N must be >= 1");
    AVQ_REQUIRE(N <= kMaxN, AVQ_ERR_UNSUPPORTED, "N must be <= 1048576");
    return AVQ_OK;
}

int hip_status(hipError_t e)
{
    if (e == hipSuccess) return AVQ_OK;
    return fail(AVQ_ERR_HIP, "HIP error: %s", hipGetErrorString(e));
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
                   float *sqnorm_out, void *stream)
{
    AVQ_REQUIRE(children && parents_out && sqnorm_out, AVQ_ERR_INVALID_ARG, "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    return hip_status(avq::launch_build_tree(children, H, M0, C, d, dtype, parents_out, sqnorm_out,
                                             (hipStream_t)stream));
}

size_t avq_assign_aggregate_workspace_size(int B, int H, int N, int M0, int C, int d)
{
    if (check_tree(H, M0, C, d, AVQ_BF16) != AVQ_OK || check_seq(B, N) != AVQ_OK) return 0;
    return avq::assign_workspace_bytes(B, H, N, M0, C, d);
}

size_t avq_operand_pack_size(int B, int H, int M0, int C, int d, int dtype)
{
    if (check_tree(H, M0, C, d, dtype) != AVQ_OK || B < 1) return 0;
    return (size_t)B * H * avq::pack_layout(M0, C, d, dtype == AVQ_BF16 ? 2 : 4).bytes;
}

int avq_assign_aggregate(const void *K, const void *V, const void *parents, const void *children,
                         const float *sqnorm, int B, int H, int N, int d, int M0, int C, int dtype,
                         unsigned flags, float *vsum_out, int32_t *count_out, int32_t *leaf_out,
                         void *pack_out, void *workspace, size_t workspace_bytes, void *stream)
{
    AVQ_REQUIRE(K && V && parents && children && sqnorm && vsum_out && count_out && pack_out && workspace,
                AVQ_ERR_INVALID_ARG, "null pointer argument");
    AVQ_REQUIRE((flags & ~(unsigned)AVQ_FLAG_FORCE_CHILD) == 0, AVQ_ERR_INVALID_ARG, "unknown flag bits");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    const size_t need = avq::assign_workspace_bytes(B, H, N, M0, C, d);
    AVQ_REQUIRE(workspace_bytes >= need, AVQ_ERR_INVALID_ARG, "workspace too small");
    AVQ_REQUIRE(((uintptr_t)workspace & 255u) == 0, AVQ_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
    const avq::AssignWorkspace ws = avq::carve_assign_workspace(workspace, B, H, N, M0, C, d);
    return hip_status(avq::launch_assign_aggregate(K, V, parents, children, sqnorm, B, H, N, d, M0, C,
                                                   dtype, flags, vsum_out, count_out, leaf_out,
                                                   pack_out, ws, (hipStream_t)stream));
}

int avq_attention_fwd(const void *Q, const void *parents, const void *children, const void *pack,
                      int B, int H, int N, int d, int M0, int C, int P, int tile, float scale,
                      int dtype, void *Y_out, int32_t *sel_out, float *importance_out, void *stream)
{
    AVQ_REQUIRE(Q && parents && children && pack && Y_out, AVQ_ERR_INVALID_ARG,
                "null pointer argument");
    int st = check_tree(H, M0, C, d, dtype);
    if (st != AVQ_OK) return st;
    st = check_seq(B, N);
    if (st != AVQ_OK) return st;
    AVQ_REQUIRE(P >= 0 && P <= M0, AVQ_ERR_INVALID_ARG, "P must satisfy 0 <= P <= M0");
    AVQ_REQUIRE(tile >= 1, AVQ_ERR_INVALID_ARG, "tile must be >= 1");
    AVQ_REQUIRE(isfinite(scale), AVQ_ERR_INVALID_ARG, "scale must be finite");
    AVQ_REQUIRE(tile == 32 || tile == 64 || tile == 128 || tile == 256, AVQ_ERR_UNSUPPORTED,
                "tile must be 32, 64, 128 or 256");
    AVQ_REQUIRE(avq::attention_child_chunk(d, M0, C, P, tile, dtype) > 0, AVQ_ERR_UNSUPPORTED,
                "codebook does not fit in LDS for this dtype/d/M0/P");
    return hip_status(avq::launch_attention_fwd(Q, parents, children, pack, B, H, N, d, M0, C, P, tile,
                                                scale, dtype, Y_out, sel_out, importance_out,
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
