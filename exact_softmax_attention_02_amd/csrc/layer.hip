// One Aaren attention layer: projections on the matrix cores (rocBLAS), then
// the many-to-many scan with a learned query per head.
//
// "Attention as an RNN" (review, proposed method): Aaren is an attention
// module whose query is a learned initial hidden state q rather than a
// projection of the input, and whose many-to-many output is the prefix scan;
// like a Transformer's attention it is stacked. Here a layer maps x [B,N,Dm]
// to o [B,N,H,d] with
//     [K | V] = x [W_K | W_V]              (one bf16 GEMM, fp32 output),
//     o[b,n,h] = scan of q_h over K[b,0..n,h], V[b,0..n,h].
// K and V stay in the GEMM's token-major layout; the scan reads them through
// its strides, so nothing is transposed. Stacking feeds o (as [B,N,H*d]) to
// the next layer as x.
#include <rocblas/rocblas.h>

#include <cstring>
#include <mutex>
#include <unordered_map>

#include "layout.h"

#define AAREN_API extern "C" __attribute__((visibility("default")))

namespace {

// One rocBLAS handle per device, created by aaren_init (rocBLAS allocates its
// own workspace then) and kept for the process; calls through it are
// serialised because a handle is not thread-safe.
std::mutex g_blas_mutex;
std::unordered_map<int, rocblas_handle> g_blas;

size_t round256(size_t x)
{
    return (x + 255) / 256 * 256;
}

}  // namespace

extern "C" aaren_status aaren_layer_fail(aaren_status s, const char *msg);

namespace aaren {

// Creates the handle and runs one small product of the layer's types and
// layout through it, so that rocBLAS has loaded its kernels for them before a
// layer call can be captured into a graph.
const char *layer_init(int device)
{
    std::lock_guard<std::mutex> lock(g_blas_mutex);
    if (g_blas.count(device))
        return nullptr;
    rocblas_handle h = nullptr;
    if (rocblas_create_handle(&h) != rocblas_status_success)
        return "rocblas_create_handle failed";
    constexpr int n = 64;
    void *buf = nullptr;
    if (hipMalloc(&buf, 2 * n * n * 2 + n * n * 4) != hipSuccess) {
        rocblas_destroy_handle(h);
        return "hipMalloc of the warm-up product failed";
    }
    const char *err = nullptr;
    if (hipMemsetAsync(buf, 0, 2 * n * n * 2 + n * n * 4, nullptr) != hipSuccess ||
        rocblas_set_stream(h, nullptr) != rocblas_status_success)
        err = "warm-up product set-up failed";
    const float alpha = 1.f, beta = 0.f;
    uint8_t *b8 = static_cast<uint8_t *>(buf);
    if (!err && rocblas_gemm_ex(h, rocblas_operation_none, rocblas_operation_none, n, n, n, &alpha,
                                b8, rocblas_datatype_bf16_r, n, b8 + n * n * 2,
                                rocblas_datatype_bf16_r, n, &beta, b8 + 2 * n * n * 2,
                                rocblas_datatype_f32_r, n, b8 + 2 * n * n * 2,
                                rocblas_datatype_f32_r, n, rocblas_datatype_f32_r,
                                rocblas_gemm_algo_standard, 0, 0) != rocblas_status_success)
        err = "warm-up product failed";
    if (hipStreamSynchronize(nullptr) != hipSuccess && !err)
        err = "warm-up product did not complete";
    (void)hipFree(buf);
    if (err) {
        rocblas_destroy_handle(h);
        return err;
    }
    g_blas[device] = h;
    return nullptr;
}

}  // namespace aaren

AAREN_API size_t aaren_layer_workspace_size(int64_t B, int64_t N, int64_t H, int64_t d)
{
    if (B < 0 || N < 0 || H < 0 || (d != 64 && d != 128))
        return 0;
    const size_t scan = aaren_scan_workspace_size(B, H, N, d);
    if (scan == 0)
        return 0;
    return round256(scan) + round256((size_t)B * N * 2 * H * d * 4);
}

AAREN_API aaren_status aaren_layer_forward(const void *x, const void *w_kv, const float *q,
                                           void *o, int64_t B, int64_t N, int64_t Dm, int64_t H,
                                           int64_t d, float scale, aaren_dtype out_dtype,
                                           void *workspace, size_t workspace_bytes,
                                           void *hip_stream)
{
    if (B < 0 || N < 0 || Dm < 0 || H < 0)
        return aaren_layer_fail(AAREN_ERR_INVALID_ARG, "negative size");
    if (d != 64 && d != 128)
        return aaren_layer_fail(AAREN_ERR_UNSUPPORTED, "supported head dimensions are 64 and 128");
    int out_code;  // read from the bytes: a C caller may pass any int
    std::memcpy(&out_code, &out_dtype, sizeof out_code);
    if (out_code != AAREN_F32 && out_code != AAREN_BF16)
        return aaren_layer_fail(AAREN_ERR_UNSUPPORTED, "unknown output dtype");
    const int64_t rows = B * N, cols = 2 * H * d;
    if (B * N == 0 || H == 0)
        return AAREN_OK;
    if (Dm == 0)
        return aaren_layer_fail(AAREN_ERR_INVALID_ARG, "Dm = 0: keys and values have no inputs");
    if (rows > 0x7fffffffLL || cols > 0x7fffffffLL || Dm > 0x7fffffffLL ||
        rows > (int64_t(1) << 62) / (cols > Dm ? cols : Dm))
        return aaren_layer_fail(AAREN_ERR_UNSUPPORTED, "sizes exceed the 32-bit GEMM interface");
    for (const void *ptr : {x, w_kv, static_cast<const void *>(q), static_cast<const void *>(o)}) {
        if (!ptr)
            return aaren_layer_fail(AAREN_ERR_INVALID_ARG, "a tensor pointer is NULL");
        if (reinterpret_cast<uintptr_t>(ptr) & 15u)
            return aaren_layer_fail(AAREN_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
    }
    const size_t need = aaren_layer_workspace_size(B, N, H, d);
    if (!workspace || workspace_bytes < need)
        return aaren_layer_fail(AAREN_ERR_WORKSPACE, "workspace too small for the layer");
    if (reinterpret_cast<uintptr_t>(workspace) & 15u)
        return aaren_layer_fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

    // [scan workspace][K|V fp32, token-major [B*N][2*H*d]]
    const size_t scan_bytes = aaren_scan_workspace_size(B, H, N, d);
    float *kv = reinterpret_cast<float *>(static_cast<uint8_t *>(workspace) + round256(scan_bytes));
    {
        int device = 0;
        if (hipGetDevice(&device) != hipSuccess)
            return aaren_layer_fail(AAREN_ERR_HIP, "hipGetDevice failed");
        std::lock_guard<std::mutex> lock(g_blas_mutex);
        // the handle (whose creation allocates) comes from aaren_init, so
        // this call allocates nothing and may be captured into a graph
        auto it = g_blas.find(device);
        if (it == g_blas.end())
            return aaren_layer_fail(AAREN_ERR_UNSUPPORTED,
                                    "aaren_init has not been called on this device (it creates "
                                    "the layer's rocBLAS handle)");
        rocblas_handle h = it->second;
        if (rocblas_set_stream(h, static_cast<hipStream_t>(hip_stream)) != rocblas_status_success)
            return aaren_layer_fail(AAREN_ERR_HIP, "rocblas_set_stream failed");
        // row-major KV[rows][cols] = x[rows][Dm] W[Dm][cols], i.e. column-major
        // KV^T = W^T x^T with the same buffers
        const float alpha = 1.f, beta = 0.f;
        const rocblas_status st = rocblas_gemm_ex(
            h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)cols,
            (rocblas_int)rows, (rocblas_int)Dm, &alpha, w_kv, rocblas_datatype_bf16_r,
            (rocblas_int)cols, x, rocblas_datatype_bf16_r, (rocblas_int)Dm, &beta, kv,
            rocblas_datatype_f32_r, (rocblas_int)cols, kv, rocblas_datatype_f32_r,
            (rocblas_int)cols, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
        if (st != rocblas_status_success)
            return aaren_layer_fail(AAREN_ERR_HIP, rocblas_status_to_string(st));
    }
    const int64_t kvs[3] = {N * cols, d, cols};      // K: row (b,n), column block h
    const int64_t os[3] = {N * H * d, d, H * d};     // o: token-major [B,N,H,d]
    return aaren_scan_strided(q, kv, kv + H * d, o, nullptr, B, H, N, d, kvs, os, scale, AAREN_F32,
                              out_dtype, workspace, scan_bytes, hip_stream);
}
