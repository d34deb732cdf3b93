// One Aaren attention layer: projections on the matrix cores (rocBLAS), then
// the many-to-many scan with a learned query per head.
//
// "Attention as an RNN" (review, proposed method): Aaren is an attention
// module whose query is a learned initial hidden state q rather than a
// projection of the input, and whose many-to-many output is the prefix scan;
// like a Transformer's attention it is stacked. Here a layer maps x [B,N,Dm]
// to o [B,N,H,d] with K = x W_K, V = x W_V and o[b,n,h] the scan of q_h over
// K[b,0..n,h], V[b,0..n,h]. The scan needs K only through the scores
// <q_h, k_n> = x_n (W_K^h q_h), so the query is folded into the weights
// first (u_h = W_K^h q_h, one column per head) and one bf16 GEMM (fp32
// output) gives V and the scores together: K is never formed, the product
// has H*d + 4H columns instead of 2*H*d, and the scan reads V and one 16-byte
// score run per row instead of K and V. u_h goes into the GEMM as three bf16
// parts, so the scores keep fp32 precision. V and the scores stay in the
// GEMM's token-major layout; the scan reads them through its strides.
// Stacking feeds o (as [B,N,H*d]) to the next layer as x.
#include <rocblas/rocblas.h>

#include <cstring>
#include <mutex>
#include <unordered_map>

#include "device.h"
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
// scan_scored_strided's argument checks alone, enqueueing nothing (api.hip)
aaren_status scan_scored_check(const float *scores, int64_t s_head_stride, const float *v,
                               void *o, int64_t B, int64_t H, int64_t N, int64_t d,
                               const int64_t *v_strides, const int64_t *o_strides,
                               aaren_dtype out_dtype, void *workspace, size_t workspace_bytes,
                               void *hip_stream);
}  // namespace aaren

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

namespace aaren {

// Columns of the layer's product: V (H*d), per head 4 score columns, then
// zero columns up to a multiple of 128. rocBLAS ran the padded product faster
// on the stacked-layer shape (B=8, N=4096, Dm=1024, H=16, d=64: 1152 columns
// 5.6% faster for the stack than 1088; 1280 slower).
int64_t layer_cols(int64_t H, int64_t d)
{
    return (H * d + 4 * H + 127) / 128 * 128;
}

// Leading dimension of the folded weights (bf16): rows start 16-byte aligned.
int64_t layer_ld(int64_t H, int64_t d)
{
    return layer_cols(H, d);
}

// The folded weights W2 [Dm][ld2]: row m holds W_V's row m and, for each
// head h, u_h[m] = c <W_K[m, h*d .. h*d+d), q_h> (c = scale * log2(e)) as
// three bf16 parts hi, mid, lo with hi + mid + lo = u_h[m] to within fp32
// rounding (each part is the bf16 rounding of what the parts before it leave),
// then a zero; zeros fill the row from column H*d + 4H to cols. x W2 then
// gives V and, in four columns per head, the three parts of c <q_h, k_n>,
// whose sum is the score.
template <int D>
__global__ __launch_bounds__(256) void layer_fold_kernel(const uint16_t *w_kv, const float *q,
                                                         uint16_t *w2, int64_t H, int64_t ld2,
                                                         int64_t cols, float c)
{
    const int64_t m = blockIdx.x, hd = H * D, nv = hd / 8;
    const int64_t npad = (cols - hd - 4 * H) / 4;  // 4-column runs of zeros
    const uint16_t *row = w_kv + m * 2 * hd;
    uint16_t *out = w2 + m * ld2;
    for (int64_t i = threadIdx.x; i < nv + H + npad; i += blockDim.x) {
        if (i < nv) {
            store16(out + 8 * i, load16(row + hd + 8 * i));
            continue;
        }
        if (i >= nv + H) {
            *reinterpret_cast<u32x2 *>(out + hd + 4 * H + 4 * (i - nv - H)) = u32x2{0, 0};
            continue;
        }
        const int64_t h = i - nv;
        float acc = 0.f;
        for (int t = 0; t < D; t += 8) {
            float w[8];
            widen<bf16>(load16(row + h * D + t), w);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                acc = __builtin_fmaf(w[e], q[h * D + t + e], acc);
        }
        const float u = c * acc;
        const uint32_t hi = bf16_bits(u);
        const float r1 = u - __uint_as_float(hi << 16);
        const uint32_t mid = bf16_bits(r1);
        const uint32_t lo = bf16_bits(r1 - __uint_as_float(mid << 16));
        *reinterpret_cast<u32x2 *>(out + hd + 4 * h) = u32x2{hi | (mid << 16), lo};
    }
}

}  // namespace aaren

AAREN_API size_t aaren_layer_workspace_size(int64_t B, int64_t N, int64_t Dm, int64_t H, int64_t d)
{
    if (B < 0 || N < 0 || Dm < 0 || H < 0 || (d != 64 && d != 128))
        return 0;
    const size_t scan = aaren_scan_workspace_size(B, H, N, d);
    if (scan == 0)
        return 0;
    const int64_t cols = aaren::layer_cols(H, d), ld = aaren::layer_ld(H, d);
    // B*N*cols*4 and Dm*ld*2 below 2^62
    const int64_t lim = int64_t(1) << 60;
    if ((B > 0 && N > lim / B) || (B * N > 0 && cols > lim / (B * N)) || (Dm > 0 && ld > lim / Dm))
        return 0;
    return round256(scan) + round256((size_t)(B * N * cols) * 4) + round256((size_t)(Dm * ld) * 2);
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
    const int64_t rows = B * N, cols = aaren::layer_cols(H, d), ld = aaren::layer_ld(H, d);
    if (B * N == 0 || H == 0)
        return AAREN_OK;
    if (Dm == 0)
        return aaren_layer_fail(AAREN_ERR_INVALID_ARG, "Dm = 0: keys and values have no inputs");
    if (rows > 0x7fffffffLL || 2 * H * d > 0x7fffffffLL || Dm > 0x7fffffffLL ||
        rows > (int64_t(1) << 62) / (2 * H * d > Dm ? 2 * H * d : Dm))
        return aaren_layer_fail(AAREN_ERR_UNSUPPORTED, "sizes exceed the 32-bit GEMM interface");
    for (const void *ptr : {x, w_kv, static_cast<const void *>(q), static_cast<const void *>(o)}) {
        if (!ptr)
            return aaren_layer_fail(AAREN_ERR_INVALID_ARG, "a tensor pointer is NULL");
        if (reinterpret_cast<uintptr_t>(ptr) & 15u)
            return aaren_layer_fail(AAREN_ERR_ALIGNMENT, "a tensor is not 16-byte aligned");
    }
    const size_t need = aaren_layer_workspace_size(B, N, Dm, H, d);
    if (need == 0)
        return aaren_layer_fail(AAREN_ERR_UNSUPPORTED, "the workspace size overflows");
    if (!workspace || workspace_bytes < need)
        return aaren_layer_fail(AAREN_ERR_WORKSPACE, "workspace too small for the layer");
    if (reinterpret_cast<uintptr_t>(workspace) & 15u)
        return aaren_layer_fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

    // [scan workspace][V and scores fp32, token-major [B*N][cols]][W2 bf16 [Dm][ld]]
    const size_t scan_bytes = aaren_scan_workspace_size(B, H, N, d);
    uint8_t *wsb = static_cast<uint8_t *>(workspace);
    float *vs = reinterpret_cast<float *>(wsb + round256(scan_bytes));
    uint16_t *w2 = reinterpret_cast<uint16_t *>(wsb + round256(scan_bytes) +
                                                round256((size_t)(rows * cols) * 4));
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const int64_t vstr[3] = {N * cols, d, cols};   // V: row (b,n), column block h
    const int64_t os[3] = {N * H * d, d, H * d};   // o: token-major [B,N,H,d]
    // the scan's own checks, before anything is enqueued
    {
        const aaren_status cs = aaren::scan_scored_check(vs + H * d, 4, vs, o, B, H, N, d, vstr,
                                                         os, out_dtype, workspace, scan_bytes,
                                                         hip_stream);
        if (cs != AAREN_OK)
            return cs;
    }
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
        if (rocblas_set_stream(h, st) != rocblas_status_success)
            return aaren_layer_fail(AAREN_ERR_HIP, "rocblas_set_stream failed");
        const float c = scale * 1.44269504088896340736f;
        if (d == 64)
            hipLaunchKernelGGL(aaren::layer_fold_kernel<64>, dim3((unsigned)Dm), dim3(256), 0, st,
                               static_cast<const uint16_t *>(w_kv), q, w2, H, ld, cols, c);
        else
            hipLaunchKernelGGL(aaren::layer_fold_kernel<128>, dim3((unsigned)Dm), dim3(256), 0, st,
                               static_cast<const uint16_t *>(w_kv), q, w2, H, ld, cols, c);
        if (hipGetLastError() != hipSuccess)
            return aaren_layer_fail(AAREN_ERR_HIP, "weight fold launch failed");
        // row-major VS[rows][cols] = x[rows][Dm] W2[Dm][cols], i.e. column-major
        // VS^T = W2^T x^T with the same buffers
        const float alpha = 1.f, beta = 0.f;
        const rocblas_status bs = rocblas_gemm_ex(
            h, rocblas_operation_none, rocblas_operation_none, (rocblas_int)cols,
            (rocblas_int)rows, (rocblas_int)Dm, &alpha, w2, rocblas_datatype_bf16_r,
            (rocblas_int)ld, x, rocblas_datatype_bf16_r, (rocblas_int)Dm, &beta, vs,
            rocblas_datatype_f32_r, (rocblas_int)cols, vs, rocblas_datatype_f32_r,
            (rocblas_int)cols, rocblas_datatype_f32_r, rocblas_gemm_algo_standard, 0, 0);
        if (bs != rocblas_status_success)
            return aaren_layer_fail(AAREN_ERR_HIP, rocblas_status_to_string(bs));
    }
    return aaren::scan_scored_strided(vs + H * d, 4, vs, o, B, H, N, d, vstr, os, out_dtype,
                                      workspace, scan_bytes, hip_stream);
}
