// Constant-memory RNN step: absorb one key/value pair per (stream, head) into
// a stored state (m, u, w) and emit o_t = w/u ("Attention as an RNN" review,
// abstract item (4)(ii) and proposed method; the update is the recurrence of
// section 2 of the "Self-attention Does Not Need O(n^2) Memory" review with
// the running-maximum shift of its section 3).
//
// Pure streaming: each (stream, head) is one lane group that reads q, k_t, v_t,
// w (16-byte slices) and m, u, and writes w, m, u and o_t. The state stays in
// natural score units (m is the running maximum of the fp32 scores).
#include "device.h"

namespace aaren {

// Absorb one pair (score s in natural units, value row vf) into the state:
// the side with the smaller maximum is scaled by e^{lo-hi}, an empty side
// (maximum -inf) weighs 0. The step and the append kernels share it, so T
// appended tokens give bit for bit the state and outputs of T steps.
template <int E>
__device__ __forceinline__ void absorb_pair(float s, const float *vf, float &m, float &u,
                                            float *wv)
{
    const bool up = s > m;
    const float hi = up ? s : m;
    const float lo = up ? m : s;
    float ex = exp2_fast((lo - hi) * kLog2e);
    ex = (lo == kNegInf) ? 0.f : ex;
    const float a = up ? ex : 1.f;
    const float pr = up ? 1.f : ex;
    u = __builtin_fmaf(u, a, pr);
#pragma unroll
    for (int e = 0; e < E; ++e)
        wv[e] = __builtin_fmaf(wv[e], a, pr * vf[e]);
    m = hi;
}

template <int D, typename Tin, typename Tout>
__global__ __launch_bounds__(256) void step_kernel(const StepParams p)
{
    using G = RowGeo<D, Tin>;
    constexpr int E = G::kElems, L = G::kLanes;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t unit = gid / L;
    const int gl = threadIdx.x % L;
    if (unit >= p.units)  // whole groups leave together: L divides 256
        return;
    const int64_t h = unit % p.H;

    float qv[E], kf[E], vf[E], wv[E];
    widen<Tin>(load_slice<D, Tin, false>(static_cast<const Tin *>(p.q) + h * D, gl), qv);
    const int64_t off = unit * D;  // column 0 of this (stream, head)
    widen<Tin>(load_slice<D, Tin, true>(static_cast<const Tin *>(p.k) + off, gl), kf);
    widen<Tin>(load_slice<D, Tin, true>(static_cast<const Tin *>(p.v) + off, gl), vf);
    float *wp = p.w + off;
    load_state<D, Tin>(wp, gl, wv);
    float m = p.m[unit], u = p.u[unit];

    float part = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e)
        part = __builtin_fmaf(qv[e] * p.scale, kf[e], part);
    absorb_pair<E>(group_sum<L>(part), vf, m, u, wv);
    store_state<D, Tin>(wp, gl, wv);
    if (gl == 0) {
        p.m[unit] = m;
        p.u[unit] = u;
    }
    if (p.o) {
        const float inv = rcp_fast(u);
        float ov[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            ov[e] = wv[e] * inv;
        store_slice<D, Tin, Tout>(static_cast<Tout *>(p.o) + off, gl, ov);
    }
}

// Absorb NB consecutive tokens of one (stream, head) into its state held in
// registers: the block's loads and scores first, then its pairs in order, each
// emitting o_t = w_t / u_t when EMIT. kp, vp, op point at the block's first
// row; rows are tstride elements apart.
template <int D, typename Tin, typename Tout, int NB, bool EMIT>
__device__ __forceinline__ void append_block(const Tin *kp, const Tin *vp, Tout *op,
                                             int64_t tstride, int gl, const float *qs, float &m,
                                             float &u, float *wv)
{
    using G = RowGeo<D, Tin>;
    constexpr int E = G::kElems, L = G::kLanes;
    u32x4 kr[NB], vr[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r)
        kr[r] = load_slice<D, Tin, true>(kp + r * tstride, gl);
#pragma unroll
    for (int r = 0; r < NB; ++r)
        vr[r] = load_slice<D, Tin, true>(vp + r * tstride, gl);
    float s[NB];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float kf[E];
        widen<Tin>(kr[r], kf);
        float part = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            part = __builtin_fmaf(qs[e], kf[e], part);
        s[r] = group_sum<L>(part);
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
        float vf[E];
        widen<Tin>(vr[r], vf);
        absorb_pair<E>(s[r], vf, m, u, wv);
        if constexpr (EMIT) {
            const float inv = rcp_fast(u);
            float ov[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                ov[e] = wv[e] * inv;
            store_slice<D, Tin, Tout>(op + r * tstride, gl, ov);
        }
    }
}

// Append `tokens` pairs to every (stream, head): a scan of the new tokens
// with the stored state as its carry-in, one lane group per (stream, head),
// walking the tokens in order, loading R at a time, then the remainder one by
// one. k, v and o are time-major ([t][unit][d], k[t] being one step's keys),
// so a wavefront reads and writes whole contiguous rows for each token. Each
// pair is absorbed with the running maximum (the state is never rescaled to a
// maximum its outputs have not reached yet, which could underflow u), with
// the step's own arithmetic.
template <int D, typename Tin, typename Tout, int R, bool EMIT>
__global__ __launch_bounds__(256) void append_kernel(const StepParams p)
{
    using G = RowGeo<D, Tin>;
    constexpr int E = G::kElems, L = G::kLanes;
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t unit = gid / L;
    const int gl = threadIdx.x % L;
    if (unit >= p.units)  // whole groups leave together: L divides 256
        return;
    const int64_t h = unit % p.H;
    const int64_t tstride = p.units * D;  // elements from one token's row to the next

    float qs[E], wv[E];
    widen<Tin>(load_slice<D, Tin, false>(static_cast<const Tin *>(p.q) + h * D, gl), qs);
#pragma unroll
    for (int e = 0; e < E; ++e)
        qs[e] *= p.scale;
    float *wp = p.w + unit * D;
    load_state<D, Tin>(wp, gl, wv);
    float m = p.m[unit], u = p.u[unit];

    const Tin *kp = static_cast<const Tin *>(p.k) + unit * D;
    const Tin *vp = static_cast<const Tin *>(p.v) + unit * D;
    Tout *op = EMIT ? static_cast<Tout *>(p.o) + unit * D : nullptr;
    int64_t t = 0;
#pragma unroll 1
    for (; t + R <= p.tokens; t += R)
        append_block<D, Tin, Tout, R, EMIT>(kp + t * tstride, vp + t * tstride,
                                            EMIT ? op + t * tstride : nullptr, tstride, gl, qs,
                                            m, u, wv);
#pragma unroll 1
    for (; t < p.tokens; ++t)
        append_block<D, Tin, Tout, 1, EMIT>(kp + t * tstride, vp + t * tstride,
                                            EMIT ? op + t * tstride : nullptr, tstride, gl, qs,
                                            m, u, wv);
    store_state<D, Tin>(wp, gl, wv);
    if (gl == 0) {
        p.m[unit] = m;
        p.u[unit] = u;
    }
}

// Empty state: m = -inf, u = 0, w = 0.
__global__ __launch_bounds__(256) void state_init_kernel(float *m, float *u, float *w,
                                                         int64_t units, int64_t D)
{
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < units; i += stride) {
        m[i] = kNegInf;
        u[i] = 0.f;
    }
    const int64_t n4 = units * D / 4;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += stride)
        store16(w + 4 * i, u32x4{0, 0, 0, 0});
}

// Zero a 16-byte aligned buffer whose size is a multiple of 16 bytes, then the tail.
__global__ __launch_bounds__(256) void fill_zero_kernel(uint8_t *p, size_t bytes)
{
    const size_t stride = (size_t)gridDim.x * 256;
    const size_t n16 = bytes / 16;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride)
        store16(p + 16 * i, u32x4{0, 0, 0, 0});
    const size_t t = n16 * 16 + (size_t)blockIdx.x * 256 + threadIdx.x;
    if (t < bytes)
        p[t] = 0;
}

template <int D, typename Tin, typename Tout>
static hipError_t step_one(const StepParams &p, hipStream_t stream)
{
    constexpr int L = RowGeo<D, Tin>::kLanes;
    const int64_t threads = p.units * L;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL((step_kernel<D, Tin, Tout>), dim3((unsigned)blocks), dim3(256), 0, stream,
                       p);
    return hipGetLastError();
}

template <int D>
static hipError_t step_dtypes(const StepParams &p, aaren_dtype in, aaren_dtype out,
                              hipStream_t stream)
{
    if (in == AAREN_F32)
        return out == AAREN_F32 ? step_one<D, float, float>(p, stream)
                                : step_one<D, float, bf16>(p, stream);
    return out == AAREN_F32 ? step_one<D, bf16, float>(p, stream)
                            : step_one<D, bf16, bf16>(p, stream);
}

hipError_t launch_step(const StepParams &p, int D, aaren_dtype in, aaren_dtype out,
                       hipStream_t stream)
{
    return D == 64 ? step_dtypes<64>(p, in, out, stream) : step_dtypes<128>(p, in, out, stream);
}

template <int D, typename Tin, typename Tout>
static hipError_t append_one(const StepParams &p, hipStream_t stream)
{
    constexpr int L = RowGeo<D, Tin>::kLanes;
    const int64_t threads = p.units * L;
    const int64_t blocks = (threads + 255) / 256;
    if (p.o)
        hipLaunchKernelGGL((append_kernel<D, Tin, Tout, 8, true>), dim3((unsigned)blocks),
                           dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((append_kernel<D, Tin, Tout, 8, false>), dim3((unsigned)blocks),
                           dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t append_dtypes(const StepParams &p, aaren_dtype in, aaren_dtype out,
                                hipStream_t stream)
{
    if (in == AAREN_F32)
        return out == AAREN_F32 ? append_one<D, float, float>(p, stream)
                                : append_one<D, float, bf16>(p, stream);
    return out == AAREN_F32 ? append_one<D, bf16, float>(p, stream)
                            : append_one<D, bf16, bf16>(p, stream);
}

hipError_t launch_append(const StepParams &p, int D, aaren_dtype in, aaren_dtype out,
                         hipStream_t stream)
{
    return D == 64 ? append_dtypes<64>(p, in, out, stream)
                   : append_dtypes<128>(p, in, out, stream);
}

static unsigned grid_for(int64_t work)
{
    int64_t b = (work + 255) / 256;
    if (b > 8192)
        b = 8192;
    return (unsigned)(b < 1 ? 1 : b);
}

hipError_t launch_state_init(float *m, float *u, float *w, int64_t units, int64_t D,
                             hipStream_t stream)
{
    const int64_t work = units * D / 4 > units ? units * D / 4 : units;
    hipLaunchKernelGGL(state_init_kernel, dim3(grid_for(work)), dim3(256), 0, stream, m, u, w,
                       units, D);
    return hipGetLastError();
}

// The next graph epoch in the workspace header (see kEpochWord).
__global__ __launch_bounds__(64) void epoch_advance_kernel(uint32_t *header)
{
    if (threadIdx.x == 0) {
        const uint32_t e = header[kEpochWord];
        header[kEpochWord] = (e < kGraphEpoch0 || e + 1 >= kGraphEpochEnd) ? kGraphEpoch0 : e + 1;
    }
}

hipError_t launch_epoch_advance(uint32_t *header, hipStream_t stream)
{
    hipLaunchKernelGGL(epoch_advance_kernel, dim3(1), dim3(64), 0, stream, header);
    return hipGetLastError();
}

// Copy a workspace's error word to *out, then clear it if asked.
__global__ __launch_bounds__(64) void workspace_status_kernel(uint32_t *header, uint32_t *out,
                                                              int reset)
{
    if (threadIdx.x == 0) {
        *out = __hip_atomic_load(header + kError, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (reset)
            __hip_atomic_store(header + kError, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

hipError_t launch_workspace_status(uint32_t *header, uint32_t *out, int reset, hipStream_t stream)
{
    hipLaunchKernelGGL(workspace_status_kernel, dim3(1), dim3(64), 0, stream, header, out, reset);
    return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream)
{
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for((int64_t)(bytes / 16) + 1)), dim3(256), 0,
                       stream, static_cast<uint8_t *>(p), bytes);
    return hipGetLastError();
}

}  // namespace aaren
