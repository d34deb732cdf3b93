// Many-to-one single-query attention (the attention of one query over all N
// key/value pairs: "Self-attention Does Not Need O(n^2) Memory" review,
// sections 1-2; "Attention as an RNN" review, abstract item (1)).
//
// Split along N: each workgroup reduces one contiguous chunk of a (b,h)
// sequence to a partial state (m, u, w); a second kernel combines the chunks'
// states per (b,h) and writes o = w/u. The pages note that the result does not
// depend on the order the pairs arrive in; only rounding does.
//
// Per iteration every lane group takes R consecutive rows (one 16-byte slice
// per lane per row), computes their scores, reduces them maximum-first and
// folds the batch into its running state, so the running maximum is rescaled
// once per batch rather than once per row. Exponentials are base 2.
#include "device.h"

namespace aaren {

template <int D, typename Tin, int R, int WAVES>
struct ReduceShape {
    using G = RowGeo<D, Tin>;
    static constexpr int E = G::kElems;
    static constexpr int L = G::kLanes;
    static constexpr int GPW = G::kGroupsPerWave;
    static constexpr int NG = WAVES * GPW;
    static constexpr int ROWS = NG * R;  // rows per workgroup iteration
    static constexpr int SLOT = slot_words(D);
};

template <int D, typename Tin, int R, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void reduce_partial_kernel(const ReduceParams p)
{
    using S = ReduceShape<D, Tin, R, WAVES>;
    constexpr int E = S::E, L = S::L, GPW = S::GPW, NG = S::NG, ROWS = S::ROWS;
    constexpr int SLOT = S::SLOT;

    __shared__ float sh_m[NG], sh_u[NG];
    __shared__ __attribute__((aligned(16))) float sh_w[NG][D];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gl = lane % L, grp = wave * GPW + lane / L;
    const int64_t unit = blockIdx.x / p.parts;
    const int64_t part = blockIdx.x - unit * p.parts;
    const int64_t begin = part * p.rows_per_part;
    int64_t end = begin + p.rows_per_part;
    end = end < p.N ? end : p.N;

    using SL = Slice<D, Tin>;
    float qv[E];
    if (p.q_unit)  // one float32 query per (b,h), at this lane's slice columns
        load_state<D, Tin>(p.q_unit + unit * D, gl, qv);
    else
        widen<Tin>(load_slice<D, Tin, false>(static_cast<const Tin *>(p.q) + (unit % p.H) * D, gl),
                   qv);
#pragma unroll
    for (int e = 0; e < E; ++e)
        qv[e] *= p.qscale;

    const Tin *kb = static_cast<const Tin *>(p.k) + unit * p.N * D;  // column 0
    const Tin *vb = static_cast<const Tin *>(p.v) + unit * p.N * D;

    float gm = kNegInf, gu = 0.f, gw[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        gw[e] = 0.f;

    for (int64_t it = begin; it < end; it += ROWS) {
        const int64_t row0 = it + (int64_t)grp * R;
        const int64_t left = end - row0;
        const int nvalid = left <= 0 ? 0 : (left >= R ? R : (int)left);
        u32x4 kr[R], vr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            kr[r] = u32x4{0, 0, 0, 0};
            vr[r] = u32x4{0, 0, 0, 0};
            if (r < nvalid) {
                kr[r] = load_slice<D, Tin, true>(kb + (row0 + r) * D, gl);
                vr[r] = load_slice<D, Tin, true>(vb + (row0 + r) * D, gl);
            }
        }
        float s[R];
        float bm = kNegInf;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float kf[E];
            widen<Tin>(kr[r], kf);
            float part_dot = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                part_dot = __builtin_fmaf(qv[e], kf[e], part_dot);
            s[r] = group_sum<L>(part_dot);
            s[r] = (r < nvalid) ? s[r] : kNegInf;
            bm = fmaxf(bm, s[r]);
        }
        if (nvalid > 0) {
            float bu = 0.f, bw[E];
#pragma unroll
            for (int e = 0; e < E; ++e)
                bw[e] = 0.f;
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float pr = (r < nvalid) ? exp2_fast(s[r] - bm) : 0.f;
                float vf[E];
                widen<Tin>(vr[r], vf);
                bu += pr;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    bw[e] = __builtin_fmaf(pr, vf[e], bw[e]);
            }
            float m, fa, fb;
            merge_weights(gm, bm, m, fa, fb);
            gu = fa * gu + fb * bu;
#pragma unroll
            for (int e = 0; e < E; ++e)
                gw[e] = fa * gw[e] + fb * bw[e];
            gm = m;
        }
    }

#pragma unroll
    for (int e = 0; e < E; ++e)
        sh_w[grp][SL::col(gl, e)] = gw[e];
    if (gl == 0) {
        sh_m[grp] = gm;
        sh_u[grp] = gu;
    }
    __syncthreads();
    if (wave == 0) {
        float am = kNegInf, au = 0.f, aw[D / 64];
#pragma unroll
        for (int c = 0; c < D / 64; ++c)
            aw[c] = 0.f;
        for (int g = 0; g < NG; ++g) {
            float m, fa, fb;
            merge_weights(am, sh_m[g], m, fa, fb);
            au = fa * au + fb * sh_u[g];
#pragma unroll
            for (int c = 0; c < D / 64; ++c)
                aw[c] = fa * aw[c] + fb * sh_w[g][lane + 64 * c];
            am = m;
        }
        float *out = p.partials + (size_t)blockIdx.x * SLOT;
#pragma unroll
        for (int c = 0; c < D / 64; ++c)
            out[2 + lane + 64 * c] = aw[c];
        if (lane == 0) {
            out[0] = am;
            out[1] = au;
        }
    }
}

// One workgroup of 1024 threads per (b,h): o = (sum_p f_p w_p) / (sum_p f_p u_p)
// with f_p = 2^(m_p - M), M the largest partial maximum. The partials (at most
// kReduceMaxParts of them) were just written; every thread issues its loads
// independently so that one workgroup drains them in a few load latencies.
constexpr int kFinalThreads = 1024;

__device__ __forceinline__ float block_reduce(float x, float *sh, bool is_max)
{
    // wave-level butterfly, then the 16 wave results through LDS
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const float y = __shfl_xor(x, off);
        x = is_max ? fmaxf(x, y) : x + y;
    }
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0)
        sh[wave] = x;
    __syncthreads();
    float r = sh[0];
    for (int i = 1; i < kFinalThreads / 64; ++i)
        r = is_max ? fmaxf(r, sh[i]) : r + sh[i];
    return r;
}

template <int D, typename Tout>
__global__ __launch_bounds__(kFinalThreads) void reduce_final_kernel(const ReduceParams p)
{
    constexpr int SLOT = slot_words(D);
    constexpr int SUB = kFinalThreads / D;  // partial subsets per column
    __shared__ float sh_f[kReduceMaxParts];
    __shared__ float sh_red[kFinalThreads / 64];
    __shared__ float sh_col[SUB][D];

    const int tid = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const float *base = p.partials + (size_t)unit * p.parts * SLOT;
    const int P = (int)p.parts;  // <= kReduceMaxParts <= kFinalThreads

    const float mi = tid < P ? base[(size_t)tid * SLOT] : kNegInf;
    const float ui = tid < P ? base[(size_t)tid * SLOT + 1] : 0.f;
    const float M = block_reduce(mi, sh_red, true);
    const float f = (mi == kNegInf) ? 0.f : exp2_fast(mi - M);
    if (tid < P)
        sh_f[tid] = f;
    const float U = block_reduce(f * ui, sh_red, false);  // syncs: sh_f is visible after

    const int col = tid % D, sub = tid / D;
    float acc = 0.f;
#pragma unroll 16
    for (int i = sub; i < P; i += SUB)
        acc = __builtin_fmaf(sh_f[i], base[(size_t)i * SLOT + 2 + col], acc);
    sh_col[sub][col] = acc;
    __syncthreads();
    if (tid < D) {
        float w = 0.f;
#pragma unroll
        for (int s = 0; s < SUB; ++s)
            w += sh_col[s][tid];
        const float val = w * rcp_fast(U);
        Tout *o = static_cast<Tout *>(p.o) + unit * D;
        if constexpr (sizeof(Tout) == 4)
            reinterpret_cast<float *>(o)[tid] = val;
        else
            reinterpret_cast<uint16_t *>(o)[tid] = (uint16_t)bf16_bits(val);
    }
    if (tid == 0) {
        if (p.m_out)
            p.m_out[unit] = M * kLn2;
        if (p.u_out)
            p.u_out[unit] = U;
    }
}

// Mean query of each (b,h) (the global-aggregation query of the pooling
// network reviewed on the efficient-transformer page: the average of the
// query projections): g = (1/N) sum_n hq[n]. Column sums in float64, each
// workgroup over one chunk of rows (the reduction's chunks), then the chunks
// added in order, so g is the same bits on every run; g is rounded to float32
// once, the precision of every query in this library.
template <int D, typename Tin>
__global__ __launch_bounds__(256) void mean_partial_kernel(const ReduceParams p)
{
    using G = RowGeo<D, Tin>;
    using SL = Slice<D, Tin>;
    constexpr int E = G::kElems, L = G::kLanes, NG = 4 * G::kGroupsPerWave;
    __shared__ double sh[NG][D];
    const int tid = threadIdx.x, gl = tid % L, grp = tid / L;
    const int64_t unit = blockIdx.x / p.parts, part = blockIdx.x - unit * p.parts;
    const int64_t begin = part * p.rows_per_part;
    int64_t end = begin + p.rows_per_part;
    end = end < p.N ? end : p.N;
    const Tin *hb = static_cast<const Tin *>(p.q) + unit * p.N * D;
    double acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        acc[e] = 0.0;
    for (int64_t row = begin + grp; row < end; row += NG) {
        float x[E];
        widen<Tin>(load_slice<D, Tin, true>(hb + row * D, gl), x);
#pragma unroll
        for (int e = 0; e < E; ++e)
            acc[e] += (double)x[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        sh[grp][SL::col(gl, e)] = acc[e];
    __syncthreads();
    if (tid < D) {
        double t = 0.0;
        for (int g = 0; g < NG; ++g)
            t += sh[g][tid];
        p.mean_partials[(size_t)blockIdx.x * D + tid] = t;
    }
}

template <int D>
__global__ __launch_bounds__(D) void mean_final_kernel(const ReduceParams p)
{
    const int col = threadIdx.x;
    const int64_t unit = blockIdx.x;
    const double *base = p.mean_partials + (size_t)unit * p.parts * D;
    double t = 0.0;
    for (int64_t i = 0; i < p.parts; ++i)
        t += base[(size_t)i * D + col];
    const float g = (float)(t / (double)p.N);
    p.q_mean[unit * D + col] = g;
    if (p.g_out)
        p.g_out[unit * D + col] = g;
}

template <int D>
static hipError_t mean_one(const ReduceParams &p, aaren_dtype in, hipStream_t stream)
{
    if (in == AAREN_F32)
        hipLaunchKernelGGL((mean_partial_kernel<D, float>), dim3((unsigned)(p.units * p.parts)),
                           dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL((mean_partial_kernel<D, bf16>), dim3((unsigned)(p.units * p.parts)),
                           dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((mean_final_kernel<D>), dim3((unsigned)p.units), dim3(D), 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_mean_query(const ReduceParams &p, int D, aaren_dtype in, hipStream_t stream)
{
    return D == 64 ? mean_one<64>(p, in, stream) : mean_one<128>(p, in, stream);
}

template <int D, typename Tin>
struct ReduceConfig {
    static constexpr int R = 8, WAVES = 8;
};

template <int D, typename Tin, typename Tout>
static hipError_t reduce_one(const ReduceParams &p, hipStream_t stream)
{
    constexpr int R = ReduceConfig<D, Tin>::R, WAVES = ReduceConfig<D, Tin>::WAVES;
    hipLaunchKernelGGL((reduce_partial_kernel<D, Tin, R, WAVES>),
                       dim3((unsigned)(p.units * p.parts)), dim3(64 * WAVES), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    hipLaunchKernelGGL((reduce_final_kernel<D, Tout>), dim3((unsigned)p.units),
                       dim3(kFinalThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t reduce_dtypes(const ReduceParams &p, aaren_dtype in, aaren_dtype out,
                                hipStream_t stream)
{
    if (in == AAREN_F32)
        return out == AAREN_F32 ? reduce_one<D, float, float>(p, stream)
                                : reduce_one<D, float, bf16>(p, stream);
    return out == AAREN_F32 ? reduce_one<D, bf16, float>(p, stream)
                            : reduce_one<D, bf16, bf16>(p, stream);
}

hipError_t launch_reduce(const ReduceParams &p, int D, aaren_dtype in, aaren_dtype out,
                         hipStream_t stream)
{
    return D == 64 ? reduce_dtypes<64>(p, in, out, stream) : reduce_dtypes<128>(p, in, out, stream);
}

template <int D, typename Tin>
static int rows_per_iteration()
{
    return ReduceShape<D, Tin, ReduceConfig<D, Tin>::R, ReduceConfig<D, Tin>::WAVES>::ROWS;
}

int reduce_rows_per_iteration(int D, aaren_dtype in)
{
    if (D == 64)
        return in == AAREN_F32 ? rows_per_iteration<64, float>() : rows_per_iteration<64, bf16>();
    return in == AAREN_F32 ? rows_per_iteration<128, float>() : rows_per_iteration<128, bf16>();
}

}  // namespace aaren
