// Device helpers for the libaaren kernels (gfx950, wave64).
//
// Row geometry: a key/value row of D elements is read 16 bytes per lane, so a
// row is spread over kLanes consecutive lanes of one wavefront ("a group") and
// one wave-wide load covers kGroupsPerWave rows. Every row the workloads use
// is 256 bytes (d=64 fp32 or d=128 bf16): 16 lanes x 16 B, 4 rows per wave.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace aaren {

// Storage type of a bfloat16 element (raw bits).
struct bf16 {
    uint16_t bits;
};

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kNegInf = -__builtin_inff();

template <int D, typename Tin>
struct RowGeo {
    static constexpr int kElems = 16 / (int)sizeof(Tin);  // elements per lane load
    static constexpr int kLanes = D / kElems;             // lanes sharing one row
    static constexpr int kGroupsPerWave = 64 / kLanes;    // rows per wave-wide load
    static_assert(kLanes >= 4 && kLanes <= 32 && (kLanes & (kLanes - 1)) == 0,
                  "a row must span 4..32 lanes");
};

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load16(const void *p)
{
    return *reinterpret_cast<const u32x4 *>(p);
}

// Streaming read of data touched once (keys, values): a non-temporal load, so
// the 16-byte slices do not displace what the caches still hold. Measured on
// the dense workload: 127 us instead of 155 us per call.
__device__ __forceinline__ u32x4 load16_stream(const void *p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ void store16(void *p, u32x4 v)
{
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Streaming write of results nobody re-reads in this call: non-temporal.
// Measured with inputs rotated beyond the 256 MB Infinity Cache: dense batch
// 143 -> 135 us, packed batch 17.1 -> 16.3 ms per call.
__device__ __forceinline__ void store16_stream(void *p, u32x4 v)
{
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Widen one 16-byte chunk into E floats (bf16 -> fp32 is exact).
template <typename T>
__device__ __forceinline__ void widen(u32x4 raw, float *out);

template <>
__device__ __forceinline__ void widen<float>(u32x4 raw, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i)
        out[i] = __uint_as_float(raw[i]);
}

template <>
__device__ __forceinline__ void widen<bf16>(u32x4 raw, float *out)
{
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        out[2 * i] = __uint_as_float(raw[i] << 16);
        out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    }
}

// fp32 -> bf16 bits, round to nearest even; NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    uint32_t x = __float_as_uint(f);
    if ((x & 0x7fffffffu) > 0x7f800000u)
        return (x >> 16) | 0x40u;
    return (x + 0x7fffu + ((x >> 16) & 1u)) >> 16;
}

// The columns a lane owns in a row of D elements: its E elements form E/4
// chunks of 4 consecutive columns, chunk c starting at column
// c * (D / (E/4)) + 4 * gl (gl = lane within its group). One wave-wide access
// of a chunk then covers a contiguous run of every row it touches, for loads
// (16 bytes of fp32 or 2 x 8 bytes of bf16 per lane) and for fp32 or bf16
// stores alike, so no store leaves a partial cache line behind.
template <int D, typename Tin>
struct Slice {
    static constexpr int E = RowGeo<D, Tin>::kElems;
    static constexpr int NC = E / 4;      // chunks per lane
    static constexpr int STRIDE = D / NC; // columns between chunks
    __device__ static constexpr int col(int gl, int e)
    {
        return (e / 4) * STRIDE + 4 * gl + (e % 4);
    }
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// The lane's 16-byte slice of a row (row points at column 0), raw bits; chunk
// c occupies words 2c..2c+1 (bf16) or all four words (fp32).
template <int D, typename Tin, bool STREAM>
__device__ __forceinline__ u32x4 load_slice(const Tin *row, int gl)
{
    if constexpr (sizeof(Tin) == 4) {
        return STREAM ? load16_stream(row + 4 * gl) : load16(row + 4 * gl);
    } else {
        const u32x2 *a = reinterpret_cast<const u32x2 *>(row + 4 * gl);
        const u32x2 *b = reinterpret_cast<const u32x2 *>(row + D / 2 + 4 * gl);
        const u32x2 x = STREAM ? __builtin_nontemporal_load(a) : *a;
        const u32x2 y = STREAM ? __builtin_nontemporal_load(b) : *b;
        return u32x4{x[0], x[1], y[0], y[1]};
    }
}

// Store the lane's E floats of a row as Tout (row points at column 0), streaming.
template <int D, typename Tin, typename Tout>
__device__ __forceinline__ void store_slice(Tout *row, int gl, const float *x)
{
    using S = Slice<D, Tin>;
#pragma unroll
    for (int c = 0; c < S::NC; ++c) {
        Tout *dst = row + c * S::STRIDE + 4 * gl;
        if constexpr (sizeof(Tout) == 4) {
            u32x4 v = {__float_as_uint(x[4 * c]), __float_as_uint(x[4 * c + 1]),
                       __float_as_uint(x[4 * c + 2]), __float_as_uint(x[4 * c + 3])};
            store16_stream(dst, v);
        } else {
            u32x2 v = {bf16_bits(x[4 * c]) | (bf16_bits(x[4 * c + 1]) << 16),
                       bf16_bits(x[4 * c + 2]) | (bf16_bits(x[4 * c + 3]) << 16)};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(dst));
        }
    }
}

// The lane's E fp32 state columns of a row (row points at column 0).
template <int D, typename Tin>
__device__ __forceinline__ void load_state(const float *row, int gl, float *x)
{
    using S = Slice<D, Tin>;
#pragma unroll
    for (int c = 0; c < S::NC; ++c)
        widen<float>(load16(row + c * S::STRIDE + 4 * gl), x + 4 * c);
}

template <int D, typename Tin>
__device__ __forceinline__ void store_state(float *row, int gl, const float *x)
{
    using S = Slice<D, Tin>;
#pragma unroll
    for (int c = 0; c < S::NC; ++c) {
        u32x4 v = {__float_as_uint(x[4 * c]), __float_as_uint(x[4 * c + 1]),
                   __float_as_uint(x[4 * c + 2]), __float_as_uint(x[4 * c + 3])};
        store16(row + c * S::STRIDE + 4 * gl, v);
    }
}

// x + (x from the lane selected by the DPP control); the whole wave is active.
template <int CTRL>
__device__ __forceinline__ float dpp_add(float x)
{
    return x + __builtin_bit_cast(
                   float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF,
                                                      0xF, true));
}

// Sum over the L lanes of a group (L = 4, 8, 16 or 32, aligned): a butterfly,
// so every lane ends with the bitwise-identical sum.
template <int L>
__device__ __forceinline__ float group_sum(float x)
{
    x = dpp_add<0xB1>(x);  // quad_perm [1,0,3,2]: lane ^ 1
    x = dpp_add<0x4E>(x);  // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (L >= 8)
        x = dpp_add<0x141>(x);  // row_half_mirror: the other quad of 8 lanes
    if constexpr (L >= 16)
        x = dpp_add<0x140>(x);  // row_mirror: the other half of 16 lanes
    if constexpr (L >= 32)
        x += __builtin_bit_cast(float,
                                __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401F));
    return x;
}

__device__ __forceinline__ float exp2_fast(float x)
{
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float log2_fast(float x)
{
    return __builtin_amdgcn_logf(x);
}

__device__ __forceinline__ float rcp_fast(float x)
{
    return __builtin_amdgcn_rcpf(x);
}

// Weights for combining two states with maxima ma and mb (log2 units):
// m = max(ma, mb), fa = 2^(ma - m), fb = 2^(mb - m). An empty side (-inf)
// gets weight 0; two empty sides give m = -inf, fa = 1, fb = 0.
__device__ __forceinline__ void merge_weights(float ma, float mb, float &m, float &fa, float &fb)
{
    const bool b_big = mb > ma;
    const float hi = b_big ? mb : ma;
    const float lo = b_big ? ma : mb;
    float e = exp2_fast(lo - hi);
    e = (lo == kNegInf) ? 0.f : e;
    fa = b_big ? e : 1.f;
    fb = b_big ? 1.f : e;
    m = hi;
}

// (m,u,w) = (m_a,u_a,w_a) (+) (m_b,u_b,w_b) over N columns, the earlier state
// on the left. Written with explicit fma so that every call site rounds the
// same way (the scan's cross-tile carry relies on that to be reproducible).
// w may alias aw or bw.
template <int N>
__device__ __forceinline__ void combine(float am, float au, const float *aw, float bm, float bu,
                                        const float *bw, float &m, float &u, float *w)
{
    float fa, fb, mm;
    merge_weights(am, bm, mm, fa, fb);
    u = __builtin_fmaf(fa, au, fb * bu);
#pragma unroll
    for (int i = 0; i < N; ++i)
        w[i] = __builtin_fmaf(fa, aw[i], fb * bw[i]);
    m = mm;
}

// 64-bit agent-scope relaxed accesses (coherent across the XCDs' L2s).
__device__ __forceinline__ void st_agent(uint64_t *p, uint64_t v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t ld_agent(const uint64_t *p)
{
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace aaren
