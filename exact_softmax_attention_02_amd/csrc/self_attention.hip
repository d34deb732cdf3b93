// Self-attention with one query per token, on the matrix cores.
//
// The memory-efficient-attention review (section 2) extends the single-query
// algorithm to self-attention by evaluating every query in turn with the same
// constant-memory recurrence; its GPU/TPU section (body lost) and its
// introduction mention chunking. Here each workgroup carries 128 queries
// through the keys 64 at a time with the same running-maximum combine as the
// single-query path: per key tile, S = scale K Q^T on the bf16 matrix cores,
// the new running maximum per query, P = e^{S - m}, and O += P V; the
// normaliser is divided out at the end. Causal: query i attends to keys 0..i.
//
// Layout choices (gfx950, wave64, v_mfma_f32_32x32x16_bf16: lane l holds 8
// consecutive k of row l%32 of A and of column l%32 of B; accumulator
// register r of lane l is row 8(r/4) + 4(l/32) + r%4, column l%32):
//  * Scores are computed transposed, S^T = K Q^T, so a query is a column: a
//    lane owns one query (l%32) and 16 keys per 32-key block, and the row
//    maximum and sum need one exchange between the two half-waves.
//  * The K rows feeding the A operand are permuted (row m of the MFMA reads
//    key kappa(m)) so that accumulator registers 8s..8s+7 of a lane hold 8
//    consecutive keys: they are then directly the B operand of
//    O^T += V^T P^T for that 16-key step, with no data movement.
//  * V^T must present 8 consecutive keys of one dimension per lane; V is
//    transposed once into the workspace by a pre-pass, so its tiles load
//    into LDS as plain rows.
//  * The value product runs in fp16 (v_mfma_f32_32x32x16_f16), whose 11
//    significant bits move an output by at most ~2^-12 max|v| where bf16's 8
//    would take ~2^-9 max|v|, the whole budget of the bf16 tolerance. V is
//    multiplied per (b,h) by a power of two 2^e that brings its largest
//    magnitude just under 2^15 (so every bf16 value of V at or above 2^-17 of
//    that scale converts exactly), and the output by 2^-e. The weights are
//    taken as 2^7 e^{s - m}: the running maximum moves only when a score
//    exceeds it by more than a factor 2^8, so they stay below 2^15, and only
//    weights under 2^-21 of the maximum fall into fp16's subnormals. The
//    normaliser sums the weights in fp32.
#include <type_traits>

#include "device.h"
#include "self_attention.h"

namespace aaren {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void *lptr;

// Fourth word of a raw buffer descriptor on gfx9-family chips (32-bit data
// format, no stride, no swizzle): buffer loads then read bytes [0, count) of
// the buffer and return zeros beyond.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32h(u32x4 a, f16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), b, c, 0, 0, 0);
}

// Partial maxima of the finite |v| over [BH][N][D], as bf16 magnitude bits
// (which order like the magnitudes; infinities and NaNs are left out, so they
// do not set the scale): part c of head bh covers keys [c*len, (c+1)*len),
// len = ceil(N / kAttnVmaxParts).
template <int D>
__global__ __launch_bounds__(256) void attn_vmax_kernel(const AttnParams p)
{
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.y;
    const int64_t len = (p.N + kAttnVmaxParts - 1) / kAttnVmaxParts;
    int64_t k0 = blockIdx.x * len, k1 = k0 + len;
    k1 = k1 < p.N ? k1 : p.N;
    k0 = k0 < k1 ? k0 : k1;
    const uint16_t *src = p.v + (bh * p.N + k0) * D;
    const int64_t chunks = (k1 - k0) * (D / 8);  // 16-byte chunks
    uint32_t mx = 0;
    auto fold = [&](u32x4 x) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            uint32_t a = x[e] & 0x7fffu, b = (x[e] >> 16) & 0x7fffu;
            a = a < 0x7f80u ? a : 0u;
            b = b < 0x7f80u ? b : 0u;
            mx = mx > a ? mx : a;
            mx = mx > b ? mx : b;
        }
    };
    // four loads in flight per thread, then the remainder
    int64_t c = tid;
    for (; c + 3 * 256 < chunks; c += 4 * 256) {
        u32x4 x[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            x[i] = load16(src + 8 * (c + 256 * i));
#pragma unroll
        for (int i = 0; i < 4; ++i)
            fold(x[i]);
    }
    for (; c < chunks; c += 256)
        fold(load16(src + 8 * c));
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mx, off);
        mx = mx > o ? mx : o;
    }
    if ((tid & 63) == 0)
        red[tid >> 6] = mx;
    __syncthreads();
    if (tid == 0) {
        uint32_t r = red[0];
        for (int w = 1; w < 4; ++w)
            r = r > red[w] ? r : red[w];
        p.vmax[bh * kAttnVmaxParts + blockIdx.x] = r;
    }
}

// The exponent e of head bh's value scale 2^e, from its partial maxima (one
// wave reads them all): the largest finite |v| < 2^(E - 126) for bf16
// exponent field E <= 254, so e = 141 - E >= -113 puts it below 2^15. Capped
// at 126 (zero or subnormal V). Infinities and NaNs stay what they are.
__device__ __forceinline__ int attn_value_exponent(const AttnParams &p, int64_t bh, int lane)
{
    uint32_t mx = p.vmax[bh * kAttnVmaxParts + lane];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        const uint32_t o = (uint32_t)__shfl_xor((int)mx, off);
        mx = mx > o ? mx : o;
    }
    const int E = (int)(mx >> 7);
    return 141 - E < 126 ? 141 - E : 126;
}

__device__ __forceinline__ float pow2f(int e)  // 2^e for -126 <= e <= 127
{
    return __uint_as_float((uint32_t)(e + 127) << 23);
}

// V [BH][N][D] bf16 -> 2^e V^T [BH][D][Np] fp16 (rounded to nearest), zero
// for keys N..Np-1. One workgroup per 64 keys x 64 dimensions.
template <int D>
__global__ __launch_bounds__(256) void attn_transpose_kernel(const AttnParams p)
{
    __shared__ uint16_t t[64][64 + 2];  // [key][dim]
    const int tid = threadIdx.x;
    const int64_t bh = blockIdx.z, key0 = (int64_t)blockIdx.x * 64, dim0 = blockIdx.y * 64;
    const float vscale = pow2f(attn_value_exponent(p, bh, tid & 63));
    for (int c = tid; c < 512; c += 256) {
        const int key = c / 8, ch = c % 8;
        u32x4 x = {0, 0, 0, 0};
        if (key0 + key < p.N)
            x = load16(p.v + ((bh * p.N + key0 + key) * D + dim0 + 8 * ch));
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const f32x2 f = {__uint_as_float(x[e] << 16) * vscale,
                             __uint_as_float(x[e] & 0xffff0000u) * vscale};
            const uint32_t h = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
            t[key][8 * ch + 2 * e] = (uint16_t)(h & 0xffffu);
            t[key][8 * ch + 2 * e + 1] = (uint16_t)(h >> 16);
        }
    }
    __syncthreads();
    for (int c = tid; c < 512; c += 256) {
        const int dim = c / 8, kc = c % 8;
        u32x4 y;
#pragma unroll
        for (int e = 0; e < 4; ++e)
            y[e] = (uint32_t)t[8 * kc + 2 * e][dim] | ((uint32_t)t[8 * kc + 2 * e + 1][dim] << 16);
        store16(p.vt + ((bh * D + dim0 + dim) * p.Np + key0 + 8 * kc), y);
    }
}

template <typename Tout>
__device__ __forceinline__ void store4(Tout *dst, float a, float b, float c, float d)
{
    if constexpr (sizeof(Tout) == 4) {
        store16(dst, u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c),
                           __float_as_uint(d)});
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        *reinterpret_cast<u32x2 *>(dst) =
            u32x2{bf16_bits(a) | (bf16_bits(b) << 16), bf16_bits(c) | (bf16_bits(d) << 16)};
    }
}

template <int D, typename Tout>
__global__ __launch_bounds__(64 * kAttnWaves, D == 64 ? 4 : 2) void self_attention_kernel(const AttnParams p)
{
    constexpr int KS = D / 16;          // 16-wide k-steps of S^T = K Q^T
    constexpr int DT = D / 32;          // 32-row tiles of O^T
    constexpr int KC = D / (8 * kAttnWaves);  // 1 KB copies per wave per tile (K and V^T each)
    // Two buffers per operand, each its own array: the tile copies below write
    // LDS asynchronously (counted by vmcnt), and the compiler makes a read of
    // LDS wait for every copy that may land in the same array. With the
    // buffers apart and the buffer index a compile-time constant (d = 128),
    // reading tile j no longer waits for tile j+1's copies.
    __shared__ __attribute__((aligned(16))) uint16_t sk0[kAttnKeys * D];
    __shared__ __attribute__((aligned(16))) uint16_t sk1[kAttnKeys * D];
    __shared__ __attribute__((aligned(16))) uint16_t sv0[D * kAttnKeys];
    __shared__ __attribute__((aligned(16))) uint16_t sv1[D * kAttnKeys];
    // a buffer index is a compile-time constant (std::integral_constant) or,
    // on the d = 64 path, an int
    auto skb = [&](auto b) -> uint16_t * {
        if constexpr (std::is_integral_v<decltype(b)>) return b ? sk1 : sk0;
        else if constexpr (decltype(b)::value == 0) return sk0;
        else return sk1;
    };
    auto svb = [&](auto b) -> uint16_t * {
        if constexpr (std::is_integral_v<decltype(b)>) return b ? sv1 : sv0;
        else if constexpr (decltype(b)::value == 0) return sv0;
        else return sv1;
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int h32 = lane >> 5, l32 = lane & 31;
    // Heads go in groups of kAttnHeadGroup (16); within a group the query
    // tiles go longest first (causal), the group's heads taking turns.
    // Workgroups are dealt to the 8 XCDs in turn, so each XCD serves two heads
    // of a group (its L2 holds their keys), and every XCD's own list runs
    // longest first across its heads, which keeps the causal tail short.
    const int64_t nqt = (p.N + kAttnQueries - 1) / kAttnQueries;
    const int64_t g0 = (int64_t)blockIdx.x / (kAttnHeadGroup * nqt) * kAttnHeadGroup;
    const int64_t gs = p.bh - g0 < kAttnHeadGroup ? p.bh - g0 : kAttnHeadGroup;
    const int64_t r = (int64_t)blockIdx.x - g0 * nqt;
    const int64_t bh = g0 + r % gs;
    const int64_t q0 = (nqt - 1 - r / gs) * kAttnQueries;
    const int64_t qi = q0 + 32 * wave + l32;  // this lane's query

    // a negative scale is moved into q (flipping a bf16 sign is exact), so the
    // scores' scale c2 below is never negative and a maximum of raw scores is
    // the maximum of scaled ones
    const uint32_t qflip = p.qscale < 0.f ? 0x80008000u : 0u;
    bf16x8 qf[KS];
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        u32x4 x = {0, 0, 0, 0};
        if (qi < p.N)
            x = load16(p.q + ((bh * p.N + qi) * D + 16 * kk + 8 * h32)) ^ qflip;
        qf[kk] = __builtin_bit_cast(bf16x8, x);
    }

    const int64_t kend = (p.causal && q0 + kAttnQueries < p.N) ? q0 + kAttnQueries : p.N;
    const int ntiles = (int)((kend + kAttnKeys - 1) / kAttnKeys);

    // Tiles go from global memory straight into LDS (buffer loads with the
    // lds flag: lane i of a wave writes 16 bytes at M0 + 16 i). Rows are
    // unpadded; the 16-byte chunks of a row are stored XOR-swizzled so that the
    // fragment reads below (16 lanes, 16 different rows, one chunk column) hit
    // 16 different bank groups: K row r (D/8 chunks) keeps chunk c at position
    // c ^ kswz(r); a V^T row (8 chunks of 8 keys) at c ^ vswz(r).
    auto kswz = [](int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); };
    auto vswz = [](int r) { return (r >> 1) & 7; };
    constexpr int KRPI = 1024 / (2 * D);  // K rows per 1 KB copy
    const uint16_t *kh = p.k + bh * p.N * D;
    const uint16_t *vth = p.vt + bh * D * p.Np;
    // Copy c of a wave fills 1 KB block kAttnWaves * c + wave of the tile, the
    // rows of its copy 0 plus 4 * kAttnWaves * c (K, d = 128) or
    // 8 * kAttnWaves * c (V^T); d = 64 takes one copy per operand. Both
    // swizzles depend on a row modulo 16 only, so every copy of a lane uses
    // copy 0's byte offset (one VGPR per operand); the rest is scalar. V^T and
    // every K tile that ends at or before N go through one buffer per head,
    // the tile's start and the copy's step as the scalar offset; neither
    // leaves that buffer (V^T reads stay in the head's padded rows). The last
    // K tile, which may pass N, gives each copy a buffer of its own whose
    // record count ends at the head's last key, so rows past N read as zeros
    // (masked later). Offsets and counts stay below 2^31 for N <= kAttnMaxN.
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int kr0 = wv * KRPI + lane / (D / 8);
    const uint32_t koff = (uint32_t)(kr0 * 2 * D + 16 * ((lane % (D / 8)) ^ kswz(kr0)));
    const int vr0 = wv * 8 + lane / 8;
    const uint32_t voff = (uint32_t)(vr0 * 2 * p.Np + 16 * ((lane % 8) ^ vswz(vr0)));
    const uint32_t vstep = (uint32_t)(16 * kAttnWaves * p.Np);  // 8 * kAttnWaves V^T rows, in bytes
    // one descriptor per head for K (tiles that end at or before N) and V^T
    const auto khr = __builtin_amdgcn_make_buffer_rsrc((void *)kh, (short)0, (int)(p.N * 2 * D), kBufferWord3);
    const auto vtr = __builtin_amdgcn_make_buffer_rsrc((void *)vth, (short)0, (int)(D * p.Np * 2), kBufferWord3);
    auto load_tile = [&](int j, auto buf) {
        const int64_t k0 = (int64_t)j * kAttnKeys;
        if (k0 + kAttnKeys <= p.N) {
#pragma unroll
            for (int c = 0; c < KC; ++c)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(khr, (lptr)(skb(buf) + (kAttnWaves * c + wv) * 512), 16,
                                                         koff, (int)(k0 * 2 * D) + 1024 * kAttnWaves * c, 0, 0);
        } else {
            // the last tile: each copy's record count ends at the head's last key
            const int64_t kbytes = (p.N - k0) * 2 * D;
#pragma unroll
            for (int c = 0; c < KC; ++c) {
                const int64_t left = kbytes - 1024 * kAttnWaves * c;
                const auto kr = __builtin_amdgcn_make_buffer_rsrc(
                    (void *)(kh + k0 * D + 512 * kAttnWaves * c), (short)0, (int)(left > 0 ? left : 0), kBufferWord3);
                __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lptr)(skb(buf) + (kAttnWaves * c + wv) * 512),
                                                         16, koff, 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < KC; ++c)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vtr, (lptr)(svb(buf) + (kAttnWaves * c + wv) * 512), 16,
                                                     voff, (int)(2 * k0) + (int)(vstep * c), 0, 0);
    };

    load_tile(0, B0{});
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    f32x16 oacc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = f32x16{};
    float m = kNegInf, lsum = 0.f;  // m in log2 units; lsum: this half-wave's keys only

    // A-operand row m = l32 of each 32-key block reads key kappa(m)
    const int krow = 16 * (l32 >> 4) + 8 * ((l32 >> 2) & 1) + 4 * ((l32 >> 3) & 1) + (l32 & 3);
    // scores are scaled inside the exponent: e^{c2 s - m}
    const float c2 = fabsf(p.qscale);

    // One key tile. EDGE: the tile holds keys past N or past some query of
    // this workgroup (causal); keys at offset >= lim from the tile's first key
    // are then masked for this lane's query (excluded from the maximum, weight
    // exactly 0).
    auto tile = [&](auto buf, int lim, auto edge_tag) {
        constexpr bool EDGE = decltype(edge_tag)::value;
        auto kfrag = [&](int t, int kk) {
            return load16(skb(buf) + (32 * t + krow) * D + 8 * ((2 * kk + h32) ^ kswz(32 * t + krow)));
        };
        f32x16 s[2] = {f32x16{}, f32x16{}};
        if constexpr (D == 128) {
            // all 16 K fragments are read before the products (the registers
            // are free at this point of the tile); read one at a time, each
            // product of the first chain waited for its own LDS read
            u32x4 kf[2][KS];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    kf[t][kk] = kfrag(t, kk);
#pragma unroll
            for (int kk = 0; kk < KS; ++kk)
#pragma unroll
                for (int t = 0; t < 2; ++t)
                    s[t] = mfma32(kf[t][kk], qf[kk], s[t]);
        } else {
            // d = 64 is held to 128 VGPRs: fragments are read at their products
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk)
                    s[t] = mfma32(kfrag(t, kk), qf[kk], s[t]);
        }
        auto key_off = [&](int t, int r) { return 32 * t + 16 * (r >> 3) + 8 * h32 + (r & 7); };
        float tx = kNegInf;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                tx = fmaxf(tx, (!EDGE || key_off(t, r) < lim) ? s[t][r] : kNegInf);
        {
            // lanes l and l ^ 32 hold the same query: v_permlane32_swap of tx
            // with itself gives one of them in each result
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(tx), __float_as_uint(tx),
                                                             false, false);
            tx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        }
        // The maximum is moved only when a score exceeds it by more than 8
        // (log2 units): the weights then stay below 2^8 (2^15 with the 2^7
        // offset), and the rescale of O (and its register traffic) is skipped
        // on most tiles. The quotient does not depend on the reference. A lane
        // whose keys are all masked has tx = -inf; with a zero scale tx * c2 is
        // NaN and the comparison keeps m.
        const float mnew = (tx * c2 > m + 8.f) ? tx * c2 : m;
        const float alpha = exp2_fast(m - mnew);  // 0 on the first tile (m = -inf)
        m = mnew;
        lsum *= alpha;
        if (__any(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                oacc[dt] *= alpha;
        }
        // O^T += V^T P^T, 16 keys per step, P = 2^7 e^{s - m} in fp16
        const float mk = mnew - 7.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
#pragma unroll
            for (int s2 = 0; s2 < 2; ++s2) {
                f32x8 pe;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    pe[e] = exp2_fast(__builtin_fmaf(s[t][8 * s2 + e], c2, -mk));
                    if (EDGE && key_off(t, 8 * s2 + e) >= lim)
                        pe[e] = 0.f;
                    lsum += pe[e];
                }
                const f16x8 ph = __builtin_convertvector(pe, f16x8);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt) {
                    const int vr = 32 * dt + l32;
                    const u32x4 a = load16(svb(buf) + vr * kAttnKeys +
                                                    8 * ((4 * t + 2 * s2 + h32) ^ vswz(vr)));
                    oacc[dt] = mfma32h(a, ph, oacc[dt]);
                }
            }
        }
    };

    // tiles 0..nfull-1 need no mask: every key is below N and, causal, below
    // every query of the workgroup
    int64_t nfull = p.N / kAttnKeys;
    if (p.causal && (q0 + 1) / kAttnKeys < nfull)
        nfull = (q0 + 1) / kAttnKeys;
    // the loops go two tiles per trip, so that every buffer index is a constant
    auto full = [&](int jj, auto buf, auto other) {
        if (jj + 1 < ntiles)
            load_tile(jj + 1, other);  // that buffer was last read before the previous barrier
        tile(buf, kAttnKeys, std::integral_constant<bool, false>{});
        __builtin_amdgcn_s_waitcnt(0);  // this wave's copies of the next tile have landed
        __syncthreads();
    };
    auto edge = [&](int jj, auto buf, auto other) {
        if (jj + 1 < ntiles)
            load_tile(jj + 1, other);
        const int64_t k0 = (int64_t)jj * kAttnKeys;
        int64_t lim = p.N - k0;
        if (p.causal && qi + 1 - k0 < lim)
            lim = qi + 1 - k0;
        tile(buf, lim < 0 ? 0 : (lim > kAttnKeys ? kAttnKeys : (int)lim),
             std::integral_constant<bool, true>{});
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    int j = 0;
    if constexpr (D == 64) {
        // held to 128 VGPRs: one loop body, the buffer chosen at run time
        for (; j < (int)nfull; ++j)
            full(j, j & 1, (j & 1) ^ 1);
        for (; j < ntiles; ++j)
            edge(j, j & 1, (j & 1) ^ 1);
    } else {
        for (; j + 1 < (int)nfull; j += 2) {
            full(j, B0{}, B1{});
            full(j + 1, B1{}, B0{});
        }
        if (j < (int)nfull) {
            full(j, B0{}, B1{});
            ++j;
        }
        // tile j is in buffer j & 1
        if ((j & 1) && j < ntiles) {
            edge(j, B1{}, B0{});
            ++j;
        }
        for (; j < ntiles; j += 2) {
            edge(j, B0{}, B1{});
            if (j + 1 < ntiles)
                edge(j + 1, B1{}, B0{});
        }
    }

    lsum += __shfl_xor(lsum, 32);
    const float vdescale = pow2f(-attn_value_exponent(p, bh, lane));
    if (qi < p.N) {
        // divide first, then undo V's scale: for a tiny V the result may be
        // subnormal, and only the last product rounds into that range
        const float inv = 1.f / lsum;
        auto out = [&](float x) { return x * inv * vdescale; };
        Tout *orow = static_cast<Tout *>(p.o) + (bh * p.N + qi) * D;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
#pragma unroll
            for (int g = 0; g < 4; ++g)
                store4<Tout>(orow + 32 * dt + 8 * g + 4 * h32, out(oacc[dt][4 * g]),
                             out(oacc[dt][4 * g + 1]), out(oacc[dt][4 * g + 2]),
                             out(oacc[dt][4 * g + 3]));
        }
        if (p.lse && h32 == 0)
            p.lse[bh * p.N + qi] = (m + (log2_fast(lsum) - 7.f)) * kLn2;
    }
}

template <int D>
static hipError_t attention_one(const AttnParams &p, aaren_dtype out, hipStream_t stream)
{
    hipLaunchKernelGGL((attn_vmax_kernel<D>), dim3((unsigned)kAttnVmaxParts, (unsigned)p.bh),
                       dim3(256), 0, stream, p);
    hipError_t e0 = hipGetLastError();
    if (e0 != hipSuccess)
        return e0;
    hipLaunchKernelGGL((attn_transpose_kernel<D>),
                       dim3((unsigned)(p.Np / 64), (unsigned)(D / 64), (unsigned)p.bh), dim3(256),
                       0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t blocks = p.bh * ((p.N + kAttnQueries - 1) / kAttnQueries);
    if (out == AAREN_F32)
        hipLaunchKernelGGL((self_attention_kernel<D, float>), dim3((unsigned)blocks),
                           dim3(64 * kAttnWaves), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((self_attention_kernel<D, bf16>), dim3((unsigned)blocks),
                           dim3(64 * kAttnWaves), 0,
                           stream, p);
    return hipGetLastError();
}

hipError_t launch_self_attention(const AttnParams &p, int D, aaren_dtype out_dtype,
                                 hipStream_t stream)
{
    return D == 64 ? attention_one<64>(p, out_dtype, stream)
                   : attention_one<128>(p, out_dtype, stream);
}

}  // namespace aaren
