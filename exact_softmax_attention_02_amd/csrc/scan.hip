// Many-to-many single-query attention as one streaming prefix scan.
//
// What is computed ("Attention as an RNN" review, abstract item (3) and
// proposed method; the recurrence is that of section 2 of the
// "Self-attention Does Not Need O(n^2) Memory" review): for every prefix
// 1..k of a sequence, o_k = sum_{i<=k} e^{s_i} v_i / sum_{i<=k} e^{s_i} with
// s_i = scale <q, k_i>. The prefix is carried as a state (m, u, w) -- running
// maximum, normaliser and weighted value sum relative to e^m -- and two states
// combine associatively: (m_a,u_a,w_a) (+) (m_b,u_b,w_b) = (m, f_a u_a + f_b u_b,
// f_a w_a + f_b w_b), m = max(m_a, m_b), f = e^{m_side - m}.
//
// Design (one HBM pass over K and V, one over O):
//  * A tile is ROWS consecutive rows of one stream (a (b,h) sequence, or one
//    head of a packed batch). A lane group of L lanes reads a 16-byte slice
//    of each of R consecutive rows per lane (see Slice in device.h), so every
//    wave-wide load or store covers whole cache lines. A dense stream ends in
//    half tiles (R/2 rows per group; dense_scan_chunks in scan_tiles.h), which
//    shortens the drain at the end of a call.
//  * Scores: per-lane partial dot products, summed over the group with a DPP
//    butterfly (no MFMA: the score is a matrix-vector product, bandwidth-bound).
//  * Pass 1 reduces each group's rows to one state (maximum first, then the
//    sums, so no chained rescaling); the groups' states go through LDS.
//  * Cross-tile carry by decoupled look-back: a tile publishes its aggregate
//    state at once, then walks back over predecessor tiles of its stream until
//    one has published an inclusive prefix, and publishes its own. A tile's
//    position along its stream comes from a per-stream ticket counter, so a
//    tile only ever waits for tiles that already run, and the counters do not
//    contend. Published words carry the call's epoch, so readers need no
//    fence and the slots never have to be reset between calls.
//  * Pass 2 re-runs each group's rows from its exclusive prefix with a running
//    maximum (outputs need the per-row maximum: a shared tile maximum would
//    underflow early rows when scores span more than ~87), normalises and
//    stores.
//  * Packed batches: a bitmap marks sequence starts; a start resets the state,
//    and the look-back stops at an aggregate that holds a start (segmented
//    scan with head flags).
//  * Scored (the layer's form): the scores arrive precomputed, three fp32
//    parts per row and head, and take the place of K's row and the dot
//    product; the rest is unchanged.
// Exponentials are base 2: q is pre-multiplied by scale*log2(e).
#include <atomic>
#include <type_traits>

#include "lookback.h"
#include "scan_tiles.h"

namespace aaren {

typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef float f32x2n __attribute__((ext_vector_type(2)));

// store_slice with bf16 outputs rounded by the chip (v_cvt_pk_bf16_f32, round
// to nearest even, two values per instruction) instead of in integer
// arithmetic: the same bits for every finite value, and the scans that write
// bf16 issue about a quarter fewer instructions (8 x 8 x 4096 fp32 -> bf16
// 37.0 against 39.2 us, 4 x 16 x 65536 bf16 -> bf16 535 against 584 us).
template <int D, typename Tin, typename Tout>
__device__ __forceinline__ void store_row(Tout *row, int gl, const float *x)
{
    if constexpr (sizeof(Tout) == 4) {
        store_slice<D, Tin, Tout>(row, gl, x);
    } else {
        using S = Slice<D, Tin>;
        auto pair = [](float a, float b) {
            return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2n{a, b}, bf16x2n));
        };
#pragma unroll
        for (int c = 0; c < S::NC; ++c) {
            const u32x2 v = {pair(x[4 * c], x[4 * c + 1]), pair(x[4 * c + 2], x[4 * c + 3])};
            __builtin_nontemporal_store(v, reinterpret_cast<u32x2 *>(row + c * S::STRIDE + 4 * gl));
        }
    }
}

template <int D, typename Tin, int R, int WAVES>
struct ScanShape {
    using G = RowGeo<D, Tin>;
    static constexpr int E = G::kElems;
    static constexpr int L = G::kLanes;
    static constexpr int GPW = G::kGroupsPerWave;
    static constexpr int NG = WAVES * GPW;  // lane groups per tile
    static constexpr int ROWS = NG * R;     // rows per tile
    static constexpr int SLOT = slot_words(D);
    static constexpr int CPL = D / 64;      // columns per lane, column-per-lane layout
    static_assert(R <= 32, "row flags are kept in 32 bits");
    static_assert(D % 64 == 0, "d = 64 or 128");
};

// SCORED: the scores come precomputed (p.scores, see ScanParams) and K is not
// read; dense fp32 values only.
// SPLIT: tiles full_chunks .. p.chunks-1 of a stream are half tiles (dense
// fp32 only); other instantiations ignore full_chunks.
template <int D, typename Tin, typename Tout, int R, int WAVES, bool SEG, bool SCORED, bool SPLIT>
__global__ __launch_bounds__(64 * WAVES) void scan_kernel(const ScanParams p, const int64_t full_chunks)
{
    using S = ScanShape<D, Tin, R, WAVES>;
    using SL = Slice<D, Tin>;
    constexpr int E = S::E, L = S::L, GPW = S::GPW, NG = S::NG, ROWS = S::ROWS;
    constexpr int SLOT = S::SLOT, CPL = S::CPL;

    __shared__ uint32_t sh_chunk;
    __shared__ float sh_gm[NG], sh_gu[NG];
    __shared__ uint32_t sh_gf[NG];
    __shared__ __attribute__((aligned(16))) float sh_gw[NG][D];
    __shared__ float sh_cm, sh_cu;
    __shared__ __attribute__((aligned(16))) float sh_cw[D];
    __shared__ LookbackWindow<D> sh_win;  // wave 0's look-back walk

    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int gl = lane % L;                     // lane within its group
    const int grp = wave * GPW + lane / L;       // group within the tile

    // Workgroups b = g*G .. g*G+G-1 serve stream g % streams (G = p.group) and
    // draw their positions along the stream from that stream's counter, so a
    // tile only ever waits for tiles whose workgroups already run (no reliance
    // on dispatch order). Consecutive workgroups go to different XCDs, so with
    // G = 8 each XCD sweeps every stream at one chunk offset: for packed
    // batches the heads of one token range, which are adjacent in memory,
    // are then read by one XCD at about the same time.
    const uint32_t stream32 = (blockIdx.x / p.group) % (uint32_t)p.streams;
    if (tid == 0)
        sh_chunk = __builtin_amdgcn_atomic_inc32(p.counters + (size_t)stream32 * kCounterStride,
                                                 p.chunks_padded - 1u, __ATOMIC_RELAXED, "agent");
    __syncthreads();
    const uint32_t chunk32 = __builtin_amdgcn_readfirstlane(sh_chunk);
    // a call captured into a graph finds its epoch in the header (advanced
    // on the device just before this launch)
    const uint32_t epoch =
        p.epoch ? p.epoch
                : __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                      p.header + kEpochWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    stress_pause(p.stress, blockIdx.x ^ (chunk32 << 12) ^ (epoch << 24));
    if (chunk32 >= (uint32_t)p.chunks && chunk32 < p.chunks_padded)
        return;  // a padding position past the end of the stream: nothing to do
    if (chunk32 >= (uint32_t)p.chunks) {  // counter not at zero: refuse to run
        if (tid == 0)
            __hip_atomic_fetch_or(p.header + kError, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t chunk = chunk32, stream = stream32;
    const int64_t tile = chunk * p.streams + stream;          // slot index
    // SPLIT: a half tile (past full_chunks) covers ROWS/2 rows, the first
    // half of the groups, R rows each. A separate instantiation, for fp32
    // inputs only: with bf16 inputs the extra arithmetic moves the compiler to
    // wait for the first rows' loads before issuing the rest.
    int64_t row0 = chunk * ROWS + (int64_t)grp * R;  // first row of this group
    int64_t lim = p.rows;
    if constexpr (SPLIT) {
        if (chunk >= full_chunks) {
            const int64_t tile_row0 = full_chunks * ROWS + (chunk - full_chunks) * (ROWS / 2);
            row0 = tile_row0 + (int64_t)grp * R;
            lim = tile_row0 + ROWS / 2 < p.rows ? tile_row0 + ROWS / 2 : p.rows;
        }
    }
    const int64_t left = lim - row0;
    const int nvalid = left <= 0 ? 0 : (left >= R ? R : (int)left);

    // ---- issue every load of the group's rows first --------------------------
    const int64_t bat = stream / p.H, head = stream - bat * p.H;
    const int64_t base = bat * p.batch_stride + head * p.head_stride + row0 * p.row_stride;  // column 0
    const Tin *kp = static_cast<const Tin *>(p.k) + base;
    const Tin *vp = static_cast<const Tin *>(p.v) + base;
    u32x4 kr[R], vr[R];  // SCORED: kr[r] holds row r's score parts
    const float *sp = nullptr;
    if constexpr (SCORED)
        sp = p.scores + bat * p.batch_stride + head * p.s_head_stride + row0 * p.row_stride;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        kr[r] = u32x4{0, 0, 0, 0};
        vr[r] = u32x4{0, 0, 0, 0};
        if (r < nvalid) {
            if constexpr (SCORED)
                kr[r] = load16_stream(sp + r * p.row_stride);
            else
                kr[r] = load_slice<D, Tin, true>(kp + r * p.row_stride, gl);
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)  // keys first: the scores need them first
        if (r < nvalid)
            vr[r] = load_slice<D, Tin, true>(vp + r * p.row_stride, gl);

    uint32_t flags = 0;  // bit r: row r of this group starts a sequence
    if constexpr (SEG) {
        if (nvalid > 0) {
            const int64_t wi = row0 >> 5;
            const int sh = (int)(row0 & 31);
            uint64_t bits = p.bitmap[wi];
            if (wi + 1 < p.bitmap_words)
                bits |= (uint64_t)p.bitmap[wi + 1] << 32;
            flags = (uint32_t)(bits >> sh);
            if (nvalid < 32)
                flags &= (1u << nvalid) - 1u;
            if constexpr (R < 32)
                flags &= (1u << R) - 1u;
        }
    }

    // ---- scores (log2 units) ---------------------------------------------------
    float s[R];
    if constexpr (SCORED) {
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float sc = (__uint_as_float(kr[r][0]) + __uint_as_float(kr[r][1])) +
                             __uint_as_float(kr[r][2]);
            s[r] = (r < nvalid) ? sc : kNegInf;
        }
    } else {
        float qv[E];
        widen<Tin>(load_slice<D, Tin, false>(static_cast<const Tin *>(p.q) + (stream % p.H) * D, gl),
                   qv);
#pragma unroll
        for (int e = 0; e < E; ++e)
            qv[e] *= p.qscale;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float kf[E];
            widen<Tin>(kr[r], kf);
            float part = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e)
                part = __builtin_fmaf(qv[e], kf[e], part);
            s[r] = group_sum<L>(part);
            s[r] = (r < nvalid) ? s[r] : kNegInf;
        }
    }

    // ---- pass 1: the group's state (from its last sequence start, if any) ------
    const int first = (SEG && flags) ? 31 - __builtin_clz(flags) : 0;
    float gm = kNegInf;
#pragma unroll
    for (int r = 0; r < R; ++r)
        gm = (r >= first) ? fmaxf(gm, s[r]) : gm;
    float gu = 0.f, gwv[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        gwv[e] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool use = (r >= first) && (r < nvalid);
        const float pr = use ? exp2_fast(s[r] - gm) : 0.f;
        float vf[E];
        widen<Tin>(vr[r], vf);
        gu += pr;
#pragma unroll
        for (int e = 0; e < E; ++e)
            gwv[e] = __builtin_fmaf(pr, vf[e], gwv[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        sh_gw[grp][SL::col(gl, e)] = gwv[e];
    if (gl == 0) {
        sh_gm[grp] = gm;
        sh_gu[grp] = gu;
        sh_gf[grp] = flags != 0;
    }
    __syncthreads();

    // ---- exclusive prefix of the groups before this one (segment-aware) --------
    auto group_prefix = [&](float &xm, float &xu, float *xw, bool &xf) {
        xm = kNegInf;
        xu = 0.f;
        xf = false;
#pragma unroll
        for (int e = 0; e < E; ++e)
            xw[e] = 0.f;
        for (int g = 0; g < grp; ++g) {
            const float bm = sh_gm[g], bu = sh_gu[g];
            const bool bf = sh_gf[g] != 0;
            float m, fa, fb;
            merge_weights(xm, bm, m, fa, fb);
            fa = bf ? 0.f : fa;  // a sequence start in g cuts what came before
            fb = bf ? 1.f : fb;
            m = bf ? bm : m;
            xu = __builtin_fmaf(fa, xu, fb * bu);
#pragma unroll
            for (int e = 0; e < E; ++e)
                xw[e] = __builtin_fmaf(fa, xw[e], fb * sh_gw[g][SL::col(gl, e)]);
            xm = m;
            xf = xf || bf;
        }
    };

    float pm, pu, pw[E];
    bool pf;
    if (wave != 0)
        group_prefix(pm, pu, pw, pf);

    if (wave == 0) {
        // tile aggregate, column-per-lane
        float am = kNegInf, au = 0.f, aw[CPL];
        bool af = false;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            aw[c] = 0.f;
        for (int g = 0; g < NG; ++g) {
            const float bm = sh_gm[g], bu = sh_gu[g];
            const bool bf = sh_gf[g] != 0;
            float m, fa, fb;
            merge_weights(am, bm, m, fa, fb);
            fa = bf ? 0.f : fa;
            fb = bf ? 1.f : fb;
            m = bf ? bm : m;
            au = __builtin_fmaf(fa, au, fb * bu);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                aw[c] = __builtin_fmaf(fa, aw[c], fb * sh_gw[g][lane + 64 * c]);
            am = m;
            af = af || bf;
        }

        uint64_t *my = p.slots + (size_t)tile * 2 * SLOT;
        float cm = kNegInf, cu = 0.f, cw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            cw[c] = 0.f;
        // The carry is needed unless this is the stream's first tile or the
        // tile's first row starts a sequence (group 0 is lanes 0..L-1 of wave 0).
        bool first_row_starts = false;
        if constexpr (SEG)
            first_row_starts = __builtin_amdgcn_readfirstlane(flags) & 1u;
        const bool need_carry = chunk > 0 && !first_row_starts;
        if (need_carry) {
            if (!af)
                publish<D>(my, epoch << 1, am, au, aw, lane);
            else
                publish<D>(my, (epoch << 1) | 1u, am, au, aw, lane);
            stress_pause(p.stress, blockIdx.x * 3u + epoch);
            // the carry is the left fold A_0 (+) ... (+) A_{j-1} of the stream's
            // earlier aggregates (from its last sequence start, packed batches)
            lookback<D, SEG, false>(p.slots, tile - p.streams, -p.streams, p.num_tiles, epoch,
                                    lane, p.header, sh_win, cm, cu, cw);
        }
        // inclusive prefix = carry (+) aggregate, unless the tile holds a start
        float im = am, iu = au, iw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            iw[c] = aw[c];
        if (!af)
            combine<CPL>(cm, cu, cw, am, au, aw, im, iu, iw);
        publish<D>(my + SLOT, epoch << 1, im, iu, iw, lane);

        if (lane == 0) {
            sh_cm = cm;
            sh_cu = cu;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            sh_cw[lane + 64 * c] = cw[c];
        group_prefix(pm, pu, pw, pf);
    }
    __syncthreads();

    // ---- pass 2: running state from carry (+) group prefix, normalise, store ---
    float xm = pm, xu = pu, xw[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        xw[e] = pw[e];
    if (!pf) {
        float cw[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            cw[e] = sh_cw[SL::col(gl, e)];
        combine<E>(sh_cm, sh_cu, cw, pm, pu, pw, xm, xu, xw);
    }

    Tout *op = static_cast<Tout *>(p.o) + bat * p.o_batch_stride + head * p.o_head_stride +
               row0 * p.o_row_stride;
    constexpr int LPL = (R + L - 1) / L;  // rows whose log-normaliser a lane stores
    float my_lse[LPL];
#pragma unroll
    for (int j = 0; j < LPL; ++j)
        my_lse[j] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (r < nvalid) {
            if constexpr (SEG) {
                if ((flags >> r) & 1u) {
                    xm = kNegInf;
                    xu = 0.f;
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        xw[e] = 0.f;
                }
            }
            const float sr = s[r];
            const bool up = sr > xm;
            const float hi = up ? sr : xm;
            const float lo = up ? xm : sr;
            const float ex = exp2_fast(lo - hi);
            const float a = up ? ex : 1.f;
            const float pr = up ? 1.f : ex;
            float vf[E];
            widen<Tin>(vr[r], vf);
            xu = __builtin_fmaf(xu, a, pr);
            const float inv = rcp_fast(xu);
            float ov[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                xw[e] = __builtin_fmaf(xw[e], a, pr * vf[e]);
                ov[e] = xw[e] * inv;
            }
            xm = hi;
            store_row<D, Tin, Tout>(op + r * p.o_row_stride, gl, ov);
            if (p.lse && r % L == gl)  // L_k = (m + log2 u) ln 2, natural units
                my_lse[r / L] = (xm + log2_fast(xu)) * kLn2;
        }
    }
    if (p.lse) {  // lane j of the group writes row j: one contiguous store per group
#pragma unroll
        for (int j = 0; j < LPL; ++j) {
            const int r = j * L + gl;
            if (r < nvalid)
                p.lse[stream * p.lse_stream_stride + (row0 + r) * p.lse_row_stride] = my_lse[j];
        }
    }

}

// One thread per 32-row bitmap word: bit b of word i is set when row 32i+b is
// the first row of a non-empty sequence.
__global__ __launch_bounds__(256) void segment_flags_kernel(const int64_t *offsets, int64_t S,
                                                            int64_t T, uint32_t *bitmap,
                                                            int64_t words)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= words)
        return;
    const int64_t lo_row = i * 32;
    const int64_t hi_row = lo_row + 32 < T ? lo_row + 32 : T;
    int64_t lo = 0, hi = S;  // first s with offsets[s] >= lo_row
    while (lo < hi) {
        const int64_t mid = (lo + hi) >> 1;
        if (offsets[mid] < lo_row)
            lo = mid + 1;
        else
            hi = mid;
    }
    uint32_t bits = 0;
    for (int64_t s = lo; s < S; ++s) {
        const int64_t o = offsets[s];
        if (o >= hi_row)
            break;
        if (o >= lo_row)
            bits |= 1u << (uint32_t)(o - lo_row);
    }
    bitmap[i] = bits;
}

template <int D, typename Tin, typename Tout, bool SEG, bool SCORED = false, bool SPLIT = false>
static hipError_t launch_one(const ScanParams &p, hipStream_t stream, int64_t full_chunks = 0)
{
    constexpr int R = 16, WAVES = 4;
    static_assert(ScanShape<D, Tin, R, WAVES>::ROWS == scan_tile_rows(D, sizeof(Tin)),
                  "tile rows disagree with the workspace sizing");
    static_assert(!SCORED || (std::is_same_v<Tin, float> && !SEG), "scored: dense fp32 values");
    static_assert(!SPLIT || (std::is_same_v<Tin, float> && !SEG && !SCORED),
                  "half tiles: dense fp32 inputs");
    hipLaunchKernelGGL((scan_kernel<D, Tin, Tout, R, WAVES, SEG, SCORED, SPLIT>),
                       dim3((unsigned)(p.streams * p.chunks_padded)), dim3(64 * WAVES), 0, stream, p,
                       full_chunks);
    return hipGetLastError();
}

template <int D, bool SEG>
static hipError_t dispatch_dtypes(const ScanParams &p, aaren_dtype in, aaren_dtype out,
                                  hipStream_t stream)
{
    if (in == AAREN_F32 && out == AAREN_F32)
        return launch_one<D, float, float, SEG>(p, stream);
    if (in == AAREN_F32 && out == AAREN_BF16)
        return launch_one<D, float, bf16, SEG>(p, stream);
    if (in == AAREN_BF16 && out == AAREN_F32)
        return launch_one<D, bf16, float, SEG>(p, stream);
    return launch_one<D, bf16, bf16, SEG>(p, stream);
}

hipError_t launch_scan_split(const ScanParams &p, int64_t full_chunks, int D, aaren_dtype out,
                             hipStream_t stream)
{
    if (D == 64)
        return out == AAREN_F32 ? launch_one<64, float, float, false, false, true>(p, stream, full_chunks)
                                : launch_one<64, float, bf16, false, false, true>(p, stream, full_chunks);
    return out == AAREN_F32 ? launch_one<128, float, float, false, false, true>(p, stream, full_chunks)
                            : launch_one<128, float, bf16, false, false, true>(p, stream, full_chunks);
}

hipError_t launch_scan(const ScanParams &p, int D, aaren_dtype in, aaren_dtype out, bool segmented,
                       hipStream_t stream)
{
    if (p.scores) {  // dense fp32 values (the caller checks)
        if (D == 64)
            return out == AAREN_F32 ? launch_one<64, float, float, false, true>(p, stream)
                                    : launch_one<64, float, bf16, false, true>(p, stream);
        return out == AAREN_F32 ? launch_one<128, float, float, false, true>(p, stream)
                                : launch_one<128, float, bf16, false, true>(p, stream);
    }
    if (D == 64)
        return segmented ? dispatch_dtypes<64, true>(p, in, out, stream)
                         : dispatch_dtypes<64, false>(p, in, out, stream);
    return segmented ? dispatch_dtypes<128, true>(p, in, out, stream)
                     : dispatch_dtypes<128, false>(p, in, out, stream);
}

int scan_rows_per_tile(int D, aaren_dtype in)
{
    return scan_tile_rows(D, in == AAREN_F32 ? 4 : 2);
}

// Workgroups of one instantiation of the dense scan that the current device
// holds at once (resident workgroups per compute unit times compute units),
// kept per device once found; 0 if the runtime cannot say (then asked again
// at the next call).
template <int D, typename Tin, typename Tout>
static int resident_one()
{
    constexpr int kMaxDev = 64;
    static std::atomic<int> known[kMaxDev];  // 0: not found yet
    int dev = 0, cus = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev)
        return 0;
    const int seen = known[dev].load(std::memory_order_relaxed);
    if (seen > 0)
        return seen;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &per_cu, reinterpret_cast<const void *>(scan_kernel<D, Tin, Tout, 16, 4, false, false, false>),
            256, 0) != hipSuccess ||
        cus <= 0 || per_cu <= 0)
        return 0;
    known[dev].store(cus * per_cu, std::memory_order_relaxed);
    return cus * per_cu;
}

int scan_resident_tiles(int D, aaren_dtype in, aaren_dtype out)
{
    if (D == 64) {
        if (in == AAREN_F32)
            return out == AAREN_F32 ? resident_one<64, float, float>() : resident_one<64, float, bf16>();
        return out == AAREN_F32 ? resident_one<64, bf16, float>() : resident_one<64, bf16, bf16>();
    }
    if (in == AAREN_F32)
        return out == AAREN_F32 ? resident_one<128, float, float>() : resident_one<128, float, bf16>();
    return out == AAREN_F32 ? resident_one<128, bf16, float>() : resident_one<128, bf16, bf16>();
}

hipError_t launch_segment_flags(const int64_t *offsets, int64_t num_seqs, int64_t total_tokens,
                                uint32_t *bitmap, int64_t words, hipStream_t stream)
{
    const int64_t blocks = (words + 255) / 256;
    hipLaunchKernelGGL(segment_flags_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, offsets,
                       num_seqs, total_tokens, bitmap, words);
    return hipGetLastError();
}

}  // namespace aaren
