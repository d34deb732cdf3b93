// Gradients of the many-to-many scan: dq, dk, dv from dloss/do.
//
// The pages present the many-to-many form as differentiable and trained in
// parallel ("Attention as an RNN" review, proposed method; the
// memory-efficient-attention review reports differentiation in its abstract
// and section 5.2, whose body is lost) but print no formula. Derived from the
// definition o_k = sum_{i<=k} p_ki v_i, p_ki = e^{s_i - L_k},
// L_k = ln sum_{j<=k} e^{s_j}, with g_k = dloss/do_k and delta_k = <g_k, o_k>:
//   dv_i = e^{s_i} sum_{k>=i} e^{-L_k} g_k
//   ds_i = <dv_i, v_i> - e^{s_i} sum_{k>=i} e^{-L_k} delta_k
//   dk_i = scale ds_i q,   dq = scale sum_i ds_i k_i.
// Both sums are suffix sums of leaves (m = -L_k, u = delta_k, w = g_k) under
// the same (m, u, w) combine as the forward scan (weights relative to the
// largest exponent), so the backward is the forward's machinery run from the
// end of each stream: tiles are claimed last-first, the look-back walks
// towards later tiles, pass 2 walks each group's rows backwards. L_k comes
// from the forward pass (aaren_scan's lse output).
//
// One HBM pass: K, V, O, dO read and dK, dV written once (plus 4 bytes of L
// per row); each tile leaves one partial dq, summed per head in a fixed order
// by a second kernel, so dq is reproducible bit for bit. Packed batches
// (one stream per head over all tokens) restart the suffix at every sequence
// end. q, K, V and dO may be bf16 (widened exactly); O, L and the gradients
// are float32.
#include <type_traits>

#include "lookback.h"

namespace aaren {

// A lane's 4 consecutive columns 4gl..4gl+3 of a row, raw: 16 bytes of fp32
// or 8 bytes of bf16, and their exact float values.
template <typename T>
using RawCols = std::conditional_t<sizeof(T) == 4, u32x4, u32x2>;

template <typename T, bool STREAM>
__device__ __forceinline__ RawCols<T> load_cols(const T *row, int gl)
{
    if constexpr (sizeof(T) == 4) {
        return STREAM ? load16_stream(row + 4 * gl) : load16(row + 4 * gl);
    } else {
        const u32x2 *a = reinterpret_cast<const u32x2 *>(row + 4 * gl);
        return STREAM ? __builtin_nontemporal_load(a) : *a;
    }
}

template <typename T>
__device__ __forceinline__ void widen_cols(RawCols<T> raw, float *out)
{
    if constexpr (sizeof(T) == 4) {
        widen<float>(raw, out);
    } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            out[2 * i] = __uint_as_float(raw[i] << 16);
            out[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
        }
    }
}

template <int D>
struct BackwardShape {
    static constexpr int E = 4;              // fp32: 4 columns per lane
    static constexpr int L = D / E;          // lanes per row
    static constexpr int GPW = 64 / L;
    static constexpr int WAVES = D == 64 ? 4 : 8;
    static constexpr int NG = WAVES * GPW;   // 16 groups
    static constexpr int R = 8;
    static constexpr int ROWS = NG * R;
    static constexpr int CPL = D / 64;
    static_assert(ROWS == backward_tile_rows(D), "tile rows disagree with the workspace sizing");
};

// Five row tensors per lane: without a bound the compiler keeps values in
// AGPRs and runs one wave per SIMD; three waves fit without spilling.
//
// SEG (packed batches): a row that ends its sequence (the next row starts
// one) takes nothing from the rows after it, so the suffix state restarts
// there. Groups and tiles carry a flag "holds a sequence end"; folding a
// flagged state onto what follows keeps the flagged state alone, exactly as
// the forward's flag-lifted combine does for sequence starts.
template <int D, bool SEG, typename Tin>
__global__ __launch_bounds__(64 * BackwardShape<D>::WAVES)
__attribute__((amdgpu_waves_per_eu(3))) void scan_backward_kernel(const BackwardParams p)
{
    const Tin *pq = static_cast<const Tin *>(p.q), *pk = static_cast<const Tin *>(p.k);
    const Tin *pv = static_cast<const Tin *>(p.v), *pg = static_cast<const Tin *>(p.g);
    using S = BackwardShape<D>;
    using SL = Slice<D, float>;
    constexpr int E = S::E, L = S::L, GPW = S::GPW, NG = S::NG, R = S::R, ROWS = S::ROWS;
    constexpr int SLOT = slot_words(D), CPL = S::CPL;

    __shared__ uint32_t sh_chunk;
    __shared__ float sh_gm[NG], sh_gu[NG];
    __shared__ uint32_t sh_gf[NG];
    __shared__ uint32_t sh_last_end;
    __shared__ __attribute__((aligned(16))) float sh_gw[NG][D];
    __shared__ float sh_cm, sh_cu;
    __shared__ __attribute__((aligned(16))) float sh_cw[D];
    __shared__ LookbackWindow<D> sh_win;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int gl = lane % L, grp = wave * GPW + lane / L;

    // position along the stream counted from its end (see the forward scan)
    const uint32_t stream32 = (blockIdx.x / p.group) % (uint32_t)p.streams;
    if (tid == 0)
        sh_chunk = __builtin_amdgcn_atomic_inc32(p.counters + (size_t)stream32 * kCounterStride,
                                                 p.chunks_padded - 1u, __ATOMIC_RELAXED, "agent");
    __syncthreads();
    const uint32_t ticket = __builtin_amdgcn_readfirstlane(sh_chunk);
    // a call captured into a graph finds its epoch in the header (advanced
    // on the device just before this launch)
    const uint32_t epoch =
        p.epoch ? p.epoch
                : __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                      p.header + kEpochWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    stress_pause(p.stress, blockIdx.x ^ (ticket << 12) ^ (epoch << 24));
    if (ticket >= (uint32_t)p.chunks && ticket < p.chunks_padded)
        return;  // a padding position: nothing to do
    if (ticket >= (uint32_t)p.chunks) {
        if (tid == 0)
            __hip_atomic_fetch_or(p.header + kError, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int64_t chunk = p.chunks - 1 - ticket, stream = stream32;
    const int64_t tile = chunk * p.streams + stream;
    const int64_t bat = stream / p.H, head = stream - bat * p.H;
    const int64_t row0 = chunk * ROWS + (int64_t)grp * R;
    const int64_t left = p.N - row0;
    const int nvalid = left <= 0 ? 0 : (left >= R ? R : (int)left);

    // column 0 of the group's first row; rows are row_stride apart
    const int64_t base = bat * p.batch_stride + head * p.head_stride + row0 * p.row_stride;
    const int64_t rs = p.row_stride;

    // bit r: row r of the group ends its sequence (row r + 1 starts one)
    uint32_t ends = 0;
    if constexpr (SEG) {
        if (nvalid > 0) {
            const int64_t wi = (row0 + 1) >> 5;
            const int sh = (int)((row0 + 1) & 31);
            uint64_t bits = wi < p.bitmap_words ? p.bitmap[wi] : 0u;
            if (wi + 1 < p.bitmap_words)
                bits |= (uint64_t)p.bitmap[wi + 1] << 32;
            ends = (uint32_t)(bits >> sh) & ((1u << nvalid) - 1u);
        }
    }

    // Every input load is unconditional: a row at or past N reads the
    // stream's last row instead (always in bounds), and its leaf exponent is
    // -inf, so it weighs exactly 0 in pass 1 and pass 2 skips it. A load
    // inside a branch would make the compiler wait at the end of the branch
    // for it and for every load issued before it.
    auto clamp_row = [&](int r) { return row0 + r < p.N ? row0 + r : p.N - 1; };
    const int64_t sbase = bat * p.batch_stride + head * p.head_stride;
    auto row_at = [&](int r) { return sbase + clamp_row(r) * rs; };

    // dO and O first: the tile's aggregate needs only them and L, so it is
    // published (and the look-back chain moves on) before K and V arrive
    RawCols<Tin> gr[R];
    u32x4 orr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        gr[r] = load_cols<Tin, true>(pg + row_at(r), gl);
        orr[r] = load_cols<float, true>(p.o + row_at(r), gl);
    }
    float lm[R];  // leaf exponent -L_r, log2 units
    const float *lse_s = p.lse + bat * p.lse_batch_stride + head * p.lse_head_stride;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float l = lse_s[clamp_row(r) * p.lse_row_stride];
        lm[r] = (r < nvalid) ? -l * kLog2e : kNegInf;
    }

    // delta_r = <g_r, o_r>
    float dl[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float gf[E], of[E];
        widen_cols<Tin>(gr[r], gf);
        widen<float>(orr[r], of);
        float b = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            b = __builtin_fmaf(gf[e], of[e], b);
        dl[r] = group_sum<L>(b);
    }

    // ---- pass 1: the group's suffix aggregate from its first row, up to its
    // first sequence end (packed), maximum first -------------------------------
    const int last = (SEG && ends) ? __builtin_ctz(ends) : R - 1;
    float gm = kNegInf;
#pragma unroll
    for (int r = 0; r < R; ++r)
        gm = (r <= last) ? fmaxf(gm, lm[r]) : gm;
    float gu = 0.f, gwv[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        gwv[e] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const float f = (r < nvalid && r <= last) ? exp2_fast(lm[r] - gm) : 0.f;
        float gf[E];
        widen_cols<Tin>(gr[r], gf);
        gu = __builtin_fmaf(f, dl[r], gu);
#pragma unroll
        for (int e = 0; e < E; ++e)
            gwv[e] = __builtin_fmaf(f, gf[e], gwv[e]);
    }
#pragma unroll
    for (int e = 0; e < E; ++e)
        sh_gw[grp][SL::col(gl, e)] = gwv[e];
    if (gl == 0) {
        sh_gm[grp] = gm;
        sh_gu[grp] = gu;
        sh_gf[grp] = ends != 0;
        if (grp == NG - 1)
            sh_last_end = (ends >> (R - 1)) & 1u;  // the tile's last row ends a sequence
    }
    // K and V land during the barrier and the look-back (O's registers are free)
    RawCols<Tin> kr[R], vr[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        kr[r] = load_cols<Tin, true>(pk + row_at(r), gl);
#pragma unroll
    for (int r = 0; r < R; ++r)
        vr[r] = load_cols<Tin, true>(pv + row_at(r), gl);
    __syncthreads();

    // fold a group state G onto X (the rows after it): G (+) X, or G alone if
    // G holds a sequence end
    auto fold_group = [&](int g, float &xm, float &xu, float *xw, bool &xf, auto col) {
        constexpr int NE = decltype(col)::value == 0 ? E : CPL;
        float yw[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e)
            yw[e] = sh_gw[g][decltype(col)::value == 0 ? SL::col(gl, e) : lane + 64 * e];
        if (SEG && sh_gf[g]) {
            xm = sh_gm[g];
            xu = sh_gu[g];
#pragma unroll
            for (int e = 0; e < NE; ++e)
                xw[e] = yw[e];
            xf = true;
        } else {
            combine<NE>(sh_gm[g], sh_gu[g], yw, xm, xu, xw, xm, xu, xw);
        }
    };
    using SliceCols = std::integral_constant<int, 0>;
    using LaneCols = std::integral_constant<int, 1>;

    // state of the groups after this one in the tile: G_{g+1} (+) ... (+) G_{NG-1}
    auto later_groups = [&](float &xm, float &xu, float *xw, bool &xf) {
        xm = kNegInf;
        xu = 0.f;
        xf = false;
#pragma unroll
        for (int e = 0; e < E; ++e)
            xw[e] = 0.f;
        for (int g = NG - 1; g > grp; --g)
            fold_group(g, xm, xu, xw, xf, SliceCols{});
    };

    float pm, pu, pw[E];
    bool pf;
    if (wave != 0)
        later_groups(pm, pu, pw, pf);

    if (wave == 0) {
        // tile aggregate, column-per-lane, folded from the last group
        float am = kNegInf, au = 0.f, aw[CPL];
        bool af = false;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            aw[c] = 0.f;
        for (int g = NG - 1; g >= 0; --g)
            fold_group(g, am, au, aw, af, LaneCols{});
        uint64_t *my = p.slots + (size_t)tile * 2 * SLOT;
        float cm = kNegInf, cu = 0.f, cw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            cw[c] = 0.f;
        // the carry is needed unless this is the stream's last tile or the
        // tile's last row ends a sequence
        const bool need_carry = chunk < p.chunks - 1 && !(SEG && sh_last_end);
        if (need_carry) {
            publish<D>(my, (epoch << 1) | (af ? 1u : 0u), am, au, aw, lane);
            stress_pause(p.stress, blockIdx.x * 3u + epoch);
            // the carry is A_{j+1} (+) ... (+) A_last, the stream's later
            // aggregates (up to the next sequence end, packed batches)
            lookback<D, SEG, true>(p.slots, tile + p.streams, p.streams, p.num_tiles, epoch,
                                   lane, p.header, sh_win, cm, cu, cw);
        }
        // inclusive suffix = aggregate (+) carry, unless the tile holds an end
        float im = am, iu = au, iw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            iw[c] = aw[c];
        if (!af)
            combine<CPL>(am, au, aw, cm, cu, cw, im, iu, iw);
        publish<D>(my + SLOT, epoch << 1, im, iu, iw, lane);
        if (lane == 0) {
            sh_cm = cm;
            sh_cu = cu;
        }
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            sh_cw[lane + 64 * c] = cw[c];
        later_groups(pm, pu, pw, pf);
    }
    __syncthreads();

    // scores, log2 units
    float qv[E], qs[E];
    widen_cols<Tin>(load_cols<Tin, false>(pq + head * D, gl), qv);
#pragma unroll
    for (int e = 0; e < E; ++e)
        qs[e] = qv[e] * p.qscale;
    float s[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        float kf[E];
        widen_cols<Tin>(kr[r], kf);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e)
            a = __builtin_fmaf(qs[e], kf[e], a);
        s[r] = group_sum<L>(a);
    }

    // ---- pass 2: rows last-first from (later groups (+) carry) ----------------
    float xm = pm, xu = pu, xw[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        xw[e] = pw[e];
    if (!pf) {
        float cw[E];
#pragma unroll
        for (int e = 0; e < E; ++e)
            cw[e] = sh_cw[SL::col(gl, e)];
        combine<E>(pm, pu, pw, sh_cm, sh_cu, cw, xm, xu, xw);
    }
    float dq_acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e)
        dq_acc[e] = 0.f;
#pragma unroll
    for (int r = R - 1; r >= 0; --r) {
        if (r < nvalid) {
            if (SEG && ((ends >> r) & 1u)) {  // the rows after this one belong to another sequence
                xm = kNegInf;
                xu = 0.f;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    xw[e] = 0.f;
            }
            float gf[E], vf[E], kf[E];
            widen_cols<Tin>(gr[r], gf);
            widen_cols<Tin>(vr[r], vf);
            widen_cols<Tin>(kr[r], kf);
            combine<E>(lm[r], dl[r], gf, xm, xu, xw, xm, xu, xw);  // leaf (+) state
            const float pw_r = exp2_fast(s[r] + xm);  // e^{s_r} times the state's scale
            float dv[E], part = 0.f;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dv[e] = pw_r * xw[e];
                part = __builtin_fmaf(dv[e], vf[e], part);
            }
            const float ds = group_sum<L>(part) - pw_r * xu;
            const float sds = p.scale * ds;
            float dk[E];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                dk[e] = sds * qv[e];
                dq_acc[e] = __builtin_fmaf(sds, kf[e], dq_acc[e]);
            }
            store_slice<D, float, float>(p.dv + base + r * rs, gl, dv);
            store_slice<D, float, float>(p.dk + base + r * rs, gl, dk);
        }
    }

    // ---- the tile's partial dq: groups summed in a fixed order ----------------
    __syncthreads();  // sh_gw is free again
#pragma unroll
    for (int e = 0; e < E; ++e)
        sh_gw[grp][SL::col(gl, e)] = dq_acc[e];
    __syncthreads();
    if (wave == 0) {
        // partials of one head are contiguous: [H][B][chunks][D]
        const int64_t B = p.streams / p.H;
        const int64_t at = (head * B + bat) * p.chunks + chunk;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float acc = 0.f;
            for (int g = 0; g < NG; ++g)
                acc += sh_gw[g][lane + 64 * c];
            p.dq_partial[(size_t)at * D + lane + 64 * c] = acc;
        }
    }
}

// dq[h] = sum of the B*chunks partials of head h, in a fixed order: thread
// (sub, c4) adds rows sub, sub + SUB, ... of columns 4c4..4c4+3, then the SUB
// subtotals are added in order. With stride > 1 it adds the rows 0, stride,
// 2 stride, ... that scan_backward_dq_slice_kernel left.
constexpr int kDqThreads = 1024;
// Heads with more partials than this (packed batches: one per 128 tokens of
// the whole batch) are summed in two levels, kDqSlice partials per workgroup
// first, so that more than one workgroup per head reads them.
constexpr int64_t kDqTwoLevel = 4096;
constexpr int64_t kDqSlice = 256;
constexpr int kDqSliceThreads = 256;

template <int D>
__global__ __launch_bounds__(kDqThreads) void scan_backward_dq_kernel(const BackwardParams p,
                                                                      int64_t stride)
{
    constexpr int V4 = D / 4, SUB = kDqThreads / V4;
    __shared__ __attribute__((aligned(16))) float sh[SUB][D];
    const int tid = threadIdx.x, c4 = tid % V4, sub = tid / V4;
    const int64_t h = blockIdx.x;
    const int64_t count = (p.streams / p.H) * p.chunks;  // partials of this head
    const int64_t rows = (count + stride - 1) / stride;
    const float *src = p.dq_partial + (size_t)h * count * D + 4 * c4;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
    for (int64_t i = sub; i < rows; i += SUB) {
        float x[4];
        widen<float>(load16(src + (size_t)(i * stride) * D), x);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            a[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        sh[sub][4 * c4 + e] = a[e];
    __syncthreads();
    if (tid < D) {
        float r = 0.f;
#pragma unroll 8
        for (int s = 0; s < SUB; ++s)
            r += sh[s][tid];
        p.dq[h * D + tid] = r;
    }
}

// First level: workgroup (g, h) adds partials g*kDqSlice .. (g+1)*kDqSlice - 1
// of head h in the same fixed order and writes the sum over the slice's first
// partial (only this workgroup touches the slice).
template <int D>
__global__ __launch_bounds__(kDqSliceThreads) void scan_backward_dq_slice_kernel(
    const BackwardParams p)
{
    constexpr int V4 = D / 4, SUB = kDqSliceThreads / V4;
    __shared__ __attribute__((aligned(16))) float sh[SUB][D];
    const int tid = threadIdx.x, c4 = tid % V4, sub = tid / V4;
    const int64_t h = blockIdx.y, g = blockIdx.x;
    const int64_t count = (p.streams / p.H) * p.chunks;
    const int64_t first = g * kDqSlice, end = first + kDqSlice < count ? first + kDqSlice : count;
    float *base = p.dq_partial + (size_t)h * count * D;
    float a[4] = {0.f, 0.f, 0.f, 0.f};
    for (int64_t i = first + sub; i < end; i += SUB) {
        float x[4];
        widen<float>(load16(base + (size_t)i * D + 4 * c4), x);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            a[e] += x[e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e)
        sh[sub][4 * c4 + e] = a[e];
    __syncthreads();  // every read of the slice is done before its first row is written
    if (tid < D) {
        float r = 0.f;
        for (int s = 0; s < SUB; ++s)
            r += sh[s][tid];
        base[(size_t)first * D + tid] = r;
    }
}

template <int D, typename Tin>
static hipError_t backward_one(const BackwardParams &p, bool segmented, hipStream_t stream)
{
    if (segmented)
        hipLaunchKernelGGL((scan_backward_kernel<D, true, Tin>),
                           dim3((unsigned)(p.streams * p.chunks_padded)),
                           dim3(64 * BackwardShape<D>::WAVES), 0, stream, p);
    else
        hipLaunchKernelGGL((scan_backward_kernel<D, false, Tin>),
                           dim3((unsigned)(p.streams * p.chunks_padded)),
                           dim3(64 * BackwardShape<D>::WAVES), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const int64_t count = (p.streams / p.H) * p.chunks;
    int64_t stride = 1;
    if (count > kDqTwoLevel) {
        hipLaunchKernelGGL((scan_backward_dq_slice_kernel<D>),
                           dim3((unsigned)((count + kDqSlice - 1) / kDqSlice), (unsigned)p.H),
                           dim3(kDqSliceThreads), 0, stream, p);
        e = hipGetLastError();
        if (e != hipSuccess)
            return e;
        stride = kDqSlice;
    }
    hipLaunchKernelGGL((scan_backward_dq_kernel<D>), dim3((unsigned)p.H), dim3(kDqThreads), 0,
                       stream, p, stride);
    return hipGetLastError();
}

hipError_t launch_scan_backward(const BackwardParams &p, int D, bool segmented, aaren_dtype in,
                                hipStream_t stream)
{
    if (in == AAREN_BF16)
        return D == 64 ? backward_one<64, bf16>(p, segmented, stream)
                       : backward_one<128, bf16>(p, segmented, stream);
    return D == 64 ? backward_one<64, float>(p, segmented, stream)
                   : backward_one<128, float>(p, segmented, stream);
}

}  // namespace aaren
