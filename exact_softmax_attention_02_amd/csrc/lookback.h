// Decoupled look-back across the tiles of a stream, shared by the forward
// (prefix) and backward (suffix) scans.
//
// Every tile publishes up to two states in its slot pair: its aggregate as
// soon as its own rows are reduced, and its inclusive state (everything from
// the stream's start, or end for a suffix scan, through this tile) once its
// carry is known. A state is slot_words(D) 64-bit words, word 0 = m,
// word 1 = u, words 2.. = w, each (tag << 32) | float bits with
// tag = epoch << 1 | flag; the epoch is unique to the call, so a word of the
// running call is told from a stale one without any fence, and relaxed
// agent-scope 64-bit accesses (coherent across the XCDs' L2s) suffice.
//
// The walk goes from the neighbouring tile outwards. It stops at the first
// tile whose inclusive state is published (or, for packed batches, whose
// aggregate holds a sequence start, which makes it inclusive), and parks the
// aggregates met on the way in an LDS window. It then folds the parked
// aggregates onto that state nearest-last, so the carry is always the same
// ordered fold of the aggregates, whatever the timing: results are
// reproducible bit for bit. Waits are bounded.
#pragma once

#include "device.h"

namespace aaren {

// Aggregates a walk may park before it waits for an inclusive state.
constexpr int kWindow = 16;

// Scheduling perturbation for tests of the look-back, off in normal use: with
// `stress` set, a workgroup pauses a pseudo-random 0..7 times 127 x 64 cycles
// (salt: something that differs between tiles and calls), so that tiles
// publish and walk in orders the hardware rarely produces by itself. The
// arguments are wave-uniform.
__device__ __forceinline__ void stress_pause(uint32_t stress, uint32_t salt)
{
    if (stress) {
        uint32_t h = salt * 0x9e3779b9u;
        h ^= h >> 15;
        h *= 0x85ebca6bu;
        h ^= h >> 13;
        const int n = (int)(h & 7u);
        for (int i = 0; i < n; ++i)
            __builtin_amdgcn_s_sleep(127);
    }
}

__device__ __forceinline__ bool tag_ok(uint64_t word, uint32_t epoch)
{
    return (uint32_t)(word >> 33) == epoch;
}

__device__ __forceinline__ float word_value(uint64_t word)
{
    return __uint_as_float((uint32_t)word);
}

// Publish a state in column-per-lane layout (lane j holds w[j + 64c]).
template <int D>
__device__ __forceinline__ void publish(uint64_t *slot, uint32_t tag, float m, float u,
                                        const float *w, int lane)
{
    const uint64_t hi = (uint64_t)tag << 32;
#pragma unroll
    for (int c = 0; c < D / 64; ++c)
        st_agent(slot + 2 + lane + 64 * c, hi | __float_as_uint(w[c]));
    if (lane == 0)
        st_agent(slot + 0, hi | __float_as_uint(m));
    if (lane == 1)
        st_agent(slot + 1, hi | __float_as_uint(u));
}

template <int D>
struct LookbackWindow {
    float m[kWindow];
    float u[kWindow];
    float w[kWindow][D];
};

// Carry of the tile whose nearest neighbour along the scan is slot `pred`
// (step = -streams for a prefix scan, +streams for a suffix scan). Called by
// one whole wavefront; returns the carry in column-per-lane layout.
// SUFFIX: the carry is the state of the tiles AFTER this one, and parked
// aggregates are folded as (aggregate (+) carry); otherwise they are folded
// as (carry (+) aggregate).
template <int D, bool SEG, bool SUFFIX>
__device__ void lookback(const uint64_t *slots, int64_t pred, int64_t step, int64_t num_tiles,
                         uint32_t epoch, int lane, uint32_t *header, LookbackWindow<D> &win,
                         float &cm, float &cu, float *cw)
{
    constexpr int SLOT = slot_words(D), CPL = D / 64;
    uint32_t polls = 0;
    int parked = 0;
    cm = kNegInf;
    cu = 0.f;
#pragma unroll
    for (int c = 0; c < CPL; ++c)
        cw[c] = 0.f;
    while (true) {
        const uint64_t *agg = slots + (size_t)pred * 2 * SLOT;
        const uint64_t *inc = agg + SLOT;
        uint64_t wi[CPL], wa[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            wi[c] = ld_agent(inc + 2 + lane + 64 * c);
            wa[c] = ld_agent(agg + 2 + lane + 64 * c);
        }
        const uint64_t imw = ld_agent(inc + 0), iuw = ld_agent(inc + 1);
        const uint64_t amw = ld_agent(agg + 0), auw = ld_agent(agg + 1);
        bool inc_ok = tag_ok(imw, epoch) && tag_ok(iuw, epoch);
        bool agg_ok = tag_ok(amw, epoch) && tag_ok(auw, epoch);
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            inc_ok = inc_ok && tag_ok(wi[c], epoch);
            agg_ok = agg_ok && tag_ok(wa[c], epoch);
        }
        inc_ok = __all(inc_ok);
        agg_ok = __all(agg_ok);
        const bool agg_starts = SEG && agg_ok && ((amw >> 32) & 1u);
        if (inc_ok || agg_starts) {
            cm = word_value(inc_ok ? imw : amw);
            cu = word_value(inc_ok ? iuw : auw);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                cw[c] = word_value(inc_ok ? wi[c] : wa[c]);
            break;
        }
        if (agg_ok && parked < kWindow) {
            const int64_t next = pred + step;
            if (next < 0 || next >= num_tiles) {  // an end tile never publishes an aggregate
                if (lane == 0)
                    __hip_atomic_fetch_or(header + kError, 2u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
            // every lane writes the same m, u and reads back only what it wrote
            win.m[parked] = word_value(amw);
            win.u[parked] = word_value(auw);
#pragma unroll
            for (int c = 0; c < CPL; ++c)
                win.w[parked][lane + 64 * c] = word_value(wa[c]);
            ++parked;
            pred = next;
            continue;
        }
        if (++polls > kMaxPolls) {  // bounded wait: give up rather than hang
            if (lane == 0)
                __hip_atomic_fetch_or(header + kError, 4u, __ATOMIC_RELAXED,
                                      __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    for (int i = parked - 1; i >= 0; --i) {
        float yw[CPL];
#pragma unroll
        for (int c = 0; c < CPL; ++c)
            yw[c] = win.w[i][lane + 64 * c];
        if constexpr (SUFFIX)
            combine<CPL>(win.m[i], win.u[i], yw, cm, cu, cw, cm, cu, cw);
        else
            combine<CPL>(cm, cu, cw, win.m[i], win.u[i], yw, cm, cu, cw);
    }
}

}  // namespace aaren
