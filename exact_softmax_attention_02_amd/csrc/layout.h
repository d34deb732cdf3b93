// Workspace layout, tile shapes and kernel parameters of libaaren (host and
// device). Nothing here is part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "aaren.h"

namespace aaren {

// ---- scan workspace ---------------------------------------------------------
// [ header: 256 B ][ ticket counters ][ segment-start bitmap (segmented only) ][ tile slots ]
// header[kError] : bits set (never cleared by a call) when a tile drew a
//                  ticket out of range (1), walked past the end of its stream
//                  (2) or gave up waiting for its predecessors (4) -- only
//                  possible with a workspace that was not zero-filled before
//                  first use or was shared by overlapping calls;
//                  aaren_workspace_status reads (and may clear) it.
// Ticket counters: one per stream, each in its own 128-byte line. A tile's
//   workgroup draws its position along the stream from its stream's counter
//   with a wrapping increment, so the counter is back at 0 when the call ends.
// Tile slots: per tile two published states ("aggregate" then "inclusive
//   prefix"), each slot_words(D) 64-bit words: word 0 = m, word 1 = u, words
//   2.. = w[0..D-1]. A word is (tag << 32) | float bits, tag = epoch << 1 |
//   flag, where the epoch is unique to each call of the process; a reader thus
//   tells a word of the running call from a stale one without any fence, and
//   the slots never need resetting. flag marks an aggregate that contains a
//   sequence start.
constexpr int kError = 3;
// header[kEpochWord]: the epoch of the last call made while its stream was
// being captured into a HIP graph. Eager calls take their epoch from a
// process-wide counter on the host (1 .. kGraphEpoch0 - 1) and pass it to the
// kernels; a captured call instead enqueues a one-thread kernel that advances
// this word (kGraphEpoch0 .. kGraphEpochEnd - 1, wrapping), and its kernels,
// given epoch 0, read the word: every replay of the graph then runs with an
// epoch of its own, and the two ranges never meet.
constexpr int kEpochWord = 4;
constexpr uint32_t kGraphEpoch0 = 1u << 30;
constexpr uint32_t kGraphEpochEnd = 0x7fffffffu;
constexpr size_t kHeaderBytes = 256;
constexpr int kCounterStride = 32;  // u32 words between ticket counters (128 B)
// polls of a predecessor's slots before a tile gives up (about a second)
constexpr uint32_t kMaxPolls = 1u << 20;

__host__ __device__ constexpr int slot_words(int D)
{
    return ((D + 2) + 7) / 8 * 8;
}

__host__ __device__ constexpr size_t round256(size_t b)
{
    return (b + 255) / 256 * 256;
}

// Rows one scan tile covers, per (d, input dtype). Row = 256 B for d=64 fp32
// and d=128 bf16; each of the 16 lane groups of a 4-wave tile owns 16 rows.
__host__ __device__ constexpr int scan_tile_rows(int D, int in_bytes)
{
    // lanes per row = D*in_bytes/16, groups per tile = 4 waves * 64 / lanes
    return (4 * 64 / (D * in_bytes / 16)) * 16;
}

// Smallest tile over the supported input dtypes (sizes the workspace query).
__host__ __device__ constexpr int scan_tile_rows_min(int D)
{
    return scan_tile_rows(D, 4) < scan_tile_rows(D, 2) ? scan_tile_rows(D, 4)
                                                       : scan_tile_rows(D, 2);
}

struct ScanParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;              // log-normaliser per row, or null
    int64_t lse_stream_stride, lse_row_stride;
    const uint32_t *bitmap;  // segment starts, one bit per row (segmented only)
    int64_t bitmap_words;
    int64_t rows;            // rows per stream: N (dense) or T (segmented)
    int64_t streams;         // B*H (dense) or H (segmented)
    int64_t H;
    // elements from the tensor start to row r of stream s = b*H + h:
    //   b * batch_stride + h * head_stride + r * row_stride
    // (k and v share one set, o has its own)
    int64_t batch_stride, head_stride, row_stride;
    int64_t o_batch_stride, o_head_stride, o_row_stride;
    // Scores given instead of keys (k unused): row r of stream s holds 4
    // floats at b * batch_stride + h * s_head_stride + r * row_stride, whose
    // first three sum to the score in log2 units (scale * log2(e) included).
    const float *scores;
    int64_t s_head_stride;
    int64_t chunks;          // tiles per stream
    uint32_t group;          // consecutive workgroups that serve one stream
    uint32_t chunks_padded;  // chunks rounded up to a multiple of group
    uint32_t num_tiles;      // streams * chunks (real tiles)
    uint32_t epoch;          // unique to this call; 0: read header[kEpochWord]
    uint32_t stress;         // nonzero: pause tiles at random (tests of the look-back)
    float qscale;            // scale * log2(e)
    uint32_t *header;
    uint32_t *counters;      // [streams * kCounterStride]
    uint64_t *slots;
};

struct StepParams {
    const void *q;
    const void *k;
    const void *v;
    float *m;
    float *u;
    float *w;
    void *o;
    int64_t units;   // S*H
    int64_t H;
    int64_t tokens;  // appended per unit (1 for a step); k, v, o are [tokens][units][d]
    float scale;
};

struct ReduceParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *m_out;
    float *u_out;
    float *partials;      // [units][parts][slot_words(d)] floats: m, u, w[d]
    const float *q_unit;  // per-unit float32 queries [units][d], or null: q [H][d] in the input dtype
    double *mean_partials;  // mean-query pass: [units][parts][d] column sums
    float *q_mean;        // mean-query pass output: [units][d]
    float *g_out;         // optional copy of q_mean for the caller
    int64_t units;        // B*H
    int64_t H;
    int64_t N;
    int64_t parts;        // chunks per unit
    int64_t rows_per_part;
    float qscale;         // scale * log2(e)
};

constexpr int kReduceMaxParts = 512;
hipError_t launch_mean_query(const ReduceParams &p, int D, aaren_dtype in, hipStream_t stream);

// Rows one backward tile covers: 128 (16 lane groups of 8 rows for d = 64,
// 16 groups over 8 waves for d = 128); five row tensors are held per lane.
__host__ __device__ constexpr int backward_tile_rows(int D)
{
    return 128 + 0 * D;
}

struct BackwardParams {
    const void *q;           // q, k, v, g: float or bf16 (the call's in_dtype)
    const void *k;
    const void *v;
    const float *o;          // the forward's output, float32
    const void *g;           // dloss/do
    const float *lse;        // log-normaliser per row, natural units
    float *dk;
    float *dv;
    float *dq_partial;       // [H][B][chunks][D], one per tile
    float *dq;               // [H][D]
    int64_t streams;         // B*H (dense) or H (packed)
    int64_t H;
    int64_t N;               // rows per stream: N (dense) or T (packed)
    // elements to row r of stream b*H + h, shared by q-side tensors k, v, o,
    // dout, dk, dv: b * batch_stride + h * head_stride + r * row_stride
    int64_t batch_stride, head_stride, row_stride;
    int64_t lse_batch_stride, lse_head_stride, lse_row_stride;
    const uint32_t *bitmap;  // sequence starts, one bit per row (packed only)
    int64_t bitmap_words;
    int64_t chunks;
    uint32_t group;
    uint32_t chunks_padded;
    uint32_t num_tiles;
    uint32_t epoch;
    uint32_t stress;         // nonzero: pause tiles at random (tests of the look-back)
    float scale;
    float qscale;            // scale * log2(e)
    uint32_t *header;
    uint32_t *counters;
    uint64_t *slots;
};

// Launchers (each validates nothing: the API layer did).
hipError_t launch_scan(const ScanParams &p, int D, aaren_dtype in, aaren_dtype out, bool segmented,
                       hipStream_t stream);

// The dense scan of fp32 values with precomputed scores (the layer's path,
// api.hip): scores[b, n, h] is 4 floats at b*v_strides[0] + h*s_head_stride +
// n*v_strides[2] whose first three sum to scale * log2(e) * <q_h, k_n>.
aaren_status scan_scored_strided(const float *scores, int64_t s_head_stride, const float *v,
                                 void *o, int64_t B, int64_t H, int64_t N, int64_t d,
                                 const int64_t *v_strides, const int64_t *o_strides,
                                 aaren_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                 void *hip_stream);
hipError_t launch_segment_flags(const int64_t *offsets, int64_t num_seqs, int64_t total_tokens,
                                uint32_t *bitmap, int64_t words, hipStream_t stream);
int scan_rows_per_tile(int D, aaren_dtype in);
hipError_t launch_step(const StepParams &p, int D, aaren_dtype in, aaren_dtype out,
                       hipStream_t stream);
hipError_t launch_append(const StepParams &p, int D, aaren_dtype in, aaren_dtype out,
                         hipStream_t stream);
hipError_t launch_state_init(float *m, float *u, float *w, int64_t units, int64_t D,
                             hipStream_t stream);
hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t stream);
hipError_t launch_epoch_advance(uint32_t *header, hipStream_t stream);
hipError_t launch_workspace_status(uint32_t *header, uint32_t *out, int reset, hipStream_t stream);
hipError_t launch_reduce(const ReduceParams &p, int D, aaren_dtype in, aaren_dtype out,
                         hipStream_t stream);
int reduce_rows_per_iteration(int D, aaren_dtype in);
// Creates the device's rocBLAS handle for the layer if it has none; returns
// null or a description of the failure.
const char *layer_init(int device);
hipError_t launch_scan_backward(const BackwardParams &p, int D, bool segmented, aaren_dtype in,
                                hipStream_t stream);

}  // namespace aaren
