// Parameters and launcher of the self-attention kernels (one query per token).
// Nothing here is part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime.h>

#include "aaren.h"

namespace aaren {

// Tile shapes: a workgroup of kAttnWaves waves takes 32 queries per wave; keys
// and values go through LDS 64 at a time, double buffered (64 KB at d = 128,
// 32 KB at d = 64). d = 128 runs 2 waves per SIMD (up to 256 VGPRs), one
// workgroup per CU, which halves the tile copies per flop against 4-wave
// workgroups; d = 64 is held to 128 VGPRs, so two workgroups per CU make 4
// waves per SIMD.
constexpr int kAttnWaves = 8;
constexpr int kAttnQueries = 32 * kAttnWaves;
constexpr int kAttnKeys = 64;
// heads whose query tiles are interleaved in the launch order
constexpr int64_t kAttnHeadGroup = 16;

// Longest sequence: the tile copies address one head's K and transposed V
// through buffer descriptors whose byte counts and offsets must stay below
// 2^31 (2^22 keys of 128 bf16 values are 2^30 bytes).
constexpr int64_t kAttnMaxN = int64_t(1) << 22;

// Rows of the transposed-value workspace are padded to a whole number of key
// tiles (the padding holds zeros).
__host__ __device__ constexpr int64_t attn_padded_keys(int64_t N)
{
    return (N + kAttnKeys - 1) / kAttnKeys * kAttnKeys;
}

// V's largest magnitude per (b,h) is reduced in this many partial maxima,
// which one wave combines.
constexpr int kAttnVmaxParts = 64;

struct AttnParams {
    const uint16_t *q;   // bf16 bits [BH][N][D]
    const uint16_t *k;   // bf16 bits [BH][N][D]
    const uint16_t *v;   // bf16 bits [BH][N][D]
    uint16_t *vt;        // workspace: fp16 bits [BH][D][Np], 2^e(b,h) V transposed, zero past N
    uint32_t *vmax;      // workspace: [BH][kAttnVmaxParts] partial max |v| (bf16 bits)
    void *o;             // [BH][N][D], float or bf16
    float *lse;          // [BH][N] or null, natural units
    int64_t bh;          // B*H
    int64_t N;
    int64_t Np;          // attn_padded_keys(N)
    float qscale;        // scale * log2(e)
    int causal;
};

hipError_t launch_self_attention(const AttnParams &p, int D, aaren_dtype out_dtype,
                                 hipStream_t stream);

}  // namespace aaren
