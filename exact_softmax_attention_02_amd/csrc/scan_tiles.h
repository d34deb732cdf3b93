// How a dense scan cuts its streams into tiles, and how many tiles the device
// runs at once (host side of scan.hip; the parameters are in layout.h).
#pragma once

#include "layout.h"

namespace aaren {

// A dense stream of n rows in tiles of `rows`: the last full tile is split in
// two half tiles, and the rows after the full tiles go in half tiles, so the
// tiles that end a call move half the bytes and finish sooner. Returns the
// stream's tile count and sets *full to the number of full tiles. At most
// two tiles more than ceil(n / rows), and never fewer for a smaller `rows`.
__host__ __device__ constexpr int64_t dense_scan_chunks(int64_t n, int64_t rows, int64_t *full)
{
    const int64_t whole = n / rows;
    const int64_t f = whole >= 2 ? whole - 1 : whole;
    const int64_t rest = n - f * rows;
    const int64_t half = rows / 2;
    *full = f;
    return f + rest / half + (rest % half != 0);
}

// Workgroups of the dense scan kernel for (D, in, out) that the current
// device holds at once; 0 if unknown.
int scan_resident_tiles(int D, aaren_dtype in, aaren_dtype out);

// The dense scan of fp32 inputs (no segments, no precomputed scores) whose
// streams end in half tiles: tiles full_chunks .. p.chunks-1 of a stream
// cover ROWS/2 rows each, from row full_chunks * ROWS on.
hipError_t launch_scan_split(const ScanParams &p, int64_t full_chunks, int D, aaren_dtype out,
                             hipStream_t stream);

}  // namespace aaren
