// C ABI of libaaren: argument validation, workspace sizing and dispatch.
// Every check runs before anything is enqueued, so a non-OK status leaves the
// outputs untouched. The kernels live in scan.hip, step.hip and reduce.hip.
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <unordered_map>

#include "layout.h"
#include "scan_tiles.h"
#include "self_attention.h"

#define AAREN_API extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[512] = "";

aaren_status fail(aaren_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

bool log_enabled()
{
    static const bool on = [] {
        const char *e = std::getenv("AAREN_LOG");
        return e && e[0] && e[0] != '0';
    }();
    return on;
}

// Test-only: AAREN_STRESS=1 makes the look-back kernels pause tiles at
// random (read at every call, so a test can switch it on and off).
uint32_t stress_enabled()
{
    const char *e = std::getenv("AAREN_STRESS");
    return (e && e[0] && e[0] != '0') ? 1u : 0u;
}

// AAREN_HALF_TILES: -1 unset (the library chooses), 0 never, 1 always (fp32)
int half_tiles_override()
{
    const char *e = std::getenv("AAREN_HALF_TILES");
    if (!e || !e[0])
        return -1;
    return e[0] != '0' ? 1 : 0;
}

bool aligned16(const void *p)
{
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// A dtype argument's value, read from its bytes: a C caller may pass any int,
// and a value outside the enumerators must not be loaded as the enum. The
// checks below therefore take dtypes by reference and read them this way.
static_assert(sizeof(aaren_dtype) == sizeof(int), "aaren_dtype is passed as an int");

int dtype_code(const aaren_dtype &t)
{
    int v;
    std::memcpy(&v, &t, sizeof v);
    return v;
}

bool dtype_ok(const aaren_dtype &t)
{
    const int v = dtype_code(t);
    return v == AAREN_F32 || v == AAREN_BF16;
}

// a*b*... without overflow past 2^62, else -1
int64_t mul_checked(std::initializer_list<int64_t> xs)
{
    int64_t r = 1;
    for (int64_t x : xs) {
        if (x < 0)
            return -1;
        if (x != 0 && r > (int64_t(1) << 62) / x)
            return -1;
        r *= x;
    }
    return r;
}

aaren_status hip_status(hipError_t e, const char *what)
{
    if (e == hipSuccess)
        return AAREN_OK;
    return fail(AAREN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

aaren_status check_common(int64_t d, const aaren_dtype &in, const aaren_dtype &out)
{
    if (d != 64 && d != 128)
        return fail(AAREN_ERR_UNSUPPORTED, "d = %lld: supported head dimensions are 64 and 128",
                    (long long)d);
    if (!dtype_ok(in) || !dtype_ok(out))
        return fail(AAREN_ERR_UNSUPPORTED, "unknown dtype (in %d, out %d)", dtype_code(in),
                    dtype_code(out));
    return AAREN_OK;
}

aaren_status check_ptr(const void *p, const char *name)
{
    if (!p)
        return fail(AAREN_ERR_INVALID_ARG, "%s is NULL", name);
    if (!aligned16(p))
        return fail(AAREN_ERR_ALIGNMENT, "%s is not 16-byte aligned", name);
    return AAREN_OK;
}

#define CHECK(expr)                          \
    do {                                     \
        aaren_status st_ = (expr);           \
        if (st_ != AAREN_OK)                 \
            return st_;                      \
    } while (0)

size_t counter_bytes(int64_t streams)
{
    return aaren::round256((size_t)streams * aaren::kCounterStride * 4);
}

size_t scan_workspace_bytes(int64_t streams, int64_t tiles, int64_t bitmap_words, int64_t d)
{
    return aaren::kHeaderBytes + counter_bytes(streams) +
           aaren::round256((size_t)bitmap_words * 4) +
           (size_t)tiles * 2 * aaren::slot_words((int)d) * 8;
}

// Each scan call tags what it publishes with an epoch no other call of this
// process uses: eager calls 1 .. kGraphEpoch0 - 1 from this counter (wrapping
// after 2^30 - 1 calls); calls captured into a HIP graph a device-side epoch
// (see kEpochWord), marked here by 0.
uint32_t next_epoch()
{
    static std::atomic<uint32_t> counter{0};
    return counter.fetch_add(1, std::memory_order_relaxed) % (aaren::kGraphEpoch0 - 1u) + 1u;
}

bool capturing(hipStream_t stream)
{
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    return hipStreamIsCapturing(stream, &st) == hipSuccess && st == hipStreamCaptureStatusActive;
}

// The call's epoch: the host's next one, or (under graph capture) 0 after
// enqueueing the device-side advance of the header's epoch word.
aaren_status call_epoch(uint32_t *header, bool captured, hipStream_t stream, uint32_t *epoch)
{
    if (!captured) {
        *epoch = next_epoch();
        return AAREN_OK;
    }
    *epoch = 0;
    return hip_status(aaren::launch_epoch_advance(header, stream), "epoch advance launch");
}

// a / b rounded up, for a >= 0 and b > 0 (no intermediate beyond a)
int64_t ceil_div(int64_t a, int64_t b)
{
    return a / b + (a % b != 0);
}

// Consecutive workgroups per stream (see scan.hip). Measured on MI355X with
// inputs beyond the Infinity Cache: packed batches fastest at 8 (one per XCD:
// the heads of a token range are adjacent in memory); the dense backward at 4.
constexpr uint32_t kGroupDense = 4;
constexpr uint32_t kGroupPacked = 8;
// Token-major layouts (heads side by side in each row, rows far apart): 8
// consecutive workgroups per head, measured on the layer's K|V (row stride
// 8 KB): 71 us against 74-79 us with 1, 2 or 4 and 73 us with 16.
constexpr uint32_t kGroupInterleaved = 8;

// Dense forward scans choose by how many rounds of resident workgroups the
// call's tiles make (tiles / resident, resident from the kernel's occupancy):
// one workgroup per stream up to 3 rounds, 2 up to 6, 4 beyond. With one per
// stream a tile's predecessor was always dispatched `streams` workgroups
// earlier and a stream's tickets are drawn one at a time, which short calls
// feel most; long calls keep neighbouring tiles of a stream on different
// XCDs. Timed interleaved on MI355X (H = 8, N = 4096, d = 64 fp32; the
// output is the same bit for bit): B = 4, 8, 16 (0.7, 1.3, 2.7 rounds)
// 20.9, 42.7, 72.9 us with 1 against 22.5, 44.9, 76.3 us with 4; B = 32 (5.3
// rounds) 136.0 us with 2 against 137.3 with 4 and 138.6 with 1; B = 128 (21
// rounds) 513.6 us with 4 against 519.5 with 2 and 525.9 with 1. d = 128 bf16:
// 1 x 8 x 16384 (1 round) 27.5 us with 1 against 31.2 with 4; 4 x 16 x 65536
// (32 rounds) 686 us with 4 against 702 with 2.
constexpr uint32_t dense_group(int64_t tiles, int resident)
{
    if (resident <= 0)
        return kGroupDense;
    if (tiles <= 3 * (int64_t)resident)
        return 1;
    if (tiles <= 6 * (int64_t)resident)
        return 2;
    return 4;
}
static_assert(dense_group(512, 768) == 1 && dense_group(2048, 768) == 1 &&
                  dense_group(4352, 768) == 2 && dense_group(16384, 512) == 4 &&
                  dense_group(100, 0) == kGroupDense,
              "B = 4 and 16 at d = 64 on 768 resident workgroups: 1; B = 32: 2; the long bf16 "
              "batch: 4; no occupancy known: the default");

// The ticket counters sit right after the header and their number depends on
// the call's shape; a call's tile slots start where its counters end. Each
// call leaves its own counters at zero, but its slots may cover bytes that a
// later call with more streams uses as counters. So the library remembers,
// per workspace, how many counter bytes are known to be zero (all of them for
// a workspace it has not seen: it was zero-filled, by contract) and clears the
// counter region before a call that needs more than that.
// A call captured into a HIP graph runs again at every replay without passing
// through here, after whatever other calls used the workspace meanwhile. So a
// captured call always records its counter clear in the graph, and a
// workspace once used under capture is never taken as clean again: every
// later call on it clears its counters first.
struct WorkspaceRecord {
    size_t clean = SIZE_MAX;  // counter bytes known to be zero (a new workspace: all)
    bool captured = false;    // used under capture: never taken as clean again
};
std::mutex g_ws_mutex;
std::unordered_map<const void *, WorkspaceRecord> g_ws;

// `own`: the record of a workspace the library keeps itself (the static
// scratch of aaren_scan_noalloc), so that such calls look nothing up and
// insert nothing; null for a caller's workspace.
aaren_status prepare_counters(void *workspace, size_t need, bool captured, hipStream_t stream,
                              WorkspaceRecord *own = nullptr)
{
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    WorkspaceRecord &rec = own ? *own : g_ws[workspace];
    rec.captured = rec.captured || captured;
    const size_t clean = rec.captured ? 0 : rec.clean;
    if (need > clean) {
        aaren_status st = hip_status(
            aaren::launch_fill_zero(static_cast<uint8_t *>(workspace) + aaren::kHeaderBytes, need,
                                    stream),
            "counter clear launch");
        if (st != AAREN_OK)
            return st;
    }
    rec.clean = need;
    return AAREN_OK;
}

// ---- the static scan workspace of aaren_scan_noalloc ---------------------------
// For callers that cannot allocate, the scan's workspace is a static device
// array: one copy per GPU, held until the process ends, shared by every
// aaren_scan_noalloc call on that GPU. On the host its name only stands in
// for the symbol: kernels and fills get the address hipGetSymbolAddress gives
// for the current device (g_scratch), never the name.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
void *g_scratch[kMaxDevices];                // guarded by g_ws_mutex
WorkspaceRecord g_scratch_record[kMaxDevices];

// Once per device, with it current: find the array's address and zero it (a
// fill kernel, then a synchronisation: no call may see it before).
aaren_status scratch_setup(int device, void **out)
{
    if (device < 0 || device >= kMaxDevices)
        return fail(AAREN_ERR_UNSUPPORTED, "device %d: at most %d devices", device, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    if (!g_scratch[device]) {
        void *ptr = nullptr;
        CHECK(hip_status(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)),
                         "hipGetSymbolAddress of the scan scratch"));
        CHECK(hip_status(aaren::launch_fill_zero(ptr, kScratchBytes, nullptr), "scratch clear"));
        CHECK(hip_status(hipDeviceSynchronize(), "scratch clear"));
        g_scratch_record[device] = WorkspaceRecord{};
        g_scratch[device] = ptr;
    }
    *out = g_scratch[device];
    return AAREN_OK;
}

}  // namespace

// Error reporting for the layer entry point (layer.hip); not exported.
extern "C" aaren_status aaren_layer_fail(aaren_status s, const char *msg)
{
    return fail(s, "%s", msg);
}

AAREN_API int aaren_version(void)
{
    return 200;  // 0.2.0
}

AAREN_API const char *aaren_status_string(aaren_status s)
{
    // a C caller may pass any int: read its bits, not the enum (whose range
    // in C++ ends at 7)
    int code;
    std::memcpy(&code, &s, sizeof code);
    switch (code) {
    case AAREN_OK: return "ok";
    case AAREN_ERR_INVALID_ARG: return "invalid argument";
    case AAREN_ERR_UNSUPPORTED: return "unsupported";
    case AAREN_ERR_ALIGNMENT: return "misaligned pointer";
    case AAREN_ERR_WORKSPACE: return "workspace too small";
    case AAREN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

AAREN_API const char *aaren_last_error(void)
{
    return g_last_error;
}

AAREN_API aaren_status aaren_init(void)
{
    int device = 0;
    CHECK(hip_status(hipGetDevice(&device), "hipGetDevice"));
    void *ws = nullptr;
    CHECK(scratch_setup(device, &ws));
    // the dense scans' resident-workgroup counts, found here once so that
    // no later call (a captured one included) needs to ask the runtime
    for (int d : {64, 128})
        for (aaren_dtype in : {AAREN_F32, AAREN_BF16})
            for (aaren_dtype out : {AAREN_F32, AAREN_BF16})
                aaren::scan_resident_tiles(d, in, out);
    if (const char *err = aaren::layer_init(device))
        return fail(AAREN_ERR_HIP, "device %d: %s", device, err);
    return AAREN_OK;
}

AAREN_API aaren_status aaren_workspace_clear(void *workspace, size_t workspace_bytes,
                                             void *hip_stream)
{
    if (workspace_bytes == 0)
        return AAREN_OK;
    CHECK(check_ptr(workspace, "workspace"));
    CHECK(hip_status(aaren::launch_fill_zero(workspace, workspace_bytes,
                                             static_cast<hipStream_t>(hip_stream)),
                     "workspace clear launch"));
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    g_ws[workspace].clean = SIZE_MAX;
    return AAREN_OK;
}

AAREN_API aaren_status aaren_workspace_status(const void *workspace, size_t workspace_bytes,
                                              uint32_t *flags, int reset, void *hip_stream)
{
    if (!workspace || !flags)
        return fail(AAREN_ERR_INVALID_ARG, "workspace or flags is NULL");
    if (!aligned16(workspace) || (reinterpret_cast<uintptr_t>(flags) & 3u))
        return fail(AAREN_ERR_ALIGNMENT, "workspace (16 B) or flags (4 B) is misaligned");
    if (workspace_bytes < aaren::kHeaderBytes)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes has no header (%zu bytes)",
                    workspace_bytes, aaren::kHeaderBytes);
    return hip_status(
        aaren::launch_workspace_status(static_cast<uint32_t *>(const_cast<void *>(workspace)),
                                       flags, reset, static_cast<hipStream_t>(hip_stream)),
        "workspace status launch");
}

// ---- dense scan ---------------------------------------------------------------

// dense_scan_chunks: full tiles, then half tiles for the last full tile and the rest
static_assert([] { int64_t f = -1; return aaren::dense_scan_chunks(4096, 256, &f) == 17 && f == 15; }(),
              "4096 rows: 15 full tiles and 2 half tiles");
static_assert([] { int64_t f = -1; return aaren::dense_scan_chunks(1000, 256, &f) == 6 && f == 2; }(),
              "1000 rows: 2 full tiles, 488 rows in 4 half tiles");
static_assert([] { int64_t f = -1; return aaren::dense_scan_chunks(300, 256, &f) == 2 && f == 1; }(),
              "300 rows: 1 full tile (one is not split), 44 rows in a half tile");
static_assert([] { int64_t f = -1; return aaren::dense_scan_chunks(0, 256, &f) == 0 && f == 0; }(),
              "no rows, no tiles");

AAREN_API size_t aaren_scan_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d)
{
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128))
        return 0;
    // the most tiles per stream any input dtype makes: the smallest tiles
    // give the most (dense_scan_chunks does not grow with the tile height)
    int64_t full = 0;
    const int64_t per_stream = aaren::dense_scan_chunks(N, aaren::scan_tile_rows_min((int)d), &full);
    const int64_t tiles = mul_checked({B, H, per_stream});
    if (tiles < 0)
        return 0;
    return scan_workspace_bytes(B * H, tiles, 0, d);
}

namespace {

// The dense scan with explicit element strides {batch, head, row} for k/v and
// for o (lse is always [B,H,N]).
// kvs == os == nullptr: contiguous [B,H,N,d] tensors.
aaren_status scan_dense(const void *q, const void *k, const void *v, void *o, float *lse,
                        int64_t B, int64_t H, int64_t N, int64_t d, const int64_t *kv_strides,
                        const int64_t *o_strides, float scale, const aaren_dtype &in_dtype,
                        const aaren_dtype &out_dtype, void *workspace, size_t workspace_bytes,
                        void *hip_stream, WorkspaceRecord *own_record = nullptr,
                        const float *scores = nullptr, int64_t s_head_stride = 0,
                        bool check_only = false)
{
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t elems = mul_checked({B, H, N, d});
    if (elems < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    if (elems == 0)
        return AAREN_OK;
    const int64_t dense[3] = {H * N * d, N * d, d};  // no overflow: B*H*N*d fits
    const int64_t *kvs = kv_strides ? kv_strides : dense, *os = o_strides ? o_strides : dense;
    const int64_t in_bytes = in_dtype == AAREN_F32 ? 4 : 2, out_bytes = out_dtype == AAREN_F32 ? 4 : 2;
    // the last row's byte offset, b*sb + h*sh + n*sn with every index at its
    // largest, must fit in 63 bits
    const int64_t last[3] = {B - 1, H - 1, N - 1};
    int64_t kv_end = 0, o_end = 0;
    for (int i = 0; i < 3; ++i) {
        if (kvs[i] < 0 || os[i] < 0)
            return fail(AAREN_ERR_INVALID_ARG, "negative stride");
        const int64_t kb = mul_checked({kvs[i], in_bytes}), ob = mul_checked({os[i], out_bytes});
        const int64_t kt = mul_checked({last[i], kb}), ot = mul_checked({last[i], ob});
        if (kb < 0 || ob < 0 || kt < 0 || ot < 0 || kt > (int64_t(1) << 62) - kv_end ||
            ot > (int64_t(1) << 62) - o_end)
            return fail(AAREN_ERR_UNSUPPORTED, "strides address beyond 2^62 bytes");
        kv_end += kt;
        o_end += ot;
        if (kb % 16 || ob % 16)
            return fail(AAREN_ERR_ALIGNMENT, "a stride is not a multiple of 16 bytes");
    }
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    if (reinterpret_cast<uintptr_t>(lse) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    if (scores) {  // 4 floats per row and head, addressed like k but for the head stride
        if (in_dtype != AAREN_F32)
            return fail(AAREN_ERR_UNSUPPORTED, "precomputed scores go with float32 values");
        CHECK(check_ptr(scores, "scores"));
        if (s_head_stride < 0 || s_head_stride % 4 ||
            mul_checked({H - 1, s_head_stride, 4}) < 0 ||
            mul_checked({H - 1, s_head_stride, 4}) > (int64_t(1) << 62) - kv_end)
            return fail(AAREN_ERR_INVALID_ARG, "score head stride");
    }
    const int rows = aaren::scan_rows_per_tile((int)d, in_dtype);
    // Full tiles only (the layer's scored scan, and calls where halves would
    // not pay), or each stream ending in half tiles; the checks below take the
    // larger grid of the two, so they do not depend on the device.
    int64_t split_full = 0;
    const int64_t plain_chunks = ceil_div(N, rows);
    const int64_t split_chunks = aaren::dense_scan_chunks(N, rows, &split_full);
    const int64_t max_tiles = B * H * split_chunks;
    const bool interleaved = kvs[1] < kvs[2];
    // the grid is largest with the largest group a dense call may take
    const uint32_t max_group = interleaved ? kGroupInterleaved : kGroupDense;
    if (B * H * (ceil_div(split_chunks, max_group) * max_group) >= 0x7fffffff)
        return fail(AAREN_ERR_UNSUPPORTED, "%lld tiles exceed the 2^31-1 launch limit",
                    (long long)max_tiles);
    const size_t need = scan_workspace_bytes(B * H, max_tiles, 0, d);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    if (check_only)
        return AAREN_OK;
    // Half tiles shorten the drain at the end of a call, but add up to two
    // tiles per stream. They are taken for fp32 inputs only (the kernel that
    // splits waits on early loads when it widens bf16), for calls of more
    // than one round of resident workgroups (in one round every tile starts
    // at once and there is no drain to shorten: B = 4 and a single sequence
    // measured 3-6% slower with halves), and where the call's tiles still
    // make the same number of rounds (one more round costs more than the
    // drain saves).
    const int resident = scores ? 0 : aaren::scan_resident_tiles((int)d, in_dtype, out_dtype);
    const int64_t plain_tiles = B * H * plain_chunks;
    const int forced = half_tiles_override();
    const bool split =
        in_dtype == AAREN_F32 && !scores &&
        (forced >= 0 ? forced == 1
                     : resident > 0 && plain_tiles > resident &&
                           ceil_div(max_tiles, resident) == ceil_div(plain_tiles, resident));
    const int64_t chunks = split ? split_chunks : plain_chunks;
    const int64_t full_chunks = split ? split_full : plain_chunks;
    const int64_t tiles = B * H * chunks;
    const uint32_t group = interleaved ? kGroupInterleaved
                           : scores    ? kGroupDense
                                       : dense_group(tiles, resident);
    const int64_t chunks_padded = ceil_div(chunks, group) * group;

    aaren::ScanParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.lse_stream_stride = N;
    p.lse_row_stride = 1;
    p.bitmap = nullptr;
    p.bitmap_words = 0;
    p.rows = N;
    p.streams = B * H;
    p.H = H;
    p.batch_stride = kvs[0];
    p.head_stride = kvs[1];
    p.row_stride = kvs[2];
    p.o_batch_stride = os[0];
    p.o_head_stride = os[1];
    p.o_row_stride = os[2];
    p.chunks = chunks;
    p.group = group;
    p.chunks_padded = (uint32_t)chunks_padded;
    p.num_tiles = (uint32_t)tiles;
    p.stress = stress_enabled();
    p.qscale = scale * 1.44269504088896340736f;
    p.scores = scores;
    p.s_head_stride = s_head_stride;
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    p.header = reinterpret_cast<uint32_t *>(ws);
    p.counters = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes);
    p.slots = reinterpret_cast<uint64_t *>(ws + aaren::kHeaderBytes + counter_bytes(B * H));
    if (log_enabled())
        fprintf(stderr,
                "[aaren] scan B=%lld H=%lld N=%lld d=%lld tiles=%lld rows/tile=%d full tiles per "
                "stream=%lld of %lld resident=%d group=%u\n",
                (long long)B, (long long)H, (long long)N, (long long)d, (long long)tiles, rows,
                (long long)full_chunks, (long long)chunks, resident, group);
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    const bool cap = capturing(st);
    CHECK(prepare_counters(workspace, counter_bytes(B * H), cap, st, own_record));
    CHECK(call_epoch(p.header, cap, st, &p.epoch));
    if (full_chunks < chunks)  // the streams end in half tiles (fp32 inputs)
        return hip_status(aaren::launch_scan_split(p, full_chunks, (int)d, out_dtype, st),
                          "scan launch");
    return hip_status(aaren::launch_scan(p, (int)d, in_dtype, out_dtype, false, st),
                      "scan launch");
}

}  // namespace

AAREN_API aaren_status aaren_scan(const void *q, const void *k, const void *v, void *o, int64_t B,
                                  int64_t H, int64_t N, int64_t d, float scale,
                                  aaren_dtype in_dtype, aaren_dtype out_dtype, void *workspace,
                                  size_t workspace_bytes, void *hip_stream)
{
    return scan_dense(q, k, v, o, nullptr, B, H, N, d, nullptr, nullptr, scale, in_dtype,
                      out_dtype, workspace, workspace_bytes, hip_stream);
}

AAREN_API aaren_status aaren_scan_lse(const void *q, const void *k, const void *v, void *o,
                                      float *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                                      float scale, aaren_dtype in_dtype, aaren_dtype out_dtype,
                                      void *workspace, size_t workspace_bytes, void *hip_stream)
{
    if (!lse)
        return fail(AAREN_ERR_INVALID_ARG, "lse is NULL (aaren_scan takes no lse)");
    return scan_dense(q, k, v, o, lse, B, H, N, d, nullptr, nullptr, scale, in_dtype, out_dtype,
                      workspace, workspace_bytes, hip_stream);
}

AAREN_API aaren_status aaren_scan_noalloc(const void *q, const void *k, const void *v, void *o,
                                          int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                          aaren_dtype in_dtype, aaren_dtype out_dtype,
                                          void *hip_stream)
{
    // what needs no device first: the workspace this shape needs must fit
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t elems = mul_checked({B, H, N, d});
    if (elems < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    if (elems == 0)
        return AAREN_OK;
    const size_t need = aaren_scan_workspace_size(B, H, N, d);
    if (need == 0 || need > kScratchBytes)
        return fail(AAREN_ERR_UNSUPPORTED,
                    "this shape needs %zu bytes of scan workspace; the static scratch holds %zu",
                    need, kScratchBytes);
    int device = 0;
    CHECK(hip_status(hipGetDevice(&device), "hipGetDevice"));
    if (device < 0 || device >= kMaxDevices)
        return fail(AAREN_ERR_UNSUPPORTED, "device %d: at most %d devices", device, kMaxDevices);
    void *ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_mutex);
        ws = g_scratch[device];
    }
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (!ws) {
        if (capturing(st))
            return fail(AAREN_ERR_UNSUPPORTED,
                        "the scan scratch of this device is not set up: call aaren_init (or "
                        "aaren_scan_noalloc once) outside graph capture first");
        CHECK(scratch_setup(device, &ws));
    }
    return scan_dense(q, k, v, o, nullptr, B, H, N, d, nullptr, nullptr, scale, in_dtype,
                      out_dtype, ws, kScratchBytes, hip_stream, &g_scratch_record[device]);
}

AAREN_API aaren_status aaren_scan_strided(const void *q, const void *k, const void *v, void *o,
                                          float *lse, int64_t B, int64_t H, int64_t N, int64_t d,
                                          const int64_t *kv_strides, const int64_t *o_strides,
                                          float scale, aaren_dtype in_dtype,
                                          aaren_dtype out_dtype, void *workspace,
                                          size_t workspace_bytes, void *hip_stream)
{
    if (!kv_strides || !o_strides)
        return fail(AAREN_ERR_INVALID_ARG, "strides are NULL");
    return scan_dense(q, k, v, o, lse, B, H, N, d, kv_strides, o_strides, scale, in_dtype,
                      out_dtype, workspace, workspace_bytes, hip_stream);
}

aaren_status aaren::scan_scored_strided(const float *scores, int64_t s_head_stride, const float *v,
                                        void *o, int64_t B, int64_t H, int64_t N, int64_t d,
                                        const int64_t *v_strides, const int64_t *o_strides,
                                        aaren_dtype out_dtype, void *workspace,
                                        size_t workspace_bytes, void *hip_stream)
{
    if (!scores || !v_strides || !o_strides)
        return fail(AAREN_ERR_INVALID_ARG, "scores or strides are NULL");
    // q and k are not read: the scores stand in for both
    return scan_dense(scores, scores, v, o, nullptr, B, H, N, d, v_strides, o_strides, 1.f,
                      AAREN_F32, out_dtype, workspace, workspace_bytes, hip_stream, nullptr, scores,
                      s_head_stride);
}

// The checks of scan_scored_strided alone: its status for these arguments,
// with nothing enqueued (the layer runs it before its own launches).
namespace aaren {
aaren_status scan_scored_check(const float *scores, int64_t s_head_stride, const float *v,
                               void *o, int64_t B, int64_t H, int64_t N, int64_t d,
                               const int64_t *v_strides, const int64_t *o_strides,
                               aaren_dtype out_dtype, void *workspace, size_t workspace_bytes,
                               void *hip_stream)
{
    if (!scores || !v_strides || !o_strides)
        return fail(AAREN_ERR_INVALID_ARG, "scores or strides are NULL");
    return scan_dense(scores, scores, v, o, nullptr, B, H, N, d, v_strides, o_strides, 1.f,
                      AAREN_F32, out_dtype, workspace, workspace_bytes, hip_stream, nullptr, scores,
                      s_head_stride, true);
}
}  // namespace aaren

// ---- backward of the dense scan -----------------------------------------------

namespace {

size_t backward_slots_bytes(int64_t tiles, int64_t d)
{
    return (size_t)tiles * 2 * aaren::slot_words((int)d) * 8;
}

}  // namespace

AAREN_API size_t aaren_scan_backward_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d)
{
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128))
        return 0;
    const int64_t tiles = mul_checked({B, H, ceil_div(N, aaren::backward_tile_rows((int)d))});
    if (tiles < 0)
        return 0;
    return aaren::kHeaderBytes + counter_bytes(B * H) + backward_slots_bytes(tiles, d) +
           aaren::round256((size_t)tiles * d * 4);
}

AAREN_API aaren_status aaren_scan_backward(const void *q, const void *k, const void *v,
                                           const void *o, const void *dout, const float *lse,
                                           float *dq, float *dk, float *dv, int64_t B, int64_t H,
                                           int64_t N, int64_t d, float scale, aaren_dtype in_dtype,
                                           void *workspace, size_t workspace_bytes,
                                           void *hip_stream)
{
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, AAREN_F32));  // q, k, v, dout: float32 or bf16
    const int64_t elems = mul_checked({B, H, N, d});
    if (elems < 0 || mul_checked({H, d}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (elems == 0) {  // no rows: dq is an empty sum
        if (H * d == 0)
            return AAREN_OK;
        CHECK(check_ptr(dq, "dq"));
        return hip_status(aaren::launch_fill_zero(dq, (size_t)(H * d) * 4, st), "dq clear launch");
    }
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    CHECK(check_ptr(dout, "dout"));
    CHECK(check_ptr(dq, "dq"));
    CHECK(check_ptr(dk, "dk"));
    CHECK(check_ptr(dv, "dv"));
    if (!lse)
        return fail(AAREN_ERR_INVALID_ARG, "lse is NULL");
    if (reinterpret_cast<uintptr_t>(lse) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    const int64_t rows = aaren::backward_tile_rows((int)d);
    const int64_t chunks = ceil_div(N, rows);
    const int64_t tiles = B * H * chunks;
    const int64_t chunks_padded = ceil_div(chunks, kGroupDense) * kGroupDense;
    if (B * H * chunks_padded >= 0x7fffffff)
        return fail(AAREN_ERR_UNSUPPORTED, "%lld tiles exceed the 2^31-1 launch limit",
                    (long long)tiles);
    const size_t need = aaren_scan_backward_workspace_size(B, H, N, d);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    aaren::BackwardParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = static_cast<const float *>(o);
    p.g = dout;
    p.lse = lse;
    p.dk = dk;
    p.dv = dv;
    p.dq = dq;
    p.streams = B * H;
    p.H = H;
    p.N = N;
    p.batch_stride = H * N * d;
    p.head_stride = N * d;
    p.row_stride = d;
    p.lse_batch_stride = H * N;
    p.lse_head_stride = N;
    p.lse_row_stride = 1;
    p.chunks = chunks;
    p.group = kGroupDense;
    p.chunks_padded = (uint32_t)chunks_padded;
    p.num_tiles = (uint32_t)tiles;
    p.stress = stress_enabled();
    p.scale = scale;
    p.qscale = scale * 1.44269504088896340736f;
    p.header = reinterpret_cast<uint32_t *>(ws);
    p.counters = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes);
    p.slots = reinterpret_cast<uint64_t *>(ws + aaren::kHeaderBytes + counter_bytes(B * H));
    p.dq_partial = reinterpret_cast<float *>(ws + aaren::kHeaderBytes + counter_bytes(B * H) +
                                             backward_slots_bytes(tiles, d));
    if (log_enabled())
        fprintf(stderr, "[aaren] scan_backward B=%lld H=%lld N=%lld d=%lld tiles=%lld\n",
                (long long)B, (long long)H, (long long)N, (long long)d, (long long)tiles);
    const bool cap = capturing(st);
    CHECK(prepare_counters(workspace, counter_bytes(B * H), cap, st));
    CHECK(call_epoch(p.header, cap, st, &p.epoch));
    return hip_status(aaren::launch_scan_backward(p, (int)d, false, in_dtype, st),
                      "scan backward launch");
}

// ---- backward of the packed scan -------------------------------------------------

AAREN_API size_t aaren_scan_segmented_backward_workspace_size(int64_t num_seqs,
                                                              int64_t total_tokens, int64_t H,
                                                              int64_t d)
{
    if (num_seqs < 0 || total_tokens < 0 || H < 0 || (d != 64 && d != 128))
        return 0;
    const int64_t tiles = mul_checked({H, ceil_div(total_tokens, aaren::backward_tile_rows((int)d))});
    if (tiles < 0)
        return 0;
    const int64_t words = ceil_div(total_tokens, 32) + 1;
    return aaren::kHeaderBytes + counter_bytes(H) + aaren::round256((size_t)words * 4) +
           backward_slots_bytes(tiles, d) + aaren::round256((size_t)tiles * d * 4);
}

AAREN_API aaren_status aaren_scan_segmented_backward(
    const void *q, const void *k, const void *v, const void *o, const void *dout,
    const float *lse, const int64_t *offsets, float *dq, float *dk, float *dv, int64_t num_seqs,
    int64_t total_tokens, int64_t H, int64_t d, float scale, aaren_dtype in_dtype,
    void *workspace, size_t workspace_bytes, void *hip_stream)
{
    const int64_t T = total_tokens;
    if (num_seqs < 0 || T < 0 || H < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (num_seqs %lld, T %lld, H %lld)",
                    (long long)num_seqs, (long long)T, (long long)H);
    CHECK(check_common(d, in_dtype, AAREN_F32));  // q, k, v, dout: float32 or bf16
    const int64_t elems = mul_checked({T, H, d});
    if (elems < 0 || mul_checked({H, d}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "T*H*d overflows");
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (elems == 0) {  // no rows: dq is an empty sum
        if (H * d == 0)
            return AAREN_OK;
        CHECK(check_ptr(dq, "dq"));
        return hip_status(aaren::launch_fill_zero(dq, (size_t)(H * d) * 4, st), "dq clear launch");
    }
    if (num_seqs == 0)
        return fail(AAREN_ERR_INVALID_ARG, "tokens but no sequences");
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    CHECK(check_ptr(dout, "dout"));
    CHECK(check_ptr(dq, "dq"));
    CHECK(check_ptr(dk, "dk"));
    CHECK(check_ptr(dv, "dv"));
    if (!lse || !offsets)
        return fail(AAREN_ERR_INVALID_ARG, "lse or offsets is NULL");
    if ((reinterpret_cast<uintptr_t>(lse) & 3u) || (reinterpret_cast<uintptr_t>(offsets) & 7u))
        return fail(AAREN_ERR_ALIGNMENT, "lse or offsets is misaligned");
    const int64_t rows = aaren::backward_tile_rows((int)d);
    const int64_t chunks = ceil_div(T, rows);
    const int64_t tiles = H * chunks;
    const int64_t chunks_padded = ceil_div(chunks, kGroupPacked) * kGroupPacked;
    if (H * chunks_padded >= 0x7fffffff)
        return fail(AAREN_ERR_UNSUPPORTED, "%lld tiles exceed the 2^31-1 launch limit",
                    (long long)tiles);
    const size_t need = aaren_scan_segmented_backward_workspace_size(num_seqs, T, H, d);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const int64_t words = ceil_div(T, 32) + 1;  // one spare word: flags look one row ahead
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes + counter_bytes(H));
    const size_t bitmap_bytes = aaren::round256((size_t)words * 4);
    aaren::BackwardParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = static_cast<const float *>(o);
    p.g = dout;
    p.lse = lse;
    p.dk = dk;
    p.dv = dv;
    p.dq = dq;
    p.streams = H;
    p.H = H;
    p.N = T;
    p.batch_stride = 0;
    p.head_stride = d;
    p.row_stride = H * d;
    p.lse_batch_stride = 0;
    p.lse_head_stride = 1;
    p.lse_row_stride = H;
    p.bitmap = bitmap;
    p.bitmap_words = words;
    p.chunks = chunks;
    p.group = kGroupPacked;
    p.chunks_padded = (uint32_t)chunks_padded;
    p.num_tiles = (uint32_t)tiles;
    p.stress = stress_enabled();
    p.scale = scale;
    p.qscale = scale * 1.44269504088896340736f;
    p.header = reinterpret_cast<uint32_t *>(ws);
    p.counters = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes);
    p.slots = reinterpret_cast<uint64_t *>(ws + aaren::kHeaderBytes + counter_bytes(H) +
                                           bitmap_bytes);
    p.dq_partial = reinterpret_cast<float *>(ws + aaren::kHeaderBytes + counter_bytes(H) +
                                             bitmap_bytes + backward_slots_bytes(tiles, d));
    if (log_enabled())
        fprintf(stderr, "[aaren] scan_segmented_backward S=%lld T=%lld H=%lld d=%lld tiles=%lld\n",
                (long long)num_seqs, (long long)T, (long long)H, (long long)d, (long long)tiles);
    const bool cap = capturing(st);
    CHECK(prepare_counters(workspace, counter_bytes(H), cap, st));
    CHECK(call_epoch(p.header, cap, st, &p.epoch));
    CHECK(hip_status(aaren::launch_segment_flags(offsets, num_seqs, T, bitmap, words, st),
                     "segment flags launch"));
    return hip_status(aaren::launch_scan_backward(p, (int)d, true, in_dtype, st),
                      "segmented scan backward launch");
}

// ---- segmented scan -------------------------------------------------------------

AAREN_API size_t aaren_scan_segmented_workspace_size(int64_t num_seqs, int64_t total_tokens,
                                                     int64_t H, int64_t d)
{
    if (num_seqs < 0 || total_tokens < 0 || H < 0 || (d != 64 && d != 128))
        return 0;
    const int64_t tiles = mul_checked({H, ceil_div(total_tokens, aaren::scan_tile_rows_min((int)d))});
    if (tiles < 0)
        return 0;
    return scan_workspace_bytes(H, tiles, ceil_div(total_tokens, 32), d);
}

namespace {

aaren_status scan_packed(const void *q, const void *k, const void *v, void *o, float *lse,
                         const int64_t *offsets, int64_t num_seqs, int64_t total_tokens, int64_t H,
                         int64_t d, float scale, const aaren_dtype &in_dtype,
                         const aaren_dtype &out_dtype, void *workspace, size_t workspace_bytes,
                         void *hip_stream)
{
    if (num_seqs < 0 || total_tokens < 0 || H < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (num_seqs %lld, T %lld, H %lld)",
                    (long long)num_seqs, (long long)total_tokens, (long long)H);
    CHECK(check_common(d, in_dtype, out_dtype));
    if (num_seqs == 0 && total_tokens != 0)
        return fail(AAREN_ERR_INVALID_ARG, "no sequences but %lld tokens", (long long)total_tokens);
    const int64_t elems = mul_checked({total_tokens, H, d});
    if (elems < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "T*H*d overflows");
    if (elems == 0)
        return AAREN_OK;
    if (!offsets)
        return fail(AAREN_ERR_INVALID_ARG, "offsets is NULL");
    if ((reinterpret_cast<uintptr_t>(offsets) & 7u) != 0)
        return fail(AAREN_ERR_ALIGNMENT, "offsets is not 8-byte aligned");
    if (reinterpret_cast<uintptr_t>(lse) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    const int rows = aaren::scan_rows_per_tile((int)d, in_dtype);
    const int64_t chunks = ceil_div(total_tokens, rows);
    const int64_t tiles = H * chunks;
    const int64_t chunks_padded = ceil_div(chunks, kGroupPacked) * kGroupPacked;
    if (H * chunks_padded >= 0x7fffffff)
        return fail(AAREN_ERR_UNSUPPORTED, "%lld tiles exceed the 2^31-1 launch limit",
                    (long long)tiles);
    const int64_t words = ceil_div(total_tokens, 32);
    const size_t need = scan_workspace_bytes(H, tiles, words, d);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");

    uint8_t *ws = static_cast<uint8_t *>(workspace);
    uint32_t *bitmap = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes + counter_bytes(H));
    aaren::ScanParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.lse_stream_stride = 1;
    p.lse_row_stride = H;
    p.bitmap = bitmap;
    p.bitmap_words = words;
    p.rows = total_tokens;
    p.streams = H;
    p.H = H;
    p.batch_stride = p.o_batch_stride = 0;  // one batch: the packed tokens
    p.head_stride = p.o_head_stride = d;
    p.row_stride = p.o_row_stride = H * d;
    p.chunks = chunks;
    p.group = kGroupPacked;
    p.chunks_padded = (uint32_t)chunks_padded;
    p.num_tiles = (uint32_t)tiles;
    p.stress = stress_enabled();
    p.qscale = scale * 1.44269504088896340736f;
    p.header = reinterpret_cast<uint32_t *>(ws);
    p.counters = reinterpret_cast<uint32_t *>(ws + aaren::kHeaderBytes);
    p.slots = reinterpret_cast<uint64_t *>(ws + aaren::kHeaderBytes + counter_bytes(H) +
                                           aaren::round256((size_t)words * 4));
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    if (log_enabled())
        fprintf(stderr, "[aaren] scan_segmented S=%lld T=%lld H=%lld d=%lld tiles=%lld\n",
                (long long)num_seqs, (long long)total_tokens, (long long)H, (long long)d,
                (long long)tiles);
    const bool cap = capturing(st);
    CHECK(prepare_counters(workspace, counter_bytes(H), cap, st));
    CHECK(call_epoch(p.header, cap, st, &p.epoch));
    CHECK(hip_status(aaren::launch_segment_flags(offsets, num_seqs, total_tokens, bitmap, words, st),
                     "segment flag launch"));
    return hip_status(aaren::launch_scan(p, (int)d, in_dtype, out_dtype, true, st),
                      "segmented scan launch");
}

}  // namespace

AAREN_API aaren_status aaren_scan_segmented(const void *q, const void *k, const void *v, void *o,
                                            const int64_t *offsets, int64_t num_seqs,
                                            int64_t total_tokens, int64_t H, int64_t d,
                                            float scale, aaren_dtype in_dtype,
                                            aaren_dtype out_dtype, void *workspace,
                                            size_t workspace_bytes, void *hip_stream)
{
    return scan_packed(q, k, v, o, nullptr, offsets, num_seqs, total_tokens, H, d, scale,
                       in_dtype, out_dtype, workspace, workspace_bytes, hip_stream);
}

AAREN_API aaren_status aaren_scan_segmented_lse(const void *q, const void *k, const void *v,
                                                void *o, float *lse, const int64_t *offsets,
                                                int64_t num_seqs, int64_t total_tokens,
                                                int64_t H, int64_t d, float scale,
                                                aaren_dtype in_dtype, aaren_dtype out_dtype,
                                                void *workspace, size_t workspace_bytes,
                                                void *hip_stream)
{
    if (!lse)
        return fail(AAREN_ERR_INVALID_ARG, "lse is NULL (aaren_scan_segmented takes no lse)");
    return scan_packed(q, k, v, o, lse, offsets, num_seqs, total_tokens, H, d, scale, in_dtype,
                       out_dtype, workspace, workspace_bytes, hip_stream);
}

// ---- RNN step -----------------------------------------------------------------

AAREN_API aaren_status aaren_state_init(float *m, float *u, float *w, int64_t S, int64_t H,
                                        int64_t d, void *hip_stream)
{
    if (S < 0 || H < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (S %lld, H %lld)", (long long)S,
                    (long long)H);
    if (d != 64 && d != 128)
        return fail(AAREN_ERR_UNSUPPORTED, "d = %lld: supported head dimensions are 64 and 128",
                    (long long)d);
    const int64_t units = mul_checked({S, H, d});
    if (units < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "S*H*d overflows");
    if (units == 0)
        return AAREN_OK;
    if (!m || !u || !w)
        return fail(AAREN_ERR_INVALID_ARG, "state pointer is NULL");
    if (!aligned16(w))
        return fail(AAREN_ERR_ALIGNMENT, "w is not 16-byte aligned");
    if ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(u)) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "m or u is not 4-byte aligned");
    return hip_status(aaren::launch_state_init(m, u, w, S * H, d,
                                               static_cast<hipStream_t>(hip_stream)),
                      "state init launch");
}

AAREN_API aaren_status aaren_step(const void *q, const void *k_t, const void *v_t, float *m,
                                  float *u, float *w, void *o_t, int64_t S, int64_t H, int64_t d,
                                  float scale, aaren_dtype in_dtype, aaren_dtype out_dtype,
                                  void *hip_stream)
{
    if (S < 0 || H < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (S %lld, H %lld)", (long long)S,
                    (long long)H);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t elems = mul_checked({S, H, d});
    if (elems < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "S*H*d overflows");
    if (elems == 0)
        return AAREN_OK;
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k_t, "k_t"));
    CHECK(check_ptr(v_t, "v_t"));
    CHECK(check_ptr(w, "w"));
    if (o_t)
        CHECK(check_ptr(o_t, "o_t"));
    if (!m || !u)
        return fail(AAREN_ERR_INVALID_ARG, "m or u is NULL");
    if ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(u)) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "m or u is not 4-byte aligned");
    aaren::StepParams p{};
    p.q = q;
    p.k = k_t;
    p.v = v_t;
    p.m = m;
    p.u = u;
    p.w = w;
    p.o = o_t;
    p.units = S * H;
    p.H = H;
    p.tokens = 1;
    p.scale = scale;
    return hip_status(aaren::launch_step(p, (int)d, in_dtype, out_dtype,
                                         static_cast<hipStream_t>(hip_stream)),
                      "step launch");
}

AAREN_API aaren_status aaren_append(const void *q, const void *k, const void *v, float *m,
                                    float *u, float *w, void *o, int64_t S, int64_t T, int64_t H,
                                    int64_t d, float scale, aaren_dtype in_dtype,
                                    aaren_dtype out_dtype, void *hip_stream)
{
    if (S < 0 || T < 0 || H < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (S %lld, T %lld, H %lld)",
                    (long long)S, (long long)T, (long long)H);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t elems = mul_checked({T, S, H, d});
    if (elems < 0 || mul_checked({S, H, d}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "T*S*H*d overflows");
    if (elems == 0)
        return AAREN_OK;
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(w, "w"));
    if (o)
        CHECK(check_ptr(o, "o"));
    if (!m || !u)
        return fail(AAREN_ERR_INVALID_ARG, "m or u is NULL");
    if ((reinterpret_cast<uintptr_t>(m) | reinterpret_cast<uintptr_t>(u)) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "m or u is not 4-byte aligned");
    aaren::StepParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.m = m;
    p.u = u;
    p.w = w;
    p.o = o;
    p.units = S * H;
    p.H = H;
    p.tokens = T;
    p.scale = scale;
    if (log_enabled())
        fprintf(stderr, "[aaren] append S=%lld T=%lld H=%lld d=%lld\n", (long long)S,
                (long long)T, (long long)H, (long long)d);
    return hip_status(aaren::launch_append(p, (int)d, in_dtype, out_dtype,
                                           static_cast<hipStream_t>(hip_stream)),
                      "append launch");
}

// ---- self-attention, one query per token -----------------------------------------

AAREN_API size_t aaren_self_attention_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d)
{
    if (B < 0 || H < 0 || N < 0 || N > aaren::kAttnMaxN || (d != 64 && d != 128))
        return 0;
    const int64_t elems = mul_checked({B, H, d, aaren::attn_padded_keys(N)});
    if (elems < 0)
        return 0;
    // [V^T fp16][partial maxima of |V|, uint32 per (b,h) and part]
    return aaren::round256((size_t)elems * 2) +
           aaren::round256((size_t)(B * H) * aaren::kAttnVmaxParts * 4);
}

AAREN_API aaren_status aaren_self_attention(const void *q, const void *k, const void *v, void *o,
                                            float *lse, int64_t B, int64_t H, int64_t N,
                                            int64_t d, float scale, int causal,
                                            aaren_dtype in_dtype, aaren_dtype out_dtype,
                                            void *workspace, size_t workspace_bytes,
                                            void *hip_stream)
{
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, out_dtype));
    if (in_dtype != AAREN_BF16)
        return fail(AAREN_ERR_UNSUPPORTED, "self-attention takes bfloat16 q, k, v");
    if (N > aaren::kAttnMaxN)
        return fail(AAREN_ERR_UNSUPPORTED, "self-attention takes N <= %lld (N = %lld)",
                    (long long)aaren::kAttnMaxN, (long long)N);
    const int64_t elems = mul_checked({B, H, N, d});
    if (elems < 0 || mul_checked({B, H, d, aaren::attn_padded_keys(N)}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    if (elems == 0)
        return AAREN_OK;
    const int64_t blocks = B * H * ((N + aaren::kAttnQueries - 1) / aaren::kAttnQueries);
    if (blocks > 0x7fffffffLL || B * H > 65535)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H = %lld or %lld query tiles exceed the launch limits",
                    (long long)(B * H), (long long)blocks);
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
        return fail(AAREN_ERR_ALIGNMENT, "lse is not 4-byte aligned");
    const size_t need = aaren_self_attention_workspace_size(B, H, N, d);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    aaren::AttnParams p{};
    p.q = static_cast<const uint16_t *>(q);
    p.k = static_cast<const uint16_t *>(k);
    p.v = static_cast<const uint16_t *>(v);
    p.vt = static_cast<uint16_t *>(workspace);
    p.vmax = reinterpret_cast<uint32_t *>(
        static_cast<uint8_t *>(workspace) +
        aaren::round256((size_t)mul_checked({B, H, d, aaren::attn_padded_keys(N)}) * 2));
    p.o = o;
    p.lse = lse;
    p.bh = B * H;
    p.N = N;
    p.Np = aaren::attn_padded_keys(N);
    p.qscale = scale * 1.44269504088896340736f;
    p.causal = causal ? 1 : 0;
    if (log_enabled())
        fprintf(stderr, "[aaren] self_attention B=%lld H=%lld N=%lld d=%lld causal=%d\n",
                (long long)B, (long long)H, (long long)N, (long long)d, p.causal);
    return hip_status(aaren::launch_self_attention(p, (int)d, out_dtype,
                                                   static_cast<hipStream_t>(hip_stream)),
                      "self-attention launch");
}

// ---- many-to-one reduction ------------------------------------------------------

namespace {

// chunks per (b,h): enough workgroups to cover the chip a few times, at least
// one iteration of rows each, at most kReduceMaxParts
int64_t reduce_parts(int64_t units, int64_t N, int64_t d)
{
    const int64_t per_iter = aaren::reduce_rows_per_iteration((int)d, AAREN_F32) <
                                     aaren::reduce_rows_per_iteration((int)d, AAREN_BF16)
                                 ? aaren::reduce_rows_per_iteration((int)d, AAREN_F32)
                                 : aaren::reduce_rows_per_iteration((int)d, AAREN_BF16);
    int64_t parts = ceil_div(2048, units > 0 ? units : 1);
    const int64_t by_rows = ceil_div(N, per_iter);
    if (parts > by_rows)
        parts = by_rows;
    if (parts > aaren::kReduceMaxParts)
        parts = aaren::kReduceMaxParts;
    return parts < 1 ? 1 : parts;
}

}  // namespace

AAREN_API size_t aaren_reduce_workspace_size(int64_t B, int64_t H, int64_t N, int64_t d)
{
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128))
        return 0;
    const int64_t units = mul_checked({B, H});
    if (units < 0)
        return 0;
    const int64_t n = mul_checked({units, reduce_parts(units, N, d), aaren::slot_words((int)d), 4});
    return n < 0 ? 0 : (size_t)n;
}

namespace {

size_t mean_query_parts_bytes(int64_t units, int64_t parts, int64_t d, size_t *reduce_b,
                              size_t *mean_b)
{
    *reduce_b = aaren::round256((size_t)units * parts * aaren::slot_words((int)d) * 4);
    *mean_b = aaren::round256((size_t)units * parts * d * 8);
    return *reduce_b + *mean_b + aaren::round256((size_t)units * d * 4);
}

}  // namespace

AAREN_API size_t aaren_mean_query_attention_workspace_size(int64_t B, int64_t H, int64_t N,
                                                           int64_t d)
{
    if (B < 0 || H < 0 || N < 0 || (d != 64 && d != 128))
        return 0;
    const int64_t units = mul_checked({B, H});
    if (units < 0 || mul_checked({B, H, N, d}) < 0)
        return 0;
    size_t rb, mb;
    return mean_query_parts_bytes(units, reduce_parts(units, N, d), d, &rb, &mb);
}

AAREN_API aaren_status aaren_mean_query_attention(const void *hq, const void *k, const void *v,
                                                  void *o, float *g_out, int64_t B, int64_t H,
                                                  int64_t N, int64_t d, float scale,
                                                  aaren_dtype in_dtype, aaren_dtype out_dtype,
                                                  void *workspace, size_t workspace_bytes,
                                                  void *hip_stream)
{
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t units = mul_checked({B, H});
    if (units < 0 || mul_checked({B, H, N, d}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    if (units == 0)
        return AAREN_OK;
    if (N == 0)
        return fail(AAREN_ERR_INVALID_ARG, "N = 0: the mean of no queries has no value");
    if (units > 0x7fffffff / aaren::kReduceMaxParts)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H = %lld is too large", (long long)units);
    CHECK(check_ptr(hq, "hq"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    if (g_out)
        CHECK(check_ptr(g_out, "g_out"));
    const int64_t parts = reduce_parts(units, N, d);
    size_t rb, mb;
    const size_t need = mean_query_parts_bytes(units, parts, d, &rb, &mb);
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    aaren::ReduceParams p{};
    p.q = hq;
    p.k = k;
    p.v = v;
    p.o = o;
    p.partials = reinterpret_cast<float *>(ws);
    p.mean_partials = reinterpret_cast<double *>(ws + rb);
    p.q_mean = reinterpret_cast<float *>(ws + rb + mb);
    p.g_out = g_out;
    p.q_unit = p.q_mean;
    p.units = units;
    p.H = H;
    p.N = N;
    p.parts = parts;
    p.rows_per_part = ceil_div(N, parts);
    p.qscale = scale * 1.44269504088896340736f;
    hipStream_t st = static_cast<hipStream_t>(hip_stream);
    CHECK(hip_status(aaren::launch_mean_query(p, (int)d, in_dtype, st), "mean-query launch"));
    return hip_status(aaren::launch_reduce(p, (int)d, in_dtype, out_dtype, st), "reduce launch");
}

AAREN_API aaren_status aaren_reduce(const void *q, const void *k, const void *v, void *o,
                                    float *m_out, float *u_out, int64_t B, int64_t H, int64_t N,
                                    int64_t d, float scale, aaren_dtype in_dtype,
                                    aaren_dtype out_dtype, void *workspace, size_t workspace_bytes,
                                    void *hip_stream)
{
    if (B < 0 || H < 0 || N < 0)
        return fail(AAREN_ERR_INVALID_ARG, "negative size (B %lld, H %lld, N %lld)",
                    (long long)B, (long long)H, (long long)N);
    CHECK(check_common(d, in_dtype, out_dtype));
    const int64_t units = mul_checked({B, H});
    if (units < 0 || mul_checked({B, H, N, d}) < 0)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H*N*d overflows");
    if (units == 0)
        return AAREN_OK;
    if (N == 0)
        return fail(AAREN_ERR_INVALID_ARG, "N = 0: attention over no pairs has no value");
    if (units > 0x7fffffff / aaren::kReduceMaxParts)
        return fail(AAREN_ERR_UNSUPPORTED, "B*H = %lld is too large", (long long)units);
    CHECK(check_ptr(q, "q"));
    CHECK(check_ptr(k, "k"));
    CHECK(check_ptr(v, "v"));
    CHECK(check_ptr(o, "o"));
    if ((reinterpret_cast<uintptr_t>(m_out) | reinterpret_cast<uintptr_t>(u_out)) & 3u)
        return fail(AAREN_ERR_ALIGNMENT, "m_out or u_out is not 4-byte aligned");
    const int64_t parts = reduce_parts(units, N, d);
    const size_t need = (size_t)units * parts * aaren::slot_words((int)d) * 4;
    if (!workspace || workspace_bytes < need)
        return fail(AAREN_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes,
                    need);
    if (!aligned16(workspace))
        return fail(AAREN_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
    aaren::ReduceParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.m_out = m_out;
    p.u_out = u_out;
    p.partials = static_cast<float *>(workspace);
    p.units = units;
    p.H = H;
    p.N = N;
    p.parts = parts;
    p.rows_per_part = ceil_div(N, parts);
    p.qscale = scale * 1.44269504088896340736f;
    if (log_enabled())
        fprintf(stderr, "[aaren] reduce B=%lld H=%lld N=%lld d=%lld parts=%lld rows/part=%lld\n",
                (long long)B, (long long)H, (long long)N, (long long)d, (long long)parts,
                (long long)p.rows_per_part);
    return hip_status(aaren::launch_reduce(p, (int)d, in_dtype, out_dtype,
                                           static_cast<hipStream_t>(hip_stream)),
                      "reduce launch");
}
