// C ABI of the dense BF16 GEMM library: argument checks, the shape-based
// plan (kernel + tile + split + launch geometry), per-device state and
// dispatch to the kernel launchers.  Declared in include/hkg.h.
#include "hkg.h"
#include "hkg_internal.h"
#include "hkg_tile_order.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cstdio>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

namespace hkg {
namespace {

// MI355X: 256 compute units in 8 XCDs of 32 (HipKittens talk notes, section
// "compute hierarchy").  The plan is a pure function of (M, N, K) on this
// device; a device that reports a different count still runs every plan
// correctly.
constexpr int kNumCUs = 256;

// Skinny path for M up to this many rows (decode shapes) when its column
// blocks of 16 fill at most two rounds of compute units (N <= 16 * 512).
// Beyond that the 4-stage 64 x 64 tile (B read once per 64 rows) keeps up
// with it on MI355X (A through LDS, rotating buffers, graph timing, the two
// interleaved): K = 4096, M = 16: N = 5120 15.6 vs 19.5 us for the tile,
// 6144 15.8 vs 19.9, 8192 17.3 vs 21.3 (K = 8192: 31.0 vs 41.2); N = 8192
// at M = 12 16.0 vs 21.2 and M = 4 14.8 vs 20.8; and past two rounds,
// M = 16: N = 12288 24.5 vs 24.2, 14336 30.3 vs 27.8, 28672 55.1 vs 51.9.  (With A loaded
// straight into registers the tile led from N = 12288, 26 vs 31 us; at
// M = 32 the tile leads: N = K = 4096 12 vs 16 us.)  Wider column blocks
// through LDS (32 and 64 columns per workgroup) were slower at every one
// of those shapes but N = 14336 (27.6 us with 64 columns).
constexpr int64_t kSkinnyMaxM = 16;
constexpr int64_t kSkinnyMaxColBlocks = 2 * kNumCUs;
// Largest split-K factor of the tile kernel.
constexpr int64_t kMaxTileSplit = 16;

// Largest dimension the kernels index with 32-bit arithmetic.
constexpr int64_t kMaxDim = INT32_MAX;

thread_local std::string g_last_hip_error;

void set_hip_error(hipError_t e, const char* where)
{
    char buf[256];
    std::snprintf(buf, sizeof buf, "%s: %s (%d)", where, hipGetErrorString(e), (int)e);
    g_last_hip_error = buf;
}

void copy_str(char* dst, size_t cap, const char* src)
{
    std::snprintf(dst, cap, "%s", src);
}

// ---------------------------------------------------------------- per device
// Library-owned scratch of one (device, stream): the split-K fp32 partials
// and arrival counters, the packed MXFP8 scales of hkg_gemm_mxfp8 and the
// row-layout copies of column-layout operands (hkg_gemm_bf16_ex).  Calls on
// one stream run in order, so they can share it; calls on different streams
// each have their own, so they do not race.
struct Workspace {
    float* ws = nullptr;          // split-K partials
    size_t ws_bytes = 0;
    int* counters = nullptr;      // split-K arrival counters (kept zero between calls)
    size_t counter_count = 0;
    uint8_t* mx_ws = nullptr;     // packed MXFP8 scales
    size_t mx_ws_bytes = 0;
    uint16_t* layout_ws = nullptr;
    size_t layout_ws_bytes = 0;
};

struct StreamKey {
    hipStream_t stream;
    std::thread::id thread;       // only for hipStreamPerThread (one stream per host thread)
    bool operator<(const StreamKey& o) const
    {
        return stream != o.stream ? std::less<hipStream_t>()(stream, o.stream) : thread < o.thread;
    }
};

struct DeviceState {
    std::once_flag once;
    hkg_status_t status = HKG_ERR_NO_DEVICE;
    std::mutex ws_mutex;
    std::map<StreamKey, Workspace> per_stream;
    // Outgrown buffers.  A launch still in flight, or a captured graph, may
    // hold their addresses, so they are released only when the library is
    // unloaded, never earlier.  Growth is geometric, so they add up to less
    // than the buffers in use.
    std::vector<void*> retired;
};

constexpr int kMaxDevices = 64;
DeviceState g_devices[kMaxDevices];

hkg_status_t current_device(int* dev_out)
{
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) {
        if (e != hipSuccess)
            set_hip_error(e, "hipGetDeviceCount");
        return HKG_ERR_NO_DEVICE;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) {
        set_hip_error(e, "hipGetDevice");
        return HKG_ERR_NO_DEVICE;
    }
    if (dev < 0 || dev >= kMaxDevices)
        return HKG_ERR_UNSUPPORTED;
    DeviceState& d = g_devices[dev];
    std::call_once(d.once, [&]() {
        hipDeviceProp_t prop;
        hipError_t pe = hipGetDeviceProperties(&prop, dev);
        if (pe != hipSuccess) {
            set_hip_error(pe, "hipGetDeviceProperties");
            d.status = HKG_ERR_HIP;
            return;
        }
        d.status = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? HKG_OK : HKG_ERR_ARCH;
    });
    *dev_out = dev;
    return d.status;
}

StreamKey stream_key(hipStream_t stream)
{
    return StreamKey{stream, stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id()};
}

// A workspace buffer may only grow outside stream capture: allocating (and
// zeroing counters) are not stream-ordered work a graph could replay, and a
// buffer allocated for one capture would be shared by every replay.
hkg_status_t check_not_capturing(hipStream_t stream, const char* what)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(stream, &cs);
    if (e != hipSuccess) {
        set_hip_error(e, "hipStreamIsCapturing");
        return HKG_ERR_HIP;
    }
    if (cs != hipStreamCaptureStatusNone) {
        char buf[256];
        std::snprintf(buf, sizeof buf,
                      "%s must grow while the stream is being captured: run the same call once "
                      "outside capture first", what);
        g_last_hip_error = buf;
        return HKG_ERR_WORKSPACE;
    }
    return HKG_OK;
}

// Grow *buf to at least `bytes` (geometrically; the old buffer is retired,
// not freed).  Called with the device's ws_mutex held.
template <typename T>
hkg_status_t grow(DeviceState& d, hipStream_t stream, T** buf, size_t* have, size_t bytes, const char* what,
                  bool zero)
{
    if (*have >= bytes)
        return HKG_OK;
    hkg_status_t st = check_not_capturing(stream, what);
    if (st != HKG_OK)
        return st;
    const size_t want = std::max(bytes, 2 * *have);
    void* p = nullptr;
    hipError_t e = hipMalloc(&p, want);
    if (e == hipSuccess && zero)
        e = hipMemset(p, 0, want);
    if (e != hipSuccess) {
        set_hip_error(e, what);
        if (p)
            (void)hipFree(p);
        return HKG_ERR_WORKSPACE;
    }
    if (*buf)
        d.retired.push_back((void*)*buf);
    *buf = (T*)p;
    *have = want;
    return HKG_OK;
}

// Split-K scratch of (dev, stream): partials of ws_bytes, `counters` zeroed
// arrival counters.
hkg_status_t get_workspace(int dev, hipStream_t stream, size_t ws_bytes, size_t counters, float** ws, int** cnt)
{
    DeviceState& d = g_devices[dev];
    std::lock_guard<std::mutex> lock(d.ws_mutex);
    Workspace& w = d.per_stream[stream_key(stream)];
    hkg_status_t st = grow(d, stream, &w.ws, &w.ws_bytes, ws_bytes, "split-K workspace", false);
    if (st != HKG_OK)
        return st;
    size_t cnt_bytes = w.counter_count * sizeof(int);
    st = grow(d, stream, &w.counters, &cnt_bytes, counters * sizeof(int), "split-K counters", true);
    if (st != HKG_OK)
        return st;
    w.counter_count = cnt_bytes / sizeof(int);
    *ws = w.ws;
    *cnt = w.counters;
    return HKG_OK;
}

// Packed-scale buffer of hkg_gemm_mxfp8 for (dev, stream).
hkg_status_t get_mx_workspace(int dev, hipStream_t stream, size_t bytes, uint8_t** out)
{
    DeviceState& d = g_devices[dev];
    std::lock_guard<std::mutex> lock(d.ws_mutex);
    Workspace& w = d.per_stream[stream_key(stream)];
    hkg_status_t st = grow(d, stream, &w.mx_ws, &w.mx_ws_bytes, bytes, "MXFP8 scale workspace", false);
    *out = w.mx_ws;
    return st;
}

// Row-layout copies of column-layout operands for (dev, stream).
hkg_status_t get_layout_workspace(int dev, hipStream_t stream, size_t bytes, uint16_t** out)
{
    DeviceState& d = g_devices[dev];
    std::lock_guard<std::mutex> lock(d.ws_mutex);
    Workspace& w = d.per_stream[stream_key(stream)];
    hkg_status_t st = grow(d, stream, &w.layout_ws, &w.layout_ws_bytes, bytes, "layout workspace", false);
    *out = w.layout_ws;
    return st;
}

// --------------------------------------------------------------------- plan
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

void fill_resources(hkg_plan_t* p, const KernelResources* r)
{
    if (!r)
        return;
    p->vgprs = r->vgprs;
    p->agprs = r->agprs;
    p->sgprs = r->sgprs;
    p->scratch_bytes = r->scratch;
    if (r->lds >= 0)
        p->lds_bytes = r->lds;          // the code object's figure (static LDS of the kernel)
}

hkg_status_t check_dims(int64_t M, int64_t N, int64_t K)
{
    if (M < 0 || N < 0 || K < 0)
        return HKG_ERR_INVALID_ARG;
    if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
        return HKG_ERR_INVALID_ARG;
    // Each of A, B and C holds fewer than 2^40 elements (2 TiB of bf16).
    const int64_t lim = (int64_t)1 << 40;
    if ((M && K >= lim / M) || (N && K >= lim / N) || (M && N >= lim / M))
        return HKG_ERR_INVALID_ARG;
    return HKG_OK;
}

void fill_tile(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N);

void plan_tile(int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    // Compute-bound shapes, largest tile first (output-tile size dominates:
    // HipKittens talk notes, Table 2; tile selection by grid fill: FlyDSL
    // "Prebuilt kernels guide", section 3c).  The 256 x 256 ping-pong tile
    // when its tiles fill at least three quarters of the compute units;
    // else, while 128 x 128 tiles outnumber the compute units, the two-stage
    // 128 x 128 tile, two workgroups per compute unit.  Measured on MI355X
    // against the 256 x 128 tile: M = 3072, N = K = 4096 (192 tiles of
    // 256 x 256) 93 vs 160 us; M = 1536 68 vs 88 us; M = 1024, N = K = 8192
    // 139 vs 159 us.
    {
        const TileShape s = tile_shape(TILE_LADDER[0]);
        const int64_t t256 = cdiv(M, s.bm) * cdiv(N, s.bn);
        if (4 * t256 >= 3 * kNumCUs) {
            // More tiles than compute units and a last round filling at most
            // half of them: that round's tiles are split in two halves of K
            // (split_k 2; run as the grouped kernel with one expert, whose
            // streamed schedule does exactly this), so it takes half a tile's
            // time.  Measured on MI355X (us, split vs whole, torch.mm):
            // 4352 x 4096 x 4096 (272 tiles) 134.2 vs 153.0 (132.6);
            // 4096 x 5120 x 4096 (320) 137.3 vs 154.3 (142.0); 4608^2 x 4096
            // (324) 139.7 vs 153.9 (142.3); 6144 x 4096 x 8192 (384) 287.5 vs
            // 303.7 (293.0); 6144 x 4096 x 4096 158.1 vs 158.9 (153.2).
            const int64_t rem = t256 % kNumCUs;
            const bool split_tail = t256 > kNumCUs && rem > 0 && 2 * rem <= kNumCUs && cdiv(K, s.bk) >= 2;
            fill_tile(p, TILE_LADDER[0], split_tail ? 2 : 1, M, N);
            return;
        }
        // One round of k-interleaved tiles (schedule 7): 128 x 256 tiles
        // when they fill 160 to 256 compute units, 128 x 128 tiles when they
        // fill 224 to 256, for K of at least 1024 and rows at most a quarter
        // padding.  Measured on MI355X (rotating buffers, us, k-interleaved
        // vs the tile it replaces, torch.mm): 2048 x 4096 x 4096 59.0 vs 63.3
        // (58.3); 1280 x 4096 x 4096 58.7 vs 65.3 (48.4); 1024 x 8192 x 8192
        // 110.4 vs 121.3 (109.7); 256 x 32768 x 4096 78.1 vs 93.1 (76.0);
        // 128 x 40960 x 4096 85.7 vs 94.7 (81.2); under 224 tiles with few
        // tile rows or K = 1024 it loses 2-3%: 768 x 8192 x 4096 69.8 vs
        // 68.2 (54.8), 640 x 8192 x 4096 66.9 vs 65.6, 1536 x 4096 x 1024
        // 19.7 vs 19.3; below K = 1024 it loses more.  128 x 128 tiles:
        // 1024 x 4096 x 4096 37.3 vs 45.4 (36.5); 512 x 8192 x 4096 44.9 vs
        // 49.0 (42.6); 1024 x 4096 x 1024 13.8 vs 16.1 (19.6).  With fewer
        // 128 x 128 tiles the streaming tiles win where they fill a round
        // (512 x 6144 x 4096, 192 tiles: 55.3 vs 39.5 for 128 x 96 tiles).
        if (K >= 1024) {
            const TileShape w = tile_shape(TILE_KINTER[0]);
            const int64_t tw = cdiv(M, w.bm) * cdiv(N, w.bn);
            const bool rows_ok = 4 * (cdiv(M, w.bm) * w.bm - M) <= cdiv(M, w.bm) * w.bm;
            if (rows_ok && 8 * tw >= 5 * kNumCUs && tw <= kNumCUs) {
                fill_tile(p, TILE_KINTER[0], 1, M, N);
                return;
            }
        }
        const TileShape t = tile_shape(TILE_LADDER[1]);
        if (cdiv(M, t.bm) * cdiv(N, t.bn) > kNumCUs) {
            fill_tile(p, TILE_LADDER[1], 1, M, N);
            return;
        }
        // 128 x 128: five stages in LDS (copies four stages ahead) from
        // K = 4096, three below: 1024 x 4096 x 4096 40.4 vs 42.7 us,
        // 1024 x 4096 x 8192 76.0 vs 79.8, 512 x 8192 x 8192 79.0 vs 82.5,
        // 1024 x 4096 x 1024 14.1 vs 13.6.
        if (K >= 1024) {
            const int v = K >= 4096 ? TILE_KINTER[2] : TILE_KINTER[1];
            const TileShape w = tile_shape(v);
            const int64_t tw = cdiv(M, w.bm) * cdiv(N, w.bn);
            const bool rows_ok = 4 * (cdiv(M, w.bm) * w.bm - M) <= cdiv(M, w.bm) * w.bm;
            if (rows_ok && 8 * tw >= 7 * kNumCUs && tw <= kNumCUs) {
                fill_tile(p, v, 1, M, N);
                return;
            }
        }
    }
    // Smaller outputs: the operands are streamed from HBM a few times at most
    // and the kernel is bound by memory, so the grid should put one workgroup
    // with a deep copy pipeline on every compute unit.  For each streaming tile, split K so
    // the grid stays within one workgroup per compute unit (at least 8 k-tiles
    // per split; split-K adds fp32 partial traffic and a reduction), then take
    // the tile with the fewest splits; on a tie, the smallest tile whose grid
    // still fits one workgroup per compute unit (each workgroup's chain of
    // loads and MFMAs is then shortest), the taller one between 128 x 64 and
    // 64 x 128.  A tile whose rows would be more than a quarter padding is
    // skipped unless it is the last one.  Measured on MI355X: M = 128,
    // N = 12288, K = 4096 (graph-timed over rotating buffers): 64 x 96
    // unsplit (exactly 256 tiles) 32.5 us, 128 x 64 unsplit (192 tiles)
    // 34.7 us, 128 x 48 (256 tiles, 2 waves) 35.9 us, 64 x 64 unsplit (384
    // tiles) 39.1 us, 128 x 128 split 2 44.8 us; M = 256, N = K = 4096:
    // 64 x 64 unsplit 21.9 us, 128 x 64 split 2 22.6 us; 256^3: 64 x 64 3.8 us,
    // 128 x 128 7.2 us; 512^3: 64 x 64 unsplit 5.1 us, split 2 6.7 us,
    // 128 x 128 split 2 13.1 us.  128 x 96 where it is the smallest tile
    // filling one round (M = 256, N = 12288: 256 tiles) against 128 x 128 (192
    // tiles): 44.7 vs 51.2 us; M = 1024, N = 3072: 41.8 vs 46.9; M = 512,
    // N = 5120: 38.9 vs 46.7; M = 128, N = 18432: 47.0 vs 53.9 (K = 4096).
    int best = -1;
    int64_t best_split = 0, best_area = 0;
    bool best_fits = false;
    const int n_stream = (int)(sizeof(STREAM_TILES) / sizeof(STREAM_TILES[0]));
    for (int i = 0; i < n_stream; ++i) {
        const int v = STREAM_TILES[i];
        const TileShape s = tile_shape(v);
        const int64_t tm = cdiv(M, s.bm), tn = cdiv(N, s.bn);
        if (i + 1 < n_stream && 4 * (tm * s.bm - M) > tm * s.bm)
            continue;
        int64_t split = 1;
        if (tm * tn < kNumCUs && M * N < ((int64_t)1 << 29) && tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched)) {   // fp32 partials addressed in 32 bits
            split = std::min<int64_t>(kNumCUs / (tm * tn), cdiv(K, s.bk) / 8);
            split = std::max<int64_t>(1, std::min<int64_t>(split, kMaxTileSplit));
        }
        const bool fits = tm * tn <= kNumCUs;
        const int64_t area = (int64_t)s.bm * s.bn;
        if (best < 0 || split < best_split ||
            (split == best_split && fits && (!best_fits || area < best_area))) {
            best = v;
            best_split = split;
            best_area = area;
            best_fits = fits;
        }
    }
    fill_tile(p, best, best_split, M, N);
}

// Fill the tile-kernel fields of p for (variant, split).
void fill_tile(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N)
{
    const TileShape s = tile_shape(variant);
    const int64_t tm = cdiv(M, s.bm), tn = cdiv(N, s.bn);
    p->kernel_id = HKG_KERNEL_TILE;
    p->variant = variant;
    p->tile_m = s.bm;
    p->tile_n = s.bn;
    p->tile_k = s.bk;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    // the persistent schedule runs at most one workgroup per compute unit
    p->grid_x = (int32_t)(s.sched == 6 ? std::min<int64_t>(tm * tn, kPersistentGrid) : tm * tn);
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    const bool split_tail = s.sched == 6 && split == 2;
    if (split_tail) {                   // one partial tile per workgroup, one grid
        p->grid_y = 1;
        p->workspace_bytes = (int64_t)p->grid_x * s.bm * s.bn * 4;
    }
    // Chiplet-aware order (talk notes, section 3): 8-tall windows, so one
    // XCD's 32 concurrent workgroups cover an 8 x 4 block of tiles, and 32
    // consecutive tiles per XCD; off when the grid is under one XCD round.
    p->xcd_window_w = tm >= 8 ? 8 : (int32_t)tm;
    p->xcd_chunk_c = (tm * tn >= 8 * 32) ? 32 : 0;
    p->lds_bytes = tile_lds_bytes(variant);
    fill_resources(p, tile_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "tile_%dx%dx%d_s%d_w%dx%d_p%d", s.bm, s.bn, s.bk,
                  s.stages, s.wm, s.wn, s.sched);
    std::snprintf(p->reason, sizeof p->reason, "%lldx%lld tiles of %dx%d (%d stages), split-K %lld on %d CUs%s",
                  (long long)tm, (long long)tn, s.bm, s.bn, s.stages, (long long)split, kNumCUs,
                  split_tail ? ", persistent, last round split in two halves of K"
                  : s.sched == 6 ? ", persistent" : s.sched == 7 ? ", k-interleaved" : "");
}

// Fill the skinny-kernel fields of p for (variant, split).
void fill_skinny(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N, const char* why)
{
    const SkinnyShape s = skinny_shape(variant);
    const int64_t col_blocks = cdiv(N, 16 * s.nblocks);
    p->kernel_id = HKG_KERNEL_SKINNY;
    p->variant = variant;
    p->tile_m = 16 * s.mblocks;
    p->tile_n = 16 * s.nblocks;
    p->tile_k = 32;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    p->grid_x = (int32_t)col_blocks;
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->xcd_window_w = 0;
    p->xcd_chunk_c = 0;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    p->lds_bytes = skinny_lds_bytes(variant);
    fill_resources(p, skinny_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "skinny_m%d_n%d_w%d_u%d_c%d%s", 16 * s.mblocks,
                  16 * s.nblocks, s.waves, s.unroll, s.cache_policy, s.a_lds ? "_lds" : "");
    std::snprintf(p->reason, sizeof p->reason, "M <= %d; %lld column blocks of %d, split-K %lld%s%s",
                  (int)kSkinnyMaxM, (long long)col_blocks, 16 * s.nblocks, (long long)split, why ? "; " : "",
                  why ? why : "");
}

void plan_skinny(int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    // Smallest A coverage (16-row blocks) that holds M; one B block per
    // workgroup; A through LDS where a variant stages it (the 16-row cover:
    // at N = K = 4096 on MI355X, 9.9 vs 11.0 us with the direct fragment
    // loads at M = 16, 9.2 vs 9.6 at M = 8, 8.9 vs 8.8 at M = 1); split K
    // across workgroups only when the column blocks underfill the device,
    // keeping at least 8 steps (256 k) per wave.
    int variant = -1, best = 1 << 30;
    for (int v = 0; v < SKINNY_NUM_VARIANTS; ++v) {
        const SkinnyShape s = skinny_shape(v);
        const int rank = 2 * s.mblocks + (s.a_lds ? 0 : 1);
        if (s.nblocks == 1 && 16 * (int64_t)s.mblocks >= M && rank < best) {
            variant = v;
            best = rank;
        }
    }
    const SkinnyShape s = skinny_shape(variant);
    const int64_t col_blocks = cdiv(N, 16 * s.nblocks);
    const int64_t steps = cdiv(K, 32);
    int64_t split = 1;
    if (col_blocks < kNumCUs) {
        split = cdiv(kNumCUs, col_blocks);
        const int64_t max_split = steps / (8 * s.waves);
        if (split > max_split)
            split = max_split;
        if (split > 64)
            split = 64;
        if (split < 1)
            split = 1;
    }
    fill_skinny(p, variant, split, M, N, nullptr);
}

void plan_generic(int64_t M, int64_t N, hkg_plan_t* p, const char* why)
{
    p->kernel_id = HKG_KERNEL_GENERIC;
    p->variant = 0;
    p->tile_m = 16;
    p->tile_n = 16;
    p->tile_k = 1;
    p->waves = 4;
    p->split_k = 1;
    p->grid_x = (int32_t)cdiv(N, 16);
    p->grid_y = (int32_t)std::min<int64_t>(cdiv(M, 16), 65535);
    p->grid_z = 1;
    p->block_x = 256;
    p->xcd_window_w = 0;
    p->xcd_chunk_c = 0;
    p->workspace_bytes = 0;
    p->lds_bytes = 0;
    fill_resources(p, generic_resources());
    copy_str(p->kernel_name, sizeof p->kernel_name, "generic");
    copy_str(p->reason, sizeof p->reason, why);
}

hkg_status_t make_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    std::memset(p, 0, sizeof *p);
    p->abi_version = HKG_ABI_VERSION;
    p->M = M;
    p->N = N;
    p->K = K;
    p->split_k = 1;
    p->vgprs = p->agprs = p->sgprs = p->scratch_bytes = -1;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    p->flops = 2.0 * (double)M * (double)N * (double)K;
    p->algorithmic_bytes = 2.0 * ((double)M * K + (double)N * K + (double)M * N);
    if (M == 0 || N == 0) {
        p->kernel_id = HKG_KERNEL_NONE;
        copy_str(p->kernel_name, sizeof p->kernel_name, "none");
        copy_str(p->reason, sizeof p->reason, "empty output");
        return HKG_OK;
    }
    if (K == 0) {
        p->kernel_id = HKG_KERNEL_ZERO;
        p->grid_x = 1;
        p->block_x = 256;
        copy_str(p->kernel_name, sizeof p->kernel_name, "zero");
        copy_str(p->reason, sizeof p->reason, "K == 0: C is the empty sum, +0");
        return HKG_OK;
    }
    if (K % 8 != 0) {
        plan_generic(M, N, p, "K % 8 != 0: fast kernels load 8 k values per 16-byte access");
        return HKG_OK;
    }
    // Buffer-resource ranges of one tile / of A must stay below 2^31 bytes.
    if (K > (int64_t)(INT32_MAX / 2) / 256) {
        plan_generic(M, N, p, "K too large for 32-bit buffer offsets of a tile");
        return HKG_OK;
    }
    if (M <= kSkinnyMaxM && cdiv(N, 16) <= kSkinnyMaxColBlocks) {
        plan_skinny(M, N, K, p);
        return HKG_OK;
    }
    plan_tile(M, N, K, p);
    const int64_t grid = (int64_t)cdiv(M, p->tile_m) * cdiv(N, p->tile_n);
    if (grid > INT32_MAX)
        plan_generic(M, N, p, "tile grid beyond 2^31 workgroups");
    return HKG_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void* a, int64_t a_bytes, const void* b, int64_t b_bytes)
{
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a_bytes > 0 && b_bytes > 0 && a0 < b0 + (uintptr_t)b_bytes && b0 < a0 + (uintptr_t)a_bytes;
}

hkg_status_t check_pointers(const void* A, const void* B, const void* C, int64_t M, int64_t N, int64_t K)
{
    const int64_t a_bytes = 2 * M * K, b_bytes = 2 * N * K, c_bytes = 2 * M * N;
    if ((a_bytes && !A) || (b_bytes && !B) || (c_bytes && !C))
        return HKG_ERR_INVALID_ARG;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes))
        return HKG_ERR_INVALID_ARG;
    return HKG_OK;
}

bool plan_matches_library(const hkg_plan_t* p)
{
    switch (p->kernel_id) {
    case HKG_KERNEL_NONE:
        return p->M == 0 || p->N == 0;
    case HKG_KERNEL_ZERO:
        return p->K == 0 && p->M > 0 && p->N > 0;
    case HKG_KERNEL_GENERIC:
        return true;
    case HKG_KERNEL_TILE: {
        if (p->variant < 0 || p->variant >= TILE_NUM_VARIANTS)
            return false;
        const TileShape s = tile_shape(p->variant);
        return p->tile_m == s.bm && p->tile_n == s.bn && p->tile_k == s.bk && p->waves == s.waves &&
               p->split_k >= 1 && p->split_k <= kMaxTileSplit &&
               (p->split_k == 1 || tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched) ||
                (s.sched == 6 && p->split_k == 2)) &&
               (p->split_k == 1 || s.sched == 6 || p->M * p->N < ((int64_t)1 << 29)) && p->xcd_window_w >= 0 &&
               p->xcd_chunk_c >= 0 && p->K > 0 && p->K % 8 == 0 && p->K <= (INT32_MAX / 2) / 256 &&
               cdiv(p->M, s.bm) * cdiv(p->N, s.bn) <= INT32_MAX;
    }
    case HKG_KERNEL_SKINNY: {
        if (p->variant < 0 || p->variant >= SKINNY_NUM_VARIANTS)
            return false;
        const SkinnyShape s = skinny_shape(p->variant);
        return p->M <= 16 * s.mblocks && p->tile_n == 16 * s.nblocks && p->split_k >= 1 && p->split_k <= 64 &&
               p->K > 0 && p->K % 8 == 0 && p->K <= (INT32_MAX / 2) / 256;
    }
    default:
        return false;
    }
}

// Split-K scratch of a split plan: from the caller's fixed buffers when
// `fixed` is given (the no-allocation entry point), else the stream's
// library workspace.
hkg_status_t split_scratch(int dev, hipStream_t stream, const FixedScratch* fixed, size_t ws_bytes, size_t counters,
                           float** ws, int** cnt)
{
    if (!fixed)
        return get_workspace(dev, stream, ws_bytes, counters, ws, cnt);
    if (ws_bytes > fixed->ws_bytes || counters > fixed->counters) {
        char buf[256];
        std::snprintf(buf, sizeof buf,
                      "split-K scratch of %zu bytes and %zu counters exceeds the fixed %zu bytes and %zu counters",
                      ws_bytes, counters, fixed->ws_bytes, fixed->counters);
        g_last_hip_error = buf;
        return HKG_ERR_WORKSPACE;
    }
    *ws = fixed->ws;
    *cnt = fixed->counter_base;
    return HKG_OK;
}

// Leading dimensions: A rows lda apart, B rows ldb apart, C rows ldc apart
// (elements); the dense calls pass K, K, N.
hkg_status_t run(const hkg_plan_t* p, const void* A, const void* B, void* C, const uint16_t* bias, int epi,
                 hipStream_t stream, int64_t lda, int64_t ldb, int64_t ldc, const FixedScratch* fixed = nullptr)
{
    const int64_t M = p->M, N = p->N, K = p->K;
    if (p->kernel_id == HKG_KERNEL_NONE)
        return HKG_OK;
    int dev = 0;
    hkg_status_t st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    const uint16_t* a = (const uint16_t*)A;
    const uint16_t* b = (const uint16_t*)B;
    uint16_t* c = (uint16_t*)C;
    hipError_t e = hipSuccess;
    switch (p->kernel_id) {
    case HKG_KERNEL_ZERO:
        e = launch_zero(c, ldc, M, N, bias, epi, stream);
        break;
    case HKG_KERNEL_GENERIC:
        e = launch_generic(a, lda, 0, b, ldb, 0, c, ldc, M, N, K, bias, epi, stream);
        break;
    case HKG_KERNEL_TILE: {
        float* ws = nullptr;
        int* counters = nullptr;
        if (tile_shape(p->variant).sched == 6 && p->split_k == 2) {
            // The persistent tile with its last round split in two halves of
            // K runs as the grouped kernel with one expert (a null offset
            // list), whose streamed schedule splits such a round.  That
            // kernel reads dense operands and takes one fp32 partial tile per
            // workgroup; with strided operands, a caller's fixed scratch, or
            // a capture during which the workspace would have to grow, the
            // plain persistent kernel runs every tile whole instead.
            bool split = lda == K && ldb == K && ldc == N && !fixed;
            if (split) {
                hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
                e = hipStreamIsCapturing(stream, &cs);
                if (e != hipSuccess) {
                    set_hip_error(e, "hipStreamIsCapturing");
                    return HKG_ERR_HIP;
                }
                const std::string before = g_last_hip_error;
                st = get_workspace(dev, stream, (size_t)p->workspace_bytes, (size_t)p->grid_x, &ws, &counters);
                if (st == HKG_ERR_WORKSPACE && cs != hipStreamCaptureStatusNone) {
                    split = false;
                    g_last_hip_error = before;
                } else if (st != HKG_OK) {
                    return st;
                }
            }
            if (split)
                e = launch_grouped(kGroupedPingPong, a, b, nullptr, 1, c, (int)M, (int)N, (int)K, p->grid_x, 1, 2, ws,
                                   counters, bias, epi, stream);
            else
                e = launch_tile(p->variant, a, b, c, (int)M, (int)N, (int)K, p->xcd_window_w, p->xcd_chunk_c, 1,
                                nullptr, nullptr, bias, epi, (int)lda, (int)ldb, (int)ldc, stream);
            break;
        }
        if (p->split_k > 1) {
            st = split_scratch(dev, stream, fixed, (size_t)p->split_k * (size_t)M * (size_t)N * sizeof(float),
                               (size_t)(cdiv(M, p->tile_m) * cdiv(N, p->tile_n)), &ws, &counters);
            if (st != HKG_OK)
                return st;
        }
        e = launch_tile(p->variant, a, b, c, (int)M, (int)N, (int)K, p->xcd_window_w, p->xcd_chunk_c,
                        p->split_k, ws, counters, bias, epi, (int)lda, (int)ldb, (int)ldc, stream);
        break;
    }
    case HKG_KERNEL_SKINNY: {
        float* ws = nullptr;
        int* counters = nullptr;
        if (p->split_k > 1) {
            st = split_scratch(dev, stream, fixed, (size_t)p->split_k * (size_t)M * (size_t)N * sizeof(float),
                               (size_t)cdiv(N, 16), &ws, &counters);
            if (st != HKG_OK)
                return st;
        }
        e = launch_skinny(p->variant, a, b, c, (int)M, (int)N, (int)K, p->split_k, ws, counters, bias, epi,
                          (int)lda, (int)ldb, (int)ldc, stream);
        break;
    }
    default:
        return HKG_ERR_UNSUPPORTED;
    }
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return HKG_OK;
}

// Every library-owned buffer is released when the library is unloaded.
struct Cleanup {
    ~Cleanup()
    {
        for (auto& d : g_devices) {
            for (auto& kv : d.per_stream) {
                Workspace& w = kv.second;
                for (void* p : {(void*)w.ws, (void*)w.counters, (void*)w.mx_ws, (void*)w.layout_ws})
                    if (p)
                        (void)hipFree(p);
            }
            d.per_stream.clear();
            for (void* p : d.retired)
                (void)hipFree(p);
            d.retired.clear();
        }
    }
} g_cleanup;

// Epilogue arguments: a known code, and for every code but NONE a bias of N
// bf16 values that is 2-byte aligned and does not overlap C.
hkg_status_t check_epilogue(const void* bias, const void* C, int64_t M, int64_t N, int32_t epi)
{
    if (epi < HKG_EPILOGUE_NONE || epi > HKG_EPILOGUE_BIAS_GELU)
        return HKG_ERR_INVALID_ARG;
    if (epi == HKG_EPILOGUE_NONE || M == 0 || N == 0)
        return HKG_OK;
    if (!bias)
        return HKG_ERR_INVALID_ARG;
    if (overlaps(C, 2 * M * N, bias, 2 * N))
        return HKG_ERR_INVALID_ARG;
    if (((uintptr_t)bias & 1u) != 0)
        return HKG_ERR_MISALIGNED;
    return HKG_OK;
}

hkg_status_t gemm(const void* A, const void* B, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                  int32_t epi, void* stream, const FixedScratch* fixed = nullptr)
{
    hkg_plan_t p;
    hkg_status_t st = make_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    st = check_pointers(A, B, C, M, N, K);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if ((p.kernel_id == HKG_KERNEL_TILE || p.kernel_id == HKG_KERNEL_SKINNY) &&
        !(aligned16(A) && aligned16(B) && aligned16(C)))
        plan_generic(M, N, &p, "pointers not 16-byte aligned");
    return run(&p, A, B, C, (const uint16_t*)bias, epi, (hipStream_t)stream, K, K, N, fixed);
}

hkg_status_t run_plan(const hkg_plan_t* plan, const void* A, const void* B, const void* bias, void* C,
                      int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    if (!plan || plan->abi_version != HKG_ABI_VERSION)
        return HKG_ERR_INVALID_ARG;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (plan->M != M || plan->N != N || plan->K != K)
        return HKG_ERR_INVALID_ARG;
    st = check_pointers(A, B, C, M, N, K);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (!plan_matches_library(plan))
        return HKG_ERR_UNSUPPORTED;
    if ((plan->kernel_id == HKG_KERNEL_TILE || plan->kernel_id == HKG_KERNEL_SKINNY) &&
        !(aligned16(A) && aligned16(B) && aligned16(C)))
        return HKG_ERR_MISALIGNED;
    return run(plan, A, B, C, (const uint16_t*)bias, epi, (hipStream_t)stream, K, K, N);
}

// ------------------------------------------------------------------- MXFP8
// Block-scaled FP8 GEMM (FlyDSL-in-PyTorch blog, MXFP section): E4M3
// operands, one E8M0 scale per 32 k, K % 128 == 0 (the scaled MFMA's k).

// Largest K whose 256-row tile still spans fewer than 2^31 bytes.
constexpr int64_t kMxMaxK = (int64_t)(INT32_MAX / 256) / 128 * 128;

bool mx_shape_supported(int64_t M, int64_t N, int64_t K)
{
    return K <= kMxMaxK && mx_packed_scale_bytes(M, K) <= INT32_MAX && mx_packed_scale_bytes(N, K) <= INT32_MAX;
}

void fill_mx_tile(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N)
{
    const TileShape s = mx_tile_shape(variant);
    const int64_t tm = cdiv(M, s.bm), tn = cdiv(N, s.bn);
    p->kernel_id = HKG_KERNEL_MX_TILE;
    p->variant = variant;
    p->tile_m = s.bm;
    p->tile_n = s.bn;
    p->tile_k = s.bk;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    p->grid_x = (int32_t)(tm * tn);
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    p->xcd_window_w = tm >= 8 ? 8 : (int32_t)tm;
    p->xcd_chunk_c = (tm * tn >= 8 * 32) ? 32 : 0;
    p->lds_bytes = mx_tile_lds_bytes(variant);
    fill_resources(p, mx_tile_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "mxtile_%dx%dx%d_s%d_w%dx%d_p%d", s.bm, s.bn, s.bk,
                  s.stages, s.wm, s.wn, s.sched);
    std::snprintf(p->reason, sizeof p->reason, "MXFP8: %lldx%lld tiles of %dx%d, split-K %lld", (long long)tm,
                  (long long)tn, s.bm, s.bn, (long long)split);
}

void fill_mx_skinny(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N)
{
    const SkinnyShape s = mx_skinny_shape(variant);
    const int64_t col_blocks = cdiv(N, 16 * s.nblocks);
    p->kernel_id = HKG_KERNEL_MX_SKINNY;
    p->variant = variant;
    p->tile_m = 16 * s.mblocks;
    p->tile_n = 16 * s.nblocks;
    p->tile_k = 128;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    p->grid_x = (int32_t)col_blocks;
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->xcd_window_w = 0;
    p->xcd_chunk_c = 0;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    p->lds_bytes = mx_skinny_lds_bytes(variant);
    fill_resources(p, mx_skinny_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "mxskinny_m%d_n%d_w%d_u%d_c%d%s", 16 * s.mblocks,
                  16 * s.nblocks, s.waves, s.unroll, s.cache_policy, s.a_lds ? "_lds" : "");
    std::snprintf(p->reason, sizeof p->reason, "MXFP8, M <= %d: %lld column blocks of %d, split-K %lld",
                  16 * s.mblocks, (long long)col_blocks, 16 * s.nblocks, (long long)split);
}

hkg_status_t make_mx_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    std::memset(p, 0, sizeof *p);
    p->abi_version = HKG_ABI_VERSION;
    p->M = M;
    p->N = N;
    p->K = K;
    p->split_k = 1;
    p->vgprs = p->agprs = p->sgprs = p->scratch_bytes = -1;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (K % 128 != 0)
        return HKG_ERR_INVALID_ARG;
    p->flops = 2.0 * (double)M * (double)N * (double)K;
    p->algorithmic_bytes = (double)M * K + (double)N * K + ((double)M + (double)N) * (double)(K / 32) +
                           2.0 * (double)M * (double)N;
    if (M == 0 || N == 0) {
        p->kernel_id = HKG_KERNEL_NONE;
        copy_str(p->kernel_name, sizeof p->kernel_name, "none");
        copy_str(p->reason, sizeof p->reason, "empty output");
        return HKG_OK;
    }
    if (K == 0) {
        p->kernel_id = HKG_KERNEL_ZERO;
        p->grid_x = 1;
        p->block_x = 256;
        copy_str(p->kernel_name, sizeof p->kernel_name, "zero");
        copy_str(p->reason, sizeof p->reason, "K == 0: C is the empty sum, +0");
        return HKG_OK;
    }
    if (!mx_shape_supported(M, N, K))
        return HKG_ERR_UNSUPPORTED;
    // Decode shapes: the skinny kernel streams B once (smallest A cover that
    // holds M; A through LDS when M fills more than half of it), split
    // across workgroups only when the column blocks leave compute units
    // idle, keeping at least 2 steps of 128 k per wave.
    int mx_variant = -1, mx_best = 1 << 30;
    for (int v = 0; v < MX_SKINNY_NUM_VARIANTS; ++v) {
        const SkinnyShape ss = mx_skinny_shape(v);
        const int rank = 2 * ss.mblocks + (ss.a_lds != (M > 8 * (int64_t)ss.mblocks ? 1 : 0));
        if (M <= 16 * (int64_t)ss.mblocks && rank < mx_best) {
            mx_variant = v;
            mx_best = rank;
        }
    }
    if (mx_variant >= 0) {
        const int v = mx_variant;
        const SkinnyShape ss = mx_skinny_shape(v);
        const int64_t col_blocks = cdiv(N, 16 * ss.nblocks);
        int64_t split = 1;
        if (col_blocks < kNumCUs) {
            split = std::min<int64_t>(cdiv(kNumCUs, col_blocks), (K / 128) / (2 * ss.waves));
            split = std::max<int64_t>(1, std::min<int64_t>(split, 64));
        }
        fill_mx_skinny(p, v, split, M, N);
        return HKG_OK;
    }
    // 256 x 256 ping-pong when its tiles fill the device; otherwise the
    // 128 x 128 tile, with split-K (at least 4 stages of 128 k per split)
    // while the grid is under one workgroup per compute unit.
    const TileShape big = mx_tile_shape(0);
    int variant = cdiv(M, big.bm) * cdiv(N, big.bn) >= kNumCUs ? 0 : 1;
    const TileShape s = mx_tile_shape(variant);
    const int64_t tiles = cdiv(M, s.bm) * cdiv(N, s.bn);
    if (tiles > INT32_MAX)
        return HKG_ERR_UNSUPPORTED;
    int64_t split = 1;
    if (tiles < kNumCUs && M * N < ((int64_t)1 << 29) && tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched)) {
        split = std::min<int64_t>(cdiv(kNumCUs, tiles), (K / 128) / 4);
        split = std::max<int64_t>(1, std::min<int64_t>(split, kMaxTileSplit));
    }
    fill_mx_tile(p, variant, split, M, N);
    return HKG_OK;
}

bool mx_plan_matches_library(const hkg_plan_t* p)
{
    switch (p->kernel_id) {
    case HKG_KERNEL_NONE:
        return p->M == 0 || p->N == 0;
    case HKG_KERNEL_ZERO:
        return p->K == 0 && p->M > 0 && p->N > 0;
    case HKG_KERNEL_MX_SKINNY: {
        if (p->variant < 0 || p->variant >= MX_SKINNY_NUM_VARIANTS)
            return false;
        const SkinnyShape s = mx_skinny_shape(p->variant);
        return p->M <= 16 * s.mblocks && p->tile_n == 16 * s.nblocks && p->split_k >= 1 && p->split_k <= 64 &&
               (p->split_k == 1 || p->M * p->N < ((int64_t)1 << 29)) && p->K > 0 && p->K % 128 == 0 &&
               mx_shape_supported(p->M, p->N, p->K);
    }
    case HKG_KERNEL_MX_TILE: {
        if (p->variant < 0 || p->variant >= MX_TILE_NUM_VARIANTS)
            return false;
        const TileShape s = mx_tile_shape(p->variant);
        return p->tile_m == s.bm && p->tile_n == s.bn && p->tile_k == s.bk && p->waves == s.waves &&
               p->split_k >= 1 && p->split_k <= kMaxTileSplit &&
               (p->split_k == 1 || tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched)) &&
               (p->split_k == 1 || p->M * p->N < ((int64_t)1 << 29)) && p->xcd_window_w >= 0 &&
               p->xcd_chunk_c >= 0 && p->K > 0 && p->K % 128 == 0 && mx_shape_supported(p->M, p->N, p->K) &&
               cdiv(p->M, s.bm) * cdiv(p->N, s.bn) <= INT32_MAX;
    }
    default:
        return false;
    }
}

// Operand checks of the block-scaled entry points: data of M x K and N x K
// bytes (MXFP4: K / 2 bytes per row), scales of `sa_bytes` and `sb_bytes`, C
// of M x N bf16; C overlaps nothing.
hkg_status_t check_mx_pointers(const void* A, const void* SA, int64_t sa_bytes, const void* B, const void* SB,
                               int64_t sb_bytes, const void* C, int64_t M, int64_t N, int64_t K, bool fp4 = false)
{
    const int64_t row = fp4 ? K / 2 : K;
    const int64_t a_bytes = M * row, b_bytes = N * row, c_bytes = 2 * M * N;
    if ((a_bytes && !A) || (b_bytes && !B) || (c_bytes && !C) || (sa_bytes && !SA) || (sb_bytes && !SB))
        return HKG_ERR_INVALID_ARG;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes) || overlaps(C, c_bytes, SA, sa_bytes) ||
        overlaps(C, c_bytes, SB, sb_bytes))
        return HKG_ERR_INVALID_ARG;
    return HKG_OK;
}

// PA, PB: packed scales, or (natural, small-M kernel only) the natural
// scale arrays.
hkg_status_t run_mx(const hkg_plan_t* p, const void* A, const uint32_t* PA, const void* B, const uint32_t* PB,
                    void* C, const uint16_t* bias, int epi, hipStream_t stream, bool natural = false)
{
    const int64_t M = p->M, N = p->N, K = p->K;
    if (p->kernel_id == HKG_KERNEL_NONE)
        return HKG_OK;
    int dev = 0;
    hkg_status_t st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    hipError_t e = hipSuccess;
    if (p->kernel_id == HKG_KERNEL_ZERO) {
        e = launch_zero((uint16_t*)C, N, M, N, bias, epi, stream);
    } else {
        float* ws = nullptr;
        int* counters = nullptr;
        if (p->split_k > 1) {
            st = get_workspace(dev, stream, (size_t)p->split_k * (size_t)M * (size_t)N * sizeof(float),
                               (size_t)(cdiv(M, p->tile_m) * cdiv(N, p->tile_n)), &ws, &counters);
            if (st != HKG_OK)
                return st;
        }
        if (p->kernel_id == HKG_KERNEL_MX_SKINNY)
            e = launch_skinny_mx(p->variant, (const uint8_t*)A, (const uint8_t*)B, (uint16_t*)C, (int)M, (int)N,
                                 (int)K, p->split_k, ws, counters, bias, epi, PA, PB, natural, stream);
        else if (p->kernel_id == HKG_KERNEL_MX4_SKINNY)
            e = launch_skinny_mx4(p->variant, (const uint8_t*)A, (const uint8_t*)B, (uint16_t*)C, (int)M, (int)N,
                                  (int)K, p->split_k, ws, counters, bias, epi, PA, PB, stream);
        else if (p->kernel_id == HKG_KERNEL_MX4_TILE)
            e = launch_tile_mx4(p->variant, (const uint8_t*)A, (const uint8_t*)B, (uint16_t*)C, (int)M, (int)N,
                                (int)K, p->xcd_window_w, p->xcd_chunk_c, p->split_k, ws, counters, bias, epi, PA,
                                PB, stream);
        else
            e = launch_tile_mx(p->variant, (const uint8_t*)A, (const uint8_t*)B, (uint16_t*)C, (int)M, (int)N,
                               (int)K, p->xcd_window_w, p->xcd_chunk_c, p->split_k, ws, counters, bias, epi, PA, PB,
                               stream);
    }
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return HKG_OK;
}

bool mx_kernel(int id)
{
    return id == HKG_KERNEL_MX_TILE || id == HKG_KERNEL_MX_SKINNY || id == HKG_KERNEL_MX4_TILE ||
           id == HKG_KERNEL_MX4_SKINNY;
}

// The MXFP8 kernels read A, B with 16-byte accesses, store C in 8-byte
// groups and reads packed scales as dwords.
bool mx_aligned(const void* A, const void* PA, const void* B, const void* PB, const void* C)
{
    return aligned16(A) && aligned16(B) && aligned16(C) && ((uintptr_t)PA & 3u) == 0 && ((uintptr_t)PB & 3u) == 0;
}

hkg_status_t gemm_mx_prepacked(const void* A, const void* PA, const void* B, const void* PB, const void* bias,
                               void* C, int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    hkg_plan_t p;
    hkg_status_t st = make_mx_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    const int64_t pa = K ? mx_packed_scale_bytes(M, K) : 0, pb = K ? mx_packed_scale_bytes(N, K) : 0;
    st = check_mx_pointers(A, PA, pa, B, PB, pb, C, M, N, K);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (mx_kernel(p.kernel_id) && !mx_aligned(A, PA, B, PB, C))
        return HKG_ERR_MISALIGNED;
    return run_mx(&p, A, (const uint32_t*)PA, B, (const uint32_t*)PB, C, (const uint16_t*)bias, epi,
                  (hipStream_t)stream);
}

hkg_status_t gemm_mx(const void* A, const void* SA, const void* B, const void* SB, const void* bias, void* C,
                     int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    hkg_plan_t p;
    hkg_status_t st = make_mx_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    st = check_mx_pointers(A, SA, M * (K / 32), B, SB, N * (K / 32), C, M, N, K);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (!mx_kernel(p.kernel_id))
        return run_mx(&p, A, nullptr, B, nullptr, C, (const uint16_t*)bias, epi, (hipStream_t)stream);
    if (!(aligned16(A) && aligned16(B) && aligned16(C)))
        return HKG_ERR_MISALIGNED;
    // The small-M kernel reads natural scales itself (dword loads): no packing.
    if (p.kernel_id == HKG_KERNEL_MX_SKINNY && ((uintptr_t)SA & 3u) == 0 && ((uintptr_t)SB & 3u) == 0)
        return run_mx(&p, A, (const uint32_t*)SA, B, (const uint32_t*)SB, C, (const uint16_t*)bias, epi,
                      (hipStream_t)stream, true);
    int dev = 0;
    st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    const int64_t pa = mx_packed_scale_bytes(M, K), pb = mx_packed_scale_bytes(N, K);
    uint8_t* ws = nullptr;
    st = get_mx_workspace(dev, (hipStream_t)stream, (size_t)(pa + pb), &ws);
    if (st != HKG_OK)
        return st;
    hipError_t e = launch_mx_pack((const uint8_t*)SA, (uint32_t*)ws, M, K, (hipStream_t)stream);
    if (e == hipSuccess)
        e = launch_mx_pack((const uint8_t*)SB, (uint32_t*)(ws + pa), N, K, (hipStream_t)stream);
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return run_mx(&p, A, (const uint32_t*)ws, B, (const uint32_t*)(ws + pa), C, (const uint16_t*)bias, epi,
                  (hipStream_t)stream);
}

// ------------------------------------------------------------------- MXFP4
// Block-scaled FP4 GEMM (the same MXFP section): E2M1 operands two per byte,
// one E8M0 scale per 32 k, K % 128 == 0; the tile kernel's MXFP4
// instantiations, scales packed as for MXFP8.

// Largest K whose 256-row tile (K / 2 bytes per row) spans fewer than 2^31
// bytes.
constexpr int64_t kMx4MaxK = (int64_t)(INT32_MAX / 256) * 2 / 128 * 128;

bool mx4_shape_supported(int64_t M, int64_t N, int64_t K)
{
    return K <= kMx4MaxK && mx_packed_scale_bytes(M, K) <= INT32_MAX && mx_packed_scale_bytes(N, K) <= INT32_MAX;
}

void fill_mx4_tile(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N)
{
    const TileShape s = mx4_tile_shape(variant);
    const int64_t tm = cdiv(M, s.bm), tn = cdiv(N, s.bn);
    p->kernel_id = HKG_KERNEL_MX4_TILE;
    p->variant = variant;
    p->tile_m = s.bm;
    p->tile_n = s.bn;
    p->tile_k = s.bk;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    p->grid_x = (int32_t)(tm * tn);
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    p->xcd_window_w = tm >= 8 ? 8 : (int32_t)tm;
    p->xcd_chunk_c = (tm * tn >= 8 * 32) ? 32 : 0;
    p->lds_bytes = mx4_tile_lds_bytes(variant);
    fill_resources(p, mx4_tile_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "mx4tile_%dx%dx%d_s%d_w%dx%d_p%d", s.bm, s.bn, s.bk,
                  s.stages, s.wm, s.wn, s.sched);
    std::snprintf(p->reason, sizeof p->reason, "MXFP4: %lldx%lld tiles of %dx%d, split-K %lld", (long long)tm,
                  (long long)tn, s.bm, s.bn, (long long)split);
}

void fill_mx4_skinny(hkg_plan_t* p, int variant, int64_t split, int64_t M, int64_t N)
{
    const SkinnyShape s = mx4_skinny_shape(variant);
    const int64_t col_blocks = cdiv(N, 16 * s.nblocks);
    p->kernel_id = HKG_KERNEL_MX4_SKINNY;
    p->variant = variant;
    p->tile_m = 16 * s.mblocks;
    p->tile_n = 16 * s.nblocks;
    p->tile_k = 256;
    p->waves = s.waves;
    p->split_k = (int32_t)split;
    p->grid_x = (int32_t)col_blocks;
    p->grid_y = (int32_t)split;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->xcd_window_w = 0;
    p->xcd_chunk_c = 0;
    p->workspace_bytes = split > 1 ? (int64_t)(split * M * N * 4) : 0;
    p->lds_bytes = mx4_skinny_lds_bytes(variant);
    fill_resources(p, mx4_skinny_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "mx4skinny_m%d_n%d_w%d_u%d_c%d%s", 16 * s.mblocks,
                  16 * s.nblocks, s.waves, s.unroll, s.cache_policy, s.a_lds ? "_lds" : "");
    std::snprintf(p->reason, sizeof p->reason, "MXFP4, M <= %d: %lld column blocks of %d, split-K %lld",
                  16 * s.mblocks, (long long)col_blocks, 16 * s.nblocks, (long long)split);
}

hkg_status_t make_mx4_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    std::memset(p, 0, sizeof *p);
    p->abi_version = HKG_ABI_VERSION;
    p->M = M;
    p->N = N;
    p->K = K;
    p->split_k = 1;
    p->vgprs = p->agprs = p->sgprs = p->scratch_bytes = -1;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (K % 128 != 0)
        return HKG_ERR_INVALID_ARG;
    p->flops = 2.0 * (double)M * (double)N * (double)K;
    p->algorithmic_bytes = ((double)M + (double)N) * (double)(K / 2) + ((double)M + (double)N) * (double)(K / 32) +
                           2.0 * (double)M * (double)N;
    if (M == 0 || N == 0) {
        p->kernel_id = HKG_KERNEL_NONE;
        copy_str(p->kernel_name, sizeof p->kernel_name, "none");
        copy_str(p->reason, sizeof p->reason, "empty output");
        return HKG_OK;
    }
    if (K == 0) {
        p->kernel_id = HKG_KERNEL_ZERO;
        p->grid_x = 1;
        p->block_x = 256;
        copy_str(p->kernel_name, sizeof p->kernel_name, "zero");
        copy_str(p->reason, sizeof p->reason, "K == 0: C is the empty sum, +0");
        return HKG_OK;
    }
    if (!mx4_shape_supported(M, N, K))
        return HKG_ERR_UNSUPPORTED;
    // Decode shapes: the small-M kernel streams B once.  Each workgroup
    // reads all of A, so the widest column block whose workgroups still
    // cover 7/8 of the compute units wins (32 x 14336 x 4096: 64 columns on
    // 224 workgroups 11.5 us, 32 columns on 448 13.4, 16 on 896 15.7; at
    // N = 8192 32 columns 12.6 vs 64 on 128 workgroups 17.2); among equal
    // widths the smaller A cover; where no width fills, the narrowest, split
    // across workgroups (at least one step of 256 k per wave).
    int mx4_variant = -1;
    bool mx4_fills = false;
    for (int v = 0; v < MX4_SKINNY_NUM_VARIANTS; ++v) {
        const SkinnyShape ss = mx4_skinny_shape(v);
        if (M > 16 * (int64_t)ss.mblocks)
            continue;
        const bool fills = cdiv(N, 16 * ss.nblocks) * 8 >= 7 * (int64_t)kNumCUs;
        if (mx4_variant < 0) {
            mx4_variant = v;
            mx4_fills = fills;
            continue;
        }
        const SkinnyShape cur = mx4_skinny_shape(mx4_variant);
        bool better;
        if (fills != mx4_fills)
            better = fills;
        else if (ss.nblocks != cur.nblocks)
            better = fills ? ss.nblocks > cur.nblocks : ss.nblocks < cur.nblocks;
        else
            better = ss.mblocks < cur.mblocks;
        if (better) {
            mx4_variant = v;
            mx4_fills = fills;
        }
    }
    if (mx4_variant >= 0) {
        const SkinnyShape ss = mx4_skinny_shape(mx4_variant);
        const int64_t col_blocks = cdiv(N, 16 * ss.nblocks);
        int64_t split = 1;
        if (!mx4_fills) {
            split = std::min<int64_t>(cdiv(kNumCUs, col_blocks), (K / 256) / ss.waves);
            split = std::max<int64_t>(1, std::min<int64_t>(split, 64));
        }
        fill_mx4_skinny(p, mx4_variant, split, M, N);
        return HKG_OK;
    }
    // 256 x 256 ping-pong when its tiles fill the device; otherwise the
    // 128 x 128 tile, with split-K (at least 2 stages of 256 k per split)
    // while the grid is under one workgroup per compute unit.
    const TileShape big = mx4_tile_shape(0);
    const int variant = cdiv(M, big.bm) * cdiv(N, big.bn) >= kNumCUs ? 0 : 1;
    const TileShape s = mx4_tile_shape(variant);
    const int64_t tiles = cdiv(M, s.bm) * cdiv(N, s.bn);
    if (tiles > INT32_MAX)
        return HKG_ERR_UNSUPPORTED;
    int64_t split = 1;
    if (tiles < kNumCUs && M * N < ((int64_t)1 << 29) && tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched)) {
        split = std::min<int64_t>(cdiv(kNumCUs, tiles), (K / 256) / 2);
        split = std::max<int64_t>(1, std::min<int64_t>(split, kMaxTileSplit));
    }
    fill_mx4_tile(p, variant, split, M, N);
    return HKG_OK;
}

bool mx4_plan_matches_library(const hkg_plan_t* p)
{
    switch (p->kernel_id) {
    case HKG_KERNEL_NONE:
        return p->M == 0 || p->N == 0;
    case HKG_KERNEL_ZERO:
        return p->K == 0 && p->M > 0 && p->N > 0;
    case HKG_KERNEL_MX4_SKINNY: {
        if (p->variant < 0 || p->variant >= MX4_SKINNY_NUM_VARIANTS)
            return false;
        const SkinnyShape s = mx4_skinny_shape(p->variant);
        return p->M <= 16 * s.mblocks && p->tile_n == 16 * s.nblocks && p->split_k >= 1 && p->split_k <= 64 &&
               (p->split_k == 1 || p->M * p->N < ((int64_t)1 << 29)) && p->K > 0 && p->K % 128 == 0 &&
               mx4_shape_supported(p->M, p->N, p->K);
    }
    case HKG_KERNEL_MX4_TILE: {
        if (p->variant < 0 || p->variant >= MX4_TILE_NUM_VARIANTS)
            return false;
        const TileShape s = mx4_tile_shape(p->variant);
        return p->tile_m == s.bm && p->tile_n == s.bn && p->tile_k == s.bk && p->waves == s.waves &&
               p->split_k >= 1 && p->split_k <= kMaxTileSplit &&
               (p->split_k == 1 || tile_split_capable(s.bm, s.bn, s.wm, s.wn, s.sched)) &&
               (p->split_k == 1 || p->M * p->N < ((int64_t)1 << 29)) && p->xcd_window_w >= 0 &&
               p->xcd_chunk_c >= 0 && p->K > 0 && p->K % 128 == 0 && mx4_shape_supported(p->M, p->N, p->K) &&
               cdiv(p->M, s.bm) * cdiv(p->N, s.bn) <= INT32_MAX;
    }
    default:
        return false;
    }
}

hkg_status_t gemm_mx4_prepacked(const void* A, const void* PA, const void* B, const void* PB, const void* bias,
                                void* C, int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    hkg_plan_t p;
    hkg_status_t st = make_mx4_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    const int64_t pa = K ? mx_packed_scale_bytes(M, K) : 0, pb = K ? mx_packed_scale_bytes(N, K) : 0;
    st = check_mx_pointers(A, PA, pa, B, PB, pb, C, M, N, K, true);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (mx_kernel(p.kernel_id) && !mx_aligned(A, PA, B, PB, C))
        return HKG_ERR_MISALIGNED;
    return run_mx(&p, A, (const uint32_t*)PA, B, (const uint32_t*)PB, C, (const uint16_t*)bias, epi,
                  (hipStream_t)stream);
}

hkg_status_t gemm_mx4(const void* A, const void* SA, const void* B, const void* SB, const void* bias, void* C,
                      int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    hkg_plan_t p;
    hkg_status_t st = make_mx4_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    st = check_mx_pointers(A, SA, M * (K / 32), B, SB, N * (K / 32), C, M, N, K, true);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (!mx_kernel(p.kernel_id))
        return run_mx(&p, A, nullptr, B, nullptr, C, (const uint16_t*)bias, epi, (hipStream_t)stream);
    if (!(aligned16(A) && aligned16(B) && aligned16(C)))
        return HKG_ERR_MISALIGNED;
    int dev = 0;
    st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    const int64_t pa = mx_packed_scale_bytes(M, K), pb = mx_packed_scale_bytes(N, K);
    uint8_t* ws = nullptr;
    st = get_mx_workspace(dev, (hipStream_t)stream, (size_t)(pa + pb), &ws);
    if (st != HKG_OK)
        return st;
    hipError_t e = launch_mx_pack((const uint8_t*)SA, (uint32_t*)ws, M, K, (hipStream_t)stream);
    if (e == hipSuccess)
        e = launch_mx_pack((const uint8_t*)SB, (uint32_t*)(ws + pa), N, K, (hipStream_t)stream);
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return run_mx(&p, A, (const uint32_t*)ws, B, (const uint32_t*)(ws + pa), C, (const uint16_t*)bias, epi,
                  (hipStream_t)stream);
}

// ------------------------------------------------- layouts and strides
// All four operand layouts (FlyDSL-in-PyTorch blog, "Dense GEMM") and leading
// dimensions.  Row layout: a(i,k) = A[i lda + k]; column layout: a(i,k) =
// A[k lda + i] (B likewise with j, ldb); C[i ldc + j].

// Bytes spanned by an operand of `rows` logical rows in a layout.
int64_t operand_extent(int64_t rows, int64_t K, int64_t ld, int col)
{
    if (rows == 0 || K == 0)
        return 0;
    return 2 * (col ? (K - 1) * ld + rows : (rows - 1) * ld + K);
}

// Largest leading dimension whose 256-row tile stays within 32-bit offsets.
constexpr int64_t kMaxLd = (int64_t)(INT32_MAX / 2) / 256;

hkg_status_t gemm_ex(const void* A, int64_t lda, int32_t a_layout, const void* B, int64_t ldb, int32_t b_layout,
                     const void* bias, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K, int32_t epi,
                     void* stream_v)
{
    hipStream_t stream = (hipStream_t)stream_v;
    hkg_plan_t p;
    hkg_status_t st = make_plan(M, N, K, &p);
    if (st != HKG_OK)
        return st;
    if ((a_layout != HKG_LAYOUT_ROW && a_layout != HKG_LAYOUT_COL) ||
        (b_layout != HKG_LAYOUT_ROW && b_layout != HKG_LAYOUT_COL))
        return HKG_ERR_INVALID_ARG;
    const int a_col = a_layout == HKG_LAYOUT_COL, b_col = b_layout == HKG_LAYOUT_COL;
    // leading dimensions at least the contiguous extent (1 for empty operands)
    if (lda < std::max<int64_t>(1, a_col ? M : K) || ldb < std::max<int64_t>(1, b_col ? N : K) ||
        ldc < std::max<int64_t>(1, N) || lda > kMaxDim || ldb > kMaxDim || ldc > kMaxDim)
        return HKG_ERR_INVALID_ARG;
    const int64_t a_bytes = operand_extent(M, K, lda, a_col), b_bytes = operand_extent(N, K, ldb, b_col);
    const int64_t c_bytes = (M && N) ? 2 * ((M - 1) * ldc + N) : 0;
    if ((a_bytes && !A) || (b_bytes && !B) || (c_bytes && !C))
        return HKG_ERR_INVALID_ARG;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes))
        return HKG_ERR_INVALID_ARG;
    st = check_epilogue(bias, C, M, N, epi);
    if (st != HKG_OK)
        return st;
    if (p.kernel_id == HKG_KERNEL_NONE)
        return HKG_OK;
    if (p.kernel_id == HKG_KERNEL_ZERO)
        return run(&p, A, B, C, (const uint16_t*)bias, epi, stream, lda, ldb, ldc);
    // Fast kernels read K-contiguous rows with 16-byte accesses: 16-byte
    // aligned pointers and leading dimensions, K % 8 == 0 (the plan's own
    // condition).  Otherwise the general kernel reads any layout directly.
    const bool fast = p.kernel_id != HKG_KERNEL_GENERIC && aligned16(A) && aligned16(B) && aligned16(C) &&
                      lda % 8 == 0 && ldb % 8 == 0 && lda <= kMaxLd && ldb <= kMaxLd;
    if (!fast) {
        int dev = 0;
        st = current_device(&dev);
        if (st != HKG_OK)
            return st;
        hipError_t e = launch_generic((const uint16_t*)A, lda, a_col, (const uint16_t*)B, ldb, b_col, (uint16_t*)C,
                                      ldc, M, N, K, (const uint16_t*)bias, epi, stream);
        if (e != hipSuccess) {
            set_hip_error(e, "kernel launch");
            return HKG_ERR_HIP;
        }
        return HKG_OK;
    }
    // Column-layout operands are first transposed into a library buffer
    // (row layout, leading dimension K), then the row-layout kernels run.
    if (a_col || b_col) {
        int dev = 0;
        st = current_device(&dev);
        if (st != HKG_OK)
            return st;
        const size_t a_ws = a_col ? (size_t)M * (size_t)K : 0, b_ws = b_col ? (size_t)N * (size_t)K : 0;
        uint16_t* ws = nullptr;
        st = get_layout_workspace(dev, stream, (a_ws + b_ws) * sizeof(uint16_t), &ws);
        if (st != HKG_OK)
            return st;
        hipError_t e = hipSuccess;
        if (a_col) {
            e = launch_transpose((const uint16_t*)A, lda, ws, K, M, K, stream);
            A = ws;
            lda = K;
        }
        if (e == hipSuccess && b_col) {
            e = launch_transpose((const uint16_t*)B, ldb, ws + a_ws, K, N, K, stream);
            B = ws + a_ws;
            ldb = K;
        }
        if (e != hipSuccess) {
            set_hip_error(e, "kernel launch");
            return HKG_ERR_HIP;
        }
    }
    return run(&p, A, B, C, (const uint16_t*)bias, epi, stream, lda, ldb, ldc);
}

// ------------------------------------------------------------ grouped GEMM
// Mixture-of-experts GEMM (FlyDSL-in-PyTorch blog, grouped GEMM section) on a
// persistent grid: expert g owns rows [offs[g-1], offs[g]) of A and C.

// Partial tiles of the grouped kernel's split last round: one per workgroup.
size_t grouped_workspace_bytes(const hkg_plan_t* p)
{
    return p->split_k == 2 ? (size_t)p->grid_x * (size_t)p->tile_m * (size_t)p->tile_n * sizeof(float) : 0;
}

void fill_grouped(hkg_plan_t* p, int variant, int64_t G, int64_t M, int64_t N, int64_t K)
{
    const TileShape s = grouped_shape(variant);
    const int64_t tn = cdiv(N, s.bn);
    // Workgroups resident at once: one per CU for the 128 KiB-LDS 256 x 256
    // tile, two for the 64 KiB 128 x 128 tile; never more than the tiles
    // the experts can have.
    const int64_t per_cu = s.bm >= 256 ? 1 : 2;
    const int64_t row_bytes = (int64_t)s.bk * 2;
    const int64_t bound = (cdiv(M, s.bm) + G) * tn;
    const int64_t grid = std::min<int64_t>(kNumCUs * per_cu, bound);
    p->kernel_id = HKG_KERNEL_GROUPED;
    p->variant = variant;
    p->tile_m = s.bm;
    p->tile_n = s.bn;
    p->tile_k = s.bk;
    p->waves = s.waves;
    // The tiles of a last round that fills at most half the grid are split
    // into two halves of K (decided on the device, where the offsets are);
    // the rounds before it run whole tiles.
    p->split_k = cdiv(K, s.bk) >= 2 ? 2 : 1;
    p->grid_x = (int32_t)std::max<int64_t>(grid, 1);
    p->grid_y = 1;
    p->grid_z = 1;
    p->block_x = s.waves * 64;
    p->workspace_bytes = (int64_t)grouped_workspace_bytes(p);
    p->xcd_window_w = 0;
    p->xcd_chunk_c = 1;                 // chiplet-contiguous walk when the grid is a multiple of 8
    // the ping-pong keeps A halves double- and B triple-buffered
    p->lds_bytes = (int32_t)(s.sched >= 5 ? 4 * (s.bm / 2) * row_bytes + 3 * s.bn * row_bytes
                                          : s.stages * (s.bm + s.bn) * row_bytes);
    fill_resources(p, grouped_resources(variant));
    std::snprintf(p->kernel_name, sizeof p->kernel_name, "grouped_%dx%dx%d_s%d_w%dx%d_p%d", s.bm, s.bn, s.bk,
                  s.stages, s.wm, s.wn, s.sched);
    std::snprintf(p->reason, sizeof p->reason,
                  "grouped: %lld experts, %d x %d tiles on a persistent grid of %lld%s", (long long)G, s.bm, s.bn,
                  (long long)grid, p->split_k == 2 ? ", a last round of at most half the grid split over K" : "");
}

hkg_status_t make_grouped_plan(int64_t G, int64_t M, int64_t N, int64_t K, hkg_plan_t* p)
{
    std::memset(p, 0, sizeof *p);
    p->abi_version = HKG_ABI_VERSION;
    p->M = M;
    p->N = N;
    p->K = K;
    p->split_k = 1;
    p->vgprs = p->agprs = p->sgprs = p->scratch_bytes = -1;
    if (G < 0 || G > kMaxDim)
        return HKG_ERR_INVALID_ARG;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (G && K >= ((int64_t)1 << 40) / G / std::max<int64_t>(N, 1))     // B holds G N K < 2^40 elements
        return HKG_ERR_INVALID_ARG;
    p->flops = 2.0 * (double)M * (double)N * (double)K;                  // at most: every row in an expert
    p->algorithmic_bytes = 2.0 * ((double)M * K + (double)G * N * K + (double)M * N);
    if (M == 0 || N == 0 || G == 0) {
        p->kernel_id = HKG_KERNEL_NONE;
        copy_str(p->kernel_name, sizeof p->kernel_name, "none");
        copy_str(p->reason, sizeof p->reason, "no rows in any expert");
        return HKG_OK;
    }
    if (K % 8 != 0 || K > (int64_t)(INT32_MAX / 2) / 256)
        return HKG_ERR_UNSUPPORTED;
    // The 256 x 256 ping-pong tile when the experts average at least 256
    // rows and those tiles fill the device; the 128 x 128 tile otherwise.
    // Measured on MI355X, ping-pong vs the 8-wave register-pipelined 256 x 256
    // tile: 8 experts x 4096 rows, N = 14336, K = 4096 1296 vs 1236 TFLOP/s;
    // 16 ragged experts, 8192 rows, N = K = 4096 960 vs 898; 8 x 1024 rows
    // 1236 vs 1237.  Its streamed form (each workgroup's tiles as one stream
    // of stages) against one tile at a time, same run: 1.5-3.6% faster on
    // every MoE shape measured (8 x 1024 rows 200.3 vs 205.1 us).
    const TileShape big = grouped_shape(kGroupedPingPong);
    const int variant =
        (M / G >= big.bm && cdiv(M, big.bm) * cdiv(N, big.bn) >= kNumCUs) ? kGroupedPingPong : kGroupedSmall;
    const TileShape s = grouped_shape(variant);
    if ((cdiv(M, s.bm) + G) * cdiv(N, s.bn) > INT32_MAX)
        return HKG_ERR_UNSUPPORTED;
    fill_grouped(p, variant, G, M, N, K);
    return HKG_OK;
}

bool grouped_plan_matches_library(const hkg_plan_t* p, int64_t G)
{
    if (p->kernel_id == HKG_KERNEL_NONE)
        return p->M == 0 || p->N == 0 || G == 0;
    if (p->kernel_id != HKG_KERNEL_GROUPED || p->variant < 0 || p->variant >= GROUPED_NUM_VARIANTS)
        return false;
    const TileShape s = grouped_shape(p->variant);
    return p->tile_m == s.bm && p->tile_n == s.bn && p->tile_k == s.bk && p->waves == s.waves &&
           (p->split_k == 1 || p->split_k == 2) &&
           p->grid_x >= 1 && p->xcd_chunk_c >= 0 && p->K % 8 == 0 && p->K <= (INT32_MAX / 2) / 256 &&
           (cdiv(p->M, s.bm) + G) * cdiv(p->N, s.bn) <= INT32_MAX;
}

hkg_status_t grouped(const hkg_plan_t* plan, const void* A, const void* B, const void* offs, const void* bias,
                     void* C, int64_t G, int64_t M, int64_t N, int64_t K, int32_t epi, void* stream)
{
    hkg_plan_t own;
    const hkg_plan_t* p = plan;
    if (!p) {
        hkg_status_t st = make_grouped_plan(G, M, N, K, &own);
        if (st != HKG_OK)
            return st;
        p = &own;
    } else {
        if (p->abi_version != HKG_ABI_VERSION || G < 0)
            return HKG_ERR_INVALID_ARG;
        hkg_status_t st = check_dims(M, N, K);
        if (st != HKG_OK)
            return st;
        if (p->M != M || p->N != N || p->K != K)
            return HKG_ERR_INVALID_ARG;
    }
    const int64_t a_bytes = 2 * M * K, b_bytes = 2 * G * N * K, c_bytes = 2 * M * N, o_bytes = 4 * G;
    if ((a_bytes && !A) || (b_bytes && !B) || (c_bytes && !C) || (o_bytes && !offs))
        return HKG_ERR_INVALID_ARG;
    if (overlaps(C, c_bytes, A, a_bytes) || overlaps(C, c_bytes, B, b_bytes) || overlaps(C, c_bytes, offs, o_bytes))
        return HKG_ERR_INVALID_ARG;
    // bias: G x N values when an epilogue is asked for
    if (epi < HKG_EPILOGUE_NONE || epi > HKG_EPILOGUE_BIAS_GELU)
        return HKG_ERR_INVALID_ARG;
    if (epi != HKG_EPILOGUE_NONE && M > 0 && N > 0 && G > 0) {
        if (!bias || overlaps(C, c_bytes, bias, 2 * G * N))
            return HKG_ERR_INVALID_ARG;
        if (((uintptr_t)bias & 1u) != 0)
            return HKG_ERR_MISALIGNED;
    }
    if (plan && !grouped_plan_matches_library(p, G))
        return HKG_ERR_UNSUPPORTED;
    if (p->kernel_id == HKG_KERNEL_NONE)
        return HKG_OK;
    if (!(aligned16(A) && aligned16(B) && aligned16(C)) || ((uintptr_t)offs & 3u) != 0)
        return HKG_ERR_MISALIGNED;
    int dev = 0;
    hkg_status_t st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    // split_k 2 permits splitting the last round; under stream capture with
    // a workspace too small for it (which may not grow then) the call runs
    // every tile whole instead, which needs no workspace.
    float* ws = nullptr;
    int* cnt = nullptr;
    int split = p->split_k;
    if (split == 2) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t ce = hipStreamIsCapturing((hipStream_t)stream, &cs);
        if (ce != hipSuccess) {
            set_hip_error(ce, "hipStreamIsCapturing");
            return HKG_ERR_HIP;
        }
        const std::string before = g_last_hip_error;
        st = get_workspace(dev, (hipStream_t)stream, grouped_workspace_bytes(p), (size_t)p->grid_x, &ws, &cnt);
        if (st == HKG_ERR_WORKSPACE && cs != hipStreamCaptureStatusNone) {
            split = 1;
            ws = nullptr;
            cnt = nullptr;
            g_last_hip_error = before;
        } else if (st != HKG_OK) {
            return st;
        }
    }
    hipError_t e = launch_grouped(p->variant, (const uint16_t*)A, (const uint16_t*)B, (const int*)offs, (int)G,
                                  (uint16_t*)C, (int)M, (int)N, (int)K, p->grid_x, p->xcd_chunk_c, split, ws, cnt,
                                  (const uint16_t*)bias, epi, (hipStream_t)stream);
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return HKG_OK;
}

}  // namespace

hkg_status_t gemm_fixed_scratch(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, void* stream,
                                const FixedScratch& scratch)
{
    return gemm(A, B, nullptr, C, M, N, K, HKG_EPILOGUE_NONE, stream, &scratch);
}

}  // namespace hkg

using namespace hkg;

extern "C" {

hkg_status_t hkg_gemm_bf16_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out)
{
    if (!out)
        return HKG_ERR_INVALID_ARG;
    return make_plan(M, N, K, out);
}

hkg_status_t hkg_gemm_bf16(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                           void* stream)
{
    return gemm(A, B, nullptr, C, M, N, K, HKG_EPILOGUE_NONE, stream);
}

hkg_status_t hkg_gemm_bf16_epilogue(const void* A, const void* B, const void* bias, void* C, int64_t M,
                                    int64_t N, int64_t K, int32_t epilogue, void* stream)
{
    return gemm(A, B, bias, C, M, N, K, epilogue, stream);
}

hkg_status_t hkg_gemm_bf16_run_plan(const hkg_plan_t* plan, const void* A, const void* B, void* C,
                                    int64_t M, int64_t N, int64_t K, void* stream)
{
    return run_plan(plan, A, B, nullptr, C, M, N, K, HKG_EPILOGUE_NONE, stream);
}

hkg_status_t hkg_gemm_bf16_run_plan_epilogue(const hkg_plan_t* plan, const void* A, const void* B,
                                             const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                             int32_t epilogue, void* stream)
{
    return run_plan(plan, A, B, bias, C, M, N, K, epilogue, stream);
}

hkg_status_t hkg_gemm_mxfp8_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out)
{
    if (!out)
        return HKG_ERR_INVALID_ARG;
    return make_mx_plan(M, N, K, out);
}

hkg_status_t hkg_gemm_mxfp8(const void* A, const void* SA, const void* B, const void* SB, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream)
{
    return gemm_mx(A, SA, B, SB, bias, C, M, N, K, epilogue, stream);
}

int64_t hkg_mx_packed_scales_bytes(int64_t rows, int64_t K)
{
    if (rows < 0 || K < 0 || K % 128 != 0 || check_dims(rows, 1, K) != HKG_OK)
        return -1;
    return mx_packed_scale_bytes(rows, K);
}

hkg_status_t hkg_mx_pack_scales(const void* S, void* P, int64_t rows, int64_t K, void* stream)
{
    const int64_t bytes = hkg_mx_packed_scales_bytes(rows, K);
    if (bytes < 0 || bytes > INT32_MAX)
        return HKG_ERR_INVALID_ARG;
    if (bytes == 0)
        return HKG_OK;
    if (!S || !P || overlaps(S, rows * (K / 32), P, bytes))
        return HKG_ERR_INVALID_ARG;
    if (((uintptr_t)P & 3u) != 0)
        return HKG_ERR_MISALIGNED;
    int dev = 0;
    hkg_status_t st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    hipError_t e = launch_mx_pack((const uint8_t*)S, (uint32_t*)P, rows, K, (hipStream_t)stream);
    if (e != hipSuccess) {
        set_hip_error(e, "kernel launch");
        return HKG_ERR_HIP;
    }
    return HKG_OK;
}

hkg_status_t hkg_gemm_mxfp8_prepacked(const void* A, const void* PA, const void* B, const void* PB,
                                      const void* bias, void* C, int64_t M, int64_t N, int64_t K, int32_t epilogue,
                                      void* stream)
{
    return gemm_mx_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue, stream);
}

hkg_status_t hkg_gemm_mxfp4_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out)
{
    if (!out)
        return HKG_ERR_INVALID_ARG;
    return make_mx4_plan(M, N, K, out);
}

hkg_status_t hkg_gemm_mxfp4(const void* A, const void* SA, const void* B, const void* SB, const void* bias, void* C,
                            int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream)
{
    return gemm_mx4(A, SA, B, SB, bias, C, M, N, K, epilogue, stream);
}

hkg_status_t hkg_gemm_mxfp4_prepacked(const void* A, const void* PA, const void* B, const void* PB,
                                      const void* bias, void* C, int64_t M, int64_t N, int64_t K, int32_t epilogue,
                                      void* stream)
{
    return gemm_mx4_prepacked(A, PA, B, PB, bias, C, M, N, K, epilogue, stream);
}

hkg_status_t hkg_gemm_mxfp8_run_plan(const hkg_plan_t* plan, const void* A, const void* PA, const void* B,
                                     const void* PB, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                     int32_t epilogue, void* stream)
{
    if (!plan || plan->abi_version != HKG_ABI_VERSION)
        return HKG_ERR_INVALID_ARG;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (plan->M != M || plan->N != N || plan->K != K || K % 128 != 0)
        return HKG_ERR_INVALID_ARG;
    const int64_t pa = K ? mx_packed_scale_bytes(M, K) : 0, pb = K ? mx_packed_scale_bytes(N, K) : 0;
    st = check_mx_pointers(A, PA, pa, B, PB, pb, C, M, N, K);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epilogue);
    if (st != HKG_OK)
        return st;
    if (!mx_plan_matches_library(plan))
        return HKG_ERR_UNSUPPORTED;
    if (mx_kernel(plan->kernel_id) && !mx_aligned(A, PA, B, PB, C))
        return HKG_ERR_MISALIGNED;
    return run_mx(plan, A, (const uint32_t*)PA, B, (const uint32_t*)PB, C, (const uint16_t*)bias, epilogue,
                  (hipStream_t)stream);
}

hkg_status_t hkg_gemm_mxfp4_run_plan(const hkg_plan_t* plan, const void* A, const void* PA, const void* B,
                                     const void* PB, const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                     int32_t epilogue, void* stream)
{
    if (!plan || plan->abi_version != HKG_ABI_VERSION)
        return HKG_ERR_INVALID_ARG;
    hkg_status_t st = check_dims(M, N, K);
    if (st != HKG_OK)
        return st;
    if (plan->M != M || plan->N != N || plan->K != K || K % 128 != 0)
        return HKG_ERR_INVALID_ARG;
    const int64_t pa = K ? mx_packed_scale_bytes(M, K) : 0, pb = K ? mx_packed_scale_bytes(N, K) : 0;
    st = check_mx_pointers(A, PA, pa, B, PB, pb, C, M, N, K, true);
    if (st != HKG_OK)
        return st;
    st = check_epilogue(bias, C, M, N, epilogue);
    if (st != HKG_OK)
        return st;
    if (!mx4_plan_matches_library(plan))
        return HKG_ERR_UNSUPPORTED;
    if (mx_kernel(plan->kernel_id) && !mx_aligned(A, PA, B, PB, C))
        return HKG_ERR_MISALIGNED;
    return run_mx(plan, A, (const uint32_t*)PA, B, (const uint32_t*)PB, C, (const uint16_t*)bias, epilogue,
                  (hipStream_t)stream);
}

hkg_status_t hkg_gemm_bf16_ex(const void* A, int64_t lda, int32_t a_layout, const void* B, int64_t ldb,
                              int32_t b_layout, const void* bias, void* C, int64_t ldc, int64_t M, int64_t N,
                              int64_t K, int32_t epilogue, void* stream)
{
    return gemm_ex(A, lda, a_layout, B, ldb, b_layout, bias, C, ldc, M, N, K, epilogue, stream);
}

hkg_status_t hkg_pack_bf16(const void* X, int64_t ldx, int32_t layout, void* Y, int64_t rows, int64_t K,
                           void* stream)
{
    if (rows < 0 || K < 0 || rows > kMaxDim || K > kMaxDim || (layout != HKG_LAYOUT_ROW && layout != HKG_LAYOUT_COL))
        return HKG_ERR_INVALID_ARG;
    if (rows == 0 || K == 0)
        return HKG_OK;
    const int col = layout == HKG_LAYOUT_COL;
    if (ldx < (col ? rows : K))
        return HKG_ERR_INVALID_ARG;
    const int64_t x_bytes = operand_extent(rows, K, ldx, col), y_bytes = 2 * rows * K;
    if (!X || !Y || overlaps(X, x_bytes, Y, y_bytes))
        return HKG_ERR_INVALID_ARG;
    int dev = 0;
    hkg_status_t st = current_device(&dev);
    if (st != HKG_OK)
        return st;
    hipError_t e;
    if (col)
        e = launch_transpose((const uint16_t*)X, ldx, (uint16_t*)Y, K, rows, K, (hipStream_t)stream);
    else
        e = hipMemcpy2DAsync(Y, (size_t)K * 2, X, (size_t)ldx * 2, (size_t)K * 2, (size_t)rows,
                             hipMemcpyDeviceToDevice, (hipStream_t)stream);
    if (e != hipSuccess) {
        set_hip_error(e, col ? "kernel launch" : "hipMemcpy2DAsync");
        return HKG_ERR_HIP;
    }
    return HKG_OK;
}

hkg_status_t hkg_grouped_gemm_bf16_plan(int64_t G, int64_t M, int64_t N, int64_t K, hkg_plan_t* out)
{
    if (!out)
        return HKG_ERR_INVALID_ARG;
    return make_grouped_plan(G, M, N, K, out);
}

hkg_status_t hkg_grouped_gemm_bf16(const void* A, const void* B, const void* offs, const void* bias, void* C,
                                   int64_t G, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream)
{
    return grouped(nullptr, A, B, offs, bias, C, G, M, N, K, epilogue, stream);
}

hkg_status_t hkg_grouped_gemm_bf16_run_plan(const hkg_plan_t* plan, const void* A, const void* B, const void* offs,
                                            const void* bias, void* C, int64_t G, int64_t M, int64_t N, int64_t K,
                                            int32_t epilogue, void* stream)
{
    if (!plan)
        return HKG_ERR_INVALID_ARG;
    return grouped(plan, A, B, offs, bias, C, G, M, N, K, epilogue, stream);
}

const char* hkg_status_string(hkg_status_t s)
{
    switch (s) {
    case HKG_OK: return "ok";
    case HKG_ERR_INVALID_ARG: return "invalid argument";
    case HKG_ERR_MISALIGNED: return "pointer or K alignment does not fit the plan's kernel";
    case HKG_ERR_UNSUPPORTED: return "plan not supported by this library";
    case HKG_ERR_NO_DEVICE: return "no HIP device";
    case HKG_ERR_ARCH: return "device is not gfx950 (MI355X)";
    case HKG_ERR_HIP: return "HIP runtime error";
    case HKG_ERR_WORKSPACE: return "workspace allocation failed";
    default: return "unknown status";
    }
}

const char* hkg_last_hip_error(void) { return g_last_hip_error.c_str(); }

int32_t hkg_abi_version(void) { return HKG_ABI_VERSION; }

// Test hook, not part of include/hkg.h: the tile kernel's workgroup -> tile
// order evaluated on the host (the same inline function the kernel uses).
int32_t hkg_internal_tile_order(int32_t b, int32_t tiles_m, int32_t tiles_n, int32_t win_w,
                                int32_t chunk_c, int32_t* tm, int32_t* tn)
{
    if (!tm || !tn || tiles_m <= 0 || tiles_n <= 0 || b < 0 || b >= tiles_m * tiles_n || win_w < 0 ||
        chunk_c < 0)
        return HKG_ERR_INVALID_ARG;
    int m = 0, n = 0;
    tile_order(b, tiles_m, tiles_n, win_w, chunk_c, m, n);
    *tm = m;
    *tn = n;
    return HKG_OK;
}

}  // extern "C"
