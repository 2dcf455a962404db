// hkg_gemm_bf16_noalloc: hkg_gemm_bf16 for callers that cannot allocate
// device memory (code under stream capture, tight serving loops, harnesses
// that forbid hipMalloc).  The split-K fp32 partials and arrival counters --
// the only scratch the dense kernels use -- live in `scratch`, a fixed array
// of this code object, instead of the stream's library workspace.
//
// The array's host-side name is not a device address: the address is taken
// once per device with hipGetSymbolAddress (each device holds its own copy)
// and only that pointer is passed to kernels.  Every call on a device shares
// the device's array, so calls that overlap in time on one device (two
// streams, or a captured graph replayed beside another call) race; calls on
// one stream are ordered.  The counters are zero when the code object is
// loaded, cleared again at set-up, and every split-K kernel returns each
// counter it used to zero, so they are zero at the start of every call; the
// partials are written before they are read.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <mutex>

#include "hkg.h"
#include "hkg_internal.h"

namespace {

// Largest split-K plan of the planner: split x tiles stays within the 256
// compute units and tiles are at most 128 x 128, so its partials take at
// most 256 x 128 x 128 x 4 bytes = 16 MiB; tile and column-block counts of
// split plans stay below 256 counters.
constexpr size_t kPartialBytes = (size_t)16 << 20;
constexpr size_t kCounters = 16384;
constexpr size_t kScratchBytes = kPartialBytes + kCounters * sizeof(int);

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_setup;
std::atomic<unsigned char*> g_ptr[kMaxDevices];

// The device address of `scratch` on the current device, set up on the
// first call there: hipGetSymbolAddress, then (outside stream capture) the
// counters cleared with a synchronous hipMemset.
hkg_status_t device_scratch(hipStream_t stream, unsigned char** out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return HKG_ERR_NO_DEVICE;
    if (dev < 0 || dev >= kMaxDevices)
        return HKG_ERR_UNSUPPORTED;
    unsigned char* p = g_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_setup);
        p = g_ptr[dev].load(std::memory_order_relaxed);
        if (!p) {
            void* addr = nullptr;
            e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
            if (e != hipSuccess || !addr)
                return HKG_ERR_HIP;
            hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
            e = hipStreamIsCapturing(stream, &cs);
            if (e != hipSuccess)
                return HKG_ERR_HIP;
            if (cs == hipStreamCaptureStatusNone) {
                e = hipMemset((unsigned char*)addr + kPartialBytes, 0, kCounters * sizeof(int));
                if (e != hipSuccess)
                    return HKG_ERR_HIP;
            }
            p = (unsigned char*)addr;
            g_ptr[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return HKG_OK;
}

}  // namespace

extern "C" hkg_status_t hkg_gemm_bf16_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N,
                                              int64_t K, void* stream)
{
    hkg_plan_t plan;
    hkg_status_t st = hkg_gemm_bf16_plan(M, N, K, &plan);
    if (st != HKG_OK)
        return st;
    hkg::FixedScratch fixed{nullptr, kPartialBytes, nullptr, kCounters};
    if (plan.split_k > 1) {            // only split plans touch the array
        unsigned char* p = nullptr;
        st = device_scratch((hipStream_t)stream, &p);
        if (st != HKG_OK)
            return st;
        fixed.ws = (float*)p;
        fixed.counter_base = (int*)(p + kPartialBytes);
    }
    return hkg::gemm_fixed_scratch(A, B, C, M, N, K, stream, fixed);
}
