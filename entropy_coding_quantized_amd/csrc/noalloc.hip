// sh_encode_noalloc: sh_encode for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid allocation).  The encode
// kernels' workspace -- the per-chunk worst-case slots, the per-chunk bit totals and the
// per-block aggregates -- lives in a file-scope device array, `scratch`, of
// kNoAllocScratchBytes on every GPU the library runs on; the caller passes only inputs and
// outputs.
//
// The array's device address is taken once per device, with that device current, by
// hipGetSymbolAddress on the entry point's first call there, and kept per device: host code
// never passes the array's own name to a kernel or a copy (in host code it is a host-side
// stand-in, not a device address).
//
// Every call on a GPU shares that GPU's array, which keeps the last call's contents.  The
// encode writes every workspace word it later reads (slots, totals and aggregates), so
// nothing needs clearing between calls.  Calls that overlap on one GPU (on different
// streams, or from different host threads) race on the array and must be serialised by
// the caller.
#include <hip/hip_runtime.h>

#include <mutex>

#include "codec_internal.hpp"

namespace shn {
namespace {

constexpr uint64_t kNoAllocScratchBytes = 64ull << 20;  // 64 MiB on every GPU used

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The array's device address on the current device (taken once per device), or null.
void* scratch_on_current_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace
}  // namespace shn

extern "C" {

uint64_t sh_encode_noalloc_scratch_bytes(void) { return shn::kNoAllocScratchBytes; }

sh_status sh_encode_noalloc(const sh_table* table, const sh_params* params, const int8_t* d_x,
                            uint64_t n, uint8_t* d_out, uint64_t out_cap,
                            sh_encode_info* d_info, int32_t* d_status, void* stream) {
    const uint64_t need = sh_encode_workspace(n, params);
    // parameters the GPU path does not take: sh_encode reports which error it is
    if (need == 0) return sh_encode(table, params, d_x, n, d_out, out_cap, nullptr, 0, d_info,
                                    d_status, stream);
    if (need > shn::kNoAllocScratchBytes) return SH_ERR_BUFFER_TOO_SMALL;
    void* ws = shn::scratch_on_current_device();
    if (!ws) return SH_ERR_HIP;
    return sh_encode(table, params, d_x, n, d_out, out_cap, ws, shn::kNoAllocScratchBytes, d_info,
                     d_status, stream);
}

}  // extern "C"
