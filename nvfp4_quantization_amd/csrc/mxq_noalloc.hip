// mxq_noalloc.hip -- the grouped NVFP4 call for callers that cannot allocate (code
// under stream capture, tight serving loops, harnesses that forbid it): the
// workspace of mxq_group_rht_quant_nvfp4 comes from a fixed device array of the
// library instead of the caller.
//
// The array `scratch` is a file-scope device variable, so every GPU the library runs
// on holds its own copy, at its own address, until the process ends.  Host code
// never passes the array's name to a kernel (in host code that name is a host-side
// stand-in, not a device address): once per device, with that device current, the
// first call on it looks up the device address with hipGetSymbolAddress and keeps
// it, and uses only that address afterwards.  The same first call clears the words
// the grouped call needs at zero (the single-read form's error word and partial
// words) with a fill kernel on the caller's stream; every finished call leaves them
// at zero again.  All calls on one GPU share that GPU's array, so calls that
// overlap on one GPU (different streams, or different host threads without
// ordering) race and must not be issued.
#include <hip/hip_runtime.h>

#include <mutex>

#include "mxq.h"
#include "mxq_internal.hpp"

namespace {

constexpr size_t kScratchBytes = MXQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
struct DeviceScratch {
    std::once_flag once;
    void* ptr = nullptr;            // device address of this device's `scratch`
    hipError_t status = hipSuccess;
};
DeviceScratch g_device[kMaxDevices];

// Zero-fill of words [0, n) (a kernel rather than a memset, so that a captured first
// call records an ordinary kernel node).
__global__ void k_clear_words(uint32_t* p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

// The scratch address of the current device, set up on the first call for it.
hipError_t device_scratch(hipStream_t stream, void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    DeviceScratch& d = g_device[dev];
    std::call_once(d.once, [&] {
        void* ptr = nullptr;
        d.status = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (d.status != hipSuccess) return;
        // the status lines, tables and single-read partial words of the grouped call:
        // the protocol words among them must start at zero
        const int64_t words = mxq::kPartialsOffset / 4;
        hipLaunchKernelGGL(k_clear_words, dim3(64), dim3(256), 0, stream, static_cast<uint32_t*>(ptr), words);
        d.status = hipGetLastError();
        if (d.status == hipSuccess) d.ptr = ptr;
    });
    *out = d.ptr;
    return d.status;
}

}  // namespace

extern "C" mxq_status mxq_group_rht_quant_nvfp4_noalloc(const uint16_t* x_bf16, int64_t k,
                                                        const int64_t* split_sections, int64_t num_sections,
                                                        uint16_t rht_sign_mask, uint32_t flags, const mxq_sr* sr,
                                                        const mxq_nvfp4_out* rowwise,
                                                        const mxq_nvfp4_out* columnwise,
                                                        const mxq_fp8_out* fp8_rowwise, void* stream) {
    // the grouped call's own checks first (nothing is enqueued), then the scratch size
    int64_t total_rows = 0;
    const mxq_status c = mxq::grouped_check(x_bf16, k, split_sections, num_sections, flags, rowwise, columnwise,
                                            fp8_rowwise, nullptr, &total_rows);
    if (c != MXQ_OK) return c;
    const size_t need = mxq_group_rht_quant_nvfp4_workspace_size(total_rows, k, num_sections, flags);
    if (need > kScratchBytes) return MXQ_ERR_UNSUPPORTED;
    void* ws = nullptr;
    if (need > 0) {
        if (device_scratch(static_cast<hipStream_t>(stream), &ws) != hipSuccess || !ws) return MXQ_ERR_HIP;
    }
    return mxq_group_rht_quant_nvfp4(x_bf16, k, split_sections, num_sections, rht_sign_mask, flags, sr, rowwise,
                                     columnwise, fp8_rowwise, ws, ws ? kScratchBytes : 0, stream);
}
