// noalloc.hip -- smcsd_round_noalloc: the SMC-SD round with its workspace in a static device
// buffer of the library, for callers that cannot allocate device memory.
//
// The buffer is a file-scope __device__ array, so every GPU the library runs on holds its own
// copy at its own address from module load until the process ends. In host code the array's
// name is only a host-side stand-in, never a device address: the device address is looked up
// once per device with hipGetSymbolAddress (that device current) and only that address is
// handed to the kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "smcsd.h"
#include "smcsd_device.h"

namespace {

static __device__ __align__(256) unsigned char scratch[SMCSD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch` per device, once looked up

// The current device's copy of the buffer.
hipError_t scratch_address(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidValue;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

extern "C" smcsd_status smcsd_round_noalloc(const smcsd_round_args* args, smcsd_stream stream) {
    if (!args) return SMCSD_ERR_ARG;
    if (args->workspace || args->workspace_bytes) return SMCSD_ERR_ARG;
    smcsd::Plan plan;
    const smcsd_status st = smcsd::check_round(args, &plan, false);
    if (st != SMCSD_OK || args->R == 0) return st;
    if (plan.bytes > (size_t)SMCSD_NOALLOC_SCRATCH_BYTES) return SMCSD_ERR_SCRATCH;
    void* ws = nullptr;
    if (scratch_address(&ws) != hipSuccess) return SMCSD_ERR_DEVICE;
    return smcsd::enqueue_round(*args, plan, static_cast<char*>(ws),
                                reinterpret_cast<hipStream_t>(stream));
}
