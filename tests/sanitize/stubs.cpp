// stubs.cpp -- the launchers of libsmcsd.so's kernels and the one HIP runtime call the host
// code makes, replaced for the sanitizer build of the host code (api.cpp) without a GPU.
// Each stub counts the call and fails like a launch would, so a test can tell that a call
// passed host validation and reached its first launch.
#include <hip/hip_runtime.h>

#include "smcsd_internal.h"

int g_stub_launches = 0;

namespace smcsd {
namespace {
hipError_t stub() {
    ++g_stub_launches;
    return hipErrorNotSupported;
}
}  // namespace
hipError_t launch_logits_tv(const Plan&, const LogitsArgs&, hipStream_t) { return stub(); }
hipError_t launch_logits_stream(const Plan&, const LogitsArgs&, hipStream_t) { return stub(); }
hipError_t launch_tv_fill(const Plan&, const LogitsArgs&, uint32_t, hipStream_t) { return stub(); }
hipError_t launch_finalize(int32_t, bool, int32_t, const FinalizeArgs&, hipStream_t) { return stub(); }
hipError_t launch_remap(int32_t, const RemapArgs&, hipStream_t) { return stub(); }
hipError_t launch_verify(int32_t, int32_t, const VerifyArgs&, hipStream_t) { return stub(); }
hipError_t launch_topk(int64_t, int32_t, const TopkArgs&, hipStream_t) { return stub(); }
hipError_t launch_topk_slices(int64_t, int32_t, const TopkArgs&, hipStream_t) { return stub(); }
hipError_t launch_pages(const PagesArgs&, int32_t, hipStream_t) { return stub(); }
hipError_t launch_bench_read(const void*, size_t, uint32_t*, int32_t, hipStream_t) { return stub(); }
hipError_t launch_bench_copy(const void*, void*, size_t, hipStream_t) { return stub(); }
}  // namespace smcsd

extern "C" hipError_t hipEventRecord(hipEvent_t, hipStream_t) {
    ++g_stub_launches;
    return hipErrorNotSupported;
}
