// k_bench.hip -- calibration kernels for measurement (include/smcsd_bench.h): a plain
// streaming read (attainable HBM read bandwidth) and a plain copy of known size (turns the
// FETCH_SIZE / WRITE_SIZE hardware counters into bytes). Not part of the round.
#include "smcsd_device.h"

namespace smcsd {
namespace {

constexpr int kBenchThreads = 256;   // workgroup size of both calibration kernels

__global__ __launch_bounds__(kBenchThreads) void k_stream_read(const u32x4* __restrict__ src, int64_t n,
                                                          uint32_t* __restrict__ sink) {
    uint32_t acc = 0u;
    const int64_t stride = (int64_t)gridDim.x * kBenchThreads;
    for (int64_t i = (int64_t)blockIdx.x * kBenchThreads + threadIdx.x; i < n; i += stride) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    sink[(int64_t)blockIdx.x * kBenchThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(kBenchThreads) void k_copy(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                   int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * kBenchThreads;
    for (int64_t i = (int64_t)blockIdx.x * kBenchThreads + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

}  // namespace

hipError_t launch_bench_read(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                             hipStream_t s) {
    k_stream_read<<<dim3((unsigned)grid), dim3(kBenchThreads), 0, s>>>(
        static_cast<const u32x4*>(src), (int64_t)(bytes / 16), sink);
    return hipGetLastError();
}

hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t s) {
    k_copy<<<dim3(2048), dim3(kBenchThreads), 0, s>>>(static_cast<const u32x4*>(src),
                                                 static_cast<u32x4*>(dst), (int64_t)(bytes / 16));
    return hipGetLastError();
}

}  // namespace smcsd
