// k_remap.hip -- page-table remap by pointer exchange.
//
// "Faster LLM Inference via Sequential Monte Carlo", section 2 (KV-cache management): a
// particle duplicated by resampling gets a copy of its source's page metadata and shares
// the source's KV pages through pointers; no KV tensor is copied. Here the metadata is a
// page table [R][N][P] of int32 page ids (negative = unused) plus a refcount per page:
//   page_table_out[r][j] = page_table_in[r][ancestors[r][j]]
//   o_i = #{j : ancestors[r][j] = i};  refcount[page] += o_i - 1 for every valid entry of
//   old row i with o_i != 1.
// Rows with o_i == 1 (kept once) cost one copy and no atomic; up to 64 particles, equal pages
// in consecutive rows of a column share one atomic. Integer atomics commute, so the
// resulting refcounts do not depend on scheduling.
#include "remap_rows.h"
#include "smcsd_device.h"

namespace smcsd {
namespace {

__global__ __launch_bounds__(kThreads) void k_remap(RemapArgs a) {
    __shared__ int32_t s_anc[SMCSD_MAX_N];
    __shared__ int32_t s_off[SMCSD_MAX_N];
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x / a.blocks_per_request;
    const int32_t part = blockIdx.x % a.blocks_per_request;
    const int32_t N = a.N, P = a.P;

    for (int32_t j = tid; j < N; j += kThreads) s_off[j] = 0;
    __syncthreads();
    for (int32_t j = tid; j < N; j += kThreads) {
        const int32_t x = a.ancestors[r * N + j];
        const bool ok = x >= 0 && x < N;
        s_anc[j] = ok ? x : -1;
        if (ok) atomicAdd(&s_off[x], 1);
        else if (part == 0) flag_error(a.error_flags, SMCSD_DEVERR_ANCESTOR);
    }
    __syncthreads();

    const int64_t NP = (int64_t)N * P;
    if (N <= 64) {
        // up to 64 particles: the request's columns split between its workgroups, one
        // refcount atomic per run of equal pages in a column (remap_columns_runs)
        const int32_t per = (P + a.blocks_per_request - 1) / a.blocks_per_request;
        const int32_t p0 = min(P, part * per);
        const int32_t p1 = min(P, p0 + per);
        remap_columns_runs(a.pt_in + r * NP, a.pt_out + r * NP, s_anc, s_off, N, P, p0, p1,
                           a.refcount, a.num_pages, a.error_flags);
        return;
    }
    const int64_t per = (NP + a.blocks_per_request - 1) / a.blocks_per_request;
    const int64_t e0 = (int64_t)part * per;
    const int64_t e1 = min(NP, e0 + per);
    remap_rows(a.pt_in + r * NP, a.pt_out + r * NP, s_anc, s_off, P, e0, e1, a.refcount,
               a.num_pages, a.error_flags);
}

}  // namespace

hipError_t launch_remap(int32_t R, const RemapArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)R * a.blocks_per_request)), block(kThreads);
    k_remap<<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
