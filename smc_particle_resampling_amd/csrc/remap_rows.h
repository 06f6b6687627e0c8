// remap_rows.h -- the page-table remap of one request, shared by k_remap and k_finalize.
//
// "Faster LLM Inference via Sequential Monte Carlo", section 2 (KV-cache management): a
// duplicated particle gets a copy of its source's page metadata and shares its KV pages.
//   out[j][c] = in[anc[j]][c];  for every valid entry of old row i with o_i != 1 (o_i the
//   number of new slots whose ancestor is i), refcount[page] += o_i - 1.
// Entries [e0, e1) of the request's N * P table, strided by the workgroup's threads. anc and
// off are the request's ancestors (all in [0, N)) and offspring counts. Integer atomics
// commute, so the refcounts do not depend on the order.
#pragma once

#include "smcsd_internal.h"

namespace smcsd {

__device__ __forceinline__ void remap_rows(const int32_t* in, int32_t* out, const int32_t* anc,
                                           const int32_t* off, int32_t P, int64_t e0, int64_t e1,
                                           int32_t* refcount, int32_t num_pages,
                                           int32_t* error_flags) {
    for (int64_t e = e0 + threadIdx.x; e < e1; e += blockDim.x) {
        const int32_t j = (int32_t)(e / P);
        const int32_t col = (int32_t)(e - (int64_t)j * P);
        const int32_t src = anc[j];
        out[e] = src >= 0 ? in[(int64_t)src * P + col] : -1;
        const int32_t page = in[e];            // old row j, column col
        const int32_t o = off[j];
        if (page >= 0 && o != 1) {
            if (page >= num_pages) {
                flag_error(error_flags, SMCSD_DEVERR_PAGE);
            } else {
                const int32_t old = atomicAdd(&refcount[page], o - 1);
                if (old + (o - 1) < 0) flag_error(error_flags, SMCSD_DEVERR_REFCOUNT);
            }
        }
    }
}

}  // namespace smcsd
