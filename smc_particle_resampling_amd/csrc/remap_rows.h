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

#include "smcsd_device.h"

namespace smcsd {

// Advances a (row, column) position by one workgroup stride over a table with P columns:
// dj = stride / P and dc = stride % P, computed once, so no entry needs a 64-bit division.
__device__ __forceinline__ void step_entry(int32_t& j, int32_t& col, int32_t dj, int32_t dc,
                                           int32_t P) {
    j += dj;
    col += dc;
    if (col >= P) {
        col -= P;
        ++j;
    }
}

__device__ __forceinline__ void remap_rows(const int32_t* in, int32_t* out, const int32_t* anc,
                                           const int32_t* off, int32_t P, int64_t e0, int64_t e1,
                                           int32_t* refcount, int32_t num_pages,
                                           int32_t* error_flags) {
    if (e0 + threadIdx.x >= e1) return;
    const int64_t first = e0 + threadIdx.x;
    int32_t j = (int32_t)(first / P);                 // the only 64-bit division
    int32_t col = (int32_t)(first - (int64_t)j * P);
    const int32_t dj = (int32_t)(blockDim.x / (uint32_t)P);
    const int32_t dc = (int32_t)(blockDim.x - (uint32_t)dj * (uint32_t)P);
    for (int64_t e = first; e < e1; e += blockDim.x) {
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
        step_entry(j, col, dj, dc, P);
    }
}

// The same remap for a whole request in one workgroup, with fewer refcount atomics: the
// table copy as above, then per column the rows are walked in order and consecutive rows
// naming the same page form a run whose net change, the sum of o_j - 1 over the run, goes to
// the page with one atomic, none when it is 0 (a prompt page kept by every row, say). Each
// page still gets the sum of o_i - 1 over every entry naming it, so the refcounts are those
// of remap_rows exactly; only the checks (a page id out of range among entries that change
// it, a refcount taken below zero) are made per run instead of per entry.
// Columns [p0, p1) of every row; a request's workgroups can split its columns between them.
__device__ __forceinline__ void remap_columns_runs(const int32_t* in, int32_t* out, const int32_t* anc,
                                                   const int32_t* off, int32_t N, int32_t P,
                                                   int32_t p0, int32_t p1, int32_t* refcount,
                                                   int32_t num_pages, int32_t* error_flags) {
    const int32_t W = p1 - p0;
    // the table copy, 8 entries a thread at a time: all 8 loads are issued before the stores
    // (the tables may alias as far as the compiler knows, so it would not reorder them)
    constexpr int kCopy = 8;
    if (W > 0) {
        int32_t j = (int32_t)(threadIdx.x / (uint32_t)W);
        int32_t col = (int32_t)(threadIdx.x - (uint32_t)j * (uint32_t)W);
        const int32_t dj = (int32_t)(blockDim.x / (uint32_t)W);
        const int32_t dc = (int32_t)(blockDim.x - (uint32_t)dj * (uint32_t)W);
        while (j < N) {
            int32_t v[kCopy];
            int64_t at[kCopy];
#pragma unroll
            for (int b = 0; b < kCopy; ++b) {
                at[b] = -1;
                if (j < N) {
                    const int32_t src = anc[j];
                    v[b] = src >= 0 ? in[(int64_t)src * P + p0 + col] : -1;
                    at[b] = (int64_t)j * P + p0 + col;
                }
                step_entry(j, col, dj, dc, W);
            }
#pragma unroll
            for (int b = 0; b < kCopy; ++b)
                if (at[b] >= 0) out[at[b]] = v[b];
        }
    }
    constexpr int kRows = 8;   // loads of a column issued together
    for (int32_t c = p0 + (int32_t)threadIdx.x; c < p1; c += blockDim.x) {
        int32_t run_page = -1, run_delta = 0;
        bool run_moves = false, bad = false, neg = false;
        auto flush = [&]() {
            if (run_page >= 0 && run_moves) {
                if (run_page >= num_pages) {
                    bad = true;
                } else if (run_delta != 0) {
                    const int32_t old = atomicAdd(&refcount[run_page], run_delta);
                    if (old + run_delta < 0) neg = true;
                }
            }
        };
        for (int32_t j0 = 0; j0 < N; j0 += kRows) {
            int32_t pg[kRows];
#pragma unroll
            for (int b = 0; b < kRows; ++b) pg[b] = j0 + b < N ? in[(int64_t)(j0 + b) * P + c] : -1;
#pragma unroll
            for (int b = 0; b < kRows; ++b) {
                if (j0 + b >= N) break;
                if (pg[b] != run_page) {
                    flush();
                    run_page = pg[b];
                    run_delta = 0;
                    run_moves = false;
                }
                const int32_t d = off[j0 + b] - 1;
                run_delta += d;
                run_moves = run_moves || d != 0;
            }
        }
        flush();
        if (bad) flag_error(error_flags, SMCSD_DEVERR_PAGE);
        if (neg) flag_error(error_flags, SMCSD_DEVERR_REFCOUNT);
    }
}

// The same remap for columns [p0, p0 + w) of a request's table of P columns, with at most
// 64 particles, held in LDS as in[j * w + c] (N * w <= kPer * blockDim.x entries), by one
// workgroup with every refcount atomic in flight at once: the copy out to out[j * P + p0 +
// c]; then one thread per column walks its rows and writes, for every entry, the net change
// of the run that ends there (0 where no run ends, the run names no page, or the change is
// 0) into dl; after a barrier every thread adds the changes of its kPer entries, one atomic
// each, and checks the results only once all of them are issued. A change fits in 16 bits:
// at most 64 rows, each o_j - 1 in [-1, 63]. A column's runs are those of
// remap_columns_runs, so the refcounts and checks are the same whichever workgroup takes
// which columns.
template <int kPer>
__device__ __forceinline__ void remap_columns_lds(const int32_t* in, int16_t* dl, int32_t w, int32_t* out,
                                                  int32_t P, int32_t p0, const int32_t* anc,
                                                  const int32_t* off, int32_t N, int32_t* refcount,
                                                  int32_t num_pages, int32_t* error_flags) {
    const int32_t NW = N * w;
    const int32_t tid = (int32_t)threadIdx.x, nt = (int32_t)blockDim.x;
    if (nt % w == 0) {
        // a thread keeps one column
        const int32_t col = tid % w, dj = nt / w;
#pragma unroll 4
        for (int32_t j = tid / w; j < N; j += dj) {
            const int32_t src = anc[j];
            out[(int64_t)j * P + p0 + col] = src >= 0 ? in[src * w + col] : -1;
        }
    } else {
        int32_t j = tid / w;
        int32_t col = tid - j * w;
        const int32_t dj = nt / w, dc = nt - dj * w;
        while (j < N) {
            const int32_t src = anc[j];
            out[(int64_t)j * P + p0 + col] = src >= 0 ? in[src * w + col] : -1;
            step_entry(j, col, dj, dc, w);
        }
    }
    // The walk has no branch but the loop's: with at most two waves a SIMD nothing hides a
    // branch's cost. Row j >= 1 closes the run that row j - 1 ended, if the page changes.
    // Lane l holds o_l - 1 (N <= 64), read per row with readlane.
    const int32_t lane = tid & 63;
    const int32_t offv = lane < N ? off[lane] - 1 : 0;
    bool bad = false;
    for (int32_t c = tid; c < w; c += nt) {
        int32_t run_page = in[c], run_delta = __builtin_amdgcn_readlane(offv, 0);
        bool run_moves = run_delta != 0;
        for (int32_t j = 1; j <= N; ++j) {
            const int32_t jc = min(j, N - 1);
            const int32_t pgr = in[jc * w + c];          // always in range; row N is past the end
            const int32_t pg = j < N ? pgr : -1;
            const int32_t od = j < N ? __builtin_amdgcn_readlane(offv, jc) : 0;
            const bool changed = j == N || pg != run_page;
            const bool counts = changed && run_page >= 0 && run_moves;
            bad = bad || (counts && run_page >= num_pages);
            dl[(j - 1) * w + c] = (int16_t)(counts && run_page < num_pages ? run_delta : 0);
            run_delta = (changed ? 0 : run_delta) + od;
            run_moves = (!changed && run_moves) || od != 0;
            run_page = pg;
        }
    }
    __syncthreads();
    int32_t old[kPer], d[kPer];
#pragma unroll
    for (int b = 0; b < kPer; ++b) {
        const int32_t e = b * nt + tid;
        d[b] = e < NW ? (int32_t)dl[e] : 0;
        old[b] = 0;
        if (d[b] != 0) old[b] = atomicAdd(&refcount[in[e]], d[b]);
    }
    bool neg = false;
#pragma unroll
    for (int b = 0; b < kPer; ++b) neg = neg || (d[b] != 0 && old[b] + d[b] < 0);
    if (bad) flag_error(error_flags, SMCSD_DEVERR_PAGE);
    if (neg) flag_error(error_flags, SMCSD_DEVERR_REFCOUNT);
}

}  // namespace smcsd
