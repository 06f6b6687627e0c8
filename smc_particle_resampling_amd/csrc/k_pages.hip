// k_pages.hip -- page lifecycle between rounds: release, copy-on-write of shared tail pages,
// fresh pages for new columns, and the KV copies that copy-on-write needs.
//
// "Faster LLM Inference via Sequential Monte Carlo", section 2 (KV-cache management): a
// particle duplicated by resampling shares its source's KV pages through page metadata. The
// page does not describe the pool around that, so the steps follow these readings:
//   - a page's refcount is -1 while free, else the number of table entries naming it; the
//     free list is a stack of page ids;
//   - release: pages at refcount 0 are pushed in increasing id and get refcount -1;
//   - copy-on-write: when a request's length is not a multiple of page_size, its partly
//     filled tail column is written next; there the lowest particle naming a page keeps it,
//     and every later particle naming it pops a fresh page that receives a copy of the KV
//     bytes (refcount 1; the shared page loses that reference);
//   - append: the columns the new length needs get fresh pages, particle by particle, column
//     by column;
//   - pops go request by request, within a request copies first (particle order), then the
//     appends; a pop from an empty list leaves the entry -1.
//
// The sequential pop order becomes a set of prefix sums, so every step is data parallel:
//   k_pages_count    one workgroup per request: which tail entries copy (a shared entry is one
//                    whose page an earlier particle of the request names) and their rank;
//                    the request's pop count. One workgroup per chunk of 4096 pages: how many
//                    pages of the chunk are released.
//   k_pages_scan     one workgroup: exclusive sums of the request pop counts and the chunk
//                    release counts; the final free count.
//   k_pages_release  one workgroup per chunk: pushes the chunk's released pages at their
//                    ranks, so the stack holds them in increasing id.
//   k_pages_apply    one workgroup per request: pop number i (over all requests) takes
//                    free_ids[F - 1 - i], F = free count after release; writes the table,
//                    the refcounts and the (source, destination) list of copies.
//   k_pages_copy     a grid-stride pass over (copy, KV tensor, 32 KiB tile): HBM-bound copy,
//                    of the whole page or (token-major pages) of the tail's filled rows.
// Integer atomics commute and every pop index is fixed by the sums, so the result is the
// same as the sequential one on every run.
#include "smcsd_device.h"

namespace smcsd {
namespace {

// Exclusive prefix sum of one int per thread over the workgroup; *total gets the sum.
// Wave prefix by shuffles, then the 8 wave totals through LDS.
__device__ int block_excl_scan(int v, int* lds, int* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d, 64);
        if (lane >= d) x += y;
    }
    __syncthreads();                       // lds may still be read by a previous call
    if (lane == 63) lds[wave] = x;
    __syncthreads();
    int before = 0, all = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int t = lds[w];
        before += w < wave ? t : 0;
        all += t;
    }
    *total = all;
    return before + x - v;
}

// Tail column of request r that the next round writes, or -1 (length a multiple of
// page_size). Lengths were checked by length_ok.
__device__ __forceinline__ int32_t tail_col(int32_t lb, int32_t page_size) {
    return (lb > 0 && lb % page_size != 0) ? (lb - 1) / page_size : -1;
}

__device__ __forceinline__ bool length_ok(int32_t lb, int32_t la, int32_t P, int32_t page_size) {
    return lb >= 0 && lb <= la && (int64_t)la <= (int64_t)P * page_size;
}

__device__ __forceinline__ int32_t ceil_div(int32_t a, int32_t b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(kThreads) void k_pages_count(PagesArgs a) {
    __shared__ int32_t s_tail[SMCSD_MAX_N];
    __shared__ int32_t s_scan[kWaves];
    const int tid = threadIdx.x;
    const int32_t N = a.N, P = a.P;
    int total;
    if ((int32_t)blockIdx.x < a.R) {
        const int32_t r = blockIdx.x;
        const int32_t lb = a.len_before[r], la = a.len_after[r];
        const bool ok = length_ok(lb, la, P, a.page_size);
        if (!ok && tid == 0) flag_error(a.error_flags, SMCSD_DEVERR_LENGTH);
        const int32_t c = ok ? tail_col(lb, a.page_size) : -1;
        const int32_t* row0 = a.page_table + (int64_t)r * N * P;
        if (c >= 0) {
            for (int32_t j = tid; j < N; j += kThreads) {
                int32_t p = row0[(int64_t)j * P + c];
                if (p >= a.num_pages) {
                    flag_error(a.error_flags, SMCSD_DEVERR_PAGE);
                    p = -1;
                }
                s_tail[j] = p;
            }
        }
        __syncthreads();
        // Particles [j0, j0 + per) belong to this thread, so ranks follow particle order.
        static_assert(SMCSD_MAX_N <= 32 * kThreads, "shared flags of a thread fit 32 bits");
        const int32_t per = (N + kThreads - 1) / kThreads;
        const int32_t j0 = min(N, tid * per), j1 = min(N, j0 + per);
        uint32_t shared_bits = 0;
        int mine = 0;
        if (c >= 0) {
            for (int32_t j = j0; j < j1; ++j) {
                const int32_t p = s_tail[j];
                bool shared = false;
                for (int32_t jj = 0; jj < j && p >= 0 && !shared; ++jj) shared = s_tail[jj] == p;
                shared_bits |= (uint32_t)shared << (j - j0);
                mine += shared;
            }
        }
        int rank = block_excl_scan(mine, s_scan, &total);
        for (int32_t j = j0; j < j1; ++j) {
            const bool shared = (shared_bits >> (j - j0)) & 1u;
            a.cow_rank[(int64_t)r * N + j] = shared ? rank : -1;
            rank += shared;
        }
        if (tid == 0) {
            const int32_t ncols = ok ? max(0, ceil_div(la, a.page_size) - ceil_div(lb, a.page_size)) : 0;
            a.req_cow[r] = total;
            a.req_pops[r] = total + N * ncols;
        }
    } else {
        const int64_t b = (int64_t)blockIdx.x - a.R;
        const int64_t p0 = b * kPageChunk;
        int mine = 0;
#pragma unroll
        for (int e = 0; e < kPageChunk / kThreads; ++e) {
            const int64_t p = p0 + (int64_t)tid * (kPageChunk / kThreads) + e;
            mine += (p < a.num_pages && a.refcount[p] == 0);
        }
        block_excl_scan(mine, s_scan, &total);
        if (tid == 0) a.chunk_cnt[b] = total;
    }
}

// In place: v[i] <- sum of v[0..i-1] over n entries, in tiles of kThreads; returns the sum.
__device__ int excl_scan_array(int32_t* v, int64_t n, int* lds) {
    int carry = 0, total;
    for (int64_t t0 = 0; t0 < n; t0 += kThreads) {
        const int64_t i = t0 + threadIdx.x;
        const int x = i < n ? v[i] : 0;
        const int before = block_excl_scan(x, lds, &total);
        if (i < n) v[i] = carry + before;
        carry += total;
    }
    return carry;
}

__global__ __launch_bounds__(kThreads) void k_pages_scan(PagesArgs a) {
    __shared__ int32_t s_scan[kWaves];
    // req_base / cow_base / chunk_off start as copies of the counts and are scanned in place.
    for (int64_t i = threadIdx.x; i < a.R; i += kThreads) {
        a.req_base[i] = a.req_pops[i];
        a.cow_base[i] = a.req_cow[i];
    }
    for (int64_t i = threadIdx.x; i < a.chunks; i += kThreads) a.chunk_off[i] = a.chunk_cnt[i];
    __syncthreads();
    const int pops = excl_scan_array(a.req_base, a.R, s_scan);
    const int cows = excl_scan_array(a.cow_base, a.R, s_scan);
    const int released = excl_scan_array(a.chunk_off, a.chunks, s_scan);
    __shared__ int32_t s_F;
    if (threadIdx.x == 0) {
        int32_t n0 = *a.n_free;
        if (n0 < 0 || n0 > a.num_pages) {
            flag_error(a.error_flags, SMCSD_DEVERR_POOL);
            n0 = min(max(n0, 0), a.num_pages);
        }
        // A consistent pool has released + n0 <= num_pages (released pages are not free).
        int32_t F = n0 + released;
        if ((int64_t)n0 + released > a.num_pages) {
            flag_error(a.error_flags, SMCSD_DEVERR_POOL);
            F = a.num_pages;
        }
        if (pops > F) flag_error(a.error_flags, SMCSD_DEVERR_POOL);
        a.hdr[0] = n0;
        a.hdr[1] = F;
        a.hdr[2] = pops;
        a.hdr[3] = cows;
        *a.n_free = max(0, F - pops);
        s_F = F;
    }
    __syncthreads();
    if (a.stats) {
        // Copies served: request r's copies are pops req_base[r] .. req_base[r] + req_cow[r] - 1.
        // Each copies `rows` token rows: the tail's filled rows with token-major pages, else all.
        const int32_t F = s_F;
        int mine = 0, mine_rows = 0;
        for (int64_t i = threadIdx.x; i < a.R; i += kThreads) {
            const int served = max(0, min(a.req_cow[i], F - a.req_base[i]));
            const int rows = a.token_rows ? a.len_before[i] % a.page_size : a.page_size;
            mine += served;
            mine_rows += served * rows;
        }
        int copied, rows_copied;
        block_excl_scan(mine, s_scan, &copied);
        block_excl_scan(mine_rows, s_scan, &rows_copied);
        if (threadIdx.x == 0) {
            a.stats[0] = F - a.hdr[0];
            a.stats[1] = min(pops, F);
            a.stats[2] = copied;
            a.stats[3] = max(0, pops - F);
            a.stats[4] = rows_copied;
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_pages_release(PagesArgs a) {
    __shared__ int32_t s_scan[kWaves];
    constexpr int kPer = kPageChunk / kThreads;
    const int64_t b = blockIdx.x;
    const int64_t p0 = b * kPageChunk + (int64_t)threadIdx.x * kPer;
    bool rel[kPer];
    int mine = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        rel[e] = p0 + e < a.num_pages && a.refcount[p0 + e] == 0;
        mine += rel[e];
    }
    int total;
    int pos = block_excl_scan(mine, s_scan, &total) + a.chunk_off[b] + a.hdr[0];
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
        if (rel[e]) {
            a.refcount[p0 + e] = -1;
            if (pos < a.num_pages) a.free_ids[pos] = (int32_t)(p0 + e);
            ++pos;
        }
    }
}

// Pops number i of the round: free_ids[F - 1 - i], or -1 when the list ran dry or holds an
// id out of range.
__device__ __forceinline__ int32_t pop_page(const PagesArgs& a, int64_t i, int32_t F) {
    if (i >= F) {
        flag_error(a.error_flags, SMCSD_DEVERR_POOL);
        return -1;
    }
    const int32_t q = a.free_ids[F - 1 - i];
    if (q < 0 || q >= a.num_pages) {
        flag_error(a.error_flags, SMCSD_DEVERR_PAGE);
        return -1;
    }
    return q;
}

__global__ __launch_bounds__(kThreads) void k_pages_apply(PagesArgs a) {
    const int32_t r = blockIdx.x;
    const int32_t N = a.N, P = a.P;
    const int32_t lb = a.len_before[r], la = a.len_after[r];
    if (!length_ok(lb, la, P, a.page_size)) return;
    const int32_t F = a.hdr[1];
    const int64_t base = a.req_base[r];
    const int32_t cow = a.req_cow[r];
    const int64_t cb = a.cow_base[r];
    int32_t* row0 = a.page_table + (int64_t)r * N * P;
    const int32_t c = tail_col(lb, a.page_size);
    const int32_t copy_bytes =
        a.token_rows ? (int32_t)((lb % a.page_size) * (a.page_bytes / a.page_size)) : (int32_t)a.page_bytes;
    if (c >= 0) {
        for (int32_t j = threadIdx.x; j < N; j += kThreads) {
            const int32_t rank = a.cow_rank[(int64_t)r * N + j];
            if (rank < 0) continue;
            int32_t* slot = row0 + (int64_t)j * P + c;
            const int32_t p = *slot;               // in [0, num_pages): checked by the count
            const int32_t q = pop_page(a, base + rank, F);
            *slot = q;
            if (q >= 0) a.refcount[q] = 1;
            const int32_t old = atomicSub(&a.refcount[p], 1);
            if (old < 1) flag_error(a.error_flags, SMCSD_DEVERR_REFCOUNT);
            a.copies[cb + rank] = PageCopy{p, q, copy_bytes, 0};
        }
    }
    const int32_t c0 = ceil_div(lb, a.page_size);
    const int32_t ncols = max(0, ceil_div(la, a.page_size) - c0);
    const int64_t n_app = (int64_t)N * ncols;
    for (int64_t e = threadIdx.x; e < n_app; e += kThreads) {
        const int32_t j = (int32_t)(e / ncols);
        const int32_t col = c0 + (int32_t)(e - (int64_t)j * ncols);
        const int32_t q = pop_page(a, base + cow + e, F);
        row0[(int64_t)j * P + col] = q;
        if (q >= 0) a.refcount[q] = 1;
    }
}

// Copies page src to page dst in every KV tensor; units are (copy, tensor, tile) triples
// taken grid-stride, the number of copies read from the scan's header.
__global__ __launch_bounds__(kThreads) void k_pages_copy(PagesArgs a) {
    const int64_t tiles = (a.page_bytes + kCopyTile - 1) / kCopyTile;
    const int64_t per_copy = tiles * a.kv_count;
    const int64_t units = (int64_t)a.hdr[3] * per_copy;
    char* kv = static_cast<char*>(a.kv);
    for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
        const int64_t ci = u / per_copy;
        const int64_t rem = u - ci * per_copy;
        const int64_t t = rem / tiles;
        const int64_t tile = rem - t * tiles;
        const PageCopy pc = a.copies[ci];
        const int64_t off = tile * kCopyTile;
        if (pc.dst < 0 || off >= pc.bytes) continue;
        const int64_t n16 = (min((int64_t)kCopyTile, (int64_t)pc.bytes - off)) / 16;
        const u32x4* src = reinterpret_cast<const u32x4*>(kv + t * a.kv_stride + pc.src * a.page_bytes + off);
        u32x4* dst = reinterpret_cast<u32x4*>(kv + t * a.kv_stride + pc.dst * a.page_bytes + off);
        constexpr int kPer = kCopyTile / 16 / kThreads;
        u32x4 v[kPer];
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kThreads;
            if (i < n16) v[k] = __builtin_nontemporal_load(src + i);
        }
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int64_t i = threadIdx.x + (int64_t)k * kThreads;
            if (i < n16) __builtin_nontemporal_store(v[k], dst + i);
        }
    }
}

}  // namespace

hipError_t launch_pages(const PagesArgs& a, int32_t copy_grid, hipStream_t s) {
    const dim3 block(kThreads);
    k_pages_count<<<dim3((unsigned)(a.R + a.chunks)), block, 0, s>>>(a);
    k_pages_scan<<<dim3(1), block, 0, s>>>(a);
    k_pages_release<<<dim3((unsigned)a.chunks), block, 0, s>>>(a);
    if (a.R > 0) k_pages_apply<<<dim3((unsigned)a.R), block, 0, s>>>(a);
    if (a.kv && copy_grid > 0) k_pages_copy<<<dim3((unsigned)copy_grid), block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
