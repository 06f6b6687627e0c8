// smcsd_internal.h -- launch plan, workspace layout, kernel argument blocks and launchers
// shared by the host code and the kernels of libsmcsd.so. Host-only declarations: the
// device helpers are in smcsd_device.h. Not installed; the public contract is
// include/smcsd.h.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "smcsd.h"

namespace smcsd {

constexpr int kThreads = 512;        // workgroup size of the round's kernels (8 wave64)
constexpr int kWaves = kThreads / 64;
constexpr int kStreamCPL = 4;        // 16-byte chunks a lane holds per row of a slice, TV off
constexpr int kTvCPL = 4;            // ... TV on (its fp32 exponentials stay in registers)
constexpr int kMaxTvSlices = 64;     // TV exchange: wave 0 reads the 2*S partial words
constexpr int kFusedRemapEntries = 16 * kThreads;   // tables the general finalize kernel remaps
constexpr int kFinalizeShare = 4 * kThreads;        // table entries a small-finalize workgroup remaps

// How one logits row is cut into 16-byte chunks and the chunks into slices, one workgroup
// per slice. Every slice is non-empty and every chunk has at least one element < V.
struct Plan {
    int32_t R = 0, N = 0, K = 0, V = 0;
    int64_t ld = 0;
    int32_t dtype = 0;
    int32_t epc = 0;         // elements per 16-byte chunk: 8 (bf16) or 4 (f32)
    int32_t chunks = 0;      // chunks per row: ceil(V / epc)
    int32_t S = 0;           // slices per row
    int32_t cps = 0;         // chunks per slice (the last slice may hold fewer)
    int64_t pairs = 0;       // R*N*K (target, draft) row pairs
    int64_t bonus_rows = 0;  // R*N bonus rows
    int64_t pair_wgs = 0;    // pairs * S
    int64_t total_wgs = 0;   // (pairs + bonus_rows) * S
    bool tv = false;
    // workspace offsets in bytes
    size_t off_ctrl = 0, off_pp = 0, off_tvp = 0, off_bp = 0, off_terms = 0, off_lw = 0, bytes = 0;
};

// Control block at the start of the workspace (zeroed before each TV launch).
struct Ctrl {
    uint32_t abort;     // set when a slice exchange timed out; later waits return at once
    uint32_t timeout;   // the wait limit, in ticks of the 100 MHz constant clock
};

// Per (row pair, slice): max and sum of exp2((z - max) * log2e/T) of target and draft.
// As two 64-bit words (mp, sp) and (mq, sq) it is also the unit of the TV slice exchange.
struct PairPart {
    float mp, sp, mq, sq;
};

// Per (bonus row, slice): best fp32 key and its vocabulary index.
struct BonusPart {
    float key;
    int32_t idx;
};

bool make_plan(int32_t R, int32_t N, int32_t K, int32_t V, int64_t ld, int32_t dtype, bool tv,
               Plan* p);

// smcsd_round in two steps: host validation (no HIP call; the workspace fields are skipped
// when check_workspace is false), then the launch sequence with its workspace at ws
// (plan.bytes bytes, 256-byte aligned). R must be > 0 for enqueue_round.
smcsd_status check_round(const smcsd_round_args* a, Plan* plan, bool check_workspace);
smcsd_status enqueue_round(const smcsd_round_args& a, const Plan& plan, char* ws, hipStream_t s);

// Arguments of the logits pass, passed by value.
struct LogitsArgs {
    const void* target;
    const void* draft;
    const float* temperature;
    const float* gumbel;
    Ctrl* ctrl;
    PairPart* pp;
    float* tvp;               // [pairs][S] each slice's share of sum |p - q| (TV)
    BonusPart* bp;
    int32_t* error_flags;
    int64_t ld;
    int64_t pairs, pair_wgs, total_wgs;
    int32_t N, K, V;
    int32_t chunks, S, cps;
    // the previous log-weights copied into the workspace by the pass (lw_n > 0: R * N of them)
    const float* lw_src;
    float* lw_copy;
    int32_t lw_n;
};

// The TV exchange wait limit: 4e8 ticks (4 s, ~10^4 times the longest expected wait), or
// the value of SMCSD_EXCHANGE_TIMEOUT_TICKS, which lets a test drive the abort path.
uint32_t exchange_timeout_ticks();

struct FinalizeArgs {
    // from the logits pass (nullptr when log_w_incr is an input)
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* temperature;
    const PairPart* pp;
    const float* tvp;
    const BonusPart* bp;
    double* terms;            // [R][N][K] per-position log-ratios (workspace)
    // weights
    const float* log_potential;  // optional [R][N], added to the increment (from partials)
    float* log_w_incr;        // out (from partials) or in
    float* log_weights;       // in/out
    // the log-weights before the round: log_weights itself, or (members > 1) a copy the
    // logits pass made, since one member overwrites log_weights while others may still read
    const float* lw_in;
    const float* uniform;
    float* log_norm;
    float* ess;
    int32_t* resampled;
    int32_t* ancestors;
    int32_t* bonus;
    int32_t* out_tokens;
    float* tv;
    int32_t* error_flags;
    // page-table remap in the same launch (pt_in == nullptr: none)
    const int32_t* pt_in;
    int32_t* pt_out;
    int32_t* refcount;
    int32_t P, num_pages;
    int64_t ld;
    int32_t N, K, V, S;
    int32_t mode;
    float ess_frac;
    // k_finalize_small: workgroups per request (request b / members, member b % members), each
    // remapping its share of the table's columns; 1 otherwise
    int32_t members;
};

// Speculative-decoding verification: the residual draw one particle still needs after the
// decide kernel (k < 0: none). The draw is in slice `slice` of row pair (particle, k), at
// `remainder` of residual mass past the slice start; lp, lq are the row's log2 normalisers
// (log2 of the temperature softmax denominators, in units of the scaled logits).
struct ResidualJob {
    int32_t k;
    int32_t slice;
    float remainder;
    float lp, lq;
};

struct VerifyArgs {
    const void* target;
    const void* draft;
    const int32_t* tokens;
    const float* temperature;
    const float* accept_u;
    const float* residual_u;
    const PairPart* pp;
    const float* tvp;
    const BonusPart* bp;
    double* terms;           // [R][N][K] workspace
    ResidualJob* jobs;       // [R][N] workspace
    int32_t* n_accepted;
    int32_t* next_token;
    float* tv;
    int32_t* error_flags;
    int64_t ld;
    int32_t N, K, V, S, cps, chunks;
};

// Gumbel-Top-K. Slices as in the TV pass (4 chunks a lane); every slice keeps its k best
// (key, index) pairs, and one workgroup per row merges the S * k candidates.
constexpr int kTopkRows = 0, kTopkBonusRows = 1, kTopkResampled = 2;
constexpr int kTopkCPL = 4;
constexpr int kMaxTopk = 64;           // == SMCSD_MAX_TOPK
constexpr int kMaxTopkSlices = 64;     // S * k candidates, at most 8 per lane of the merge

struct TopkArgs {
    const void* logits;
    const float* temperature;
    const float* gumbel;
    BonusPart* cand;       // [rows][S][k] workspace
    int32_t* out_tokens;
    float* out_keys;
    // Row map. kTopkRows: logits row i, temperature[i]. kTopkBonusRows: the round's bonus
    // rows, row i = (r, j) reads target row i*(K+1) + K and temperature[r]. kTopkResampled:
    // the bonus after resampling, target row ((r*N + ancestors[i])*(K+1) + K).
    int32_t row_mode;
    const int32_t* ancestors;
    int32_t* slot_tokens;  // optional [rows][K+1]: column K receives the token
    int32_t* error_flags;
    int64_t ld;
    int32_t V, k, chunks, S, cps;
    int32_t N, K;
    // kTopkBonusRows ahead of a TV pass: the pass's control word ({0, timeout} to *ctrl) and
    // its fill_n exchange words (all ones) are written here, which saves the pass a launch.
    // fill_words nullptr: nothing is written.
    Ctrl* ctrl;
    uint32_t* fill_words;
    int64_t fill_n;
    uint32_t timeout;
    // kTopkBonusRows ahead of a pass: lw_n > 0 copies the previous log-weights as the pass
    // would (LogitsArgs::lw_src)
    const float* lw_src;
    float* lw_copy;
    int32_t lw_n;
};

// Page lifecycle between rounds. Workspace: a header (free count before and after release,
// pops, copies), per-request counts and offsets, per-particle copy ranks, per-chunk release
// counts and offsets, and the list of (source, destination) page copies.
constexpr int kPageChunk = 4096;       // pages per workgroup of the release count / push
constexpr int kCopyTile = 32768;       // bytes per workgroup step of the KV page copy

// One copy-on-write: source and destination page, bytes to copy in each KV tensor (-1
// destination: the pop found the list empty, nothing to copy).
struct PageCopy {
    int32_t src, dst;
    int32_t bytes, pad;
};

struct PagesArgs {
    const int32_t* len_before;
    const int32_t* len_after;
    int32_t* page_table;
    int32_t* refcount;
    int32_t* free_ids;
    int32_t* n_free;
    void* kv;
    int64_t page_bytes, kv_stride;
    int32_t kv_count;
    int32_t token_rows;    // nonzero: copy only the tail's filled token rows
    int32_t* hdr;          // [4]: free count before release, after release, pops, copies
    int32_t* req_cow;      // [R]
    int32_t* req_pops;     // [R]
    int32_t* req_base;     // [R] first pop of the request
    int32_t* cow_base;     // [R] first copy of the request
    int32_t* cow_rank;     // [R][N] copy rank within the request, -1 = no copy
    int32_t* chunk_cnt;    // [chunks]
    int32_t* chunk_off;    // [chunks]
    PageCopy* copies;      // [R*N]
    int32_t* stats;        // optional [5]: released, pops served, copies served, pops unserved,
                           // token rows the served copies cover (per KV tensor)
    int32_t* error_flags;
    int32_t R, N, P, page_size, num_pages, chunks;
};

struct RemapArgs {
    const int32_t* ancestors;
    const int32_t* pt_in;
    int32_t* pt_out;
    int32_t* refcount;
    int32_t* error_flags;
    int32_t N, P, num_pages, blocks_per_request;
};

// Host launchers (defined next to their kernels). Return hipSuccess or the launch error.
// Ctrl of a TV pass: abort 0 and the wait limit (one small kernel, graph-capturable).
// The logits pass: TV on (row pairs only, persistent cooperative grid) or TV off (row pairs
// and bonus rows, one workgroup per (row, slice)).
hipError_t launch_logits_tv(const Plan& plan, const LogitsArgs& a, hipStream_t s);
hipError_t launch_logits_stream(const Plan& plan, const LogitsArgs& a, hipStream_t s);
hipError_t launch_tv_fill(const Plan& plan, const LogitsArgs& a, uint32_t timeout, hipStream_t s);
hipError_t launch_finalize(int32_t R, bool from_partials, int32_t dtype, const FinalizeArgs& a,
                           hipStream_t s);
hipError_t launch_remap(int32_t R, const RemapArgs& a, hipStream_t s);
hipError_t launch_verify(int32_t R, int32_t dtype, const VerifyArgs& a, hipStream_t s);
hipError_t launch_topk(int64_t rows, int32_t dtype, const TopkArgs& a, hipStream_t s);
// The slice pass alone (k = 1 candidates per (row, slice) in a.cand), for the round's bonus.
hipError_t launch_topk_slices(int64_t rows, int32_t dtype, const TopkArgs& a, hipStream_t s);
hipError_t launch_pages(const PagesArgs& a, int32_t copy_grid, hipStream_t s);
hipError_t launch_bench_read(const void* src, size_t bytes, uint32_t* sink, int32_t grid,
                             hipStream_t s);
hipError_t launch_bench_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

}  // namespace smcsd
