// api.cpp -- the C ABI of libsmcsd.so (include/smcsd.h): argument validation, the launch
// plan, workspace layout and the launch sequence of one SMC-SD round.
//
// Validation is plain host code and makes no HIP call, so argument errors come back
// synchronously, before anything is enqueued, on any machine.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstdint>
#include <cstring>

#include "smcsd.h"
#include "smcsd_bench.h"
#include "smcsd_internal.h"

namespace smcsd {

static size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

uint32_t exchange_timeout_ticks() {
    const char* v = std::getenv("SMCSD_EXCHANGE_TIMEOUT_TICKS");
    if (v && *v) {
        char* end = nullptr;
        const unsigned long long t = std::strtoull(v, &end, 10);
        if (end && *end == '\0') return (uint32_t)std::min<unsigned long long>(t, UINT32_MAX);
    }
    return 400000000u;
}

bool make_plan(int32_t R, int32_t N, int32_t K, int32_t V, int64_t ld, int32_t dtype, bool tv,
               Plan* p) {
    if (R < 0 || N < 1 || N > SMCSD_MAX_N || K < 1 || K > SMCSD_MAX_K || V < 1) return false;
    if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return false;
    Plan q;
    q.R = R;
    q.N = N;
    q.K = K;
    q.V = V;
    q.ld = ld;
    q.dtype = dtype;
    q.tv = tv;
    q.epc = dtype == SMCSD_F32 ? 4 : 8;
    q.chunks = (int32_t)(((int64_t)V + q.epc - 1) / q.epc);
    const int32_t per_slice = kThreads * (tv ? kTvCPL : kStreamCPL);
    const int32_t s0 = (q.chunks + per_slice - 1) / per_slice;
    q.cps = (q.chunks + s0 - 1) / s0;
    q.S = (q.chunks + q.cps - 1) / q.cps;   // no empty slice
    q.pairs = (int64_t)R * N * K;          // < 2^49: R < 2^31, N <= 2^10, K <= 2^8
    q.bonus_rows = (int64_t)R * N;
    // grid range: (pairs + bonus rows) * S workgroups below 2^31, checked before multiplying
    if (q.pairs + q.bonus_rows >= (int64_t)INT32_MAX / q.S) return false;
    q.pair_wgs = q.pairs * q.S;
    q.total_wgs = (q.pairs + q.bonus_rows) * q.S;
    if (tv && q.S > kMaxTvSlices) return false;               // V > 1048576 (bf16) with TV
    size_t off = 0;
    q.off_ctrl = off;
    off = align256(off + sizeof(Ctrl));
    q.off_pp = off;
    off = align256(off + sizeof(PairPart) * (size_t)q.pair_wgs);
    q.off_tvp = off;
    off = align256(off + (tv ? sizeof(float) * (size_t)q.pair_wgs : 0));   // per (pair, slice)
    q.off_bp = off;
    off = align256(off + sizeof(BonusPart) * (size_t)(q.bonus_rows * q.S));
    q.off_terms = off;
    off = align256(off + sizeof(double) * (size_t)q.pairs);
    q.off_lw = off;   // the previous log-weights, for a finalize split over several workgroups
    off = align256(off + sizeof(float) * (size_t)R * N);
    q.bytes = off;
    *p = q;
    return true;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

// Validates a round's arguments and makes its plan. The workspace fields are checked too
// unless the caller brings its own buffer (check_workspace false). No HIP call.
smcsd_status check_round(const smcsd_round_args* a, Plan* plan, bool check_workspace) {
    if (!a) return SMCSD_ERR_ARG;
    if (a->R < 0 || a->N < 1 || a->K < 1 || a->V < 1 || a->reserved0 != 0) return SMCSD_ERR_ARG;
    if (a->dtype != SMCSD_F32 && a->dtype != SMCSD_BF16) return SMCSD_ERR_ARG;
    if (a->mode < SMCSD_RESAMPLE_ALWAYS || a->mode > SMCSD_RESAMPLE_NEVER) return SMCSD_ERR_ARG;
    if (a->mode == SMCSD_RESAMPLE_ESS && !(a->ess_frac > 0.0f && a->ess_frac <= 1.0f))
        return SMCSD_ERR_ARG;
    const int64_t epc = a->dtype == SMCSD_F32 ? 4 : 8;
    if (a->ld < a->V || a->ld % epc != 0) return SMCSD_ERR_ARG;
    if (a->N > SMCSD_MAX_N || a->K > SMCSD_MAX_K) return SMCSD_ERR_UNSUPPORTED;
    if (a->R == 0) return SMCSD_OK;
    // gumbel NULL: no bonus inside the pass (bonus may then be NULL too)
    if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->temperature ||
        !a->uniform || !a->log_weights || !a->log_w_incr || !a->log_norm || !a->ess ||
        !a->resampled || !a->ancestors || (a->gumbel && !a->bonus))
        return SMCSD_ERR_ARG;
    if (!aligned16(a->target_logits) || !aligned16(a->draft_logits) || !aligned16(a->gumbel))
        return SMCSD_ERR_ARG;
    if (a->page_table_in) {
        if (a->P < 1 || a->num_pages < 1 || !a->page_table_out || !a->refcount)
            return SMCSD_ERR_ARG;
        const size_t tb = sizeof(int32_t) * (size_t)a->R * a->N * a->P;
        if (overlap(a->page_table_in, tb, a->page_table_out, tb)) return SMCSD_ERR_ARG;
    }
    if (!make_plan(a->R, a->N, a->K, a->V, a->ld, a->dtype, a->tv != nullptr, plan))
        return SMCSD_ERR_UNSUPPORTED;
    if (check_workspace) {
        if (!a->workspace || a->workspace_bytes < plan->bytes) return SMCSD_ERR_WORKSPACE;
        if (reinterpret_cast<uintptr_t>(a->workspace) & 255u) return SMCSD_ERR_WORKSPACE;
    }
    if (!a->gumbel) {                       // the logits pass reads no bonus row
        plan->bonus_rows = 0;
        plan->total_wgs = plan->pair_wgs;
    }
    return SMCSD_OK;
}

static size_t verify_jobs_offset(const Plan& p) { return p.bytes; }

static size_t verify_bytes(const Plan& p) {
    return verify_jobs_offset(p) + align256(sizeof(ResidualJob) * (size_t)p.R * p.N);
}

static smcsd_status check_verify(const smcsd_verify_args* a, Plan* plan) {
    if (!a) return SMCSD_ERR_ARG;
    if (a->R < 0 || a->N < 1 || a->K < 1 || a->V < 1 || a->reserved0 != 0) return SMCSD_ERR_ARG;
    if (a->dtype != SMCSD_F32 && a->dtype != SMCSD_BF16) return SMCSD_ERR_ARG;
    const int64_t epc = a->dtype == SMCSD_F32 ? 4 : 8;
    if (a->ld < a->V || a->ld % epc != 0) return SMCSD_ERR_ARG;
    if (a->N > SMCSD_MAX_N || a->K > SMCSD_MAX_K) return SMCSD_ERR_UNSUPPORTED;
    if (a->R == 0) return SMCSD_OK;
    if (!a->target_logits || !a->draft_logits || !a->draft_tokens || !a->temperature ||
        !a->gumbel || !a->accept_uniform || !a->residual_uniform || !a->n_accepted ||
        !a->next_token)
        return SMCSD_ERR_ARG;
    if (!aligned16(a->target_logits) || !aligned16(a->draft_logits) || !aligned16(a->gumbel))
        return SMCSD_ERR_ARG;
    if (!make_plan(a->R, a->N, a->K, a->V, a->ld, a->dtype, true, plan))
        return SMCSD_ERR_UNSUPPORTED;
    if (!a->workspace || a->workspace_bytes < verify_bytes(*plan)) return SMCSD_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(a->workspace) & 255u) return SMCSD_ERR_WORKSPACE;
    return SMCSD_OK;
}

// The logits pass. With TV the row pairs run in the cooperative exchange kernel and the
// bonus rows (if any) in the Gumbel-Top-K slice kernel with k = 1, whose (key, index) per
// (row, slice) lands in the same BonusPart layout (its slicing equals the TV plan's).
// A persistent grid's share of the bonus rows ran slower than this ordinary grid.
static_assert(kTvCPL == kTopkCPL, "bonus slices of the TV plan are Gumbel-Top-K slices");

static hipError_t record(smcsd_event ev, hipStream_t s) {
    return ev ? hipEventRecord(reinterpret_cast<hipEvent_t>(ev), s) : hipSuccess;
}

// The logits pass of a round, bracketed by the optional timing events (split: see
// smcsd_round_args). TV off: one kernel. TV on: the bonus rows first, in the Gumbel-Top-K
// slice kernel, which also resets the control word and the exchange words of the row-pair
// kernel that follows (a fill kernel does that when there are no bonus rows), then the row
// pairs. Kernels, not memset nodes, so the sequence can be captured in a graph.
static hipError_t launch_logits_pass(const Plan& plan, const LogitsArgs& la, hipStream_t s,
                                     smcsd_event begin, smcsd_event split, smcsd_event end) {
    hipError_t e = hipSuccess;
    if (!plan.tv) {
        if ((e = record(begin, s)) != hipSuccess || (e = launch_logits_stream(plan, la, s)) != hipSuccess ||
            (e = record(split, s)) != hipSuccess)
            return e;
        return record(end, s);
    }
    Plan pairs = plan;
    pairs.bonus_rows = 0;
    pairs.total_wgs = plan.pair_wgs;
    LogitsArgs lp = la;
    lp.total_wgs = la.pair_wgs;
    const uint32_t timeout = exchange_timeout_ticks();
    if (plan.bonus_rows == 0) {
        if ((e = launch_tv_fill(plan, la, timeout, s)) != hipSuccess || (e = record(begin, s)) != hipSuccess ||
            (e = launch_logits_tv(pairs, lp, s)) != hipSuccess || (e = record(split, s)) != hipSuccess)
            return e;
        return record(end, s);
    }
    TopkArgs t{};
    t.logits = la.target;
    t.temperature = la.temperature;
    t.gumbel = la.gumbel;
    t.cand = la.bp;
    t.out_tokens = nullptr;
    t.row_mode = kTopkBonusRows;
    t.ld = la.ld;
    t.V = la.V;
    t.k = 1;
    t.chunks = plan.chunks;
    t.S = plan.S;
    t.cps = plan.cps;
    t.N = la.N;
    t.K = la.K;
    t.ctrl = la.ctrl;
    t.fill_words = reinterpret_cast<uint32_t*>(la.pp);
    t.fill_n = plan.pair_wgs * (int64_t)(sizeof(PairPart) / 4);
    t.timeout = timeout;
    t.lw_src = la.lw_src;
    t.lw_copy = la.lw_copy;
    t.lw_n = la.lw_n;
    if ((e = record(begin, s)) != hipSuccess || (e = launch_topk_slices(plan.bonus_rows, plan.dtype, t, s)) != hipSuccess ||
        (e = record(split, s)) != hipSuccess || (e = launch_logits_tv(pairs, lp, s)) != hipSuccess)
        return e;
    return record(end, s);
}

// Slices of a Gumbel-Top-K row: as the TV pass (512 lanes x 4 chunks at most per slice).
static bool topk_plan(int32_t rows, int32_t V, int32_t dtype, int32_t k, int32_t* chunks,
                      int32_t* S, int32_t* cps, size_t* bytes) {
    if (rows < 0 || V < 1 || k < 1 || k > kMaxTopk || k > V) return false;
    if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return false;
    const int32_t epc = dtype == SMCSD_F32 ? 4 : 8;
    const int32_t c = (int32_t)(((int64_t)V + epc - 1) / epc);
    const int32_t per_slice = kThreads * kTopkCPL;
    const int32_t s0 = (c + per_slice - 1) / per_slice;
    const int32_t q = (c + s0 - 1) / s0;
    const int32_t s = (c + q - 1) / q;
    if (s > kMaxTopkSlices) return false;
    if ((int64_t)rows * s >= (int64_t)INT32_MAX) return false;
    *chunks = c;
    *S = s;
    *cps = q;
    *bytes = align256(sizeof(BonusPart) * (size_t)rows * s * k);
    return true;
}

}  // namespace smcsd

using namespace smcsd;

extern "C" {

size_t smcsd_round_args_size(void) { return sizeof(smcsd_round_args); }

const char* smcsd_status_string(int32_t s) {
    switch (s) {
    case SMCSD_OK: return "ok";
    case SMCSD_ERR_ARG: return "invalid argument";
    case SMCSD_ERR_UNSUPPORTED: return "unsupported size";
    case SMCSD_ERR_WORKSPACE: return "workspace missing, too small or misaligned";
    case SMCSD_ERR_DEVICE: return "HIP launch or runtime error";
    case SMCSD_ERR_SCRATCH: return "request needs more than the library's static scratch buffer";
    }
    return "unknown status";
}

size_t smcsd_workspace_size(int32_t R, int32_t N, int32_t K, int32_t V, int32_t dtype,
                            int32_t tv_enabled) {
    Plan p;
    const int64_t epc = dtype == SMCSD_F32 ? 4 : 8;
    if (!make_plan(R, N, K, V, ((int64_t)V + epc - 1) / epc * epc, dtype, tv_enabled != 0, &p))
        return 0;
    return p.bytes;
}

smcsd_status smcsd_round(const smcsd_round_args* args, smcsd_stream stream) {
    Plan plan;
    const smcsd_status st = check_round(args, &plan, true);
    if (st != SMCSD_OK || args->R == 0) return st;
    return enqueue_round(*args, plan, static_cast<char*>(args->workspace),
                         reinterpret_cast<hipStream_t>(stream));
}

}  // extern "C"

namespace smcsd {

// The logits pass's argument block of a validated round.
static LogitsArgs logits_args(const smcsd_round_args& a, const Plan& plan, char* ws) {
    LogitsArgs la{};
    la.target = a.target_logits;
    la.draft = a.draft_logits;
    la.temperature = a.temperature;
    la.gumbel = a.gumbel;
    la.ctrl = reinterpret_cast<Ctrl*>(ws + plan.off_ctrl);
    la.pp = reinterpret_cast<PairPart*>(ws + plan.off_pp);
    la.tvp = reinterpret_cast<float*>(ws + plan.off_tvp);
    la.bp = reinterpret_cast<BonusPart*>(ws + plan.off_bp);
    la.error_flags = a.error_flags;
    la.ld = a.ld;
    la.pairs = plan.pairs;
    la.pair_wgs = plan.pair_wgs;
    la.total_wgs = plan.total_wgs;
    la.N = a.N;
    la.K = a.K;
    la.V = a.V;
    la.chunks = plan.chunks;
    la.S = plan.S;
    la.cps = plan.cps;
    return la;
}

// Workgroups a request for the small finalize kernel: enough that each member's share of the
// table's columns is at most kFinalizeShare entries, 1 without a table; 0 when the small
// kernel does not take the round (the general finalize then remaps tables of at most
// kFusedRemapEntries entries and k_remap the larger ones).
static int32_t finalize_members(const smcsd_round_args& a) {
    if (a.N > 64 || a.N * a.K > kThreads) return 0;
    if (!a.page_table_in || (int64_t)a.N * a.P <= kFinalizeShare) return 1;
    const int64_t cols = kFinalizeShare / a.N;   // >= 32 columns a member (N <= 64)
    const int64_t m = ((int64_t)a.P + cols - 1) / cols;
    return (int64_t)a.R * m <= INT32_MAX ? (int32_t)m : 0;   // one launch's grid
}

smcsd_status enqueue_round(const smcsd_round_args& a, const Plan& plan, char* ws, hipStream_t s) {
    LogitsArgs la = logits_args(a, plan, ws);
    const int32_t members = finalize_members(a);
    if (members > 1) {   // the pass copies the previous log-weights for the members to read
        la.lw_src = a.log_weights;
        la.lw_copy = reinterpret_cast<float*>(ws + plan.off_lw);
        la.lw_n = a.R * a.N;
    }
    hipError_t e = launch_logits_pass(plan, la, s, a.timing_begin, a.timing_split, a.timing_end);
    if (e != hipSuccess) return SMCSD_ERR_DEVICE;

    FinalizeArgs fa{};
    fa.target = a.target_logits;
    fa.draft = a.draft_logits;
    fa.tokens = a.draft_tokens;
    fa.temperature = a.temperature;
    fa.pp = la.pp;
    fa.tvp = plan.tv ? la.tvp : nullptr;
    fa.bp = a.gumbel ? la.bp : nullptr;
    fa.terms = reinterpret_cast<double*>(ws + plan.off_terms);
    fa.log_potential = a.log_potential;
    fa.log_w_incr = a.log_w_incr;
    fa.log_weights = a.log_weights;
    fa.uniform = a.uniform;
    fa.log_norm = a.log_norm;
    fa.ess = a.ess;
    fa.resampled = a.resampled;
    fa.ancestors = a.ancestors;
    fa.bonus = a.bonus;
    fa.out_tokens = a.out_tokens;
    fa.tv = a.tv;
    fa.error_flags = a.error_flags;
    fa.ld = a.ld;
    fa.N = a.N;
    fa.K = a.K;
    fa.V = a.V;
    fa.S = plan.S;
    fa.mode = a.mode;
    fa.ess_frac = a.ess_frac;
    fa.members = std::max(members, 1);
    fa.lw_in = members > 1 ? la.lw_copy : a.log_weights;
    // The finalize remaps the table in the same launch, which saves one: the small kernel
    // any table (split by columns over its members), the general one tables of at most 16
    // entries a thread; larger ones there keep the separate remap kernel.
    const int64_t table_entries = (int64_t)a.N * a.P;
    const bool fused_remap = a.page_table_in && (members > 0 || table_entries <= kFusedRemapEntries);
    if (fused_remap) {
        fa.pt_in = a.page_table_in;
        fa.pt_out = a.page_table_out;
        fa.refcount = a.refcount;
        fa.P = a.P;
        fa.num_pages = a.num_pages;
    }
    e = launch_finalize(a.R, true, a.dtype, fa, s);
    if (e != hipSuccess) return SMCSD_ERR_DEVICE;
    if (a.page_table_in && !fused_remap) {
        RemapArgs ra{};
        ra.ancestors = a.ancestors;
        ra.pt_in = a.page_table_in;
        ra.pt_out = a.page_table_out;
        ra.refcount = a.refcount;
        ra.error_flags = a.error_flags;
        ra.N = a.N;
        ra.P = a.P;
        ra.num_pages = a.num_pages;
        ra.blocks_per_request = (int32_t)std::max<int64_t>(1, (table_entries + 2047) / 2048);
        e = launch_remap(a.R, ra, s);
        if (e != hipSuccess) return SMCSD_ERR_DEVICE;
    }
    return SMCSD_OK;
}

}  // namespace smcsd

extern "C" {

smcsd_status smcsd_resample(int32_t R, int32_t N, const float* log_w_incr, float* log_weights,
                            const float* uniform, int32_t mode, float ess_frac,
                            float* log_norm, float* ess, int32_t* resampled,
                            int32_t* ancestors, smcsd_stream stream) {
    if (R < 0 || N < 1) return SMCSD_ERR_ARG;
    if (mode < SMCSD_RESAMPLE_ALWAYS || mode > SMCSD_RESAMPLE_NEVER) return SMCSD_ERR_ARG;
    if (mode == SMCSD_RESAMPLE_ESS && !(ess_frac > 0.0f && ess_frac <= 1.0f)) return SMCSD_ERR_ARG;
    if (N > SMCSD_MAX_N) return SMCSD_ERR_UNSUPPORTED;
    if (R == 0) return SMCSD_OK;
    if (!log_w_incr || !log_weights || !uniform || !log_norm || !ess || !resampled || !ancestors)
        return SMCSD_ERR_ARG;
    FinalizeArgs fa{};
    fa.log_w_incr = const_cast<float*>(log_w_incr);
    fa.log_weights = log_weights;
    fa.lw_in = log_weights;
    fa.members = 1;
    fa.uniform = uniform;
    fa.log_norm = log_norm;
    fa.ess = ess;
    fa.resampled = resampled;
    fa.ancestors = ancestors;
    fa.N = N;
    fa.K = 0;
    fa.mode = mode;
    fa.ess_frac = ess_frac;
    const hipError_t e = launch_finalize(R, false, SMCSD_F32, fa, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMCSD_OK : SMCSD_ERR_DEVICE;
}

smcsd_status smcsd_remap_pages(int32_t R, int32_t N, int32_t P, const int32_t* ancestors,
                               const int32_t* page_table_in, int32_t* page_table_out,
                               int32_t* refcount, int32_t num_pages, int32_t* error_flags,
                               smcsd_stream stream) {
    if (R < 0 || N < 1 || P < 1 || num_pages < 1) return SMCSD_ERR_ARG;
    if (N > SMCSD_MAX_N) return SMCSD_ERR_UNSUPPORTED;
    if (R == 0) return SMCSD_OK;
    if (!ancestors || !page_table_in || !page_table_out || !refcount) return SMCSD_ERR_ARG;
    if ((int64_t)R * (((int64_t)N * P + 2047) / 2048) >= (int64_t)INT32_MAX) return SMCSD_ERR_UNSUPPORTED;
    const size_t tb = sizeof(int32_t) * (size_t)R * N * P;   // < 2^31 * 2048 * 4 bytes
    if (overlap(page_table_in, tb, page_table_out, tb)) return SMCSD_ERR_ARG;
    RemapArgs ra{};
    ra.ancestors = ancestors;
    ra.pt_in = page_table_in;
    ra.pt_out = page_table_out;
    ra.refcount = refcount;
    ra.error_flags = error_flags;
    ra.N = N;
    ra.P = P;
    ra.num_pages = num_pages;
    ra.blocks_per_request = (int32_t)std::max<int64_t>(1, ((int64_t)N * P + 2047) / 2048);
    const hipError_t e = launch_remap(R, ra, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMCSD_OK : SMCSD_ERR_DEVICE;
}

// Workspace of the page lifecycle; false if the sizes are invalid or too large.
struct PagesLayout {
    int64_t chunks = 0;
    size_t off_hdr = 0, off_req = 0, off_rank = 0, off_chunk = 0, off_copies = 0, bytes = 0;
};

static bool pages_layout(int32_t R, int32_t N, int32_t P, int32_t num_pages, PagesLayout* L) {
    if (R < 0 || N < 1 || P < 1 || num_pages < 1) return false;
    if (N > SMCSD_MAX_N) return false;
    // Pops, page-table offsets and grid sizes are int32 on the device.
    if ((int64_t)R * N * P >= (int64_t)INT32_MAX) return false;
    L->chunks = ((int64_t)num_pages + kPageChunk - 1) / kPageChunk;
    if ((int64_t)R + L->chunks >= (int64_t)INT32_MAX) return false;
    size_t o = 0;
    L->off_hdr = o;
    o = align256(o + 4 * sizeof(int32_t));
    L->off_req = o;                                   // req_cow, req_pops, req_base, cow_base
    o = align256(o + 4 * sizeof(int32_t) * (size_t)R);
    L->off_rank = o;
    o = align256(o + sizeof(int32_t) * (size_t)R * N);
    L->off_chunk = o;                                 // chunk_cnt, chunk_off
    o = align256(o + 2 * sizeof(int32_t) * (size_t)L->chunks);
    L->off_copies = o;
    o = align256(o + sizeof(PageCopy) * (size_t)R * N);
    L->bytes = o;
    return true;
}

size_t smcsd_pages_workspace_size(int32_t R, int32_t N, int32_t P, int32_t num_pages) {
    PagesLayout L;
    return pages_layout(R, N, P, num_pages, &L) ? L.bytes : 0;
}

smcsd_status smcsd_pages_advance(int32_t R, int32_t N, int32_t P, int32_t page_size,
                                 const int32_t* len_before, const int32_t* len_after,
                                 int32_t* page_table, int32_t num_pages, int32_t* refcount,
                                 int32_t* free_ids, int32_t* n_free, void* kv,
                                 int64_t page_bytes, int32_t kv_count, int64_t kv_stride,
                                 int32_t token_rows, void* workspace, size_t workspace_bytes,
                                 int32_t* stats,
                                 int32_t* error_flags, smcsd_stream stream) {
    if (R < 0 || N < 1 || P < 1 || page_size < 1 || num_pages < 1) return SMCSD_ERR_ARG;
    PagesLayout L;
    if (!pages_layout(R, N, P, num_pages, &L)) return SMCSD_ERR_UNSUPPORTED;
    if (!refcount || !free_ids || !n_free) return SMCSD_ERR_ARG;
    if (R > 0 && (!len_before || !len_after || !page_table)) return SMCSD_ERR_ARG;
    int64_t max_units = 0;
    if (kv) {
        if (page_bytes < 16 || page_bytes % 16 != 0 || !aligned16(kv) || kv_count < 1)
            return SMCSD_ERR_ARG;
        if (page_bytes > INT32_MAX) return SMCSD_ERR_UNSUPPORTED;
        // token rows: page_size rows of page_bytes / page_size bytes, each a multiple of 16
        if (token_rows && (page_bytes % page_size != 0 || (page_bytes / page_size) % 16 != 0))
            return SMCSD_ERR_ARG;
        if (page_bytes > INT64_MAX / num_pages) return SMCSD_ERR_ARG;
        if (kv_count > 1 && (kv_stride % 16 != 0 || kv_stride < page_bytes * num_pages))
            return SMCSD_ERR_ARG;
        const int64_t tiles = (page_bytes + kCopyTile - 1) / kCopyTile;
        max_units = (int64_t)R * N * kv_count * tiles;
    }
    if (!workspace || workspace_bytes < L.bytes) return SMCSD_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SMCSD_ERR_WORKSPACE;
    const size_t pb = sizeof(int32_t) * (size_t)num_pages;
    const size_t tb = sizeof(int32_t) * (size_t)R * N * P;
    const void* bufs[6] = {page_table, refcount, free_ids, n_free, workspace, stats};
    const size_t sizes[6] = {tb, pb, pb, sizeof(int32_t), L.bytes, 5 * sizeof(int32_t)};
    for (int i = 0; i < 6; ++i)
        for (int k = i + 1; k < 6; ++k)
            if (bufs[i] && bufs[k] && overlap(bufs[i], sizes[i], bufs[k], sizes[k]))
                return SMCSD_ERR_ARG;
    char* ws = static_cast<char*>(workspace);
    PagesArgs a{};
    a.len_before = len_before;
    a.len_after = len_after;
    a.page_table = page_table;
    a.refcount = refcount;
    a.free_ids = free_ids;
    a.n_free = n_free;
    a.kv = kv;
    a.page_bytes = page_bytes;
    a.kv_stride = kv_stride;
    a.kv_count = kv ? kv_count : 0;
    a.token_rows = token_rows != 0;
    int32_t* req = reinterpret_cast<int32_t*>(ws + L.off_req);
    a.hdr = reinterpret_cast<int32_t*>(ws + L.off_hdr);
    a.req_cow = req;
    a.req_pops = req + R;
    a.req_base = req + 2 * (size_t)R;
    a.cow_base = req + 3 * (size_t)R;
    a.cow_rank = reinterpret_cast<int32_t*>(ws + L.off_rank);
    a.chunk_cnt = reinterpret_cast<int32_t*>(ws + L.off_chunk);
    a.chunk_off = a.chunk_cnt + L.chunks;
    a.copies = reinterpret_cast<PageCopy*>(ws + L.off_copies);
    a.stats = stats;
    a.error_flags = error_flags;
    a.R = R;
    a.N = N;
    a.P = P;
    a.page_size = page_size;
    a.num_pages = num_pages;
    a.chunks = (int32_t)L.chunks;
    // The copy kernel strides over the device-side number of copies; 2048 workgroups
    // (8 per CU) keep every CU streaming when there are many.
    const int32_t copy_grid = (int32_t)std::min<int64_t>(max_units, 2048);
    const hipError_t e = launch_pages(a, copy_grid, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMCSD_OK : SMCSD_ERR_DEVICE;
}

smcsd_status smcsd_bench_stream_read(const void* src, size_t bytes, uint32_t* sink,
                                     int32_t grid, smcsd_stream stream) {
    if (!src || !sink || grid < 1 || bytes % 16 != 0 || !aligned16(src)) return SMCSD_ERR_ARG;
    const hipError_t e = launch_bench_read(src, bytes, sink, grid, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMCSD_OK : SMCSD_ERR_DEVICE;
}

smcsd_status smcsd_bench_logits_pass(const smcsd_round_args* args, int32_t repeats,
                                     smcsd_stream stream) {
    if (repeats < 1) return SMCSD_ERR_ARG;
    Plan plan;
    const smcsd_status st = check_round(args, &plan, true);
    if (st != SMCSD_OK || args->R == 0) return st;
    const LogitsArgs la = logits_args(*args, plan, static_cast<char*>(args->workspace));
    const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    for (int32_t i = 0; i < repeats; ++i)
        if (launch_logits_pass(plan, la, s, nullptr, nullptr, nullptr) != hipSuccess) return SMCSD_ERR_DEVICE;
    return SMCSD_OK;
}

smcsd_status smcsd_bench_copy(const void* src, void* dst, size_t bytes, smcsd_stream stream) {
    if (!src || !dst || bytes % 16 != 0 || !aligned16(src) || !aligned16(dst)) return SMCSD_ERR_ARG;
    if (overlap(src, bytes, dst, bytes)) return SMCSD_ERR_ARG;
    const hipError_t e = launch_bench_copy(src, dst, bytes, reinterpret_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMCSD_OK : SMCSD_ERR_DEVICE;
}

size_t smcsd_verify_args_size(void) { return sizeof(smcsd_verify_args); }

size_t smcsd_verify_workspace_size(int32_t R, int32_t N, int32_t K, int32_t V, int32_t dtype) {
    Plan p;
    const int64_t epc = dtype == SMCSD_F32 ? 4 : 8;
    if (!make_plan(R, N, K, V, ((int64_t)V + epc - 1) / epc * epc, dtype, true, &p)) return 0;
    return verify_bytes(p);
}

smcsd_status smcsd_sd_verify(const smcsd_verify_args* args, smcsd_stream stream) {
    Plan plan;
    const smcsd_status st = check_verify(args, &plan);
    if (st != SMCSD_OK || args->R == 0) return st;
    const smcsd_verify_args& a = *args;
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* ws = static_cast<char*>(a.workspace);

    LogitsArgs la{};
    la.target = a.target_logits;
    la.draft = a.draft_logits;
    la.temperature = a.temperature;
    la.gumbel = a.gumbel;
    la.ctrl = reinterpret_cast<Ctrl*>(ws + plan.off_ctrl);
    la.pp = reinterpret_cast<PairPart*>(ws + plan.off_pp);
    la.tvp = reinterpret_cast<float*>(ws + plan.off_tvp);
    la.bp = reinterpret_cast<BonusPart*>(ws + plan.off_bp);
    la.error_flags = a.error_flags;
    la.ld = a.ld;
    la.pairs = plan.pairs;
    la.pair_wgs = plan.pair_wgs;
    la.total_wgs = plan.total_wgs;
    la.N = a.N;
    la.K = a.K;
    la.V = a.V;
    la.chunks = plan.chunks;
    la.S = plan.S;
    la.cps = plan.cps;
    if (launch_logits_pass(plan, la, s, a.timing_begin, nullptr, a.timing_end) != hipSuccess)
        return SMCSD_ERR_DEVICE;

    VerifyArgs va{};
    va.target = a.target_logits;
    va.draft = a.draft_logits;
    va.tokens = a.draft_tokens;
    va.temperature = a.temperature;
    va.accept_u = a.accept_uniform;
    va.residual_u = a.residual_uniform;
    va.pp = la.pp;
    va.tvp = la.tvp;
    va.bp = la.bp;
    va.terms = reinterpret_cast<double*>(ws + plan.off_terms);
    va.jobs = reinterpret_cast<ResidualJob*>(ws + verify_jobs_offset(plan));
    va.n_accepted = a.n_accepted;
    va.next_token = a.next_token;
    va.tv = a.tv;
    va.error_flags = a.error_flags;
    va.ld = a.ld;
    va.N = a.N;
    va.K = a.K;
    va.V = a.V;
    va.S = plan.S;
    va.cps = plan.cps;
    va.chunks = plan.chunks;
    if (launch_verify(a.R, a.dtype, va, s) != hipSuccess) return SMCSD_ERR_DEVICE;
    return SMCSD_OK;
}

size_t smcsd_bonus_workspace_size(int32_t R, int32_t N, int32_t V, int32_t dtype) {
    if (R < 0 || N < 1 || N > SMCSD_MAX_N || (int64_t)R * N >= (int64_t)INT32_MAX) return 0;
    int32_t chunks, S, cps;
    size_t bytes;
    if (!topk_plan(R * N, V, dtype, 1, &chunks, &S, &cps, &bytes)) return 0;
    return bytes > 0 ? bytes : 256;
}

smcsd_status smcsd_bonus_resampled(int32_t R, int32_t N, int32_t K, int32_t V, int64_t ld,
                                   int32_t dtype, const void* target_logits,
                                   const float* temperature, const int32_t* ancestors,
                                   const float* gumbel, int32_t* bonus, int32_t* out_tokens,
                                   void* workspace, size_t workspace_bytes,
                                   int32_t* error_flags, smcsd_stream stream) {
    if (R < 0 || N < 1 || K < 1 || V < 1) return SMCSD_ERR_ARG;
    if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_ARG;
    const int64_t epc = dtype == SMCSD_F32 ? 4 : 8;
    if (ld < V || ld % epc != 0) return SMCSD_ERR_ARG;
    if (N > SMCSD_MAX_N || K > SMCSD_MAX_K) return SMCSD_ERR_UNSUPPORTED;
    if ((int64_t)R * N >= (int64_t)INT32_MAX) return SMCSD_ERR_UNSUPPORTED;
    int32_t chunks, S, cps;
    size_t bytes;
    if (!topk_plan(R * N, V, dtype, 1, &chunks, &S, &cps, &bytes)) return SMCSD_ERR_UNSUPPORTED;
    if (R == 0) return SMCSD_OK;
    if (!target_logits || !temperature || !ancestors || !gumbel || !bonus) return SMCSD_ERR_ARG;
    if (!aligned16(target_logits) || !aligned16(gumbel)) return SMCSD_ERR_ARG;
    if (!workspace || workspace_bytes < bytes) return SMCSD_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SMCSD_ERR_WORKSPACE;
    TopkArgs a{};
    a.logits = target_logits;
    a.temperature = temperature;
    a.gumbel = gumbel;
    a.cand = static_cast<BonusPart*>(workspace);
    a.out_tokens = bonus;
    a.row_mode = kTopkResampled;
    a.ancestors = ancestors;
    a.slot_tokens = out_tokens;
    a.error_flags = error_flags;
    a.ld = ld;
    a.V = V;
    a.k = 1;
    a.chunks = chunks;
    a.S = S;
    a.cps = cps;
    a.N = N;
    a.K = K;
    if (launch_topk((int64_t)R * N, dtype, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return SMCSD_ERR_DEVICE;
    return SMCSD_OK;
}

size_t smcsd_topk_workspace_size(int32_t rows, int32_t V, int32_t dtype, int32_t k) {
    int32_t chunks, S, cps;
    size_t bytes;
    if (!topk_plan(rows, V, dtype, k, &chunks, &S, &cps, &bytes)) return 0;
    return bytes > 0 ? bytes : 256;
}

smcsd_status smcsd_gumbel_topk(int32_t rows, int32_t V, int64_t ld, int32_t dtype,
                               const void* logits, const float* temperature, const float* gumbel,
                               int32_t k, int32_t* out_tokens, float* out_keys, void* workspace,
                               size_t workspace_bytes, smcsd_stream stream) {
    if (rows < 0 || V < 1 || k < 1) return SMCSD_ERR_ARG;
    if (dtype != SMCSD_F32 && dtype != SMCSD_BF16) return SMCSD_ERR_ARG;
    const int64_t epc = dtype == SMCSD_F32 ? 4 : 8;
    if (ld < V || ld % epc != 0 || k > V) return SMCSD_ERR_ARG;
    int32_t chunks, S, cps;
    size_t bytes;
    if (!topk_plan(rows, V, dtype, k, &chunks, &S, &cps, &bytes)) return SMCSD_ERR_UNSUPPORTED;
    if (rows == 0) return SMCSD_OK;
    if (!logits || !temperature || !gumbel || !out_tokens) return SMCSD_ERR_ARG;
    if (!aligned16(logits) || !aligned16(gumbel)) return SMCSD_ERR_ARG;
    if (!workspace || workspace_bytes < bytes) return SMCSD_ERR_WORKSPACE;
    if (reinterpret_cast<uintptr_t>(workspace) & 255u) return SMCSD_ERR_WORKSPACE;
    TopkArgs a{};
    a.logits = logits;
    a.temperature = temperature;
    a.gumbel = gumbel;
    a.cand = static_cast<BonusPart*>(workspace);
    a.out_tokens = out_tokens;
    a.out_keys = out_keys;
    a.ld = ld;
    a.V = V;
    a.k = k;
    a.chunks = chunks;
    a.S = S;
    a.cps = cps;
    if (launch_topk(rows, dtype, a, reinterpret_cast<hipStream_t>(stream)) != hipSuccess)
        return SMCSD_ERR_DEVICE;
    return SMCSD_OK;
}

}  // extern "C"
