// k_finalize.hip -- per-request end of an SMC-SD round: importance weights, normalisation,
// ESS, the resample decision, systematic resampling and the tokens each new slot keeps.
//
// "Faster LLM Inference via Sequential Monte Carlo", section 2: every particle gets an
// importance weight instead of accept/reject; low-weight particles are evicted and
// high-weight ones duplicated back to N; each round keeps K drafted tokens plus one bonus
// token. One workgroup handles one request. The slice partials of the logits pass are
// combined in fixed slice order, and everything per request runs in double precision: the
// log-weights, logsumexp, ESS and the inclusive prefix sum of the weights. A boundary tie
// U_j == C_i therefore resolves the same way on every run. When the round carries a page
// table, the same workgroup then remaps its request's table rows through the ancestors
// (pointer exchange, as k_remap does), which saves the round a launch.
//
// Two kernels. k_finalize_small takes the common case (at most one position a thread and
// at most 64 particles) with everything of the request in LDS: it runs once per round on
// one workgroup per request, so its time is latency, and it keeps the chain of dependent
// steps and the instructions it executes few. k_finalize takes every other size, and the
// resampling of given increments (smcsd_resample).
#include <algorithm>

#include "finalize_common.h"
#include "remap_rows.h"

namespace smcsd {
namespace {

template <int DT, bool FROM_PARTIALS>
__global__ __launch_bounds__(kThreads) void k_finalize(FinalizeArgs a) {
    __shared__ double s_l[SMCSD_MAX_N];    // l_i = log_weights_i + log_w_incr_i
    __shared__ double s_c[SMCSD_MAX_N];    // W_i, then C_i
    __shared__ int32_t s_bonus[SMCSD_MAX_N];
    __shared__ int32_t s_anc[SMCSD_MAX_N];   // ancestors, for the page-table remap
    __shared__ int32_t s_off[SMCSD_MAX_N];   // offspring counts o_i
    __shared__ double s_logZ;
    __shared__ int32_t s_rs;
    __shared__ double s_red[2 * kWaves];       // per-wave partials of the block reductions
    __shared__ int32_t s_pt[kFusedRemapEntries];   // the request's input page table
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int32_t N = a.N, K = a.K;
    // The request's uniform, loaded now: nothing of the round writes it.
    const double u_r = (double)a.uniform[r];

    // The input page table does not depend on this round's ancestors, so its loads (16 a
    // thread at most; launch_finalize takes no larger table) are issued first; they arrive
    // while the weights are computed and go to LDS, from where the remap at the end reads
    // them instead of waiting on global memory.
    constexpr int kPtRegs = kFusedRemapEntries / kThreads;
    const int64_t NP = a.pt_in ? (int64_t)N * a.P : 0;
    const bool staged = NP > 0;
    int32_t ptv[kPtRegs];
    if (staged) {
#pragma unroll
        for (int b = 0; b < kPtRegs; ++b) {
            const int64_t e = (int64_t)b * kThreads + tid;
            if (e < NP) ptv[b] = a.pt_in[r * NP + e];
        }
    }

    if constexpr (FROM_PARTIALS) {
        const float T = a.temperature[r];
        const float c = kLog2e / T;             // the scale the logits pass used
        const double invT = 1.0 / (double)T;
        // one thread per (particle, position): the position's log p(x) - log q(x) and TV.
        // The token, the S slice parts and (with TV) the first 16 float4 of the position's
        // S * kWaves partials are all loaded before any of them is used, so a thread waits
        // for memory a few times rather than once per load. Every sum keeps its order.
        for (int32_t ik = tid; ik < N * K; ik += kThreads) {
            const int32_t i = ik / K, k = ik - i * K;
            const int64_t ri = r * N + i;
            const int64_t u = ri * K + k;
            PositionLoads L;
            issue_position(a, u, L);
            a.terms[u] = position_term<DT>(a, ri, u, k, L, c, invT);
        }
        if (staged) {
#pragma unroll
            for (int b = 0; b < kPtRegs; ++b) {
                const int64_t e = (int64_t)b * kThreads + tid;
                if (e < NP) s_pt[e] = ptv[b];
            }
        }
        // one thread per particle: its bonus token. When the positions leave enough threads
        // idle, the waves after theirs take the particles, so these loads overlap the ones
        // above (a wave of their own issues them at once).
        const int32_t pos_end = (N * K + 63) / 64 * 64;
        const int32_t boff = pos_end + N <= kThreads ? pos_end : 0;
        for (int32_t i = tid - boff; i < N; i += kThreads)
            if (i >= 0) s_bonus[i] = bonus_of(a, r * N + i);
        __syncthreads();   // terms written above are read by other threads below
        for (int32_t i = tid; i < N; i += kThreads) {
            const int64_t ri = r * N + i;
            double lw = 0.0;
            for (int32_t k0 = 0; k0 < K; k0 += 8) {   // k in order, loads in batches of 8
                double w[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    if (k0 + b < K) w[b] = a.terms[ri * K + k0 + b];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    if (k0 + b < K) lw += w[b];
            }
            if (a.log_potential) lw += (double)a.log_potential[ri];
            a.log_w_incr[ri] = (float)lw;
            s_l[i] = (double)a.log_weights[ri] + lw;
        }
    } else {
        if (staged) {
#pragma unroll
            for (int b = 0; b < kPtRegs; ++b) {
                const int64_t e = (int64_t)b * kThreads + tid;
                if (e < NP) s_pt[e] = ptv[b];
            }
        }
        for (int32_t i = tid; i < N; i += kThreads)
            s_l[i] = (double)a.log_weights[r * N + i] + (double)a.log_w_incr[r * N + i];
    }
    for (int32_t i = tid; i < N; i += kThreads) s_off[i] = 0;
    __syncthreads();

    if (N <= 64) {
        if (tid < 64) weights_wave(a, r, N, s_l, s_c, &s_logZ, &s_rs);
    } else {
        // more than 64 particles: the whole workgroup, each thread on the particles 2t and
        // 2t + 1 (N <= 2 * kThreads); every reduction and the scan combine in one fixed
        // order (the thread's pair, a butterfly within each wave, the waves in index order)
        static_assert(SMCSD_MAX_N <= 2 * kThreads, "two particles a thread");
        const int lane = tid & 63, wv = tid >> 6;
        const int i0 = 2 * tid, i1 = 2 * tid + 1;
        const double l0 = i0 < N ? s_l[i0] : -INFINITY;
        const double l1 = i1 < N ? s_l[i1] : -INFINITY;
        double m = fmax(l0, l1);
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) m = fmax(m, __shfl_xor(m, d));
        if (lane == 0) s_red[wv] = m;
        __syncthreads();
        m = s_red[0];
        for (int t = 1; t < kWaves; ++t) m = fmax(m, s_red[t]);
        const double e0 = i0 < N ? exp(l0 - m) : 0.0;
        const double e1 = i1 < N ? exp(l1 - m) : 0.0;
        double se = e0 + e1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) se += __shfl_xor(se, d);
        __syncthreads();                       // s_red is reused
        if (lane == 0) s_red[wv] = se;
        __syncthreads();
        se = s_red[0];
        for (int t = 1; t < kWaves; ++t) se += s_red[t];
        const double w0 = e0 / se, w1 = e1 / se;
        double s2 = w0 * w0 + w1 * w1;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) s2 += __shfl_xor(s2, d);
        // inclusive prefix sums: the thread's pair, a scan over the lanes, then the waves
        const double pair = w0 + w1;
        double acc = pair;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const double o = __shfl_up(acc, d);
            if (lane >= d) acc += o;
        }
        __syncthreads();                       // s_red is reused
        if (lane == 0) s_red[wv] = s2;
        if (lane == 63) s_red[kWaves + wv] = acc;   // the wave's total weight
        __syncthreads();
        s2 = s_red[0];
        for (int t = 1; t < kWaves; ++t) s2 += s_red[t];
        double base = 0.0;
        for (int t = 0; t < wv; ++t) base += s_red[kWaves + t];
        // C at particle 2t + 1 is base + acc; C just before particle 2t is the previous
        // lane's value, computed by the same operations; C at 2t lies between the two (min
        // keeps the sums non-decreasing whatever the roundings)
        double excl = __shfl_up(acc, 1);
        if (lane == 0) excl = 0.0;
        const double c1 = base + acc;
        const double c0 = fmin((base + excl) + w0, c1);
        const double logZ = m + log(se);
        const double ess = 1.0 / s2;
        const int32_t rs = a.mode == SMCSD_RESAMPLE_ALWAYS ||
                           (a.mode == SMCSD_RESAMPLE_ESS && ess < (double)a.ess_frac * (double)N);
        if (i0 < N) s_c[i0] = rs ? c0 : w0;
        if (i1 < N) s_c[i1] = rs ? c1 : w1;
        if (tid == 0) {
            a.log_norm[r] = (float)logZ;
            a.ess[r] = (float)ess;
            a.resampled[r] = rs;
            s_logZ = logZ;
            s_rs = rs;
        }
    }
    __syncthreads();

    const int32_t rs = s_rs;
    const double logZ = s_logZ;
    for (int32_t j = tid; j < N; j += kThreads) {
        const int32_t anc = rs ? ancestor_of(j, u_r, N, s_c) : j;
        a.ancestors[r * N + j] = anc;
        s_anc[j] = anc;
        if (a.pt_in) atomicAdd(&s_off[anc], 1);
        a.log_weights[r * N + j] = rs ? (float)(-log((double)N)) : (float)(s_l[j] - logZ);
        if constexpr (FROM_PARTIALS) {
            if (a.out_tokens) {
                int32_t* dst = a.out_tokens + (r * N + j) * (K + 1);
                const int32_t* src = a.tokens + (r * N + anc) * K;
                for (int32_t k0 = 0; k0 < K; k0 += 8) {   // loads of a batch before its stores
                    int32_t t[8];
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        if (k0 + b < K) t[b] = src[k0 + b];
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        if (k0 + b < K) dst[k0 + b] = t[b];
                }
                dst[K] = s_bonus[anc];
            }
        }
    }

    // the request's page-table remap, when the round carries a small table, read from LDS
    if (a.pt_in) {
        __syncthreads();
        int32_t* out = a.pt_out + r * NP;
        // up to 64 particles: one atomic per run of equal pages in a column; more particles
        // would make each column's walk long, so one atomic per entry there
        if (N <= 64)
            remap_columns_runs(s_pt, out, s_anc, s_off, N, a.P, 0, a.P, a.refcount, a.num_pages,
                               a.error_flags);
        else
            remap_rows(s_pt, out, s_anc, s_off, a.P, 0, NP, a.refcount, a.num_pages, a.error_flags);
    }
}

// The common case, at most one position a thread (N * K <= kThreads) and at most 64
// particles, as one short kernel with every value of the request in LDS. Same results as
// k_finalize. Every load that depends on no other load (the uniform, the page table, the
// previous log-weights, each position's token, slice parts and TV partials, the bonus
// parts) is issued before the first wait; the gather of the two logits at the token is the
// only dependent one. A kernel's instruction cache is cold when it starts, so the code that
// runs is kept short: this kernel is mostly latency.
// A table of more than kFinalizeShare entries (N * P) is split by columns over a.members
// workgroups a request (a larger share a workgroup measured slower: the remap's column walk
// and atomics took 7 of the kernel's 16 us on 8192 entries): each member does the request's arithmetic
// itself (the same inputs and instructions give the same bits), copies its rows j % members
// of out_tokens and remaps its columns; member 0 alone writes the request's other outputs.
// The previous log-weights then come from a copy (a.lw_in), since member 0 overwrites
// log_weights while the others may still read them.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_finalize_small(FinalizeArgs a) {
    constexpr int kMaxN = 64;
    constexpr int kPtRegs = kFinalizeShare / kThreads;
    __shared__ double s_term[kThreads];    // the positions' log-ratios
    __shared__ int32_t s_tok[kThreads];    // the drafted tokens
    __shared__ double s_l[kMaxN];          // l_i = log_weights_i + log_w_incr_i
    __shared__ double s_c[kMaxN];          // W_i, then C_i
    __shared__ int32_t s_bonus[kMaxN];
    __shared__ int32_t s_anc[kMaxN];
    __shared__ int32_t s_off[kMaxN];       // offspring counts o_i
    __shared__ int32_t s_pt[kFinalizeShare];   // this member's columns of the input page table
    __shared__ int16_t s_dl[kFinalizeShare];   // refcount change of the run ending at each entry
    __shared__ double s_logZ;
    __shared__ int32_t s_rs;
    const int tid = threadIdx.x;
    const int32_t gs = a.members;
    const int64_t r = blockIdx.x / gs;
    const int32_t gi = (int32_t)(blockIdx.x - r * gs);
    const bool lead = gi == 0;
    const int32_t N = a.N, K = a.K, NK = N * K;
    const double u_r = (double)a.uniform[r];
    const float T = a.temperature[r];
    const int64_t NP = a.pt_in ? (int64_t)N * a.P : 0;   // the request's whole table
    // this member's columns [p0, p0 + w) of it, staged as s_pt[j * w + c] (N * w entries)
    const int32_t p0 = NP > 0 ? (int32_t)((int64_t)a.P * gi / gs) : 0;
    const int32_t w = NP > 0 ? (int32_t)((int64_t)a.P * (gi + 1) / gs) - p0 : 0;
    const int32_t NW = N * w;
    double lw_prev = 0.0, lpot = 0.0;
    if (tid < N) {
        lw_prev = (double)a.lw_in[r * N + tid];
        if (a.log_potential) lpot = (double)a.log_potential[r * N + tid];
    }
    // thread tid < NK: position (i, k); the particles' bonus parts go to the waves after the
    // positions' when they fit (a wave of their own issues its loads at once), else to the
    // position threads after their position. The page table, needed last, is loaded after
    // the positions' values, so that those come first.
    const int32_t pos_end = (NK + 63) / 64 * 64;
    const int32_t boff = pos_end + N <= kThreads ? pos_end : 0;
    PositionLoads L;
    const int32_t i = tid < NK ? tid / K : 0, k = tid - i * K;
    const int64_t ri = r * N + i, u = ri * K + k;
    if (tid < NK) issue_position(a, u, L);
    int32_t ptv[kPtRegs];
#pragma unroll
    for (int b = 0; b < kPtRegs; ++b) {
        const int32_t e = b * kThreads + tid;
        if (e < NW) {
            const int32_t j = e / w;
            ptv[b] = a.pt_in[r * NP + (int64_t)j * a.P + p0 + (e - j * w)];
        }
    }
    if (tid < NK) {
        s_term[tid] = position_term<DT>(a, ri, u, k, L, kLog2e / T, 1.0 / (double)T);
        s_tok[tid] = L.x;
    }
    if (tid >= boff && tid < boff + N) s_bonus[tid - boff] = bonus_of(a, r * N + (tid - boff), lead);
#pragma unroll
    for (int b = 0; b < kPtRegs; ++b) {
        const int32_t e = b * kThreads + tid;
        if (e < NW) s_pt[e] = ptv[b];
    }
    if (tid < N) s_off[tid] = 0;
    __syncthreads();
    if (tid < N) {
        double lw = 0.0;
        for (int32_t k = 0; k < K; ++k) lw += s_term[tid * K + k];
        if (a.log_potential) lw += lpot;
        if (lead) a.log_w_incr[r * N + tid] = (float)lw;
        s_l[tid] = lw_prev + lw;
    }
    __syncthreads();
    if (tid < 64) weights_wave(a, r, N, s_l, s_c, &s_logZ, &s_rs, lead);
    __syncthreads();
    if (tid < N) {
        const int32_t j = tid;
        const int32_t anc = s_rs ? ancestor_of(j, u_r, N, s_c) : j;
        s_anc[j] = anc;
        if (NW > 0) atomicAdd(&s_off[anc], 1);
        if (lead) {
            a.ancestors[r * N + j] = anc;
            a.log_weights[r * N + j] = s_rs ? (float)(-log((double)N)) : (float)(s_l[j] - s_logZ);
        }
        if (a.out_tokens && j % gs == gi) {
            int32_t* dst = a.out_tokens + (r * N + j) * (K + 1);
            for (int32_t k = 0; k < K; ++k) dst[k] = s_tok[anc * K + k];
            dst[K] = s_bonus[anc];
        }
    }
    if (NW > 0) {
        __syncthreads();
        remap_columns_lds<kPtRegs>(s_pt, s_dl, w, a.pt_out + r * NP, a.P, p0, s_anc, s_off, N, a.refcount,
                                   a.num_pages, a.error_flags);
    }
}

}  // namespace

hipError_t launch_finalize(int32_t R, bool from_partials, int32_t dtype, const FinalizeArgs& a,
                           hipStream_t s) {
    const bool small = from_partials && a.N <= 64 && a.N * a.K <= kThreads;
    // the page table is staged in LDS, a member's share of its columns at a time (k_finalize:
    // one member); larger shares go to launch_remap instead
    if (!small && a.members > 1) return hipErrorInvalidValue;
    const int32_t gs = std::max(a.members, 1);
    if (a.pt_in && (int64_t)a.N * ((a.P + gs - 1) / gs) > (small ? kFinalizeShare : kFusedRemapEntries))
        return hipErrorInvalidValue;
    const dim3 grid((unsigned)((int64_t)R * gs)), block(kThreads);
    if (small) {
        if (dtype == SMCSD_BF16) k_finalize_small<SMCSD_BF16><<<grid, block, 0, s>>>(a);
        else k_finalize_small<SMCSD_F32><<<grid, block, 0, s>>>(a);
    } else if (!from_partials) {
        k_finalize<SMCSD_F32, false><<<grid, block, 0, s>>>(a);
    } else if (dtype == SMCSD_BF16) {
        k_finalize<SMCSD_BF16, true><<<grid, block, 0, s>>>(a);
    } else {
        k_finalize<SMCSD_F32, true><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace smcsd
