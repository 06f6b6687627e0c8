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
#include "remap_rows.h"
#include "smcsd_device.h"

namespace smcsd {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

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
        constexpr int kTvRegs = 16;
        for (int32_t ik = tid; ik < N * K; ik += kThreads) {
            const int32_t i = ik / K, k = ik - i * K;
            const int64_t ri = r * N + i;
            const int64_t u = ri * K + k;
            const int32_t x = a.tokens[u];
            const PairPart* part = a.pp + u * a.S;
            PairPart v[kPartRegs];
            load_parts(part, a.S, v);
            // the position's block of partials starts at a multiple of 32 floats
            const float4* tp = a.tv ? reinterpret_cast<const float4*>(a.tvp + u * a.S * kWaves) : nullptr;
            const int n4 = a.tv ? a.S * kWaves / 4 : 0;
            float4 tv4[kTvRegs];
#pragma unroll
            for (int t = 0; t < kTvRegs; ++t)
                if (t < n4) tv4[t] = tp[t];
            float Mp, Mq;
            double Sp, Sq;
            pair_norms_from(part, v, a.S, c, Mp, Mq, Sp, Sq);
            double term = 0.0;
            if (x < 0 || x >= a.V) {
                flag_error(a.error_flags, SMCSD_DEVERR_TOKEN);
            } else {
                // (zp[x] - Mp)/T - log Sp  -  ((zq[x] - Mq)/T - log Sq)
                const double zp = logit_at<DT>(a.target, ri * (K + 1) + k, a.ld, x);
                const double zq = logit_at<DT>(a.draft, u, a.ld, x);
                term = ((zp - (double)Mp) - (zq - (double)Mq)) * invT - (log(Sp) - log(Sq));
            }
            a.terms[u] = term;
            if (a.tv) {
                double t2 = 0.0;
                auto add4 = [&](const float4& f) {
                    t2 += (double)f.x;
                    t2 += (double)f.y;
                    t2 += (double)f.z;
                    t2 += (double)f.w;
                };
#pragma unroll
                for (int t = 0; t < kTvRegs; ++t)
                    if (t < n4) add4(tv4[t]);
                for (int t0 = kTvRegs; t0 < n4; t0 += 8) {
                    float4 w[8];
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        if (t0 + b < n4) w[b] = tp[t0 + b];
#pragma unroll
                    for (int b = 0; b < 8; ++b)
                        if (t0 + b < n4) add4(w[b]);
                }
                a.tv[u] = (float)fmin(fmax(0.5 * t2, 0.0), 1.0);
            }
        }
        if (staged) {
#pragma unroll
            for (int b = 0; b < kPtRegs; ++b) {
                const int64_t e = (int64_t)b * kThreads + tid;
                if (e < NP) s_pt[e] = ptv[b];
            }
        }
        // one thread per particle: its bonus token, the best (key, index) over the slices
        // (none without noise: out_tokens then get -1 in column K); slices in batches of 8.
        // When the positions leave enough threads idle, those threads take the particles, so
        // these loads overlap the ones above.
        const int32_t boff = N * K + N <= kThreads ? N * K : 0;
        for (int32_t i = tid - boff; i < N; i += kThreads) {
            if (i < 0) continue;
            if (!a.bp) {
                s_bonus[i] = -1;
                continue;
            }
            const BonusPart* bpart = a.bp + (r * N + i) * a.S;
            float best = -INFINITY;
            int32_t besti = INT32_MAX;
            for (int t0 = 0; t0 < a.S; t0 += 8) {
                BonusPart w[8];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    if (t0 + b < a.S) w[b] = bpart[t0 + b];
#pragma unroll
                for (int b = 0; b < 8; ++b)
                    if (t0 + b < a.S && (t0 + b == 0 || better(w[b].key, w[b].idx, best, besti))) {
                        best = w[b].key;
                        besti = w[b].idx;
                    }
            }
            if (besti < 0 || besti >= a.V) besti = 0;   // only if every key was NaN
            a.bonus[r * N + i] = besti;
            s_bonus[i] = besti;
        }
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
        // one wave, lane i = particle i: butterfly reductions (every lane ends with the same
        // bits) and an inclusive prefix scan of the weights, all in double precision
        if (tid < 64) {
            const int i = tid;
            const double l = i < N ? s_l[i] : -INFINITY;
            double m = l;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) m = fmax(m, __shfl_xor(m, d));
            const double e = i < N ? exp(l - m) : 0.0;
            double se = e;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) se += __shfl_xor(se, d);
            const double w = e / se;
            double s2 = w * w;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) s2 += __shfl_xor(s2, d);
            const double logZ = m + log(se);
            const double ess = 1.0 / s2;
            const int32_t rs = a.mode == SMCSD_RESAMPLE_ALWAYS ||
                               (a.mode == SMCSD_RESAMPLE_ESS && ess < (double)a.ess_frac * (double)N);
            double acc = w;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const double o = __shfl_up(acc, d);
                if (i >= d) acc += o;
            }
            if (i < N) s_c[i] = rs ? acc : w;
            if (i == 0) {
                a.log_norm[r] = (float)logZ;
                a.ess[r] = (float)ess;
                a.resampled[r] = rs;
                s_logZ = logZ;
                s_rs = rs;
            }
        }
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
    const double u = (double)a.uniform[r];
    for (int32_t j = tid; j < N; j += kThreads) {
        int32_t anc = j;
        if (rs) {
            // min{i : U_j < C_i}, the last index standing in for "none" (clamp to N-1)
            const double U = ((double)j + u) / (double)N;
            int32_t lo = 0, hi = N - 1;
            while (lo < hi) {
                const int32_t mid = (lo + hi) >> 1;
                if (U < s_c[mid]) hi = mid;
                else lo = mid + 1;
            }
            anc = lo;
        }
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

}  // namespace

hipError_t launch_finalize(int32_t R, bool from_partials, int32_t dtype, const FinalizeArgs& a,
                           hipStream_t s) {
    // the page table is staged in LDS: larger ones go to launch_remap instead
    if (a.pt_in && (int64_t)a.N * a.P > kFusedRemapEntries) return hipErrorInvalidValue;
    const dim3 grid((unsigned)R), block(kThreads);
    if (!from_partials) {
        k_finalize<SMCSD_F32, false><<<grid, block, 0, s>>>(a);
    } else if (dtype == SMCSD_BF16) {
        k_finalize<SMCSD_BF16, true><<<grid, block, 0, s>>>(a);
    } else {
        k_finalize<SMCSD_F32, true><<<grid, block, 0, s>>>(a);
    }
    return hipGetLastError();
}

}  // namespace smcsd
