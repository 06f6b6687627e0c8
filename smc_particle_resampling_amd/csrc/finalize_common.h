// finalize_common.h -- the per-request arithmetic of a round's end, shared by the finalize
// kernels (k_finalize.hip): one position's log-ratio and TV from its slice partials, a
// particle's bonus token from its slices' best keys, the weight reductions of up to 64
// particles in one wave, and systematic resampling's search. "Faster LLM Inference via
// Sequential Monte Carlo", section 2.
#pragma once

#include "smcsd_device.h"

namespace smcsd {
namespace {

constexpr int kTvRegs = 16;   // per-slice TV partials of a position held in registers

// The loads of one position (token, its S slice parts, the first kTvRegs of its per-slice
// sums of |p - q|), issued together; nothing here waits for them.
struct PositionLoads {
    int32_t x;
    PairPart v[kPartRegs];
    float tvs[kTvRegs];
};

__device__ __forceinline__ void issue_position(const FinalizeArgs& a, int64_t u, PositionLoads& L) {
    L.x = a.tokens[u];
    load_parts(a.pp + u * a.S, a.S, L.v);
    if (a.tv) {
        const float* tp = a.tvp + u * a.S;
#pragma unroll
        for (int t = 0; t < kTvRegs; ++t)
            if (t < a.S) L.tvs[t] = tp[t];
    }
}

// The two logits at position u's token x (row ri * (K + 1) + k of the target, row u of the
// draft); 0 when x is out of range, which the term reports.
template <int DT>
__device__ __forceinline__ void token_logits(const FinalizeArgs& a, int64_t ri, int64_t u, int32_t k,
                                             int32_t x, double& zp, double& zq) {
    zp = 0.0;
    zq = 0.0;
    if (x >= 0 && x < a.V) {
        zp = logit_at<DT>(a.target, ri * (a.K + 1) + k, a.ld, x);
        zq = logit_at<DT>(a.draft, u, a.ld, x);
    }
}

// The position's log p(x) - log q(x) = (zp[x] - Mp)/T - log Sp - ((zq[x] - Mq)/T - log Sq)
// from its slice parts and the two logits at x, 0 with an error flag when the token is out
// of range; and, with TV, its total-variation distance, written to a.tv (partials summed in
// order).
__device__ __forceinline__ double position_term_from(const FinalizeArgs& a, int64_t u, const PositionLoads& L,
                                                     double zp, double zq, float c, double invT) {
    float Mp, Mq;
    double Sp, Sq;
    pair_norms_from(a.pp + u * a.S, L.v, a.S, c, Mp, Mq, Sp, Sq);
    double term = 0.0;
    if (L.x < 0 || L.x >= a.V)
        flag_error(a.error_flags, SMCSD_DEVERR_TOKEN);
    else
        term = ((zp - (double)Mp) - (zq - (double)Mq)) * invT - (log(Sp) - log(Sq));
    if (a.tv) {
        const float* tp = a.tvp + u * a.S;
        double t2 = 0.0;
#pragma unroll
        for (int t = 0; t < kTvRegs; ++t)
            if (t < a.S) t2 += (double)L.tvs[t];
        for (int t0 = kTvRegs; t0 < a.S; t0 += 8) {
            float w[8];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if (t0 + b < a.S) w[b] = tp[t0 + b];
#pragma unroll
            for (int b = 0; b < 8; ++b)
                if (t0 + b < a.S) t2 += (double)w[b];
        }
        a.tv[u] = (float)fmin(fmax(0.5 * t2, 0.0), 1.0);
    }
    return term;
}

template <int DT>
__device__ __forceinline__ double position_term(const FinalizeArgs& a, int64_t ri, int64_t u, int32_t k,
                                                const PositionLoads& L, float c, double invT) {
    double zp, zq;
    token_logits<DT>(a, ri, u, k, L.x, zp, zq);
    return position_term_from(a, u, L, zp, zq, c, invT);
}

// Particle ri's bonus token: the best (key, index) over its S slices, slices in batches of
// 8 (-1 without noise: out_tokens then get -1 in column K). Written to a.bonus too if store.
__device__ __forceinline__ int32_t bonus_of(const FinalizeArgs& a, int64_t ri, bool store = true) {
    if (!a.bp) return -1;
    const BonusPart* bpart = a.bp + ri * a.S;
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
    if (store) a.bonus[ri] = besti;
    return besti;
}

// Up to 64 particles, one wave, lane i = particle i (l_i in s_l): DPP reductions (every lane
// ends with the same bits) and an inclusive prefix scan of the weights, all in double
// precision. Writes C_i (resampling) or W_i to s_c and, if store, the request's outputs.
__device__ __forceinline__ void weights_wave(const FinalizeArgs& a, int64_t r, int32_t N, const double* s_l,
                                             double* s_c, double* s_logZ, int32_t* s_rs, bool store = true) {
    const int i = threadIdx.x;
    const double l = i < N ? s_l[i] : -INFINITY;
    const double m = wave_max_f64(l);
    const double e = i < N ? exp(l - m) : 0.0;
    const double se = wave_sum_f64(e);
    const double w = e / se;
    const double s2 = wave_sum_f64(w * w);
    const double logZ = m + log(se);
    const double ess = 1.0 / s2;
    const int32_t rs = a.mode == SMCSD_RESAMPLE_ALWAYS ||
                       (a.mode == SMCSD_RESAMPLE_ESS && ess < (double)a.ess_frac * (double)N);
    const double acc = wave_scan_f64(w);
    if (i < N) s_c[i] = rs ? acc : w;
    if (i == 0) {
        if (store) {
            a.log_norm[r] = (float)logZ;
            a.ess[r] = (float)ess;
            a.resampled[r] = rs;
        }
        *s_logZ = logZ;
        *s_rs = rs;
    }
}

// Systematic resampling: slot j's ancestor min{i : U_j < C_i}, U_j = (j + u) / N, the last
// index standing in for "none" (clamp to N - 1).
__device__ __forceinline__ int32_t ancestor_of(int32_t j, double u, int32_t N, const double* s_c) {
    const double U = ((double)j + u) / (double)N;
    int32_t lo = 0, hi = N - 1;
    while (lo < hi) {
        const int32_t mid = (lo + hi) >> 1;
        if (U < s_c[mid]) hi = mid;
        else lo = mid + 1;
    }
    return lo;
}

}  // namespace
}  // namespace smcsd
