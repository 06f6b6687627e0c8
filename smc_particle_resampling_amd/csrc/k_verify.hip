// k_verify.hip -- standard speculative-decoding verification on the partials of the TV pass.
//
// The baseline the SMC-SD page compares against ("Faster LLM Inference via Sequential Monte
// Carlo", section 1): the target verifies the drafted tokens in order and the first rejection
// ends the block. Standard speculative sampling: accept x_k iff u_k < min(1, p_k(x_k)/q_k(x_k));
// at the first rejection k*, draw the next token from the residual max(p - q, 0) (inverse CDF
// over increasing v with one uniform b); if every token is accepted, the next token is the
// bonus draw from p.
//
// The residual mass of a position is its TV distance, so the TV pass of the round already
// holds, per slice, the mass sum_v |p - q| (per wave) and the slice's p and q masses; the
// slice's residual mass is (|p - q| + p - q) / 2 summed over the slice. The decide kernel
// (one workgroup per request) takes the acceptance decisions and picks the slice of the
// residual draw; the residual kernel (one workgroup per particle) scans that one slice of
// the rejected row in increasing v to find the token.
#include "smcsd_device.h"

namespace smcsd {
namespace {

// 1 - 2^t for t <= 0, without cancellation as t -> 0. For t >= -1 it is -(e^x - 1) at
// x = t ln 2 by the Taylor series of e^x - 1 through x^9, written in t (coefficients
// ln2^n / n!; the truncation is below 1e-8 relative there, and Horner's rounding keeps the
// result within about 2 ulp); below -1 it is 1 - 2^t directly, which is then at least 0.5.
__device__ __forceinline__ float one_minus_exp2(float t) {
    constexpr float c[9] = {0.69314718f,    0.24022651f,    0.055504110f,
                            0.0096181286f,  0.0013333558f,  1.5403530e-4f,
                            1.5252734e-5f,  1.3215487e-6f,  1.0178086e-7f};
    float p = c[8];
#pragma unroll
    for (int n = 7; n >= 0; --n) p = fmaf(t, p, c[n]);
    return t >= -1.0f ? -t * p : 1.0f - __builtin_amdgcn_exp2f(t);
}

template <int DT>
__global__ __launch_bounds__(kThreads) void k_verify_decide(VerifyArgs a) {
    const int tid = threadIdx.x;
    const int64_t r = blockIdx.x;
    const int32_t N = a.N, K = a.K;
    const float T = a.temperature[r];
    const float c = kLog2e / T;
    const double invT = 1.0 / (double)T;

    // one thread per (particle, position): log p(x_k) - log q(x_k) and the position's TV
    for (int32_t ik = tid; ik < N * K; ik += kThreads) {
        const int32_t i = ik / K, k = ik - i * K;
        const int64_t ri = r * N + i;
        const int64_t u = ri * K + k;
        float Mp, Mq;
        double Sp, Sq;
        pair_norms(a.pp + u * a.S, a.S, c, Mp, Mq, Sp, Sq);
        double term = 0.0;
        const int32_t x = a.tokens[u];
        if (x < 0 || x >= a.V) {
            flag_error(a.error_flags, SMCSD_DEVERR_TOKEN);
        } else {
            const double zp = logit_at<DT>(a.target, ri * (K + 1) + k, a.ld, x);
            const double zq = logit_at<DT>(a.draft, u, a.ld, x);
            term = ((zp - (double)Mp) - (zq - (double)Mq)) * invT - (log(Sp) - log(Sq));
        }
        a.terms[u] = term;
        if (a.tv) {
            double t2 = 0.0;
            for (int t = 0; t < a.S; ++t) t2 += (double)a.tvp[u * a.S + t];
            a.tv[u] = (float)fmin(fmax(0.5 * t2, 0.0), 1.0);
        }
    }
    __syncthreads();

    // one thread per particle: the first rejection, then the bonus or the residual's slice
    for (int32_t i = tid; i < N; i += kThreads) {
        const int64_t ri = r * N + i;
        int32_t ks = K;
        for (int32_t k = 0; k < K; ++k) {
            const double m = fmin(1.0, exp(a.terms[ri * K + k]));
            if (!((double)a.accept_u[ri * K + k] < m)) {
                ks = k;
                break;
            }
        }
        a.n_accepted[ri] = ks;
        ResidualJob job{-1, 0, 0.0f, 0.0f, 0.0f};
        if (ks == K) {
            const BonusPart* bpart = a.bp + ri * a.S;
            float best = bpart[0].key;
            int32_t besti = bpart[0].idx;
            for (int t = 1; t < a.S; ++t)
                if (better(bpart[t].key, bpart[t].idx, best, besti)) {
                    best = bpart[t].key;
                    besti = bpart[t].idx;
                }
            a.next_token[ri] = (besti < 0 || besti >= a.V) ? 0 : besti;
        } else {
            const int64_t u = ri * K + ks;
            const PairPart* part = a.pp + u * a.S;
            float Mp, Mq;
            double Sp, Sq;
            pair_norms(part, a.S, c, Mp, Mq, Sp, Sq);
            // residual mass of slice t: (sum|p - q| + P_t - Q_t) / 2, never below 0
            auto slice_res = [&](int t) {
                const double d = (double)a.tvp[u * a.S + t];
                const double P = (double)part[t].sp * (double)__builtin_amdgcn_exp2f((part[t].mp - Mp) * c) / Sp;
                const double Q = (double)part[t].sq * (double)__builtin_amdgcn_exp2f((part[t].mq - Mq) * c) / Sq;
                return fmax(0.5 * (d + P - Q), 0.0);
            };
            double R = 0.0;
            for (int t = 0; t < a.S; ++t) R += slice_res(t);
            const double target = (double)a.residual_u[ri] * R;
            double acc = 0.0, before = 0.0;
            int ts = -1, last = 0;
            for (int t = 0; t < a.S; ++t) {
                const double m = slice_res(t);
                if (m > 0.0) last = t;
                if (ts < 0 && target < acc + m) {
                    ts = t;
                    before = acc;
                }
                acc += m;
            }
            job.k = ks;
            job.slice = ts >= 0 ? ts : last;
            // past the end by rounding: the scan then falls back to the slice's last token
            // with positive residual
            job.remainder = ts >= 0 ? (float)(target - before) : INFINITY;
            job.lp = (float)((double)Mp * (double)c + log2(Sp));
            job.lq = (float)((double)Mq * (double)c + log2(Sq));
            a.next_token[ri] = -1;
        }
        a.jobs[ri] = job;
    }
}

// Inclusive prefix sum over the 64 lanes of a wave (lane order).
__device__ __forceinline__ float wave_inclusive_scan(float v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// One workgroup per particle; returns at once for particles without a residual draw.
template <int DT>
__global__ __launch_bounds__(kThreads) void k_residual(VerifyArgs a) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
    constexpr size_t ESZ = DT == SMCSD_F32 ? 4 : 2;
    __shared__ float wsum[kWaves];
    __shared__ int32_t wlast[kWaves];
    __shared__ int32_t found;
    const int64_t ri = blockIdx.x;
    const ResidualJob job = a.jobs[ri];
    if (job.k < 0) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r = ri / a.N;
    const float c = kLog2e / a.temperature[r];
    const int64_t u = ri * a.K + job.k;
    const char* zp = static_cast<const char*>(a.target) + (size_t)((ri * (a.K + 1) + job.k) * a.ld) * ESZ;
    const char* zq = static_cast<const char*>(a.draft) + (size_t)(u * a.ld) * ESZ;
    const int c0 = job.slice * a.cps;
    const int c1 = min(c0 + a.cps, a.chunks);
    if (tid == 0) found = -1;

    float base = 0.0f;     // residual mass of the slice before chunk group j
    int32_t last = -1;     // this lane's last index with positive residual
    for (int j = 0; j < kTvCPL; ++j) {
        const int ch = c0 + j * kThreads + tid;
        float rv[EPC];
        float s = 0.0f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) rv[e] = 0.0f;
        if (ch < c1) {
            const u32x4 P = *(reinterpret_cast<const u32x4*>(zp) + ch);
            const u32x4 Q = *(reinterpret_cast<const u32x4*>(zq) + ch);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                const int32_t v = ch * EPC + e;
                if (v < a.V) {
                    // log2 p(v), log2 q(v); p - q = p * (1 - 2^(lq2 - lp2)) without cancellation
                    const float lp2 = chunk_elem<DT>(P, e) * c - job.lp;
                    const float lq2 = chunk_elem<DT>(Q, e) * c - job.lq;
                    if (lp2 > lq2) {
                        rv[e] = __builtin_amdgcn_exp2f(lp2) * one_minus_exp2(lq2 - lp2);
                        if (rv[e] > 0.0f) last = v;
                    }
                }
                s += rv[e];
            }
        }
        // this lane's interval [lo, hi) of the slice's cumulative residual
        const float incl = wave_inclusive_scan(s);
        if (lane == 63) wsum[wave] = incl;
        __syncthreads();
        float wbase = 0.0f, total = 0.0f;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) wbase += wsum[w];
            total += wsum[w];
        }
        const float excl = __shfl_up(incl, 1, 64);
        const float lo = base + (wbase + (lane == 0 ? 0.0f : excl));
        const float hi = base + (wbase + incl);
        if (s > 0.0f && job.remainder >= lo && job.remainder < hi) {
            float acc = lo;
            int32_t pick = -1, lastpos = -1;
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if (rv[e] > 0.0f) lastpos = ch * EPC + e;
                acc += rv[e];
                if (pick < 0 && rv[e] > 0.0f && job.remainder < acc) pick = ch * EPC + e;
            }
            found = pick >= 0 ? pick : lastpos;
        }
        __syncthreads();
        if (found >= 0) break;
        base += total;
    }
    if (found < 0) {
        // rounding left the target past the slice's mass: its last token with residual > 0
        int32_t m = last;
        for (int d = 32; d >= 1; d >>= 1) m = max(m, __shfl_xor(m, d, 64));
        if (lane == 0) wlast[wave] = m;
        __syncthreads();
        if (tid == 0) {
            int32_t b = -1;
            for (int w = 0; w < kWaves; ++w) b = max(b, wlast[w]);
            found = b >= 0 ? b : c0 * EPC;
        }
        __syncthreads();
    }
    if (tid == 0) a.next_token[ri] = found;
}

}  // namespace

hipError_t launch_verify(int32_t R, int32_t dtype, const VerifyArgs& a, hipStream_t s) {
    if (R <= 0) return hipSuccess;
    const dim3 block(kThreads);
    if (dtype == SMCSD_BF16) k_verify_decide<SMCSD_BF16><<<dim3((unsigned)R), block, 0, s>>>(a);
    else k_verify_decide<SMCSD_F32><<<dim3((unsigned)R), block, 0, s>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid((unsigned)((int64_t)R * a.N));
    if (dtype == SMCSD_BF16) k_residual<SMCSD_BF16><<<grid, block, 0, s>>>(a);
    else k_residual<SMCSD_F32><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
