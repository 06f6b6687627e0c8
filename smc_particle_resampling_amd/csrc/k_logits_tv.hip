// k_logits_tv.hip -- the logits pass with TV on: normalisers and the per-position total
// variation of every row pair in one HBM pass (the slices of a row pair swap partials).
//   phase 1: each wave takes the maximum m of z over its own share of the slice, then
//            e = exp2((z - m) * log2e/T) and its sum, for p and q, so nothing waits between
//            the loads and the exponentials.
//   phase 2: the S workgroups of the row pair swap their (m, sum) partials and combine them
//            in one fixed order into the row's maxima M and sums S. With
//            f = exp2((m - M) * log2e/T) (m of the wave that computed the e values) the
//            |p - q| terms are (f_p / S_p) |e_p - rho e_q|, rho = (f_q S_p) / (f_p S_q).
//            The e values stay in fp32 registers from phase 1, so phase 2 costs one fma and
//            one add per element and no exponential. rho is exactly 1 when the two rows are
//            equal, and then TV is exactly 0.
// When every slice fills all its chunk groups but the last and V is a multiple of the chunk
// width, nothing is masked: a lane past the slice end re-reads an inside chunk and its
// exponentials are shifted by -inf.
//
// Launch shape. The S workgroups of a row pair must be resident together to swap partials,
// so the pass runs as a persistent cooperative grid (hipLaunchCooperativeKernel guarantees
// co-residency) over the row pairs only. It has C clusters of S consecutive workgroups (4
// chunks a lane, so the fp32 e values fit in registers), and each cluster walks the row
// pairs c, c+C, c+2C, ... in lockstep. The loads of a cluster's next row pair are issued
// while the current one is exchanged and finished. The round's bonus rows run before it, as
// an ordinary grid of the Gumbel-Top-K slice kernel, which also resets this kernel's control
// word and exchange words. A wall-clock limit bounds every wait. A workgroup that times out
// raises SMCSD_DEVERR_EXCHANGE and an abort flag, every later wait returns at once, and the
// kernel always drains.
#include <algorithm>
#include <atomic>

#include "logits_common.h"

namespace smcsd {
namespace {

// Slice exchange of the TV pass. Every (row pair, slice) partial is two 64-bit words, (max,
// sum) of the target row and of the draft row. Before the launch, every word holds kEmpty,
// a bit pattern no partial can take. A slice publishes its two words with relaxed
// agent-scope atomic stores. Wave 0 of every slice polls all 2S words of its row pair with
// relaxed agent-scope atomic loads until none is kEmpty. Each value is read from the very
// location it was stored to, so coherence of that location suffices: no release/acquire
// fences, which on this GPU would write back or invalidate a whole L2 per exchange.
constexpr uint64_t kEmpty = ~0ull;

__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ float word_lo(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float word_hi(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }

// Wave 0 only: one poll of the nwords (<= 128) words of a row pair, with the abort flag in the
// same round trip. Returns true (wave-uniform) once every word is published, the pass was
// aborted, or the wait has lasted longer than the limit (then it raises the abort flag and
// SMCSD_DEVERR_EXCHANGE). On true, lds holds the words.
__device__ bool poll_slices(const uint64_t* words, int nwords, Ctrl* ctrl, int32_t* error_flags,
                            uint64_t* lds, uint64_t t0) {
    const int lane = threadIdx.x & 63;
    const uint64_t v0 = lane < nwords
                            ? __hip_atomic_load(words + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0ull;
    const uint64_t v1 = lane + 64 < nwords
                            ? __hip_atomic_load(words + lane + 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                            : 0ull;
    // the control word: abort flag (low half) and wait limit (high half)
    uint64_t* cw = reinterpret_cast<uint64_t*>(ctrl);
    const uint64_t c = __hip_atomic_load(cw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    bool done = !__any(v0 == kEmpty || v1 == kEmpty) || (uint32_t)c != 0;
    if (!done && wall_clock64() - t0 > (c >> 32)) {
        if (lane == 0) {
            __hip_atomic_store(cw, (c & 0xFFFFFFFF00000000ull) | 1ull, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
            flag_error(error_flags, SMCSD_DEVERR_EXCHANGE);
        }
        done = true;
    }
    if (done) {
        if (lane < nwords) lds[lane] = v0;
        if (lane + 64 < nwords) lds[lane + 64] = v1;
    }
    return done;
}

// The -inf padding of one workgroup's slice, fixed for the whole persistent loop (every row
// has the same length): which chunk groups run past the slice end (a uniform bit per group),
// whether this lane's chunk of such a group lies inside, and which lane holds the row's
// partial tail chunk, if any. Applying it is one select per word of a partial group.
template <int DT, int CPL>
struct SliceMask {
    uint32_t partial;      // bit j: chunk group j has lanes past the slice end (uniform)
    bool inside[CPL];      // this lane's chunk of group j is inside the slice
    bool has_tail;         // the slice holds the row's last chunk and V is not a multiple of
                           // the chunk width (uniform)
    int tail_j;            // chunk group of that chunk if this lane holds it, else -1
    uint32_t keep[4];      // per word of the tail chunk: bits kept (uniform)

    // Fast path: the slice fills every chunk group but the last and holds no partial tail
    // chunk. Then nothing is masked: a lane past the slice end in the last group re-reads the
    // slice's last chunk (its byte offset voff_last), which leaves every maximum unchanged,
    // and its exponentials get a shift of -inf (last_inside false), so they are 0.
    bool last_inside;      // this lane's chunk of the last group lies inside the slice
    int voff_last;         // byte offset of this lane's load in the last group

    __device__ __forceinline__ SliceMask(int c0, int c1, int V) {
        constexpr int EPC = Elem<DT>::EPC;
        const int tid = threadIdx.x;
        const int n = c1 - c0;
        partial = 0;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            if ((j + 1) * kThreads > n) partial |= 1u << j;
            inside[j] = j * kThreads + tid < n;
        }
        has_tail = (int64_t)c1 * EPC > V;
        tail_j = -1;
        const int nv = V - (c1 - 1) * EPC;   // valid elements of the last chunk
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (DT == SMCSD_F32) keep[w] = w < nv ? 0xFFFFFFFFu : 0u;
            else keep[w] = 2 * w + 1 < nv ? 0xFFFFFFFFu : 2 * w < nv ? 0x0000FFFFu : 0u;
        }
        if (has_tail) {
            const int last = c1 - 1 - c0;
            if (last % kThreads == tid) tail_j = last / kThreads;
        }
        constexpr int kLast = (CPL - 1) * kThreads;   // first chunk of the last group
        const bool fast = n > kLast && !has_tail;
        last_inside = kLast + tid < n;
        voff_last = ((fast ? min(kLast + tid, n - 1) : kLast + tid) - kLast) * 16;
    }

    // -inf bits are exactly the complement of the kept bits within each element, so the
    // padding is (x & keep) | (kNegInf & ~keep)
    __device__ __forceinline__ void apply(u32x4 (&R)[CPL]) const {
        const uint32_t ni = Elem<DT>::kNegInf;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (partial & (1u << j)) {
#pragma unroll
                for (int w = 0; w < 4; ++w) R[j][w] = inside[j] ? R[j][w] : ni;
            }
        if (has_tail) {
#pragma unroll
            for (int j = 0; j < CPL; ++j)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    const uint32_t m = (R[j][w] & keep[w]) | (ni & ~keep[w]);
                    R[j][w] = tail_j == j ? m : R[j][w];
                }
        }
    }
};

// The rows of row pair u: with g = u / K (request * N + particle) and k = u - g * K, the
// target row is g * (K + 1) + k = u + g and the draft row is u. Row pairs number fewer than
// 2^31 (the grid bound of the plan), so 32-bit division suffices.
template <int DT>
__device__ __forceinline__ void pair_rows(const LogitsArgs& a, uint32_t u, int c0, const char*& zp,
                                          const char*& zq) {
    constexpr size_t ESZ = Elem<DT>::ESZ;
    const uint32_t g = u / (uint32_t)a.K;
    zp = static_cast<const char*>(a.target) + ((size_t)(u + g) * a.ld + (size_t)c0 * Elem<DT>::EPC) * ESZ;
    zq = static_cast<const char*>(a.draft) + ((size_t)u * a.ld + (size_t)c0 * Elem<DT>::EPC) * ESZ;
}

// Issue the loads of this lane's chunks of the slice that starts at `row` (c0 already
// applied) and holds n chunks. voff_last is the lane's byte offset within the last chunk
// group (SliceMask::voff_last).
template <int CPL>
__device__ __forceinline__ void issue_at(u32x4 (&R)[CPL], const char* row, int n, int voff_last) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(row), 0, n * 16,
                                                                       kRsrcWord3);
    const int voff = (int)threadIdx.x * 16;
#pragma unroll
    for (int j = 0; j < CPL - 1; ++j)
        R[j] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, j * kThreads * 16, kLoadNontemporal);
    R[CPL - 1] = __builtin_amdgcn_raw_buffer_load_b128(r, voff_last, (CPL - 1) * kThreads * 16,
                                                       kLoadNontemporal);
}

// LDS of the TV pass: the wave partials (max p, sum p, max q, sum q) of the current row pair,
// its exchange words and the row sums wave 0 makes of them, and the previous row pair's
// per-wave sums of |p - q|. Reuse by the next row pair needs no third barrier: wave 0 reads
// wpart and xch before the exchange barrier, and the next row pair rewrites them only after
// that barrier; wave 0 rewrites norm only after the next row pair's first barrier, which
// every wave reaches after its last read of norm; tvw is written at the end of a row pair,
// read by wave 0 between the next row pair's two barriers and rewritten after the second.
struct TvLds {
    float4 wpart[kWaves];
    uint64_t xch[2 * kMaxTvSlices];
    float4 norm;   // the row pair's (max p, sum p, max q, sum q), from wave 0
    float tvw[kWaves];
};

// The slice's share of sum |p - q| of row pair u: the eight wave sums in wave order, one
// float per (row pair, slice) in a.tvp. Called by one whole wave; lane 0 stores.
__device__ __forceinline__ void store_slice_tv(const LogitsArgs& a, const TvLds& sh, uint32_t u, int s) {
    float t = sh.tvw[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) t += sh.tvw[w];
    if ((threadIdx.x & 63) == 0) a.tvp[(size_t)u * a.S + s] = t;
}

// TV on: partials, exchange, and this slice's share of sum |p - q|, one partial per wave.
// Each wave shifts its exponentials by the maximum of its own share of the slice, so nothing
// waits between the loads and the exponentials; wave 0 combines the eight wave partials into
// the slice partial it publishes, and in phase 2 each wave scales its terms by its own
// f = exp2((m_wave - M_row) c). P and Q hold this slice's loads, issued one row pair earlier;
// as soon as a chunk group's values are exponentials, the loads of row pair `next` go into
// that group's registers, in flight during the rest of phase 1, the exchange and phase 2.
// Two barriers per row pair: wave partials, exchange words. Wave 0 stores the previous row
// pair's share of sum |p - q| (prev; -1: none) right after it publishes (measured 1% faster
// there than in wave 1 or wave 7 during the wait, and than one store per wave).

template <int DT, bool kFast>
__device__ void pair_slice_tv(const LogitsArgs& a, uint32_t u, int s, int64_t prev, int64_t next,
                              const SliceMask<DT, kTvCPL>& mask, int c0, int n, u32x4 (&P)[kTvCPL],
                              u32x4 (&Q)[kTvCPL], TvLds& sh, uint32_t& r_lo, float& c_r,
                              float& early_mp, float& early_mq) {
    constexpr int NE = kTvCPL * Elem<DT>::EPC;
    constexpr int EPC = Elem<DT>::EPC;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    // log2(e)/T, divided once per request (row pairs of one request follow each other):
    // r_lo is the first row pair of the request c_r belongs to
    const uint32_t nk = (uint32_t)a.N * (uint32_t)a.K;
    if (u - r_lo >= nk) {
        const uint32_t r = u / nk;
        r_lo = r * nk;
        c_r = kLog2e / load_constant(a.temperature, r);
    }
    const float c = c_r;
    float Ep[NE], Eq[NE];
    // Wave priority: highest until this slice's partials are published (the other slices of
    // the row pair wait for them), lowest while polling, in between after the exchange (that
    // work delays only this slice's next publish). Without it the pass took 7% longer.
    __builtin_amdgcn_s_setprio(3);
    // The padding is applied to copies, so that P and Q stay the registers the next row
    // pair's loads land in (in-place masking made the compiler copy them back, 32 moves).
    u32x4 Pm[kTvCPL], Qm[kTvCPL];
#pragma unroll
    for (int j = 0; j < kTvCPL; ++j) {
        Pm[j] = P[j];
        Qm[j] = Q[j];
    }
    if constexpr (!kFast) {
        mask.apply(Pm);
        mask.apply(Qm);
    }
    // the wave maxima, unless this wave took them while it waited for the previous row
    // pair's exchange (early_mp is NaN when it did not)
    const bool have_early = kFast && early_mp == early_mp;
    const float mpw = have_early ? early_mp : wave_share_max<DT, kTvCPL>(Pm);
    const float mqw = have_early ? early_mq : wave_share_max<DT, kTvCPL>(Qm);
    // The next row pair's loads go into P and Q chunk group by chunk group, each right after
    // the group's exponentials: early, without copies of the registers they overwrite, and
    // without a branch (with no next row pair the buffer range is empty and the loads read
    // nothing), so the order below holds.
    const char *zpn, *zqn;
    pair_rows<DT>(a, next >= 0 ? (uint32_t)next : u, c0, zpn, zqn);
    const int nn = next >= 0 ? n * 16 : 0;
    const __amdgpu_buffer_rsrc_t rp = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(zpn), 0, nn, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(zqn), 0, nn, kRsrcWord3);
    const int voff = tid * 16;
    float s0 = 0.0f, s1 = 0.0f, q0 = 0.0f, q1 = 0.0f;
    {
        const float nmp = mpw == -INFINITY ? 0.0f : -mpw * c;
        const float nmq = mqw == -INFINITY ? 0.0f : -mqw * c;
        // fast path: the re-read chunk of a lane past the slice end contributes exp2(-inf) = 0
        const float nmp_last = !kFast || mask.last_inside ? nmp : -INFINITY;
        const float nmq_last = !kFast || mask.last_inside ? nmq : -INFINITY;
#pragma unroll
        for (int j = 0; j < kTvCPL; ++j) {
            const float np = j == kTvCPL - 1 ? nmp_last : nmp;
            const float nq = j == kTvCPL - 1 ? nmq_last : nmq;
#pragma unroll
            for (int e = 0; e < EPC; e += 2) {
                const int x = j * EPC + e;
                Ep[x] = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Pm[j], e), c, np));
                Ep[x + 1] = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Pm[j], e + 1), c, np));
                Eq[x] = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Qm[j], e), c, nq));
                Eq[x + 1] = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Qm[j], e + 1), c, nq));
                s0 += Ep[x];
                s1 += Ep[x + 1];
                q0 += Eq[x];
                q1 += Eq[x + 1];
            }
            const int vo = j == kTvCPL - 1 ? mask.voff_last : voff;
            P[j] = __builtin_amdgcn_raw_buffer_load_b128(rp, vo, j * kThreads * 16, kLoadNontemporal);
            Q[j] = __builtin_amdgcn_raw_buffer_load_b128(rq, vo, j * kThreads * 16, kLoadNontemporal);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const float spw = wave_sum(s0 + s1), sqw = wave_sum(q0 + q1);
    if (lane == 0) sh.wpart[w] = make_float4(mpw, spw, mqw, sqw);
    __syncthreads();
    if (tid < 64) {
        const float4 wpv = lane < kWaves ? sh.wpart[lane] : make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
        const float mp = readlane_f32(row_max(wpv.x), 0);
        const float mq = readlane_f32(row_max(wpv.z), 0);
        // a wave whose share is all -inf holds (-inf, 0): it adds 0, also when the whole slice
        // is -inf (mp = -inf would make its scale exp2(NaN))
        const float sp = readlane_f32(
            row_sum(wpv.x == -INFINITY ? 0.0f : wpv.y * __builtin_amdgcn_exp2f((wpv.x - mp) * c)), 0);
        const float sq = readlane_f32(
            row_sum(wpv.z == -INFINITY ? 0.0f : wpv.w * __builtin_amdgcn_exp2f((wpv.z - mq) * c)), 0);
        uint64_t* words = reinterpret_cast<uint64_t*>(a.pp + (size_t)u * a.S);
        if (lane == 0) {
            __hip_atomic_store(words + 2 * s, pack2(mp, sp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(words + 2 * s + 1, pack2(mq, sq), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        __builtin_amdgcn_s_setprio(0);
        // the previous row pair's share of sum |p - q|, while the other slices publish
        if (prev >= 0) store_slice_tv(a, sh, (uint32_t)prev, s);
        const uint64_t t0 = wall_clock64();
        while (!poll_slices(words, 2 * a.S, a.ctrl, a.error_flags, sh.xch, t0)) __builtin_amdgcn_s_sleep(1);
        // the row maxima and sums from the S slice partials, once for the workgroup: lane t
        // holds slice t (lanes without a slice hold (-inf, 0), which adds nothing)
        const uint64_t kNone = pack2(-INFINITY, 0.0f);
        const uint64_t wp = lane < a.S ? sh.xch[2 * lane] : kNone;
        const uint64_t wq = lane < a.S ? sh.xch[2 * lane + 1] : kNone;
        float Mp, Mq, Sp, Sq;
        if (a.S <= 16) {
            Mp = readlane_f32(row_max(word_lo(wp)), 0);
            Mq = readlane_f32(row_max(word_lo(wq)), 0);
            Sp = readlane_f32(row_sum(word_hi(wp) * __builtin_amdgcn_exp2f((word_lo(wp) - Mp) * c)), 0);
            Sq = readlane_f32(row_sum(word_hi(wq) * __builtin_amdgcn_exp2f((word_lo(wq) - Mq) * c)), 0);
        } else {
            Mp = wave_max(word_lo(wp));
            Mq = wave_max(word_lo(wq));
            Sp = wave_sum(word_hi(wp) * __builtin_amdgcn_exp2f((word_lo(wp) - Mp) * c));
            Sq = wave_sum(word_hi(wq) * __builtin_amdgcn_exp2f((word_lo(wq) - Mq) * c));
        }
        if (lane == 0) sh.norm = make_float4(Mp, Sp, Mq, Sq);
    }
    // Waves 1..7 would only wait here while wave 0 takes the exchange: they take the next
    // row pair's wave maxima now (its loads are in P and Q), which moves 2 x 29 of their
    // instructions per row pair off the path to the next publish. Wave 0 keeps its own in
    // phase 1: taken here they would delay the exchange barrier for everyone (measured
    // slower). With the mask-free slices only (masking would need copies held until then).
    early_mp = early_mq = __builtin_nanf("");
    if (kFast && tid >= 64 && next >= 0) {
        early_mp = wave_share_max<DT, kTvCPL>(P);
        early_mq = wave_share_max<DT, kTvCPL>(Q);
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(1);
    const float4 nrm = sh.norm;
    const float Mp = nrm.x, Sp = nrm.y, Mq = nrm.z, Sq = nrm.w;
    const float fp = __builtin_amdgcn_exp2f((mpw - Mp) * c);
    const float fq = __builtin_amdgcn_exp2f((mqw - Mq) * c);
    const bool p_major = fp * Sq >= fq * Sp;
    const float num = p_major ? fq * Sp : fp * Sq;
    const float den = p_major ? fp * Sq : fq * Sp;
    // equal rows: rho exactly 1, so TV is exactly 0 (a reciprocal would not give that)
    const float rho = num == den ? 1.0f : den > 0.0f ? num * __builtin_amdgcn_rcpf(den) : 0.0f;
    const float scale = p_major ? fp * __builtin_amdgcn_rcpf(Sp) : fq * __builtin_amdgcn_rcpf(Sq);
    float acc0 = 0.0f, acc1 = 0.0f;
    if (p_major) {
#pragma unroll
        for (int e = 0; e < NE; e += 2) {
            acc0 += fabsf(fmaf(-rho, Eq[e], Ep[e]));
            acc1 += fabsf(fmaf(-rho, Eq[e + 1], Ep[e + 1]));
        }
    } else {
#pragma unroll
        for (int e = 0; e < NE; e += 2) {
            acc0 += fabsf(fmaf(-rho, Ep[e], Eq[e]));
            acc1 += fabsf(fmaf(-rho, Ep[e + 1], Eq[e + 1]));
        }
    }
    const float acc = wave_sum(acc0 + acc1);
    if (lane == 0) sh.tvw[w] = acc * scale;
}

// TV on: persistent cooperative grid, gridDim.x = C * S. kFast: every slice takes the fast
// path of SliceMask (chosen on the host by tv_fast_path).
template <int DT, bool kFast>
__global__ __launch_bounds__(kThreads, 4) void k_logits_tv(LogitsArgs a) {
    __shared__ TvLds sh;
    const int s = (int)(blockIdx.x % (unsigned)a.S);
    const int64_t C = gridDim.x / (unsigned)a.S;
    const int64_t cluster = blockIdx.x / (unsigned)a.S;
    if (cluster >= a.pairs) return;
    const int c0 = s * a.cps;
    const int c1 = min(c0 + a.cps, a.chunks);
    const SliceMask<DT, kTvCPL> mask(c0, c1, a.V);
    u32x4 P[kTvCPL], Q[kTvCPL];
    {
        const char *zp, *zq;
        pair_rows<DT>(a, (uint32_t)cluster, c0, zp, zq);
        issue_at<kTvCPL>(P, zp, c1 - c0, mask.voff_last);
        issue_at<kTvCPL>(Q, zq, c1 - c0, mask.voff_last);
    }
    const uint32_t nk = (uint32_t)a.N * (uint32_t)a.K;
    uint32_t r_lo = (uint32_t)cluster / nk * nk;   // first row pair of the current request
    float c_r = kLog2e / load_constant(a.temperature, (uint32_t)cluster / nk);
    float early_mp = __builtin_nanf(""), early_mq = __builtin_nanf("");
    int64_t it = cluster;
    for (; it < a.pairs; it += C)
        pair_slice_tv<DT, kFast>(a, (uint32_t)it, s, it - C, it + C < a.pairs ? it + C : -1, mask,
                                 c0, c1 - c0, P, Q, sh, r_lo, c_r, early_mp, early_mq);
    // the last row pair's share of sum |p - q|
    __syncthreads();
    if (threadIdx.x < 64) store_slice_tv(a, sh, (uint32_t)(it - C), s);
}

// Before a TV pass without bonus rows: the control word (abort flag 0, the wait limit) and
// every exchange word at the all-ones "empty" pattern, in one launch; with lw_n > 0 also the
// copy of the previous log-weights (LogitsArgs::lw_src).
__global__ void k_fill_tv(Ctrl* ctrl, uint32_t timeout, uint32_t* words, int64_t n, const float* lw_src,
                          float* lw_copy, int32_t lw_n) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *ctrl = Ctrl{0u, timeout};
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < lw_n; i += (int64_t)gridDim.x * blockDim.x)
        lw_copy[i] = lw_src[i];
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        words[i] = ~0u;
}

}  // namespace

// Whether every slice of the plan takes SliceMask's fast path: each fills all chunk groups
// but the last, and V is a multiple of the chunk width (no partial tail chunk).
static bool tv_fast_path(const Plan& plan) {
    const int32_t last = plan.chunks - (plan.S - 1) * plan.cps;   // the last slice's chunks
    return plan.V % plan.epc == 0 && last > (kTvCPL - 1) * kThreads;
}

// Workgroups of k_logits_tv<DT, kFast> that fit on the current device at once (cached per
// device).
template <int DT, bool kFast>
static int64_t coop_capacity() {
    static std::atomic<int64_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int per_cu = 0, cus = 0, coop = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_logits_tv<DT, kFast>),
                                                     kThreads, 0) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop)
        return 0;
    const int64_t c = (int64_t)per_cu * cus;
    if (dev < 64) cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

hipError_t launch_tv_fill(const Plan& plan, const LogitsArgs& a, uint32_t timeout, hipStream_t s) {
    const int64_t n = (int64_t)(plan.pair_wgs * sizeof(PairPart) / 4);
    const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>((n + kThreads - 1) / kThreads, 1024));
    k_fill_tv<<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(a.ctrl, timeout,
                                                               reinterpret_cast<uint32_t*>(a.pp), n, a.lw_src,
                                                               a.lw_copy, a.lw_n);
    return hipGetLastError();
}

// The row pairs only: the round hands the bonus rows to the Gumbel-Top-K slice kernel.
template <int DT, bool kFast>
static hipError_t launch_tv(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    const int64_t cap = coop_capacity<DT, kFast>();
    const int64_t clusters = std::min<int64_t>(cap / plan.S, plan.pairs);
    if (clusters < 1) return hipErrorCooperativeLaunchTooLarge;
    LogitsArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_logits_tv<DT, kFast>),
                                      dim3((unsigned)(clusters * plan.S)), dim3(kThreads), params, 0, s);
}

hipError_t launch_logits_tv(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    const bool fast = tv_fast_path(plan);
    if (plan.dtype == SMCSD_BF16)
        return fast ? launch_tv<SMCSD_BF16, true>(plan, a, s) : launch_tv<SMCSD_BF16, false>(plan, a, s);
    return fast ? launch_tv<SMCSD_F32, true>(plan, a, s) : launch_tv<SMCSD_F32, false>(plan, a, s);
}

}  // namespace smcsd
