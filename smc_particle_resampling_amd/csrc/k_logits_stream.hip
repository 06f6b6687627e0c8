// k_logits_stream.hip -- the logits pass with TV off: every (row, slice) is an independent
// workgroup of an ordinary grid, 4 chunks a lane. A row-pair slice reduces the target and the
// draft row to their slice partials (max, sum of exp2((z - m) * log2e/T)); a bonus slice
// reduces a bonus row and its noise row to the slice's Gumbel-max (key, index). Each wave
// shifts its exponentials by the maximum of its own share of the slice, so nothing waits
// between the loads and the exponentials; wave 0 combines the eight wave partials.
#include "logits_common.h"

namespace smcsd {
namespace {

struct PairLoc {
    int64_t r;
    const char* zp;
    const char* zq;
    int c0, c1;
};

template <int DT>
__device__ __forceinline__ PairLoc pair_location(const LogitsArgs& a, int64_t u, int s) {
    constexpr size_t ESZ = Elem<DT>::ESZ;
    const int64_t nk = (int64_t)a.N * a.K;
    const int64_t r = u / nk;
    const int64_t ik = u - r * nk;
    const int64_t i = ik / a.K;
    const int64_t k = ik - i * a.K;
    PairLoc L;
    L.r = r;
    L.zp = static_cast<const char*>(a.target) + (size_t)(((r * a.N + i) * (a.K + 1) + k) * a.ld) * ESZ;
    L.zq = static_cast<const char*>(a.draft) + (size_t)(((r * a.N + i) * a.K + k) * a.ld) * ESZ;
    L.c0 = s * a.cps;
    L.c1 = min(L.c0 + a.cps, a.chunks);
    return L;
}

// Every lane of each 16-lane row ends with the row's best (key, index), as in row_max.
__device__ __forceinline__ void argmax_step(float& k, int32_t& i, float ok, int32_t oi) {
    if (better(ok, oi, k, i)) {
        k = ok;
        i = oi;
    }
}
__device__ __forceinline__ void row_argmax(float& k, int32_t& i) {
    argmax_step(k, i, dpp_f32<kDppXor1>(k), dpp_i32<kDppXor1>(i));
    argmax_step(k, i, dpp_f32<kDppXor2>(k), dpp_i32<kDppXor2>(i));
    argmax_step(k, i, dpp_f32<kDppRowHalfMirror>(k), dpp_i32<kDppRowHalfMirror>(i));
    argmax_step(k, i, dpp_f32<kDppRowMirror>(k), dpp_i32<kDppRowMirror>(i));
}

// Bonus rows. A workgroup handles slice s of a bonus row two chunks per lane at a time (a
// "piece"). key = z/T + G with one
// rounding; -inf for positions outside the slice or >= V. A lane visits its indices in
// increasing order, so the strict comparison keeps the lowest index among equal keys.
struct BonusRow {
    const char* zrow;
    const char* grow;
    float invT;
    int c0, c1;
};

template <int DT>
__device__ __forceinline__ BonusRow bonus_row(const LogitsArgs& a, int64_t b, int s) {
    constexpr size_t ESZ = Elem<DT>::ESZ;
    BonusRow B;
    B.zrow = static_cast<const char*>(a.target) + (size_t)((b * (a.K + 1) + a.K) * a.ld) * ESZ;
    B.grow = reinterpret_cast<const char*>(a.gumbel + (size_t)b * a.ld);
    B.invT = __fdiv_rn(1.0f, load_constant(a.temperature, b / a.N));
    B.c0 = s * a.cps;
    B.c1 = min(B.c0 + a.cps, a.chunks);
    return B;
}

// Chunk groups j0 and j0 + 1 of this lane (two chunks keep the noise, twice the bytes of
// the logits, from piling up in registers).
template <int DT>
__device__ __forceinline__ void bonus_piece(const LogitsArgs& a, const BonusRow& B, int j0,
                                            float& best, int32_t& besti) {
    constexpr int EPC = Elem<DT>::EPC;
    const int tid = threadIdx.x;
    u32x4 Z[2];
    u32x4 g[2][EPC / 4];
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int ch = B.c0 + (j0 + jj) * kThreads + tid;
        const uint32_t ni = Elem<DT>::kNegInf;
        Z[jj] = u32x4{ni, ni, ni, ni};
#pragma unroll
        for (int h = 0; h < EPC / 4; ++h) g[jj][h] = u32x4{0u, 0u, 0u, 0u};
        if (ch < B.c1) {
            Z[jj] = load_chunk(B.zrow, ch);
#pragma unroll
            for (int h = 0; h < EPC / 4; ++h) g[jj][h] = load_chunk(B.grow, (int64_t)ch * (EPC / 4) + h);
            const int nv = a.V - ch * EPC;
            if (nv < EPC) Z[jj] = mask_tail<DT>(Z[jj], nv);
        }
    }
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
        const int ch = B.c0 + (j0 + jj) * kThreads + tid;
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            const float key = fmaf(chunk_elem<DT>(Z[jj], e), B.invT, __uint_as_float(g[jj][e >> 2][e & 3]));
            const bool win = key > best;
            best = win ? key : best;
            besti = win ? ch * EPC + e : besti;
        }
    }
}

// Block argmax of the lanes' (key, index) and its store. (key, index) with the lower index
// winning ties is a total order, so the result does not depend on the order of the steps.
__device__ void bonus_finish(const LogitsArgs& a, int64_t b, int s, float best, int32_t besti,
                             float* red, int32_t* redi) {
    const int tid = threadIdx.x;
    row_argmax(best, besti);
    float k = readlane_f32(best, 0);
    int32_t i = __builtin_amdgcn_readlane(besti, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16) {
        const float ok = readlane_f32(best, r);
        const int32_t oi = __builtin_amdgcn_readlane(besti, r);
        if (better(ok, oi, k, i)) {
            k = ok;
            i = oi;
        }
    }
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        red[w] = k;
        redi[w] = i;
    }
    __syncthreads();
    if (tid == 0) {
        for (int t = 1; t < kWaves; ++t)
            if (better(red[t], redi[t], k, i)) {
                k = red[t];
                i = redi[t];
            }
        a.bp[b * a.S + s] = BonusPart{k, i};
    }
    __syncthreads();   // red / redi are reused by the next call
}

template <int DT, int CPL>
__device__ void bonus_slice(const LogitsArgs& a, int64_t b, int s, float* red, int32_t* redi) {
    const BonusRow B = bonus_row<DT>(a, b, s);
    float best = -INFINITY;
    int32_t besti = INT32_MAX;
#pragma unroll 1
    for (int j0 = 0; j0 < CPL; j0 += 2) bonus_piece<DT>(a, B, j0, best, besti);
    bonus_finish(a, b, s, best, besti, red, redi);
}
// TV off: slice partials only. Each wave shifts its exponentials by the maximum of its own
// share (no barrier between the loads and the exponentials); wave 0 combines the eight wave
// partials into the slice partial after the one barrier.
template <int DT>
__device__ void pair_slice_stream(const LogitsArgs& a, int64_t u, int s, float4* wpart) {
    const PairLoc L = pair_location<DT>(a, u, s);
    const float c = kLog2e / load_constant(a.temperature, L.r);   // exp(z/T) = exp2(z * c)
    const int lane = threadIdx.x & 63;
    u32x4 P[kStreamCPL], Q[kStreamCPL];
    issue_slice<kStreamCPL>(P, L.zp, L.c0, L.c1);
    issue_slice<kStreamCPL>(Q, L.zq, L.c0, L.c1);
    mask_slice<DT, kStreamCPL>(P, L.c0, L.c1, a.V);
    mask_slice<DT, kStreamCPL>(Q, L.c0, L.c1, a.V);
    const float mpw = wave_share_max<DT, kStreamCPL>(P);
    const float mqw = wave_share_max<DT, kStreamCPL>(Q);
    // a wave whose share is all padding has maximum -inf: shift 0, so its terms are 0
    const float spw = wave_sum(slice_sumexp<DT, kStreamCPL>(P, c, mpw == -INFINITY ? 0.0f : -mpw * c));
    const float sqw = wave_sum(slice_sumexp<DT, kStreamCPL>(Q, c, mqw == -INFINITY ? 0.0f : -mqw * c));
    if (lane == 0) wpart[threadIdx.x >> 6] = make_float4(mpw, spw, mqw, sqw);
    __syncthreads();
    if (threadIdx.x < 64) {
        const float4 wpv = lane < kWaves ? wpart[lane] : make_float4(-INFINITY, 0.0f, -INFINITY, 0.0f);
        const float mp = readlane_f32(row_max(wpv.x), 0);
        const float mq = readlane_f32(row_max(wpv.z), 0);
        // a wave whose share is all -inf holds (-inf, 0): it adds 0, also when the whole slice
        // is -inf (mp = -inf would make its scale exp2(NaN))
        const float sp = readlane_f32(
            row_sum(wpv.x == -INFINITY ? 0.0f : wpv.y * __builtin_amdgcn_exp2f((wpv.x - mp) * c)), 0);
        const float sq = readlane_f32(
            row_sum(wpv.z == -INFINITY ? 0.0f : wpv.w * __builtin_amdgcn_exp2f((wpv.z - mq) * c)), 0);
        if (lane == 0) a.pp[u * a.S + s] = PairPart{mp, sp, mq, sq};
    }
}

// TV off: one workgroup per (row, slice).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_logits_stream(LogitsArgs a) {
    __shared__ float red[kWaves];
    __shared__ int32_t redi[kWaves];
    __shared__ float4 wpart[kWaves];
    // the bonus slices (a logits row and its noise row, 1.5 times a row pair's bytes) are
    // dispatched first, so that the grid's tail holds the lighter row-pair slices
    const int64_t t = blockIdx.x;
    const int64_t bonus_wgs = a.total_wgs - a.pair_wgs;
    // the previous log-weights, for a finalize that overwrites them while other workgroups of
    // the request still read them (a grid-stride copy, nothing for most workgroups)
    for (int64_t i = t * kThreads + threadIdx.x; i < a.lw_n; i += (int64_t)gridDim.x * kThreads)
        a.lw_copy[i] = a.lw_src[i];
    if (t < bonus_wgs) {
        bonus_slice<DT, kStreamCPL>(a, t / a.S, (int)(t % a.S), red, redi);
    } else if (t < a.total_wgs) {
        const int64_t tp = t - bonus_wgs;
        pair_slice_stream<DT>(a, tp / a.S, (int)(tp % a.S), wpart);
    }
}

}  // namespace

hipError_t launch_logits_stream(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    const dim3 grid((unsigned)plan.total_wgs), block(kThreads);
    if (plan.dtype == SMCSD_BF16) k_logits_stream<SMCSD_BF16><<<grid, block, 0, s>>>(a);
    else k_logits_stream<SMCSD_F32><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
