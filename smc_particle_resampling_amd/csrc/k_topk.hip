// k_topk.hip -- Gumbel-Top-K: k tokens drawn without replacement from softmax(z/T) in one
// step, as the STAND page describes for drafting (method item 2): add precomputed, cached
// Gumbel noise to the log-probabilities and keep the indices of the k largest sums. Adding
// the row's normaliser to every key changes no ranking, so the keys are the bonus token's,
// key_v = fl32(fma(z_v, fl32(1/T), G_v)), ranked by decreasing key and then increasing index
// (a total order, so the selection is exact and deterministic).
//
// Pass 1: one 512-thread workgroup per (row, slice), 4 chunks a lane as in the TV pass. Each
// lane holds its keys in registers and its own best; k rounds of a block argmax over the
// lanes' bests pick the slice's k best, and only the lane that lost its best rescans. Pass 2:
// one workgroup per row takes the S * k candidates the same way.
#include "smcsd_device.h"

namespace smcsd {
namespace {

__device__ __forceinline__ void argmax_step(float& k, int32_t& i, float ok, int32_t oi) {
    if (better(ok, oi, k, i)) {
        k = ok;
        i = oi;
    }
}

// Block argmax of every lane's (key, index); all threads get the winner. lds holds 2 *
// kWaves entries per buffer; callers alternate buffers between rounds, so one barrier per
// round suffices.
__device__ __forceinline__ void block_argmax(float& k, int32_t& i, float* lk, int32_t* li) {
    argmax_step(k, i, dpp_f32<kDppXor1>(k), dpp_i32<kDppXor1>(i));
    argmax_step(k, i, dpp_f32<kDppXor2>(k), dpp_i32<kDppXor2>(i));
    argmax_step(k, i, dpp_f32<kDppRowHalfMirror>(k), dpp_i32<kDppRowHalfMirror>(i));
    argmax_step(k, i, dpp_f32<kDppRowMirror>(k), dpp_i32<kDppRowMirror>(i));
    float bk = readlane_f32(k, 0);
    int32_t bi = __builtin_amdgcn_readlane(i, 0);
#pragma unroll
    for (int r = 16; r < 64; r += 16)
        argmax_step(bk, bi, readlane_f32(k, r), __builtin_amdgcn_readlane(i, r));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        lk[w] = bk;
        li[w] = bi;
    }
    __syncthreads();
    bk = lk[0];
    bi = li[0];
    for (int t = 1; t < kWaves; ++t) argmax_step(bk, bi, lk[t], li[t]);
    k = bk;
    i = bi;
}

// The lane's best among n (key, index) pairs held in registers.
template <int n>
__device__ __forceinline__ void lane_best(const float (&key)[n], const int32_t (&idx)[n], float& bk,
                                          int32_t& bi) {
    bk = -INFINITY;
    bi = INT32_MAX;
#pragma unroll
    for (int e = 0; e < n; ++e) argmax_step(bk, bi, key[e], idx[e]);
}

// k rounds of selection over keys held in registers; writes the winners to out (k entries).
template <int n>
__device__ __forceinline__ void select_k(float (&key)[n], int32_t (&idx)[n], int k,
                                         BonusPart* out, float* lk, int32_t* li) {
    float bk;
    int32_t bi;
    lane_best<n>(key, idx, bk, bi);
    for (int it = 0; it < k; ++it) {
        float wk = bk;
        int32_t wi = bi;
        const int buf = (it & 1) * kWaves;
        block_argmax(wk, wi, lk + buf, li + buf);
        if (threadIdx.x == 0) out[it] = BonusPart{wk, wk == -INFINITY ? INT32_MAX : wi};
        if (bi == wi && bk != -INFINITY) {
            // this lane held the winner: drop it and rescan
#pragma unroll
            for (int e = 0; e < n; ++e)
                if (idx[e] == wi) key[e] = -INFINITY;
            lane_best<n>(key, idx, bk, bi);
        }
    }
}

// The lane's best position among n keys whose indices increase with the position: the first
// position holding the maximum (-1 if every key is -inf).
template <int n>
__device__ __forceinline__ int lane_best_pos(const float (&key)[n], float& bk) {
    float m = key[0];
#pragma unroll
    for (int e = 1; e < n; ++e) m = fmaxf(m, key[e]);
    int pos = -1;
#pragma unroll
    for (int e = n - 1; e >= 0; --e) pos = key[e] == m ? e : pos;
    bk = m;
    return m == -INFINITY ? -1 : pos;
}

// MODE is TopkArgs::row_mode as a template parameter, so the plain kernel carries none of the
// row-map arithmetic. 8 waves per SIMD (4 workgroups per CU) are asked for explicitly: the
// row map had raised the SGPR count enough to cost one, and the pass 10%.
template <int DT, int MODE>
__global__ __launch_bounds__(kThreads, 8) void k_topk_slice(TopkArgs a) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
    constexpr size_t ESZ = DT == SMCSD_F32 ? 4 : 2;
    constexpr int n = kTopkCPL * EPC;
    __shared__ float lk[2 * kWaves];
    __shared__ int32_t li[2 * kWaves];
    const uint32_t row32 = blockIdx.x / (unsigned)a.S;   // rows * S < 2^31
    const int64_t row = row32;
    const int s = (int)(blockIdx.x % (unsigned)a.S);
    const int tid = threadIdx.x;
    int64_t lrow = row, trow = row;
    if constexpr (MODE != kTopkRows) {
        const uint32_t r = row32 / (uint32_t)a.N;         // the request
        uint32_t src = row32;                              // its particle row
        if constexpr (MODE == kTopkResampled) {
            const int32_t x = a.ancestors[row];
            if (x < 0 || x >= a.N) return;   // the merge writes -1 for this row
            src = r * (uint32_t)a.N + (uint32_t)x;
        }
        trow = r;
        lrow = (int64_t)src * (a.K + 1) + a.K;
    }
    if constexpr (MODE == kTopkBonusRows) {
        if (a.fill_words) {
            if (blockIdx.x == 0 && tid == 0) *a.ctrl = Ctrl{0u, a.timeout};
            for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.lw_n; i += (int64_t)gridDim.x * kThreads)
                a.lw_copy[i] = a.lw_src[i];
            for (int64_t i = (int64_t)blockIdx.x * kThreads + tid; i < a.fill_n;
                 i += (int64_t)gridDim.x * kThreads)
                a.fill_words[i] = ~0u;
        }
    }
    const char* zrow = static_cast<const char*>(a.logits) + (size_t)(lrow * a.ld) * ESZ;
    const float* grow = a.gumbel + (size_t)row * a.ld;
    const float invT = __fdiv_rn(1.0f, a.temperature[trow]);
    const int c0 = s * a.cps;
    const int c1 = min(c0 + a.cps, a.chunks);
    float key[n];
#pragma unroll
    for (int j = 0; j < kTopkCPL; ++j) {
        const int ch = c0 + j * kThreads + tid;
        u32x4 Z = u32x4{0u, 0u, 0u, 0u};
        u32x4 G[EPC / 4];
#pragma unroll
        for (int h = 0; h < EPC / 4; ++h) G[h] = u32x4{0u, 0u, 0u, 0u};
        if (ch < c1) {
            Z = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(zrow) + ch);
#pragma unroll
            for (int h = 0; h < EPC / 4; ++h)
                G[h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(grow) + (int64_t)ch * (EPC / 4) + h);
        }
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
            const int32_t v = ch * EPC + e;
            const bool in = ch < c1 && v < a.V;
            key[j * EPC + e] = in ? fmaf(chunk_elem<DT>(Z, e), invT, __uint_as_float(G[e >> 2][e & 3]))
                                  : -INFINITY;
        }
    }
    // k rounds: block argmax of the lanes' bests; the winning lane drops that key and finds
    // its next best. A lane's keys are in increasing index order (chunk group, then element).
    BonusPart* out = a.cand + (row * a.S + s) * a.k;
    float bk;
    int pos = lane_best_pos<n>(key, bk);
    auto index_of = [&](int p) {
        return p < 0 ? INT32_MAX : (c0 + (p / EPC) * kThreads + tid) * EPC + p % EPC;
    };
    for (int it = 0; it < a.k; ++it) {
        float wk = bk;
        int32_t wi = index_of(pos);
        const int32_t mine = wi;
        const int buf = (it & 1) * kWaves;
        block_argmax(wk, wi, lk + buf, li + buf);
        if (tid == 0) out[it] = BonusPart{wk, wk == -INFINITY ? INT32_MAX : wi};
        if (pos >= 0 && mine == wi) {
#pragma unroll
            for (int e = 0; e < n; ++e) key[e] = e == pos ? -INFINITY : key[e];
            pos = lane_best_pos<n>(key, bk);
        }
    }
}

template <int MODE>
__global__ __launch_bounds__(kThreads) void k_topk_merge(TopkArgs a) {
    constexpr int n = kMaxTopk * kMaxTopkSlices / kThreads;   // 8 candidates a lane at most
    __shared__ float lk[2 * kWaves];
    __shared__ int32_t li[2 * kWaves];
    __shared__ BonusPart res[kMaxTopk];
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    if constexpr (MODE == kTopkResampled) {
        const int32_t x = a.ancestors[row];
        if (x < 0 || x >= a.N) {
            if (tid == 0) {
                flag_error(a.error_flags, SMCSD_DEVERR_ANCESTOR);
                a.out_tokens[row] = -1;
                if (a.slot_tokens) a.slot_tokens[row * (a.K + 1) + a.K] = -1;
            }
            return;
        }
    }
    const int m = a.S * a.k;
    const BonusPart* c = a.cand + row * m;
    float key[n];
    int32_t idx[n];
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const int t = e * kThreads + tid;
        key[e] = t < m ? c[t].key : -INFINITY;
        idx[e] = t < m ? c[t].idx : INT32_MAX;
    }
    select_k<n>(key, idx, a.k, res, lk, li);
    __syncthreads();
    for (int j = tid; j < a.k; j += kThreads) {
        a.out_tokens[row * a.k + j] = res[j].idx;
        if (a.out_keys) a.out_keys[row * a.k + j] = res[j].key;
    }
    if (a.slot_tokens && tid == 0) a.slot_tokens[row * (a.K + 1) + a.K] = res[0].idx;
}

}  // namespace

hipError_t launch_topk(int64_t rows, int32_t dtype, const TopkArgs& a, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const dim3 block(kThreads);
    const dim3 g1((unsigned)(rows * a.S));
    if (a.row_mode == kTopkResampled) {
        if (dtype == SMCSD_BF16) k_topk_slice<SMCSD_BF16, kTopkResampled><<<g1, block, 0, s>>>(a);
        else k_topk_slice<SMCSD_F32, kTopkResampled><<<g1, block, 0, s>>>(a);
    } else {
        if (dtype == SMCSD_BF16) k_topk_slice<SMCSD_BF16, kTopkRows><<<g1, block, 0, s>>>(a);
        else k_topk_slice<SMCSD_F32, kTopkRows><<<g1, block, 0, s>>>(a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.row_mode == kTopkResampled) k_topk_merge<kTopkResampled><<<dim3((unsigned)rows), block, 0, s>>>(a);
    else k_topk_merge<kTopkRows><<<dim3((unsigned)rows), block, 0, s>>>(a);
    return hipGetLastError();
}

hipError_t launch_topk_slices(int64_t rows, int32_t dtype, const TopkArgs& a, hipStream_t s) {
    if (rows <= 0) return hipSuccess;
    const dim3 block(kThreads), grid((unsigned)(rows * a.S));
    if (dtype == SMCSD_BF16) k_topk_slice<SMCSD_BF16, kTopkBonusRows><<<grid, block, 0, s>>>(a);
    else k_topk_slice<SMCSD_F32, kTopkBonusRows><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
