// k_topk.hip -- Gumbel-Top-K: k tokens drawn without replacement from softmax(z/T) in one
// step, as the STAND page describes for drafting (method item 2): add precomputed, cached
// Gumbel noise to the log-probabilities and keep the indices of the k largest sums. Adding
// the row's normaliser to every key changes no ranking, so the keys are the bonus token's,
// key_v = fl32(fma(z_v, fl32(1/T), G_v)), ranked by decreasing key and then increasing index
// (a total order, so the selection is exact and deterministic).
//
// Pass 1: one 512-thread workgroup per (row, slice), 4 chunks a lane as in the TV pass. Each
// lane holds its keys in registers, the best of each chunk group and its own best; k rounds
// of a block argmax over the lanes' bests pick the slice's k best, and only the lane that
// lost its best rescans, and only the group it lost it from. Pass 2: one wave per row takes
// the S * k candidates of its row by k rounds of a wave argmax (one workgroup per row, by
// block rounds, when they exceed 8 a lane).
//
// Both passes rank a (key, index) pair as one 64-bit word whose unsigned order is the
// ranking: the key's bits mapped to an order-preserving unsigned value (both zeros as +0) in
// the high half, the complement of the index in the low half, so that one 64-bit compare
// decides a step. Pass 1 ranks by the index within its slice (chunk group, lane, element),
// which orders as the index in the row does.
#include "smcsd_device.h"

namespace smcsd {
namespace {

__device__ __forceinline__ uint64_t rank_word(float k, int32_t i) {
    uint32_t b = __float_as_uint(k);
    b = (b << 1) == 0u ? 0u : b;   // -0 ranks as +0
    b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((uint64_t)b << 32) | (uint32_t)~(uint32_t)i;
}
__device__ __forceinline__ float rank_key(uint64_t w) {
    const uint32_t b = (uint32_t)(w >> 32);
    return __uint_as_float((b & 0x80000000u) ? (b & 0x7fffffffu) : ~b);
}
__device__ __forceinline__ int32_t rank_idx(uint64_t w) { return (int32_t)~(uint32_t)w; }
// The word of an absent entry (key -inf, index INT32_MAX); every present entry ranks above
// it, and 0 ranks below everything.
constexpr uint64_t kAbsentWord = (uint64_t(0x007fffffu) << 32) | 0x80000000u;

template <int kCtrl>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, kCtrl, 0xF, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), kCtrl, 0xF, 0xF, true);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t max_u64(uint64_t x, uint64_t y) { return x > y ? x : y; }

// The wave's largest word (every lane active), uniform.
__device__ __forceinline__ uint64_t wave_best(uint64_t w) {
    w = max_u64(w, dpp_u64<kDppXor1>(w));
    w = max_u64(w, dpp_u64<kDppXor2>(w));
    w = max_u64(w, dpp_u64<kDppRowHalfMirror>(w));
    w = max_u64(w, dpp_u64<kDppRowMirror>(w));
    return max_u64(max_u64(readlane_u64(w, 0), readlane_u64(w, 16)),
                   max_u64(readlane_u64(w, 32), readlane_u64(w, 48)));
}

// k rounds of a wave argmax over n words a lane (0 = no entry); round it leaves its winner
// in lane it's res (lanes it < k; k <= 64). A lane drops a present winner it holds and takes
// its next best; absent entries are never dropped, so once only they remain every further
// round returns kAbsentWord.
template <int n>
__device__ __forceinline__ uint64_t wave_select(uint64_t (&c)[n], int k) {
    const int lane = threadIdx.x & 63;
    uint64_t lb = c[0];
#pragma unroll
    for (int e = 1; e < n; ++e) lb = max_u64(lb, c[e]);
    uint64_t res = kAbsentWord;
    for (int it = 0; it < k; ++it) {
        const uint64_t best = wave_best(lb);
        if (lane == it) res = best;
        if (it + 1 < k && lb == best && best != kAbsentWord) {
#pragma unroll
            for (int e = 0; e < n; ++e) c[e] = c[e] == best ? 0 : c[e];
            lb = c[0];
#pragma unroll
            for (int e = 1; e < n; ++e) lb = max_u64(lb, c[e]);
        }
    }
    return res;
}

// The block's largest word (all threads, every lane active); lw holds kWaves words. Callers
// alternate two buffers between rounds, so one barrier per round suffices.
__device__ __forceinline__ uint64_t block_best(uint64_t w, uint64_t* lw) {
    w = wave_best(w);
    if ((threadIdx.x & 63) == 0) lw[threadIdx.x >> 6] = w;
    __syncthreads();
    uint64_t b = lw[0];
#pragma unroll
    for (int t = 1; t < kWaves; ++t) b = max_u64(b, lw[t]);
    return b;
}

// Best of chunk group j of a lane's keys (EPC keys from j * EPC): its maximum, and the first
// position holding it in bits 4j..4j+3 of gp.
template <int DT>
__device__ __forceinline__ void group_best(const float (&key)[kTopkCPL * (DT == SMCSD_F32 ? 4 : 8)], int j,
                                           float& gk, uint32_t& gp) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
    float m = key[j * EPC];
#pragma unroll
    for (int e = 1; e < EPC; ++e) m = fmaxf(m, key[j * EPC + e]);
    uint32_t p = 0;
#pragma unroll
    for (int e = EPC - 1; e >= 0; --e) p = key[j * EPC + e] == m ? (uint32_t)e : p;
    gk = m;
    gp = (gp & ~(0xfu << (4 * j))) | (p << (4 * j));
}

// Drops key e of group j (sets it to -inf) and takes the group's best again.
template <int DT>
__device__ __forceinline__ void drop_in_group(float (&key)[kTopkCPL * (DT == SMCSD_F32 ? 4 : 8)], int j, int e,
                                              float& gk, uint32_t& gp) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
#pragma unroll
    for (int x = 0; x < EPC; ++x) key[j * EPC + x] = x == e ? -INFINITY : key[j * EPC + x];
    group_best<DT>(key, j, gk, gp);
}

// The lane's best position from its groups' bests (groups in increasing index order): the
// first group holding the maximum; -1 if every key is -inf.
template <int EPC>
__device__ __forceinline__ int lane_best_of_groups(const float (&gk)[kTopkCPL], uint32_t gp, float& bk) {
    float m = gk[0];
#pragma unroll
    for (int j = 1; j < kTopkCPL; ++j) m = fmaxf(m, gk[j]);
    int pos = -1;
#pragma unroll
    for (int j = kTopkCPL - 1; j >= 0; --j) pos = gk[j] == m ? j * EPC + (int)((gp >> (4 * j)) & 0xfu) : pos;
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
    __shared__ uint64_t cw[2 * kWaves];
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
    // k rounds of a block argmax over the lanes' bests (as rank words); the winning lane drops
    // that key and finds its next best. A lane's keys are in increasing index order (chunk
    // group, then element), so its first maximum is its best; it keeps each group's best, and
    // a drop rescans only the dropped key's group.
    float gk[kTopkCPL];
    uint32_t gp = 0;
#pragma unroll
    for (int j = 0; j < kTopkCPL; ++j) group_best<DT>(key, j, gk[j], gp);
    float bk;
    int pos = lane_best_of_groups<EPC>(gk, gp, bk);
    for (int it = 0; it < a.k; ++it) {
        // ranked by the index within the slice, (group, lane, element) in that order
        const uint64_t mine =
            pos < 0 ? kAbsentWord : rank_word(bk, (pos / EPC) * (kThreads * EPC) + tid * EPC + pos % EPC);
        const uint64_t best = block_best(mine, cw + (it & 1) * kWaves);
        if (tid == 0) {
            const float rk = rank_key(best);
            a.cand[(row * a.S + s) * a.k + it] =
                BonusPart{rk, rk == -INFINITY ? INT32_MAX : c0 * EPC + rank_idx(best)};
        }
        if (it + 1 < a.k && pos >= 0 && mine == best) {
            const int g = pos / EPC, e = pos % EPC;
#pragma unroll
            for (int j = 0; j < kTopkCPL; ++j)
                if (j == g) drop_in_group<DT>(key, j, e, gk[j], gp);
            pos = lane_best_of_groups<EPC>(gk, gp, bk);
        }
    }
}

// Pass 2 with one wave a row, for S * k <= 512 candidates (8 a lane).
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_topk_merge_wave(TopkArgs a, int64_t rows) {
    constexpr int n = kWaves * kMaxTopk / 64;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (row >= rows) return;
    if constexpr (MODE == kTopkResampled) {
        const int32_t x = a.ancestors[row];
        if (x < 0 || x >= a.N) {
            if (lane == 0) {
                flag_error(a.error_flags, SMCSD_DEVERR_ANCESTOR);
                a.out_tokens[row] = -1;
                if (a.slot_tokens) a.slot_tokens[row * (a.K + 1) + a.K] = -1;
            }
            return;
        }
    }
    const int m = a.S * a.k;
    const BonusPart* cr = a.cand + row * m;
    uint64_t c[n];
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const int t = e * 64 + lane;
        c[e] = t < m ? rank_word(cr[t].key, cr[t].idx) : 0;
    }
    const uint64_t res = wave_select<n>(c, a.k);
    const float rk = rank_key(res);
    const int32_t ri = rk == -INFINITY ? INT32_MAX : rank_idx(res);
    if (lane < a.k) {
        a.out_tokens[row * a.k + lane] = ri;
        if (a.out_keys) a.out_keys[row * a.k + lane] = rk;
    }
    if (a.slot_tokens && lane == 0) a.slot_tokens[row * (a.K + 1) + a.K] = ri;
}

// Pass 2 with one workgroup a row, for more than 512 candidates (at most 8 a lane).
template <int MODE>
__global__ __launch_bounds__(kThreads) void k_topk_merge(TopkArgs a) {
    constexpr int n = kMaxTopk * kMaxTopkSlices / kThreads;
    __shared__ uint64_t cw[2 * kWaves];
    __shared__ uint64_t res[kMaxTopk];
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
    const BonusPart* cr = a.cand + row * m;
    uint64_t c[n];
#pragma unroll
    for (int e = 0; e < n; ++e) {
        const int t = e * kThreads + tid;
        c[e] = t < m ? rank_word(cr[t].key, cr[t].idx) : 0;
    }
    uint64_t lb = c[0];
#pragma unroll
    for (int e = 1; e < n; ++e) lb = max_u64(lb, c[e]);
    for (int it = 0; it < a.k; ++it) {
        const uint64_t best = block_best(lb, cw + (it & 1) * kWaves);
        if (tid == 0) res[it] = best;
        if (it + 1 < a.k && lb == best && best != kAbsentWord) {
#pragma unroll
            for (int e = 0; e < n; ++e) c[e] = c[e] == best ? 0 : c[e];
            lb = c[0];
#pragma unroll
            for (int e = 1; e < n; ++e) lb = max_u64(lb, c[e]);
        }
    }
    __syncthreads();
    for (int j = tid; j < a.k; j += kThreads) {
        const float rk = rank_key(res[j]);
        const int32_t ri = rk == -INFINITY ? INT32_MAX : rank_idx(res[j]);
        a.out_tokens[row * a.k + j] = ri;
        if (a.out_keys) a.out_keys[row * a.k + j] = rk;
        if (a.slot_tokens && j == 0) a.slot_tokens[row * (a.K + 1) + a.K] = ri;
    }
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
    if ((int64_t)a.S * a.k <= kWaves * kMaxTopk) {
        const dim3 g2((unsigned)((rows + kWaves - 1) / kWaves));
        if (a.row_mode == kTopkResampled) k_topk_merge_wave<kTopkResampled><<<g2, block, 0, s>>>(a, rows);
        else k_topk_merge_wave<kTopkRows><<<g2, block, 0, s>>>(a, rows);
    } else if (a.row_mode == kTopkResampled) {
        k_topk_merge<kTopkResampled><<<dim3((unsigned)rows), block, 0, s>>>(a);
    } else {
        k_topk_merge<kTopkRows><<<dim3((unsigned)rows), block, 0, s>>>(a);
    }
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
