// k_logits.hip -- the logits pass of one SMC-SD round: the one kernel that touches the
// logits, i.e. nearly every byte of the round.
//
// For every drafted position it reduces the target row and the draft row over the whole
// vocabulary. It produces their temperature log-softmax normalisers, which the importance
// weights of "Faster LLM Inference via Sequential Monte Carlo" (section 2) need, and, when
// asked, the total-variation distance between the two distributions (the block-divergence
// signal of the METASD page, section 2). For every particle it also reduces the bonus row
// with its precomputed Gumbel noise to the Gumbel-max token (STAND page, method item 2).
//
// Work decomposition. A row is cut into 16-byte chunks and the chunks into S slices of at
// most 256 lanes x 8 chunks. One 256-thread workgroup handles one slice of one row pair
// (target row k, draft row k), or one slice of one bonus row plus its noise row. A slice
// is read once with 16-byte non-temporal loads and kept in registers (64 VGPRs a lane for
// a bf16 pair). Then:
//   phase 1: slice max of z and sum of exp2((z - max) * log2e/T) for p and q -> partials;
//   phase 2 (TV only): the S workgroups of a row pair swap partials through the workspace,
//            all combine them in the same fixed order into the row's normalisers, and each
//            sums |p - q| over its own slice from registers. No logit is read twice.
// The final combination over slices (normalisers, weights, argmax) happens in the
// finalize kernel, in fixed order, so every result is deterministic.
//
// Launch shapes. Without TV, every (row, slice) is an independent workgroup of an ordinary
// grid. With TV, the S workgroups of a row pair must be resident at the same time to swap
// partials, so the TV pass runs as a persistent cooperative grid
// (hipLaunchCooperativeKernel, which guarantees co-residency): C clusters of S consecutive
// workgroups, each cluster walking the row pairs c, c+C, c+2C, ... in lockstep, then its
// share of the bonus rows. A wall-clock limit still bounds every wait; a workgroup that
// times out raises SMCSD_DEVERR_EXCHANGE and an abort flag, every later wait returns at
// once, and the kernel always drains.
#include <algorithm>
#include <atomic>

#include "smcsd_internal.h"

namespace smcsd {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;
// 4e8 ticks of the 100 MHz constant clock: 4 s, ~10^4 times the longest expected wait.
constexpr uint64_t kExchangeTimeoutTicks = 400000000ull;

__device__ __forceinline__ u32x4 load_chunk(const char* row, int64_t chunk) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + chunk);
}

// Slice exchange of the TV pass. Every (row pair, slice) partial is two 64-bit words, (max,
// sum) of the target row and of the draft row. Before the launch, every word holds kEmpty,
// a bit pattern no finite partial can take. A slice publishes its two words with relaxed
// agent-scope atomic stores. Wave 0 of every slice polls all 2S words of its row pair with
// relaxed agent-scope atomic loads until none is kEmpty. Each value is read from the very
// location it was stored to, so coherence of that location suffices: no release/acquire
// fences, which on this GPU would write back or invalidate a whole L2 per exchange.
constexpr uint64_t kEmpty = ~0ull;

__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}

// Wave 0 only. Copies the 2S words of row pair u into lds[0..2S) once all are published.
__device__ void wait_for_slices(const uint64_t* words, int nwords, Ctrl* ctrl,
                                int32_t* error_flags, uint64_t* lds) {
    const int lane = threadIdx.x & 63;
    const uint64_t t0 = wall_clock64();
    uint64_t v = 0;
    while (true) {
        v = lane < nwords ? __hip_atomic_load(words + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                          : 0ull;
        if (!__any(v == kEmpty)) break;
        if (__hip_atomic_load(&ctrl->abort, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) break;
        if (wall_clock64() - t0 > kExchangeTimeoutTicks) {
            if (lane == 0) {
                __hip_atomic_store(&ctrl->abort, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                flag_error(error_flags, SMCSD_DEVERR_EXCHANGE);
            }
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    if (lane < nwords) lds[lane] = v;
}

template <int DT, bool TV>
__device__ void pair_slice(const LogitsArgs& a, int64_t u, int s, float* red, float* bcast,
                           uint64_t* xch) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
    constexpr size_t ESZ = DT == SMCSD_F32 ? 4 : 2;
    const int tid = threadIdx.x;
    const int64_t nk = (int64_t)a.N * a.K;
    const int64_t r = u / nk;
    const int64_t ik = u - r * nk;
    const int64_t i = ik / a.K;
    const int64_t k = ik - i * a.K;
    const char* zp = static_cast<const char*>(a.target) +
                     (size_t)(((r * a.N + i) * (a.K + 1) + k) * a.ld) * ESZ;
    const char* zq = static_cast<const char*>(a.draft) +
                     (size_t)(((r * a.N + i) * a.K + k) * a.ld) * ESZ;
    const float c = kLog2e / a.temperature[r];   // exp(z/T) = exp2(z * c)
    const int c0 = s * a.cps;
    const int c1 = min(c0 + a.cps, a.chunks);

    u32x4 P[kChunksPerLane], Q[kChunksPerLane];
#pragma unroll
    for (int j = 0; j < kChunksPerLane; ++j) {
        const int ch = c0 + j * kThreads + tid;
        if (ch < c1) {
            P[j] = load_chunk(zp, ch);
            Q[j] = load_chunk(zq, ch);
        } else {
            P[j] = u32x4{0u, 0u, 0u, 0u};
            Q[j] = u32x4{0u, 0u, 0u, 0u};
        }
    }

    // phase 1a: slice maxima (elements >= V in the row's last chunk are skipped)
    float mp = -INFINITY, mq = -INFINITY;
#pragma unroll
    for (int j = 0; j < kChunksPerLane; ++j) {
        const int ch = c0 + j * kThreads + tid;
        if (ch < c1) {
            const int nv = min(EPC, a.V - ch * EPC);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if (e < nv) {
                    mp = fmaxf(mp, chunk_elem<DT>(P[j], e));
                    mq = fmaxf(mq, chunk_elem<DT>(Q[j], e));
                }
            }
        }
    }
    mp = block_max(mp, red);
    mq = block_max(mq, red);

    // phase 1b: sums of exp2((z - max) * c)
    const float nmp = -mp * c, nmq = -mq * c;
    float sp = 0.0f, sq = 0.0f;
#pragma unroll
    for (int j = 0; j < kChunksPerLane; ++j) {
        const int ch = c0 + j * kThreads + tid;
        if (ch < c1) {
            const int nv = min(EPC, a.V - ch * EPC);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if (e < nv) {
                    sp += __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(P[j], e), c, nmp));
                    sq += __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Q[j], e), c, nmq));
                }
            }
        }
    }
    sp = block_sum(sp, red);
    sq = block_sum(sq, red);
    if constexpr (!TV) {
        if (tid == 0) a.pp[u * a.S + s] = PairPart{mp, sp, mq, sq};
    } else {
        uint64_t* words = reinterpret_cast<uint64_t*>(a.pp + u * a.S);
        if (tid == 0) {
            __hip_atomic_store(words + 2 * s, pack2(mp, sp), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(words + 2 * s + 1, pack2(mq, sq), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if (tid < 64) wait_for_slices(words, 2 * a.S, a.ctrl, a.error_flags, xch);
        __syncthreads();
        if (tid == 0) {
            // the row's normalisers from all slices, in slice order
            float Mp = -INFINITY, Mq = -INFINITY;
            for (int t = 0; t < a.S; ++t) {
                Mp = fmaxf(Mp, __uint_as_float((uint32_t)xch[2 * t]));
                Mq = fmaxf(Mq, __uint_as_float((uint32_t)xch[2 * t + 1]));
            }
            float Sp = 0.0f, Sq = 0.0f;
            for (int t = 0; t < a.S; ++t) {
                const float mpt = __uint_as_float((uint32_t)xch[2 * t]);
                const float spt = __uint_as_float((uint32_t)(xch[2 * t] >> 32));
                const float mqt = __uint_as_float((uint32_t)xch[2 * t + 1]);
                const float sqt = __uint_as_float((uint32_t)(xch[2 * t + 1] >> 32));
                Sp += spt * __builtin_amdgcn_exp2f((mpt - Mp) * c);
                Sq += sqt * __builtin_amdgcn_exp2f((mqt - Mq) * c);
            }
            bcast[0] = Mp;
            bcast[1] = Mq;
            bcast[2] = Sp / Sq;
            bcast[3] = 1.0f / Sp;
        }
        __syncthreads();
        const float nMp = -bcast[0] * c, nMq = -bcast[1] * c, ratio = bcast[2];
        // phase 2, from registers: with e = exp2(z c - M c), p = e_p / Sp and q = e_q / Sq, so
        // sum |p - q| = (1/Sp) sum |e_p - (Sp/Sq) e_q|: one fma per element, and exactly 0
        // when the draft row equals the target row (the ratio is then exactly 1).
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < kChunksPerLane; ++j) {
            const int ch = c0 + j * kThreads + tid;
            if (ch < c1) {
                const int nv = min(EPC, a.V - ch * EPC);
#pragma unroll
                for (int e = 0; e < EPC; ++e) {
                    if (e < nv) {
                        const float ep = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(P[j], e), c, nMp));
                        const float eq = __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(Q[j], e), c, nMq));
                        acc += fabsf(fmaf(-ratio, eq, ep));
                    }
                }
            }
        }
        acc = block_sum(acc, red);
        if (tid == 0) a.tvp[u * a.S + s] = acc * bcast[3];
    }
}

template <int DT>
__device__ void bonus_slice(const LogitsArgs& a, int64_t b, int s, float* red, int32_t* redi) {
    constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;
    constexpr size_t ESZ = DT == SMCSD_F32 ? 4 : 2;
    const int tid = threadIdx.x;
    const int64_t r = b / a.N;
    const char* zrow = static_cast<const char*>(a.target) +
                       (size_t)((b * (a.K + 1) + a.K) * a.ld) * ESZ;
    const char* grow = reinterpret_cast<const char*>(a.gumbel + (size_t)b * a.ld);
    const float invT = __fdiv_rn(1.0f, a.temperature[r]);
    const int c0 = s * a.cps;
    const int c1 = min(c0 + a.cps, a.chunks);

    float best = -INFINITY;
    int32_t besti = INT32_MAX;
#pragma unroll 2
    for (int j = 0; j < kChunksPerLane; ++j) {
        const int ch = c0 + j * kThreads + tid;
        if (ch < c1) {
            const u32x4 z = load_chunk(zrow, ch);
            u32x4 g[EPC / 4];
#pragma unroll
            for (int h = 0; h < EPC / 4; ++h) g[h] = load_chunk(grow, (int64_t)ch * (EPC / 4) + h);
            const int nv = min(EPC, a.V - ch * EPC);
#pragma unroll
            for (int e = 0; e < EPC; ++e) {
                if (e < nv) {
                    const float key = fmaf(chunk_elem<DT>(z, e), invT, __uint_as_float(g[e >> 2][e & 3]));
                    if (key > best) {   // a lane visits its indices in increasing order
                        best = key;
                        besti = ch * EPC + e;
                    }
                }
            }
        }
    }
    // block argmax in fixed order
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ok = __shfl_xor(best, off, 64);
        const int32_t oi = __shfl_xor(besti, off, 64);
        if (better(ok, oi, best, besti)) {
            best = ok;
            besti = oi;
        }
    }
    const int w = tid >> 6;
    if ((tid & 63) == 0) {
        red[w] = best;
        redi[w] = besti;
    }
    __syncthreads();
    if (tid == 0) {
        for (int t = 1; t < kWaves; ++t)
            if (better(red[t], redi[t], best, besti)) {
                best = red[t];
                besti = redi[t];
            }
        a.bp[b * a.S + s] = BonusPart{best, besti};
    }
}

// TV off: one workgroup per (row, slice).
template <int DT>
__global__ __launch_bounds__(kThreads) void k_logits_stream(LogitsArgs a) {
    __shared__ float red[kWaves];
    __shared__ int32_t redi[kWaves];
    __shared__ float bcast[4];
    const int64_t t = blockIdx.x;
    if (t < a.pair_wgs) {
        pair_slice<DT, false>(a, t / a.S, (int)(t % a.S), red, bcast, nullptr);
    } else if (t < a.total_wgs) {
        const int64_t tb = t - a.pair_wgs;
        bonus_slice<DT>(a, tb / a.S, (int)(tb % a.S), red, redi);
    }
}

// TV on: persistent cooperative grid, gridDim.x = C * S.
template <int DT>
__global__ __launch_bounds__(kThreads, 4) void k_logits_tv(LogitsArgs a) {
    __shared__ float red[kWaves];
    __shared__ int32_t redi[kWaves];
    __shared__ float bcast[4];
    __shared__ uint64_t xch[2 * kMaxTvSlices];
    const int s = (int)(blockIdx.x % (unsigned)a.S);
    const int64_t cluster = blockIdx.x / (unsigned)a.S;
    const int64_t clusters = gridDim.x / (unsigned)a.S;
    const int64_t items = a.pairs + (a.total_wgs - a.pair_wgs) / a.S;
    for (int64_t it = cluster; it < items; it += clusters) {
        if (it < a.pairs) pair_slice<DT, true>(a, it, s, red, bcast, xch);
        else bonus_slice<DT>(a, it - a.pairs, s, red, redi);
        __syncthreads();   // red / bcast are reused by the next item
    }
}

__global__ void k_fill_words(uint32_t* p, int64_t n, uint32_t value) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = value;
}

}  // namespace

hipError_t launch_fill_words(uint32_t* p, int64_t n, uint32_t value, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 1024);
    k_fill_words<<<dim3((unsigned)blocks), dim3(kThreads), 0, s>>>(p, n, value);
    return hipGetLastError();
}

// Workgroups of k_logits_tv<DT> that fit on the current device at once (cached per device).
template <int DT>
static int64_t coop_capacity() {
    static std::atomic<int64_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int64_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int per_cu = 0, cus = 0, coop = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(&k_logits_tv<DT>),
                                                     kThreads, 0) != hipSuccess)
        return 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    if (hipDeviceGetAttribute(&coop, hipDeviceAttributeCooperativeLaunch, dev) != hipSuccess || !coop)
        return 0;
    const int64_t c = (int64_t)per_cu * cus;
    if (dev < 64) cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

template <int DT>
static hipError_t launch_tv(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    const int64_t cap = coop_capacity<DT>();
    const int64_t items = plan.pairs + plan.bonus_rows;
    const int64_t clusters = std::min<int64_t>(cap / plan.S, items);
    if (clusters < 1) return hipErrorCooperativeLaunchTooLarge;
    LogitsArgs copy = a;
    void* params[] = {&copy};
    return hipLaunchCooperativeKernel(reinterpret_cast<const void*>(&k_logits_tv<DT>),
                                      dim3((unsigned)(clusters * plan.S)), dim3(kThreads), params, 0, s);
}

hipError_t launch_logits(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    if (plan.tv) {
        return plan.dtype == SMCSD_BF16 ? launch_tv<SMCSD_BF16>(plan, a, s)
                                        : launch_tv<SMCSD_F32>(plan, a, s);
    }
    const dim3 grid((unsigned)plan.total_wgs), block(kThreads);
    if (plan.dtype == SMCSD_BF16) k_logits_stream<SMCSD_BF16><<<grid, block, 0, s>>>(a);
    else k_logits_stream<SMCSD_F32><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
