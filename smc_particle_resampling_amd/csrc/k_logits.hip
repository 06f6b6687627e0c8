// k_logits.hip -- the logits pass of one SMC-SD round: the one kernel that touches the
// logits, i.e. nearly every byte of the round.
//
// For every drafted position it reduces the target row and the draft row over the whole
// vocabulary. It produces their temperature log-softmax normalisers, which the importance
// weights of "Faster LLM Inference via Sequential Monte Carlo" (section 2) need, and, when
// asked, the total-variation distance between the two distributions (the block-divergence
// signal of the METASD page, section 2). It can also reduce every particle's bonus row with
// its precomputed Gumbel noise to the Gumbel-max token (STAND page, method item 2): the round
// does so here without TV, and with TV hands those rows to the Gumbel-Top-K slice kernel
// (k = 1), which runs them faster than this grid's tail would.
//
// Work decomposition. A row is cut into 16-byte chunks and the chunks into S slices. One
// 512-thread workgroup (8 wave64) handles one slice of one row pair (target row k, draft row
// k) or one slice of one bonus row plus its noise row. Each lane loads its CPL chunks of both
// rows with 16-byte non-temporal buffer loads. Chunks outside the slice and elements >= V
// become -inf, which adds nothing to any max, sum, TV or argmax, so the arithmetic has no
// per-element branch. (The TV pass avoids even that where it can: when every slice fills all
// its chunk groups but the last and V is a multiple of the chunk width, a lane past the slice
// end re-reads an inside chunk and its exponentials are shifted by -inf.)
//   phase 1: the maximum m of z over a share of the slice, then e = exp2((z - m) * log2e/T)
//            and its sum, for p and q. TV off: the share is the slice (one workgroup max).
//            TV on: each wave's own share, so nothing waits between loads and exponentials.
//   phase 2 (TV only): the S workgroups of the row pair swap their (m, sum) partials and
//            combine them in one fixed order into the row's maxima M and sums S. With
//            f = exp2((m - M) * log2e/T) (m of the wave that computed the e values) the
//            |p - q| terms are (f_p / S_p) |e_p - rho e_q|, rho = (f_q S_p) / (f_p S_q).
//            The e values stay in fp32 registers from phase 1, so phase 2 costs one fma and
//            one add per element and no exponential. rho is exactly 1 when the two rows are
//            equal, and then TV is exactly 0.
// The finalize kernel combines slices (normalisers, weights, TV, argmax) in fixed order, so
// every result is deterministic.
//
// Launch shapes. Without TV, every (row, slice) is an independent workgroup of an ordinary
// grid (8 chunks a lane). With TV, the S workgroups of a row pair must be resident together
// to swap partials, so the pass runs as a persistent cooperative grid
// (hipLaunchCooperativeKernel guarantees co-residency) over the row pairs only. It has C
// clusters of S consecutive workgroups (4 chunks a lane, so the fp32 e values fit in
// registers), and each cluster walks the row pairs c, c+C, c+2C, ... in lockstep. The loads
// of a cluster's next row pair are issued while the current one is exchanged and finished.
// The round's bonus rows run before it, as an ordinary grid of the Gumbel-Top-K slice kernel,
// which also resets this kernel's control word and exchange words.
// A wall-clock limit bounds every wait. A workgroup that times out raises
// SMCSD_DEVERR_EXCHANGE and an abort flag, every later wait returns at once, and the kernel
// always drains.
#include <algorithm>
#include <atomic>

#include "smcsd_device.h"

namespace smcsd {
namespace {

constexpr float kLog2e = 1.44269504088896340736f;

template <int DT>
struct Elem {
    static constexpr int EPC = DT == SMCSD_F32 ? 4 : 8;              // elements per chunk
    static constexpr size_t ESZ = DT == SMCSD_F32 ? 4 : 2;           // bytes per element
    static constexpr uint32_t kNegInf = DT == SMCSD_F32 ? 0xFF800000u : 0xFF80FF80u;
};

// A per-request value that no kernel of the round writes (the temperatures), read through
// the scalar cache. A plain load would be a vector load, and waiting for it would also wait
// for every logits load issued before it.
__device__ __forceinline__ float load_constant(const float* p, int64_t i) {
    return ((const __attribute__((address_space(4))) float*)p)[i];
}

__device__ __forceinline__ u32x4 load_chunk(const char* row, int64_t chunk) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(row) + chunk);
}

// A chunk whose elements >= nv are replaced by -inf (nv < EPC: the row's tail chunk).
template <int DT>
__device__ __forceinline__ u32x4 mask_tail(u32x4 c, int nv) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        if constexpr (DT == SMCSD_F32) {
            if (w >= nv) c[w] = 0xFF800000u;
        } else {
            if (2 * w >= nv) c[w] = 0xFF80FF80u;
            else if (2 * w + 1 >= nv) c[w] = (c[w] & 0x0000FFFFu) | 0xFF800000u;
        }
    }
    return c;
}

// Slice loads go through a buffer resource that covers exactly the slice [c0, c1) of a row:
// one scalar base, one lane offset (16 * lane) shared by every load, the chunk group in the
// scalar offset, and the hardware range check returning zeros past the slice end (no
// memory access there). Word 3 is the gfx9-family raw-buffer setting (32-bit data format,
// no swizzle); cache policy 2 marks the loads non-temporal.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kLoadNontemporal = 2;

// Issue the loads of the CPL chunks this lane owns in slice [c0, c1) of a row (chunk
// c0 + j * kThreads + lane). They may still be in flight on return.
template <int CPL>
__device__ __forceinline__ void issue_slice(u32x4 (&R)[CPL], const char* row, int c0, int c1) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(row) + (size_t)c0 * 16, 0, (c1 - c0) * 16, kRsrcWord3);
    const int voff = (int)threadIdx.x * 16;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
        R[j] = __builtin_amdgcn_raw_buffer_load_b128(r, voff, j * kThreads * 16, kLoadNontemporal);
}

// After the loads: chunks past the slice end and elements >= V (only in the row's last
// chunk, when V is not a multiple of EPC) become -inf. The branches are uniform.
template <int DT, int CPL>
__device__ __forceinline__ void mask_slice(u32x4 (&R)[CPL], int c0, int c1, int V) {
    constexpr int EPC = Elem<DT>::EPC;
    const int tid = threadIdx.x;
    const int n = c1 - c0;
    const uint32_t ni = Elem<DT>::kNegInf;
#pragma unroll
    for (int j = 0; j < CPL; ++j)
        if ((j + 1) * kThreads > n && j * kThreads + tid >= n) R[j] = u32x4{ni, ni, ni, ni};
    if ((int64_t)c1 * EPC > V) {
        const int last = c1 - 1 - c0;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
            if (j * kThreads + tid == last) R[j] = mask_tail<DT>(R[j], V - (c1 - 1) * EPC);
    }
}

typedef short i16x2 __attribute__((ext_vector_type(2)));

// sum over the slice of exp2(z * c - m * c)
template <int DT, int CPL>
__device__ __forceinline__ float slice_sumexp(const u32x4 (&R)[CPL], float c, float nmc) {
    float s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
#pragma unroll
        for (int e = 0; e < Elem<DT>::EPC; e += 2) {
            s0 += __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(R[j], e), c, nmc));
            s1 += __builtin_amdgcn_exp2f(fmaf(chunk_elem<DT>(R[j], e + 1), c, nmc));
        }
    }
    return s0 + s1;
}

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

// Wave-wide integer max / min by DPP row steps, then the four row results.
__device__ __forceinline__ int32_t wave_max_i32(int32_t v) {
    v = max(v, dpp_i32<kDppXor1>(v));
    v = max(v, dpp_i32<kDppXor2>(v));
    v = max(v, dpp_i32<kDppRowHalfMirror>(v));
    v = max(v, dpp_i32<kDppRowMirror>(v));
    return max(max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               max(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}
__device__ __forceinline__ int32_t wave_min_i32(int32_t v) {
    v = min(v, dpp_i32<kDppXor1>(v));
    v = min(v, dpp_i32<kDppXor2>(v));
    v = min(v, dpp_i32<kDppRowHalfMirror>(v));
    v = min(v, dpp_i32<kDppRowMirror>(v));
    return min(min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 16)),
               min(__builtin_amdgcn_readlane(v, 32), __builtin_amdgcn_readlane(v, 48)));
}

// Maximum of this wave's share of a slice (wave-uniform). bf16: the packed int16 max alone
// decides whenever the wave holds a non-negative value (those order like their int16 bits
// and beat every negative); only a wave whose share is entirely negative takes the int16
// min as well (negative values order in reverse). -inf padding (int16 -128) never wins
// either way while a finite value is present.
template <int DT, int CPL>
__device__ __forceinline__ float wave_share_max(const u32x4 (&R)[CPL]) {
    if constexpr (DT == SMCSD_F32) {
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int w = 0; w < 4; w += 2)
                m = fmaxf(m, fmaxf(__uint_as_float(R[j][w]), __uint_as_float(R[j][w + 1])));
        return wave_max(m);
    } else {
        i16x2 mx = {(short)-32768, (short)-32768};
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t word = R[j][w];
                mx = __builtin_elementwise_max(mx, __builtin_bit_cast(i16x2, word));
            }
        const int32_t hi = wave_max_i32(mx[0] > mx[1] ? mx[0] : mx[1]);
        if (hi >= 0) return __uint_as_float((uint32_t)hi << 16);
        i16x2 mn = {(short)32767, (short)32767};
#pragma unroll
        for (int j = 0; j < CPL; ++j)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t word = R[j][w];
                mn = __builtin_elementwise_min(mn, __builtin_bit_cast(i16x2, word));
            }
        const int32_t lo = wave_min_i32(mn[0] < mn[1] ? mn[0] : mn[1]);
        return __uint_as_float(((uint32_t)lo & 0xFFFFu) << 16);
    }
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
    if (t < bonus_wgs) {
        bonus_slice<DT, kStreamCPL>(a, t / a.S, (int)(t % a.S), red, redi);
    } else if (t < a.total_wgs) {
        const int64_t tp = t - bonus_wgs;
        pair_slice_stream<DT>(a, tp / a.S, (int)(tp % a.S), wpart);
    }
}

// Before a TV pass without bonus rows: the control word (abort flag 0, the wait limit) and
// every exchange word at the all-ones "empty" pattern, in one launch.
__global__ void k_fill_tv(Ctrl* ctrl, uint32_t timeout, uint32_t* words, int64_t n) {
    if (blockIdx.x == 0 && threadIdx.x == 0) *ctrl = Ctrl{0u, timeout};
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
                                                               reinterpret_cast<uint32_t*>(a.pp), n);
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

hipError_t launch_logits(const Plan& plan, const LogitsArgs& a, hipStream_t s) {
    if (plan.tv) {
        const bool fast = tv_fast_path(plan);
        if (plan.dtype == SMCSD_BF16)
            return fast ? launch_tv<SMCSD_BF16, true>(plan, a, s) : launch_tv<SMCSD_BF16, false>(plan, a, s);
        return fast ? launch_tv<SMCSD_F32, true>(plan, a, s) : launch_tv<SMCSD_F32, false>(plan, a, s);
    }
    const dim3 grid((unsigned)plan.total_wgs), block(kThreads);
    if (plan.dtype == SMCSD_BF16) k_logits_stream<SMCSD_BF16><<<grid, block, 0, s>>>(a);
    else k_logits_stream<SMCSD_F32><<<grid, block, 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace smcsd
