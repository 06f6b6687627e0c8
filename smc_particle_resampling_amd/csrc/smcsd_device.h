// smcsd_device.h -- device helpers shared by the kernels of libsmcsd.so: chunk widening,
// DPP wave reductions, error flags and the slice-partial combines. Included by the .hip
// sources only; the host-side plan and argument blocks are in smcsd_internal.h.
#pragma once

#include "smcsd_internal.h"

namespace smcsd {
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.44269504088896340736f;   // exp(x) = exp2(x * log2e)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Element e (0..epc-1) of a 16-byte chunk as f32 (exact widening for bf16).
template <int DT>
__device__ __forceinline__ float chunk_elem(const u32x4& c, int e) {
    if constexpr (DT == SMCSD_F32) {
        return __uint_as_float(c[e]);
    } else {
        const uint32_t w = c[e >> 1];
        return (e & 1) ? bf16_hi(w) : bf16_lo(w);
    }
}

__device__ __forceinline__ void flag_error(int32_t* flags, uint32_t bit) {
    if (flags) atomicOr(reinterpret_cast<unsigned int*>(flags), bit);
}

// Cross-lane reductions by DPP moves, which stay in the VALU (no LDS round trip as with
// ds_bpermute). Steps xor 1 and xor 2 (quad permutes), then the half-row mirror (lane i of
// 8 reads 7 - i) and the row mirror (lane i of 16 reads 15 - i): after them every lane of a
// 16-lane row holds the row's result, because each step combines two disjoint groups whose
// results every lane already holds. The four row results are then read from lanes 0, 16,
// 32 and 48 and combined in that order. The order is fixed, so a sum is bit-identical from
// run to run, and the result is uniform (a scalar register).
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

template <int kCtrl>
__device__ __forceinline__ float dpp_f32(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), kCtrl,
                                                                 0xF, 0xF, true));
}
template <int kCtrl>
__device__ __forceinline__ int32_t dpp_i32(int32_t v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, true);
}
__device__ __forceinline__ float readlane_f32(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float row_max(float v) {
    v = fmaxf(v, dpp_f32<kDppXor1>(v));
    v = fmaxf(v, dpp_f32<kDppXor2>(v));
    v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
    return fmaxf(v, dpp_f32<kDppRowMirror>(v));
}
__device__ __forceinline__ float row_sum(float v) {
    v += dpp_f32<kDppXor1>(v);
    v += dpp_f32<kDppXor2>(v);
    v += dpp_f32<kDppRowHalfMirror>(v);
    return v + dpp_f32<kDppRowMirror>(v);
}

// Whole-wave max and sum; every lane must be active. The result is wave-uniform.
__device__ __forceinline__ float wave_max(float v) {
    v = row_max(v);
    return fmaxf(fmaxf(readlane_f32(v, 0), readlane_f32(v, 16)),
                 fmaxf(readlane_f32(v, 32), readlane_f32(v, 48)));
}
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum(v);
    return ((readlane_f32(v, 0) + readlane_f32(v, 16)) + readlane_f32(v, 32)) + readlane_f32(v, 48);
}

// The same reductions in double precision, each DPP step moving the two 32-bit halves.
// Row masks: kRows selects the 16-lane rows the step writes; the others receive 0.
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142;   // lane 15 of each row to the whole next row
constexpr int kDppRowBcast31 = 0x143;   // lane 31 to rows 2 and 3

template <int kCtrl, int kRows = 0xF>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)b, kCtrl, kRows, 0xF, true);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(b >> 32), kCtrl, kRows, 0xF, true);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), lane);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
// Whole-wave max and sum of doubles (every lane active), uniform and bit-identical from run
// to run, in the order of wave_max and wave_sum.
__device__ __forceinline__ double wave_max_f64(double v) {
    v = fmax(v, dpp_f64<kDppXor1>(v));
    v = fmax(v, dpp_f64<kDppXor2>(v));
    v = fmax(v, dpp_f64<kDppRowHalfMirror>(v));
    v = fmax(v, dpp_f64<kDppRowMirror>(v));
    return fmax(fmax(readlane_f64(v, 0), readlane_f64(v, 16)), fmax(readlane_f64(v, 32), readlane_f64(v, 48)));
}
__device__ __forceinline__ double wave_sum_f64(double v) {
    v += dpp_f64<kDppXor1>(v);
    v += dpp_f64<kDppXor2>(v);
    v += dpp_f64<kDppRowHalfMirror>(v);
    v += dpp_f64<kDppRowMirror>(v);
    return ((readlane_f64(v, 0) + readlane_f64(v, 16)) + readlane_f64(v, 32)) + readlane_f64(v, 48);
}
// Inclusive prefix sum over the 64 lanes (every lane active): a scan within each row (lane k
// adds lane k - d for d = 1, 2, 4, 8; lanes with k < d add 0), then row 1 and row 3 add the
// totals of rows 0 and 2, then rows 2 and 3 add lane 31 (the total of rows 0 and 1). A fixed
// order, so the sums are bit-identical from run to run.
__device__ __forceinline__ double wave_scan_f64(double v) {
    v += dpp_f64<kDppRowShr1>(v);
    v += dpp_f64<kDppRowShr2>(v);
    v += dpp_f64<kDppRowShr4>(v);
    v += dpp_f64<kDppRowShr8>(v);
    v += dpp_f64<kDppRowBcast15, 0xA>(v);
    v += dpp_f64<kDppRowBcast31, 0xC>(v);
    return v;
}

// One logit of a row, widened exactly to double.
template <int DT>
__device__ __forceinline__ double logit_at(const void* base, int64_t row, int64_t ld, int32_t v) {
    if constexpr (DT == SMCSD_F32) {
        return (double)static_cast<const float*>(base)[row * ld + v];
    } else {
        const uint16_t bits = static_cast<const uint16_t*>(base)[row * ld + v];
        return (double)__uint_as_float((uint32_t)bits << 16);
    }
}

// Row maxima and softmax denominators of one row pair from its S slice partials, in slice
// order: M = max_t m_t, S = sum_t s_t * exp2((m_t - M) * c) accumulated in double.
// The first kPartRegs slice parts of a position are loaded together into registers, so a
// thread has them all in flight at once; slices beyond those are loaded in batches of 8.
constexpr int kPartRegs = 16;

__device__ __forceinline__ void load_parts(const PairPart* part, int S, PairPart (&v)[kPartRegs]) {
#pragma unroll
    for (int t = 0; t < kPartRegs; ++t)
        if (t < S) v[t] = part[t];
}

// Row maxima and sums of one position from its S slice parts; v holds the first kPartRegs
// of them (load_parts). The sums take the slices in order 0..S-1.
__device__ __forceinline__ void pair_norms_from(const PairPart* part, const PairPart (&v)[kPartRegs],
                                                int S, float c, float& Mp, float& Mq, double& Sp,
                                                double& Sq) {
    Mp = -INFINITY;
    Mq = -INFINITY;
#pragma unroll
    for (int t = 0; t < kPartRegs; ++t)
        if (t < S) {
            Mp = fmaxf(Mp, v[t].mp);
            Mq = fmaxf(Mq, v[t].mq);
        }
    for (int t0 = kPartRegs; t0 < S; t0 += 8) {
        PairPart w[8];
#pragma unroll
        for (int b = 0; b < 8; ++b)
            if (t0 + b < S) w[b] = part[t0 + b];
#pragma unroll
        for (int b = 0; b < 8; ++b)
            if (t0 + b < S) {
                Mp = fmaxf(Mp, w[b].mp);
                Mq = fmaxf(Mq, w[b].mq);
            }
    }
    Sp = 0.0;
    Sq = 0.0;
#pragma unroll
    for (int t = 0; t < kPartRegs; ++t)
        if (t < S) {
            Sp += (double)(v[t].sp * __builtin_amdgcn_exp2f((v[t].mp - Mp) * c));
            Sq += (double)(v[t].sq * __builtin_amdgcn_exp2f((v[t].mq - Mq) * c));
        }
    for (int t0 = kPartRegs; t0 < S; t0 += 8) {
        PairPart w[8];
#pragma unroll
        for (int b = 0; b < 8; ++b)
            if (t0 + b < S) w[b] = part[t0 + b];
#pragma unroll
        for (int b = 0; b < 8; ++b)
            if (t0 + b < S) {
                Sp += (double)(w[b].sp * __builtin_amdgcn_exp2f((w[b].mp - Mp) * c));
                Sq += (double)(w[b].sq * __builtin_amdgcn_exp2f((w[b].mq - Mq) * c));
            }
    }
}

__device__ __forceinline__ void pair_norms(const PairPart* part, int S, float c, float& Mp,
                                           float& Mq, double& Sp, double& Sq) {
    PairPart v[kPartRegs];
    load_parts(part, S, v);
    pair_norms_from(part, v, S, c, Mp, Mq, Sp, Sq);
}

// (key, index) argmax: the larger key wins, the lower index wins on equal keys.
__device__ __forceinline__ bool better(float k1, int32_t i1, float k2, int32_t i2) {
    return k1 > k2 || (k1 == k2 && i1 < i2);
}

}  // namespace smcsd
