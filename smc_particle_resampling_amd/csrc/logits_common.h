// logits_common.h -- what the two logits-pass kernels share (k_logits_tv.hip, TV on, and
// k_logits_stream.hip, TV off): element widths, the 16-byte slice loads, -inf padding, and
// the wave reductions over a slice's chunks.
//
// The logits pass of one SMC-SD round is the one pass that touches the logits, i.e. nearly
// every byte of the round. For every drafted position it reduces the target row and the
// draft row over the whole vocabulary. It produces their temperature log-softmax
// normalisers, which the importance weights of "Faster LLM Inference via Sequential Monte
// Carlo" (section 2) need, and, when asked, the total-variation distance between the two
// distributions (the block-divergence signal of the METASD page, section 2). It also
// reduces every particle's bonus row with its precomputed Gumbel noise to the Gumbel-max
// token (STAND page, method item 2): the stream kernel does so itself, and with TV the
// round hands those rows to the Gumbel-Top-K slice kernel (k = 1).
//
// Work decomposition. A row is cut into 16-byte chunks and the chunks into S slices. One
// 512-thread workgroup (8 wave64) handles one slice of one row pair (target row k, draft row
// k) or one slice of one bonus row plus its noise row. Each lane loads its CPL chunks of both
// rows with 16-byte non-temporal buffer loads. Chunks outside the slice and elements >= V
// become -inf, which adds nothing to any max, sum, TV or argmax, so the arithmetic has no
// per-element branch. The finalize kernel combines slices (normalisers, weights, TV,
// argmax) in fixed order, so every result is deterministic.
// Included by the two .hip sources only, inside namespace smcsd's anonymous namespace.
#pragma once

#include "smcsd_device.h"

namespace smcsd {
namespace {

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

}  // namespace
}  // namespace smcsd
