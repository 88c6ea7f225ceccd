// common.hpp -- device helpers shared by the draft, verify and schedule
// kernels for gfx950 (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "../../include/dspark.h"
#include "kernels.hpp"

namespace dspark {

constexpr int kWave = 64;
constexpr uint32_t kTagDraft = 0;
constexpr uint32_t kTagAccept = 1;
constexpr uint32_t kTagResample = 2;
constexpr uint32_t kTagDraftBlock = 3;
// Draft tokens are drawn by Gumbel-max in two levels: blocks of kDraftBlock
// consecutive vocabulary entries compete with key log(block mass) + G (tag 3,
// counter word = block index), then the token is the Gumbel-argmax of the
// logits inside the winning block (tag 0, word = entry).  Exact in distribution
// for any partition; only the winning block needs per-entry draws.
constexpr int kDraftBlock = 64;
// The verifier's residual, fallback and bonus draws use the same 64-entry
// blocks: block keys with tag-4 draws (word = block index), then tag-2 draws
// (word = entry) inside the winning block.
constexpr uint32_t kTagVerifyBlock = 4;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------- loads
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}

// ---------------------------------------------------------------- Philox
// Philox4x32-10 (Salmon et al., SC'11, section 3): ten rounds of two 32x32->64
// multiplies; the high halves are mixed into the other two words with the
// round key, the words are re-ordered, and the key advances by two Weyl
// constants per round.
struct u32x4 {
    uint32_t x, y, z, w;
};

// Three-way xor in one gfx950 VALU op (v_bitop3_b32, truth table 0x96 = odd parity).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                          uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
        const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
        const uint32_t n0 = xor3(static_cast<uint32_t>(p1 >> 32), c1, k0);
        const uint32_t n2 = xor3(static_cast<uint32_t>(p0 >> 32), c3, k1);
        c1 = static_cast<uint32_t>(p1);
        c3 = static_cast<uint32_t>(p0);
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return {c0, c1, c2, c3};
}

// Block of four draws for vocab indices 4q .. 4q+3.
__device__ __forceinline__ u32x4 philox_block(uint64_t seed, uint32_t b, uint32_t pos,
                                              uint32_t tag, uint32_t q) {
    return philox10(q, pos, b, tag, static_cast<uint32_t>(seed),
                    static_cast<uint32_t>(seed >> 32));
}

__device__ __forceinline__ uint32_t pick(const u32x4& r, int i) {
    return i == 0 ? r.x : (i == 1 ? r.y : (i == 2 ? r.z : r.w));
}

// u = ((w >> 9) + 0.5) 2^-23, exact in fp32 (24 significant bits).  The top 23
// bits of w become the mantissa of f = 1 + (w >> 9) 2^-23 (one align-bit op
// puts 0x7F above them: exponent field 127), and f - (1 - 2^-24) is exact
// because both operands lie within a factor of two of each other.
__device__ __forceinline__ float uniform_of(uint32_t w) {
    const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9));
    return f - 0x1.fffffep-1f;
}

__device__ __forceinline__ float gumbel_of(uint32_t w) {
    return -logf(-logf(uniform_of(w)));
}

// Same Gumbel from the hardware base-2 logarithm.  Both logarithm arguments
// are normal floats (u >= 2^-24 and -ln u >= 5.9e-8), so no denormal handling
// is needed; the result agrees with the fp64 value to a few fp32 ulps.
__device__ __forceinline__ float gumbel_fast(uint32_t w) {
    const float a = -__builtin_amdgcn_logf(uniform_of(w)) * kLn2;
    return -__builtin_amdgcn_logf(a) * kLn2;
}

// Tag-3 draws of draft blocks 4 (blk / 4) .. 4 (blk / 4) + 3: block blk takes
// word blk % 4 of Philox block blk / 4.
__device__ __forceinline__ u32x4 block_draws(uint64_t seed, uint32_t b, uint32_t pos,
                                             uint32_t blk) {
    return philox_block(seed, b, pos, kTagDraftBlock, blk >> 2);
}

// Base-2 Gumbel -log2(-log2 u) of a draft block's draw word: log2(e) G up to a
// constant shared by every block of the row.
__device__ __forceinline__ float block_gumbel2(uint32_t word) {
    const float l1 = __builtin_amdgcn_logf(uniform_of(word));
    return -__builtin_amdgcn_logf(-l1);
}

// ---------------------------------------------------------------- row state
// Partial reduction state of one logits row over a subset of the vocabulary:
// online-softmax max m and sum s = sum exp(z - m); the winner of a keyed
// argmax (its key, a value carried with it, its index): a perturbed entry, a
// draft block (key = log-mass + Gumbel, index = block start) or, for T == 0,
// the largest logit.  Ties go to the smaller index.
struct RowState {
    float m;
    float s;
    float pert;
    float zb;
    int idx;
};

__device__ __forceinline__ RowState row_empty() {
    return {-INFINITY, 0.0f, -INFINITY, -INFINITY, 0x7fffffff};
}

__device__ __forceinline__ bool beats(float p1, int i1, float p0, int i0) {
    return p1 > p0 || (p1 == p0 && i1 < i0);
}

// The rescaling factors exp(m_a - m) lie in (0, 1]: the hardware exp2 of the
// log2(e)-scaled difference is enough (no range reduction needed).
__device__ __forceinline__ void row_merge(RowState& a, const RowState& b) {
    const float m = fmaxf(a.m, b.m);
    if (m != -INFINITY) {
        const float sa =
            (a.m == -INFINITY) ? 0.0f : a.s * __builtin_amdgcn_exp2f((a.m - m) * kLog2e);
        const float sb =
            (b.m == -INFINITY) ? 0.0f : b.s * __builtin_amdgcn_exp2f((b.m - m) * kLog2e);
        a.s = sa + sb;
        a.m = m;
    }
    if (beats(b.pert, b.idx, a.pert, a.idx)) {
        a.pert = b.pert;
        a.zb = b.zb;
        a.idx = b.idx;
    }
}

// Partner of each lane at step STEP of a wavefront all-reduce, by register
// exchanges only (no LDS): steps 0 and 1 swap lanes within quads (l ^ 1,
// l ^ 2, DPP quad_perm), step 2 mirrors each group of 8 (l ^ 7, DPP
// row_half_mirror), step 3 each row of 16 (l ^ 15, DPP row_mirror), step 4
// swaps adjacent rows of 16 (l ^ 16, v_permlane16_swap) and step 5 the halves
// (l ^ 32, v_permlane32_swap).  The six masks are linearly independent bit
// patterns, so after steps 0..s a commutative merge at every step leaves the
// total of each aligned group of 2^(s+1) lanes in all of them.
template <int STEP>
__device__ __forceinline__ uint32_t xlane(uint32_t x) {
    if constexpr (STEP == 0) {
        return __builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false);
    } else if constexpr (STEP == 1) {
        return __builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false);
    } else if constexpr (STEP == 2) {
        return __builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false);
    } else if constexpr (STEP == 3) {
        return __builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false);
    } else if constexpr (STEP == 4) {
        // rows 2 q + 1 of the first result and rows 2 q of the second hold the
        // other row of each pair
        const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
        return ((threadIdx.x >> 4) & 1) ? r[0] : r[1];
    } else {
        const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return ((threadIdx.x >> 5) & 1) ? r[0] : r[1];
    }
}

template <int STEP>
__device__ __forceinline__ float xlane_f(float x) {
    return __uint_as_float(xlane<STEP>(__float_as_uint(x)));
}
template <int STEP>
__device__ __forceinline__ int xlane_i(int x) {
    return static_cast<int>(xlane<STEP>(static_cast<uint32_t>(x)));
}

template <int STEP>
__device__ __forceinline__ RowState xlane_row(const RowState& a) {
    return {xlane_f<STEP>(a.m), xlane_f<STEP>(a.s), xlane_f<STEP>(a.pert), xlane_f<STEP>(a.zb),
            xlane_i<STEP>(a.idx)};
}

// Every lane ends with the wavefront's merged state (bit-identical in all
// lanes: each step merges a symmetric pair with a commutative rule).
__device__ __forceinline__ void wave_reduce_row(RowState& a) {
    row_merge(a, xlane_row<0>(a));
    row_merge(a, xlane_row<1>(a));
    row_merge(a, xlane_row<2>(a));
    row_merge(a, xlane_row<3>(a));
    row_merge(a, xlane_row<4>(a));
    row_merge(a, xlane_row<5>(a));
}

// Workgroup reduction of one RowState per thread; the result is valid in
// thread 0.  red must hold one RowState per wavefront.
template <int NT>
__device__ __forceinline__ RowState block_reduce_row(RowState st, RowState* red) {
    wave_reduce_row(st);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = st;
    __syncthreads();
    if (tid == 0) {
#pragma unroll
        for (int w = 1; w < NT / kWave; ++w) row_merge(st, red[w]);
    }
    return st;
}


__device__ __forceinline__ void store_partial(PartialBuf p, size_t slot, const RowState& a) {
    p.v[slot] = make_float4(a.m, a.s, a.pert, a.zb);
    p.idx[slot] = a.idx;
}

__device__ __forceinline__ RowState load_partial(PartialBuf p, size_t slot) {
    const float4 v = p.v[slot];
    return {v.x, v.y, v.z, v.w, p.idx[slot]};
}

__device__ __forceinline__ float inv_temperature(float T) { return 1.0f / T; }

// Token ids and lengths come from device memory the host cannot check; they are
// clamped before they index anything.
__device__ __forceinline__ int clamp_token(int x, int V) { return min(max(x, 0), V - 1); }
__device__ __forceinline__ int clamp_len(int L, int K) { return min(max(L, 0), K); }

}  // namespace dspark
