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
// Every draw is a Gumbel-max over the whole vocabulary with one key per entry:
// draft x_k = argmax_v z_v + G(tag 0, v); residual, fallback and bonus draws
// use tag 2.  Keys are formed in base 2 (see entry_l2).
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

__device__ __forceinline__ float inv_temperature(float T) { return 1.0f / T; }

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

// Philox4x32-10 for the counters (q, pos, b, tag) of one (request, position,
// tag) with only the first counter word q varying, as when a lane walks the
// vocabulary: the parts of rounds 1-3 that depend on pos, b, tag and the key
// alone are computed once (philox_row), so one block of four draws
// (philox_row_block) costs 37 VALU operations instead of 40.  The rounds are the
// ones of philox10, written out with those parts folded in.
struct PhiloxRow {
    uint32_t k0, k1;   // key words (seed low, seed high)
    uint32_t c3k;      // round 1: tag ^ k1
    uint32_t x0, x1k;  // round 1 outputs 0 and 1 (x1 already xored with round 2's k0)
    uint32_t h0k, l0;  // round 2: hi(M0 x0) ^ round 2's k1, lo(M0 x0)
    uint32_t l0k;      // round 3: lo(M0 x0) ^ round 3's k1
};

__device__ __forceinline__ PhiloxRow philox_row(uint64_t seed, uint32_t b, uint32_t pos,
                                                uint32_t tag) {
    PhiloxRow r;
    r.k0 = static_cast<uint32_t>(seed);
    r.k1 = static_cast<uint32_t>(seed >> 32);
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * b;
    r.x0 = static_cast<uint32_t>(p1 >> 32) ^ pos ^ r.k0;
    r.x1k = static_cast<uint32_t>(p1) ^ (r.k0 + 0x9E3779B9u);
    r.c3k = tag ^ r.k1;
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * r.x0;
    r.h0k = static_cast<uint32_t>(p0 >> 32) ^ (r.k1 + 0xBB67AE85u);
    r.l0 = static_cast<uint32_t>(p0);
    r.l0k = r.l0 ^ (r.k1 + 2u * 0xBB67AE85u);
    return r;
}

// The block for counter word q in stages, so that a caller can spread its
// rounds over other work: philox_head runs rounds 1-3 (where the fixed parts
// of the counter are folded in), philox_round(i) round i = 4..10 with the key
// advanced i - 1 times.
struct PhiloxState {
    uint32_t c0, c1, c2, c3;
};

__device__ __forceinline__ PhiloxState philox_head(const PhiloxRow& r, uint32_t q) {
    // round 1: x0, x1 come from (pos, b); x2, x3 from q
    const uint64_t a0 = static_cast<uint64_t>(0xD2511F53u) * q;
    const uint32_t x2 = static_cast<uint32_t>(a0 >> 32) ^ r.c3k;
    const uint32_t x3 = static_cast<uint32_t>(a0);
    // round 2: M0 x0 is fixed
    const uint64_t a1 = static_cast<uint64_t>(0xCD9E8D57u) * x2;
    const uint32_t c0 = static_cast<uint32_t>(a1 >> 32) ^ r.x1k;
    const uint32_t c1 = static_cast<uint32_t>(a1);
    const uint32_t c2 = x3 ^ r.h0k;
    // round 3: the previous word 3 (lo(M0 x0)) is fixed
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
    return {xor3(static_cast<uint32_t>(p1 >> 32), c1, r.k0 + 2u * 0x9E3779B9u),
            static_cast<uint32_t>(p1), static_cast<uint32_t>(p0 >> 32) ^ r.l0k,
            static_cast<uint32_t>(p0)};
}

__device__ __forceinline__ void philox_round(PhiloxState& p, const PhiloxRow& r, int i) {
    const uint64_t p0 = static_cast<uint64_t>(0xD2511F53u) * p.c0;
    const uint64_t p1 = static_cast<uint64_t>(0xCD9E8D57u) * p.c2;
    const uint32_t n0 =
        xor3(static_cast<uint32_t>(p1 >> 32), p.c1, r.k0 + static_cast<uint32_t>(i - 1) * 0x9E3779B9u);
    const uint32_t n2 =
        xor3(static_cast<uint32_t>(p0 >> 32), p.c3, r.k1 + static_cast<uint32_t>(i - 1) * 0xBB67AE85u);
    p.c1 = static_cast<uint32_t>(p1);
    p.c3 = static_cast<uint32_t>(p0);
    p.c0 = n0;
    p.c2 = n2;
}

__device__ __forceinline__ uint32_t state_word(const PhiloxState& p, int w) {
    return w == 0 ? p.c0 : (w == 1 ? p.c1 : (w == 2 ? p.c2 : p.c3));
}

// Draws for vocabulary entries 4 q .. 4 q + 3 (word v & 3 of block q = v >> 2).
__device__ __forceinline__ u32x4 philox_row_block(const PhiloxRow& r, uint32_t q) {
    PhiloxState p = philox_head(r, q);
#pragma unroll
    for (int i = 4; i <= 10; ++i) philox_round(p, r, i);
    return {p.c0, p.c1, p.c2, p.c3};
}

// Per-lane constants of the entry key.  A sampled lane (T > 0) forms
// key = s c2 - log2(-log2 u) with c2 = log2(e) / T: log2(e) (z + G) plus a
// constant shared by the row, so it orders entries as z + G does.  A greedy
// lane (T == 0) that runs the same code (a wavefront mixing both) takes c2 = 1
// and u = 1/2, so -log2(-log2 u) = 0 and its key is s itself: the argmax.
struct KeyLane {
    float c2;
    float umul, uoff;  // u = f umul + uoff from f = 1 + (w >> 9) 2^-23
};

__device__ __forceinline__ KeyLane key_lane(float T) {
    if (T > 0.0f) return {inv_temperature(T) * kLog2e, 1.0f, -0x1.fffffep-1f};
    return {1.0f, 0.0f, 0.5f};
}

// log2(-log2 u) of a draw word; -log2(-log2 u) = log2(e) G - log2(log2 e).
// Both logarithm arguments are normal floats (u >= 2^-24, -log2 u >= 8.6e-8).
__device__ __forceinline__ float entry_l2(uint32_t w, const KeyLane& kl) {
    const float f = __uint_as_float(__builtin_amdgcn_alignbit(0x7Fu, w, 9));
    const float l1 = __builtin_amdgcn_logf(fmaf(f, kl.umul, kl.uoff));
    return __builtin_amdgcn_logf(-l1);
}

// Residual and fallback keys of the verifier's draw after a rejection at row
// j* (and the bonus draw of a listed full acceptance, which is the fallback
// draw over row L_b + 1).  Per entry, in base 2 with c2 = log2(e) / T:
//   a  = log2 p_t = t c2 - lse_t log2(e)
//   dm = log2 p_d - log2 p_t = (s - t) c2 + (lse_t - lse_d) log2(e)
//   fallback  kf = a - log2(-log2 u)
//   residual  kr = kf + log2(1 - 2^dm)      (entries with p_t > p_d, dm < 0)
// with the entry's tag-2 draw: log2(e) (y + G) and log2(e) (log(p_t - p_d) + G)
// up to constants shared by the row.  dm is formed from the logit difference so
// that a target row equal to the draft row gives every such entry the same dm.
// The verifier's residual list: the sampled first rejections at
// list[0 .. count[0]) and the sampled full acceptances (whose next token is the
// bonus draw) from the back, list[B - 1 - i] for i < count[1].  Slot s in
// [0, n), n = count[0] + count[1], names one listed request.  Slots come in
// groups of 256 (a workgroup row of the residual strip kernels); each group
// takes its share of the rejections, first, then of the full acceptances:
// group [start, end) holds rejection ranks [q(start), q(end)), q(x) =
// floor(count[0] x / n).  So the groups carry like work (a rejection
// recomputes its draft row, a full acceptance keys the target row alone), and
// a wavefront holds one kind of request (but for the one at the boundary).
__device__ __forceinline__ int listed_count(const int32_t* count) { return count[0] + count[1]; }

__device__ __forceinline__ int listed_request(const int32_t* list, const int32_t* count, int B,
                                              int s) {
    const int nr = count[0], n = count[0] + count[1];
    if (n <= 0) return list[B - 1];  // no listed request: an in-range stand-in
    const int start = s & ~255, end = min(start + 256, n);
    const int q0 = static_cast<int>(static_cast<int64_t>(nr) * start / n);
    const int q1 = static_cast<int>(static_cast<int64_t>(nr) * end / n);
    const int o = s - start;
    if (o < q1 - q0) return list[q0 + o];
    return list[B - 1 - ((start - q0) + (o - (q1 - q0)))];
}

struct ResRow {
    float c2;    // log2(e) / T
    float lt2;   // lse_t log2(e)
    float dl;    // (lse_t - lse_d) log2(e)
    bool bonus;  // a listed full acceptance: fallback keys only
    KeyLane kl;
    PhiloxRow ph;
};

struct ResBest {
    float br, bf;  // best residual / fallback key
    int ir, jf;    // and its entry
};

__device__ __forceinline__ ResBest res_empty() {
    return {-INFINITY, -INFINITY, 0x7fffffff, 0x7fffffff};
}

// One entry (s = base + bias, tv = target logit, w = its draw word); entries
// arrive in increasing order (strict comparisons keep the smallest on ties).
__device__ __forceinline__ void residual_entry(ResBest& rb, float sv, float tv, uint32_t w, int v,
                                               const ResRow& R) {
    const float a = fmaf(tv, R.c2, -R.lt2);
    const float dm = fmaf(sv - tv, R.c2, R.dl);
    const float kf = a - entry_l2(w, R.kl);
    // past V both logits are -inf: a = kf = -inf and dm is NaN (no residual key)
    const float kr = (dm < 0.0f && !R.bonus)
                         ? kf + __builtin_amdgcn_logf(1.0f - __builtin_amdgcn_exp2f(dm))
                         : -INFINITY;
    if (kr > rb.br) {
        rb.br = kr;
        rb.ir = v;
    }
    if (kf > rb.bf) {
        rb.bf = kf;
        rb.jf = v;
    }
}

// ---------------------------------------------------------------- row state
// Partial reduction state of one logits row over a subset of the vocabulary:
// online-softmax max m and sum s = sum exp(z - m); the winner of a keyed
// argmax (its key, a value carried with it, its index): the entry with the
// largest perturbed key (its own Gumbel draw) or, for T == 0, the largest
// logit.  Ties go to the smaller index.
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

// Token ids and lengths come from device memory the host cannot check; they are
// clamped before they index anything.
__device__ __forceinline__ int clamp_token(int x, int V) { return min(max(x, 0), V - 1); }
__device__ __forceinline__ int clamp_len(int L, int K) { return min(max(L, 0), K); }

}  // namespace dspark
