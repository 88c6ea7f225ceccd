// draft_mfma.hip -- MFMA strip kernels for bf16 logits and factors (rank a
// multiple of 16, V a multiple of 8): the Markov-head draft step, parallel
// drafting and the verification residual.
//
// All need, per (request, vocabulary entry), the transition bias of the
// previous token: bias^T[v, b] = sum_i W[i, v] A[x_prev[b], i].  It is a dense
// contraction (M = V, N = requests, K = r), so it runs on
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation and never leaves registers;
// the epilogue consumes the accumulators directly.
//
// Workgroup = NWAVES wavefronts = a persistent walk over 128-entry vocabulary
// strips x 32*NWAVES requests.  The strip of W (r x 128 bf16) is staged in LDS
// and shared by the waves; each wave owns 32 requests (one MFMA column tile).
// The rank-256 kernel works a strip as four tiles in two 64-entry halves with
// transposing LDS reads, software-pipelined a tile at a time (the bias MFMAs of
// one tile interleaved with the per-entry draws of the one before); the
// runtime-rank kernel keeps four 32-row
// tiles per strip, where row m of tile t is entry v = strip start + 4 m + t:
//   - an A-operand lane (row m) reads 4 consecutive entries of 8 rank rows
//     with one 8-byte LDS read per row, and the 16 lanes of an LDS pass read
//     128 consecutive bytes (no bank conflicts);
//   - output lane l holds rows 8 (i / 4) + 4 (l / 32) + i % 4 of every tile, so
//     its accumulator i covers the 4 consecutive entries
//     v = start + 32 (i / 4) + 16 (l / 32) + 4 (i % 4) + t, t = 0..3: exactly
//     one Philox block, and the lane's 64 entries are four runs of 16.
#include <algorithm>
#include <atomic>

#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kStripV = kMfmaStrip;  // 128 vocabulary entries per strip
// s_waitcnt operand (gfx9 encoding): vector-memory count <= 4, export and LDS
// counts not waited on
constexpr int kWaitVm4 = 4 | (7 << 4) | (15 << 8);
constexpr int kPitch = kStripV;  // LDS row pitch in bf16 elements (256 bytes)

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 q) { return __builtin_bit_cast(bf16x8, q); }
__device__ __forceinline__ uint32_t dword_of(const uint4& q, int i) {
    return i == 0 ? q.x : (i == 1 ? q.y : (i == 2 ? q.z : q.w));
}

// Entry offset of accumulator i, tile t within a lane's strip half.
__device__ __forceinline__ constexpr int entry_of(int i, int t) {
    return 32 * (i >> 2) + 4 * (i & 3) + t;
}

// The lane's 64 bf16 logits of one row: runs a = 0..3 of 16 entries at
// row[vh + 32 a], two 16-byte loads each.  Every load is in bounds and
// unconditional (chunks past the end of the row are read from its last chunk;
// V % 8 == 0, V >= 8).  In a strip that crosses V (tail != 0) those chunks are
// then replaced by bf16 -inf, so entries past V carry the logit -inf and need
// no mask downstream.
__device__ __forceinline__ void load_lane_logits(uint4 (&q)[8], const uint16_t* row, int vh,
                                                 int V, bool tail) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int v = vh + 32 * (c >> 1) + 8 * (c & 1);
        q[c] = *reinterpret_cast<const uint4*>(row + min(v, V - 8));
    }
    if (tail) {
        const uint32_t ninf2 = 0xFF80FF80u;  // two bf16 -inf
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int v = vh + 32 * (c >> 1) + 8 * (c & 1);
            if (v >= V) q[c] = make_uint4(ninf2, ninf2, ninf2, ninf2);
        }
    }
}

// Logit of accumulator i, tile t from load_lane_logits' registers.
__device__ __forceinline__ float logit_at(const uint4 (&q)[8], int i, int t) {
    const int o = 4 * (i & 3) + t;  // offset inside the 16-entry run i / 4
    const uint32_t dw = dword_of(q[2 * (i >> 2) + (o >> 3)], (o & 7) >> 1);
    return __uint_as_float((o & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
}

// Stage W[0:r, v0:v0+128] in LDS (row pitch 256 bytes) with direct global->LDS
// loads: one wave instruction moves 1 KiB, four rank rows of the strip, and
// lane i's 16 bytes land at the instruction's LDS base + 16 i.  No VGPR holds
// the data.  Chunks past the end of the vocabulary are read from the row's last
// chunk (V % 8 == 0), so the bias of entries >= V is finite; their logits are
// -inf.  The caller waits for the loads and synchronises before reading.
template <int NWAVES>
__device__ __forceinline__ void stage_w(uint16_t* w_sh, const uint16_t* __restrict__ W, int r,
                                        int V, int v0) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int v = min(v0 + 8 * (lane & 15), V - 8);
    const uint16_t* src = W + static_cast<size_t>(lane >> 4) * V + v;
    for (int j = wave; j < r / 4; j += NWAVES) {
        __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(4 * j) * V,
                                         w_sh + 4 * j * kPitch, 16, 0, 0);
    }
}

// acc[t] = (W^T tile t of the strip) x (factor row arow); arow points at the
// lane's 8-element rank slice (A row + 8 * (lane / 32)).  The LDS rows and the
// factor fragment of the next rank step are read one step ahead, so each
// step's MFMAs do not wait on its own LDS reads.
__device__ __forceinline__ void mfma_step(f32x16 (&acc)[4], const uint2 (&d)[8], uint4 bq) {
    // 8 rank rows x 4 entries -> four vectors of 8 rank values
    const bf16x8 bv = as_bf16x8(bq);
    uint4 a;
    a = make_uint4(__builtin_amdgcn_perm(d[1].x, d[0].x, 0x05040100u),
                   __builtin_amdgcn_perm(d[3].x, d[2].x, 0x05040100u),
                   __builtin_amdgcn_perm(d[5].x, d[4].x, 0x05040100u),
                   __builtin_amdgcn_perm(d[7].x, d[6].x, 0x05040100u));
    acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bv, acc[0], 0, 0, 0);
    a = make_uint4(__builtin_amdgcn_perm(d[1].x, d[0].x, 0x07060302u),
                   __builtin_amdgcn_perm(d[3].x, d[2].x, 0x07060302u),
                   __builtin_amdgcn_perm(d[5].x, d[4].x, 0x07060302u),
                   __builtin_amdgcn_perm(d[7].x, d[6].x, 0x07060302u));
    acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bv, acc[1], 0, 0, 0);
    a = make_uint4(__builtin_amdgcn_perm(d[1].y, d[0].y, 0x05040100u),
                   __builtin_amdgcn_perm(d[3].y, d[2].y, 0x05040100u),
                   __builtin_amdgcn_perm(d[5].y, d[4].y, 0x05040100u),
                   __builtin_amdgcn_perm(d[7].y, d[6].y, 0x05040100u));
    acc[2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bv, acc[2], 0, 0, 0);
    a = make_uint4(__builtin_amdgcn_perm(d[1].y, d[0].y, 0x07060302u),
                   __builtin_amdgcn_perm(d[3].y, d[2].y, 0x07060302u),
                   __builtin_amdgcn_perm(d[5].y, d[4].y, 0x07060302u),
                   __builtin_amdgcn_perm(d[7].y, d[6].y, 0x07060302u));
    acc[3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bv, acc[3], 0, 0, 0);
}

__device__ __forceinline__ void lds_rows(uint2 (&d)[8], const uint16_t* wl, int kk) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
        d[j] = *reinterpret_cast<const uint2*>(wl + (kk * 16 + j) * kPitch);
}

__device__ __forceinline__ uint4 factor_frag(const uint16_t* arow, int kk, int ksteps) {
    return *reinterpret_cast<const uint4*>(arow + 16 * min(kk, ksteps - 1));
}

__device__ __forceinline__ void bias_tiles(f32x16 (&acc)[4], const uint16_t* w_sh,
                                           const uint16_t* arow, int r, int lane) {
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] = 0.0f;
    const uint16_t* wl = w_sh + (8 * (lane >> 5)) * kPitch + 4 * (lane & 31);
    const int ksteps = r / 16;
    // factor fragments come from L2, so they are fetched four rank steps ahead;
    // indices past the last step are clamped (in bounds, never used)
    uint4 q0 = factor_frag(arow, 0, ksteps), q1 = factor_frag(arow, 1, ksteps);
    uint4 q2 = factor_frag(arow, 2, ksteps), q3 = factor_frag(arow, 3, ksteps);
    uint2 d[8];
    lds_rows(d, wl, 0);
    int kk = 0;
    for (; kk + 2 <= ksteps; kk += 2) {
        uint2 e[8];
        lds_rows(e, wl, kk + 1);
        mfma_step(acc, d, q0);
        q0 = factor_frag(arow, kk + 4, ksteps);
        lds_rows(d, wl, min(kk + 2, ksteps - 1));
        mfma_step(acc, e, q1);
        q1 = factor_frag(arow, kk + 5, ksteps);
        const uint4 t0 = q0, t1 = q1;
        q0 = q2;
        q1 = q3;
        q2 = t0;
        q3 = t1;
    }
    if (kk < ksteps) mfma_step(acc, d, q0);
}

// ------------------------------------------------------------------ draft
// Running state of a lane over the entries it visits: the online-softmax
// partial in base 2 (m2 = the largest s c2 seen, s = sum of 2^(s c2 - m2)) and
// the best entry key (s c2 - log2(-log2 u), see KeyLane) with its entry.  A
// greedy lane's key is its logit, and its softmax fields are unused.  lane_row
// turns the state into the row partial the combine merges (m on the z scale;
// zb is not carried: the combine recovers z of the winner from its key).
struct LaneRun {
    float m2;
    float s;
    float key;
    int idx;
};

__device__ __forceinline__ LaneRun lane_empty() { return {-INFINITY, 0.0f, -INFINITY, 0x7fffffff}; }

__device__ __forceinline__ RowState lane_row(const LaneRun& r) {
    return {r.m2 == -INFINITY ? -INFINITY : r.m2 * kLn2, r.s, r.key, 0.0f, r.idx};
}

// Fold a chunk's softmax partial (chunk maximum mx of s, sum of 2^(s c2 - mc)
// with mc = mx c2, or mx = -inf for a chunk with no entry below V) and its best
// key into the lane state (ties to the smaller entry: the two MFMA tiles of a
// half interleave in entry order).
__device__ __forceinline__ void fold_chunk(LaneRun& run, float mx, float mc, float sum, float hb,
                                           int hi) {
    // select-only (no branch), so that the fold stays in the scheduling region
    // of the MFMAs it is interleaved with; with M = -inf both sides hold no
    // entry and exp2(-inf) = 0 keeps the sum at 0
    const float mh = (mx == -INFINITY) ? -INFINITY : mc;
    const float M = fmaxf(run.m2, mh);
    const float Mr = (M == -INFINITY) ? 0.0f : M;
    run.s = run.s * __builtin_amdgcn_exp2f(run.m2 - Mr) + sum * __builtin_amdgcn_exp2f(mh - Mr);
    run.m2 = M;
    const bool take = beats(hb, hi, run.key, run.idx);
    run.key = take ? hb : run.key;
    run.idx = take ? hi : run.idx;
}

// Epilogue of the runtime-rank kernel for one lane (one request, 64 entries
// vh + entry_of(i, t)): s = base + bias (-inf past V), then per entry the
// softmax term and the key (KeyLane); the four tiles of accumulator i are the
// four consecutive entries of one Philox block.  A greedy lane only takes the
// argmax of s.
__device__ __forceinline__ void draft_epilogue(LaneRun& run, f32x16 (&acc)[4], const uint4 (&bl)[8],
                                               int vh, bool greedy, const KeyLane& kl,
                                               const PhiloxRow& ph) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float sv = logit_at(bl, i, t) + acc[t][i];
            acc[t][i] = sv;
            mx = fmaxf(mx, sv);
        }
    }
    float hb = -INFINITY;
    int hi = 0;
    if (greedy) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (acc[t][i] > hb) {
                    hb = acc[t][i];
                    hi = entry_of(i, t);
                }
        if (hb > run.key) {
            run.key = hb;
            run.idx = vh + hi;
        }
        return;
    }
    const float mc = (mx == -INFINITY) ? 0.0f : mx * kl.c2;
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const u32x4 rnd = philox_row_block(ph, static_cast<uint32_t>((vh + entry_of(i, 0)) >> 2));
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float sv = acc[t][i];
            sum += __builtin_amdgcn_exp2f(fmaf(sv, kl.c2, -mc));
            const float key = fmaf(sv, kl.c2, -entry_l2(pick(rnd, t), kl));
            if (key > hb) {
                hb = key;
                hi = entry_of(i, t);
            }
        }
    }
    fold_chunk(run, mx, mc, sum, hb, vh + hi);
}

// One workgroup per (part, request group), persistent over the strips
// part, part + n_parts, ...: while the waves run the bias MFMAs and the epilogue
// of one strip, the next strip's W is already on its way into the other LDS
// buffer and its logits into registers.  Each lane folds the strips it visits
// into one running state, so a request gets n_parts partials per step.
template <int NWAVES>
__global__ __launch_bounds__(64 * NWAVES)
void draft_strip_mfma(const uint16_t* __restrict__ base, const uint16_t* __restrict__ A,
                      const uint16_t* __restrict__ W, const int32_t* __restrict__ prev,
                      int prev_stride, const float* __restrict__ temperature,
                      const int32_t* __restrict__ order, uint64_t seed, int B, int K, int V,
                      int r, int k, PartialBuf part, int n_strips, int n_parts) {
    extern __shared__ uint16_t w_sh[];  // two buffers of [r][kPitch]
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5;
    const int slot = (blockIdx.y * NWAVES + (threadIdx.x >> 6)) * 32 + (lane & 31);
    const bool active = slot < B;
    // lanes past B run request 0's row (every wave takes part in the MFMAs and
    // barriers) and store nothing
    const int b = active ? order[slot] : 0;
    const int p = clamp_token(prev[static_cast<size_t>(b) * prev_stride], V);
    const float T = temperature[b];
    const bool greedy = !(T > 0.0f);
    const KeyLane kl = key_lane(T);
    const PhiloxRow ph = philox_row(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(k + 1),
                                    kTagDraft);
    const uint16_t* arow = A + static_cast<size_t>(p) * r + 8 * kh;
    const uint16_t* brow = base + (static_cast<size_t>(b) * K + k) * V;
    const int buf_elems = r * kPitch;

    int s = blockIdx.x;  // < n_strips: the launch has n_parts <= n_strips
    stage_w<NWAVES>(w_sh, W, r, V, s * kStripV);
    uint4 bl[8];
    load_lane_logits(bl, brow, s * kStripV + 16 * kh, V, s * kStripV + kStripV > V);
    LaneRun lr = lane_empty();
    int buf = 0;
    for (;;) {
        // this strip's W (all waves' shares) and logits have landed, and every
        // wave is done with the other buffer
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        const int sn = s + n_parts;
        const bool more = sn < n_strips;
        f32x16 acc[4];
        bias_tiles(acc, w_sh + buf * buf_elems, arow, r, lane);
        // The next strip's W and logits are requested only now: the vector
        // memory counter retires loads in order, so a prefetch issued before
        // the factor-fragment loads of the MFMA loop would stall that loop
        // until the whole prefetch had landed.
        uint4 bn[8];
        if (more) {
            stage_w<NWAVES>(w_sh + (buf ^ 1) * buf_elems, W, r, V, sn * kStripV);
            load_lane_logits(bn, brow, sn * kStripV + 16 * kh, V, sn * kStripV + kStripV > V);
        }
        // lane entries: strip start + 16 kh + entry_of(i, t)
        draft_epilogue(lr, acc, bl, s * kStripV + 16 * kh, greedy, kl, ph);
        if (!more) break;
#pragma unroll
        for (int c = 0; c < 8; ++c) bl[c] = bn[c];
        buf ^= 1;
        s = sn;
    }
    // lanes l and l + 32 hold the two halves of every strip for one request
    RowState run = lane_row(lr);
    row_merge(run, xlane_row<5>(run));
    if (active && kh == 0)
        store_partial(part, static_cast<size_t>(b) * n_parts + blockIdx.x, run);
}

// ------------------------------------------------- draft: strip in two halves
// Half h of a 128-entry strip is two 32-row tiles.  Row m of tile t is entry
// v0 + 64 h + 16 (m / 8) + 8 ((m / 4) % 2) + 4 (t ^ ((m / 8) % 2)) + m % 4, so
// output lane l's accumulator i of tile t is entry v0 + 64 h + 16 (i / 4)
// + 8 (l / 32) + 4 (t ^ ((i / 4) % 2)) + i % 4: for each run a = i / 4 the lane
// holds the 8 consecutive entries 16 a + 8 (l / 32) + 0..7, one 16-byte logit
// chunk, half of it from each tile.  Working on one half at a time keeps 32
// accumulators live, which leaves room to hold the factor fragments in
// registers.
//
// The A operand (8 consecutive ranks of one entry per lane) comes straight
// from the [rank][entry] strip in LDS through gfx950's transposing LDS read
// (ds_read_b64_tr_b16): within a group of 16 lanes, lane i names 4 consecutive
// bf16 of one row, and lane j receives element j % 4 of the rows named by
// lanes j / 4, j / 4 + 4, j / 4 + 8, j / 4 + 12.  So if lane i of a group names
// rank row R + i / 4 at entry c0(i % 4), lane j receives ranks R .. R + 3 of
// entry c0(j / 4) + j % 4; two such reads give an operand.  The 16 lanes of a
// group name 4 rows x 4 eight-byte pieces, 128 bytes in all.  The strip's
// 16-byte granules are stored XOR-swizzled within each 256-byte rank row
// (granule g of row k at position p = f(g) ^ s(k % 4), with f flipping bit 3
// of g when bit 2 is set and s(u) = 4 (u % 2) + 2 (u / 2)), and a lane naming
// piece q of row u reads the (t ^ (q / 2))-th eight-byte half of its granule
// for tile t: together these put the 16 pieces of a group on 16 distinct
// 8-byte bank slots of a 128-byte line (and the two groups of a 32-lane half
// on different 128-byte halves of the row).
//
// KS = r / 16 rank steps, fixed at compile time so that the step loop is fully
// unrolled without guards (per-step guards split it into branches that stall
// the MFMA pipeline).

__device__ __forceinline__ constexpr int tr_row_swizzle(int u) { return 4 * (u & 1) + 2 * (u >> 1); }
__device__ __forceinline__ constexpr int tr_granule_flip(int g) { return g ^ ((g & 4) << 1); }

// Stage W[0:r, v0:v0+128] in LDS in the swizzled layout above.  As in stage_w,
// one wave instruction fills four rank rows (1 KiB) and lane i's 16 bytes land
// at the instruction's base + 16 i: lane i fills position i % 16 of row
// 4 j + i / 16, so it fetches the granule stored there (f is its own inverse).
template <int NWAVES>
__device__ __forceinline__ void stage_w_tr(uint16_t* w_sh, const uint16_t* __restrict__ W, int r,
                                           int V, int v0) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = tr_granule_flip((lane & 15) ^ tr_row_swizzle(lane >> 4));
    const int v = min(v0 + 8 * g, V - 8);
    const uint16_t* src = W + static_cast<size_t>(lane >> 4) * V + v;
    for (int j = wave; j < r / 4; j += NWAVES) {
        __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(4 * j) * V,
                                         w_sh + 4 * j * kPitch, 16, 0, 0);
    }
}

// The same with the rank fixed at compile time (r = 16 KS, 4 KS a multiple of
// NWAVES): each wave issues exactly 4 KS / NWAVES direct loads, so the
// compiler can count the loads issued after any earlier one and wait for that
// one alone (with a runtime trip count it waits for every outstanding load).
template <int NWAVES, int KS>
__device__ __forceinline__ void stage_w_tr_fixed(uint16_t* w_sh, const uint16_t* __restrict__ W,
                                                 int V, int v0) {
    static_assert((4 * KS) % NWAVES == 0, "whole rank rows per wave");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = tr_granule_flip((lane & 15) ^ tr_row_swizzle(lane >> 4));
    const int v = min(v0 + 8 * g, V - 8);
    const uint16_t* src = W + static_cast<size_t>(lane >> 4) * V + v;
#pragma unroll
    for (int i = 0; i < 4 * KS / NWAVES; ++i) {
        const int j = wave + i * NWAVES;
        __builtin_amdgcn_global_load_lds(src + static_cast<size_t>(4 * j) * V,
                                         w_sh + 4 * j * kPitch, 16, 0, 0);
    }
}

// Element offset in a strip buffer of the row piece this lane names for half h,
// tile t, rank step 0: lane = 32 kh + 16 gm + 4 u + q reads rank row 8 kh + u
// at entry 64 h + 32 gm + 16 (q / 2) + 8 (q % 2) + 4 (t ^ (q / 2)) (granule
// g = 8 h + 4 gm + q, stored at f(g) ^ s(u), and the 8-byte half t ^ (q / 2)
// of it).  Rank step kk is 16 rows further, ranks + 4 are 4 rows further.
__device__ __forceinline__ int tr_offset(int lane, int h, int t) {
    const int kh = lane >> 5, gm = (lane >> 4) & 1, u = (lane >> 2) & 3, q = lane & 3;
    const int g = 8 * h + 4 * gm + q;
    return (8 * kh + u) * kPitch + 8 * (tr_granule_flip(g) ^ tr_row_swizzle(u)) +
           4 * (t ^ (q >> 1));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_tr16(const uint16_t* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Accumulator i of tile t holds entry 16 (i / 4) + 4 (t ^ ((i / 4) % 2)) + i % 4
// of the lane's half, which is element 4 (t ^ ((i / 4) % 2)) + i % 4 of logit
// chunk i / 4 (q = the half's four chunks): the accumulators start from the
// logits, so the MFMAs leave s = base + bias in them.
__device__ __forceinline__ void acc_from_logits(f32x16 (&acc)[2], const uint4 (&q)[4]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t dw = dword_of(q[i >> 2], 2 * (t ^ ((i >> 2) & 1)) + ((i & 3) >> 1));
            acc[t][i] = __uint_as_float((i & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
        }
    }
}

// wt[t] = strip buffer + tr_offset(lane, h, t); acc holds the half's logits.
template <int KS>
__device__ __forceinline__ void bias_half(f32x16 (&acc)[2], const uint16_t* const (&wt)[2],
                                          const uint4 (&afr)[KS]) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const bf16x8 bv = as_bf16x8(afr[kk]);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint2 lo = lds_tr16(wt[t] + kk * 16 * kPitch);
            const uint2 hi = lds_tr16(wt[t] + kk * 16 * kPitch + 4 * kPitch);
            const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), bv, acc[t], 0, 0, 0);
        }
    }
}

// The lane's 64 logits of one strip: chunk 4 h + a holds entries
// v0 + 64 h + 16 a + 8 kh .. + 7.  Loads are in bounds (the last chunk of the
// row stands in past V) and chunks past V become bf16 -inf.
__device__ __forceinline__ void load_strip_logits(uint4 (&q)[8], const uint16_t* row, int v0,
                                                  int kh, int V) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const int v = v0 + 64 * (c >> 2) + 16 * (c & 3) + 8 * kh;
        q[c] = *reinterpret_cast<const uint4*>(row + min(v, V - 8));
    }
    if (v0 + kStripV > V) {
        const uint32_t ninf2 = 0xFF80FF80u;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int v = v0 + 64 * (c >> 2) + 16 * (c & 3) + 8 * kh;
            if (v >= V) q[c] = make_uint4(ninf2, ninf2, ninf2, ninf2);
        }
    }
}

// Chunks 4 h .. 4 h + 3 of a lane's strip logits: the logits of half h.
__device__ __forceinline__ const uint4 (&half_of(const uint4 (&q)[8], int h))[4] {
    return *reinterpret_cast<const uint4(*)[4]>(&q[4 * h]);
}

// Chunks c0 .. c1 - 1 of load_strip_logits without the tail fix-up, so that a
// strip's loads can be spread over the phases of the previous strip.
__device__ __forceinline__ void load_logit_chunks(uint4 (&q)[8], const uint16_t* row, int v0,
                                                  int kh, int V, int c0, int c1) {
#pragma unroll
    for (int c = c0; c < c1; ++c) {
        const int v = v0 + 64 * (c >> 2) + 16 * (c & 3) + 8 * kh;
        q[c] = *reinterpret_cast<const uint4*>(row + min(v, V - 8));
    }
}

// The tail fix-up of load_strip_logits, once the loads have landed.
__device__ __forceinline__ void logit_tail(uint4 (&q)[8], int v0, int kh, int V) {
    if (v0 + kStripV > V) {
        const uint32_t ninf2 = 0xFF80FF80u;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int v = v0 + 64 * (c >> 2) + 16 * (c & 3) + 8 * kh;
            if (v >= V) q[c] = make_uint4(ninf2, ninf2, ninf2, ninf2);
        }
    }
}

// One half (entries vh + 16 a + 4 tt + w, with acc_from_logits' layout: run
// a = i / 4, tt = t ^ (a % 2), w = i % 4) into the running state.  acc holds
// s = base + bias.  Sampled form (any wavefront with a sampled lane): per entry
// the softmax term and the key s c2 - log2(-log2 u) with its own tag-0 draw
// (KeyLane: greedy lanes get the key s); the four entries w = 0..3 of one
// (a, tt) are one Philox block.  Entries are visited in increasing order.
__device__ __forceinline__ void sample_half(LaneRun& run, const f32x16 (&acc)[2], int vh,
                                            const KeyLane& kl, const PhiloxRow& ph) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i)
#pragma unroll
        for (int t = 0; t < 2; ++t) mx = fmaxf(mx, acc[t][i]);
    const float mc = (mx == -INFINITY) ? 0.0f : mx * kl.c2;
    float sum = 0.0f, hb = -INFINITY;
    int hi = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = tt ^ (a & 1);
            const u32x4 rnd =
                philox_row_block(ph, static_cast<uint32_t>(vh >> 2) + 4 * a + tt);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sv = acc[t][4 * a + w];
                sum += __builtin_amdgcn_exp2f(fmaf(sv, kl.c2, -mc));
                const float key = fmaf(sv, kl.c2, -entry_l2(pick(rnd, w), kl));
                if (key > hb) {
                    hb = key;
                    hi = 16 * a + 4 * tt + w;
                }
            }
        }
    }
    fold_chunk(run, mx, mc, sum, hb, vh + hi);
}

// Greedy form (every lane of the wavefront has T == 0): the first entry, in
// increasing order, that holds the largest logit.
__device__ __forceinline__ void greedy_half(LaneRun& run, const f32x16 (&acc)[2], int vh) {
    float hb = -INFINITY;
    int hi = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float sv = acc[tt ^ (a & 1)][4 * a + w];
                if (sv > hb) {
                    hb = sv;
                    hi = 16 * a + 4 * tt + w;
                }
            }
    if (hb > run.key) {
        run.key = hb;
        run.idx = vh + hi;
    }
}

// Eight bf16 -inf: the logit chunk that stands in for chunks past V.
__device__ uint4 kNegInfChunk = {0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};

// Chunks a = 0..3 of half h of a lane's strip logits (entries v0 + 64 h +
// 16 a + 8 kh .. + 7).  A chunk past V is read from kNegInfChunk, so entries
// past V carry the logit -inf with no fix-up after the loads land (a fix-up
// would make the waits for these loads coarser than they need to be).
__device__ __forceinline__ void load_half(uint4 (&q)[4], const uint16_t* row, int v0, int h,
                                          int kh, int V) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int v = v0 + 64 * h + 16 * a + 8 * kh;
        const uint4* p = (v < V) ? reinterpret_cast<const uint4*>(row + v) : &kNegInfChunk;
        q[a] = *p;
    }
}

// The first strip's logits of a launch, coalesced.  Every CU asks for its
// first strip at once, and per-lane loads (32 rows x 32 bytes per instruction)
// make four times the cache requests of whole row pieces.  So the wave's 32
// rows x 256 bytes go by direct loads into LDS (the second W buffer, free
// until the first strip's barrier), 16 lanes per row piece: chunk c of row j
// lands in slot c ^ (j % 16), which spreads the lanes of a later read over all
// banks.  Then each lane reads its eight chunks (those of load_half, with the
// same -inf chunks past V) into L0 / L1.
__device__ __forceinline__ void first_strip_logits(uint4 (&L0)[4], uint4 (&L1)[4], uint16_t* lds,
                                                   const uint16_t* brow, int v0, int kh, int V) {
    const int lane = threadIdx.x & 63;
    uint16_t* wl = lds + (threadIdx.x >> 6) * 32 * kStripV;  // the wave's 32 rows (8 KiB)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 4 * q + (lane >> 4);
        const uint16_t* rp = reinterpret_cast<const uint16_t*>(
            __shfl(reinterpret_cast<unsigned long long>(brow), row, kWave));
        const int v = v0 + 8 * ((lane & 15) ^ (row & 15));
        const void* src = (v < V) ? static_cast<const void*>(rp + v)
                                  : static_cast<const void*>(&kNegInfChunk);
        __builtin_amdgcn_global_load_lds(src, wl + q * 4 * kStripV, 16, 0, 0);
    }
    // the wave's own direct loads have landed: wait for every load it has out
    __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));
    asm volatile("" ::: "memory");
    const int j = lane & 31;
    const uint16_t* rl = wl + j * kStripV;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        L0[a] = *reinterpret_cast<const uint4*>(rl + 8 * ((2 * a + kh) ^ (j & 15)));
        L1[a] = *reinterpret_cast<const uint4*>(rl + 8 * ((8 + 2 * a + kh) ^ (j & 15)));
    }
    // every read of the buffer is done before this wave meets the first strip's
    // barrier, after which the next strip's W goes into it
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (0x3 << 14));
}

// The -inf fix-up for chunks past V, for callers that load with the row's
// last chunk standing in (the residual kernel).
__device__ __forceinline__ void tail_half(uint4 (&q)[4], int v0, int h, int kh, int V) {
    if (v0 + kStripV > V) {
        const uint32_t ninf2 = 0xFF80FF80u;
#pragma unroll
        for (int a = 0; a < 4; ++a)
            if (v0 + 64 * h + 16 * a + 8 * kh >= V) q[a] = make_uint4(ninf2, ninf2, ninf2, ninf2);
    }
}

// ------------------------------------------- rank 256: one MFMA tile at a time
// Tile t of a half is accumulator set acc[t] of acc_from_logits' layout: its
// accumulator i = 4 a + w holds entry vh + 16 a + 4 (t ^ (a % 2)) + w, element
// 4 (t ^ (a % 2)) + w of logit chunk a.  The sixteen entries of a tile are four
// Philox blocks, visited in increasing order.

__device__ __forceinline__ void tile_from_logits(f32x16& acc, const uint4 (&q)[4], int t) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t dw = dword_of(q[i >> 2], 2 * (t ^ ((i >> 2) & 1)) + ((i & 3) >> 1));
        acc[i] = __uint_as_float((i & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
    }
}

template <int KS>
__device__ __forceinline__ void bias_tile(f32x16& acc, const uint16_t* wt,
                                          const uint4 (&afr)[KS]) {
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        const uint2 lo = lds_tr16(wt + kk * 16 * kPitch);
        const uint2 hi = lds_tr16(wt + kk * 16 * kPitch + 4 * kPitch);
        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(afr[kk]), acc, 0, 0,
                                                      0);
    }
}

__device__ __forceinline__ void sample_tile(LaneRun& run, const f32x16& acc, int vh, int t,
                                            const KeyLane& kl, const PhiloxRow& ph) {
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, acc[i]);
    const float mc = (mx == -INFINITY) ? 0.0f : mx * kl.c2;
    float sum = 0.0f, hb = -INFINITY;
    int hi = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int o = 16 * a + 4 * (t ^ (a & 1));
        const u32x4 rnd = philox_row_block(ph, static_cast<uint32_t>((vh + o) >> 2));
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sv = acc[4 * a + w];
            sum += __builtin_amdgcn_exp2f(fmaf(sv, kl.c2, -mc));
            const float key = fmaf(sv, kl.c2, -entry_l2(pick(rnd, w), kl));
            if (key > hb) {
                hb = key;
                hi = o + w;
            }
        }
    }
    fold_chunk(run, mx, mc, sum, hb, vh + hi);
}

__device__ __forceinline__ void greedy_tile(LaneRun& run, const f32x16& acc, int vh, int t) {
    float hb = -INFINITY;
    int hi = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int w = 0; w < 4; ++w)
            if (acc[4 * a + w] > hb) {
                hb = acc[4 * a + w];
                hi = 16 * a + 4 * (t ^ (a & 1)) + w;
            }
    if (beats(hb, vh + hi, run.key, run.idx)) {
        run.key = hb;
        run.idx = vh + hi;
    }
}

// Software pipeline of the rank-256 draft kernel, one unit per MFMA tile (a
// strip is four: half 0 tiles 0 and 1, half 1 tiles 0 and 1).  Unit u runs the
// KS bias MFMAs of its own tile into one accumulator set and, in the same
// instruction stream, the per-entry sampling of unit u - 1 from the other set.
// A wavefront issues in order, so MFMAs grouped in a phase of their own stall
// it (each waits for the matrix core and for its transposing LDS reads) while
// its VALU work waits behind them; the unit is therefore cut into KS slices
// fenced by sched_barrier, slice kk holding the MFMA of rank step kk (its
// operands read two slices earlier), entry kk % 4 of Philox block kk / 4 and a
// quarter of the rounds of the next block.  Measured on its own (two
// wavefronts per SIMD, operands in LDS) this takes 4.3K cycles per pair of
// tiles against 4.75K with the MFMAs in a phase of their own and 3.8K for the
// sampling alone.  Pipelining per tile rather than per half keeps two
// accumulator sets at 32 registers.
template <int KS, bool GREEDY, bool SAMPLE>
__device__ __forceinline__ void rk_unit(f32x16& accm, const uint16_t* wt, const uint4 (&afr)[KS],
                                        const f32x16& accs, LaneRun& run, int vs, int ts,
                                        const KeyLane& kl, const PhiloxRow& ph) {
    static_assert(KS == 16, "the slice schedule covers 16 rank steps (four Philox blocks)");
    constexpr bool kSample = SAMPLE && !GREEDY;
    uint2 lo[3], hi[3];
    lo[0] = lds_tr16(wt);
    hi[0] = lds_tr16(wt + 4 * kPitch);
    lo[1] = lds_tr16(wt + 16 * kPitch);
    hi[1] = lds_tr16(wt + 16 * kPitch + 4 * kPitch);
    float mx = -INFINITY, mc = 0.0f, sum = 0.0f, hb = -INFINITY;
    int he = 0;
    PhiloxState cur{}, nxt{};
    if constexpr (kSample) {
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, accs[i]);
        mc = (mx == -INFINITY) ? 0.0f : mx * kl.c2;
        nxt = philox_head(ph, static_cast<uint32_t>((vs + 4 * ts) >> 2));
#pragma unroll
        for (int i = 4; i <= 10; ++i) philox_round(nxt, ph, i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + 2 < KS) {
            lo[(kk + 2) % 3] = lds_tr16(wt + (kk + 2) * 16 * kPitch);
            hi[(kk + 2) % 3] = lds_tr16(wt + (kk + 2) * 16 * kPitch + 4 * kPitch);
        }
        const uint4 a = make_uint4(lo[kk % 3].x, lo[kk % 3].y, hi[kk % 3].x, hi[kk % 3].y);
        accm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(afr[kk]), accm, 0, 0,
                                                       0);
        if constexpr (kSample) {
            // entry w of block g (tile entries 16 g + 4 (ts ^ (g % 2)) + w)
            const int g = kk >> 2, w = kk & 3;
            if (w == 0) cur = nxt;
            const int o = 16 * g + 4 * (ts ^ (g & 1));
            const float sv = accs[4 * g + w];
            sum += __builtin_amdgcn_exp2f(fmaf(sv, kl.c2, -mc));
            const float key = fmaf(sv, kl.c2, -entry_l2(state_word(cur, w), kl));
            if (key > hb) {
                hb = key;
                he = o + w;
            }
            // a quarter of block g + 1's rounds
            if (g < 3) {
                const int gn = g + 1;
                if (w == 0) {
                    nxt = philox_head(ph, static_cast<uint32_t>((vs + 16 * gn + 4 * (ts ^ (gn & 1))) >> 2));
                    philox_round(nxt, ph, 4);
                } else {
                    philox_round(nxt, ph, 2 * w + 3);
                    philox_round(nxt, ph, 2 * w + 4);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kSample) fold_chunk(run, mx, mc, sum, hb, vs + he);
    if constexpr (SAMPLE && GREEDY) greedy_tile(run, accs, vs, ts);
}

// Load balancing of the rank-256 draft kernel.  Wavefronts w and w + 4 of a
// workgroup share a SIMD, and requests are visited greedy first, so with a
// third of the requests greedy two SIMDs hold two sampled wavefronts each
// while the other two hold a greedy one (argmax only) beside a sampled one.
// A sampled wavefront on a loaded SIMD then hands the last tile of every strip
// but the final one to the greedy wavefront of a light SIMD: it writes the
// tile's s values (16 per lane, 4 KiB) to LDS before the next strip's barrier,
// and the helper draws that tile's keys and softmax terms for the same lanes
// after the barrier, with the owner's request constants, into states of its
// own that are merged into the owner's at the end.  Every key is computed by
// the same code either way, so the draw does not depend on who takes a tile.
constexpr int kRoleNone = 0;    // samples all its tiles
constexpr int kRoleHelped = 1;  // hands the last tile of each strip to a helper
constexpr int kRoleHelper = 2;  // greedy wavefront drawing two helped tiles per strip
// s_waitcnt operand: vector-memory count <= 4 and every LDS access complete
constexpr int kWaitVm4Lds = 4 | (7 << 4) | (0 << 8);
// Handoff slots: [strip parity][helped index 0..3][4 float4 per lane][64 lanes].
constexpr int kHandoffSlots = 2 * 4 * 4 * 64;

// Barrier for LDS traffic only: waits for this wave's LDS accesses, not for
// its outstanding global loads (which __syncthreads' fence would drain).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xF | (7 << 4) | (0 << 8) | (0x3 << 14));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// A helper's constants and running states for the lanes of the two wavefronts
// it serves (helped indices h and h + 2 for helper wavefront h).
struct Helper {
    KeyLane kl[2];
    PhiloxRow ph[2];
    LaneRun run[2];
};

__device__ __forceinline__ float4* handoff_slot(float4* hs, int par, int idx) {
    return hs + (par * 4 + idx) * 4 * 64;
}

__device__ __forceinline__ void put_tile(float4* slot, const f32x16& acc, int lane) {
#pragma unroll
    for (int c = 0; c < 4; ++c)
        slot[c * 64 + lane] = make_float4(acc[4 * c], acc[4 * c + 1], acc[4 * c + 2], acc[4 * c + 3]);
}

__device__ __forceinline__ void get_tile(f32x16& acc, const float4* slot, int lane) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const float4 q = slot[c * 64 + lane];
        acc[4 * c] = q.x;
        acc[4 * c + 1] = q.y;
        acc[4 * c + 2] = q.z;
        acc[4 * c + 3] = q.w;
    }
}

// Merge of two lane states (the softmax partials rescaled to the larger
// maximum; the key by beats(), so the result does not depend on the order).
__device__ __forceinline__ void run_merge(LaneRun& a, const LaneRun& b) {
    const float M = fmaxf(a.m2, b.m2);
    const float Mr = (M == -INFINITY) ? 0.0f : M;
    a.s = a.s * __builtin_amdgcn_exp2f(a.m2 - Mr) + b.s * __builtin_amdgcn_exp2f(b.m2 - Mr);
    a.m2 = M;
    if (beats(b.key, b.idx, a.key, a.idx)) {
        a.key = b.key;
        a.idx = b.idx;
    }
}

// One strip of draft_strip_mfma_rk: this strip's W is in `cur`, the next
// strip's goes into `nxt`.  The caller alternates two static LDS arrays, so
// every LDS access here names one array: the compiler then sees that the
// transposing reads of `cur` cannot alias the direct loads into `nxt`, and
// issues the MFMAs without first waiting for the next strip's W.  L0 / L1
// hold this strip's half-0 / half-1 logits on entry and the next strip's on
// return (each is reloaded once both of its tiles are unpacked); accB holds the
// previous strip's last tile (unsampled) on entry, and this strip's on return.
// FIRST: no previous tile to sample.  PAR: the strip's parity (the handoff
// slot it writes or reads).  Returns false after the last strip.
template <int NWAVES, int KS, bool GREEDY, bool FIRST, int ROLE, int PAR>
__device__ __forceinline__ bool rk_strip(const uint16_t* cur, uint16_t* nxt, int& s, uint4 (&L0)[4],
                                         uint4 (&L1)[4], f32x16& accA, f32x16& accB, int& vsB,
                                         LaneRun& run, const uint16_t* __restrict__ W,
                                         const uint16_t* brow, const uint4 (&afr)[KS],
                                         const int (&tro)[2][2], const KeyLane& kl,
                                         const PhiloxRow& ph, int V, int kh, int n_strips,
                                         int n_parts, float4* hs, int hidx, Helper& H) {
    const int lane = threadIdx.x & 63;
    // the previous strip's last tile goes to the helper
    if constexpr (ROLE == kRoleHelped && !FIRST) put_tile(handoff_slot(hs, PAR, hidx), accB, lane);
    // This strip's W (all waves' shares) and half-0 logits have landed, and
    // every wave is done with the other buffer.  The wave's loads were issued
    // in the order W, half-0 logits, half-1 logits (the slices' scheduling
    // fences keep them there), so waiting until at most the four half-1 loads
    // are outstanding covers the first two: those were requested about four
    // tiles ago, the half-1 logits one tile ago, and they are first used two
    // tiles from now.  The bare barrier (no release fence, which would wait
    // for every outstanding load) is enough: each wave has waited for its own
    // direct-to-LDS loads of this strip, every LDS read of the other buffer has
    // been consumed by an MFMA before it, and the empty asm keeps the compiler
    // from moving memory accesses across it.  A helped wave also waits for its
    // handoff writes, so the helper reads them after the barrier.
    if constexpr (ROLE == kRoleHelped)
        __builtin_amdgcn_s_waitcnt(kWaitVm4Lds);
    else
        __builtin_amdgcn_s_waitcnt(kWaitVm4);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    const int v0 = s * kStripV;
    const int sn = s + n_parts;
    const bool more = sn < n_strips;
    // the next strip's W and logits (after the last strip: this one's again,
    // into the unused buffer and registers, so that every path issues the
    // same loads and the waits can count them)
    const int vn = more ? sn * kStripV : v0;
    stage_w_tr_fixed<NWAVES, KS>(nxt, W, V, vn);
    const int vh0 = v0 + 8 * kh, vh1 = v0 + 64 + 8 * kh;
    tile_from_logits(accA, L0, 0);
    if constexpr (ROLE == kRoleHelped)
        rk_unit<KS, GREEDY, false>(accA, cur + tro[0][0], afr, accB, run, vsB, 1, kl, ph);
    else
        rk_unit<KS, GREEDY, !FIRST>(accA, cur + tro[0][0], afr, accB, run, vsB, 1, kl, ph);
    // a helper draws the two handed-off tiles of the previous strip, one after
    // each of its first two units (the lanes' entry offsets are its own vsB)
    if constexpr (ROLE == kRoleHelper && !FIRST) {
        f32x16 acch;
        get_tile(acch, handoff_slot(hs, PAR, threadIdx.x >> 6), lane);
        sample_tile(H.run[0], acch, vsB, 1, H.kl[0], H.ph[0]);
    }
    tile_from_logits(accB, L0, 1);
    load_half(L0, brow, vn, 0, kh, V);
    rk_unit<KS, GREEDY, true>(accB, cur + tro[0][1], afr, accA, run, vh0, 0, kl, ph);
    if constexpr (ROLE == kRoleHelper && !FIRST) {
        f32x16 acch;
        get_tile(acch, handoff_slot(hs, PAR, (threadIdx.x >> 6) + 2), lane);
        sample_tile(H.run[1], acch, vsB, 1, H.kl[1], H.ph[1]);
    }
    tile_from_logits(accA, L1, 0);
    rk_unit<KS, GREEDY, true>(accA, cur + tro[1][0], afr, accB, run, vh0, 1, kl, ph);
    tile_from_logits(accB, L1, 1);
    load_half(L1, brow, vn, 1, kh, V);
    rk_unit<KS, GREEDY, true>(accB, cur + tro[1][1], afr, accA, run, vh1, 0, kl, ph);
    vsB = vh1;
    if (!more) return false;
    s = sn;
    return true;
}

template <int NWAVES, int KS, bool GREEDY, int ROLE>
__device__ __forceinline__ void rk_strips(uint16_t* w_a, uint16_t* w_b, int s, LaneRun& run,
                                          const uint16_t* __restrict__ W, const uint16_t* brow,
                                          const uint4 (&afr)[KS], const int (&tro)[2][2],
                                          const KeyLane& kl, const PhiloxRow& ph, int V, int kh,
                                          int n_strips, int n_parts, float4* hs, int hidx,
                                          Helper& H) {
    stage_w_tr_fixed<NWAVES, KS>(w_a, W, V, s * kStripV);
    uint4 L0[4], L1[4];
    first_strip_logits(L0, L1, w_b, brow, s * kStripV, kh, V);
    f32x16 accA, accB;
    int vsB = 0;
    // strips alternate between w_a (parity 0) and w_b (parity 1)
    if (rk_strip<NWAVES, KS, GREEDY, true, ROLE, 0>(w_a, w_b, s, L0, L1, accA, accB, vsB, run, W,
                                                    brow, afr, tro, kl, ph, V, kh, n_strips,
                                                    n_parts, hs, hidx, H)) {
        while (rk_strip<NWAVES, KS, GREEDY, false, ROLE, 1>(w_b, w_a, s, L0, L1, accA, accB, vsB,
                                                            run, W, brow, afr, tro, kl, ph, V, kh,
                                                            n_strips, n_parts, hs, hidx, H) &&
               rk_strip<NWAVES, KS, GREEDY, false, ROLE, 0>(w_a, w_b, s, L0, L1, accA, accB, vsB,
                                                            run, W, brow, afr, tro, kl, ph, V, kh,
                                                            n_strips, n_parts, hs, hidx, H)) {
        }
    }
    // the last tile (half 1, tile 1): never handed off
    if constexpr (GREEDY)
        greedy_tile(run, accB, vsB, 1);
    else
        sample_tile(run, accB, vsB, 1, kl, ph);
}

// One workgroup per (part, request group), persistent over the strips part,
// part + n_parts, ...: the factor fragments of each lane's request are loaded
// once and stay in registers, so the MFMA loops issue no vector-memory loads.
// The next strip's W (into the other LDS array) is requested as soon as a
// strip starts, and each half's logits as soon as the registers of the same
// half of the current strip are free.  Each lane folds the halves and strips
// it visits into one running state, so a request gets n_parts partials per
// step.  A wavefront whose lanes are all greedy (T == 0) runs the key-free
// argmax epilogue.  With eight wavefronts, greedy ones take tiles from the
// sampled wavefronts of loaded SIMDs (the handoff above).
template <int NWAVES, int KS>
__global__ __launch_bounds__(64 * NWAVES)
void draft_strip_mfma_rk(const uint16_t* __restrict__ base, const uint16_t* __restrict__ A,
                      const uint16_t* __restrict__ W, const int32_t* __restrict__ prev,
                      int prev_stride, const float* __restrict__ temperature,
                      const int32_t* __restrict__ order, uint64_t seed, int B, int K, int V,
                      int r, int k, PartialBuf part, int n_strips, int n_parts) {
    constexpr bool kBalance = NWAVES == 8;
    // the two W buffers, [16 KS][kPitch] each (r == 16 KS), and the handoff
    // slots (160 KiB in all with eight wavefronts)
    __shared__ __attribute__((aligned(16))) uint16_t w_a[16 * KS * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t w_b[16 * KS * kPitch];
    __shared__ float4 hs[kBalance ? kHandoffSlots : 1];
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5;
    const int wave = threadIdx.x >> 6;
    const int slot = (blockIdx.y * NWAVES + wave) * 32 + (lane & 31);
    const bool active = slot < B;
    // lanes past B run request 0's row (every wave takes part in the MFMAs and
    // barriers) and store nothing
    const int b = active ? order[slot] : 0;
    const int p = clamp_token(prev[static_cast<size_t>(b) * prev_stride], V);
    const float T = temperature[b];
    const KeyLane kl = key_lane(T);
    const PhiloxRow ph = philox_row(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(k + 1),
                                    kTagDraft);
    // one epilogue per wavefront: the greedy one when no lane samples
    const bool wave_greedy = __all(!active || !(T > 0.0f));
    // Roles: helper h in {0, 1} (greedy) serves wavefronts h + 2 and h + 6
    // (one SIMD) when both sample.  The flags go through the handoff slots,
    // which are first written after the first strip's barrier.
    int role = kRoleNone;
    int hidx = 0;
    Helper H;
    if constexpr (kBalance) {
        int* flags = reinterpret_cast<int*>(hs);
        if (lane == 0) flags[wave] = wave_greedy ? 1 : 0;
        lds_barrier();
        const int h = wave & 1;
        const bool pair = flags[h] && !flags[h + 2] && !flags[h + 6];
        if (wave < 2 && pair) role = kRoleHelper;
        if (wave >= 2 && (wave & 3) >= 2 && pair) {
            role = kRoleHelped;
            hidx = (wave < 4) ? wave - 2 : wave - 4;
        }
        if (role == kRoleHelper) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int hslot = (blockIdx.y * NWAVES + wave + 2 + 4 * j) * 32 + (lane & 31);
                const int hb = hslot < B ? order[hslot] : 0;
                H.kl[j] = key_lane(temperature[hb]);
                H.ph[j] = philox_row(seed, static_cast<uint32_t>(hb), static_cast<uint32_t>(k + 1),
                                     kTagDraft);
                H.run[j] = lane_empty();
            }
        }
    }
    const uint16_t* arow = A + static_cast<size_t>(p) * r + 8 * kh;
    const uint16_t* brow = base + (static_cast<size_t>(b) * K + k) * V;
    uint4 afr[KS];  // r == 16 KS
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) afr[kk] = *reinterpret_cast<const uint4*>(arow + 16 * kk);
    const int tro[2][2] = {{tr_offset(lane, 0, 0), tr_offset(lane, 0, 1)},
                           {tr_offset(lane, 1, 0), tr_offset(lane, 1, 1)}};
    LaneRun lr = lane_empty();
    const int s = blockIdx.x;  // < n_strips: the launch has n_parts <= n_strips
    // With balancing every wavefront meets two more barriers after its strips:
    // after the first every handoff slot has been read, and the helpers' states
    // for the helped lanes go through LDS to be merged into the owners'.
    if (wave_greedy) {
        if (kBalance && role == kRoleHelper) {
            rk_strips<NWAVES, KS, true, kRoleHelper>(w_a, w_b, s, lr, W, brow, afr, tro, kl, ph, V,
                                                     kh, n_strips, n_parts, hs, hidx, H);
            lds_barrier();
#pragma unroll
            for (int j = 0; j < 2; ++j)
                hs[(wave + 2 * j) * 64 + lane] =
                    make_float4(H.run[j].m2, H.run[j].s, H.run[j].key, __int_as_float(H.run[j].idx));
            lds_barrier();
        } else {
            rk_strips<NWAVES, KS, true, kRoleNone>(w_a, w_b, s, lr, W, brow, afr, tro, kl, ph, V,
                                                   kh, n_strips, n_parts, hs, hidx, H);
            if constexpr (kBalance) {
                lds_barrier();
                lds_barrier();
            }
        }
    } else {
        if (kBalance && role == kRoleHelped) {
            rk_strips<NWAVES, KS, false, kRoleHelped>(w_a, w_b, s, lr, W, brow, afr, tro, kl, ph,
                                                      V, kh, n_strips, n_parts, hs, hidx, H);
            lds_barrier();
            lds_barrier();
            const float4 q = hs[hidx * 64 + lane];
            run_merge(lr, LaneRun{q.x, q.y, q.z, __float_as_int(q.w)});
        } else {
            rk_strips<NWAVES, KS, false, kRoleNone>(w_a, w_b, s, lr, W, brow, afr, tro, kl, ph, V,
                                                    kh, n_strips, n_parts, hs, hidx, H);
            if constexpr (kBalance) {
                lds_barrier();
                lds_barrier();
            }
        }
    }
    // lanes l and l + 32 hold the two halves of every strip for one request
    RowState run = lane_row(lr);
    row_merge(run, xlane_row<5>(run));
    if (active && kh == 0)
        store_partial(part, static_cast<size_t>(b) * n_parts + blockIdx.x, run);
}

// ------------------------------------------ parallel drafting (no Markov head)
// With no transition factors the draft distribution of position k is
// softmax(base_k / T) on its own, so all B K rows are drawn in one launch:
// the same half-strip sampler (sample_half / greedy_half) on zero bias, lanes
// walking the strips of their row.  Slot s is row (order[s / K], s % K); partials are
// stored per row.
template <int NWAVES>
__global__ __launch_bounds__(64 * NWAVES)
void draft_rows_parallel(const uint16_t* __restrict__ base, const float* __restrict__ temperature,
                         const int32_t* __restrict__ order, uint64_t seed, int B, int K, int V,
                         PartialBuf part, int n_strips, int n_parts) {
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5;
    const int rows = B * K;
    const int slot = (blockIdx.y * NWAVES + (threadIdx.x >> 6)) * 32 + (lane & 31);
    const bool active = slot < rows;
    const int sl = active ? slot : 0;
    const int b = order[sl / K];
    const int k = sl - (sl / K) * K;
    const int row = b * K + k;
    const float T = temperature[b];
    const KeyLane kl = key_lane(T);
    const PhiloxRow ph = philox_row(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(k + 1),
                                    kTagDraft);
    const bool wave_greedy = __all(!active || !(T > 0.0f));
    const uint16_t* brow = base + static_cast<size_t>(row) * V;
    LaneRun lr = lane_empty();
    for (int s = blockIdx.x; s < n_strips; s += n_parts) {
        uint4 bl[8];
        load_strip_logits(bl, brow, s * kStripV, kh, V);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            f32x16 acc[2];
            acc_from_logits(acc, half_of(bl, h));
            if (wave_greedy)
                greedy_half(lr, acc, s * kStripV + 64 * h + 8 * kh);
            else
                sample_half(lr, acc, s * kStripV + 64 * h + 8 * kh, kl, ph);
        }
    }
    RowState run = lane_row(lr);
    row_merge(run, xlane_row<5>(run));
    if (active && kh == 0) store_partial(part, static_cast<size_t>(row) * n_parts + blockIdx.x, run);
}

// --------------------------------------------------------------- residual
// For every request whose first rejection is at j* = a_b + 1 (sampled, T > 0):
// recompute the draft logits at j* (previous token x_{j*-1}), read the target
// row, and draw from normalise(max(0, p_t - p_d)) and, as the fallback for a
// residual without positive mass, from p_t: per entry the keys
//   fallback  kf = log2 p_t - log2(-log2 u)
//   residual  kr = kf + log2(1 - p_d / p_t)   (entries with p_t > p_d only)
// with the entry's tag-2 draw at position j*, kept as two running argmaxes.
// In base 2 with c = log2(e) / T: a = log2 p_t = t c - lse_t log2(e), and
// dm = log2 p_d - log2 p_t = (s - t) c + (lse_t - lse_d) log2(e), formed from
// the logit difference so that a target row equal to the draft row gives the
// same dm for every such entry.  These keys are log2(e) (log r + G) and
// log2(e) (y + G) up to constants shared by the row.  Rejected requests are
// listed in `list` (count entries), and so are sampled requests that accepted
// every drafted token: their bonus token is exactly the fallback draw over
// row L_b + 1, and they take no residual key.
// verify_residual_combine merges the partials into the next token.  The key
// arithmetic is residual_entry (common.hpp).
// Persistent like the draft kernel: one workgroup per (part, slot group) walks
// the strips part, part + n_parts, ... with W double-buffered in LDS.
template <int NWAVES>
__global__ __launch_bounds__(64 * NWAVES) void residual_strip_mfma(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ target,
    const int64_t* __restrict__ row_off, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ prev_token, const float* __restrict__ draft_lse,
    const float* __restrict__ temperature, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ list, const int32_t* __restrict__ count_ptr,
    const int32_t* __restrict__ lengths, const float* __restrict__ lse_tab, uint64_t seed, int B,
    int K,
    int V, int r, PartialBuf res, PartialBuf fall, int n_strips, int n_parts) {
    extern __shared__ uint16_t w_sh[];  // two buffers of [r][kPitch]
    const int count = listed_count(count_ptr);
    const int slot0 = blockIdx.y * NWAVES * 32;
    if (slot0 >= count) return;  // whole workgroup idle
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5;
    const int slot = slot0 + (threadIdx.x >> 6) * 32 + (lane & 31);
    const bool active = slot < count;
    // waves wholly past the list only help stage W and meet the barriers
    const bool wave_busy = slot0 + (threadIdx.x >> 6) * 32 < count;
    // lanes past the list run request list[0]'s rows and store nothing
    const int b = listed_request(list, count_ptr, B, active ? slot : 0);
    const int js = accepted[b] + 1;
    // js > L_b: a full acceptance listed for its bonus, which is this kernel's
    // fallback draw over row L_b + 1; it takes no residual draw, and its draft
    // side reads row 1 as an in-range stand-in
    const bool bonus = js > (lengths ? clamp_len(lengths[b], K) : K);
    const int jd = bonus ? 1 : js;
    const int p = clamp_token((jd == 1) ? prev_token[b]
                                        : tokens[static_cast<size_t>(b) * K + jd - 2],
                              V);
    const float T = temperature[b];
    ResRow R;
    R.c2 = inv_temperature(T) * kLog2e;
    R.lt2 = lse_tab[static_cast<size_t>(b) * (K + 1) + js - 1] * kLog2e;
    R.dl = R.lt2 - draft_lse[static_cast<size_t>(b) * K + jd - 1] * kLog2e;
    R.bonus = bonus;
    R.kl = key_lane(T);
    R.ph = philox_row(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(js), kTagResample);
    const uint16_t* arow = A + static_cast<size_t>(p) * r + 8 * kh;
    const uint16_t* brow = base + (static_cast<size_t>(b) * K + jd - 1) * V;
    const uint16_t* trow = target + (row_off[b] + js - 1) * static_cast<int64_t>(V);
    const int buf_elems = r * kPitch;

    int s = blockIdx.x;  // < n_strips: the launch has n_parts <= n_strips
    stage_w<NWAVES>(w_sh, W, r, V, s * kStripV);
    ResBest best = res_empty();
    int buf = 0;
    for (;;) {
        __builtin_amdgcn_s_waitcnt(0);  // this strip's W (all waves' shares) has landed
        __syncthreads();
        const int sn = s + n_parts;
        const bool more = sn < n_strips;
        if (!wave_busy) {
            if (more) stage_w<NWAVES>(w_sh + (buf ^ 1) * buf_elems, W, r, V, sn * kStripV);
            if (!more) break;
            buf ^= 1;
            s = sn;
            continue;
        }
        const int v0 = s * kStripV;
        const int vh = v0 + 16 * kh;
        const bool tail = v0 + kStripV > V;
        uint4 bl[8], tl[8];
        load_lane_logits(bl, brow, vh, V, tail);
        load_lane_logits(tl, trow, vh, V, tail);
        f32x16 acc[4];
        bias_tiles(acc, w_sh + buf * buf_elems, arow, r, lane);
        // requested after the MFMA loop's factor loads (in-order load counter)
        if (more) stage_w<NWAVES>(w_sh + (buf ^ 1) * buf_elems, W, r, V, sn * kStripV);
        // accumulator i of tile t is entry vh + entry_of(i, t); the four tiles
        // of accumulator i are the four entries of one Philox block
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const u32x4 rnd =
                philox_row_block(R.ph, static_cast<uint32_t>((vh + entry_of(i, 0)) >> 2));
#pragma unroll
            for (int t = 0; t < 4; ++t)
                residual_entry(best, logit_at(bl, i, t) + acc[t][i], logit_at(tl, i, t),
                               pick(rnd, t), vh + entry_of(i, t), R);
        }
        if (!more) break;
        buf ^= 1;
        s = sn;
    }
    RowState sr{-INFINITY, 0.0f, best.br, 0.0f, best.ir};
    RowState sf{-INFINITY, 0.0f, best.bf, 0.0f, best.jf};
    row_merge(sr, xlane_row<5>(sr));
    row_merge(sf, xlane_row<5>(sf));
    if (active && kh == 0) {
        store_partial(res, static_cast<size_t>(slot) * n_parts + blockIdx.x, sr);
        store_partial(fall, static_cast<size_t>(slot) * n_parts + blockIdx.x, sf);
    }
}

// ------------------------------------------------------------ visit order
// Requests are visited greedy (T == 0) first, then sampled, each kind in
// request order, so a wavefront rarely mixes the two epilogues.  With more
// than one request group (kOrderGroup slots each, one workgroup row of the
// strip kernels) every group takes its share of the greedy requests, greedy
// first: group g holds greedy ranks [Q(g), Q(g + 1)), Q(g) = floor(n_greedy
// g kOrderGroup / B), then the sampled ones that fill it.  Groups of one
// kind only would give the launch workgroups of very different length.
// One workgroup.
constexpr int kOrderGroup = 256;

__device__ __forceinline__ int order_slot(int rank, bool greedy, int n_greedy, int B) {
    auto q = [&](int slot) {
        return static_cast<int>(static_cast<int64_t>(n_greedy) * slot / B);
    };
    int g = 0;
    while (true) {
        const int end = min((g + 1) * kOrderGroup, B);
        if (greedy ? rank < q(end) : rank < end - q(end)) break;
        ++g;
    }
    const int start = g * kOrderGroup;
    const int q0 = q(start), q1 = q(min(start + kOrderGroup, B));
    return greedy ? start + (rank - q0) : start + (q1 - q0) + (rank - (start - q0));
}

__global__ __launch_bounds__(1024) void temperature_order(const float* __restrict__ temperature,
                                                          int B, int32_t* __restrict__ order) {
    __shared__ int sh[1024 / kWave];
    __shared__ int sh_total;
    const int tid = threadIdx.x;
    int local = 0;
    for (int b = tid; b < B; b += 1024) local += !(temperature[b] > 0.0f);
    for (int msk = 32; msk >= 1; msk >>= 1) local += __shfl_xor(local, msk, kWave);
    if ((tid & 63) == 0) sh[tid >> 6] = local;
    __syncthreads();
    if (tid == 0) {
        int t = 0;
        for (int w = 0; w < 1024 / kWave; ++w) t += sh[w];
        sh_total = t;
    }
    __syncthreads();
    const int n_greedy = sh_total;
    int off_g = 0, off_s = 0;  // ranks among the greedy / sampled requests
    for (int c0 = 0; c0 < B; c0 += 1024) {
        const int b = c0 + tid;
        const int g = (b < B) && !(temperature[b] > 0.0f);
        const int s = (b < B) && !g;
        int ig = g, is = s;
        const int lane = tid & 63;
        for (int d = 1; d < kWave; d <<= 1) {
            const int og = __shfl_up(ig, d, kWave);
            const int os = __shfl_up(is, d, kWave);
            if (lane >= d) {
                ig += og;
                is += os;
            }
        }
        __syncthreads();
        if (lane == 63) sh[tid >> 6] = ig | (is << 16);
        __syncthreads();
        int bg = 0, bs = 0, tg = 0, ts = 0;
        for (int w = 0; w < 1024 / kWave; ++w) {
            const int vg = sh[w] & 0xFFFF, vs = sh[w] >> 16;
            if (w < (tid >> 6)) {
                bg += vg;
                bs += vs;
            }
            tg += vg;
            ts += vs;
        }
        if (g) order[order_slot(off_g + bg + ig - 1, true, n_greedy, B)] = b;
        if (s) order[order_slot(off_s + bs + is - 1, false, n_greedy, B)] = b;
        off_g += tg;
        off_s += ts;
    }
}

// ------------------------------------------------- residual: rank 256
// The residual strip of residual_strip_mfma for rank 256, built like
// draft_strip_mfma_rk: factor fragments in registers (the MFMA loops issue no
// vector-memory loads), W double-buffered in two static LDS arrays, and a
// strip worked in two 64-entry halves.  The base and target
// logits of a half are loaded one phase ahead into registers that the phase
// before has freed: a strip's half-1 base logits go out before the next
// strip's W, so waiting for them never waits for that W.

// Keys of one half (see residual_strip_mfma): acc holds s = base + bias, tq
// the target logits in the same entry layout (acc_from_logits): entry
// vh + 16 a + 4 tt + w is accumulator 4 a + w of tile tt ^ (a % 2) and element
// 4 tt + w of chunk a.
__device__ __forceinline__ void residual_half(ResBest& rb, const f32x16 (&acc)[2],
                                              const uint4 (&tq)[4], int vh, const ResRow& R) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 rnd = philox_row_block(R.ph, static_cast<uint32_t>(vh >> 2) + 4 * a + tt);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t dw = dword_of(tq[a], 2 * tt + (w >> 1));
                const float tv = __uint_as_float((w & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
                residual_entry(rb, acc[tt ^ (a & 1)][4 * a + w], tv, pick(rnd, w),
                               vh + 16 * a + 4 * tt + w, R);
            }
        }
    }
}

// Fallback keys only, for a wavefront of listed full acceptances (their bonus
// draw is the fallback draw over row L_b + 1): the same keys as residual_half
// gives them, with no draft row.
__device__ __forceinline__ void bonus_half(ResBest& rb, const uint4 (&tq)[4], int vh,
                                           const ResRow& R) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const u32x4 rnd = philox_row_block(R.ph, static_cast<uint32_t>(vh >> 2) + 4 * a + tt);
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const uint32_t dw = dword_of(tq[a], 2 * tt + (w >> 1));
                const float tv = __uint_as_float((w & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
                const float kf = fmaf(tv, R.c2, -R.lt2) - entry_l2(pick(rnd, w), R.kl);
                if (kf > rb.bf) {
                    rb.bf = kf;
                    rb.jf = vh + 16 * a + 4 * tt + w;
                }
            }
        }
    }
}

struct ResLane {
    const uint16_t* brow;
    const uint16_t* trow;
    ResRow R;
    ResBest best;
};

// One strip of a wave with no draft row to recompute: this strip's W is in
// `cur`, the next strip's goes into `nxt`.  A wave with no listed request only
// stages its share of W; a wave of listed full acceptances (bonus_only) also
// keys the target row alone (t0 holds this strip's half-0 target logits on
// entry and the next strip's on return).  The barrier and W staging match
// residual_rk_pipe's, so waves of both kinds share a workgroup.
template <int NWAVES, int KS>
__device__ __forceinline__ bool residual_rk_light(const uint16_t* cur, uint16_t* nxt, int& s,
                                                  uint4 (&t0)[4], ResLane& L,
                                                  const uint16_t* __restrict__ W, int V, int kh,
                                                  int n_strips, int n_parts, bool bonus_only) {
    // this strip's W (all waves' shares) and logits have landed, and every
    // wave is done with the other buffer
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int v0 = s * kStripV;
    const int sn = s + n_parts;
    const bool more = sn < n_strips;
    if (!bonus_only) {
        if (!more) return false;
        stage_w_tr<NWAVES>(nxt, W, 16 * KS, V, sn * kStripV);
        s = sn;
        return true;
    }
    uint4 t1[4];
    load_half(t1, L.trow, v0, 1, kh, V);
    if (more) stage_w_tr<NWAVES>(nxt, W, 16 * KS, V, sn * kStripV);
    bonus_half(L.best, t0, v0 + 8 * kh, L.R);
    if (more) load_half(t0, L.trow, sn * kStripV, 0, kh, V);
    bonus_half(L.best, t1, v0 + 64 + 8 * kh, L.R);
    if (!more) return false;
    s = sn;
    return true;
}

// Four bf16 -inf: the piece that stands in for tile pieces past V.
__device__ uint2 kNegInfPiece = {0xFF80FF80u, 0xFF80FF80u};

// The four 8-byte pieces of one tile's entries in a row (acc_from_logits'
// layout): piece g holds entries 16 g + 4 (ts ^ (g % 2)) + 0..3 of the lane's
// half, whose values accumulator 4 g + w of the tile holds.  A piece starts
// on a multiple of 4 and V is a multiple of 8, so a piece is wholly below V or
// wholly past it; pieces past V read the -inf piece.
__device__ __forceinline__ void load_tile(uint2 (&q)[4], const uint16_t* row, int v0, int h, int ts,
                                          int kh, int V) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int v = v0 + 64 * h + 16 * g + 8 * kh + 4 * (ts ^ (g & 1));
        const uint2* p = (v < V) ? reinterpret_cast<const uint2*>(row + v) : &kNegInfPiece;
        q[g] = *p;
    }
}

__device__ __forceinline__ float piece_value(const uint2 (&q)[4], int g, int w) {
    const uint32_t dw = (w >> 1) ? q[g].y : q[g].x;
    return __uint_as_float((w & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
}

__device__ __forceinline__ void tile_from_pieces(f32x16& acc, const uint2 (&q)[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int w = 0; w < 4; ++w) acc[4 * g + w] = piece_value(q, g, w);
}

// The residual counterpart of rk_unit: the KS bias MFMAs of one tile into accm
// and, in the same instruction stream, the residual and fallback keys of the
// tile before (accs, with its target pieces tq) into rb, cut into KS slices
// fenced by sched_barrier (slice kk: the MFMA of rank step kk, entry kk of the
// previous tile, an eighth of the next draw block's Philox rounds).
template <int KS, bool SAMPLE>
__device__ __forceinline__ void res_unit(f32x16& accm, const uint16_t* wt, const uint4 (&afr)[KS],
                                         const f32x16& accs, const uint2 (&tq)[4], ResBest& rb,
                                         int vs, int ts, const ResRow& R) {
    static_assert(KS == 16, "the slice schedule covers 16 rank steps (four Philox blocks)");
    uint2 lo[3], hi[3];
    lo[0] = lds_tr16(wt);
    hi[0] = lds_tr16(wt + 4 * kPitch);
    lo[1] = lds_tr16(wt + 16 * kPitch);
    hi[1] = lds_tr16(wt + 16 * kPitch + 4 * kPitch);
    PhiloxState cur{}, nxt{};
    if constexpr (SAMPLE) {
        nxt = philox_head(R.ph, static_cast<uint32_t>((vs + 4 * ts) >> 2));
#pragma unroll
        for (int i = 4; i <= 10; ++i) philox_round(nxt, R.ph, i);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
        if (kk + 2 < KS) {
            lo[(kk + 2) % 3] = lds_tr16(wt + (kk + 2) * 16 * kPitch);
            hi[(kk + 2) % 3] = lds_tr16(wt + (kk + 2) * 16 * kPitch + 4 * kPitch);
        }
        const uint4 a = make_uint4(lo[kk % 3].x, lo[kk % 3].y, hi[kk % 3].x, hi[kk % 3].y);
        accm = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(afr[kk]), accm, 0, 0,
                                                       0);
        if constexpr (SAMPLE) {
            const int g = kk >> 2, w = kk & 3;
            if (w == 0) cur = nxt;
            const int o = 16 * g + 4 * (ts ^ (g & 1));
            residual_entry(rb, accs[4 * g + w], piece_value(tq, g, w), state_word(cur, w),
                           vs + o + w, R);
            if (g < 3) {
                const int gn = g + 1;
                if (w == 0) {
                    nxt = philox_head(R.ph,
                                      static_cast<uint32_t>((vs + 16 * gn + 4 * (ts ^ (gn & 1))) >> 2));
                    philox_round(nxt, R.ph, 4);
                } else {
                    philox_round(nxt, R.ph, 2 * w + 3);
                    philox_round(nxt, R.ph, 2 * w + 4);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The keys of one tile with no MFMAs beside them (the last tile of a launch).
__device__ __forceinline__ void res_tile(ResBest& rb, const f32x16& acc, const uint2 (&tq)[4],
                                         int vs, int ts, const ResRow& R) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const int o = 16 * g + 4 * (ts ^ (g & 1));
        const u32x4 rnd = philox_row_block(R.ph, static_cast<uint32_t>((vs + o) >> 2));
#pragma unroll
        for (int w = 0; w < 4; ++w)
            residual_entry(rb, acc[4 * g + w], piece_value(tq, g, w), pick(rnd, w), vs + o + w, R);
    }
}

// One strip of a wave that recomputes draft rows, software-pipelined a tile at
// a time like rk_strip (tiles 0..3 = half 0 tiles 0, 1, half 1 tiles 0, 1):
// this strip's W is in `cur`, the next strip's goes into `nxt`.  Base logits go
// by half as in rk_strip (L0 / L1 hold this strip's halves on entry and the
// next strip's on return, each reloaded once both of its tiles are unpacked);
// target logits go by tile in a two-slot ring, Tq[u % 2] holding tile u's
// pieces, requested one tile ahead (as soon as tile u - 2 is keyed).  On entry
// T0 holds this strip's tile 0, T1 the previous strip's tile 3 and accB that
// tile's s (unkeyed); on return the same for the next strip.
template <int NWAVES, int KS, bool FIRST>
__device__ __forceinline__ bool residual_rk_pipe(const uint16_t* cur, uint16_t* nxt, int& s,
                                                 uint4 (&L0)[4], uint4 (&L1)[4], uint2 (&T0)[4],
                                                 uint2 (&T1)[4], f32x16& accA, f32x16& accB,
                                                 int& vsB, ResLane& L,
                                                 const uint16_t* __restrict__ W,
                                                 const uint4 (&afr)[KS], const int (&tro)[2][2],
                                                 int V, int kh, int n_strips, int n_parts) {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int v0 = s * kStripV;
    const int sn = s + n_parts;
    const bool more = sn < n_strips;
    const int vn = more ? sn * kStripV : v0;  // past the last strip: in-range loads, unused
    if (more) stage_w_tr<NWAVES>(nxt, W, 16 * KS, V, sn * kStripV);
    const int vh0 = v0 + 8 * kh, vh1 = v0 + 64 + 8 * kh;
    // tile 0 (keys the previous strip's tile 3)
    tile_from_logits(accA, L0, 0);
    res_unit<KS, !FIRST>(accA, cur + tro[0][0], afr, accB, T1, L.best, vsB, 1, L.R);
    load_tile(T1, L.trow, v0, 0, 1, kh, V);  // tile 1
    // tile 1 (keys tile 0)
    tile_from_logits(accB, L0, 1);
    load_half(L0, L.brow, vn, 0, kh, V);  // next strip's half 0
    res_unit<KS, true>(accB, cur + tro[0][1], afr, accA, T0, L.best, vh0, 0, L.R);
    load_tile(T0, L.trow, v0, 1, 0, kh, V);  // tile 2
    // tile 2 (keys tile 1)
    tile_from_logits(accA, L1, 0);
    res_unit<KS, true>(accA, cur + tro[1][0], afr, accB, T1, L.best, vh0, 1, L.R);
    load_tile(T1, L.trow, v0, 1, 1, kh, V);  // tile 3
    // tile 3 (keys tile 2)
    tile_from_logits(accB, L1, 1);
    load_half(L1, L.brow, vn, 1, kh, V);  // next strip's half 1
    res_unit<KS, true>(accB, cur + tro[1][1], afr, accA, T0, L.best, vh1, 0, L.R);
    load_tile(T0, L.trow, vn, 0, 0, kh, V);  // next strip's tile 0
    vsB = vh1;
    if (!more) return false;
    s = sn;
    return true;
}

template <int NWAVES, int KS>
__global__ __launch_bounds__(64 * NWAVES) void residual_strip_mfma_rk(
    const uint16_t* __restrict__ base, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ W, const uint16_t* __restrict__ target,
    const int64_t* __restrict__ row_off, const int32_t* __restrict__ tokens,
    const int32_t* __restrict__ prev_token, const float* __restrict__ draft_lse,
    const float* __restrict__ temperature, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ list, const int32_t* __restrict__ count_ptr,
    const int32_t* __restrict__ lengths, const float* __restrict__ lse_tab, uint64_t seed, int B,
    int K,
    int V, int r, PartialBuf res, PartialBuf fall, int n_strips, int n_wgs) {
    __shared__ __attribute__((aligned(16))) uint16_t w_a[16 * KS * kPitch];
    __shared__ __attribute__((aligned(16))) uint16_t w_b[16 * KS * kPitch];
    // The listed requests fill `groups` request groups; the n_wgs workgroups
    // of the grid are split over those groups only (the list's length is
    // known on the device alone), so that every CU works however long it is.
    // The launch has n_wgs >= the groups B requests can fill, so n_parts >= 1
    // parts of every group are covered.
    const int count = listed_count(count_ptr);
    const int groups = (count + NWAVES * 32 - 1) / (NWAVES * 32);
    if (groups == 0) return;
    const int n_parts = residual_parts(n_strips, n_wgs, groups);
    const int group = blockIdx.x / n_parts;
    const int part = blockIdx.x - group * n_parts;
    if (group >= groups) return;  // whole workgroup idle
    const int slot0 = group * NWAVES * 32;
    const int lane = threadIdx.x & 63;
    const int kh = lane >> 5;
    const int slot = slot0 + (threadIdx.x >> 6) * 32 + (lane & 31);
    const bool active = slot < count;
    // waves wholly past the list only stage W and meet the barriers
    const bool busy = slot0 + (threadIdx.x >> 6) * 32 < count;
    // lanes past the list run request list[0]'s rows and store nothing
    ResLane L;
    const int b = listed_request(list, count_ptr, B, active ? slot : 0);
    const int js = accepted[b] + 1;
    // js > L_b: a listed full acceptance (its bonus is the fallback draw over
    // row L_b + 1); its draft side reads row 1 as an in-range stand-in
    const bool bonus = js > (lengths ? clamp_len(lengths[b], K) : K);
    const int jd = bonus ? 1 : js;
    const int p =
        clamp_token((jd == 1) ? prev_token[b] : tokens[static_cast<size_t>(b) * K + jd - 2], V);
    const float T = temperature[b];
    L.R.c2 = inv_temperature(T) * kLog2e;
    L.R.lt2 = lse_tab[static_cast<size_t>(b) * (K + 1) + js - 1] * kLog2e;
    L.R.dl = L.R.lt2 - draft_lse[static_cast<size_t>(b) * K + jd - 1] * kLog2e;
    L.R.bonus = bonus;
    L.R.kl = key_lane(T);
    L.R.ph = philox_row(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(js), kTagResample);
    L.brow = base + (static_cast<size_t>(b) * K + jd - 1) * V;
    L.trow = target + (row_off[b] + js - 1) * static_cast<int64_t>(V);
    L.best = res_empty();
    const uint16_t* arow = A + static_cast<size_t>(p) * r + 8 * kh;
    // a wave whose listed requests are all full acceptances needs no draft row
    const bool bonus_only = busy && __all(!active || bonus);
    uint4 afr[KS];
    uint4 b0[4], t0[4];
    int s = part;  // < n_strips: n_parts <= n_strips
    if (busy && !bonus_only) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) afr[kk] = *reinterpret_cast<const uint4*>(arow + 16 * kk);
    }
    const int tro[2][2] = {{tr_offset(lane, 0, 0), tr_offset(lane, 0, 1)},
                           {tr_offset(lane, 1, 0), tr_offset(lane, 1, 1)}};
    stage_w_tr<NWAVES>(w_a, W, r, V, s * kStripV);
    if (busy && !bonus_only) {
        uint4 B0[4], B1[4];
        uint2 T0[4], T1[4];
        load_half(B0, L.brow, s * kStripV, 0, kh, V);
        load_half(B1, L.brow, s * kStripV, 1, kh, V);
        load_tile(T0, L.trow, s * kStripV, 0, 0, kh, V);
        f32x16 accA, accB;
        int vsB = 0;
        // strips alternate between w_a and w_b
        if (residual_rk_pipe<NWAVES, KS, true>(w_a, w_b, s, B0, B1, T0, T1, accA, accB, vsB, L, W,
                                               afr, tro, V, kh, n_strips, n_parts)) {
            while (residual_rk_pipe<NWAVES, KS, false>(w_b, w_a, s, B0, B1, T0, T1, accA, accB,
                                                       vsB, L, W, afr, tro, V, kh, n_strips,
                                                       n_parts) &&
                   residual_rk_pipe<NWAVES, KS, false>(w_a, w_b, s, B0, B1, T0, T1, accA, accB,
                                                       vsB, L, W, afr, tro, V, kh, n_strips,
                                                       n_parts)) {
            }
        }
        res_tile(L.best, accB, T1, vsB, 1, L.R);  // the last tile (half 1, tile 1)
    } else {
        if (busy) load_half(t0, L.trow, s * kStripV, 0, kh, V);
        while (residual_rk_light<NWAVES, KS>(w_a, w_b, s, t0, L, W, V, kh, n_strips, n_parts,
                                             bonus_only) &&
               residual_rk_light<NWAVES, KS>(w_b, w_a, s, t0, L, W, V, kh, n_strips, n_parts,
                                             bonus_only)) {
        }
    }
    // lanes l and l + 32 hold the two halves of every strip for one request
    RowState sr{-INFINITY, 0.0f, L.best.br, 0.0f, L.best.ir};
    RowState sf{-INFINITY, 0.0f, L.best.bf, 0.0f, L.best.jf};
    row_merge(sr, xlane_row<5>(sr));
    row_merge(sf, xlane_row<5>(sf));
    if (active && kh == 0) {
        store_partial(res, static_cast<size_t>(slot) * n_parts + part, sr);
        store_partial(fall, static_cast<size_t>(slot) * n_parts + part, sf);
    }
}

constexpr int kMaxLds = 160 * 1024;

// Devices a kernel's LDS limit has been raised on (the attribute is per device;
// raising it twice is harmless, so concurrent first calls need no lock).
struct LdsReady {
    std::atomic<bool> dev[64] = {};
};

// Let the kernel take all the LDS its static arrays leave, once per device.
template <typename Kern>
hipError_t allow_big_lds(Kern* kern, LdsReady& ready) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const bool track = dev >= 0 && dev < 64;
    if (track && ready.dev[dev].load(std::memory_order_acquire)) return hipSuccess;
    hipFuncAttributes fa;
    e = hipFuncGetAttributes(&fa, reinterpret_cast<const void*>(kern));
    if (e != hipSuccess) return e;
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLds - static_cast<int>(fa.sharedSizeBytes));
    if (e == hipSuccess && track) ready.dev[dev].store(true, std::memory_order_release);
    return e;
}

// `lds` is the dynamic LDS of the launch (0 for a kernel whose W buffers are
// static arrays).
template <int NWAVES, typename Kern>
hipError_t launch_draft_strip(Kern* kern, LdsReady& lds_ok, size_t lds, const DraftArgs& a,
                              const int32_t* prev, int prev_stride, int k, const int32_t* order,
                              PartialBuf part, int n_strips, int* n_parts) {
    hipError_t e = allow_big_lds(kern, lds_ok);
    if (e != hipSuccess) return e;
    // one resident workgroup per CU (the two W buffers take most of the LDS)
    const int groups = static_cast<int>(ceil_div(a.B, 32 * NWAVES));
    const int parts = std::max(1, std::min(n_strips, device_cus() / groups));
    *n_parts = parts;
    dim3 grid(static_cast<unsigned>(parts), static_cast<unsigned>(groups));
    hipLaunchKernelGGL(kern, grid, dim3(64 * NWAVES), lds, a.stream,
                       static_cast<const uint16_t*>(a.base), static_cast<const uint16_t*>(a.A),
                       static_cast<const uint16_t*>(a.W), prev, prev_stride, a.temperature, order,
                       a.seed, a.B, a.K, a.V, a.r, k, part, n_strips, parts);
    return hipGetLastError();
}

// Rank 256 takes the register-factor kernel; other ranks the runtime-rank one.
template <int NWAVES>
hipError_t launch_draft_step_nw(const DraftArgs& a, const int32_t* prev, int prev_stride, int k,
                                const int32_t* order, PartialBuf part, int n_strips,
                                int* n_parts) {
    if (a.r == 256) {
        static LdsReady lds_ok;
        return launch_draft_strip<NWAVES>(&draft_strip_mfma_rk<NWAVES, 16>, lds_ok, 0, a, prev,
                                          prev_stride, k, order, part, n_strips, n_parts);
    }
    static LdsReady lds_ok;
    const size_t lds = 2 * sizeof(uint16_t) * static_cast<size_t>(a.r) * kPitch;
    return launch_draft_strip<NWAVES>(&draft_strip_mfma<NWAVES>, lds_ok, lds, a, prev, prev_stride,
                                      k, order, part, n_strips, n_parts);
}

template <int NWAVES>
hipError_t launch_residual_strip(const ResidualArgs& a, ResGeom* geom) {
    const VerifyArgs& v = *a.v;
    if (v.r == 256) {
        static LdsReady lds_rk;
        hipError_t e = allow_big_lds(&residual_strip_mfma_rk<NWAVES, 16>, lds_rk);
        if (e != hipSuccess) return e;
        // one workgroup per CU, split on the device over the groups the list
        // fills, and at least one per request group the list can fill
        const int wgs =
            std::max(device_cus(), static_cast<int>(ceil_div(v.B, 32 * NWAVES)));
        *geom = ResGeom{0, wgs, NWAVES};
        hipLaunchKernelGGL((residual_strip_mfma_rk<NWAVES, 16>), dim3(static_cast<unsigned>(wgs)),
                           dim3(64 * NWAVES), 0, v.stream, static_cast<const uint16_t*>(v.base),
                           static_cast<const uint16_t*>(v.A), static_cast<const uint16_t*>(v.W),
                           static_cast<const uint16_t*>(v.target), v.row_off, v.tokens,
                           v.prev_token, v.draft_lse, v.temperature, v.accepted, a.list, a.count,
                           v.lengths, a.lse_tab, v.seed, v.B, v.K, v.V, v.r, a.res, a.fall, a.n_strips,
                           wgs);
        return hipGetLastError();
    }
    static LdsReady lds_ok;
    hipError_t e = allow_big_lds(&residual_strip_mfma<NWAVES>, lds_ok);
    if (e != hipSuccess) return e;
    const size_t lds = 2 * sizeof(uint16_t) * static_cast<size_t>(v.r) * kPitch;
    const int groups = static_cast<int>(ceil_div(v.B, 32 * NWAVES));
    const int parts = std::max(1, std::min(a.n_strips, device_cus() / groups));
    *geom = ResGeom{parts, 0, NWAVES};
    dim3 grid(static_cast<unsigned>(parts), static_cast<unsigned>(groups));
    hipLaunchKernelGGL(residual_strip_mfma<NWAVES>, grid, dim3(64 * NWAVES), lds, v.stream,
                       static_cast<const uint16_t*>(v.base), static_cast<const uint16_t*>(v.A),
                       static_cast<const uint16_t*>(v.W), static_cast<const uint16_t*>(v.target),
                       v.row_off, v.tokens, v.prev_token, v.draft_lse, v.temperature, v.accepted,
                       a.list, a.count, v.lengths, a.lse_tab, v.seed, v.B, v.K, v.V, v.r, a.res, a.fall,
                       a.n_strips, parts);
    return hipGetLastError();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

// Compute units of the current device, queried once per device (a racing
// first query stores the same value).
int device_cus() {
    static std::atomic<int> cus[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cus[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cus[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

int mfma_draft_strip() { return kStripV; }

bool parallel_supported(const DraftArgs& a) {
    return a.logit_dt == DSPARK_BF16 && a.V % 8 == 0 && aligned16(a.base);
}

hipError_t launch_draft_parallel(const DraftArgs& a, PartialBuf part, size_t part_capacity,
                                 const int32_t* order) {
    constexpr int NW = 8;
    const int64_t rows = static_cast<int64_t>(a.B) * a.K;
    const int n_strips = static_cast<int>(ceil_div(a.V, kStripV));
    const int groups = static_cast<int>(ceil_div(rows, 32 * NW));
    // a few workgroups per CU (no LDS), and no more partials than the workspace holds
    int parts = std::max(1, std::min(n_strips, 4 * device_cus() / groups));
    parts = static_cast<int>(
        std::max<int64_t>(1, std::min<int64_t>(parts, static_cast<int64_t>(part_capacity) / rows)));
    hipLaunchKernelGGL(draft_rows_parallel<NW>, dim3(static_cast<unsigned>(parts),
                                                     static_cast<unsigned>(groups)),
                       dim3(64 * NW), 0, a.stream, static_cast<const uint16_t*>(a.base),
                       a.temperature, order, a.seed, a.B, a.K, a.V, part, n_strips, parts);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_draft_combine(a, part, parts, static_cast<int>(rows), -1);
}

bool mfma_supported(const DraftArgs& a) {
    // two LDS buffers of r x 128 bf16 must fit in 160 KiB
    return a.factor_dt == DSPARK_BF16 && a.logit_dt == DSPARK_BF16 && a.r % 16 == 0 &&
           a.r <= 256 && a.V % 8 == 0 && aligned16(a.base) && aligned16(a.A) && aligned16(a.W);
}

bool residual_mfma_supported(const VerifyArgs& a) {
    return a.A != nullptr && a.factor_dt == DSPARK_BF16 && a.logit_dt == DSPARK_BF16 && a.r % 16 == 0 &&
           a.r <= 256 && a.V % 8 == 0 && aligned16(a.base) && aligned16(a.A) &&
           aligned16(a.W) && aligned16(a.target);
}

hipError_t launch_temperature_order(const float* temperature, int B, int32_t* order,
                                    hipStream_t stream) {
    hipLaunchKernelGGL(temperature_order, dim3(1), dim3(1024), 0, stream, temperature, B, order);
    return hipGetLastError();
}

hipError_t launch_draft_mfma_step(const DraftArgs& a, const int32_t* prev, int prev_stride, int k,
                                  const int32_t* order, PartialBuf part, int n_strips,
                                  int* n_parts) {
    if (a.B > 128)
        return launch_draft_step_nw<8>(a, prev, prev_stride, k, order, part, n_strips, n_parts);
    if (a.B > 64)
        return launch_draft_step_nw<4>(a, prev, prev_stride, k, order, part, n_strips, n_parts);
    return launch_draft_step_nw<2>(a, prev, prev_stride, k, order, part, n_strips, n_parts);
}

hipError_t launch_residual_mfma(const ResidualArgs& a, ResGeom* geom) {
    if (a.v->B > 128) return launch_residual_strip<8>(a, geom);
    if (a.v->B > 64) return launch_residual_strip<4>(a, geom);
    return launch_residual_strip<2>(a, geom);
}

}  // namespace dspark
