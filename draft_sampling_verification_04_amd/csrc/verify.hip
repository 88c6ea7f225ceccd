// verify.hip -- lossless rejection-sampling verification with strict prefix
// semantics (yage.ai DSpark analysis, paragraphs on prefix matching and on
// rejection sampling needing the exact draft probability; legalagi.cn reading,
// section 3).
//
// Request b verifies rows j = 1 .. L_b + 1 of the target (row L_b + 1 is the
// bonus row).  With y = t / T and p_t = softmax(y):
//   accept x_j  iff  log u_j < log p_t(x_j) - log p_d(x_j)   (T > 0)
//               iff  x_j == argmax t_j                        (T == 0)
//   a_b = leading accepts;  a_b < L_b: next ~ normalise(max(0, p_t - p_d)) at
//   j* = a_b + 1 (Gumbel-max over log of the positive residual entries, falling
//   back to p_t when no residual mass is left);  a_b = L_b: next ~ p_t of row
//   L_b + 1.  Every draw takes one tag-2 Philox draw per vocabulary entry.
//
// Launches: (1) one workgroup per (request, row) streams the target row once
// with 16-byte loads: log-normaliser, accept bit, argmax, and (when no residual
// kernel runs) the bonus Gumbel-max on row L_b + 1; (2) one thread per request
// finds the first rejection and lists the requests that need a draw; (3) the
// listed requests recompute their draft row at j* (rank-r bias on MFMA for
// bf16, VALU otherwise) and stream the target row j* again, split in
// vocabulary strips, keeping the best residual and fallback keys; (4) the
// strips are folded into the next token.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kResRows = 8;  // rejected requests per workgroup of the VALU residual kernel

struct VerifyWs {
    int32_t* accept;  // [B][K+1]
    int32_t* arg;     // [B][K+1] row argmax (T == 0)
    float* lse;       // [B][K+1] target log-normaliser per row
    int32_t* bonus;   // [B] next token candidate from row L_b + 1
    int32_t* list;    // [B] requests that need a residual draw
    int32_t* count;   // [1]
    PartialBuf res;   // [B][n_strips] residual Gumbel-max partials
    PartialBuf fall;  // [B][n_strips] fallback (p_t) Gumbel-max partials
};

// 16 bytes of a target row.  Target rows are streamed once per verify, so the
// loads are non-temporal: they then displace fewer cached lines, which took
// verify_rows from 241.5 to 231.7 us on the long-draft rows (1.32 GB), the time
// of the same loads with no arithmetic at all.
__device__ __forceinline__ uint4 load_stream16(const void* p) {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u t = __builtin_nontemporal_load(static_cast<const v4u*>(p));
    return make_uint4(t.x, t.y, t.z, t.w);
}

// Eight consecutive logits of a row as floats; `vec` = the row is 16-byte
// aligned and V is a multiple of the vector width, so a chunk starting below V
// is whole.  Entries past V read as -inf.
template <typename LT>
__device__ __forceinline__ void load8(const LT* row, int v0, int V, bool vec, float (&x)[8]);

template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* row, int v0, int V, bool vec,
                                              float (&x)[8]) {
    if (vec) {
        const uint4 q = load_stream16(row + v0);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[2 * i] = __uint_as_float(w[i] << 16);
            x[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (v0 + i < V) ? to_f32(row[v0 + i]) : -INFINITY;
    }
}

template <>
__device__ __forceinline__ void load8<float>(const float* row, int v0, int V, bool vec,
                                             float (&x)[8]) {
    if (vec) {
        const uint4 a = load_stream16(row + v0);
        const uint4 b = load_stream16(row + v0 + 4);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
        x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
        x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = (v0 + i < V) ? row[v0 + i] : -INFINITY;
    }
}

// Chunk v0 .. v0 + 7 of a row for the verify loop; entries past V read as
// -inf, which changes no maximum, sum of exponentials or argmax.  VEC
// (16-byte aligned rows, V % 8 == 0): an unconditional load, from the row's
// last chunk when v0 is past V, so that the loads of one loop iteration go out
// together with no branch between them.  Otherwise entries are read one by
// one below V.
template <typename LT, bool VEC>
__device__ __forceinline__ void row_chunk(const LT* row, int v0, int V, float (&x)[8]) {
    if constexpr (VEC) {
        load8<LT>(row, min(v0, V - 8), V, true, x);
        const bool past = v0 >= V;
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = past ? -INFINITY : x[e];
    } else {
        load8<LT>(row, v0, V, false, x);
    }
}

// The (request, row) of this workgroup, or live = false when the row cannot
// decide the request (past L_b + 1, out of range, or after a rejection found
// by an earlier launch).  Called by every thread of the workgroup.
struct RowJob {
    int b, j;
    int64_t row;
    float T;
    bool greedy, bonus, live;
};

__device__ __forceinline__ RowJob row_begin(const int64_t* __restrict__ row_off,
                                            const int32_t* __restrict__ lengths,
                                            const float* __restrict__ temperature, int K,
                                            int64_t n_rows, VerifyWs ws, int j_lo, int span) {
    RowJob job{};
    const int64_t id = blockIdx.x;
    // the residual list starts empty; verify_resolve appends to it after the
    // last launch of the row kernels
    if (j_lo == 1 && id == 0 && threadIdx.x < 2) ws.count[threadIdx.x] = 0;
    // this launch covers positions j_lo .. j_lo + span - 1 of every request
    job.b = static_cast<int>(id / span);
    job.j = static_cast<int>(id - static_cast<int64_t>(job.b) * span) + j_lo;
    const int L = lengths ? clamp_len(lengths[job.b], K) : K;
    job.live = false;
    if (job.j > L + 1) return job;
    if (row_off[job.b] < 0 || row_off[job.b] + L + 1 > n_rows) return job;  // reported by verify_resolve
    // Strict prefix: row j matters only while rows 1 .. j - 1 are all accepted.
    // Rows of earlier launches are decided (thread i reads row i + 1's flag);
    // a rejected one among them ends the request.
    if (j_lo > 1) {
        const int32_t* acc = ws.accept + static_cast<size_t>(job.b) * (K + 1);
        const bool rejected = threadIdx.x < j_lo - 1 && !acc[threadIdx.x];
        if (__syncthreads_or(rejected)) return job;
    }
    job.row = row_off[job.b] + (job.j - 1);
    job.T = temperature[job.b];
    job.greedy = !(job.T > 0.0f);
    job.bonus = (job.j == L + 1);
    job.live = true;
    return job;
}

// The end of a verified row, once its state is reduced (thread 0): the target
// log-normaliser, and the accept test of the drafted token (or the bonus
// candidate on row L_b + 1).
template <typename LT>
__device__ __forceinline__ void row_finish(const RowState& st, const LT* trow, int64_t row, int b,
                                           int j, bool greedy, bool bonus, float T,
                                           const int32_t* __restrict__ tokens,
                                           const float* __restrict__ draft_logp, uint64_t seed,
                                           int K, int V, float* __restrict__ row_lse_t,
                                           float* __restrict__ row_logratio, VerifyWs ws) {
    const size_t slot = static_cast<size_t>(b) * (K + 1) + (j - 1);
    const float lse_t = greedy ? st.pert : st.m + logf(st.s);
    ws.lse[slot] = lse_t;
    if (row_lse_t) row_lse_t[row] = lse_t;
    if (bonus) {
        ws.bonus[b] = st.idx;
        if (row_logratio) row_logratio[row] = 0.0f;
    } else {
        const int x = clamp_token(tokens[static_cast<size_t>(b) * K + (j - 1)], V);
        int acc;
        float ratio;
        if (!greedy) {
            const float yx = to_f32(trow[x]) * inv_temperature(T);
            ratio = (yx - lse_t) - draft_logp[static_cast<size_t>(b) * K + (j - 1)];
            const u32x4 rnd = philox_block(seed, b, j, kTagAccept, 0);
            acc = logf(uniform_of(rnd.x)) < ratio;
        } else {
            acc = (x == st.idx);
            ratio = acc ? 0.0f : -INFINITY;
        }
        ws.accept[slot] = acc;
        ws.arg[slot] = st.idx;
        if (row_logratio) row_logratio[row] = ratio;
    }
}

// verify_rows: one 512-thread workgroup per visited row with four 16-byte
// loads in flight per lane (512 threads measured best among 64 / 256 / 512 /
// 1024; four loads 4% faster than two on the long-draft step, 40 VGPRs -> 56).
constexpr int kVRowThreads = 512;
constexpr int kVRowUnroll = 4;

// One target row (job.live): its normaliser, argmax or bonus draw, reduced
// over the workgroup, and the row's end (row_finish).  Called by every thread.
template <typename LT, bool VEC>
__device__ __forceinline__ void verify_row(const RowJob& job, const LT* __restrict__ target,
                                           const int32_t* __restrict__ tokens,
                                           const float* __restrict__ draft_logp, uint64_t seed,
                                           int K, int V, bool bonus_draw,
                                           float* __restrict__ row_lse_t,
                                           float* __restrict__ row_logratio, VerifyWs ws,
                                           RowState* red) {
    const int b = job.b, j = job.j;
    const int64_t row = job.row;
    const float T = job.T;
    const bool greedy = job.greedy, bonus = job.bonus;
    // the sampled bonus draw is made here only when the residual kernel does
    // not make it (bonus_draw); the normaliser is always computed
    const bool draw = bonus && bonus_draw;
    const LT* trow = target + row * static_cast<int64_t>(V);
    RowState st = row_empty();
    if (greedy) {
        // argmax of t, smallest index on ties (visited in increasing v per thread)
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int c0 = threadIdx.x * 8; c0 < V; c0 += kVRowThreads * 8 * kVRowUnroll) {
            float xs[kVRowUnroll][8];
#pragma unroll
            for (int u = 0; u < kVRowUnroll; ++u) {
                const int v0 = c0 + u * kVRowThreads * 8;
                row_chunk<LT, VEC>(trow, v0, V, xs[u]);
            }
#pragma unroll
            for (int u = 0; u < kVRowUnroll; ++u) {
                const int v0 = c0 + u * kVRowThreads * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (xs[u][e] > best) {
                        best = xs[u][e];
                        bi = v0 + e;
                    }
                }
            }
        }
        st.pert = best;
        st.zb = best;
        st.idx = bi;
    } else {
        // log sum_v exp(t_v / T) around the running maximum m of t:
        // s = sum 2^((t - m) c) with c = log2(e) / T
        const float it = inv_temperature(T);
        const float c = it * kLog2e;
        const KeyLane kl = key_lane(T);
        const PhiloxRow ph = draw ? philox_row(seed, static_cast<uint32_t>(b),
                                               static_cast<uint32_t>(j), kTagResample)
                                  : PhiloxRow{};
        float m = -INFINITY, s = 0.0f;
        float best = -INFINITY;
        int bi = 0x7fffffff;
        for (int c0 = threadIdx.x * 8; c0 < V; c0 += kVRowThreads * 8 * kVRowUnroll) {
          float xs[kVRowUnroll][8];
#pragma unroll
          for (int u = 0; u < kVRowUnroll; ++u) {
            const int v0 = c0 + u * kVRowThreads * 8;
            row_chunk<LT, VEC>(trow, v0, V, xs[u]);
          }
#pragma unroll
          for (int u = 0; u < kVRowUnroll; ++u) {
            const int v0 = c0 + u * kVRowThreads * 8;
            const float (&x)[8] = xs[u];
            float cm = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                             fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
            if (cm > m) {
                s *= __builtin_amdgcn_exp2f((m - cm) * c);
                m = cm;
            }
            // a thread may meet a chunk wholly past the row (-inf) before any
            // entry: then m = -inf and the reference is 0
            const float mc = (m == -INFINITY) ? 0.0f : m * c;
#pragma unroll
            for (int e = 0; e < 8; ++e) s += __builtin_amdgcn_exp2f(fmaf(x[e], c, -mc));
            if (draw && v0 < V) {
                // bonus draw: key t c - log2(-log2 u) per entry (tag 2), two
                // Philox blocks per chunk; entries past V read -inf
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const u32x4 rnd = philox_row_block(ph, static_cast<uint32_t>(v0 >> 2) + h);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float key = fmaf(x[4 * h + e], c, -entry_l2(pick(rnd, e), kl));
                        if (key > best) {
                            best = key;
                            bi = v0 + 4 * h + e;
                        }
                    }
                }
            }
          }
        }
        // express (m, s) on the y = t / T scale for the shared merge
        st.m = m * it;
        st.s = s;
        st.pert = best;
        st.zb = best;
        st.idx = bi;
    }
    st = block_reduce_row<kVRowThreads>(st, red);
    if (threadIdx.x == 0)
        row_finish(st, trow, row, b, j, greedy, bonus, T, tokens, draft_logp, seed, K, V, row_lse_t,
                   row_logratio, ws);
}

template <typename LT, bool VEC>
__global__ __launch_bounds__(kVRowThreads) void verify_rows(
    const LT* __restrict__ target, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ tokens,
    const float* __restrict__ draft_logp, const float* __restrict__ temperature, uint64_t seed,
    int K, int V, int64_t n_rows, bool bonus_draw, float* __restrict__ row_lse_t,
    float* __restrict__ row_logratio, VerifyWs ws, int j_lo, int span) {
    __shared__ RowState red[kVRowThreads / kWave];
    const RowJob job = row_begin(row_off, lengths, temperature, K, n_rows, ws, j_lo, span);
    if (!job.live) return;
    verify_row<LT, VEC>(job, target, tokens, draft_logp, seed, K, V, bonus_draw, row_lse_t,
                        row_logratio, ws, red);
}

// The second launch of the decisive rows (positions j_lo .. L_b + 1, after
// the launch of positions 1 .. j_lo - 1) over a fixed grid: every workgroup
// first lists, in LDS, the rows still needed, those of the requests whose rows
// 1 .. j_lo - 1 were all accepted, then takes rows blockIdx.x, blockIdx.x +
// gridDim.x, ... of that list.  A one-row-per-workgroup grid over every
// (request, position) spent most of its workgroups on requests already
// rejected.  B <= kTailMaxB.
constexpr int kTailMaxB = 4096;

template <typename LT, bool VEC>
__global__ __launch_bounds__(kVRowThreads) void verify_rows_tail(
    const LT* __restrict__ target, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ tokens,
    const float* __restrict__ draft_logp, const float* __restrict__ temperature, uint64_t seed,
    int B, int K, int V, int64_t n_rows, bool bonus_draw, VerifyWs ws, int j_lo) {
    __shared__ RowState red[kVRowThreads / kWave];
    __shared__ int pre[kTailMaxB];  // exclusive prefix of the rows each request needs
    __shared__ int wsum[kVRowThreads / kWave];
    __shared__ int total;
    constexpr int kPer = kTailMaxB / kVRowThreads;  // requests per thread
    int cnt[kPer];
    int mine = 0;
    const int b0 = threadIdx.x * kPer;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = b0 + i;
        int n = 0;
        if (b < B) {
            const int L = lengths ? clamp_len(lengths[b], K) : K;
            const int64_t o = row_off[b];
            if (L + 1 >= j_lo && o >= 0 && o + L + 1 <= n_rows) {
                n = L + 2 - j_lo;
                const int32_t* acc = ws.accept + static_cast<size_t>(b) * (K + 1);
                for (int q = 0; q < j_lo - 1; ++q) n = acc[q] ? n : 0;
            }
        }
        cnt[i] = n;
        mine += n;
    }
    // exclusive scan of the per-thread totals: within each wavefront, then
    // over the wavefront totals
    const int lane = threadIdx.x & (kWave - 1);
    int inc = mine;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(inc, d, kWave);
        if (lane >= d) inc += o;
    }
    if (lane == kWave - 1) wsum[threadIdx.x / kWave] = inc;
    __syncthreads();
    int before = 0, all = 0;
    for (int w = 0; w < kVRowThreads / kWave; ++w) {
        before += (w < static_cast<int>(threadIdx.x / kWave)) ? wsum[w] : 0;
        all += wsum[w];
    }
    int run = before + inc - mine;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        if (b0 + i < B) pre[b0 + i] = run;
        run += cnt[i];
    }
    if (threadIdx.x == 0) total = all;
    __syncthreads();
    const int n_jobs = total;
    for (int q = blockIdx.x; q < n_jobs; q += gridDim.x) {
        // the request of list entry q: the last b with pre[b] <= q
        int lo = 0, hi = B - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (pre[mid] <= q)
                lo = mid;
            else
                hi = mid - 1;
        }
        RowJob job{};
        job.b = lo;
        job.j = j_lo + (q - pre[lo]);
        const int L = lengths ? clamp_len(lengths[job.b], K) : K;
        job.row = row_off[job.b] + (job.j - 1);
        job.T = temperature[job.b];
        job.greedy = !(job.T > 0.0f);
        job.bonus = (job.j == L + 1);
        job.live = true;
        verify_row<LT, VEC>(job, target, tokens, draft_logp, seed, K, V, bonus_draw, nullptr,
                            nullptr, ws, red);
        __syncthreads();  // red is reused by the next row
    }
}

__global__ __launch_bounds__(256) void verify_resolve(int B, int K, int64_t n_rows,
                                                     const int64_t* __restrict__ row_off,
                                                     const int32_t* __restrict__ lengths,
                                                     const float* __restrict__ temperature,
                                                     bool bonus_in_list, VerifyWs ws,
                                                     int32_t* __restrict__ accepted,
                                                     int32_t* __restrict__ next_token) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= B) return;
    const int L = lengths ? clamp_len(lengths[b], K) : K;
    if (row_off[b] < 0 || row_off[b] + L + 1 > n_rows) {
        accepted[b] = 0;
        next_token[b] = -1;
        return;
    }
    const int32_t* acc = ws.accept + static_cast<size_t>(b) * (K + 1);
    int a = 0;
    while (a < L && acc[a]) ++a;
    accepted[b] = a;
    const bool sampled = temperature[b] > 0.0f;
    if (a == L && !(sampled && bonus_in_list)) {
        next_token[b] = ws.bonus[b];
    } else if (!sampled) {
        next_token[b] = ws.arg[static_cast<size_t>(b) * (K + 1) + a];
    } else if (a < L) {
        // a sampled first rejection: from the front of the list
        ws.list[atomicAdd(&ws.count[0], 1)] = b;
    } else {
        // (bonus_in_list) a sampled full acceptance whose bonus the residual
        // kernel draws as its fallback: from the back of the list
        ws.list[B - 1 - atomicAdd(&ws.count[1], 1)] = b;
    }
}

// Residual strip kernel, VALU form (fp32 inputs, or shapes the MFMA form does
// not take): workgroup = (8 rejected requests) x (1024 vocabulary entries);
// each thread keeps the best residual and fallback keys of its 4 entries.
template <typename LT, typename FT>
__global__ __launch_bounds__(256) void verify_residual_valu(
    const LT* __restrict__ base, const FT* __restrict__ A, const FT* __restrict__ W,
    const LT* __restrict__ target, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ prev_token,
    const float* __restrict__ draft_lse, const float* __restrict__ temperature,
    const int32_t* __restrict__ accepted, uint64_t seed, int B, int K, int V, int r, VerifyWs ws,
    int n_strips) {
    extern __shared__ float a_sh[];  // [kResRows][r]
    __shared__ RowState red_r[4][kResRows];
    __shared__ RowState red_f[4][kResRows];
    const int tid = threadIdx.x;
    const int slot0 = blockIdx.x * kResRows;
    const int count = listed_count(ws.count);
    if (slot0 >= count) return;
    const int nrows = min(kResRows, count - slot0);
    const int strip = blockIdx.y;
    for (int e = tid; e < kResRows * r; e += 256) {
        const int g = e / r;
        const int i = e - g * r;
        float a = 0.0f;
        if (A != nullptr && g < nrows) {
            const int b = listed_request(ws.list, ws.count, B, slot0 + g);
            const int js = accepted[b] + 1;
            const int p = clamp_token(
                (js == 1) ? prev_token[b] : tokens[static_cast<size_t>(b) * K + js - 2], V);
            a = to_f32(A[static_cast<size_t>(p) * r + i]);
        }
        a_sh[e] = a;
    }
    __syncthreads();
    const int v0 = strip * kValuStrip + tid * 4;
    float acc[kResRows][4];
#pragma unroll
    for (int g = 0; g < kResRows; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = 0.0f;
    if (A != nullptr && v0 < V) {  // A = W = NULL: no transition bias
        for (int i = 0; i < r; ++i) {
            const FT* wr = W + static_cast<size_t>(i) * V + v0;
            float w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = (v0 + t < V) ? to_f32(wr[t]) : 0.0f;
#pragma unroll
            for (int g = 0; g < kResRows; ++g) {
                const float a = a_sh[g * r + i];
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[g][t] = fmaf(a, w[t], acc[g][t]);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < kResRows; ++g) {
        if (g >= nrows) break;
        const int b = listed_request(ws.list, ws.count, B, slot0 + g);
        const int js = accepted[b] + 1;
        const float T = temperature[b];
        // keys of the thread's 4 entries (one Philox block), see residual_entry
        ResRow R;
        R.c2 = inv_temperature(T) * kLog2e;
        R.lt2 = ws.lse[static_cast<size_t>(b) * (K + 1) + js - 1] * kLog2e;
        R.dl = R.lt2 - draft_lse[static_cast<size_t>(b) * K + js - 1] * kLog2e;
        R.bonus = false;
        R.kl = key_lane(T);
        ResBest best = res_empty();
        if (v0 < V) {
            const LT* br = base + (static_cast<size_t>(b) * K + js - 1) * V + v0;
            const LT* tr = target + (row_off[b] + js - 1) * static_cast<int64_t>(V) + v0;
            const u32x4 rnd = philox_block(seed, b, js, kTagResample, v0 >> 2);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (v0 + t >= V) continue;
                residual_entry(best, to_f32(br[t]) + acc[g][t], to_f32(tr[t]), pick(rnd, t),
                               v0 + t, R);
            }
        }
        RowState sr{-INFINITY, 0.0f, best.br, 0.0f, best.ir};
        RowState sf{-INFINITY, 0.0f, best.bf, 0.0f, best.jf};
        wave_reduce_row(sr);
        wave_reduce_row(sf);
        if ((tid & 63) == 0) {
            red_r[tid >> 6][g] = sr;
            red_f[tid >> 6][g] = sf;
        }
    }
    __syncthreads();
    if (tid < nrows) {
        RowState sr = red_r[0][tid];
        RowState sf = red_f[0][tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
            row_merge(sr, red_r[w][tid]);
            row_merge(sf, red_f[w][tid]);
        }
        const size_t o = static_cast<size_t>(slot0 + tid) * n_strips + strip;
        store_partial(ws.res, o, sr);
        store_partial(ws.fall, o, sf);
    }
}

// Fold the residual strips of each listed request into its next token: the
// winner of the residual keys when any entry had positive residual mass, else
// the winner of the fallback keys (for a listed full acceptance, its bonus).
// One wavefront per listed request.  The partials per request are g.n_parts,
// or with g.wgs > 0 the split residual_parts makes of the list's length.
__global__ __launch_bounds__(kWave) void verify_residual_combine(VerifyWs ws, int B, int n_strips_v,
                                                                 ResGeom g,
                                                                 int32_t* __restrict__ next_token) {
    const int slot = blockIdx.x;
    const int count = listed_count(ws.count);
    if (slot >= count) return;
    const int n_strips =
        g.wgs > 0 ? residual_parts(n_strips_v, g.wgs, (count + 32 * g.nw - 1) / (32 * g.nw))
                  : g.n_parts;
    const int lane = threadIdx.x;
    RowState sr = row_empty();
    RowState sf = row_empty();
    const size_t o = static_cast<size_t>(slot) * n_strips;
    int s = lane;
    for (; s + kWave < n_strips; s += 2 * kWave) {
        const RowState r0 = load_partial(ws.res, o + s), r1 = load_partial(ws.res, o + s + kWave);
        const RowState f0 = load_partial(ws.fall, o + s),
                       f1 = load_partial(ws.fall, o + s + kWave);
        row_merge(sr, r0);
        row_merge(sr, r1);
        row_merge(sf, f0);
        row_merge(sf, f1);
    }
    for (; s < n_strips; s += kWave) {
        row_merge(sr, load_partial(ws.res, o + s));
        row_merge(sf, load_partial(ws.fall, o + s));
    }
    wave_reduce_row(sr);
    wave_reduce_row(sf);
    if (lane == 0)
        next_token[listed_request(ws.list, ws.count, B, slot)] =
            (sr.pert > -INFINITY) ? sr.idx : sf.idx;
}

struct WsLayout {
    size_t accept, arg, lse, bonus, list, count, res_v, res_i, fall_v, fall_i, total;
};

WsLayout verify_layout(int B, int K, int V) {
    WsLayout l;
    const size_t rows = static_cast<size_t>(B) * (K + 1);
    const size_t np = static_cast<size_t>(B) * ceil_div(V, kMfmaStrip);
    size_t o = 0;
    l.accept = o; o += align256(rows * 4);
    l.arg = o; o += align256(rows * 4);
    l.lse = o; o += align256(rows * 4);
    l.bonus = o; o += align256(static_cast<size_t>(B) * 4);
    l.list = o; o += align256(static_cast<size_t>(B) * 4);
    l.count = o; o += 256;
    l.res_v = o; o += align256(np * 16);
    l.res_i = o; o += align256(np * 4);
    l.fall_v = o; o += align256(np * 16);
    l.fall_i = o; o += align256(np * 4);
    l.total = o;
    return l;
}

template <typename LT, typename FT>
void launch_residual_valu(const VerifyArgs& a, const VerifyWs& ws, int n_strips) {
    dim3 grid(static_cast<unsigned>(ceil_div(a.B, kResRows)), static_cast<unsigned>(n_strips));
    const size_t lds = sizeof(float) * kResRows * a.r;
    hipLaunchKernelGGL((verify_residual_valu<LT, FT>), grid, dim3(256), lds, a.stream,
                       static_cast<const LT*>(a.base), static_cast<const FT*>(a.A),
                       static_cast<const FT*>(a.W), static_cast<const LT*>(a.target), a.row_off,
                       a.tokens, a.prev_token, a.draft_lse, a.temperature, a.accepted, a.seed, a.B,
                       a.K, a.V, a.r, ws, n_strips);
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

size_t verify_workspace_bytes(int B, int K, int V, int r) {
    (void)r;
    return verify_layout(B, K, V).total;
}

// Positions j_lo .. j_lo + span - 1 of one verify_rows launch when only the
// rows that decide the result are read: positions 1-4, then 5 .. K + 1.  Each
// launch costs about 27 us however few rows it holds, so more, smaller launches
// lost (four launches 1-2, 3-4, 5-8, 9-17 took 134 us per long-draft step,
// these two 114 us; 1-3/4-6/7-17, 1-4/5-8/9-17, 1-5/6-17 and 1-6/7-17 took
// 123-129 us).
int verify_rows_chunk(int j_lo, int K) {
    const int left = K + 2 - j_lo;  // positions j_lo .. K + 1
    return (j_lo == 1) ? std::min(4, left) : left;
}

hipError_t launch_verify(const VerifyArgs& a) {
    if (a.B == 0) return hipSuccess;
    const WsLayout l = verify_layout(a.B, a.K, a.V);
    char* w = static_cast<char*>(a.ws);
    VerifyWs ws;
    ws.accept = reinterpret_cast<int32_t*>(w + l.accept);
    ws.arg = reinterpret_cast<int32_t*>(w + l.arg);
    ws.lse = reinterpret_cast<float*>(w + l.lse);
    ws.bonus = reinterpret_cast<int32_t*>(w + l.bonus);
    ws.list = reinterpret_cast<int32_t*>(w + l.list);
    ws.count = reinterpret_cast<int32_t*>(w + l.count);
    ws.res = {reinterpret_cast<float4*>(w + l.res_v), reinterpret_cast<int32_t*>(w + l.res_i)};
    ws.fall = {reinterpret_cast<float4*>(w + l.fall_v), reinterpret_cast<int32_t*>(w + l.fall_i)};

    // whole 16-byte chunks of every row: the branch-free load path
    const bool vec = aligned16(a.target) && a.V % 8 == 0;
    // With draft rows and the MFMA residual kernel, the sampled bonus draws are
    // made there (its fallback draw over row L_b + 1 is the bonus draw), only
    // for the requests that accepted every drafted token.
    const bool bonus_in_residual = a.K > 0 && residual_mfma_supported(a);
    // With the per-row outputs requested every row is read (one launch over all
    // positions).  Without them only the rows that can decide the result are:
    // positions go in two launches (verify_rows_chunk) and a request whose
    // first rejection lies in the first takes no part in the second.
    const bool every_row = a.row_lse_t != nullptr || a.row_logratio != nullptr;
    hipError_t e = hipSuccess;
    for (int j_lo = 1; j_lo <= a.K + 1;) {
        const int span = every_row ? a.K + 1 : verify_rows_chunk(j_lo, a.K);
        const dim3 rows_grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * span));
        ProfScope rows_scope(DSPARK_KERNEL_VERIFY_ROWS, a.stream);
        if (!every_row && j_lo > 1 && a.B <= kTailMaxB) {
            // the rows still needed, listed by every workgroup of a fixed grid
            // (four 512-thread workgroups per CU)
            const int64_t most = static_cast<int64_t>(a.B) * span;
            const dim3 tail_grid(static_cast<unsigned>(std::max<int64_t>(
                1, std::min<int64_t>(most, 4 * static_cast<int64_t>(device_cus())))));
            if (a.logit_dt == DSPARK_BF16)
                hipLaunchKernelGGL((vec ? verify_rows_tail<bf16_t, true> : verify_rows_tail<bf16_t, false>),
                                   tail_grid, dim3(kVRowThreads), 0, a.stream,
                                   static_cast<const bf16_t*>(a.target), a.row_off, a.lengths,
                                   a.tokens, a.draft_logp, a.temperature, a.seed, a.B, a.K, a.V,
                                   a.n_rows, !bonus_in_residual, ws, j_lo);
            else
                hipLaunchKernelGGL((vec ? verify_rows_tail<float, true> : verify_rows_tail<float, false>),
                                   tail_grid, dim3(kVRowThreads), 0, a.stream,
                                   static_cast<const float*>(a.target), a.row_off, a.lengths,
                                   a.tokens, a.draft_logp, a.temperature, a.seed, a.B, a.K, a.V,
                                   a.n_rows, !bonus_in_residual, ws, j_lo);
        } else if (a.logit_dt == DSPARK_BF16) {
            hipLaunchKernelGGL((vec ? verify_rows<bf16_t, true> : verify_rows<bf16_t, false>),
                               rows_grid, dim3(kVRowThreads), 0, a.stream,
                               static_cast<const bf16_t*>(a.target), a.row_off, a.lengths,
                               a.tokens, a.draft_logp, a.temperature, a.seed, a.K, a.V, a.n_rows,
                               !bonus_in_residual, a.row_lse_t, a.row_logratio, ws, j_lo, span);
        } else {
            hipLaunchKernelGGL((vec ? verify_rows<float, true> : verify_rows<float, false>),
                               rows_grid, dim3(kVRowThreads), 0, a.stream,
                               static_cast<const float*>(a.target), a.row_off, a.lengths,
                               a.tokens, a.draft_logp, a.temperature, a.seed, a.K, a.V, a.n_rows,
                               !bonus_in_residual, a.row_lse_t, a.row_logratio, ws, j_lo, span);
        }
        e = hipGetLastError();
        if (e != hipSuccess) return e;
        prof_end(rows_scope.slot, a.stream);
        rows_scope.slot = -1;
        j_lo += span;
    }
    {
        ProfScope resolve_scope(DSPARK_KERNEL_VERIFY_RESOLVE, a.stream);
        hipLaunchKernelGGL(verify_resolve, dim3(static_cast<unsigned>(ceil_div(a.B, 256))), dim3(256),
                           0, a.stream, a.B, a.K, a.n_rows, a.row_off, a.lengths, a.temperature,
                           bonus_in_residual, ws, a.accepted, a.next_token);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.K == 0) return hipSuccess;  // no draft rows: every next token is a bonus draw
    int n_strips;
    ResGeom geom{0, 0, 0};  // partials per listed request
    ProfScope res_scope(DSPARK_KERNEL_RESIDUAL_STRIP, a.stream);
    if (residual_mfma_supported(a)) {
        n_strips = static_cast<int>(ceil_div(a.V, kMfmaStrip));
        ResidualArgs ra{&a, ws.list, ws.count, ws.lse, ws.res, ws.fall, n_strips};
        e = launch_residual_mfma(ra, &geom);
        if (e != hipSuccess) return e;
    } else {
        n_strips = static_cast<int>(ceil_div(a.V, kValuStrip));
        geom.n_parts = n_strips;
        if (a.logit_dt == DSPARK_BF16 && a.factor_dt == DSPARK_BF16)
            launch_residual_valu<bf16_t, bf16_t>(a, ws, n_strips);
        else if (a.logit_dt == DSPARK_BF16)
            launch_residual_valu<bf16_t, float>(a, ws, n_strips);
        else if (a.factor_dt == DSPARK_BF16)
            launch_residual_valu<float, bf16_t>(a, ws, n_strips);
        else
            launch_residual_valu<float, float>(a, ws, n_strips);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    prof_end(res_scope.slot, a.stream);
    res_scope.slot = -1;
    ProfScope combine_scope(DSPARK_KERNEL_RESIDUAL_COMBINE, a.stream);
    hipLaunchKernelGGL(verify_residual_combine, dim3(static_cast<unsigned>(a.B)), dim3(kWave), 0,
                       a.stream, ws, a.B, n_strips, geom, a.next_token);
    return hipGetLastError();
}

}  // namespace dspark
