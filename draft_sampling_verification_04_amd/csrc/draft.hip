// draft.hip -- Markov-head draft sampling (yage.ai DSpark analysis, paragraph on
// the first-order Markov head; freeaitool DSpark guide, section 3.1).
//
// Per draft position k (sequential, x_k feeds position k+1):
//   bias_v = A[x_{k-1}, :] . W[:, v]     rank-r transition lookup
//   z_v    = (base[b, k, v] + bias_v) * (1/T_b)
//   x_k    = argmax_v z_v + G_v          (T > 0: Gumbel-max, one tag-0 draw per entry)
//          = argmax_v base + bias        (T == 0)
//   lse_d  = log sum_v exp(z_v),  log p_d(x_k) = z_{x_k} - lse_d
//
// Each position is two launches: a strip kernel that produces, per request and
// vocabulary strip (or part of strips), an online-softmax partial with the best
// entry key (RowState), and a combine kernel that folds them into lse_d and
// x_k and writes log p_d.  The strip kernel exists in two forms: a VALU form
// for any factor dtype and rank, and an MFMA form (draft_mfma.hip) for bf16
// factors.  Keys are base 2: s c - log2(-log2 u) with c = log2(e) / T orders
// entries as z + G does (KeyLane).
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kValuRows = 8;  // requests per workgroup of the VALU strip kernel

// VALU strip kernel: workgroup = (8 requests) x (1024 vocabulary entries); each
// thread owns 4 consecutive entries (one Philox block) for all 8 requests and
// accumulates their transition bias in fp32 from factor rows staged in LDS.
// The partial's key is the best entry key, its index that entry.
template <typename LT, typename FT>
__global__ __launch_bounds__(256) void draft_strip_valu(
    const LT* __restrict__ base, const FT* __restrict__ A, const FT* __restrict__ W,
    const int32_t* __restrict__ prev, int prev_stride, const float* __restrict__ temperature,
    uint64_t seed, int B, int K, int V, int r, int k, PartialBuf part, int n_strips) {
    extern __shared__ float a_sh[];  // [kValuRows][r] gathered factor rows
    __shared__ RowState red[4][kValuRows];
    const int tid = threadIdx.x;
    const int b0 = blockIdx.x * kValuRows;
    const int strip = blockIdx.y;
    const int nrows = min(kValuRows, B - b0);
    for (int e = tid; e < kValuRows * r; e += 256) {
        const int g = e / r;
        const int i = e - g * r;
        float a = 0.0f;
        if (g < nrows) {
            const int p = clamp_token(prev[static_cast<size_t>(b0 + g) * prev_stride], V);
            a = to_f32(A[static_cast<size_t>(p) * r + i]);
        }
        a_sh[e] = a;
    }
    __syncthreads();

    const int v0 = strip * kValuStrip + tid * 4;
    float acc[kValuRows][4];
#pragma unroll
    for (int g = 0; g < kValuRows; ++g)
#pragma unroll
        for (int t = 0; t < 4; ++t) acc[g][t] = 0.0f;
    if (v0 < V) {
        for (int i = 0; i < r; ++i) {
            const FT* wr = W + static_cast<size_t>(i) * V + v0;
            float w[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) w[t] = (v0 + t < V) ? to_f32(wr[t]) : 0.0f;
#pragma unroll
            for (int g = 0; g < kValuRows; ++g) {
                const float a = a_sh[g * r + i];
#pragma unroll
                for (int t = 0; t < 4; ++t) acc[g][t] = fmaf(a, w[t], acc[g][t]);
            }
        }
    }

#pragma unroll
    for (int g = 0; g < kValuRows; ++g) {
        if (g >= nrows) break;  // uniform: every thread handles the same requests
        const int b = b0 + g;
        const float T = temperature[b];
        RowState st = row_empty();
        float s[4];
        const LT* br = base + (static_cast<size_t>(b) * K + k) * V + v0;
#pragma unroll
        for (int t = 0; t < 4; ++t)
            s[t] = (v0 + t < V) ? to_f32(br[t]) + acc[g][t] : -INFINITY;
        if (T > 0.0f) {
            // the thread's softmax partial over its 4 entries (on the z scale)
            // and the best of their keys s c - log2(-log2 u) (one Philox block)
            const KeyLane kl = key_lane(T);
            const float it = inv_temperature(T);
            float m = -INFINITY;
#pragma unroll
            for (int t = 0; t < 4; ++t) m = fmaxf(m, s[t] * it);
            float sum = 0.0f;
            if (m != -INFINITY) {
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (v0 + t < V) sum += expf(s[t] * it - m);
            }
            st.m = m;
            st.s = sum;
            if (v0 < V) {
                const u32x4 rnd = philox_block(seed, b, k + 1, kTagDraft, v0 >> 2);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float key = fmaf(s[t], kl.c2, -entry_l2(pick(rnd, t), kl));
                    if (v0 + t < V && key > st.pert) {
                        st.pert = key;
                        st.idx = v0 + t;
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (v0 + t < V && beats(s[t], v0 + t, st.pert, st.idx)) {
                    st.pert = s[t];
                    st.idx = v0 + t;
                }
            }
        }
        wave_reduce_row(st);
        if ((tid & 63) == 0) red[tid >> 6][g] = st;
    }
    __syncthreads();
    if (tid < nrows) {
        RowState st = red[0][tid];
#pragma unroll
        for (int w = 1; w < 4; ++w) row_merge(st, red[w][tid]);
        store_partial(part, static_cast<size_t>(b0 + tid) * n_strips + strip, st);
    }
}

// Fold the partials of each row into its token (one wavefront per row, one
// wavefront per workgroup, so that the rows spread over every CU's memory
// pipeline).  Rows are requests at step k (k >= 0: partial row b, output
// b K + k) or, for parallel drafting (k < 0, no factors), every (request,
// position) row q = b K + k'.  The winner of the merged partials is x_k (the
// largest key, smallest entry on ties).  T == 0: its key is the logit, so
// lse_d is the row maximum and log p_d = 0.  T > 0: lse_d = m + log s, and
// z_x log2(e) = key + log2(-log2 u_x), the winner's own draw recomputed here
// (the key is that sum rounded once), so log p_d = z_x - lse_d needs no logit
// or bias load.
__global__ __launch_bounds__(kWave) void draft_combine(
    PartialBuf part, int n_parts, const float* __restrict__ temperature, uint64_t seed,
    int n_rows, int K, int k, int32_t* __restrict__ tokens, float* __restrict__ logp,
    float* __restrict__ lse) {
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x;
    if (row >= n_rows) return;  // whole wavefront
    const int b = (k >= 0) ? row : row / K;
    const int pos = (k >= 0) ? k + 1 : row % K + 1;
    const size_t o = (k >= 0) ? static_cast<size_t>(b) * K + k : static_cast<size_t>(row);
    RowState st = row_empty();
    {
        const size_t pr = static_cast<size_t>(row) * n_parts;
        int s = lane;
        for (; s + 3 * kWave < n_parts; s += 4 * kWave) {
            RowState q[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) q[u] = load_partial(part, pr + s + u * kWave);
#pragma unroll
            for (int u = 0; u < 4; ++u) row_merge(st, q[u]);
        }
        for (; s < n_parts; s += kWave) row_merge(st, load_partial(part, pr + s));
    }
    wave_reduce_row(st);  // every lane holds the row's state
    if (lane != 0) return;
    const float T = temperature[b];
    tokens[o] = st.idx;
    if (!(T > 0.0f)) {
        if (lse) lse[o] = st.pert;
        if (logp) logp[o] = 0.0f;
        return;
    }
    const float l = st.m + logf(st.s);
    if (lse) lse[o] = l;
    if (logp) {
        const KeyLane kl = key_lane(T);
        const uint32_t x = static_cast<uint32_t>(st.idx);
        const u32x4 rnd =
            philox_block(seed, static_cast<uint32_t>(b), static_cast<uint32_t>(pos), kTagDraft,
                         x >> 2);
        logp[o] = (st.pert + entry_l2(pick(rnd, static_cast<int>(x & 3u)), kl)) * kLn2 - l;
    }
}

template <typename LT, typename FT>
void launch_valu_strip(const DraftArgs& a, const int32_t* prev, int prev_stride, int k,
                       PartialBuf part, int n_strips) {
    dim3 grid(static_cast<unsigned>(ceil_div(a.B, kValuRows)), static_cast<unsigned>(n_strips));
    const size_t lds = sizeof(float) * kValuRows * a.r;
    hipLaunchKernelGGL((draft_strip_valu<LT, FT>), grid, dim3(256), lds, a.stream,
                       static_cast<const LT*>(a.base), static_cast<const FT*>(a.A),
                       static_cast<const FT*>(a.W), prev, prev_stride, a.temperature, a.seed, a.B,
                       a.K, a.V, a.r, k, part, n_strips);
}

void launch_combine(const DraftArgs& a, PartialBuf part, int n_parts, int n_rows, int k) {
    hipLaunchKernelGGL(draft_combine, dim3(static_cast<unsigned>(n_rows)), dim3(kWave), 0,
                       a.stream, part, n_parts, a.temperature, a.seed, n_rows, a.K, k, a.tokens,
                       a.logp, a.lse);
}

}  // namespace

hipError_t launch_draft_combine(const DraftArgs& a, PartialBuf part, int n_parts, int n_rows, int k) {
    launch_combine(a, part, n_parts, n_rows, k);
    return hipGetLastError();
}

// Implemented in draft_mfma.hip.
bool mfma_supported(const DraftArgs& a);
int mfma_draft_strip();
bool parallel_supported(const DraftArgs& a);
hipError_t launch_draft_parallel(const DraftArgs& a, PartialBuf part, size_t part_capacity,
                                 const int32_t* order);
hipError_t launch_temperature_order(const float* temperature, int B, int32_t* order,
                                    hipStream_t stream);
hipError_t launch_draft_mfma_step(const DraftArgs& a, const int32_t* prev, int prev_stride, int k,
                                  const int32_t* order, PartialBuf part, int n_strips,
                                  int* n_parts);

namespace {

struct DraftWs {
    PartialBuf part;
    int32_t* order;
};

// Partial records reserved: B max(ceil(V / 64), K), enough for one per
// (request, strip) of the narrowest strip and for the parallel path's rows.
size_t partial_capacity(int B, int K, int V) {
    return static_cast<size_t>(B) * std::max<int64_t>(ceil_div(V, kMinStrip), K);
}

DraftWs draft_ws(void* ws, int B, int K, int V) {
    const size_t n = partial_capacity(B, K, V);
    char* w = static_cast<char*>(ws);
    DraftWs d;
    size_t o = 0;
    d.part.v = reinterpret_cast<float4*>(w + o);
    o += align256(n * sizeof(float4));
    d.part.idx = reinterpret_cast<int32_t*>(w + o);
    o += align256(n * sizeof(int32_t));
    d.order = reinterpret_cast<int32_t*>(w + o);
    return d;
}

}  // namespace

size_t draft_workspace_bytes(int B, int K, int V, int r) {
    (void)r;
    const size_t n = partial_capacity(B, K, V);
    return align256(n * sizeof(float4)) + align256(n * sizeof(int32_t)) +
           align256(static_cast<size_t>(B) * sizeof(int32_t));
}

bool draft_uses_mfma(const DraftArgs& a) { return mfma_supported(a); }

hipError_t launch_draft(const DraftArgs& a) {
    if (a.B == 0 || a.K == 0) return hipSuccess;
    if (a.A == nullptr && a.W == nullptr) {  // parallel drafting: no Markov head
        const DraftWs ws = draft_ws(a.ws, a.B, a.K, a.V);
        hipError_t e = launch_temperature_order(a.temperature, a.B, ws.order, a.stream);
        if (e != hipSuccess) return e;
        ProfScope scope(DSPARK_KERNEL_DRAFT_STRIP, a.stream);
        return launch_draft_parallel(a, ws.part, partial_capacity(a.B, a.K, a.V), ws.order);
    }
    const bool mfma = draft_uses_mfma(a);
    const int n_strips = static_cast<int>(ceil_div(a.V, mfma ? mfma_draft_strip() : kValuStrip));
    const DraftWs ws = draft_ws(a.ws, a.B, a.K, a.V);
    if (mfma) {
        hipError_t e = launch_temperature_order(a.temperature, a.B, ws.order, a.stream);
        if (e != hipSuccess) return e;
    }
    for (int k = 0; k < a.K; ++k) {
        const int32_t* prev = (k == 0) ? a.prev_token : a.tokens + (k - 1);
        const int prev_stride = (k == 0) ? 1 : a.K;
        ProfScope strip_scope(DSPARK_KERNEL_DRAFT_STRIP, a.stream);
        int n_parts = n_strips;  // partials per request written by this step
        if (mfma) {
            hipError_t e = launch_draft_mfma_step(a, prev, prev_stride, k, ws.order, ws.part,
                                                  n_strips, &n_parts);
            if (e != hipSuccess) return e;
        } else if (a.logit_dt == DSPARK_BF16 && a.factor_dt == DSPARK_BF16) {
            launch_valu_strip<bf16_t, bf16_t>(a, prev, prev_stride, k, ws.part, n_strips);
        } else if (a.logit_dt == DSPARK_BF16) {
            launch_valu_strip<bf16_t, float>(a, prev, prev_stride, k, ws.part, n_strips);
        } else if (a.factor_dt == DSPARK_BF16) {
            launch_valu_strip<float, bf16_t>(a, prev, prev_stride, k, ws.part, n_strips);
        } else {
            launch_valu_strip<float, float>(a, prev, prev_stride, k, ws.part, n_strips);
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        prof_end(strip_scope.slot, a.stream);
        strip_scope.slot = -1;
        ProfScope combine_scope(DSPARK_KERNEL_DRAFT_COMBINE, a.stream);
        e = launch_draft_combine(a, ws.part, n_parts, a.B, k);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dspark
