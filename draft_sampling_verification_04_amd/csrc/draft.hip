// draft.hip -- Markov-head draft sampling (yage.ai DSpark analysis, paragraph on
// the first-order Markov head; freeaitool DSpark guide, section 3.1).
//
// Per draft position k (sequential, x_k feeds position k+1):
//   bias_v = A[x_{k-1}, :] . W[:, v]     rank-r transition lookup
//   z_v    = (base[b, k, v] + bias_v) * (1/T_b)
//   x_k    = argmax_v z_v + G_v          Philox-keyed Gumbel-max (T > 0)
//          = argmax_v base + bias        (T == 0)
//   lse_d  = log sum_v exp(z_v),  log p_d(x_k) = z_{x_k} - lse_d
//
// Each position is two launches: a strip kernel that produces, per request and
// vocabulary strip, an online-softmax / Gumbel-max partial (RowState), and a
// combine kernel that folds the strips of each request into x_k, log p_d, lse_d.
// The strip kernel exists in two forms: a VALU form for any factor dtype and
// rank, and an MFMA form (draft_mfma.hip) for bf16 factors.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kValuRows = 8;  // requests per workgroup of the VALU strip kernel

// VALU strip kernel: workgroup = (8 requests) x (1024 vocabulary entries); each
// thread owns 4 consecutive entries (one Philox block) for all 8 requests and
// accumulates their transition bias in fp32 from factor rows staged in LDS.
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
        if (g >= nrows) break;
        const int b = b0 + g;
        const float T = temperature[b];
        RowState st = row_empty();
        if (v0 < V) {
            const LT* br = base + (static_cast<size_t>(b) * K + k) * V + v0;
            float s[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) s[t] = (v0 + t < V) ? to_f32(br[t]) + acc[g][t] : -INFINITY;
            if (T > 0.0f) {
                const float it = inv_temperature(T);
                float z[4];
                float m = -INFINITY;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    z[t] = s[t] * it;
                    m = fmaxf(m, z[t]);
                }
                float sum = 0.0f;
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (v0 + t < V) sum += expf(z[t] - m);
                st.m = m;
                st.s = sum;
                const u32x4 rnd = philox_block(seed, b, k + 1, kTagDraft, v0 >> 2);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (v0 + t < V) {
                        const float p = z[t] + gumbel_of(pick(rnd, t));
                        if (beats(p, v0 + t, st.pert, st.idx)) {
                            st.pert = p;
                            st.zb = z[t];
                            st.idx = v0 + t;
                        }
                    }
                }
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (v0 + t < V && beats(s[t], v0 + t, st.pert, st.idx)) {
                        st.pert = s[t];
                        st.zb = s[t];
                        st.idx = v0 + t;
                    }
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

// Fold the strips of each request (one 256-thread workgroup per request) and
// write x_k, log p_d(x_k) and lse_d.
constexpr int kCombineThreads = 256;

__global__ __launch_bounds__(kCombineThreads) void draft_combine(
    PartialBuf part, int n_strips, const float* __restrict__ temperature, int K, int k,
    int32_t* __restrict__ tokens, float* __restrict__ logp, float* __restrict__ lse) {
    __shared__ RowState red[kCombineThreads / kWave];
    const int b = blockIdx.x;
    RowState st = row_empty();
    for (int s = threadIdx.x; s < n_strips; s += kCombineThreads)
        row_merge(st, load_partial(part, static_cast<size_t>(b) * n_strips + s));
    st = block_reduce_row<kCombineThreads>(st, red);
    if (threadIdx.x == 0) {
        const size_t o = static_cast<size_t>(b) * K + k;
        tokens[o] = st.idx;
        if (temperature[b] > 0.0f) {
            const float l = st.m + logf(st.s);
            if (lse) lse[o] = l;
            if (logp) logp[o] = st.zb - l;
        } else {
            if (lse) lse[o] = st.pert;
            if (logp) logp[o] = 0.0f;
        }
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

}  // namespace

// Implemented in draft_mfma.hip.
bool mfma_supported(const DraftArgs& a);
int mfma_draft_strip();
hipError_t launch_draft_combine_mfma(const DraftArgs& a, PartialBuf part, int n_parts, int k,
                                    float* lse_ws);
hipError_t launch_draft_logp_mfma(const DraftArgs& a, const float* lse_ws);
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
    float* lse;  // [B, K] lse_d, kept for the deferred log-probabilities
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
    o += align256(static_cast<size_t>(B) * sizeof(int32_t));
    d.lse = reinterpret_cast<float*>(w + o);
    return d;
}

}  // namespace

size_t draft_workspace_bytes(int B, int K, int V, int r) {
    (void)r;
    const size_t n = partial_capacity(B, K, V);
    return align256(n * sizeof(float4)) + align256(n * sizeof(int32_t)) +
           align256(static_cast<size_t>(B) * sizeof(int32_t)) +
           align256(static_cast<size_t>(B) * K * sizeof(float));
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
        if (mfma) {
            e = launch_draft_combine_mfma(a, ws.part, n_parts, k, ws.lse);
        } else {
            hipLaunchKernelGGL(draft_combine, dim3(static_cast<unsigned>(a.B)),
                               dim3(kCombineThreads), 0, a.stream, ws.part, n_parts,
                               a.temperature, a.K, k, a.tokens, a.logp, a.lse);
            e = hipGetLastError();
        }
        if (e != hipSuccess) return e;
    }
    if (mfma && a.logp) {
        ProfScope logp_scope(DSPARK_KERNEL_DRAFT_LOGP, a.stream);
        hipError_t e = launch_draft_logp_mfma(a, ws.lse);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace dspark
