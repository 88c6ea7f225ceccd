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
//   j* = a_b + 1 (Gumbel-max over log of the positive residual, falling back to
//   p_t when no residual mass is left);  a_b = L_b: next ~ p_t of row L_b + 1.
//
// Launches: (1) one workgroup per (request, row) streams the target row once:
// log-normaliser, accept bit, argmax, and the bonus Gumbel-max on row L_b + 1;
// (2) one thread per request finds the first rejection; (3) rejected sampled
// requests recompute their draft row at j* (rank-r bias + base) and stream the
// target row again for the residual Gumbel-max, split in vocabulary strips;
// (4) the strips are folded into the next token.
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kRowThreads = 256;
constexpr int kResRows = 8;  // rejected requests per workgroup of the residual kernel

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

__device__ __forceinline__ void block_reduce_row(RowState& st, RowState* red /* [4] */) {
    wave_reduce_row(st);
    const int tid = threadIdx.x;
    if ((tid & 63) == 0) red[tid >> 6] = st;
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < kRowThreads / kWave; ++w) row_merge(st, red[w]);
    }
}

template <typename LT>
__global__ __launch_bounds__(kRowThreads) void verify_rows(
    const LT* __restrict__ target, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ lengths, const int32_t* __restrict__ tokens,
    const float* __restrict__ draft_logp, const float* __restrict__ temperature, uint64_t seed,
    int K, int V, int64_t n_rows, float* __restrict__ row_lse_t, float* __restrict__ row_logratio,
    VerifyWs ws) {
    __shared__ RowState red[kRowThreads / kWave];
    const int64_t id = blockIdx.x;
    const int b = static_cast<int>(id / (K + 1));
    const int j = static_cast<int>(id - static_cast<int64_t>(b) * (K + 1)) + 1;
    const int L = lengths ? clamp_len(lengths[b], K) : K;
    if (j > L + 1) return;
    if (row_off[b] < 0 || row_off[b] + L + 1 > n_rows) return;  // reported by verify_resolve
    const int64_t row = row_off[b] + (j - 1);
    const float T = temperature[b];
    const bool greedy = !(T > 0.0f);
    const float it = greedy ? 1.0f : inv_temperature(T);
    const bool bonus = (j == L + 1);
    const LT* trow = target + row * static_cast<int64_t>(V);
    RowState st = row_empty();
    for (int v0 = threadIdx.x * 4; v0 < V; v0 += kRowThreads * 4) {
        float y[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = (v0 + t < V) ? to_f32(trow[v0 + t]) * it : -INFINITY;
        if (!greedy) {
            float m = st.m;
#pragma unroll
            for (int t = 0; t < 4; ++t) m = fmaxf(m, y[t]);
            float sum = (st.m == -INFINITY) ? 0.0f : st.s * expf(st.m - m);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (v0 + t < V) sum += expf(y[t] - m);
            st.m = m;
            st.s = sum;
            if (bonus) {
                const u32x4 rnd = philox_block(seed, b, j, kTagResample, v0 >> 2);
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (v0 + t < V) {
                        const float p = y[t] + gumbel_of(pick(rnd, t));
                        if (beats(p, v0 + t, st.pert, st.idx)) {
                            st.pert = p;
                            st.zb = y[t];
                            st.idx = v0 + t;
                        }
                    }
                }
            }
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (v0 + t < V && beats(y[t], v0 + t, st.pert, st.idx)) {
                    st.pert = y[t];
                    st.zb = y[t];
                    st.idx = v0 + t;
                }
            }
        }
    }
    block_reduce_row(st, red);
    if (threadIdx.x == 0) {
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
                const float yx = to_f32(trow[x]) * it;
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
}

__global__ void fill_i32(int32_t* p, int n, int32_t v) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

__global__ __launch_bounds__(256) void verify_resolve(int B, int K, int64_t n_rows,
                                                     const int64_t* __restrict__ row_off,
                                                     const int32_t* __restrict__ lengths,
                                                     const float* __restrict__ temperature,
                                                     VerifyWs ws, int32_t* __restrict__ accepted,
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
    if (a == L) {
        next_token[b] = ws.bonus[b];
    } else if (!(temperature[b] > 0.0f)) {
        next_token[b] = ws.arg[static_cast<size_t>(b) * (K + 1) + a];
    } else {
        const int slot = atomicAdd(ws.count, 1);
        ws.list[slot] = b;
    }
}

// Residual strip kernel (VALU form): workgroup = (8 rejected requests) x (1024
// vocabulary entries).  Recomputes the draft row at j* = a_b + 1 and streams the
// target row j*: r_v = max(0, p_t - p_d), Gumbel-max of log r_v (tag 2, position
// j*); in parallel the fallback Gumbel-max of y (same draws).
template <typename LT, typename FT>
__global__ __launch_bounds__(256) void verify_residual_valu(
    const LT* __restrict__ base, const FT* __restrict__ A, const FT* __restrict__ W,
    const LT* __restrict__ target, const int64_t* __restrict__ row_off,
    const int32_t* __restrict__ tokens, const int32_t* __restrict__ prev_token,
    const float* __restrict__ draft_lse, const float* __restrict__ temperature,
    const int32_t* __restrict__ accepted, uint64_t seed, int K, int V, int r, VerifyWs ws,
    int n_strips) {
    extern __shared__ float a_sh[];  // [kResRows][r]
    __shared__ RowState red_r[4][kResRows];
    __shared__ RowState red_f[4][kResRows];
    const int tid = threadIdx.x;
    const int slot0 = blockIdx.x * kResRows;
    const int count = *ws.count;
    if (slot0 >= count) return;
    const int nrows = min(kResRows, count - slot0);
    const int strip = blockIdx.y;
    for (int e = tid; e < kResRows * r; e += 256) {
        const int g = e / r;
        const int i = e - g * r;
        float a = 0.0f;
        if (g < nrows) {
            const int b = ws.list[slot0 + g];
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
    if (v0 < V) {
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
        const int b = ws.list[slot0 + g];
        const int js = accepted[b] + 1;
        const float it = inv_temperature(temperature[b]);
        const float lse_d = draft_lse[static_cast<size_t>(b) * K + js - 1];
        const float lse_t = ws.lse[static_cast<size_t>(b) * (K + 1) + js - 1];
        RowState sr = row_empty();
        RowState sf = row_empty();
        if (v0 < V) {
            const LT* br = base + (static_cast<size_t>(b) * K + js - 1) * V + v0;
            const LT* tr = target + (row_off[b] + js - 1) * static_cast<int64_t>(V) + v0;
            const u32x4 rnd = philox_block(seed, b, js, kTagResample, v0 >> 2);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (v0 + t >= V) continue;
                const float z = (to_f32(br[t]) + acc[g][t]) * it;
                const float y = to_f32(tr[t]) * it;
                const float g_v = gumbel_of(pick(rnd, t));
                const float res = expf(y - lse_t) - expf(z - lse_d);
                if (res > 0.0f) {
                    const float p = logf(res) + g_v;
                    if (beats(p, v0 + t, sr.pert, sr.idx)) {
                        sr.pert = p;
                        sr.zb = p;
                        sr.idx = v0 + t;
                    }
                }
                const float pf = y + g_v;
                if (beats(pf, v0 + t, sf.pert, sf.idx)) {
                    sf.pert = pf;
                    sf.zb = y;
                    sf.idx = v0 + t;
                }
            }
        }
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

__global__ __launch_bounds__(64) void verify_residual_combine(VerifyWs ws, int n_strips,
                                                             int32_t* __restrict__ next_token) {
    const int slot = blockIdx.x;
    if (slot >= *ws.count) return;
    const int lane = threadIdx.x;
    RowState sr = row_empty();
    RowState sf = row_empty();
    for (int s = lane; s < n_strips; s += kWave) {
        row_merge(sr, load_partial(ws.res, static_cast<size_t>(slot) * n_strips + s));
        row_merge(sf, load_partial(ws.fall, static_cast<size_t>(slot) * n_strips + s));
    }
    wave_reduce_row(sr);
    wave_reduce_row(sf);
    if (lane == 0) {
        const int b = ws.list[slot];
        next_token[b] = (sr.pert > -INFINITY) ? sr.idx : sf.idx;
    }
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
                       a.tokens, a.prev_token, a.draft_lse, a.temperature, a.accepted, a.seed, a.K,
                       a.V, a.r, ws, n_strips);
}

}  // namespace

size_t verify_workspace_bytes(int B, int K, int V, int r) {
    (void)r;
    return verify_layout(B, K, V).total;
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

    hipLaunchKernelGGL(fill_i32, dim3(1), dim3(64), 0, a.stream, ws.count, 1, 0);
    const dim3 rows_grid(static_cast<unsigned>(static_cast<int64_t>(a.B) * (a.K + 1)));
    if (a.logit_dt == DSPARK_BF16) {
        hipLaunchKernelGGL(verify_rows<bf16_t>, rows_grid, dim3(kRowThreads), 0, a.stream,
                           static_cast<const bf16_t*>(a.target), a.row_off, a.lengths, a.tokens,
                           a.draft_logp, a.temperature, a.seed, a.K, a.V, a.n_rows, a.row_lse_t,
                           a.row_logratio, ws);
    } else {
        hipLaunchKernelGGL(verify_rows<float>, rows_grid, dim3(kRowThreads), 0, a.stream,
                           static_cast<const float*>(a.target), a.row_off, a.lengths, a.tokens,
                           a.draft_logp, a.temperature, a.seed, a.K, a.V, a.n_rows, a.row_lse_t,
                           a.row_logratio, ws);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(verify_resolve, dim3(static_cast<unsigned>(ceil_div(a.B, 256))), dim3(256),
                       0, a.stream, a.B, a.K, a.n_rows, a.row_off, a.lengths, a.temperature, ws,
                       a.accepted,
                       a.next_token);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n_strips = static_cast<int>(ceil_div(a.V, kValuStrip));
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
    hipLaunchKernelGGL(verify_residual_combine, dim3(static_cast<unsigned>(a.B)), dim3(kWave), 0,
                       a.stream, ws, n_strips, a.next_token);
    return hipGetLastError();
}

}  // namespace dspark
