// schedule.hip -- confidence-scheduled prefix selection (freeaitool DSpark
// guide, sections 4.1-4.2; yage.ai DSpark analysis, scheduler paragraph;
// legalagi.cn reading, section 5).
//
//   S[b][k] = c[b][0] * ... * c[b][k]         sequential fp32 products
//   D = max(0, budget - B)                     the budget counts the B roots
//   items taken in order (S desc, k asc, b asc) while taken < D and S > 0 and,
//   with a throughput curve tau(N), while (B + sum S) / tau(B + taken) rises
//   strictly; the first failure stops the walk.
//   L_b = taken items of request b (prefix-closed: S never rises along k);
//   row_offsets = exclusive scan of L_b + 1.
//
// One workgroup of 1024 threads does the whole selection; the input is at most
// a few hundred KB, so the kernel is latency-bound.  The order is encoded in a
// 64-bit key: high word ~bits(S) (S > 0 is a positive float, so its bit pattern
// is monotone), low word k * B + b.  Without a curve the D-th smallest key is
// found by an 8-pass byte-wise radix select and L_b counts keys at or below it.
// With a curve the candidates are sorted (bitonic, in workspace memory) and
// the strict-rise test is evaluated at every rank from an fp64 prefix sum.
#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 1024;
constexpr uint64_t kNoKey = ~0ull;

struct Curve {
    int n;
    double cn[kMaxCurvePoints];
    double ct[kMaxCurvePoints];
};

__device__ double curve_tau(const Curve& c, double N) {
    if (c.n <= 0) return 1.0;
    if (c.n == 1 || N <= c.cn[0]) return c.ct[0];
    for (int i = 1; i < c.n; ++i) {
        if (N <= c.cn[i]) {
            const double f = (N - c.cn[i - 1]) / (c.cn[i] - c.cn[i - 1]);
            return c.ct[i - 1] + f * (c.ct[i] - c.ct[i - 1]);
        }
    }
    const double slope = (c.ct[c.n - 1] - c.ct[c.n - 2]) / (c.cn[c.n - 1] - c.cn[c.n - 2]);
    return c.ct[c.n - 1] + slope * (N - c.cn[c.n - 1]);
}

__device__ __forceinline__ float key_survival(uint64_t key) {
    return __uint_as_float(0xFFFFFFFFu - static_cast<uint32_t>(key >> 32));
}

// Block-wide sum of one value per thread (all threads get the result).
template <typename T>
__device__ T block_sum(T v, T* sh /* [kThreads / kWave] */) {
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    const int tid = threadIdx.x;
    __syncthreads();
    if ((tid & 63) == 0) sh[tid >> 6] = v;
    __syncthreads();
    T t = 0;
    for (int w = 0; w < kThreads / kWave; ++w) t += sh[w];
    __syncthreads();
    return t;
}

// Block-wide exclusive scan of one value per thread (thread order).
template <typename T>
__device__ T block_exclusive_scan(T v, T* sh /* [kThreads / kWave] */, T* total) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    T incl = v;
    for (int d = 1; d < kWave; d <<= 1) {
        const T o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    __syncthreads();
    if (lane == 63) sh[tid >> 6] = incl;
    __syncthreads();
    T before = 0;
    T all = 0;
    for (int w = 0; w < kThreads / kWave; ++w) {
        if (w < (tid >> 6)) before += sh[w];
        all += sh[w];
    }
    __syncthreads();
    if (total) *total = all;
    return before + incl - v;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(
    const float* __restrict__ conf, int B, int K, long long budget, Curve curve,
    int32_t* __restrict__ lengths, int64_t* __restrict__ row_offsets, float* __restrict__ survival,
    uint64_t* __restrict__ keys, uint64_t* __restrict__ sorted, int sort_cap) {
    __shared__ unsigned hist[256];
    __shared__ unsigned long long sh_u64[kThreads / kWave];
    __shared__ double sh_f64[kThreads / kWave];
    __shared__ unsigned sh_sel, sh_want, sh_ncand;
    __shared__ unsigned long long sh_stop;
    const int tid = threadIdx.x;
    const long long n_items = static_cast<long long>(B) * K;

    // 1. survival products and keys
    unsigned long long n_pos_local = 0;
    for (int b = tid; b < B; b += kThreads) {
        float S = 1.0f;
        for (int k = 0; k < K; ++k) {
            const size_t o = static_cast<size_t>(b) * K + k;
            S = S * conf[o];
            if (survival) survival[o] = S;
            const bool pos = S > 0.0f;
            keys[o] = pos ? (static_cast<uint64_t>(0xFFFFFFFFu - __float_as_uint(S)) << 32) |
                                static_cast<uint32_t>(k * B + b)
                          : kNoKey;
            n_pos_local += pos;
        }
        lengths[b] = 0;
    }
    const unsigned long long n_pos = block_sum<unsigned long long>(n_pos_local, sh_u64);
    const long long D = budget - B > 0 ? budget - B : 0;
    const long long dsel = D < static_cast<long long>(n_pos) ? D : static_cast<long long>(n_pos);

    // 2. threshold key: every candidate has key <= theta
    uint64_t theta;
    if (dsel == 0) {
        theta = 0;  // keys of positive S are > 0: nothing is taken
    } else if (dsel == static_cast<long long>(n_pos)) {
        theta = kNoKey - 1;
    } else {
        uint64_t prefix = 0, mask = 0;
        unsigned want = static_cast<unsigned>(dsel - 1);  // 0-based rank
        for (int d = 7; d >= 0; --d) {
            for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
            __syncthreads();
            for (long long i = tid; i < n_items; i += kThreads) {
                const uint64_t key = keys[i];
                if (key != kNoKey && (key & mask) == prefix)
                    atomicAdd(&hist[(key >> (8 * d)) & 255u], 1u);
            }
            __syncthreads();
            if (tid == 0) {
                unsigned c = 0;
                unsigned sel = 255;
                for (unsigned t = 0; t < 256; ++t) {
                    if (c + hist[t] > want) {
                        sel = t;
                        break;
                    }
                    c += hist[t];
                }
                sh_sel = sel;
                sh_want = want - c;
            }
            __syncthreads();
            prefix |= static_cast<uint64_t>(sh_sel) << (8 * d);
            mask |= 255ull << (8 * d);
            want = sh_want;
            __syncthreads();
        }
        theta = prefix;
    }

    if (curve.n <= 0) {
        // 3a. L_b = number of candidate keys of request b
        for (int b = tid; b < B; b += kThreads) {
            int L = 0;
            for (int k = 0; k < K; ++k) {
                const uint64_t key = keys[static_cast<size_t>(b) * K + k];
                L += (key != kNoKey && key <= theta);
            }
            lengths[b] = L;
        }
    } else if (dsel > 0) {
        // 3b. sort the candidates, then the strict-rise test at every rank
        if (tid == 0) sh_ncand = 0;
        __syncthreads();
        for (long long i = tid; i < n_items; i += kThreads) {
            const uint64_t key = keys[i];
            if (key != kNoKey && key <= theta) sorted[atomicAdd(&sh_ncand, 1u)] = key;
        }
        __syncthreads();
        const int n = static_cast<int>(sh_ncand);  // == dsel
        int npow = 1;
        while (npow < n) npow <<= 1;
        for (int i = n + tid; i < npow && i < sort_cap; i += kThreads) sorted[i] = kNoKey;
        __syncthreads();
        for (int size = 2; size <= npow; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < npow; i += kThreads) {
                    const int partner = i ^ stride;
                    if (partner > i) {
                        const bool up = (i & size) == 0;
                        const uint64_t x = sorted[i], y = sorted[partner];
                        if ((x > y) == up) {
                            sorted[i] = y;
                            sorted[partner] = x;
                        }
                    }
                }
                __syncthreads();
            }
        }
        // prefix sums of S in rank order, chunked per thread
        const int chunk = (n + kThreads - 1) / kThreads;
        const int lo = min(n, tid * chunk), hi = min(n, lo + chunk);
        double local = 0.0;
        for (int i = lo; i < hi; ++i) local += static_cast<double>(key_survival(sorted[i]));
        const double before = block_exclusive_scan<double>(local, sh_f64, nullptr);
        if (tid == 0) sh_stop = static_cast<unsigned long long>(n);
        __syncthreads();
        double E = static_cast<double>(B) + before;
        for (int i = lo; i < hi; ++i) {
            const double S = static_cast<double>(key_survival(sorted[i]));
            const double N = static_cast<double>(B) + i;
            const double f_now = E / curve_tau(curve, N);
            const double f_next = (E + S) / curve_tau(curve, N + 1.0);
            if (!(f_next > f_now)) {
                atomicMin(&sh_stop, static_cast<unsigned long long>(i));
                break;
            }
            E += S;
        }
        __syncthreads();
        const int stop = static_cast<int>(sh_stop);
        for (int i = tid; i < stop; i += kThreads) {
            const uint32_t low = static_cast<uint32_t>(sorted[i]);
            atomicAdd(&lengths[low % static_cast<uint32_t>(B)], 1);
        }
    }
    __syncthreads();

    // 4. row_offsets = exclusive scan of L_b + 1
    const int chunk = (B + kThreads - 1) / kThreads;
    const int lo = min(B, tid * chunk), hi = min(B, lo + chunk);
    long long local = 0;
    for (int b = lo; b < hi; ++b) local += lengths[b] + 1;
    long long total = 0;
    const long long before =
        block_exclusive_scan<long long>(local, reinterpret_cast<long long*>(sh_u64), &total);
    long long run = before;
    for (int b = lo; b < hi; ++b) {
        row_offsets[b] = run;
        run += lengths[b] + 1;
    }
    if (tid == 0) row_offsets[B] = total;
}

}  // namespace

size_t schedule_workspace_bytes(int B, int K) {
    const size_t n = static_cast<size_t>(B) * K;
    size_t npow = 1;
    while (npow < n) npow <<= 1;
    return align256(n * 8) + align256(npow * 8);
}

hipError_t launch_schedule(const ScheduleArgs& a) {
    const size_t n = static_cast<size_t>(a.B) * a.K;
    uint64_t* keys = static_cast<uint64_t*>(a.ws);
    uint64_t* sorted = reinterpret_cast<uint64_t*>(static_cast<char*>(a.ws) + align256(n * 8));
    size_t npow = 1;
    while (npow < n) npow <<= 1;
    Curve c;
    c.n = a.n_points;
    for (int i = 0; i < kMaxCurvePoints; ++i) {
        c.cn[i] = i < a.n_points ? a.curve_n[i] : 0.0;
        c.ct[i] = i < a.n_points ? a.curve_tau[i] : 0.0;
    }
    ProfScope scope(DSPARK_KERNEL_SCHEDULE, a.stream);
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.conf, a.B, a.K,
                       static_cast<long long>(a.budget), c, a.lengths, a.row_offsets, a.survival,
                       keys, sorted, static_cast<int>(npow));
    return hipGetLastError();
}

}  // namespace dspark
