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
// With a curve the candidates are sorted (bitonic) and the strict-rise test is
// evaluated at every rank from an fp64 prefix sum; the key at the stop rank
// becomes the threshold.  Up to 16384 candidates (of at most 32768 items) are
// sorted by their high words only, in registers and LDS (compare-exchange
// partners in the same wavefront swap by register exchange, only strides
// across wavefronts pass through LDS): the walk depends only on the S
// sequence, and the exact threshold key is then selected among the keys that
// share the stop item's S.  Larger inputs sort whole keys in workspace memory.
// A curve that is one positive constant over every batch size the walk can
// reach ([B, B + D]) cannot stop it before D while the taken S are far above
// the fp64 rounding of the running total: then the D-th key is the threshold
// and nothing is sorted.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace dspark {
namespace {

constexpr int kThreads = 1024;
constexpr uint64_t kNoKey = ~0ull;
constexpr int kSortWords = 32768;  // LDS sort buffer: 128 KB (staging, high words)
constexpr int kSortMax = 16384;    // most candidates sorted in LDS (16 per thread)
constexpr int kKeyRegs = 32;     // keys per thread kept in registers while B * K <= 32768

struct Curve {
    int n;
    int flat;  // tau is one positive constant on [B, B + D] (set by the launcher)
    double cn[kMaxCurvePoints];
    double ct[kMaxCurvePoints];
};

__host__ __device__ double curve_tau(const Curve& c, double N) {
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

// Register exchange with lane ^ m (m a power of two < 64).
__device__ __forceinline__ uint32_t lane_xor(uint32_t x, int m) {
    switch (m) {
        case 1: return xlane<0>(x);
        case 2: return xlane<1>(x);
        case 16: return xlane<4>(x);
        case 32: return xlane<5>(x);
        default: return __shfl_xor(x, m, kWave);
    }
}

// One bitonic stage of stride S < E inside a thread's E registers.
template <int E, int S>
__device__ __forceinline__ void stage_in_thread(uint32_t (&v)[E], int base, int size) {
    if constexpr (S < E) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & S) == 0) {
                const bool up = ((base + e) & size) == 0;
                const uint32_t a = v[e], b = v[e | S];
                v[e] = up ? min(a, b) : max(a, b);
                v[e | S] = up ? max(a, b) : min(a, b);
            }
        }
    }
}

// Ascending bitonic sort of the E * kThreads words in sh.  Thread t holds
// positions t E .. t E + E - 1 in registers; the partner of position i at a
// stage of stride s is i ^ s, in the same thread for s < E, in lane ^ (s / E)
// of the same wavefront for s < 64 E, otherwise read back through LDS.
template <int E>
__device__ void sort_words_lds(uint32_t* sh) {
    constexpr int npow = E * kThreads;
    const int base = threadIdx.x * E;
    uint32_t v[E];
#pragma unroll
    for (int e = 0; e < E; ++e) v[e] = sh[base + e];
    for (int size = 2; size <= npow; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            if (stride >= kWave * E) {
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) sh[base + e] = v[e];
                __syncthreads();
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = base + e;
                    const uint32_t p = sh[i ^ stride];
                    const bool keep_min = ((i & stride) == 0) == ((i & size) == 0);
                    v[e] = keep_min ? min(v[e], p) : max(v[e], p);
                }
            } else if (stride >= E) {
                const int m = stride / E;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int i = base + e;
                    const uint32_t p = lane_xor(v[e], m);
                    const bool keep_min = ((i & stride) == 0) == ((i & size) == 0);
                    v[e] = keep_min ? min(v[e], p) : max(v[e], p);
                }
            } else {
                switch (stride) {
                    case 1: stage_in_thread<E, 1>(v, base, size); break;
                    case 2: stage_in_thread<E, 2>(v, base, size); break;
                    case 4: stage_in_thread<E, 4>(v, base, size); break;
                    case 8: stage_in_thread<E, 8>(v, base, size); break;
                    default: stage_in_thread<E, 16>(v, base, size); break;
                }
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e) sh[base + e] = v[e];
    __syncthreads();
}

__device__ __forceinline__ float survival_of(uint64_t key) { return key_survival(key); }
__device__ __forceinline__ float survival_of(uint32_t word) {
    return __uint_as_float(0xFFFFFFFFu - word);
}

// Strict-rise test over the n sorted candidates (ascending keys or high words
// = descending S): the first rank whose item does not raise
// (B + sum S) / tau(B + taken) stops the walk.  Returns that rank (n if none).
template <typename T>
__device__ __forceinline__ int curve_stop(const T* srt, int n, int B, const Curve& curve,
                                          double* sh_f64, unsigned long long* sh_stop) {
    const int tid = threadIdx.x;
    const int chunk = (n + kThreads - 1) / kThreads;
    const int lo = min(n, tid * chunk), hi = min(n, lo + chunk);
    double local = 0.0;
    for (int i = lo; i < hi; ++i) local += static_cast<double>(survival_of(srt[i]));
    const double before = block_exclusive_scan<double>(local, sh_f64, nullptr);
    if (tid == 0) *sh_stop = static_cast<unsigned long long>(n);
    __syncthreads();
    double E = static_cast<double>(B) + before;
    for (int i = lo; i < hi; ++i) {
        const double S = static_cast<double>(survival_of(srt[i]));
        const double N = static_cast<double>(B) + i;
        const double f_now = E / curve_tau(curve, N);
        const double f_next = (E + S) / curve_tau(curve, N + 1.0);
        if (!(f_next > f_now)) {
            atomicMin(sh_stop, static_cast<unsigned long long>(i));
            break;
        }
        E += S;
    }
    __syncthreads();
    const int stop = static_cast<int>(*sh_stop);
    __syncthreads();
    return stop;
}

// Histogram add for one key per lane: the lanes that share the first hitting
// lane's digit add once (the high digits of ~bits(S) are few, so most lanes
// of a wavefront share one), the others add one each.
__device__ __forceinline__ void hist_add(unsigned* hist, bool hit, unsigned dig) {
    const unsigned long long hits = __ballot(hit);
    if (hits) {
        const int leader = __ffsll(static_cast<long long>(hits)) - 1;
        const unsigned ld = __shfl(dig, leader, kWave);
        const unsigned long long same = __ballot(hit && dig == ld);
        if ((threadIdx.x & 63) == leader)
            atomicAdd(&hist[ld], static_cast<unsigned>(__popcll(same)));
        else if (hit && dig != ld)
            atomicAdd(&hist[dig], 1u);
    }
}

// Slot of this lane's key in a compacted list (one counter add per wavefront);
// -1 for a lane that holds no key.
__device__ __forceinline__ int compact_slot(unsigned* counter, bool take) {
    const unsigned long long takes = __ballot(take);
    if (!takes) return -1;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll(static_cast<long long>(takes)) - 1;
    unsigned base = 0;
    if (lane == leader) base = atomicAdd(counter, static_cast<unsigned>(__popcll(takes)));
    base = __shfl(base, leader, kWave);
    const unsigned long long below = lane ? (takes & (~0ull >> (64 - lane))) : 0ull;
    return take ? static_cast<int>(base + __popcll(below)) : -1;
}

__global__ __launch_bounds__(kThreads) void schedule_kernel(
    const float* __restrict__ conf, int B, int K, long long budget, Curve curve,
    int32_t* __restrict__ lengths, int64_t* __restrict__ row_offsets, float* __restrict__ survival,
    uint64_t* __restrict__ keys, uint64_t* __restrict__ sorted, int sort_cap) {
    __shared__ uint64_t sh_sort[kSortWords / 2];
    __shared__ unsigned hist[256];
    __shared__ unsigned long long sh_u64[kThreads / kWave];
    __shared__ double sh_f64[kThreads / kWave];
    __shared__ unsigned sh_sel, sh_want, sh_cnt, sh_ncand;
    __shared__ unsigned long long sh_stop, sh_theta;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const long long n_items = static_cast<long long>(B) * K;

    // 1. survival products and keys; L_b starts as the count of positive S in
    // row b (the length when every positive item is taken).  While B * K
    // floats fit in the sort buffer, conf is staged there so that the global
    // loads and stores are coalesced and only the sequential products walk the
    // rows (row b is stored rotated by b mod K, so that the lanes of a
    // wavefront, one row each, spread over the banks); larger batches walk the
    // rows in global memory.
    unsigned long long n_pos_local = 0;
    int my_len = 0;  // L of request tid (used while B <= kThreads)
    uint32_t kh[kKeyRegs];  // see below
#pragma unroll
    for (int j = 0; j < kKeyRegs; ++j) kh[j] = 0xFFFFFFFFu;
    const unsigned uK = static_cast<unsigned>(K > 0 ? K : 1);
    const bool staged = n_items <= static_cast<long long>(kThreads) * kKeyRegs;
    const long long D = budget - B > 0 ? budget - B : 0;
    // the budget holds every item and no curve can stop the walk: every
    // positive item is taken, which is known before anything is counted, so
    // no keys are written and no total is formed
    const bool all_fit = curve.n <= 0 && D >= n_items;
    // stage slot of item (b, k)
    auto slot_of = [&](unsigned b, unsigned k) -> unsigned {
        unsigned c = k + (b - (b / uK) * uK);
        if (c >= uK) c -= uK;
        return b * uK + c;
    };
    if (staged) {
        // eight loads in flight per thread: a load-then-store loop waits for
        // each load in turn (16 to 32 round trips at the scheduled batch sizes)
        float* stage = reinterpret_cast<float*>(sh_sort);
        constexpr int kStageBatch = 8;
        for (long long o0 = tid; o0 < n_items; o0 += static_cast<long long>(kThreads) * kStageBatch) {
            float v[kStageBatch];
#pragma unroll
            for (int u = 0; u < kStageBatch; ++u) {
                const long long o = o0 + static_cast<long long>(u) * kThreads;
                v[u] = o < n_items ? conf[o] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < kStageBatch; ++u) {
                const long long o = o0 + static_cast<long long>(u) * kThreads;
                if (o < n_items) {
                    const unsigned b = static_cast<unsigned>(o) / uK;
                    const unsigned k = static_cast<unsigned>(o) - b * uK;
                    stage[slot_of(b, k)] = v[u];
                }
            }
        }
        __syncthreads();
        for (int b = tid; b < B; b += kThreads) {
            float S = 1.0f;
            int pos_b = 0;
            const unsigned base = static_cast<unsigned>(b) * uK;
            unsigned c = static_cast<unsigned>(b) - (static_cast<unsigned>(b) / uK) * uK;
            for (int k = 0; k < K; ++k) {
                S = S * stage[base + c];
                stage[base + c] = S;
                pos_b += S > 0.0f;
                if (++c == uK) c = 0;
            }
            n_pos_local += pos_b;
            lengths[b] = pos_b;
            if (b == tid) my_len = pos_b;
        }
        __syncthreads();
        // B * K <= 32768: register slot j of thread tid is item tid + j * kThreads
#pragma unroll
        for (int j = 0; j < kKeyRegs; ++j) {
            const unsigned o = static_cast<unsigned>(tid + j * kThreads);
            if (static_cast<long long>(j) * kThreads < n_items && o < n_items) {
                const unsigned b = o / uK, k = o - b * uK;
                const float S = stage[slot_of(b, k)];
                if (survival) survival[o] = S;
                if (!all_fit) {
                    const uint32_t h = S > 0.0f ? 0xFFFFFFFFu - __float_as_uint(S) : 0xFFFFFFFFu;
                    keys[o] = h != 0xFFFFFFFFu ? (static_cast<uint64_t>(h) << 32) | (k * B + b)
                                               : kNoKey;
                    kh[j] = h;
                }
            }
        }
    } else {
        for (int b = tid; b < B; b += kThreads) {
            float S = 1.0f;
            int pos_b = 0;
            for (int k = 0; k < K; ++k) {
                const size_t o = static_cast<size_t>(b) * K + k;
                S = S * conf[o];
                if (survival) survival[o] = S;
                const bool pos = S > 0.0f;
                if (!all_fit)
                    keys[o] = pos ? (static_cast<uint64_t>(0xFFFFFFFFu - __float_as_uint(S)) << 32) |
                                        static_cast<uint32_t>(k * B + b)
                                  : kNoKey;
                pos_b += pos;
            }
            n_pos_local += pos_b;
            lengths[b] = pos_b;
            if (b == tid) my_len = pos_b;
        }
    }
    const unsigned long long n_pos =
        all_fit ? 0ull : block_sum<unsigned long long>(n_pos_local, sh_u64);
    const long long dsel =
        all_fit ? 0 : (D < static_cast<long long>(n_pos) ? D : static_cast<long long>(n_pos));
    // every positive item is taken: L_b is already set
    const bool take_all =
        all_fit || (dsel == static_cast<long long>(n_pos) && (curve.n <= 0 || dsel == 0));

    // while a threshold search or a sort follows, up to 32768 keys keep their
    // high word ~bits(S) in registers (key i in slot i / kThreads of thread
    // i % kThreads; 0xFFFFFFFF = no key), filled above when staged and read
    // back here otherwise; the low word k * B + b follows from i = b * K + k
    // where it is needed
    const bool in_regs =
        !take_all && dsel > 0 && n_items <= static_cast<long long>(kThreads) * kKeyRegs;
    if (in_regs && !staged) {
#pragma unroll
        for (int j = 0; j < kKeyRegs; ++j) {
            const long long i = tid + static_cast<long long>(j) * kThreads;
            kh[j] = i < n_items ? static_cast<uint32_t>(keys[i] >> 32) : 0xFFFFFFFFu;
        }
    }
    auto full_key = [&](int j) -> uint64_t {  // key of register slot j (which holds one)
        const unsigned i = static_cast<unsigned>(tid + j * kThreads);
        const unsigned b = i / static_cast<unsigned>(K), k = i - b * static_cast<unsigned>(K);
        return (static_cast<uint64_t>(kh[j]) << 32) | (k * static_cast<unsigned>(B) + b);
    };

    // Key of rank `want` (0-based) among the keys with (key & mask) == prefix
    // and key <= limit, by byte-wise radix passes from byte dtop down.  The
    // limit is tested only in passes below byte 4, so a caller with a limit
    // short of kNoKey - 1 starts at byte 3 (its prefix fixes the high word).
    // regs: read the high words from registers (else every key from memory).
    auto select_key = [&](uint64_t prefix, uint64_t mask, unsigned want, int dtop,
                          uint64_t limit, bool regs) -> uint64_t {
        for (int d = dtop; d >= 0; --d) {
            for (int i = tid; i < 256; i += kThreads) hist[i] = 0;
            // the register words are marked as rewritten in every pass, so
            // what is derived from them (per-slot masks and addresses, 32 of
            // each) is not hoisted out of the loop into spilled registers
            int tid_o = tid;
            asm volatile("" : "+v"(tid_o));
#pragma unroll
            for (int j = 0; j < kKeyRegs; ++j) asm volatile("" : "+v"(kh[j]));
            __syncthreads();
            if (regs) {
#pragma unroll
                for (int j = 0; j < kKeyRegs; ++j) {
                    if (static_cast<long long>(j) * kThreads >= n_items) continue;
                    const bool has = kh[j] != 0xFFFFFFFFu;
                    // bytes 4..7 are the high word; bytes 0..3 (reached only
                    // when survival values tie) read the whole key again
                    const uint64_t key =
                        d >= 4 ? static_cast<uint64_t>(kh[j]) << 32
                               : (has ? keys[tid_o + static_cast<long long>(j) * kThreads] : kNoKey);
                    hist_add(hist, has && (key & mask) == prefix && (d >= 4 || key <= limit),
                             static_cast<unsigned>(key >> (8 * d)) & 255u);
                }
            } else {
                for (long long i0 = 0; i0 < n_items; i0 += kThreads) {
                    const long long i = i0 + tid;
                    const uint64_t key = i < n_items ? keys[i] : kNoKey;
                    hist_add(hist, key != kNoKey && (key & mask) == prefix && key <= limit,
                             static_cast<unsigned>(key >> (8 * d)) & 255u);
                }
            }
            __syncthreads();
            // the bin that holds rank `want`: wavefront 0 scans 4 bins per lane
            if (tid < kWave) {
                const unsigned h0 = hist[4 * lane], h1 = hist[4 * lane + 1];
                const unsigned h2 = hist[4 * lane + 2], h3 = hist[4 * lane + 3];
                const unsigned own = h0 + h1 + h2 + h3;
                unsigned incl = own;
                for (int dd = 1; dd < kWave; dd <<= 1) {
                    const unsigned o = __shfl_up(incl, dd, kWave);
                    if (lane >= dd) incl += o;
                }
                const unsigned excl = incl - own;
                if (excl <= want && want < incl) {
                    unsigned c = excl, sel = 4 * lane;
                    if (c + h0 <= want) {
                        c += h0;
                        ++sel;
                        if (c + h1 <= want) {
                            c += h1;
                            ++sel;
                            if (c + h2 <= want) {
                                c += h2;
                                ++sel;
                            }
                        }
                    }
                    sh_sel = sel;
                    sh_want = want - c;
                    sh_cnt = hist[sel];
                } else if (lane == kWave - 1 && incl <= want) {
                    sh_sel = 255;  // unreachable: rank `want` lies among the prefix's keys
                    sh_want = want - incl;
                    sh_cnt = 0;
                }
            }
            __syncthreads();
            prefix |= static_cast<uint64_t>(sh_sel) << (8 * d);
            mask |= 255ull << (8 * d);
            want = sh_want;
            const unsigned cnt = sh_cnt;
            __syncthreads();
            if (cnt == 1 && d > 0) {
                // the selected bin holds one key: it is the one
                if (regs) {
                    const uint64_t hmask = mask & 0xFFFFFFFF00000000ull;
#pragma unroll
                    for (int j = 0; j < kKeyRegs; ++j) {
                        if (kh[j] != 0xFFFFFFFFu &&
                            ((static_cast<uint64_t>(kh[j]) << 32) & hmask) == (prefix & hmask)) {
                            const uint64_t key = keys[tid_o + static_cast<long long>(j) * kThreads];
                            if ((key & mask) == prefix && key <= limit) sh_theta = key;
                        }
                    }
                } else {
                    for (long long i = tid; i < n_items; i += kThreads) {
                        const uint64_t key = keys[i];
                        if (key != kNoKey && (key & mask) == prefix && key <= limit) sh_theta = key;
                    }
                }
                __syncthreads();
                const uint64_t found = sh_theta;
                __syncthreads();
                return found;
            }
        }
        return prefix;
    };

    // 2. threshold key: every candidate has key <= theta
    uint64_t theta;
    if (dsel == 0) {
        theta = 0;  // keys of positive S are > 0: nothing is taken
    } else if (dsel == static_cast<long long>(n_pos)) {
        theta = kNoKey - 1;
    } else {
        theta = select_key(0, 0, static_cast<unsigned>(dsel - 1), 7, kNoKey - 1, in_regs);
    }

    // With tau one positive constant over every batch size the walk visits
    // ([B, B + D]), the objective (B + sum S) / tau rises strictly exactly
    // when a taken S does not vanish against the fp64 running total (at most
    // B + dsel).  When the smallest candidate S is at least (B + dsel) 2^-40,
    // no comparison comes near rounding and the walk takes all dsel
    // candidates: the threshold found above stands and nothing is sorted.
    const bool flat_walk =
        curve.n > 0 && curve.flat && dsel > 0 && dsel < static_cast<long long>(n_pos) &&
        static_cast<double>(survival_of(static_cast<uint32_t>(theta >> 32))) >=
            static_cast<double>(B + dsel) * 0x1p-40;
    if (curve.n > 0 && dsel > 0 && !flat_walk) {
        // 3. sort the candidates; the strict-rise test sets the threshold
        int npow = kThreads;
        while (npow < dsel) npow <<= 1;
        if (tid == 0) sh_ncand = 0;
        __syncthreads();
        if (in_regs && npow <= kSortMax) {
            // B * K <= 32768 and at most 16384 candidates: their high words
            // ~bits(S) are sorted in LDS.  The walk needs only the S sequence, which equal
            // S values leave unchanged; the exact threshold key follows from
            // the stop rank.
            uint32_t* sh_w = reinterpret_cast<uint32_t*>(sh_sort);
            const uint32_t th = static_cast<uint32_t>(theta >> 32);
#pragma unroll
            for (int j = 0; j < kKeyRegs; ++j) {
                if (static_cast<long long>(j) * kThreads < n_items) {
                    const uint32_t h = kh[j];
                    bool take = h != 0xFFFFFFFFu && h <= th;
                    if (take && h == th) take = full_key(j) <= theta;
                    const int slot = compact_slot(&sh_ncand, take);
                    if (slot >= 0 && slot < kSortWords) sh_w[slot] = h;
                }
            }
            __syncthreads();
            const int n = static_cast<int>(sh_ncand);  // == dsel
            for (int i = n + tid; i < npow; i += kThreads) sh_w[i] = 0xFFFFFFFFu;
            __syncthreads();
            switch (npow / kThreads) {
                case 1: sort_words_lds<1>(sh_w); break;
                case 2: sort_words_lds<2>(sh_w); break;
                case 4: sort_words_lds<4>(sh_w); break;
                case 8: sort_words_lds<8>(sh_w); break;
                default: sort_words_lds<16>(sh_w); break;
            }
            const int stop = curve_stop(sh_w, n, B, curve, sh_f64, &sh_stop);
            if (stop == 0) {
                theta = 0;
            } else {
                // the stop-th key: the candidates with a smaller high word, then
                // rank `r` among those that share the stop item's high word
                const uint32_t hs = sh_w[stop - 1];
                int lo = 0, hi = stop - 1;  // first index holding hs
                while (lo < hi) {
                    const int mid = (lo + hi) >> 1;
                    if (sh_w[mid] < hs) lo = mid + 1; else hi = mid;
                }
                const bool unique = lo == stop - 1 && (stop == n || sh_w[stop] != hs);
                __syncthreads();
                // (keys read back from memory: the register words end at the
                // compaction, which leaves the sort its registers)
                if (unique) {
                    for (long long i = tid; i < n_items; i += kThreads) {
                        const uint64_t key = keys[i];
                        if (key != kNoKey && static_cast<uint32_t>(key >> 32) == hs && key <= theta)
                            sh_theta = key;
                    }
                    __syncthreads();
                    theta = sh_theta;
                } else {
                    theta = select_key(static_cast<uint64_t>(hs) << 32, 0xFFFFFFFF00000000ull,
                                       static_cast<unsigned>(stop - 1 - lo), 3, theta, false);
                }
            }
        } else {
            for (long long i0 = 0; i0 < n_items; i0 += kThreads) {
                const long long i = i0 + tid;
                const uint64_t key = i < n_items ? keys[i] : kNoKey;
                const int slot = compact_slot(&sh_ncand, key != kNoKey && key <= theta);
                if (slot >= 0) sorted[slot] = key;
            }
            __syncthreads();
            const int n = static_cast<int>(sh_ncand);  // == dsel
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
            const int stop = curve_stop(sorted, n, B, curve, sh_f64, &sh_stop);
            theta = stop > 0 ? sorted[stop - 1] : 0;
        }
    }

    // 4. otherwise L_b = number of candidate keys of request b (the taken
    // items: keys at or below the threshold)
    if (!take_all) {
        for (int b = tid; b < B; b += kThreads) {
            int L = 0;
            const uint64_t* row = keys + static_cast<size_t>(b) * K;
            for (int k0 = 0; k0 < K; k0 += 8) {  // eight loads in flight, none conditional
                uint64_t kv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) kv[u] = row[min(k0 + u, K - 1)];
#pragma unroll
                for (int u = 0; u < 8; ++u)
                    L += (k0 + u < K && kv[u] != kNoKey && kv[u] <= theta);
            }
            lengths[b] = L;
            if (b == tid) my_len = L;
        }
    }
    __syncthreads();

    // 5. row_offsets = exclusive scan of L_b + 1 (thread tid holds L of request
    // tid while B <= kThreads; larger batches read the lengths back in chunks)
    if (B <= kThreads) {
        long long total = 0;
        const long long v = tid < B ? my_len + 1 : 0;
        const long long before =
            block_exclusive_scan<long long>(v, reinterpret_cast<long long*>(sh_u64), &total);
        if (tid < B) row_offsets[tid] = before;
        if (tid == 0) row_offsets[B] = total;
    } else {
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
    // tau is constant on [B, B + D] when it takes one value at both ends and
    // at every point inside (piecewise linear between the points)
    c.flat = 0;
    if (c.n > 0) {
        const double lo = static_cast<double>(a.B);
        const double hi = lo + static_cast<double>(std::max<long long>(0, a.budget - a.B));
        const double t0 = curve_tau(c, lo);
        bool flat = t0 > 0.0 && curve_tau(c, hi) == t0;
        for (int i = 0; i < c.n && flat; ++i)
            if (c.cn[i] > lo && c.cn[i] < hi && c.ct[i] != t0) flat = false;
        c.flat = flat ? 1 : 0;
    }
    ProfScope scope(DSPARK_KERNEL_SCHEDULE, a.stream);
    hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kThreads), 0, a.stream, a.conf, a.B, a.K,
                       static_cast<long long>(a.budget), c, a.lengths, a.row_offsets, a.survival,
                       keys, sorted, static_cast<int>(npow));
    return hipGetLastError();
}

}  // namespace dspark
