// profile.hip -- optional per-kernel timing with HIP events (dspark_profile_*).
//
// While a profiling session is open, every launch of a kernel whose bit is set
// in the session mask is bracketed by two hipEvents recorded on the stream the
// kernel is launched on, so the elapsed time between them is that launch's
// duration as the stream saw it.  The events are created when the session
// opens (a fixed pool; launches beyond it are counted but not timed) and are
// read and destroyed when it closes.  With no session open the hooks cost one
// relaxed atomic load per launch.
#include <atomic>
#include <mutex>
#include <vector>

#include "kernels.hpp"

namespace dspark {
namespace {

struct Record {
    int kernel;
    hipEvent_t start;
    hipEvent_t stop;
};

struct Session {
    std::mutex mu;
    std::atomic<uint32_t> mask{0};
    std::vector<hipEvent_t> pool;  // 2 * capacity events
    std::vector<Record> used;
    int64_t launches[DSPARK_KERNEL_COUNT] = {};
};

Session& session() {
    static Session s;
    return s;
}

}  // namespace

int prof_begin(int kernel, hipStream_t stream) {
    Session& s = session();
    if ((s.mask.load(std::memory_order_relaxed) & (1u << kernel)) == 0) return -1;
    std::lock_guard<std::mutex> g(s.mu);
    if ((s.mask.load(std::memory_order_relaxed) & (1u << kernel)) == 0) return -1;
    ++s.launches[kernel];
    const size_t slot = s.used.size();
    if (2 * slot + 1 >= s.pool.size()) return -1;
    Record r{kernel, s.pool[2 * slot], s.pool[2 * slot + 1]};
    if (hipEventRecord(r.start, stream) != hipSuccess) return -1;
    s.used.push_back(r);
    return static_cast<int>(slot);
}

void prof_end(int slot, hipStream_t stream) {
    if (slot < 0) return;
    Session& s = session();
    std::lock_guard<std::mutex> g(s.mu);
    if (static_cast<size_t>(slot) < s.used.size())
        (void)hipEventRecord(s.used[slot].stop, stream);
}

hipError_t profile_open(uint32_t mask, int32_t capacity) {
    Session& s = session();
    std::lock_guard<std::mutex> g(s.mu);
    if (mask == 0 || s.mask.load() != 0) return hipErrorInvalidValue;
    for (hipEvent_t ev : s.pool) (void)hipEventDestroy(ev);
    s.pool.assign(2 * static_cast<size_t>(capacity), nullptr);
    for (size_t i = 0; i < s.pool.size(); ++i) {
        hipError_t e = hipEventCreate(&s.pool[i]);
        if (e != hipSuccess) {
            for (size_t j = 0; j < i; ++j) (void)hipEventDestroy(s.pool[j]);
            s.pool.clear();
            return e;
        }
    }
    s.used.clear();
    for (int64_t& n : s.launches) n = 0;
    s.mask.store(mask);
    return hipSuccess;
}

hipError_t profile_close(double* total_ms, int64_t* launches, int64_t* timed) {
    Session& s = session();
    std::lock_guard<std::mutex> g(s.mu);
    s.mask.store(0);
    hipError_t err = hipSuccess;
    for (int k = 0; k < DSPARK_KERNEL_COUNT; ++k) {
        if (total_ms) total_ms[k] = 0.0;
        if (launches) launches[k] = s.launches[k];
        if (timed) timed[k] = 0;
    }
    for (const Record& r : s.used) {
        float ms = 0.0f;
        hipError_t e = hipEventSynchronize(r.stop);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.start, r.stop);
        if (e != hipSuccess) {
            err = e;
            continue;
        }
        if (total_ms) total_ms[r.kernel] += ms;
        if (timed) ++timed[r.kernel];
    }
    for (hipEvent_t ev : s.pool) (void)hipEventDestroy(ev);
    s.pool.clear();
    s.used.clear();
    return err;
}

}  // namespace dspark
