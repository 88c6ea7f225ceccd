// api.hip -- exported C ABI (include/dspark.h): argument validation, workspace
// sizing and dispatch to the kernel launchers.  Nothing here allocates device
// memory or synchronises the stream.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "kernels.hpp"

// Scratch memory of dspark_draft_sample_noalloc, one copy per device (loaded
// with the code object; held until the process ends).  Host code never uses
// this name as an address: it holds a host-side stand-in.  The device address
// comes from hipGetSymbolAddress, once per device (noalloc_scratch below).
static __device__ __align__(256) unsigned char scratch[DSPARK_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_last_error[512] = "";

dspark_status fail(dspark_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

dspark_status ok() {
    g_last_error[0] = '\0';
    return DSPARK_OK;
}

bool valid_dtype(dspark_dtype d) { return d == DSPARK_F32 || d == DSPARK_BF16; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

dspark_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(DSPARK_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};  // device address of `scratch` per device

// Device address of the current device's copy of `scratch`, looked up on the
// first call on that device (with it current) and kept.
hipError_t noalloc_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (p == nullptr) return hipErrorInvalidSymbol;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

// Validation shared by both draft entry points; fills everything in a but
// the workspace.  Returns DSPARK_OK with *nothing = true for empty problems.
dspark_status draft_checked(const char* who, const void* base_logits, dspark_dtype logit_dt,
                            const void* A, const void* W, dspark_dtype factor_dt,
                            const int32_t* prev_token, const float* temperature, uint64_t seed,
                            int32_t B, int32_t K, int32_t V, int32_t r, int32_t* draft_tokens,
                            float* draft_logp, float* draft_lse, void* stream,
                            dspark::DraftArgs* a, bool* nothing) {
    *nothing = false;
    if (!valid_dtype(logit_dt) || !valid_dtype(factor_dt))
        return fail(DSPARK_ERR_UNSUPPORTED_DTYPE, "%s: unsupported dtype (%d, %d)", who,
                    static_cast<int>(logit_dt), static_cast<int>(factor_dt));
    if (B < 0 || K < 0) return fail(DSPARK_ERR_INVALID_ARG, "%s: B=%d K=%d", who, B, K);
    if (V < 1 || V >= (1 << 30)) return fail(DSPARK_ERR_INVALID_ARG, "%s: V=%d", who, V);
    if (r < 1 || r > 1024) return fail(DSPARK_ERR_INVALID_ARG, "%s: r=%d", who, r);
    if (B == 0 || K == 0) {
        *nothing = true;
        return ok();
    }
    if (!base_logits || !prev_token || !temperature || !draft_tokens)
        return fail(DSPARK_ERR_INVALID_ARG, "%s: NULL required pointer", who);
    if ((A == nullptr) != (W == nullptr))
        return fail(DSPARK_ERR_INVALID_ARG, "%s: A and W must both be set or both NULL", who);
    if (static_cast<int64_t>(B) * K > (int64_t{1} << 31))
        return fail(DSPARK_ERR_INVALID_ARG, "%s: B*K too large", who);
    *a = dspark::DraftArgs{base_logits, logit_dt,     A,         W,          factor_dt,
                           prev_token,  temperature,  seed,      B,          K,
                           V,           r,            draft_tokens, draft_logp, draft_lse,
                           nullptr,     0,            static_cast<hipStream_t>(stream)};
    if (!A && !dspark::parallel_supported(*a))
        return fail(DSPARK_ERR_INVALID_ARG,
                    "%s: drafting without factors needs bf16 logits, V %% 8 == 0 and a "
                    "16-byte aligned base", who);
    return ok();
}

}  // namespace

extern "C" {

const char* dspark_version(void) { return "dspark-mi355x 0.1.0 (gfx950)"; }

const char* dspark_last_error(void) { return g_last_error; }

size_t dspark_draft_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t r) {
    if (B < 0 || K < 0 || V < 1 || r < 1) return 0;
    return dspark::draft_workspace_bytes(B, K, V, r);
}

dspark_status dspark_draft_sample(const void* base_logits, dspark_dtype logit_dt, const void* A,
                                  const void* W, dspark_dtype factor_dt,
                                  const int32_t* prev_token, const float* temperature,
                                  uint64_t seed, int32_t B, int32_t K, int32_t V, int32_t r,
                                  int32_t* draft_tokens, float* draft_logp, float* draft_lse,
                                  void* workspace, size_t ws_bytes, void* stream) {
    dspark::DraftArgs a;
    bool nothing = false;
    dspark_status st = draft_checked("draft_sample", base_logits, logit_dt, A, W, factor_dt,
                                     prev_token, temperature, seed, B, K, V, r, draft_tokens,
                                     draft_logp, draft_lse, stream, &a, &nothing);
    if (st != DSPARK_OK || nothing) return st;
    const size_t need = dspark::draft_workspace_bytes(B, K, V, r);
    if (!workspace || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE_TOO_SMALL, "draft_sample: workspace %zu < %zu bytes",
                    ws_bytes, need);
    if (!aligned(workspace, 256))
        return fail(DSPARK_ERR_INVALID_ARG, "draft_sample: workspace not 256-byte aligned");
    a.ws = workspace;
    a.ws_bytes = ws_bytes;
    return hip_status(dspark::launch_draft(a), "draft_sample");
}

dspark_status dspark_draft_sample_noalloc(const void* base_logits, dspark_dtype logit_dt,
                                          const void* A, const void* W, dspark_dtype factor_dt,
                                          const int32_t* prev_token, const float* temperature,
                                          uint64_t seed, int32_t B, int32_t K, int32_t V,
                                          int32_t r, int32_t* draft_tokens, float* draft_logp,
                                          float* draft_lse, void* stream) {
    dspark::DraftArgs a;
    bool nothing = false;
    dspark_status st = draft_checked("draft_sample_noalloc", base_logits, logit_dt, A, W,
                                     factor_dt, prev_token, temperature, seed, B, K, V, r,
                                     draft_tokens, draft_logp, draft_lse, stream, &a, &nothing);
    if (st != DSPARK_OK || nothing) return st;
    const size_t need = dspark::draft_workspace_bytes(B, K, V, r);
    const size_t have = DSPARK_NOALLOC_SCRATCH_BYTES;
    if (need > have)
        return fail(DSPARK_ERR_WORKSPACE_TOO_SMALL,
                    "draft_sample_noalloc: these sizes need %zu bytes of scratch, more than the "
                    "%zu the library holds per device; call dspark_draft_sample with a workspace",
                    need, have);
    void* ptr = nullptr;
    hipError_t e = noalloc_scratch(&ptr);
    if (e != hipSuccess) return hip_status(e, "draft_sample_noalloc: scratch address");
    a.ws = ptr;
    a.ws_bytes = have;
    return hip_status(dspark::launch_draft(a), "draft_sample_noalloc");
}

size_t dspark_schedule_workspace_bytes(int32_t B, int32_t K) {
    if (B < 0 || K < 0) return 0;
    return dspark::schedule_workspace_bytes(B, K);
}

dspark_status dspark_schedule(const float* conf, int32_t B, int32_t K, int64_t budget_tokens,
                              const float* curve_n, const float* curve_latency, int32_t n_points,
                              int32_t* lengths, int64_t* row_offsets, float* survival,
                              void* workspace, size_t ws_bytes, void* stream) {
    if (B < 0 || K < 0 || K > 64)
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: B=%d K=%d (0 <= K <= 64)", B, K);
    if (static_cast<int64_t>(B) * K > (int64_t{1} << 22))
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: B*K too large");
    if (n_points < 0 || n_points > dspark::kMaxCurvePoints)
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: n_points=%d", n_points);
    if (n_points > 0 && (!curve_n || !curve_latency))
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: NULL curve arrays with n_points > 0");
    if (!lengths || !row_offsets || (B > 0 && K > 0 && !conf))
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: NULL required pointer");
    dspark::ScheduleArgs a;
    a.n_points = n_points;
    for (int i = 0; i < n_points; ++i) {
        a.curve_n[i] = curve_n[i];
        a.curve_tau[i] = curve_latency[i];
        if (!(curve_latency[i] > 0.0f) || (i > 0 && !(curve_n[i] > curve_n[i - 1])))
            return fail(DSPARK_ERR_INVALID_ARG,
                        "schedule: curve needs increasing N and positive latency");
    }
    const size_t need = dspark::schedule_workspace_bytes(B, K);
    if (ws_bytes < need || (need > 0 && !workspace))
        return fail(DSPARK_ERR_WORKSPACE_TOO_SMALL, "schedule: workspace %zu < %zu bytes",
                    ws_bytes, need);
    if (workspace && !aligned(workspace, 256))
        return fail(DSPARK_ERR_INVALID_ARG, "schedule: workspace not 256-byte aligned");
    a.conf = conf;
    a.B = B;
    a.K = K;
    a.budget = budget_tokens;
    a.lengths = lengths;
    a.row_offsets = row_offsets;
    a.survival = survival;
    a.ws = workspace;
    a.ws_bytes = ws_bytes;
    a.stream = static_cast<hipStream_t>(stream);
    return hip_status(dspark::launch_schedule(a), "schedule");
}

size_t dspark_verify_workspace_bytes(int32_t B, int32_t K, int32_t V, int32_t r) {
    if (B < 0 || K < 0 || V < 1 || r < 1) return 0;
    return dspark::verify_workspace_bytes(B, K, V, r);
}

dspark_status dspark_verify(const int32_t* draft_tokens, const int32_t* prev_token,
                            const float* draft_logp, const float* draft_lse,
                            const void* base_logits, dspark_dtype logit_dt, const void* A,
                            const void* W, dspark_dtype factor_dt, const void* target_logits,
                            int64_t n_target_rows, const int64_t* target_row_offsets,
                            const int32_t* lengths,
                            const float* temperature, uint64_t seed, int32_t B, int32_t K,
                            int32_t V, int32_t r, int32_t* accepted, int32_t* next_token,
                            float* row_lse_t, float* row_logratio, void* workspace,
                            size_t ws_bytes, void* stream) {
    if (!valid_dtype(logit_dt) || !valid_dtype(factor_dt))
        return fail(DSPARK_ERR_UNSUPPORTED_DTYPE, "verify: unsupported dtype (%d, %d)",
                    static_cast<int>(logit_dt), static_cast<int>(factor_dt));
    if (B < 0 || K < 0) return fail(DSPARK_ERR_INVALID_ARG, "verify: B=%d K=%d", B, K);
    if (V < 1 || V >= (1 << 30)) return fail(DSPARK_ERR_INVALID_ARG, "verify: V=%d", V);
    if (r < 1 || r > 1024) return fail(DSPARK_ERR_INVALID_ARG, "verify: r=%d", r);
    if (n_target_rows < 0) return fail(DSPARK_ERR_INVALID_ARG, "verify: n_target_rows < 0");
    if (B == 0) return ok();
    if (!prev_token || !target_logits || !target_row_offsets || !temperature || !accepted ||
        !next_token)
        return fail(DSPARK_ERR_INVALID_ARG, "verify: NULL required pointer");
    if (K > 0 && (!draft_tokens || !draft_logp || !draft_lse || !base_logits))
        return fail(DSPARK_ERR_INVALID_ARG, "verify: NULL draft input");
    if ((A == nullptr) != (W == nullptr))
        return fail(DSPARK_ERR_INVALID_ARG, "verify: A and W must both be set or both NULL");
    if (static_cast<int64_t>(B) * (K + 1) > (int64_t{1} << 31))
        return fail(DSPARK_ERR_INVALID_ARG, "verify: B*(K+1) too large");
    const size_t need = dspark::verify_workspace_bytes(B, K, V, r);
    if (!workspace || ws_bytes < need)
        return fail(DSPARK_ERR_WORKSPACE_TOO_SMALL, "verify: workspace %zu < %zu bytes", ws_bytes,
                    need);
    if (!aligned(workspace, 256))
        return fail(DSPARK_ERR_INVALID_ARG, "verify: workspace not 256-byte aligned");
    dspark::VerifyArgs a{draft_tokens, prev_token,  draft_logp,  draft_lse,      base_logits,
                         logit_dt,     A,           W,           factor_dt,      target_logits,
                         n_target_rows, target_row_offsets,        lengths,     temperature,    seed,
                         B,            K,           V,           r,              accepted,
                         next_token,   row_lse_t,   row_logratio, workspace,     ws_bytes,
                         static_cast<hipStream_t>(stream)};
    return hip_status(dspark::launch_verify(a), "verify");
}

dspark_status dspark_profile_begin(uint32_t kernel_mask, int32_t max_launches) {
    if (kernel_mask == 0 || max_launches < 1 || max_launches > (1 << 20))
        return fail(DSPARK_ERR_INVALID_ARG, "profile: mask=0x%x max_launches=%d", kernel_mask,
                    max_launches);
    hipError_t e = dspark::profile_open(kernel_mask, max_launches);
    if (e == hipErrorInvalidValue)
        return fail(DSPARK_ERR_INVALID_ARG, "profile: a session is already open");
    return hip_status(e, "profile_begin");
}

dspark_status dspark_profile_end(double* total_ms, int64_t* launches, int64_t* timed) {
    return hip_status(dspark::profile_close(total_ms, launches, timed), "profile_end");
}

}  // extern "C"
