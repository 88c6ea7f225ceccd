// kernels.hpp -- host-side launchers of the HIP kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/dspark.h"

namespace dspark {

// Vocabulary entries per partial (one workgroup strip) of the two draft paths.
constexpr int kValuStrip = 1024;  // 256 threads x 4 entries
constexpr int kMfmaStrip = 128;   // 4 MFMA row tiles of 32
constexpr int kMinStrip = 64;     // narrowest strip of any draft path (sizes the partials)

// Stored per-strip reduction partials: (max, sum, perturbed best, logit at the
// best) as float4 plus the best index.
struct PartialBuf {
    float4* v;
    int32_t* idx;
};

// Event timing hooks (profile.hip): prof_begin returns a slot (or -1 when the
// kernel is not being timed) to hand to prof_end after the launch.
int prof_begin(int kernel, hipStream_t stream);
void prof_end(int slot, hipStream_t stream);
hipError_t profile_open(uint32_t mask, int32_t capacity);
hipError_t profile_close(double* total_ms, int64_t* launches, int64_t* timed);

struct ProfScope {
    int slot;
    hipStream_t stream;
    ProfScope(int kernel, hipStream_t s) : slot(prof_begin(kernel, s)), stream(s) {}
    ~ProfScope() { prof_end(slot, stream); }
};

inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct DraftArgs {
    const void* base;
    dspark_dtype logit_dt;
    const void* A;
    const void* W;
    dspark_dtype factor_dt;
    const int32_t* prev_token;
    const float* temperature;
    uint64_t seed;
    int B, K, V, r;
    int32_t* tokens;
    float* logp;
    float* lse;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

size_t draft_workspace_bytes(int B, int K, int V, int r);
bool draft_uses_mfma(const DraftArgs& a);
bool parallel_supported(const DraftArgs& a);
hipError_t launch_draft(const DraftArgs& a);
// Fold the per-row partials into each row's token (draft.hip): k >= 0 is step
// k of the Markov head (rows = requests); k < 0 is parallel drafting (rows =
// B K, no factors).
hipError_t launch_draft_combine(const DraftArgs& a, PartialBuf part, int n_parts, int n_rows, int k);

struct VerifyArgs {
    const int32_t* tokens;
    const int32_t* prev_token;
    const float* draft_logp;
    const float* draft_lse;
    const void* base;
    dspark_dtype logit_dt;
    const void* A;
    const void* W;
    dspark_dtype factor_dt;
    const void* target;
    int64_t n_rows;
    const int64_t* row_off;
    const int32_t* lengths;
    const float* temperature;
    uint64_t seed;
    int B, K, V, r;
    int32_t* accepted;
    int32_t* next_token;
    float* row_lse_t;
    float* row_logratio;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

size_t verify_workspace_bytes(int B, int K, int V, int r);

// Residual draw for the rejected sampled requests (MFMA path).
struct ResidualArgs {
    const VerifyArgs* v;
    const int32_t* list;   // rejected requests
    const int32_t* count;  // device count of list entries
    const float* lse_tab;  // [B][K+1] target log-normalisers
    PartialBuf res;
    PartialBuf fall;
    int n_strips;
};
bool residual_mfma_supported(const VerifyArgs& a);
// How the residual strip partials of one listed request are laid out: n_parts
// per request, or (wgs > 0) a split of a wgs-workgroup grid over the request
// groups of nw wavefronts the list fills, known only on the device
// (residual_parts).
struct ResGeom {
    int n_parts;
    int wgs;
    int nw;
};
// Parts per request group when the list fills `groups` groups of a grid of
// `wgs` workgroups over n_strips strips.
__host__ __device__ inline int residual_parts(int n_strips, int wgs, int groups) {
    const int p = wgs / (groups > 0 ? groups : 1);
    return p < 1 ? 1 : (p < n_strips ? p : n_strips);
}
hipError_t launch_residual_mfma(const ResidualArgs& a, ResGeom* geom);
hipError_t launch_verify(const VerifyArgs& a);
// Compute units of the current device (queried once per device).
int device_cus();

constexpr int kMaxCurvePoints = 64;

struct ScheduleArgs {
    const float* conf;
    int B, K;
    int64_t budget;
    int n_points;
    double curve_n[kMaxCurvePoints];
    double curve_tau[kMaxCurvePoints];
    int32_t* lengths;
    int64_t* row_offsets;
    float* survival;
    void* ws;
    size_t ws_bytes;
    hipStream_t stream;
};

size_t schedule_workspace_bytes(int B, int K);
hipError_t launch_schedule(const ScheduleArgs& a);

}  // namespace dspark
