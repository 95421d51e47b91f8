// Host-side launchers of the libspecverify kernels (internal; the C ABI in
// sv_api.cpp validates arguments before calling these).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "libspecverify.h"

namespace sv {

// Outputs of sv_pack_varlen, written by the budget's last kernel when given.
struct PackTargets {
    const int32_t* last_token;
    const int32_t* draft_tokens;
    int32_t* cu_rows;
    int32_t* row_req;
    int32_t* row_pos;
    int32_t* packed_tokens;
};

hipError_t launch_budget(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                         const float* cost, int t_base, int n_bonus, int32_t* kept,
                         int32_t* budget, float* survival, int32_t* dev_error, void* ws,
                         const PackTargets* pack, hipStream_t stream);
hipError_t launch_allocate(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                           const int32_t* budget_in, int32_t* kept, int32_t* budget_used,
                           float* survival, int32_t* dev_error, void* ws,
                           const PackTargets* pack, hipStream_t stream);
size_t budget_workspace_bytes(int n_req, int k_max);

hipError_t launch_uniform_k(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                            const float* cost, int t_base, int n_bonus, int32_t* kept,
                            int32_t* k_out, double* scores, int32_t* dev_error,
                            hipStream_t stream);

hipError_t launch_pack(const int32_t* kept, const int32_t* last_token,
                       const int32_t* draft_tokens, int n_req, int k_max, int32_t* cu_rows,
                       int32_t* row_req, int32_t* row_pos, int32_t* packed_tokens,
                       int32_t* dev_error, hipStream_t stream);

struct VerifyArgs {
    const void* target;
    int64_t target_ld;
    int64_t target_rows;
    const void* draft;
    int64_t draft_ld;
    sv_dtype dtype;
    int vocab;
    const int32_t* draft_tokens;
    const int32_t* cu_rows;
    int n_req;
    int k_max;
    sv_mode mode;
    float temperature;
    uint64_t seed;
    uint64_t step;
    int32_t* out_tokens;
    int32_t* out_accepted;
    float* out_p_draft;
    float* out_q_draft;
    float* out_residual_mass;
    float* out_q_entropy;
    float* out_q_max;
    int32_t* dev_error;
    void* ws;
    int stages;  // bit 0: pass 1 (row statistics), bit 1: pass 2 (decide and draw)
};

size_t verify_workspace_bytes(int n_req, int k_max);
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
// sv_verify's host checks of everything but the workspace (sv_api.cpp): SV_OK means
// a launch may follow (nothing to launch when n_req = 0).
sv_status check_verify(const VerifyArgs& a);
// The status of a call's launches (sv_api.cpp): SV_ERR_LAUNCH if the runtime
// refused one; with SV_FORCE_SYNC set (and the stream not capturing) the call
// also waits for the stream and reports a failed kernel the same way.
sv_status finish_launch(hipError_t e, hipStream_t stream);

hipError_t launch_accept_stats(const int32_t* accepted, const int32_t* cu_rows, int n_req,
                               int k_max, uint64_t* attempted, uint64_t* accepted_at,
                               uint64_t* totals, hipStream_t stream);
hipError_t launch_calibrate_update(float* theta, const float* q_draft, const float* q_entropy,
                                   const float* q_max, const int32_t* accepted,
                                   const int32_t* cu_rows, int n_req, int k_max, float lr,
                                   int32_t* count_out, hipStream_t stream);
hipError_t launch_calibrate_predict(const float* theta, const float* q_draft,
                                    const float* q_entropy, const float* q_max, int n_req,
                                    int k_max, float* conf, hipStream_t stream);

hipError_t launch_philox_uniforms(uint64_t seed, uint64_t step, int n_req, int n_pos, float* u,
                                  float* v, hipStream_t stream);

}  // namespace sv
