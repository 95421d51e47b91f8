// C ABI of libspecverify: host-side validation, then launches on the caller's
// stream.  Every check here runs before any HIP call, so a rejected call
// touches neither the device nor any output.  Two environment variables serve
// debugging only: SV_FORCE_SYNC (wait after the launches, report a failed
// kernel) and SV_DEBUG_CHECKS (copy the index inputs to the host and refuse
// what the kernels would flag in dev_error); both are skipped while the
// stream is being captured into a graph.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "libspecverify.h"
#include "sv_launch.h"

namespace {

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// A debug variable is on when set to anything but empty or "0".
bool env_on(const char* name) {
    const char* v = std::getenv(name);
    return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
}

// Waiting on a stream that is being captured would end the capture.
bool capturing(hipStream_t s) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &st) != hipSuccess) return true;  // unknown: do not wait
    return st != hipStreamCaptureStatusNone;
}

bool debug_checks(hipStream_t s) { return env_on("SV_DEBUG_CHECKS") && !capturing(s); }

// n int32 values of device array d, on the host, in stream order.
bool fetch(std::vector<int32_t>& h, const int32_t* d, int64_t n, hipStream_t s) {
    h.assign((size_t)n, 0);
    if (n == 0) return true;
    if (hipMemcpyAsync(h.data(), d, (size_t)n * sizeof(int32_t), hipMemcpyDeviceToHost, s) !=
        hipSuccess)
        return false;
    return hipStreamSynchronize(s) == hipSuccess;
}

// Debug checks of counts in [0, k_max] (draft lengths: SV_DEV_BAD_DRAFT_LEN;
// kept counts: SV_DEV_BAD_KEPT).
sv_status check_counts(const int32_t* counts, int32_t n, int32_t k_max, hipStream_t s) {
    if (n == 0 || !debug_checks(s)) return SV_OK;
    std::vector<int32_t> h;
    if (!fetch(h, counts, n, s)) return SV_ERR_LAUNCH;
    for (int32_t v : h)
        if (v < 0 || v > k_max) return SV_ERR_DATA;
    return SV_OK;
}

// Debug checks of a verify call's row offsets and kept draft ids, as the
// kernels test them (SV_DEV_BAD_CU_ROWS, SV_DEV_BAD_TOKEN).
sv_status check_verify_data(const sv::VerifyArgs& v, hipStream_t s) {
    if (v.n_req == 0 || !debug_checks(s)) return SV_OK;
    std::vector<int32_t> cu, tok;
    if (!fetch(cu, v.cu_rows, (int64_t)v.n_req + 1, s)) return SV_ERR_LAUNCH;
    if (v.k_max > 0 && !fetch(tok, v.draft_tokens, (int64_t)v.n_req * v.k_max, s))
        return SV_ERR_LAUNCH;
    for (int32_t r = 0; r < v.n_req; ++r) {
        const int64_t lo = cu[r], hi = cu[r + 1], b = hi - lo - 1;
        if (lo < 0 || b < 0 || b > v.k_max || hi > v.target_rows) return SV_ERR_DATA;
        for (int64_t j = 0; j < b; ++j) {
            const int32_t d = tok[(size_t)r * v.k_max + j];
            if (d < 0 || d >= v.vocab) return SV_ERR_DATA;
        }
    }
    return SV_OK;
}

}  // namespace

namespace sv {

sv_status finish_launch(hipError_t e, hipStream_t stream) {
    if (e != hipSuccess) return SV_ERR_LAUNCH;
    if (env_on("SV_FORCE_SYNC") && !capturing(stream)) {
        // the wait's own status carries a failed kernel; an error left by
        // some earlier, unrelated call is not this call's
        if (hipStreamSynchronize(stream) != hipSuccess) return SV_ERR_LAUNCH;
    }
    return SV_OK;
}

sv_status check_verify(const VerifyArgs& v) {
    if (v.dtype != SV_F32 && v.dtype != SV_BF16) return SV_ERR_DTYPE;
    if (v.mode != SV_STOCHASTIC && v.mode != SV_GREEDY) return SV_ERR_VALUE;
    if (v.n_req < 0 || v.k_max < 0 || v.k_max > SV_MAX_DRAFT) return SV_ERR_SHAPE;
    if ((int64_t)v.n_req * (2 * v.k_max + 1) > SV_MAX_VERIFY_SLOTS) return SV_ERR_SHAPE;
    if (v.vocab < 1 || v.vocab > SV_MAX_VOCAB) return SV_ERR_SHAPE;
    if (v.target_rows < 0 || v.target_ld < v.vocab) return SV_ERR_SHAPE;
    const bool stochastic = v.mode == SV_STOCHASTIC;
    if (stochastic && v.draft_ld < v.vocab) return SV_ERR_SHAPE;
    if (stochastic && (!std::isfinite(v.temperature) || !(v.temperature > 0.0f)))
        return SV_ERR_VALUE;
    if (v.n_req == 0) return SV_OK;
    if (v.target == nullptr || v.cu_rows == nullptr || v.out_tokens == nullptr ||
        v.out_accepted == nullptr)
        return SV_ERR_NULL;
    if (v.k_max > 0 && v.draft_tokens == nullptr) return SV_ERR_NULL;
    if (stochastic && v.k_max > 0 && v.draft == nullptr) return SV_ERR_NULL;
    // the largest element offset a kernel may form must fit int64
    if ((double)v.target_rows * (double)v.target_ld > 9.0e18) return SV_ERR_SHAPE;
    // log2(e) / T must be a finite fp32
    if (stochastic && (1.4426950408889634 / (double)v.temperature) > 3.0e38) return SV_ERR_VALUE;
    return SV_OK;
}

}  // namespace sv

extern "C" {

const char* sv_status_str(sv_status s) {
    switch (s) {
        case SV_OK: return "ok";
        case SV_ERR_NULL: return "a required pointer is NULL";
        case SV_ERR_SHAPE: return "a size or stride is out of range";
        case SV_ERR_DTYPE: return "unknown dtype";
        case SV_ERR_VALUE: return "a scalar argument is out of range";
        case SV_ERR_WORKSPACE: return "workspace missing or too small";
        case SV_ERR_LAUNCH: return "the HIP runtime refused a kernel launch, or one failed";
        case SV_ERR_CAPACITY: return "the batch needs more than the static workspace holds";
        case SV_ERR_DATA: return "index data on the device is inconsistent (SV_DEBUG_CHECKS)";
        default: break;  // the range markers and any other int
    }
    return "unknown status";
}

size_t sv_budget_workspace_bytes(int32_t n_req, int32_t k_max) {
    if (n_req < 0 || k_max < 0 || n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return 0;
    return sv::budget_workspace_bytes(n_req, k_max);
}

size_t sv_verify_workspace_bytes(int32_t n_req, int32_t k_max) {
    if (n_req < 0 || k_max < 0 || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * (2 * k_max + 1) > SV_MAX_VERIFY_SLOTS)
        return 0;
    return sv::verify_workspace_bytes(n_req, k_max);
}

sv_status sv_cost_table_prepare(const float* raw, int32_t raw_len, int32_t granule, float* out,
                                int32_t out_len) {
    if (raw == nullptr || out == nullptr) return SV_ERR_NULL;
    if (granule < 1 || out_len < 1 || raw_len < 1) return SV_ERR_SHAPE;
    const int64_t last_padded = ((int64_t)(out_len - 1) + granule - 1) / granule * granule;
    if ((int64_t)raw_len < last_padded + 1) return SV_ERR_SHAPE;
    for (int32_t t = 0; t < raw_len; ++t)
        if (!std::isfinite(raw[t]) || !(raw[t] > 0.0f)) return SV_ERR_VALUE;
    // running maximum up to each padded size, read at ceil_g(t)
    float running = raw[0];
    int64_t filled = 0;  // raw entries folded into `running`
    for (int32_t t = 0; t < out_len; ++t) {
        const int64_t padded = ((int64_t)t + granule - 1) / granule * granule;
        while (filled <= padded) {
            if (raw[filled] > running) running = raw[filled];
            ++filled;
        }
        out[t] = running;
    }
    return SV_OK;
}

sv_status sv_budget_select(const float* conf, const int32_t* draft_len, int32_t n_req,
                           int32_t k_max, const float* cost, int32_t cost_len, int32_t t_base,
                           int32_t n_bonus, int32_t* kept, int32_t* budget, float* survival,
                           int32_t* dev_error, void* ws, size_t ws_bytes, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    if (cost == nullptr || budget == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (draft_len == nullptr || kept == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && conf == nullptr) return SV_ERR_NULL;
    if (n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return SV_ERR_SHAPE;
    if (t_base < 0 || n_bonus < 0) return SV_ERR_VALUE;
    if ((int64_t)cost_len < (int64_t)t_base + (int64_t)n_req * k_max + 1) return SV_ERR_SHAPE;
    const size_t need = sv::budget_workspace_bytes(n_req, k_max);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return SV_ERR_WORKSPACE;
    const sv_status dc = check_counts(draft_len, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_budget(conf, draft_len, n_req, k_max, cost, t_base, n_bonus,
                                           kept, budget, survival, dev_error, ws, nullptr,
                                           as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

// The outputs of sv_pack_varlen for the fused calls (sizes: the budget's).
static sv_status check_pack_outputs(int32_t n_req, int32_t k_max, const int32_t* last_token,
                                    const int32_t* draft_tokens, const int32_t* cu_rows,
                                    const int32_t* row_req, const int32_t* row_pos,
                                    const int32_t* packed_tokens) {
    if (cu_rows == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (last_token == nullptr || row_req == nullptr || row_pos == nullptr ||
                      packed_tokens == nullptr))
        return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && draft_tokens == nullptr) return SV_ERR_NULL;
    return SV_OK;
}

sv_status sv_budget_select_pack(const float* conf, const int32_t* draft_len, int32_t n_req,
                                int32_t k_max, const float* cost, int32_t cost_len,
                                int32_t t_base, int32_t n_bonus, const int32_t* last_token,
                                const int32_t* draft_tokens, int32_t* kept, int32_t* budget,
                                float* survival, int32_t* cu_rows, int32_t* row_req,
                                int32_t* row_pos, int32_t* packed_tokens, int32_t* dev_error,
                                void* ws, size_t ws_bytes, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    const sv_status ps = check_pack_outputs(n_req, k_max, last_token, draft_tokens, cu_rows,
                                            row_req, row_pos, packed_tokens);
    if (ps != SV_OK) return ps;
    if (cost == nullptr || budget == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (draft_len == nullptr || kept == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && conf == nullptr) return SV_ERR_NULL;
    if (n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return SV_ERR_SHAPE;
    if (t_base < 0 || n_bonus < 0) return SV_ERR_VALUE;
    if ((int64_t)cost_len < (int64_t)t_base + (int64_t)n_req * k_max + 1) return SV_ERR_SHAPE;
    const size_t need = sv::budget_workspace_bytes(n_req, k_max);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return SV_ERR_WORKSPACE;
    const sv::PackTargets pack{last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens};
    const sv_status dc = check_counts(draft_len, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_budget(conf, draft_len, n_req, k_max, cost, t_base, n_bonus,
                                           kept, budget, survival, dev_error, ws, &pack,
                                           as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_budget_allocate(const float* conf, const int32_t* draft_len, int32_t n_req,
                             int32_t k_max, const int32_t* budget_in, int32_t* kept,
                             int32_t* budget_used, float* survival, int32_t* dev_error, void* ws,
                             size_t ws_bytes, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    if (budget_in == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (draft_len == nullptr || kept == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && conf == nullptr) return SV_ERR_NULL;
    if (n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return SV_ERR_SHAPE;
    const size_t need = sv::budget_workspace_bytes(n_req, k_max);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return SV_ERR_WORKSPACE;
    const sv_status dc = check_counts(draft_len, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_allocate(conf, draft_len, n_req, k_max, budget_in, kept,
                                             budget_used, survival, dev_error, ws, nullptr,
                                             as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_budget_allocate_pack(const float* conf, const int32_t* draft_len, int32_t n_req,
                                  int32_t k_max, const int32_t* budget_in,
                                  const int32_t* last_token, const int32_t* draft_tokens,
                                  int32_t* kept, int32_t* budget_used, float* survival,
                                  int32_t* cu_rows, int32_t* row_req, int32_t* row_pos,
                                  int32_t* packed_tokens, int32_t* dev_error, void* ws,
                                  size_t ws_bytes, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    const sv_status ps = check_pack_outputs(n_req, k_max, last_token, draft_tokens, cu_rows,
                                            row_req, row_pos, packed_tokens);
    if (ps != SV_OK) return ps;
    if (budget_in == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (draft_len == nullptr || kept == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && conf == nullptr) return SV_ERR_NULL;
    if (n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return SV_ERR_SHAPE;
    const size_t need = sv::budget_workspace_bytes(n_req, k_max);
    if (need > 0 && (ws == nullptr || ws_bytes < need)) return SV_ERR_WORKSPACE;
    const sv::PackTargets pack{last_token, draft_tokens, cu_rows, row_req, row_pos, packed_tokens};
    const sv_status dc = check_counts(draft_len, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_allocate(conf, draft_len, n_req, k_max, budget_in, kept,
                                             budget_used, survival, dev_error, ws, &pack,
                                             as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_uniform_k_select(const float* conf, const int32_t* draft_len, int32_t n_req,
                              int32_t k_max, const float* cost, int32_t cost_len, int32_t t_base,
                              int32_t n_bonus, int32_t* kept, int32_t* k_out, double* scores,
                              int32_t* dev_error, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    if (cost == nullptr || k_out == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (draft_len == nullptr || kept == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && conf == nullptr) return SV_ERR_NULL;
    if (n_req > SV_MAX_BUDGET_SLOTS || k_max > SV_MAX_DRAFT ||
        (int64_t)n_req * k_max > SV_MAX_BUDGET_SLOTS)
        return SV_ERR_SHAPE;
    if (t_base < 0 || n_bonus < 0) return SV_ERR_VALUE;
    if ((int64_t)cost_len < (int64_t)t_base + (int64_t)n_req * k_max + 1) return SV_ERR_SHAPE;
    const sv_status dc = check_counts(draft_len, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_uniform_k(conf, draft_len, n_req, k_max, cost, t_base, n_bonus,
                                              kept, k_out, scores, dev_error, as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_pack_varlen(const int32_t* kept, const int32_t* last_token,
                         const int32_t* draft_tokens, int32_t n_req, int32_t k_max,
                         int32_t* cu_rows, int32_t* row_req, int32_t* row_pos,
                         int32_t* packed_tokens, int32_t* dev_error, void* stream) {
    if (n_req < 0 || k_max < 0) return SV_ERR_SHAPE;
    if ((int64_t)n_req * (k_max + 1) > INT32_MAX) return SV_ERR_SHAPE;
    if (cu_rows == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (kept == nullptr || last_token == nullptr || row_req == nullptr ||
                      row_pos == nullptr || packed_tokens == nullptr))
        return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && draft_tokens == nullptr) return SV_ERR_NULL;
    const sv_status dc = check_counts(kept, n_req, k_max, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_pack(kept, last_token, draft_tokens, n_req, k_max, cu_rows,
                                         row_req, row_pos, packed_tokens, dev_error,
                                         as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_verify_stages(const void* target_logits, int64_t target_ld, int64_t target_rows,
                           const void* draft_logits, int64_t draft_ld, sv_dtype dtype,
                           int32_t vocab, const int32_t* draft_tokens, const int32_t* cu_rows,
                           int32_t n_req, int32_t k_max, sv_mode mode, float temperature,
                           uint64_t seed, uint64_t step, int32_t* out_tokens,
                           int32_t* out_accepted, float* out_p_draft, float* out_q_draft,
                           float* out_residual_mass, float* out_q_entropy, float* out_q_max,
                           int32_t* dev_error, void* ws, size_t ws_bytes, int32_t stages,
                           void* stream) {
    if (stages < 1 || stages > 3) return SV_ERR_VALUE;
    const sv::VerifyArgs a{target_logits, target_ld,    target_rows,  draft_logits, draft_ld,
                           dtype,         vocab,        draft_tokens, cu_rows,      n_req,
                           k_max,         mode,         temperature,  seed,         step,
                           out_tokens,    out_accepted, out_p_draft,  out_q_draft,
                           out_residual_mass, out_q_entropy, out_q_max, dev_error,  ws,
                           stages};
    const sv_status st = sv::check_verify(a);
    if (st != SV_OK || n_req == 0) return st;
    const size_t need = sv::verify_workspace_bytes(n_req, k_max);
    if (ws == nullptr || ws_bytes < need) return SV_ERR_WORKSPACE;
    const sv_status dc = check_verify_data(a, as_stream(stream));
    if (dc != SV_OK) return dc;
    const hipError_t e = sv::launch_verify(a, as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_verify(const void* target_logits, int64_t target_ld, int64_t target_rows,
                    const void* draft_logits, int64_t draft_ld, sv_dtype dtype, int32_t vocab,
                    const int32_t* draft_tokens, const int32_t* cu_rows, int32_t n_req,
                    int32_t k_max, sv_mode mode, float temperature, uint64_t seed, uint64_t step,
                    int32_t* out_tokens, int32_t* out_accepted, float* out_p_draft,
                    float* out_q_draft, float* out_residual_mass, float* out_q_entropy,
                    float* out_q_max, int32_t* dev_error, void* ws, size_t ws_bytes,
                    void* stream) {
    return sv_verify_stages(target_logits, target_ld, target_rows, draft_logits, draft_ld, dtype,
                            vocab, draft_tokens, cu_rows, n_req, k_max, mode, temperature, seed,
                            step, out_tokens, out_accepted, out_p_draft, out_q_draft,
                            out_residual_mass, out_q_entropy, out_q_max, dev_error, ws, ws_bytes,
                            3, stream);
}

sv_status sv_accept_stats(const int32_t* accepted, const int32_t* cu_rows, int32_t n_req,
                          int32_t k_max, uint64_t* attempted, uint64_t* accepted_at,
                          uint64_t* totals, void* stream) {
    if (n_req < 0 || k_max < 0 || k_max > SV_MAX_DRAFT) return SV_ERR_SHAPE;
    if (totals == nullptr || (k_max > 0 && (attempted == nullptr || accepted_at == nullptr)))
        return SV_ERR_NULL;
    if (n_req > 0 && (accepted == nullptr || cu_rows == nullptr)) return SV_ERR_NULL;
    const hipError_t e = sv::launch_accept_stats(accepted, cu_rows, n_req, k_max, attempted,
                                                 accepted_at, totals, as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_calibrate_update(float* theta, const float* q_draft, const float* q_entropy,
                              const float* q_max, const int32_t* accepted,
                              const int32_t* cu_rows, int32_t n_req, int32_t k_max, float lr,
                              int32_t* count_out, void* stream) {
    if (n_req < 0 || k_max < 0 || k_max > SV_MAX_DRAFT) return SV_ERR_SHAPE;
    if (!std::isfinite(lr) || lr < 0.0f) return SV_ERR_VALUE;
    if (theta == nullptr) return SV_ERR_NULL;
    if (n_req > 0 && (accepted == nullptr || cu_rows == nullptr)) return SV_ERR_NULL;
    if (n_req > 0 && k_max > 0 && q_draft == nullptr) return SV_ERR_NULL;
    const hipError_t e = sv::launch_calibrate_update(theta, q_draft, q_entropy, q_max, accepted,
                                                     cu_rows, n_req, k_max, lr, count_out,
                                                     as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_calibrate_predict(const float* theta, const float* q_draft, const float* q_entropy,
                               const float* q_max, int32_t n_req, int32_t k_max, float* conf,
                               void* stream) {
    if (n_req < 0 || k_max < 0 || k_max > SV_MAX_DRAFT) return SV_ERR_SHAPE;
    if ((int64_t)n_req * k_max > 0 && (theta == nullptr || q_draft == nullptr || conf == nullptr))
        return SV_ERR_NULL;
    const hipError_t e = sv::launch_calibrate_predict(theta, q_draft, q_entropy, q_max, n_req,
                                                      k_max, conf, as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

sv_status sv_philox_uniforms(uint64_t seed, uint64_t step, int32_t n_req, int32_t n_pos,
                             float* u, float* v, void* stream) {
    if (n_req < 0 || n_pos < 0) return SV_ERR_SHAPE;
    if ((int64_t)n_req * n_pos > 0 && (u == nullptr || v == nullptr)) return SV_ERR_NULL;
    const hipError_t e = sv::launch_philox_uniforms(seed, step, n_req, n_pos, u, v,
                                                    as_stream(stream));
    return sv::finish_launch(e, as_stream(stream));
}

}  // extern "C"
