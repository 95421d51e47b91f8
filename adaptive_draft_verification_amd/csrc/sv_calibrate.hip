// Acceptance statistics and online calibration of the per-position acceptance
// estimates (gfx950).
//
// FOS blog "추측 디코딩과 vLLM 적응형 검증": section "켜는 방법과 제약" (for
// model-based drafters without a confidence head, a small logistic model
// predicts acceptance from the draft's logits and is recalibrated while
// serving from the actual verification results), the measurement checklist
// (per-position acceptance rate, mean acceptance length) and section "평균
// 수락 길이".
//
// A request r with b_r kept drafts and L_r accepted verified positions
// 0 .. min(L_r, b_r - 1): those below L_r were accepted, position L_r (when
// L_r < b_r) rejected.  Requests whose outcome is not a verify result
// (L_r < 0 after a fault, or outside 0 <= L_r <= b_r <= k_max) are skipped.
// The model: c_j = sigmoid(alpha_j + beta * x), x = log2 q(d_j) clamped to
// [-64, 0] (the draft's own log-probability of its token).
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr float kXMin = -64.0f;

__device__ __forceinline__ bool outcome(const int32_t* accepted, const int32_t* cu_rows, int r,
                                        int k_max, int* b, int* L) {
    *b = cu_rows[r + 1] - cu_rows[r] - 1;
    *L = accepted[r];
    return *L >= 0 && *L <= *b && *b <= k_max;
}

__device__ __forceinline__ float feature(float q) {
    if (!(q > 0.0f)) return kXMin;  // 0, negative or NaN
    return fminf(0.0f, fmaxf(kXMin, log2f(q)));
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

// Block-wide sum of one float per thread in a fixed order (DPP within each
// wave, then the wave totals in wave order).  Every thread gets the sum.
__device__ float block_sum(float v, float* red) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const float w = wave_sum_dpp(v, lane);
    if (lane == 0) red[wave] = w;
    __syncthreads();
    float t = red[0];
    for (int i = 1; i < kWaves; ++i) t += red[i];
    __syncthreads();
    return t;
}

__global__ __launch_bounds__(kThreads) void accept_stats_kernel(
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ cu_rows, int n_req,
    int k_max, unsigned long long* attempted, unsigned long long* accepted_at,
    unsigned long long* totals) {
    __shared__ unsigned int att_s[SV_MAX_DRAFT], acc_s[SV_MAX_DRAFT];
    __shared__ unsigned long long req_s, emit_s;
    const int tid = threadIdx.x;
    if (tid < SV_MAX_DRAFT) {
        att_s[tid] = 0u;
        acc_s[tid] = 0u;
    }
    if (tid == 0) {
        req_s = 0ull;
        emit_s = 0ull;
    }
    __syncthreads();
    unsigned long long my_req = 0, my_emit = 0;
    for (int r = tid; r < n_req; r += kThreads) {
        int b, L;
        if (!outcome(accepted, cu_rows, r, k_max, &b, &L)) continue;
        ++my_req;
        my_emit += (unsigned long long)(L + 1);
        const int last = L < b - 1 ? L : b - 1;  // verified positions 0 .. last
        for (int j = 0; j <= last; ++j) {
            atomicAdd(&att_s[j], 1u);
            if (j < L) atomicAdd(&acc_s[j], 1u);
        }
    }
    if (my_req) atomicAdd(&req_s, my_req);
    if (my_emit) atomicAdd(&emit_s, my_emit);
    __syncthreads();
    if (tid < k_max) {
        if (att_s[tid]) atomicAdd(&attempted[tid], (unsigned long long)att_s[tid]);
        if (acc_s[tid]) atomicAdd(&accepted_at[tid], (unsigned long long)acc_s[tid]);
    }
    if (tid == 0) {
        atomicAdd(&totals[0], req_s);
        atomicAdd(&totals[1], emit_s);
    }
}

// One gradient step on the mean log-loss of the verified positions:
// theta <- theta - lr * grad / N.  One workgroup; each gradient component is
// a fixed-order block sum (deterministic).
__global__ __launch_bounds__(kThreads) void calibrate_update_kernel(
    float* theta, const float* __restrict__ q_draft, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ cu_rows, int n_req, int k_max, float lr, int32_t* count_out) {
    __shared__ float th[SV_MAX_DRAFT + 1];
    __shared__ float red[kWaves];
    __shared__ float grad[SV_MAX_DRAFT + 1];
    __shared__ int cnt_s;
    const int tid = threadIdx.x;
    if (tid <= k_max) th[tid] = theta[tid];
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    const float beta = th[k_max];
    float g_beta = 0.0f;
    int my_cnt = 0;
    for (int j = 0; j < k_max; ++j) {
        // this thread's requests, in order, that verified position j
        float g = 0.0f;
        for (int r = tid; r < n_req; r += kThreads) {
            int b, L;
            if (!outcome(accepted, cu_rows, r, k_max, &b, &L)) continue;
            if (j > L || j >= b) continue;
            const float x = feature(q_draft[(int64_t)r * k_max + j]);
            const float err = sigmoid(th[j] + beta * x) - (j < L ? 1.0f : 0.0f);
            g += err;
            g_beta += err * x;
            ++my_cnt;
        }
        g = block_sum(g, red);
        if (tid == 0) grad[j] = g;
    }
    g_beta = block_sum(g_beta, red);
    if (my_cnt) atomicAdd(&cnt_s, my_cnt);
    __syncthreads();
    const int count = cnt_s;
    if (tid <= k_max && count > 0) {
        const float g = tid < k_max ? grad[tid] : g_beta;
        theta[tid] = th[tid] - lr * (g / (float)count);
    }
    if (tid == 0 && count_out != nullptr) count_out[0] = count;
}

__global__ void calibrate_predict_kernel(const float* __restrict__ theta,
                                         const float* __restrict__ q_draft, int n_req, int k_max,
                                         float* __restrict__ conf) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n_req * k_max) return;
    const int j = (int)(i % k_max);
    conf[i] = sigmoid(theta[j] + theta[k_max] * feature(q_draft[i]));
}

}  // namespace

hipError_t launch_accept_stats(const int32_t* accepted, const int32_t* cu_rows, int n_req,
                               int k_max, uint64_t* attempted, uint64_t* accepted_at,
                               uint64_t* totals, hipStream_t stream) {
    hipLaunchKernelGGL(accept_stats_kernel, dim3(1), dim3(kThreads), 0, stream, accepted,
                       cu_rows, n_req, k_max, reinterpret_cast<unsigned long long*>(attempted),
                       reinterpret_cast<unsigned long long*>(accepted_at),
                       reinterpret_cast<unsigned long long*>(totals));
    return hipGetLastError();
}

hipError_t launch_calibrate_update(float* theta, const float* q_draft, const int32_t* accepted,
                                   const int32_t* cu_rows, int n_req, int k_max, float lr,
                                   int32_t* count_out, hipStream_t stream) {
    hipLaunchKernelGGL(calibrate_update_kernel, dim3(1), dim3(kThreads), 0, stream, theta,
                       q_draft, accepted, cu_rows, n_req, k_max, lr, count_out);
    return hipGetLastError();
}

hipError_t launch_calibrate_predict(const float* theta, const float* q_draft, int n_req,
                                    int k_max, float* conf, hipStream_t stream) {
    const int64_t n = (int64_t)n_req * k_max;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(calibrate_predict_kernel, dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, stream, theta, q_draft, n_req, k_max, conf);
    return hipGetLastError();
}

}  // namespace sv
