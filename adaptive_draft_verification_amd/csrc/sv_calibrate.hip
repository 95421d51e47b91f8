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
// The model: c_j = sigmoid(alpha_j + beta_1 x_1 + beta_2 x_2 + beta_3 x_3) over
// three features of draft row j: x_1 = log2 q(d_j) clamped to [-64, 0] (the
// draft's own log-probability of its token), x_2 = the row's entropy in bits
// clamped to [0, 64], x_3 = its largest probability clamped to [0, 1]; a
// feature array left out (null) reads as 0.  theta = [alpha_0 ..
// alpha_{k_max-1}, beta_1, beta_2, beta_3].
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

constexpr int kFeat = 3;

struct Features {
    const float* q;    // q(d_j), [n, k_max]
    const float* ent;  // draft-row entropy in bits, [n, k_max] or null
    const float* pmax; // draft-row largest probability, [n, k_max] or null
};

__device__ __forceinline__ void features(const Features& f, int64_t i, float* x) {
    const float q = f.q[i];
    x[0] = q > 0.0f ? fminf(0.0f, fmaxf(kXMin, log2f(q))) : kXMin;  // 0, negative or NaN: floor
    const float h = f.ent ? f.ent[i] : 0.0f;
    x[1] = h > 0.0f ? fminf(64.0f, h) : 0.0f;
    const float m = f.pmax ? f.pmax[i] : 0.0f;
    x[2] = m > 0.0f ? fminf(1.0f, m) : 0.0f;
}

__device__ __forceinline__ float logit(const float* th, int j, int k_max, const float* x) {
    return th[j] + th[k_max] * x[0] + th[k_max + 1] * x[1] + th[k_max + 2] * x[2];
}

__device__ __forceinline__ float sigmoid(float z) { return 1.0f / (1.0f + expf(-z)); }

__global__ __launch_bounds__(kThreads) void accept_stats_kernel(
    const int32_t* __restrict__ accepted, const int32_t* __restrict__ cu_rows, int n_req,
    int k_max, unsigned long long* attempted, unsigned long long* accepted_at,
    unsigned long long* totals) {
    __shared__ unsigned int att_s[SV_MAX_DRAFT], acc_s[SV_MAX_DRAFT];
    __shared__ unsigned long long req_s, emit_s;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
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
    // whole waves step through the requests together, so that a ballot per
    // position counts a wave's 64 requests at once (one LDS add per wave)
    for (int base = tid - lane; base < n_req; base += kThreads) {
        const int r = base + lane;
        int b = 0, L = -1;
        const bool ok = r < n_req && outcome(accepted, cu_rows, r, k_max, &b, &L);
        const int last = !ok ? -1 : (L < b - 1 ? L : b - 1);  // verified positions 0 .. last
        if (ok) {
            ++my_req;
            my_emit += (unsigned long long)(L + 1);
        }
        for (int j = 0; j < k_max; ++j) {
            const uint64_t ver = __ballot(j <= last);
            if (ver == 0) break;  // positions only shrink from here (uniform)
            const uint64_t acc = __ballot(j <= last && j < L);
            if (lane == 0) {
                atomicAdd(&att_s[j], (unsigned int)__popcll(ver));
                if (acc) atomicAdd(&acc_s[j], (unsigned int)__popcll(acc));
            }
        }
    }
    // one LDS add per wave for the totals as well
    my_req = wave_sum_dpp(my_req, lane);
    my_emit = wave_sum_dpp(my_emit, lane);
    if (lane == 0 && my_req) {
        atomicAdd(&req_s, my_req);
        atomicAdd(&emit_s, my_emit);
    }
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
// theta <- theta - lr * grad / N.  One workgroup, one pass: wave w takes the
// positions j = w, w + 16, ...; its lanes walk the requests r = lane,
// lane + 64, ... in order, so each alpha component is a fixed-order sum (the
// lanes' partial sums, then a DPP wave sum) and each beta component the waves'
// sums added in wave order: deterministic, with no barrier per position.
__global__ __launch_bounds__(kThreads) void calibrate_update_kernel(
    float* theta, Features f, const int32_t* __restrict__ accepted,
    const int32_t* __restrict__ cu_rows, int n_req, int k_max, float lr, int32_t* count_out) {
    __shared__ float th[SV_MAX_DRAFT + kFeat];
    __shared__ float grad[SV_MAX_DRAFT + kFeat];
    __shared__ float beta_w[kWaves][kFeat];
    __shared__ int cnt_s;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    if (tid < k_max + kFeat) th[tid] = theta[tid];
    if (tid == 0) cnt_s = 0;
    __syncthreads();
    float g_beta[kFeat] = {0.0f, 0.0f, 0.0f};
    int my_cnt = 0;
    for (int j = wave; j < k_max; j += kWaves) {
        float g = 0.0f;
        for (int r = lane; r < n_req; r += kWave) {
            int b, L;
            if (!outcome(accepted, cu_rows, r, k_max, &b, &L)) continue;
            if (j > L || j >= b) continue;  // position j not verified for r
            float x[kFeat];
            features(f, (int64_t)r * k_max + j, x);
            const float err = sigmoid(logit(th, j, k_max, x)) - (j < L ? 1.0f : 0.0f);
            g += err;
#pragma unroll
            for (int i = 0; i < kFeat; ++i) g_beta[i] += err * x[i];
            ++my_cnt;
        }
        g = wave_sum_dpp(g, lane);
        if (lane == 0) grad[j] = g;
    }
#pragma unroll
    for (int i = 0; i < kFeat; ++i) {
        const float gw = wave_sum_dpp(g_beta[i], lane);
        if (lane == 0) beta_w[wave][i] = gw;
    }
    my_cnt = wave_sum_dpp(my_cnt, lane);  // one LDS add per wave
    if (lane == 0 && my_cnt) atomicAdd(&cnt_s, my_cnt);
    __syncthreads();
    if (tid < kFeat) {
        float t = beta_w[0][tid];
        for (int w = 1; w < kWaves; ++w) t += beta_w[w][tid];
        grad[k_max + tid] = t;
    }
    __syncthreads();
    const int count = cnt_s;
    if (tid < k_max + kFeat && count > 0) theta[tid] = th[tid] - lr * (grad[tid] / (float)count);
    if (tid == 0 && count_out != nullptr) count_out[0] = count;
}

__global__ void calibrate_predict_kernel(const float* __restrict__ theta, Features f, int n_req,
                                         int k_max, float* __restrict__ conf) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n_req * k_max) return;
    float x[kFeat];
    features(f, i, x);
    conf[i] = sigmoid(logit(theta, (int)(i % k_max), k_max, x));
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

hipError_t launch_calibrate_update(float* theta, const float* q_draft, const float* q_entropy,
                                   const float* q_max, const int32_t* accepted,
                                   const int32_t* cu_rows, int n_req, int k_max, float lr,
                                   int32_t* count_out, hipStream_t stream) {
    const Features f{q_draft, q_entropy, q_max};
    hipLaunchKernelGGL(calibrate_update_kernel, dim3(1), dim3(kThreads), 0, stream, theta, f,
                       accepted, cu_rows, n_req, k_max, lr, count_out);
    return hipGetLastError();
}

hipError_t launch_calibrate_predict(const float* theta, const float* q_draft,
                                    const float* q_entropy, const float* q_max, int n_req,
                                    int k_max, float* conf, hipStream_t stream) {
    const int64_t n = (int64_t)n_req * k_max;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    const Features f{q_draft, q_entropy, q_max};
    hipLaunchKernelGGL(calibrate_predict_kernel, dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, stream, theta, f, n_req, k_max, conf);
    return hipGetLastError();
}

}  // namespace sv
