// Adaptive verification budget on one workgroup (gfx950).
//
// FOS blog "추측 디코딩과 vLLM 적응형 검증", section "적응형 검증 > 동작",
// steps 1-3; agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive
// Verification)", section "DSpark 신뢰도 스케줄링 메커니즘" (Global Top-B
// Selection, Budget Calculation).
//
// At most SV_MAX_BUDGET_SLOTS draft slots: the whole problem lives in LDS.
//   1. survival products per request (one thread walks one request's
//      positions in order, fp32 round-to-nearest, no contraction);
//   2. 64-bit keys (~survival bits << 32 | slot id) sorted ascending by a
//      bitonic network in LDS: descending survival, then request, then
//      position — a total order, so the sort is deterministic;
//   3. fixed-point prefix sums sum floor(s * 2^40) in uint64 (exact, order
//      free), fp64 scores (n_bonus + S * 2^-40) / cost[t_base + B], and the
//      first maximiser;
//   4. kept counts by integer LDS atomics over the first B ranks.
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kBudgetThreads = 1024;
constexpr int kBudgetWaves = kBudgetThreads / kWave;

__device__ __forceinline__ float clamp_confidence(float c) {
    // NaN and negatives -> 0, above 1 -> 1 (the test below is false for NaN).
    if (!(c >= 0.0f)) return 0.0f;
    return c > 1.0f ? 1.0f : c;
}

// Block-wide exclusive scan of one uint64 per thread; returns the exclusive
// prefix and writes the block total to *total.
__device__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* wave_tot, uint64_t* total) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint64_t incl = wave_incl_scan<uint64_t>(v, lane);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint64_t t = lane < kBudgetWaves ? wave_tot[lane] : 0ull;
        t = wave_incl_scan<uint64_t>(t, lane);
        if (lane < kBudgetWaves) wave_tot[lane] = t;  // inclusive totals per wave
    }
    __syncthreads();
    const uint64_t before_wave = wave == 0 ? 0ull : wave_tot[wave - 1];
    *total = wave_tot[kBudgetWaves - 1];
    return before_wave + incl - v;
}

__global__ __launch_bounds__(kBudgetThreads) void budget_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ draft_len, int n_req, int k_max,
    const float* __restrict__ cost, int t_base, int n_bonus, int32_t* __restrict__ kept,
    int32_t* __restrict__ budget, float* __restrict__ survival, int32_t* dev_error) {
    __shared__ uint64_t keys[SV_MAX_BUDGET_SLOTS];
    __shared__ int32_t kept_s[SV_MAX_BUDGET_SLOTS];
    __shared__ uint64_t wave_tot[kBudgetWaves];
    __shared__ int32_t total_slots_s;
    __shared__ int32_t err_s;
    __shared__ double best_score_s[kBudgetWaves];
    __shared__ int32_t best_b_s[kBudgetWaves];

    const int tid = threadIdx.x;
    const int n_slots = n_req * k_max;
    int npow2 = 1;
    while (npow2 < n_slots) npow2 <<= 1;

    if (tid == 0) {
        total_slots_s = 0;
        err_s = 0;
    }
    __syncthreads();

    // 1. survival and keys
    int my_err = 0;
    int my_total = 0;
    for (int r = tid; r < n_req; r += kBudgetThreads) {
        int K = draft_len[r];
        if (K < 0 || K > k_max) {
            my_err |= SV_DEV_BAD_DRAFT_LEN;
            K = K < 0 ? 0 : k_max;
        }
        my_total += K;
        kept_s[r] = 0;
        float s = 1.0f;
        for (int j = 0; j < k_max; ++j) {
            const int slot = r * k_max + j;
            if (j < K) {
                s = __fmul_rn(s, clamp_confidence(conf[slot]));
                keys[slot] = ((uint64_t)(0xffffffffu - __float_as_uint(s)) << 32) | (uint32_t)slot;
                if (survival) survival[slot] = s;
            } else {
                keys[slot] = ~0ull;
                if (survival) survival[slot] = 0.0f;
            }
        }
    }
    for (int i = n_slots + tid; i < npow2; i += kBudgetThreads) keys[i] = ~0ull;
    if (my_total) atomicAdd(&total_slots_s, my_total);
    if (my_err) atomicOr(&err_s, my_err);
    __syncthreads();

    // 2. bitonic sort, ascending
    for (int k = 2; k <= npow2; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            for (int i = tid; i < (npow2 >> 1); i += kBudgetThreads) {
                const int lo = 2 * i - (i & (j - 1));
                const int hi = lo + j;
                const bool ascending = (lo & k) == 0;
                const uint64_t x = keys[lo], y = keys[hi];
                if ((x > y) == ascending) {
                    keys[lo] = y;
                    keys[hi] = x;
                }
            }
            __syncthreads();
        }
    }

    // 3. fixed-point prefix sums over ranks, scores, first maximiser.
    // Thread t owns the contiguous ranks [t*per, (t+1)*per).
    const int total = total_slots_s;
    const int per = (npow2 + kBudgetThreads - 1) / kBudgetThreads;
    const int first = tid * per;
    uint64_t local = 0;
    for (int q = 0; q < per; ++q) {
        const int rank = first + q;
        if (rank < total) {
            const float sv = __uint_as_float(0xffffffffu - (uint32_t)(keys[rank] >> 32));
            local += (uint64_t)(sv * 0x1p40f);  // exact scaling, truncation = floor
        }
    }
    uint64_t block_total;
    uint64_t run = block_excl_scan_u64(local, wave_tot, &block_total);

    double best = -__builtin_inf();
    int best_b = 0x7fffffff;
    int cost_err = 0;
    if (tid == 0) {  // B = 0
        const float c0 = cost[t_base];
        if (c0 > 0.0f && is_finite_bits(c0)) {
            best = (double)n_bonus / (double)c0;
        } else {
            cost_err = SV_DEV_BAD_COST;
        }
        best_b = 0;
    }
    for (int q = 0; q < per; ++q) {
        const int rank = first + q;
        if (rank < total) {
            const float sv = __uint_as_float(0xffffffffu - (uint32_t)(keys[rank] >> 32));
            run += (uint64_t)(sv * 0x1p40f);
            const int b = rank + 1;
            const float cb = cost[t_base + b];
            double sc = -__builtin_inf();
            if (cb > 0.0f && is_finite_bits(cb)) {
                sc = __dadd_rn((double)n_bonus, __dmul_rn((double)run, 0x1p-40));
                sc = __ddiv_rn(sc, (double)cb);
            } else {
                cost_err = SV_DEV_BAD_COST;
            }
            if (sc > best || (sc == best && b < best_b)) {
                best = sc;
                best_b = b;
            }
        }
    }
    // block argmax: larger score, then smaller B
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const double ob = __shfl_xor(best, o);
        const int obb = __shfl_xor(best_b, o);
        if (ob > best || (ob == best && obb < best_b)) {
            best = ob;
            best_b = obb;
        }
    }
    if (cost_err) atomicOr(&err_s, cost_err);
    if (lane == 0) {
        best_score_s[wave] = best;
        best_b_s[wave] = best_b;
    }
    __syncthreads();
    if (wave == 0) {
        best = lane < kBudgetWaves ? best_score_s[lane] : -__builtin_inf();
        best_b = lane < kBudgetWaves ? best_b_s[lane] : 0x7fffffff;
#pragma unroll
        for (int o = kWave / 2; o > 0; o >>= 1) {
            const double ob = __shfl_xor(best, o);
            const int obb = __shfl_xor(best_b, o);
            if (ob > best || (ob == best && obb < best_b)) {
                best = ob;
                best_b = obb;
            }
        }
        if (lane == 0) best_b_s[0] = best_b;
    }
    __syncthreads();
    const int B = best_b_s[0];

    // 4. kept counts
    for (int rank = tid; rank < B; rank += kBudgetThreads) {
        const int slot = (int)(uint32_t)keys[rank];
        atomicAdd(&kept_s[slot / k_max], 1);
    }
    __syncthreads();
    for (int r = tid; r < n_req; r += kBudgetThreads) kept[r] = kept_s[r];
    if (tid == 0) {
        budget[0] = B;
        raise_error(dev_error, err_s);
    }
}

}  // namespace

hipError_t launch_budget(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                         const float* cost, int t_base, int n_bonus, int32_t* kept,
                         int32_t* budget, float* survival, int32_t* dev_error,
                         hipStream_t stream) {
    hipLaunchKernelGGL(budget_kernel, dim3(1), dim3(kBudgetThreads), 0, stream, conf, draft_len,
                       n_req, k_max, cost, t_base, n_bonus, kept, budget, survival, dev_error);
    return hipGetLastError();
}

}  // namespace sv
