// Adaptive verification budget on one workgroup (gfx950).
//
// FOS blog "추측 디코딩과 vLLM 적응형 검증", section "적응형 검증 > 동작",
// steps 1-3; agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive
// Verification)", section "DSpark 신뢰도 스케줄링 메커니즘" (Global Top-B
// Selection, Budget Calculation).
//
// At most SV_MAX_BUDGET_SLOTS draft slots, so the whole problem lives on one
// CU:
//   0. every global input is requested up front (confidences, draft lengths,
//      and the cost entries of this thread's ranks) so their latencies
//      overlap;
//   1. one thread per request forms the survival products in position order
//      (fp32 round-to-nearest, no contraction) and writes that request's
//      keys — (bits that fall as survival rises) << 32 | slot id, unique —
//      as one ascending run: survival never rises with position, so every
//      request's run is already sorted;
//   2. a merge tree joins the runs pairwise, ceil(log2 n) levels, two LDS
//      buffers in turn: each key lands at (its index in its run) + (number of
//      keys below it in the partner run), found by one binary search — exact
//      and order free because keys are unique.  The order is survival
//      descending, then request, then position;
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
// Keys of slots past a request's draft length: above every real key (whose
// high word is at most 0x7fffffff), unique through the slot id.
constexpr uint64_t kPadKey = 0x8000000000000000ull;

__device__ __forceinline__ float clamp_confidence(float c) {
    // NaN, negatives and -0 -> +0; above 1 -> 1.
    if (!(c > 0.0f)) return 0.0f;
    return c > 1.0f ? 1.0f : c;
}

// Survival s in [0, 1] -> high key word that grows as s falls (s >= +0).
__device__ __forceinline__ uint64_t survival_key(float s, int slot) {
    return ((uint64_t)(0x7fffffffu - __float_as_uint(s)) << 32) | (uint32_t)slot;
}

__device__ __forceinline__ float key_survival(uint64_t key) {
    return __uint_as_float(0x7fffffffu - (uint32_t)(key >> 32));
}

// Number of keys in seg[0 .. len) below `key` (seg ascending, keys unique).
__device__ __forceinline__ int lower_bound(const uint64_t* seg, int len, uint64_t key) {
    int lo = 0;
    while (len > 0) {
        const int half = len >> 1;
        if (seg[lo + half] < key) {
            lo += half + 1;
            len -= half + 1;
        } else {
            len = half;
        }
    }
    return lo;
}

// Block-wide exclusive scan of one uint64 per thread.
__device__ uint64_t block_excl_scan_u64(uint64_t v, uint64_t* wave_tot) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    const uint64_t incl = wave_incl_scan<uint64_t>(v, lane);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    if (wave == 0) {
        uint64_t t = lane < kBudgetWaves ? wave_tot[lane] : 0ull;
        t = wave_incl_scan<uint64_t>(t, lane);
        if (lane < kBudgetWaves) wave_tot[lane] = t;
    }
    __syncthreads();
    return (wave == 0 ? 0ull : wave_tot[wave - 1]) + incl - v;
}

// E = ranks per thread (contiguous), n_req * k_max <= 1024 * E.
template <int E>
__global__ __launch_bounds__(kBudgetThreads) void budget_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ draft_len, int n_req, int k_max,
    const float* __restrict__ cost, int t_base, int n_bonus, int32_t* __restrict__ kept,
    int32_t* __restrict__ budget, float* __restrict__ survival, int32_t* dev_error) {
    __shared__ uint64_t buf[2][SV_MAX_BUDGET_SLOTS];
    __shared__ uint64_t wave_tot[kBudgetWaves];
    __shared__ double best_score_s[kBudgetWaves];
    __shared__ int32_t best_b_s[kBudgetWaves];
    __shared__ int32_t total_slots_s, err_s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n_slots = n_req * k_max;
    const int first_rank = tid * E;
    float* conf_s = reinterpret_cast<float*>(buf[1]);  // staging, dead before buf[1] is used

    // 0. requests for every global input this thread will need
    float cst[E];
#pragma unroll
    for (int q = 0; q < E; ++q) {
        const int rank = first_rank + q;
        cst[q] = rank < n_slots ? cost[t_base + rank + 1] : 1.0f;
    }
    const float cost0 = cost[t_base];
    constexpr int kMaxReqPerThread = SV_MAX_BUDGET_SLOTS / kBudgetThreads;
    int dl[kMaxReqPerThread];
#pragma unroll
    for (int i = 0; i < kMaxReqPerThread; ++i) {
        const int r = tid + i * kBudgetThreads;
        dl[i] = r < n_req ? draft_len[r] : 0;
    }
    for (int i = tid; i < n_slots; i += kBudgetThreads) conf_s[i] = conf[i];
    if (tid == 0) {
        total_slots_s = 0;
        err_s = 0;
    }
    __syncthreads();

    // 1. survival products and the per-request sorted runs of keys (buf[0])
    int my_err = 0, my_total = 0;
#pragma unroll
    for (int i = 0; i < kMaxReqPerThread; ++i) {
        const int r = tid + i * kBudgetThreads;
        if (r >= n_req) break;
        int K = dl[i];
        if (K < 0 || K > k_max) {
            my_err |= SV_DEV_BAD_DRAFT_LEN;
            K = K < 0 ? 0 : k_max;
        }
        my_total += K;
        float s = 1.0f;
        for (int j = 0; j < k_max; ++j) {
            const int slot = r * k_max + j;
            if (j < K) {
                s = __fmul_rn(s, clamp_confidence(conf_s[slot]));
                buf[0][slot] = survival_key(s, slot);
                if (survival != nullptr) survival[slot] = s;
            } else {
                buf[0][slot] = kPadKey | (uint32_t)slot;
                if (survival != nullptr) survival[slot] = 0.0f;
            }
        }
    }
    if (my_total) atomicAdd(&total_slots_s, my_total);
    // cost entries are checked here so their loads complete under this phase
    int cost_bad = 0;
#pragma unroll
    for (int q = 0; q < E; ++q) cost_bad |= (cst[q] > 0.0f && is_finite_bits(cst[q])) ? 0 : 1 << q;
    const bool cost0_bad = !(cost0 > 0.0f && is_finite_bits(cost0));
    if (my_err) atomicOr(&err_s, my_err);
    __syncthreads();

    // 2. merge tree over runs of k_max << level slots
    int src = 0;
    for (int run = k_max; run < n_slots; run <<= 1) {
        const uint64_t* in = buf[src];
        uint64_t* out = buf[src ^ 1];
#pragma unroll
        for (int q = 0; q < E; ++q) {
            const int p = first_rank + q;
            if (p < n_slots) {
                const uint64_t key = in[p];
                const int r_idx = p / run;
                const int pair_base = (r_idx & ~1) * run;
                const int partner = (r_idx ^ 1) * run;
                int pos = p - pair_base;  // own index in run, plus left run if right
                if (partner < n_slots) {
                    const int plen = min(run, n_slots - partner);
                    pos = (p - r_idx * run) + lower_bound(in + partner, plen, key);
                }
                out[pair_base + pos] = key;
            }
        }
        src ^= 1;
        __syncthreads();
    }
    const uint64_t* sorted = buf[src];
    int32_t* kept_s = reinterpret_cast<int32_t*>(buf[src ^ 1]);
    for (int r = tid; r < n_req; r += kBudgetThreads) kept_s[r] = 0;

    // 3. fixed-point prefix sums over ranks, scores, first maximiser
    const int total = total_slots_s;
    uint64_t fx[E];
    uint64_t local = 0;
#pragma unroll
    for (int q = 0; q < E; ++q) {
        fx[q] = 0;
        if (first_rank + q < total) fx[q] = (uint64_t)(key_survival(sorted[first_rank + q]) * 0x1p40f);
        local += fx[q];  // exact scaling; truncation = floor
    }
    uint64_t run_sum = block_excl_scan_u64(local, wave_tot);

    double best = -__builtin_inf();
    int best_b = 0x7fffffff;
    int cost_err = 0;
    if (tid == 0) {  // B = 0
        if (!cost0_bad)
            best = (double)n_bonus / (double)cost0;
        else
            cost_err = SV_DEV_BAD_COST;
        best_b = 0;
    }
#pragma unroll
    for (int q = 0; q < E; ++q) {
        const int rank = first_rank + q;
        if (rank < total) {
            run_sum += fx[q];
            const int b = rank + 1;
            double sc = -__builtin_inf();
            if (!((cost_bad >> q) & 1)) {
                sc = __dadd_rn((double)n_bonus, __dmul_rn((double)run_sum, 0x1p-40));
                sc = __ddiv_rn(sc, (double)cst[q]);
            } else {
                cost_err = SV_DEV_BAD_COST;
            }
            if (sc > best || (sc == best && b < best_b)) {
                best = sc;
                best_b = b;
            }
        }
    }
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
#pragma unroll
    for (int q = 0; q < E; ++q)
        if (first_rank + q < B) atomicAdd(&kept_s[(int)(uint32_t)sorted[first_rank + q] / k_max], 1);
    __syncthreads();
    for (int r = tid; r < n_req; r += kBudgetThreads) kept[r] = kept_s[r];
    if (tid == 0) {
        budget[0] = B;
        raise_error(dev_error, err_s);
    }
}

template <int E>
void launch_e(const float* conf, const int32_t* draft_len, int n_req, int k_max,
              const float* cost, int t_base, int n_bonus, int32_t* kept, int32_t* budget,
              float* survival, int32_t* dev_error, hipStream_t stream) {
    hipLaunchKernelGGL(budget_kernel<E>, dim3(1), dim3(kBudgetThreads), 0, stream, conf,
                       draft_len, n_req, k_max, cost, t_base, n_bonus, kept, budget, survival,
                       dev_error);
}

}  // namespace

hipError_t launch_budget(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                         const float* cost, int t_base, int n_bonus, int32_t* kept,
                         int32_t* budget, float* survival, int32_t* dev_error,
                         hipStream_t stream) {
    const int n_slots = n_req * k_max;
    if (n_slots <= kBudgetThreads)
        launch_e<1>(conf, draft_len, n_req, k_max, cost, t_base, n_bonus, kept, budget, survival,
                    dev_error, stream);
    else if (n_slots <= 2 * kBudgetThreads)
        launch_e<2>(conf, draft_len, n_req, k_max, cost, t_base, n_bonus, kept, budget, survival,
                    dev_error, stream);
    else if (n_slots <= 4 * kBudgetThreads)
        launch_e<4>(conf, draft_len, n_req, k_max, cost, t_base, n_bonus, kept, budget, survival,
                    dev_error, stream);
    else
        launch_e<8>(conf, draft_len, n_req, k_max, cost, t_base, n_bonus, kept, budget, survival,
                    dev_error, stream);
    return hipGetLastError();
}

}  // namespace sv
