// Adaptive verification budget (gfx950).
//
// FOS blog "추측 디코딩과 vLLM 적응형 검증", section "적응형 검증 > 동작",
// steps 1-3; agentlens "vLLM DSpark을 활용한 적응형 검증(Adaptive
// Verification)", section "DSpark 신뢰도 스케줄링 메커니즘" (Global Top-B
// Selection, Budget Calculation).
//
// Every draft slot gets a unique 64-bit key, (bits that fall as survival
// rises) << 32 | slot id, so that ascending keys are the global order —
// survival descending, then request, then position.  A slot's place in that
// order is the number of keys below its own, which the GPU counts in
// parallel instead of sorting:
//
//   rank kernel — one 1024-thread workgroup per 16 query slots.  Each
//     workgroup stages every confidence in LDS with coalesced loads, forms
//     every survival product (one thread per request, position order, fp32
//     round-to-nearest, no contraction — identical bits in every
//     workgroup) and keeps the keys in LDS.  Each wave then ranks one query
//     slot: every lane holds one key of each 64-key chunk of the batch, one
//     compare per chunk, and the population count of the ballot adds 64
//     comparisons at once.  It writes each query's rank and places its
//     survival at that rank in the workspace.
//   finish kernel — one workgroup (DPP wave scans): the fixed-point prefix sums
//     sum floor(s * 2^40) over the rank-ordered survivals (exact uint64,
//     order free), the fp64 scores (n_bonus + S * 2^-40) / cost[t_base + B],
//     the first maximiser B and the kept counts #{j : rank(r, j) < B}.
//
// Workspace: [0] total real slots (int32), then ranks [n_slots] int32 and the
// rank-ordered survivals [n_slots] fp32.  Every word the finish kernel reads
// is written by the rank kernel of the same call, so it needs no clearing.
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;                        // 16
constexpr int kQueries = kWaves;                                // query slots per rank workgroup
// conf rows padded to an odd stride: n_req * (k_max | 1) floats, largest at
// k_max = 2 (4096 requests x 3)
constexpr int kConfLds = SV_MAX_BUDGET_SLOTS + SV_MAX_BUDGET_SLOTS / 2;
constexpr int kPerThread = SV_MAX_BUDGET_SLOTS / kThreads;      // 8
constexpr size_t kHeaderBytes = 16;

__device__ __forceinline__ float clamp_confidence(float c) {
    // NaN, negatives and -0 -> +0; above 1 -> 1.
    if (!(c > 0.0f)) return 0.0f;
    return c > 1.0f ? 1.0f : c;
}

// Survival s in [0, 1] -> key whose high word grows as s falls.
__device__ __forceinline__ uint64_t survival_key(float s, int slot) {
    return ((uint64_t)(0x7fffffffu - __float_as_uint(s)) << 32) | (uint32_t)slot;
}

__device__ __forceinline__ float key_survival(uint64_t key) {
    return __uint_as_float(0x7fffffffu - (uint32_t)(key >> 32));
}

constexpr uint64_t kNoSlot = ~0ull;  // past draft_len: after every real key

__device__ __forceinline__ int clamp_len(int K, int k_max) { return K < 0 ? 0 : (K > k_max ? k_max : K); }

struct BudgetWs {
    int32_t* total;
    int32_t* rank;
    float* sorted;
};

__device__ __forceinline__ BudgetWs budget_ws(void* ws, int n_slots) {
    char* base = static_cast<char*>(ws);
    BudgetWs w;
    w.total = reinterpret_cast<int32_t*>(base);
    w.rank = reinterpret_cast<int32_t*>(base + kHeaderBytes);
    w.sorted = reinterpret_cast<float*>(base + kHeaderBytes + (size_t)n_slots * sizeof(int32_t));
    return w;
}

__global__ __launch_bounds__(kThreads) void rank_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ draft_len, int n_req, int k_max,
    float* __restrict__ survival, int32_t* dev_error, void* ws) {
    // confidences at r * kp + j with an odd row stride kp (conflict-free LDS
    // reads when lanes walk consecutive requests); keys transposed, j * n_req + r
    __shared__ float conf_s[kConfLds];
    __shared__ uint64_t keys[SV_MAX_BUDGET_SLOTS];
    __shared__ int32_t total_s, err_s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n_slots = n_req * k_max;
    const int kp = k_max | 1;
    const bool lead = blockIdx.x == 0;  // writes survival, total and the error bits
    const BudgetWs w = budget_ws(ws, n_slots);

    // every global input requested at once: confidences (coalesced) and the
    // draft lengths of the requests this thread will chain
    float c[kPerThread];
    int32_t dl[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int x = tid + q * kThreads;
        c[q] = x < n_slots ? conf[x] : 0.0f;
        dl[q] = x < n_req ? draft_len[x] : 0;
    }
    if (tid == 0) {
        total_s = 0;
        err_s = 0;
    }
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int x = tid + q * kThreads;
        if (x < n_slots) {
            const int r = x / k_max;
            conf_s[r * kp + (x - r * k_max)] = clamp_confidence(c[q]);
        }
    }
    __syncthreads();

    // survival products, one thread per request
    int my_total = 0, my_err = 0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int r = tid + q * kThreads;
        if (r < n_req) {
            const int K = clamp_len(dl[q], k_max);
            if (K != dl[q]) my_err |= SV_DEV_BAD_DRAFT_LEN;
            my_total += K;
            float s = 1.0f;
            // eight positions at a time: their confidences are read before the
            // products are chained, so the LDS reads overlap
            for (int j0 = 0; j0 < k_max; j0 += 8) {
                float cv[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) cv[u] = j0 + u < K ? conf_s[r * kp + j0 + u] : 1.0f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int j = j0 + u;
                    if (j >= k_max) break;
                    if (j < K) s = __fmul_rn(s, cv[u]);
                    keys[j * n_req + r] = j < K ? survival_key(s, r * k_max + j) : kNoSlot;
                }
            }
        }
    }
    if (lead) {
        // one LDS atomic per wave (contended per-thread LDS atomics serialise)
        my_total = wave_sum_dpp(my_total, lane);
        my_err = wave_or_int(my_err);
        if (lane == 0) {
            if (my_total) atomicAdd(&total_s, my_total);
            if (my_err) atomicOr(&err_s, my_err);
        }
    }
    __syncthreads();
    if (lead) {
        // after the last barrier, so that no barrier waits for these stores
        if (tid == 0) {
            w.total[0] = total_s;
            raise_error(dev_error, err_s);
        }
        if (survival != nullptr) {
#pragma unroll
            for (int q = 0; q < kPerThread; ++q) {
                const int x = tid + q * kThreads;
                if (x < n_slots) {
                    const int r = x / k_max;
                    const uint64_t key = keys[(x - r * k_max) * n_req + r];
                    survival[x] = key != kNoSlot ? key_survival(key) : 0.0f;
                }
            }
        }
    }

    // wave `wave` ranks one query slot: every lane holds one key of each
    // 64-key chunk, one compare per chunk, and the population count of the
    // ballot adds 64 comparisons at once (the key order in LDS is irrelevant)
    const int x = blockIdx.x * kQueries + wave;
    if (x >= n_slots) return;  // wave-uniform; no barrier follows
    const int xr = x / k_max;
    const uint64_t v = keys[(x - xr * k_max) * n_req + xr];  // same address in every lane
    const uint64_t qk = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)) << 32) |
                        __builtin_amdgcn_readfirstlane((uint32_t)v);
    int cnt = 0;
    int base = 0;
    for (; base + 4 * kWave <= n_slots; base += 4 * kWave) {
        uint64_t ref[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ref[u] = keys[base + u * kWave + lane];
#pragma unroll
        for (int u = 0; u < 4; ++u) cnt += __popcll(__ballot(ref[u] < qk));
    }
    for (; base < n_slots; base += kWave) {
        const int i = base + lane;
        const uint64_t ref = i < n_slots ? keys[i] : kNoSlot;
        cnt += __popcll(__ballot(ref < qk));
    }
    if (lane == 0) {
        w.rank[x] = cnt;
        if (qk != kNoSlot) w.sorted[cnt] = key_survival(qk);
    }
}

// The per-wave totals tot[0 .. kWaves) in LDS: the sum over the waves before
// `wave`, and (*all) over every wave.  Lane v reads tot[v] once and a DPP wave
// scan does the rest, instead of a chain of dependent LDS reads.
template <typename T>
__device__ __forceinline__ T waves_before(const T* tot, int wave, int lane, T* all) {
    const T x = lane < kWaves ? tot[lane] : T(0);
    const T incl = wave_incl_sum_dpp<T>(x, lane);
    *all = lane63(incl);
    return readlane_t(incl - x, wave);
}

// A wave's best (score, B): the larger score, then the smaller B.
struct Cand {
    double score;
    int32_t b;
    int32_t pad;
};

struct MaxOpD {
    __device__ __forceinline__ double operator()(double a, double b) const { return fmax(a, b); }
};

// kept[r] = #{j : rank(r, j) < B}.  A request's real slots rank in position
// order (survival never rises along a chain, ties go to the lower slot) and
// its slots past draft_len rank at `total` or later, never before B <= total,
// so the kept slots are a prefix: the request's count is written by the slot
// that ends it (in budget, its successor not), or by slot 0 when slot 0 is
// not in budget.  rk[q], rk1[q]: the ranks of slot tid + 1024 q and of the
// slot after it.  kept_s (LDS, or null) gets a copy; no barrier inside.
__device__ __forceinline__ void write_kept(const int32_t* rk, const int32_t* rk1, int per, int B,
                                           int n_req, int k_max, int32_t* __restrict__ kept,
                                           uint8_t* kept_s) {
    const int tid = threadIdx.x;
    const int n_slots = n_req * k_max;
    if (k_max == 0) {
        for (int r = tid; r < n_req; r += kThreads) {
            kept[r] = 0;
            if (kept_s != nullptr) kept_s[r] = 0;
        }
        return;
    }
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        if (q >= per) break;  // uniform
        const int x = tid + q * kThreads;
        if (x < n_slots) {
            const int r = x / k_max, j = x - r * k_max;
            const bool in = rk[q] < B;
            const bool next_in = j + 1 < k_max && rk1[q] < B;
            int k_in = -1;
            if (j == 0 && !in) k_in = 0;
            if (in && !next_in) k_in = j + 1;
            if (k_in >= 0) {
                kept[r] = k_in;
                if (kept_s != nullptr) kept_s[r] = (uint8_t)k_in;
            }
        }
    }
}

// ------------------------------------------------- packing in the same launch
// The varlen layout of sv_pack_varlen (agentlens page, section "기술적 구현
// 및 CUDA Graphs", item Graph Capture; section "설정 및 재현": capacity
// (k + 1) * n), written by the workgroup that has just counted the kept
// slots, from its LDS copy of them: one launch fewer on the step's path.
struct PackOut {
    const int32_t* last_token;    // [n]
    const int32_t* draft_tokens;  // [n, k_max]
    int32_t* cu_rows;             // [n + 1]
    int32_t* row_req;             // [n (k_max + 1)]
    int32_t* row_pos;
    int32_t* packed_tokens;
};

// Ids the packing will copy, loaded at the start of the kernel so that their
// latency hides under the budget's own work: the draft id of slot
// tid + 1024 q and the last token of request tid + 1024 q.
struct PackIds {
    int32_t dtok[kPerThread];
    int32_t ltok[kPerThread];
};

__device__ __forceinline__ void pack_prefetch(const PackOut& po, int n_req, int k_max,
                                              PackIds& ids) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int x = tid + q * kThreads;
        ids.dtok[q] = x < n_req * k_max ? po.draft_tokens[x] : -1;
        ids.ltok[q] = x < n_req ? po.last_token[x] : -1;
    }
}

// Called by every thread after write_kept and a barrier (kept_s complete in
// LDS).  cu_s: LDS, n_req + 1 entries; wave_tot: LDS, kWaves entries.
__device__ void pack_from_lds(const uint8_t* kept_s, int n_req, int k_max, const PackOut& po,
                              const PackIds& ids, int32_t* cu_s, int32_t* wave_tot) {
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    // rows per request (kept + 1): thread t sums requests [t per, t per + per)
    const int per = (n_req + kThreads - 1) / kThreads;
    const int first = tid * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (first + i < n_req) local += (int)kept_s[first + i] + 1;
    const int incl = wave_incl_sum_dpp(local, lane);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    int total = 0;
    int start = incl - local + waves_before(wave_tot, wave, lane, &total);
    for (int i = 0; i < per; ++i) {
        const int r = first + i;
        if (r < n_req) {
            cu_s[r] = start;
            po.cu_rows[r] = start;
            start += (int)kept_s[r] + 1;
        }
    }
    if (tid == 0) po.cu_rows[n_req] = total;
    __syncthreads();
    // row 0 of each request: its last token; row 1 + j: draft j, if kept
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int r = tid + q * kThreads;
        if (r < n_req) {
            const int row = cu_s[r];
            po.row_req[row] = r;
            po.row_pos[row] = 0;
            po.packed_tokens[row] = ids.ltok[q];
        }
        const int x = tid + q * kThreads;
        if (x < n_req * k_max) {
            const int rr = x / k_max, j = x - rr * k_max;
            if (j < (int)kept_s[rr]) {
                const int row = cu_s[rr] + 1 + j;
                po.row_req[row] = rr;
                po.row_pos[row] = j + 1;
                po.packed_tokens[row] = ids.dtok[q];
            }
        }
    }
    const int cap = n_req * (k_max + 1);
    for (int row = total + tid; row < cap; row += kThreads) {
        po.row_req[row] = -1;
        po.row_pos[row] = -1;
        po.packed_tokens[row] = -1;
    }
}

template <bool PACK>
__global__ __launch_bounds__(kThreads) void finish_kernel(
    int n_req, int k_max, const float* __restrict__ cost, int t_base, int n_bonus,
    int32_t* __restrict__ kept, int32_t* __restrict__ budget, int32_t* dev_error, void* ws,
    PackOut po) {
    __shared__ uint8_t kept_s[PACK ? SV_MAX_BUDGET_SLOTS : 1];
    __shared__ int32_t cu_s[PACK ? SV_MAX_BUDGET_SLOTS : 1];
    __shared__ int32_t pack_tot[kWaves];
    __shared__ uint64_t wave_tot[kWaves];
    __shared__ Cand wave_best[kWaves];
    __shared__ int32_t err_s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = tid / kWave;
    const int n_slots = n_req * k_max;
    const BudgetWs w = budget_ws(ws, n_slots);
    // this thread's ranks: [first, first + per), per = ceil(n_slots / 1024)
    const int per = (n_slots + kThreads - 1) / kThreads;
    const int first = tid * per;

    // every load first: rank-ordered survivals and cost entries of this
    // thread's ranks, the ranks of slots tid + 1024 q and of their successors,
    // the total
    float srt[kPerThread], cst[kPerThread];
    int32_t rk[kPerThread], rk1[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        srt[q] = 0.0f;
        cst[q] = 1.0f;
        rk[q] = 0;
        rk1[q] = 0;
        if (q >= per) continue;  // uniform: per = ceil(n_slots / 1024)
        const int rank = first + q;
        if (rank < n_slots) {
            srt[q] = w.sorted[rank];
            cst[q] = cost[t_base + rank + 1];
        }
        const int x = tid + q * kThreads;
        if (x < n_slots) rk[q] = w.rank[x];
        if (x + 1 < n_slots) rk1[q] = w.rank[x + 1];
    }
    const float cost0 = cost[t_base];
    const int total = n_slots > 0 ? w.total[0] : 0;
    if (tid == 0) err_s = 0;
    PackIds ids;
    if (PACK) pack_prefetch(po, n_req, k_max, ids);

    uint64_t fx[kPerThread];
    uint64_t local = 0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        // s * 2^40 is exact in fp32; the conversion truncates = floor
        fx[q] = (q < per && first + q < total) ? (uint64_t)(srt[q] * 0x1p40f) : 0ull;
        local += fx[q];
    }
    // block exclusive scan: DPP wave scan, then the totals of earlier waves
    const uint64_t incl = wave_incl_sum_dpp<uint64_t>(local, lane);
    if (lane == kWave - 1) wave_tot[wave] = incl;
    __syncthreads();
    uint64_t all_waves;  // unused here
    uint64_t run_sum = incl - local + waves_before(wave_tot, wave, lane, &all_waves);
    (void)all_waves;

    // this thread's best candidate; its B values rise with the thread and the
    // lane, so the first maximiser of the block is the lowest lane holding the
    // maximum score (strict > keeps a thread's smaller B on a tie)
    double bs = -__builtin_inf();
    int bb = 0x7fffffff;
    int cost_err = 0;
    if (tid == 0) {  // B = 0
        if (cost0 > 0.0f && is_finite_bits(cost0))
            bs = (double)n_bonus / (double)cost0;
        else
            cost_err = SV_DEV_BAD_COST;
        bb = 0;
    }
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        if (q >= per) break;  // uniform
        const int rank = first + q;
        if (rank < total) {
            run_sum += fx[q];
            if (cst[q] > 0.0f && is_finite_bits(cst[q])) {
                // run_sum < 2^53 and 2^-40 is a power of two: the product is exact
                const double sc = ((double)n_bonus + (double)run_sum * 0x1p-40) / (double)cst[q];
                if (sc > bs) {
                    bs = sc;
                    bb = rank + 1;
                }
            } else {
                cost_err = SV_DEV_BAD_COST;
            }
        }
    }
    {
        const double m = lane63(wave_scan_dpp(bs, lane, MaxOpD{}));
        const int wb = __builtin_amdgcn_readlane(bb, __builtin_ctzll(__ballot(bs == m)));
        if (cost_err) atomicOr(&err_s, cost_err);
        if (lane == 0) wave_best[wave] = Cand{m, wb, 0};
    }
    __syncthreads();
    // every wave reduces the 16 wave winners itself (waves in B order too): no
    // further barrier
    const double cs = lane < kWaves ? wave_best[lane].score : -__builtin_inf();
    const int cb = lane < kWaves ? wave_best[lane].b : 0x7fffffff;
    const double cm = lane63(wave_scan_dpp(cs, lane, MaxOpD{}));
    const int B = __builtin_amdgcn_readlane(cb, __builtin_ctzll(__ballot(cs == cm)));
    write_kept(rk, rk1, per, B, n_req, k_max, kept, PACK ? kept_s : nullptr);
    if (tid == 0) {
        budget[0] = B;
        raise_error(dev_error, err_s);
    }
    if (PACK) {
        __syncthreads();
        pack_from_lds(kept_s, n_req, k_max, po, ids, cu_s, pack_tot);
    }
}

// Allocation of a budget sized elsewhere (agentlens page, section "DSpark
// 신뢰도 스케줄링 메커니즘", item Execution Pipeline: B comes from the
// previous step's confidences, the slots from the current ones): the first
// min(max(B, 0), total) slots of the rank kernel's order.  One workgroup.
template <bool PACK>
__global__ __launch_bounds__(kThreads) void allocate_kernel(int n_req, int k_max,
                                                            const int32_t* __restrict__ budget_in,
                                                            int32_t* __restrict__ kept,
                                                            int32_t* budget_used, void* ws,
                                                            PackOut po) {
    __shared__ uint8_t kept_s[PACK ? SV_MAX_BUDGET_SLOTS : 1];
    __shared__ int32_t cu_s[PACK ? SV_MAX_BUDGET_SLOTS : 1];
    __shared__ int32_t pack_tot[kWaves];
    const int tid = threadIdx.x;
    PackIds ids;
    if (PACK) pack_prefetch(po, n_req, k_max, ids);
    const int n_slots = n_req * k_max;
    const BudgetWs w = budget_ws(ws, n_slots);
    const int per = (n_slots + kThreads - 1) / kThreads;
    int32_t rk[kPerThread], rk1[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        rk[q] = 0;
        rk1[q] = 0;
        if (q >= per) continue;  // uniform
        const int x = tid + q * kThreads;
        if (x < n_slots) rk[q] = w.rank[x];
        if (x + 1 < n_slots) rk1[q] = w.rank[x + 1];
    }
    const int total = n_slots > 0 ? w.total[0] : 0;
    const int b_in = budget_in[0];
    const int B = b_in < 0 ? 0 : (b_in > total ? total : b_in);
    write_kept(rk, rk1, per, B, n_req, k_max, kept, PACK ? kept_s : nullptr);
    if (tid == 0 && budget_used != nullptr) budget_used[0] = B;
    if (PACK) {
        __syncthreads();
        pack_from_lds(kept_s, n_req, k_max, po, ids, cu_s, pack_tot);
    }
}

// One draft length for the whole batch ("Hardware-Aware Dynamic Speculative
// Decoding (DSD), feat. Cohere", section "동적 추측 디코딩(DSD)의 핵심
// 아이디어": K chosen by goodput = acceptance length / step latency).  One
// workgroup: confidences staged in LDS; one thread per request forms its
// survival chain, stores floor(s * 2^40) of position j at column j of an LDS
// table (0 past draft_len) and counts its clamped draft length in a small
// histogram; wave w then sums columns w, w + 16, ... (a DPP wave sum of
// exact uint64 fixed-point values: order free, no contended atomics).
// Thread K forms S(K) = sum of columns j < K and T(K) = drafts verified at K
// (from the histogram), and the score (n_bonus + S * 2^-40) / cost[t_base + T]
// in IEEE fp64; the first maximiser is K*, and kept[r] = min(K*, K_r).
__global__ __launch_bounds__(kThreads) void uniform_k_kernel(
    const float* __restrict__ conf, const int32_t* __restrict__ draft_len, int n_req, int k_max,
    const float* __restrict__ cost, int t_base, int n_bonus, int32_t* __restrict__ kept,
    int32_t* __restrict__ k_out, double* __restrict__ scores, int32_t* dev_error) {
    __shared__ float conf_s[kConfLds];
    __shared__ uint64_t fx_s[SV_MAX_BUDGET_SLOTS];  // column j at j * n_req
    __shared__ unsigned long long col_sum[SV_MAX_DRAFT];
    __shared__ int32_t len_hist[SV_MAX_DRAFT + 1];
    __shared__ double score_s[SV_MAX_DRAFT + 1];
    __shared__ int32_t err_s, best_s;

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const int n_slots = n_req * k_max;
    const int kp = k_max | 1;
    float c[kPerThread];
    int32_t dl[kPerThread];
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int x = tid + q * kThreads;
        c[q] = x < n_slots ? conf[x] : 0.0f;
        dl[q] = x < n_req ? draft_len[x] : 0;
    }
    if (tid <= SV_MAX_DRAFT) len_hist[tid] = 0;
    if (tid == 0) err_s = 0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int x = tid + q * kThreads;
        if (x < n_slots) {
            const int r = x / k_max;
            conf_s[r * kp + (x - r * k_max)] = clamp_confidence(c[q]);
        }
    }
    __syncthreads();

    int my_err = 0;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int r = tid + q * kThreads;
        if (r < n_req) {
            const int K = clamp_len(dl[q], k_max);
            if (K != dl[q]) my_err |= SV_DEV_BAD_DRAFT_LEN;

            float sv = 1.0f;
            for (int j = 0; j < k_max; ++j) {
                uint64_t f = 0;
                if (j < K) {
                    sv = __fmul_rn(sv, conf_s[r * kp + j]);
                    // s * 2^40 is exact in fp32; the conversion truncates = floor
                    f = (uint64_t)(sv * 0x1p40f);
                }
                fx_s[j * n_req + r] = f;
            }
        }
    }
    // the histogram of clamped draft lengths: a ballot per length counts a
    // wave's requests at once (one LDS add per wave and length)
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int base = tid - lane + q * kThreads;
        if (base >= n_req) break;  // uniform
        const int r = base + lane;
        const int K = r < n_req ? clamp_len(dl[q], k_max) : -1;
        for (int len = 0; len <= k_max; ++len) {
            const uint64_t m = __ballot(K == len);
            if (lane == 0 && m) atomicAdd(&len_hist[len], (int)__popcll(m));
        }
    }
    my_err = wave_or_int(my_err);
    if (lane == 0 && my_err) atomicOr(&err_s, my_err);
    __syncthreads();

    for (int j = wave; j < k_max; j += kWaves) {
        uint64_t part = 0;
        for (int r = lane; r < n_req; r += kWave) part += fx_s[j * n_req + r];
        part = wave_sum_dpp(part, lane);
        if (lane == 0) col_sum[j] = part;
    }
    __syncthreads();

    if (tid <= k_max) {
        const int K = tid;
        unsigned long long S = 0ull;
        int T = 0;
        for (int j = 0; j < K; ++j) S += col_sum[j];
        // drafts verified at K: sum over requests of min(K, K_r)
        for (int len = 1; len <= k_max; ++len) T += len_hist[len] * (len < K ? len : K);
        const float cst = cost[t_base + T];
        double sc = -__builtin_inf();
        if (cst > 0.0f && is_finite_bits(cst)) {
            // S < 2^53 and 2^-40 is a power of two: the product is exact
            sc = ((double)n_bonus + (double)S * 0x1p-40) / (double)cst;
        } else {
            atomicOr(&err_s, SV_DEV_BAD_COST);
        }
        score_s[K] = sc;
        if (scores != nullptr) scores[K] = sc;
    }
    __syncthreads();
    if (tid == 0) {
        int best = 0;
        for (int K = 1; K <= k_max; ++K)
            if (score_s[K] > score_s[best]) best = K;  // the first maximiser
        best_s = best;
        k_out[0] = best;
        raise_error(dev_error, err_s);
    }
    __syncthreads();
    const int best = best_s;
#pragma unroll
    for (int q = 0; q < kPerThread; ++q) {
        const int r = tid + q * kThreads;
        if (r < n_req) {
            const int K = clamp_len(dl[q], k_max);
            kept[r] = K < best ? K : best;
        }
    }
}

}  // namespace

size_t budget_workspace_bytes(int n_req, int k_max) {
    if (n_req <= 0 || k_max < 0) return 0;
    return kHeaderBytes + (size_t)n_req * (size_t)k_max * (sizeof(int32_t) + sizeof(float));
}

hipError_t launch_rank(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                       float* survival, int32_t* dev_error, void* ws, hipStream_t stream) {
    if (n_req == 0) return hipSuccess;
    const int n_slots = n_req * k_max;
    const unsigned blocks = (unsigned)(n_slots > 0 ? (n_slots + kQueries - 1) / kQueries : 1);
    hipLaunchKernelGGL(rank_kernel, dim3(blocks), dim3(kThreads), 0, stream, conf, draft_len,
                       n_req, k_max, survival, dev_error, ws);
    return hipGetLastError();
}

hipError_t launch_budget(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                         const float* cost, int t_base, int n_bonus, int32_t* kept,
                         int32_t* budget, float* survival, int32_t* dev_error, void* ws,
                         const PackTargets* pack, hipStream_t stream) {
    const hipError_t e = launch_rank(conf, draft_len, n_req, k_max, survival, dev_error, ws,
                                     stream);
    if (e != hipSuccess) return e;
    if (pack != nullptr) {
        const PackOut po{pack->last_token, pack->draft_tokens, pack->cu_rows,
                         pack->row_req,    pack->row_pos,      pack->packed_tokens};
        hipLaunchKernelGGL(finish_kernel<true>, dim3(1), dim3(kThreads), 0, stream, n_req, k_max,
                           cost, t_base, n_bonus, kept, budget, dev_error, ws, po);
    } else {
        hipLaunchKernelGGL(finish_kernel<false>, dim3(1), dim3(kThreads), 0, stream, n_req,
                           k_max, cost, t_base, n_bonus, kept, budget, dev_error, ws, PackOut{});
    }
    return hipGetLastError();
}

hipError_t launch_allocate(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                           const int32_t* budget_in, int32_t* kept, int32_t* budget_used,
                           float* survival, int32_t* dev_error, void* ws,
                           const PackTargets* pack, hipStream_t stream) {
    const hipError_t e = launch_rank(conf, draft_len, n_req, k_max, survival, dev_error, ws,
                                     stream);
    if (e != hipSuccess) return e;
    if (pack != nullptr) {
        const PackOut po{pack->last_token, pack->draft_tokens, pack->cu_rows,
                         pack->row_req,    pack->row_pos,      pack->packed_tokens};
        hipLaunchKernelGGL(allocate_kernel<true>, dim3(1), dim3(kThreads), 0, stream, n_req,
                           k_max, budget_in, kept, budget_used, ws, po);
    } else {
        hipLaunchKernelGGL(allocate_kernel<false>, dim3(1), dim3(kThreads), 0, stream, n_req,
                           k_max, budget_in, kept, budget_used, ws, PackOut{});
    }
    return hipGetLastError();
}

}  // namespace sv

namespace sv {

hipError_t launch_uniform_k(const float* conf, const int32_t* draft_len, int n_req, int k_max,
                            const float* cost, int t_base, int n_bonus, int32_t* kept,
                            int32_t* k_out, double* scores, int32_t* dev_error,
                            hipStream_t stream) {
    hipLaunchKernelGGL(uniform_k_kernel, dim3(1), dim3(kThreads), 0, stream, conf, draft_len,
                       n_req, k_max, cost, t_base, n_bonus, kept, k_out, scores, dev_error);
    return hipGetLastError();
}

}  // namespace sv
