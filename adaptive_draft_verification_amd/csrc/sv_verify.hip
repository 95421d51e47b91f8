// Full-vocabulary verification of the kept rows (gfx950, wave64).
//
// What is computed follows the FOS blog "추측 디코딩과 vLLM 적응형 검증":
// section "추측 디코딩이란" (accept from the front up to the first mismatch,
// the target's own token fills the mismatch or follows the last draft),
// section "속도, 메모리, 정확도에 주는 영향", row 정확도 (rejection sampling
// keeps the target's law: accept with probability min(1, p/q), otherwise draw
// from the normalised residual max(0, p - q)), and section "평균 수락 길이"
// (the bonus token).
//
// Pass 1, one 256-thread workgroup per candidate row: target rows 0..b and
// (stochastic) draft rows 0..b-1 of each request.  The grid is the host-known
// capacity; workgroups of rows past a request's kept count do nothing.  The
// grid runs position-major from the last draft position down to position 0,
// so the rows pass 2 most often reads again (the first rejections happen
// early) are the last ones streamed and are still in the Infinity Cache.
//
// Row statistics.  The row is streamed once with 16-byte loads.  Stochastic
// rows keep, per thread, an offset taken from the max of the thread's first
// 16-byte chunk and accumulate exp2(z * log2(e)/T - offset) in independent
// fp32 partial sums, so the hot loop has no per-element max; per-thread
// (offset, sum) pairs merge by rescaling in a fixed tree.  If that shortcut
// overflows (a later logit more than ~88/T above the first chunk's max) the
// row is redone exactly (max pass, then sum pass).  Greedy rows track the
// running max and the lowest index reaching it.  Faults: NaN, +inf, or no
// finite mass.
//
// Pass 2, one 1024-thread workgroup per request.  Wave 0 draws the Philox
// uniforms of the kept positions, tests u < 2^(log2 p(d) - log2 q(d)) (greedy:
// d == argmax) and takes the first rejection with a ballot.  The token at L
// is drawn by inverse CDF over the residual row (or the bonus row): one sweep
// sums weights per 8192-id tile (one wave reduction per tile, no barriers,
// several tiles in flight), a wave scan over tile sums finds the tile holding
// v * W, and only that tile is read again, with a block-wide exclusive scan.
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

constexpr int kThreads = 256;                        // pass 1 workgroup
constexpr int kUnroll = 4;                           // pass 1: 16-byte loads in flight per thread
constexpr int kP2Threads = 1024;                     // pass 2 workgroup (stochastic)
constexpr int kP2Waves = kP2Threads / kWave;
constexpr int kTile = kP2Threads * 8;                // ids per tile of the draw
constexpr int kMaxTiles = SV_MAX_VOCAB / kTile;      // 128
constexpr int kTilesPerLane = kMaxTiles / kWave;     // tile scan: 2 tiles per lane of one wave
constexpr int kDrawUnroll = 4;                       // tiles in flight per thread in the sweep
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInf = __builtin_inff();

template <sv_dtype DT>
struct Vec;

template <>
struct Vec<SV_BF16> {
    static constexpr int kElems = 8;
    static constexpr int kBytes = 2;
    using raw_t = uint4;
    __device__ static __forceinline__ void unpack(const raw_t& w, float* x) {
        x[0] = bf16_lo(w.x);
        x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y);
        x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z);
        x[5] = bf16_hi(w.z);
        x[6] = bf16_lo(w.w);
        x[7] = bf16_hi(w.w);
    }
    __device__ static __forceinline__ float load1(const char* row, int i) {
        const uint16_t h = reinterpret_cast<const uint16_t*>(row)[i];
        return __uint_as_float((uint32_t)h << 16);
    }
};

template <>
struct Vec<SV_F32> {
    static constexpr int kElems = 4;
    static constexpr int kBytes = 4;
    using raw_t = float4;
    __device__ static __forceinline__ void unpack(const raw_t& w, float* x) {
        x[0] = w.x;
        x[1] = w.y;
        x[2] = w.z;
        x[3] = w.w;
    }
    __device__ static __forceinline__ float load1(const char* row, int i) {
        return reinterpret_cast<const float*>(row)[i];
    }
};


// Merge two (offset, sum) pairs: both sums re-expressed against the larger offset.
__device__ __forceinline__ void merge_as(float& a, float& s, float a2, float s2) {
    const float m = fmaxf(a, a2);
    s = s * fast_exp2(a - m) + s2 * fast_exp2(a2 - m);
    a = m;
}

// Exact two-pass row statistics (fallback): offset = max * c, then the sum.
template <sv_dtype DT>
__device__ void row_stats_exact(const char* row, int vocab, float c, float* red, float* out_a,
                                float* out_s) {
    using V = Vec<DT>;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    float m = -kInf;
    for (int e = tid; e < vocab; e += kThreads) m = fmaxf(m, V::load1(row, e));
    m = wave_max(m);
    if (lane == 0) red[wave] = m;
    __syncthreads();
    float mx = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) mx = fmaxf(mx, red[w]);
    __syncthreads();
    const float a = mx * c;
    float s = 0.0f;
    for (int e = tid; e < vocab; e += kThreads) s += fast_exp2(fmaf(V::load1(row, e), c, -a));
    s = wave_sum(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    float tot = red[0];
    for (int w = 1; w < kThreads / kWave; ++w) tot += red[w];
    *out_a = a;
    *out_s = tot;
}

// One-pass row statistics; returns through out_a/out_s (identical in every thread).
template <sv_dtype DT>
__device__ void row_stats_stochastic(const char* row, int vocab, float c, float* red,
                                     float* out_a, float* out_s) {
    using V = Vec<DT>;
    using raw_t = typename V::raw_t;
    constexpr int E = V::kElems;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    const int nvec = aligned ? vocab / E : 0;
    const raw_t* vrow = reinterpret_cast<const raw_t*>(row);

    float acc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) acc[k] = 0.0f;
    float a_t = 0.0f;
    int i = tid;
    if (i < nvec) {
        float x[E];
        V::unpack(vrow[i], x);
        float m = x[0];
#pragma unroll
        for (int k = 1; k < E; ++k) m = fmaxf(m, x[k]);
        a_t = (m == -kInf) ? 0.0f : m * c;
#pragma unroll
        for (int k = 0; k < E; ++k) acc[k] += fast_exp2(fmaf(x[k], c, -a_t));
        i += kThreads;
    } else {
        const int e = nvec * E + tid;
        if (e < vocab) {
            const float m = V::load1(row, e);
            a_t = (m == -kInf) ? 0.0f : m * c;
        }
    }
    for (; i + (kUnroll - 1) * kThreads < nvec; i += kUnroll * kThreads) {
        raw_t w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) w[u] = vrow[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[E];
            V::unpack(w[u], x);
#pragma unroll
            for (int k = 0; k < E; ++k) acc[k] += fast_exp2(fmaf(x[k], c, -a_t));
        }
    }
    for (; i < nvec; i += kThreads) {
        float x[E];
        V::unpack(vrow[i], x);
#pragma unroll
        for (int k = 0; k < E; ++k) acc[k] += fast_exp2(fmaf(x[k], c, -a_t));
    }
    for (int e = nvec * E + tid; e < vocab; e += kThreads)
        acc[0] += fast_exp2(fmaf(V::load1(row, e), c, -a_t));

    float s = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) s += acc[k];

    float a = a_t;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float a2 = __shfl_xor(a, o), s2 = __shfl_xor(s, o);
        merge_as(a, s, a2, s2);
    }
    if (lane == 0) {
        red[2 * wave] = a;
        red[2 * wave + 1] = s;
    }
    __syncthreads();
    float A = red[0], S = red[1];
    for (int w = 1; w < kThreads / kWave; ++w) merge_as(A, S, red[2 * w], red[2 * w + 1]);
    __syncthreads();
    if (!(S > 0.0f) || !is_finite_bits(S) || !is_finite_bits(A)) {
        row_stats_exact<DT>(row, vocab, c, red, &A, &S);  // block-uniform branch
    }
    *out_a = A;
    *out_s = S;
}

// Greedy: (max, lowest index reaching it) and whether the row holds a NaN.
template <sv_dtype DT>
__device__ void row_argmax(const char* row, int vocab, float* redf, int* redi, float* out_max,
                           int* out_idx, bool* out_nan) {
    using V = Vec<DT>;
    using raw_t = typename V::raw_t;
    constexpr int E = V::kElems;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    const int nvec = aligned ? vocab / E : 0;
    const raw_t* vrow = reinterpret_cast<const raw_t*>(row);

    float best = -kInf;
    int bidx = 0x7fffffff;
    bool nan = false;
    int i = tid;
    for (; i + (kUnroll - 1) * kThreads < nvec; i += kUnroll * kThreads) {
        raw_t w[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) w[u] = vrow[i + u * kThreads];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            float x[E];
            V::unpack(w[u], x);
            float cm = x[0];
#pragma unroll
            for (int k = 1; k < E; ++k) {
                cm = fmaxf(cm, x[k]);
                nan |= x[k] != x[k];
            }
            nan |= x[0] != x[0];
            if (cm > best) {
                best = cm;
                int pos = E - 1;
#pragma unroll
                for (int k = E - 1; k >= 0; --k)
                    if (x[k] == cm) pos = k;
                bidx = (i + u * kThreads) * E + pos;
            }
        }
    }
    for (; i < nvec; i += kThreads) {
        float x[E];
        V::unpack(vrow[i], x);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            nan |= x[k] != x[k];
            if (x[k] > best) {
                best = x[k];
                bidx = i * E + k;
            }
        }
    }
    for (int e = nvec * E + tid; e < vocab; e += kThreads) {
        const float x = V::load1(row, e);
        nan |= x != x;
        if (x > best) {
            best = x;
            bidx = e;
        }
    }
    int nan_i = nan ? 1 : 0;
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) {
        const float b2 = __shfl_xor(best, o);
        const int i2 = __shfl_xor(bidx, o);
        nan_i |= __shfl_xor(nan_i, o);
        if (b2 > best || (b2 == best && i2 < bidx)) {
            best = b2;
            bidx = i2;
        }
    }
    if (lane == 0) {
        redf[wave] = best;
        redi[2 * wave] = bidx;
        redi[2 * wave + 1] = nan_i;
    }
    __syncthreads();
    best = redf[0];
    bidx = redi[0];
    nan_i = redi[1];
    for (int w = 1; w < kThreads / kWave; ++w) {
        const float b2 = redf[w];
        const int i2 = redi[2 * w];
        nan_i |= redi[2 * w + 1];
        if (b2 > best || (b2 == best && i2 < bidx)) {
            best = b2;
            bidx = i2;
        }
    }
    *out_max = best;
    *out_idx = bidx;
    *out_nan = nan_i != 0;
}

struct Args {
    const char* target;
    int64_t target_ld_bytes;
    int64_t target_rows;
    const char* draft;
    int64_t draft_ld_bytes;
    int vocab;
    const int32_t* draft_tokens;
    const int32_t* cu_rows;
    int k_max;
    float c;  // log2(e) / T
    uint64_t seed;
    uint64_t step;
    RowStat* stats;  // [n, 2*k_max + 1]
    int32_t* out_tokens;
    int32_t* out_accepted;
    float* out_p;
    float* out_q;
    float* out_resid;
    int32_t* dev_error;
};

// ------------------------------------------------------------------ the draw

// 8 consecutive ids starting at e (logit -inf past the row end: weight 0).
template <sv_dtype DT>
__device__ __forceinline__ void load8(const char* row, int vocab, int e, bool aligned, float* x) {
    using V = Vec<DT>;
    if (aligned && e + 8 <= vocab) {
        const typename V::raw_t* vr = reinterpret_cast<const typename V::raw_t*>(row);
        constexpr int per = 8 / V::kElems;
#pragma unroll
        for (int q = 0; q < per; ++q) V::unpack(vr[e / V::kElems + q], x + q * V::kElems);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) x[k] = e + k < vocab ? V::load1(row, e + k) : -kInf;
    }
}

// 8 ids as raw 16-byte words (fast path: aligned, fully inside the row).
template <sv_dtype DT>
struct Raw8 {
    typename Vec<DT>::raw_t w[8 / Vec<DT>::kElems];
    __device__ __forceinline__ void fetch(const char* row, int e) {
        const typename Vec<DT>::raw_t* vr = reinterpret_cast<const typename Vec<DT>::raw_t*>(row);
#pragma unroll
        for (int q = 0; q < 8 / Vec<DT>::kElems; ++q) w[q] = vr[e / Vec<DT>::kElems + q];
    }
    __device__ __forceinline__ void unpack(float* x) const {
#pragma unroll
        for (int q = 0; q < 8 / Vec<DT>::kElems; ++q) Vec<DT>::unpack(w[q], x + q * Vec<DT>::kElems);
    }
};

// Weights of 8 ids: residual max(0, p - q) or (unnormalised) target mass.
template <bool RESID>
__device__ __forceinline__ void weights_from(const float* zp, const float* zq, float c, float ap,
                                             float isp, float aq, float isq, float* w) {
    if (RESID) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float p = fast_exp2(fmaf(zp[k], c, -ap)) * isp;
            const float q = fast_exp2(fmaf(zq[k], c, -aq)) * isq;
            w[k] = fmaxf(0.0f, p - q);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = fast_exp2(fmaf(zp[k], c, -ap));
    }
}

struct DrawSmem {
    float wsum[kMaxTiles * kP2Waves];  // per tile, per wave partial sums
    float wtot[kP2Waves];
    int cand;
    int lastpos;
    int tile;
    float base;
    float target;
    float total;
};

// Per-thread sum of 8 weights, in id order.
__device__ __forceinline__ float sum8(const float* w) {
    float s = w[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) s += w[k];
    return s;
}

// Inverse-CDF draw over one row's weights (RESID: residual of two rows).
// *mass gets the weight total.  Returns -2 if the total is not positive.
template <sv_dtype DT, bool RESID>
__device__ int draw_row(const char* prow, const char* qrow, int vocab, float c, float ap,
                        float isp, float aq, float isq, float v, DrawSmem& sm, float* mass) {
    constexpr int U = kDrawUnroll;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const bool aligned = ((reinterpret_cast<uintptr_t>(prow) | reinterpret_cast<uintptr_t>(qrow)) &
                          15) == 0;
    const int ntiles = (vocab + kTile - 1) / kTile;

    // sweep: U tiles' loads in flight before any is reduced
    for (int t0 = 0; t0 < ntiles; t0 += U) {
        float s[U];
        if (aligned && (t0 + U) * kTile <= vocab) {
            Raw8<DT> rp[U], rq[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = (t0 + u) * kTile + tid * 8;
                rp[u].fetch(prow, e);
                if (RESID) rq[u].fetch(qrow, e);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                float zp[8], zq[8], w[8];
                rp[u].unpack(zp);
                if (RESID) rq[u].unpack(zq);
                weights_from<RESID>(zp, zq, c, ap, isp, aq, isq, w);
                s[u] = sum8(w);
            }
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int e = (t0 + u) * kTile + tid * 8;
                float zp[8], zq[8], w[8];
                load8<DT>(prow, vocab, e, aligned, zp);
                if (RESID) load8<DT>(qrow, vocab, e, aligned, zq);
                weights_from<RESID>(zp, zq, c, ap, isp, aq, isq, w);
                s[u] = sum8(w);
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t0 + u >= ntiles) break;
            const float ws = wave_sum(s[u]);
            if (lane == 0) sm.wsum[(t0 + u) * kP2Waves + wave] = ws;
        }
    }
    __syncthreads();
    if (wave == 0) {
        // tile totals in a fixed order; lane l owns tiles [l*TPL, (l+1)*TPL)
        float tot[kTilesPerLane];
        float lane_sum = 0.0f;
#pragma unroll
        for (int i = 0; i < kTilesPerLane; ++i) {
            const int k = lane * kTilesPerLane + i;
            float t = 0.0f;
            if (k < ntiles)
                for (int w = 0; w < kP2Waves; ++w) t += sm.wsum[k * kP2Waves + w];
            tot[i] = t;
            lane_sum += t;
        }
        const float incl = wave_incl_scan<float>(lane_sum, lane);
        float excl = __shfl_up(incl, 1);
        if (lane == 0) excl = 0.0f;
        const float W = __shfl(incl, kWave - 1);
        const float tgt = v * W;
        // first tile of this lane whose inclusive sum passes tgt, and the sum before it
        int hit_tile = -1, last_pos_tile = -1;
        float run = excl, hit_base = 0.0f;
#pragma unroll
        for (int i = 0; i < kTilesPerLane; ++i) {
            const int k = lane * kTilesPerLane + i;
            const float before = run;
            run += tot[i];
            if (k < ntiles && hit_tile < 0 && run > tgt) {
                hit_tile = k;
                hit_base = before;
            }
            if (k < ntiles && tot[i] > 0.0f) last_pos_tile = k;
        }
        const uint64_t hits = __ballot(hit_tile >= 0);
        const uint64_t pos = __ballot(last_pos_tile >= 0);
        if (lane == 0) {
            sm.total = W;
            sm.target = tgt;
            sm.cand = 0x7fffffff;
            sm.lastpos = -1;
            sm.tile = -1;
            sm.base = 0.0f;
        }
        if (hits) {
            if (lane == __builtin_ctzll(hits)) {
                sm.tile = hit_tile;
                sm.base = hit_base;
            }
        } else if (pos) {
            // rounding left v * W at or above the total: last id of positive weight
            if (lane == 63 - __builtin_clzll(pos)) sm.tile = -1 - last_pos_tile;
        }
    }
    __syncthreads();
    *mass = sm.total;
    if (!(sm.total > 0.0f)) {
        __syncthreads();  // every thread has read sm before a second call rewrites it
        return -2;
    }
    const int tile_code = sm.tile;
    const bool crossing = tile_code >= 0;
    const int tile = crossing ? tile_code : -1 - tile_code;
    const float tgt = sm.target;
    const int e = tile * kTile + tid * 8;
    float zp[8], zq[8], w[8];
    load8<DT>(prow, vocab, e, aligned, zp);
    if (RESID) load8<DT>(qrow, vocab, e, aligned, zq);
    weights_from<RESID>(zp, zq, c, ap, isp, aq, isq, w);
    const float s = sum8(w);
    // block exclusive scan of the per-thread sums
    const float incl = wave_incl_scan<float>(s, lane);
    float excl = __shfl_up(incl, 1);
    if (lane == 0) excl = 0.0f;
    if (lane == kWave - 1) sm.wtot[wave] = incl;
    __syncthreads();
    float before = sm.base;
    for (int w2 = 0; w2 < wave; ++w2) before += sm.wtot[w2];
    float run = before + excl;
    int cand = 0x7fffffff, lastpos = -1;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        run += w[k];
        // Only an id of positive weight can be drawn: the scanned prefix and
        // the per-thread sums round differently, so a thread may start above
        // v * W; its first positive id is then the crossing.
        const bool positive = w[k] > 0.0f && e + k < vocab;
        if (crossing && positive && run > tgt && cand == 0x7fffffff) cand = e + k;
        if (positive) lastpos = e + k;
    }
    cand = wave_min_int(cand);
    lastpos = wave_max_int(lastpos);
    if (lane == 0) {
        atomicMin(&sm.cand, cand);
        atomicMax(&sm.lastpos, lastpos);
    }
    __syncthreads();
    const int tok = sm.cand != 0x7fffffff ? sm.cand : sm.lastpos;
    __syncthreads();  // sm is reused by a possible second call
    return tok;
}

// ------------------------------------------------------- finishing a request

// A faulty request writes -1 to every output of its own and reports its bits.
__device__ void emit_fault(const Args& a, int r, int bits) {
    const int tid = threadIdx.x;
    int32_t* tok_out = a.out_tokens + (int64_t)r * (a.k_max + 1);
    for (int j = tid; j <= a.k_max; j += blockDim.x) tok_out[j] = -1;
    for (int j = tid; j < a.k_max; j += blockDim.x) {
        if (a.out_p) a.out_p[(int64_t)r * a.k_max + j] = -1.0f;
        if (a.out_q) a.out_q[(int64_t)r * a.k_max + j] = -1.0f;
    }
    if (tid == 0) {
        a.out_accepted[r] = -1;
        if (a.out_resid) a.out_resid[r] = -1.0f;
        raise_error(a.dev_error, bits);
    }
}

struct FinishSmem {
    DrawSmem draw;
    int L, b, lo, fault;
};

template <sv_dtype DT, bool GREEDY>
__device__ void finish_request(const Args& a, int r, FinishSmem& sm) {
    const int tid = threadIdx.x;
    const int k_max = a.k_max;
    const RowStat* st = a.stats + (int64_t)r * (2 * k_max + 1);
    if (tid < kWave) {
        const int lane = tid;
        const int lo = a.cu_rows[r], hi = a.cu_rows[r + 1];
        const int b = hi - lo - 1;
        int fault = 0;
        bool acc = true;
        if (lo < 0 || b < 0 || b > k_max || (int64_t)hi > a.target_rows) {
            fault = SV_DEV_BAD_CU_ROWS;
        } else {
            const int j = lane;
            if (j < b) {
                const int d = a.draft_tokens[(int64_t)r * k_max + j];
                if (d < 0 || d >= a.vocab) fault |= SV_DEV_BAD_TOKEN;
                const RowStat ts = st[j];
                if (GREEDY) {
                    if (ts.idx < 0) fault |= SV_DEV_NONFINITE;
                    acc = ts.idx == d;
                } else {
                    const RowStat ds = st[k_max + 1 + j];
                    if (!(ts.s > 0.0f) || !(ds.s > 0.0f)) fault |= SV_DEV_NONFINITE;
                    float u, v;
                    draw_uniforms(a.seed, a.step, (uint32_t)r, (uint32_t)j, &u, &v);
                    // u < min(1, p/q), the ratio taken from log2 p - log2 q so that
                    // probabilities below fp32's normal range do not decide it
                    acc = u < exp2f(ts.lpd - ds.lpd);
                }
            }
            if (lane == 0 && (GREEDY ? st[b].idx < 0 : !(st[b].s > 0.0f)))
                fault |= SV_DEV_NONFINITE;
        }
        fault = wave_or_int(fault);
        const uint64_t rej = __ballot(!acc);
        if (lane == 0) {
            sm.L = rej ? __builtin_ctzll(rej) : b;
            sm.b = b;
            sm.lo = lo;
            sm.fault = fault;
        }
    }
    __syncthreads();
    if (sm.fault) {
        emit_fault(a, r, sm.fault);
        return;
    }
    const int L = sm.L, b = sm.b, lo = sm.lo;
    int token;
    float mass = -1.0f;
    if (GREEDY) {
        token = st[L].idx;
    } else {
        float u, v;
        draw_uniforms(a.seed, a.step, (uint32_t)r, (uint32_t)L, &u, &v);
        const RowStat tp = st[L];
        const char* prow = a.target + ((int64_t)lo + L) * a.target_ld_bytes;
        if (L < b) {
            const RowStat tq = st[k_max + 1 + L];
            const char* qrow = a.draft + ((int64_t)r * k_max + L) * a.draft_ld_bytes;
            token = draw_row<DT, true>(prow, qrow, a.vocab, a.c, tp.a, 1.0f / tp.s, tq.a,
                                       1.0f / tq.s, v, sm.draw, &mass);
            if (token == -2) {  // zero residual mass: draw from p instead
                float unused;
                token = draw_row<DT, false>(prow, prow, a.vocab, a.c, tp.a, 1.0f, 0.0f, 1.0f, v,
                                            sm.draw, &unused);
            }
        } else {
            float unused;
            token = draw_row<DT, false>(prow, prow, a.vocab, a.c, tp.a, 1.0f, 0.0f, 1.0f, v,
                                        sm.draw, &unused);
        }
    }
    if (token < 0) {  // no id carries weight: only reachable through a numeric fault
        emit_fault(a, r, SV_DEV_NONFINITE);
        return;
    }
    int32_t* tok_out = a.out_tokens + (int64_t)r * (k_max + 1);
    for (int j = tid; j <= k_max; j += blockDim.x) {
        int t = -1;
        if (j < L) t = a.draft_tokens[(int64_t)r * k_max + j];
        else if (j == L) t = token;
        tok_out[j] = t;
    }
    for (int j = tid; j < k_max; j += blockDim.x) {
        float p = -1.0f, q = -1.0f;
        if (!GREEDY && j < b) {
            p = st[j].pd;
            q = st[k_max + 1 + j].pd;
        }
        if (a.out_p) a.out_p[(int64_t)r * k_max + j] = p;
        if (a.out_q) a.out_q[(int64_t)r * k_max + j] = q;
    }
    if (tid == 0) {
        a.out_accepted[r] = L;
        if (a.out_resid) a.out_resid[r] = (!GREEDY && L < b) ? mass : -1.0f;
    }
}

// ------------------------------------------------------------------ kernels

// Pass-1 workgroup g -> (request, slot).  Groups of n workgroups run the same
// row kind for every request: target row K first, then for j = K-1 .. 0 draft
// row j and target row j.  Slots: target j = j, draft j = k_max + 1 + j.
__device__ __forceinline__ void pass1_slot(int g, int n_req, int k_max, bool greedy, int* r,
                                           int* slot) {
    const int grp = g / n_req;
    *r = g - grp * n_req;
    if (greedy) {
        *slot = k_max - grp;
        return;
    }
    if (grp == 0) {
        *slot = k_max;
        return;
    }
    const int j = k_max - 1 - (grp - 1) / 2;
    *slot = ((grp - 1) & 1) == 0 ? k_max + 1 + j : j;
}

template <sv_dtype DT, bool GREEDY>
__global__ __launch_bounds__(kThreads) void rowstats_kernel(Args a, int n_req) {
    __shared__ float redf[2 * (kThreads / kWave)];
    __shared__ int redi[2 * (kThreads / kWave)];
    int r, slot;
    pass1_slot(blockIdx.x, n_req, a.k_max, GREEDY, &r, &slot);
    const int lo = a.cu_rows[r], hi = a.cu_rows[r + 1];
    const int b = hi - lo - 1;
    if (lo < 0 || b < 0 || b > a.k_max || (int64_t)hi > a.target_rows) return;
    const bool is_draft = slot > a.k_max;
    const int j = is_draft ? slot - a.k_max - 1 : slot;
    if (is_draft ? (j >= b) : (j > b)) return;
    const char* row = is_draft ? a.draft + ((int64_t)r * a.k_max + j) * a.draft_ld_bytes
                               : a.target + ((int64_t)lo + j) * a.target_ld_bytes;
    RowStat* out = a.stats + (int64_t)r * (2 * a.k_max + 1) + slot;
    if (GREEDY) {
        float mx;
        int idx;
        bool nan;
        row_argmax<DT>(row, a.vocab, redf, redi, &mx, &idx, &nan);
        if (threadIdx.x == 0) {
            const bool fault = nan || mx == kInf || mx == -kInf;
            RowStat st{};
            st.a = mx;
            st.idx = fault ? -1 : idx;
            *out = st;
        }
        return;
    }
    // the draft id's logit is fetched up front so its latency hides under the stream
    const int d = j < b ? a.draft_tokens[(int64_t)r * a.k_max + j] : -1;
    const bool want_pd = d >= 0 && d < a.vocab;
    float zd = 0.0f;
    if (threadIdx.x == 0 && want_pd) zd = Vec<DT>::load1(row, d);
    float A, S;
    row_stats_stochastic<DT>(row, a.vocab, a.c, redf, &A, &S);
    if (threadIdx.x == 0) {
        const bool fault = !(S > 0.0f) || !is_finite_bits(S) || !is_finite_bits(A);
        const float y = fmaf(zd, a.c, -A);
        RowStat st;
        st.a = A;
        st.s = fault ? -1.0f : S;
        st.pd = want_pd ? exp2f(y) / S : -1.0f;
        st.lpd = want_pd ? y - log2f(S) : -kInf;
        *out = st;
    }
}

template <sv_dtype DT, bool GREEDY>
__global__ __launch_bounds__(GREEDY ? kWave : kP2Threads) void decide_kernel(Args a) {
    __shared__ FinishSmem fin;
    finish_request<DT, GREEDY>(a, blockIdx.x, fin);
}

template <sv_dtype DT, bool GREEDY>
hipError_t launch_typed(const VerifyArgs& v, hipStream_t stream) {
    const int esize = Vec<DT>::kBytes;
    Args a{static_cast<const char*>(v.target), v.target_ld * esize, v.target_rows,
           static_cast<const char*>(v.draft), v.draft_ld * esize, v.vocab, v.draft_tokens,
           v.cu_rows, v.k_max, kLog2e / v.temperature, v.seed, v.step,
           static_cast<RowStat*>(v.ws), v.out_tokens, v.out_accepted, v.out_p_draft,
           v.out_q_draft, v.out_residual_mass, v.dev_error};
    const int slots = GREEDY ? v.k_max + 1 : 2 * v.k_max + 1;
    if (v.stages & 1) {
        hipLaunchKernelGGL((rowstats_kernel<DT, GREEDY>), dim3((unsigned)(v.n_req * slots)),
                           dim3(kThreads), 0, stream, a, v.n_req);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (!(v.stages & 2)) return hipSuccess;
    hipLaunchKernelGGL((decide_kernel<DT, GREEDY>), dim3((unsigned)v.n_req),
                       dim3(GREEDY ? kWave : kP2Threads), 0, stream, a);
    return hipGetLastError();
}

__global__ void philox_uniforms_kernel(uint64_t seed, uint64_t step, int n_req, int n_pos,
                                       float* u, float* v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)n_req * n_pos) return;
    const int r = (int)(i / n_pos), j = (int)(i - (int64_t)r * n_pos);
    float uu, vv;
    draw_uniforms(seed, step, (uint32_t)r, (uint32_t)j, &uu, &vv);
    u[i] = uu;
    v[i] = vv;
}

}  // namespace

size_t verify_workspace_bytes(int n_req, int k_max) {
    return (size_t)n_req * (size_t)(2 * k_max + 1) * sizeof(RowStat);
}

hipError_t launch_verify(const VerifyArgs& v, hipStream_t stream) {
    if (v.n_req == 0) return hipSuccess;
    VerifyArgs w = v;
    if (v.mode == SV_GREEDY) w.temperature = 1.0f;
    if (v.dtype == SV_BF16)
        return v.mode == SV_GREEDY ? launch_typed<SV_BF16, true>(w, stream)
                                   : launch_typed<SV_BF16, false>(w, stream);
    return v.mode == SV_GREEDY ? launch_typed<SV_F32, true>(w, stream)
                               : launch_typed<SV_F32, false>(w, stream);
}

hipError_t launch_philox_uniforms(uint64_t seed, uint64_t step, int n_req, int n_pos, float* u,
                                  float* v, hipStream_t stream) {
    const int64_t n = (int64_t)n_req * n_pos;
    if (n == 0) return hipSuccess;
    const int threads = 256;
    hipLaunchKernelGGL(philox_uniforms_kernel, dim3((unsigned)((n + threads - 1) / threads)),
                       dim3(threads), 0, stream, seed, step, n_req, n_pos, u, v);
    return hipGetLastError();
}

}  // namespace sv
