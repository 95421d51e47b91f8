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
// Pass 1, one 512-thread workgroup per row part: target rows
// 0..b and (stochastic) draft rows 0..b-1 of each request.  The grid is the
// host-known capacity.  With well-formed offsets workgroup u takes the u-th
// existing row part (target rows in packed order, then draft rows), so the
// workgroups without a row sit at the end of the grid and exit at once;
// other offsets keep a (position, request) order whose checks reject bad
// requests one by one.
//
// Row statistics.  The row is streamed once with 16-byte non-temporal loads
// (each byte is read once; keeping it out of the caches measurably raises
// the streaming rate).  Stochastic rows keep, per thread, an integer offset
// and accumulate exp2(z * log2(e)/T - offset) in independent fp32 partial
// sums; the exponents of each 16-byte chunk are checked before use and the
// offset moves up (rescaling the sums exactly) when one would enter above 8,
// so the largest terms are computed from small, accurately rounded
// exponents.  Per-thread (offset, sum) pairs merge by exact power-of-two
// scalings in a fixed tree.  A part holding a NaN or +inf, or no finite
// mass, is redone exactly (max pass, then sum pass).  Greedy rows track the
// running max and the lowest index reaching it.  Faults: NaN, +inf, or no
// finite mass.
//
// Pass 2, one 1024-thread workgroup per request.  Wave 0 draws the Philox
// uniforms of the kept positions, tests u < 2^(log2 p(d) - log2 q(d)) (greedy:
// d == argmax) and takes the first rejection with a ballot.  The token at L
// is drawn by inverse CDF over the residual row (or the bonus row): waves
// claim super-groups (512 ids; 1024 on a bf16 bonus row) from an LDS
// counter and stream them (the next
// one's loads in flight while the current one is summed, no barrier in the
// stream), each super-group's sum goes to LDS, and wave 0 walks the sums in
// id order and reads only the crossing super-group again.  The bonus row's
// total is pass 1's sum, so its draw stops claiming once the super-groups
// already summed pass v * W.
#include "sv_device.h"
#include "sv_launch.h"

namespace sv {
namespace {

// Launch shapes (overridable at build time for tuning sweeps).  Measured on
// MI355X, 256 requests x 8 rows x 129280 bf16: non-temporal pass-1 loads move
// the stream from ~5.8 to ~6.5 TB/s; 512-thread workgroups beat 256 and 1024;
// with the dense order, parts of up to 131072 ids (one per row here) beat
// 65536 (74.7 vs 76.8 us) and smaller parts lose more (3 parts 81, 4 parts
// 88 us); five loads in flight per thread beat four (73.1-73.5 against
// 74.4-74.7 us adaptive, 147.8 against 149.9 full K) and three, six and eight;
// draft rows with features keep four (five costs them occupancy); bf16 draw super-groups of 512 ids per
// wave beat 1024 (28.4 vs 29.1 us: finer claims even out the waves' ends and
// the second look is shorter), 1536 (30.4) and 2048 (35.2).
#ifndef SV_PASS1_THREADS
#define SV_PASS1_THREADS 512
#endif
#ifndef SV_PASS1_UNROLL
#define SV_PASS1_UNROLL 5
#endif
#ifndef SV_PASS1_NONTEMPORAL
#define SV_PASS1_NONTEMPORAL 1
#endif
#ifndef SV_DRAW_UNROLL
#define SV_DRAW_UNROLL 1
#endif
constexpr int kThreads = SV_PASS1_THREADS;           // pass 1 workgroup
constexpr int kUnroll = SV_PASS1_UNROLL;             // pass 1: 16-byte loads in flight per thread
constexpr int kFeatUnroll = 4;  // draft rows with features: two more sums per element, fewer loads
constexpr int kP2Threads = 1024;                     // pass 2 workgroup (stochastic)
constexpr int kP2Waves = kP2Threads / kWave;
constexpr int kDrawUnroll = SV_DRAW_UNROLL;          // 8-id groups per lane per super-group
// Greedy pass 1 (target rows only, a max per element instead of an exp):
// 512-thread workgroups with six 16-byte loads in flight per thread (full K,
// 2048 rows of 129280 bf16: 80.5 us against 83.0 with 256 threads and 85 with
// 1024; the adaptive batch 43.0 against 43.2); half-row parts, eight loads in
// flight and a scheduling barrier after the loads all lost.
#ifndef SV_GREEDY_THREADS
#define SV_GREEDY_THREADS 512
#endif
#ifndef SV_GREEDY_UNROLL
#define SV_GREEDY_UNROLL 6
#endif

constexpr int kGreedyThreads = SV_GREEDY_THREADS;
constexpr int kGreedyUnroll = SV_GREEDY_UNROLL;
template <bool GREEDY>
constexpr int pass1_threads() { return GREEDY ? kGreedyThreads : kThreads; }

// One 16-byte load of streamed row data (optionally non-temporal: read once,
// no point keeping it in the caches).
template <typename T>
__device__ __forceinline__ T stream_load(const T* p) {
    static_assert(sizeof(T) == 16, "16-byte loads only");
#if SV_PASS1_NONTEMPORAL
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    T out;
    __builtin_memcpy(&out, &v, 16);
    return out;
#else
    return *p;
#endif
}
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


// s * 2^d for an integer d <= 0, exact (v_ldexp_f32): every offset is an
// integer, so moving a sum between offsets rounds nothing.  d below -256
// (a pair without mass, below) gives 0.
__device__ __forceinline__ float scale_exp2(float s, float d) {
    return ldexpf(s, (int)fmaxf(d, -256.0f));
}

// Offset of a pair without mass (a thread that met no finite logit): far
// below any real offset, so that merging it scales its zero sum by 0 and
// leaves the other pair as it was; two such pairs merge to one.
constexpr float kNoMass = -1.0e30f;

// Highest exponent t = y - a at which a pass-1 term enters before its
// thread's offset moves up: with |t| < 8 for the largest terms, the rounding
// of t (half an ulp of t) costs them at most 2^-22 ln 2 of their value.
#ifndef SV_REOFFSET
#define SV_REOFFSET 8.0f
#endif
#ifndef SV_REOFFSET_HEADROOM
#define SV_REOFFSET_HEADROOM 7.0f
#endif
constexpr float kReoffset = SV_REOFFSET;
// A moved offset sits this far above the logit that moved it, so that the
// next move needs a logit kReoffset + kHeadroom higher: measured on 256 x 8
// rows of 129280 bf16 N(0, 3^2) logits, a window (-8, 8] costs pass 1
// ~0.6 us against ~2 us for (-1, 4] (moves in most chunks' waves).
constexpr float kHeadroom = SV_REOFFSET_HEADROOM;

// Merge two (offset, sum) pairs: both sums re-expressed against the larger
// offset (exact scalings; the one rounding is the add).  A NaN sum propagates.
__device__ __forceinline__ void merge_as(float& a, float& s, float a2, float s2) {
    const float m = fmaxf(a, a2);
    s = scale_exp2(s, a - m) + scale_exp2(s2, a2 - m);
    a = m;
}

// Draft-row features carry e = sum_x 2^(t_x) t_x, t_x = y_x - a, next to the
// (offset a, sum s) pair; moving the offset from a to m turns e into
// 2^(a - m) (e + (a - m) s).  s and a come out bit for bit as in merge_as.
__device__ __forceinline__ void merge_ase(float& a, float& s, float& e, float a2, float s2,
                                          float e2) {
    const float m = fmaxf(a, a2);
    const float d1 = fmaxf(a - m, -256.0f), d2 = fmaxf(a2 - m, -256.0f);
    e = scale_exp2(fmaf(d1, s, e), d1) + scale_exp2(fmaf(d2, s2, e2), d2);
    s = scale_exp2(s, d1) + scale_exp2(s2, d2);
    a = m;
}

// The merges as scan operators (earlier lane t, later lane v) for the DPP wave
// reductions: a fixed combination order, the same in the plain and the
// feature variants, so that (a, s) agree bit for bit between them.
struct AS {
    float a, s;
};
struct ASEM {
    float a, s, e, mx;
};
struct MergeAsOp {
    __device__ __forceinline__ AS operator()(AS t, AS v) const {
        merge_as(v.a, v.s, t.a, t.s);
        return v;
    }
};
struct MergeAseOp {
    __device__ __forceinline__ ASEM operator()(ASEM t, ASEM v) const {
        merge_ase(v.a, v.s, v.e, t.a, t.s, t.e);
        v.mx = fmaxf(v.mx, t.mx);
        return v;
    }
};

// Lower clamp of t in the entropy term: an id of logit -inf has weight 0 and
// must add 0, not 0 * -inf.
constexpr float kTFloor = -256.0f;

// Feature side of a part: e (above) and the part's largest logit.
struct FeatAcc {
    float e = 0.0f;
    float mx = -__builtin_inff();
};

// Exact two-pass statistics (fallback): offset = ceil(max * c), then the sum.
// A range holding a NaN or +inf returns S = NaN; one whose logits are all -inf
// returns (A, S) = (-inf, 0).
template <sv_dtype DT, bool FEAT = false>
__device__ void row_stats_exact(const char* row, int vocab, float c, float* red, float* out_a,
                                float* out_s, FeatAcc* feat = nullptr) {
    using V = Vec<DT>;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    float m = -kInf;
    int nan = 0;
    for (int e = tid; e < vocab; e += kThreads) {
        const float x = V::load1(row, e);
        m = fmaxf(m, x);
        nan |= x != x;
    }
    m = wave_max(m);
    nan = wave_or_int(nan);
    if (lane == 0) {
        red[2 * wave] = m;
        red[2 * wave + 1] = nan ? 1.0f : 0.0f;
    }
    __syncthreads();
    float mx = red[0];
    bool any_nan = red[1] != 0.0f;
    for (int w = 1; w < kThreads / kWave; ++w) {
        mx = fmaxf(mx, red[2 * w]);
        any_nan |= red[2 * w + 1] != 0.0f;
    }
    __syncthreads();
    if (any_nan || mx == kInf) {  // block-uniform
        *out_a = 0.0f;
        *out_s = __builtin_nanf("");
        return;
    }
    if (mx == -kInf) {
        *out_a = -kInf;
        *out_s = 0.0f;
        return;
    }
    const float a = ceilf(mx * c);
    float s = 0.0f, ef = 0.0f;
    for (int e = tid; e < vocab; e += kThreads) {
        const float t = fmaf(V::load1(row, e), c, -a);
        const float w = fast_exp2(t);
        s += w;
        if (FEAT) ef = fmaf(w, fmaxf(t, kTFloor), ef);
    }
    s = wave_sum(s);
    if (FEAT) ef = wave_sum(ef);
    if (lane == 0) {
        red[2 * wave] = s;
        red[2 * wave + 1] = ef;
    }
    __syncthreads();
    float tot = red[0], etot = red[1];
    for (int w = 1; w < kThreads / kWave; ++w) {
        tot += red[2 * w];
        etot += red[2 * w + 1];
    }
    *out_a = a;
    *out_s = tot;
    if (FEAT) {
        feat->e = etot;
        feat->mx = mx;
    }
}

// One-pass row statistics; returns through out_a/out_s (identical in every
// thread).  FEAT also accumulates the entropy term and the largest logit (two
// more VALU operations per element) into *feat; (a, s) come out bit for bit
// as without it.  dtok (or null): where the position's draft id is; thread 0
// reads it before the stream's first load and, once the first chunk is in
// (the id with it), the id's logit if the id lies in this part (ids id0 ..
// id0 + vocab - 1), into *zd: no wave waits for the id before it streams.
template <sv_dtype DT, bool FEAT = false>
__device__ void row_stats_stochastic(const char* row, int vocab, float c, float* red,
                                     float* out_a, float* out_s,
                                     FeatAcc* feat = nullptr, const int32_t* dtok = nullptr,
                                     float* zd = nullptr, int id0 = 0) {
    using V = Vec<DT>;
    using raw_t = typename V::raw_t;
    constexpr int E = V::kElems;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15) == 0;
    const int nvec = aligned ? vocab / E : 0;
    const raw_t* vrow = reinterpret_cast<const raw_t*>(row);

    float acc[E], eacc[E];
#pragma unroll
    for (int k = 0; k < E; ++k) {
        acc[k] = 0.0f;
        eacc[k] = 0.0f;
    }
    float mx = -kInf;
    // The thread's offset: an integer, kNoMass until its first finite logit.
    // Every term enters at t = y - a_t <= kReoffset (a chunk whose largest
    // logit would enter higher first moves the offset to ceil(y_max) +
    // kHeadroom), so the thread's largest terms have |t| < 8 and their
    // exponents round to within 2^-22 however far the row's peak lies above
    // its first logits; no sum can overflow.
    float a_t = kNoMass;
    auto reoffset = [&](float a_new) {
        const float d = fmaxf(a_t - a_new, -256.0f);  // an integer below 0
#pragma unroll
        for (int k = 0; k < E; ++k) {
            if (FEAT) eacc[k] = scale_exp2(fmaf(d, acc[k], eacc[k]), d);
            acc[k] = scale_exp2(acc[k], d);
        }
        a_t = a_new;
    };
    // one element at exponent t: its weight into acc, and with FEAT its
    // entropy term
    auto add = [&](float t, int k) {
        const float w = fast_exp2(t);
        acc[k] += w;
        if (FEAT) eacc[k] = fmaf(w, fmaxf(t, kTFloor), eacc[k]);
    };
    // one 16-byte chunk (E elements), checked before any exponent is used
    // (no branch taken unless some lane's chunk enters too high): plain rows
    // check the max of the exponents against the current offset; with FEAT
    // the chunk's largest logit, which the features keep anyway
    auto take = [&](const raw_t& raw) {
        float x[E], t[E];
        V::unpack(raw, x);
        if (FEAT) {
            float y = x[0];
#pragma unroll
            for (int k = 1; k < E; ++k) y = fmaxf(y, x[k]);
            mx = fmaxf(mx, y);
            if (fmaf(y, c, -a_t) > kReoffset) reoffset(ceilf(y * c) + kHeadroom);
#pragma unroll
            for (int k = 0; k < E; ++k) t[k] = fmaf(x[k], c, -a_t);
        } else {
#pragma unroll
            for (int k = 0; k < E; ++k) t[k] = fmaf(x[k], c, -a_t);
            float m = t[0];
#pragma unroll
            for (int k = 1; k < E; ++k) m = fmaxf(m, t[k]);
            if (m > kReoffset) {
                float y = x[0];
#pragma unroll
                for (int k = 1; k < E; ++k) y = fmaxf(y, x[k]);
                reoffset(ceilf(y * c) + kHeadroom);
#pragma unroll
                for (int k = 0; k < E; ++k) t[k] = fmaf(x[k], c, -a_t);
            }
        }
#pragma unroll
        for (int k = 0; k < E; ++k) add(t[k], k);
    };
    auto take1 = [&](float x) {
        if (FEAT) mx = fmaxf(mx, x);
        if (fmaf(x, c, -a_t) > kReoffset) reoffset(ceilf(x * c) + kHeadroom);
        add(fmaf(x, c, -a_t), 0);
    };
    int did = -1;
    if (tid == 0 && dtok != nullptr) did = *dtok;
    int i = tid;
    if (i < nvec) {
        take(stream_load(vrow + i));
        i += kThreads;
    }
    if (tid == 0 && did >= id0 && did - id0 < vocab) *zd = V::load1(row, did - id0);
    // loads in flight per thread (the feature sums need registers of their own)
    constexpr int U = FEAT ? kFeatUnroll : kUnroll;
    for (; i + (U - 1) * kThreads < nvec; i += U * kThreads) {
        raw_t w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = stream_load(vrow + i + u * kThreads);
#pragma unroll
        for (int u = 0; u < U; ++u) take(w[u]);
    }
    for (; i < nvec; i += kThreads) take(stream_load(vrow + i));
    for (int e = nvec * E + tid; e < vocab; e += kThreads) take1(V::load1(row, e));

    float s = 0.0f, ef = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        s += acc[k];
        if (FEAT) ef += eacc[k];
    }

    // a thread that met no finite logit (s = 0) must not move the offset
    float a = s == 0.0f ? kNoMass : a_t;
    if (FEAT) {
        const ASEM w = lane63(wave_scan_dpp(ASEM{a, s, ef, mx}, lane, MergeAseOp{}));
        a = w.a;
        s = w.s;
        ef = w.e;
        mx = w.mx;
    } else {
        const AS w = lane63(wave_scan_dpp(AS{a, s}, lane, MergeAsOp{}));
        a = w.a;
        s = w.s;
    }
    if (lane == 0) {
        red[4 * wave] = a;
        red[4 * wave + 1] = s;
        if (FEAT) {
            red[4 * wave + 2] = ef;
            red[4 * wave + 3] = mx;
        }
    }
    __syncthreads();
    float A = red[0], S = red[1], EF = FEAT ? red[2] : 0.0f, MX = FEAT ? red[3] : -kInf;
    for (int w = 1; w < kThreads / kWave; ++w) {
        if (FEAT) {
            merge_ase(A, S, EF, red[4 * w], red[4 * w + 1], red[4 * w + 2]);
            MX = fmaxf(MX, red[4 * w + 3]);
        } else {
            merge_as(A, S, red[4 * w], red[4 * w + 1]);
        }
    }
    __syncthreads();
    // Exact path (block-uniform): a NaN or +inf, no mass, or a sum that is
    // not finite.
    if (!(S > 0.0f) || !is_finite_bits(S) || !is_finite_bits(A) ||
        (FEAT && !is_finite_bits(EF))) {
        row_stats_exact<DT, FEAT>(row, vocab, c, red, &A, &S, feat);
    } else {
        // S brought to [1/2, 1) by moving the offset by a whole number (both
        // exact): the part's largest terms then sit within a few units of
        // t = 0 in the second pass and in p(d), whatever headroom the threads
        // kept, and the second pass's sums of 2^(y - A) cannot overflow.
        int k;
        frexpf(S, &k);
        if (FEAT) EF = ldexpf(fmaf(-(float)k, S, EF), -k);
        S = ldexpf(S, -k);
        A += (float)k;
        if (FEAT) {
            feat->e = EF;
            feat->mx = MX;
        }
    }
    *out_a = A;
    *out_s = S;
}

// (max, lowest index reaching it, NaN seen) as a scan operator.
struct ArgMax {
    float best;
    int idx;
    int nan;
};
struct ArgMaxOp {
    __device__ __forceinline__ ArgMax operator()(ArgMax t, ArgMax v) const {
        v.nan |= t.nan;
        if (t.best > v.best || (t.best == v.best && t.idx < v.idx)) {
            v.best = t.best;
            v.idx = t.idx;
        }
        return v;
    }
};

// Greedy: (max, lowest index reaching it) and whether the row holds a NaN.
template <sv_dtype DT, int T, int U>
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
    for (; i + (U - 1) * T < nvec; i += U * T) {
        raw_t w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = stream_load(vrow + i + u * T);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float x[E];
            V::unpack(w[u], x);
            // IEEE maximum propagates NaN (v_maximum3_f32), so one test per
            // chunk finds a NaN; a NaN chunk never beats the running max
            float cm = x[0];
#pragma unroll
            for (int k = 1; k < E; ++k) cm = __builtin_elementwise_maximum(cm, x[k]);
            nan |= cm != cm;
            if (cm > best) {
                best = cm;
                int pos = E - 1;
#pragma unroll
                for (int k = E - 1; k >= 0; --k)
                    if (x[k] == cm) pos = k;
                bidx = (i + u * T) * E + pos;
            }
        }
    }
    for (; i < nvec; i += T) {
        float x[E];
        V::unpack(stream_load(vrow + i), x);
#pragma unroll
        for (int k = 0; k < E; ++k) {
            nan |= x[k] != x[k];
            if (x[k] > best) {
                best = x[k];
                bidx = i * E + k;
            }
        }
    }
    for (int e = nvec * E + tid; e < vocab; e += T) {
        const float x = V::load1(row, e);
        nan |= x != x;
        if (x > best) {
            best = x;
            bidx = e;
        }
    }
    int nan_i = nan ? 1 : 0;
    {
        const ArgMax w = lane63(wave_scan_dpp(ArgMax{best, bidx, nan_i}, lane, ArgMaxOp{}));
        best = w.best;
        bidx = w.idx;
        nan_i = w.nan;
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
    for (int w = 1; w < T / kWave; ++w) {
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

// Per-part statistics written by verify pass 1 and merged by pass 2.  A row
// is cut into row_parts(vocab) contiguous parts of part_len ids (a multiple
// of 8, so every part starts 16-byte aligned), one workgroup each.
//   a   : stochastic: offset, max_x z_x * log2(e)/T over the part (up to
//         rounding), -inf for a part without a finite logit; greedy: the
//         part's max logit;
//   s   : stochastic: sum_x exp2(z_x * log2(e)/T - a) over the part; 0 for a
//         part without a finite logit; -1 if the part holds a NaN or +inf;
//   zd  : stochastic: the logit of the position's draft id when it lies in
//         this part;
//   idx : greedy: the lowest id reaching the part's max (INT_MAX if every
//         logit is -inf), -1 if the part holds a NaN.
struct alignas(16) PartStat {
    float a;
    float s;
    float zd;
    int32_t idx;
};
// Draft-row features of one part (stochastic mode, when asked for):
//   e  : sum_x 2^(t_x) t_x, t_x = z_x * log2(e)/T - a (a the part's offset);
//   mx : the part's largest logit.
struct alignas(8) FeatPart {
    float e;
    float mx;
};
constexpr int kMaxParts = 8;
#ifndef SV_PART_IDS
#define SV_PART_IDS 131072
#endif
#ifndef SV_GREEDY_PART_IDS
#define SV_GREEDY_PART_IDS SV_PART_IDS
#endif
constexpr int kPartIds = SV_PART_IDS;  // parts of about this many ids
constexpr int kGreedyPartIds = SV_GREEDY_PART_IDS;

__device__ __forceinline__ int part_len(int vocab, int parts) {
    return ((vocab + parts - 1) / parts + 7) & ~7;
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
    int parts;  // row parts (pass-1 workgroups per row)
    float c;  // log2(e) / T
    uint64_t seed;
    uint64_t step;
    PartStat* stats;  // [n, 2*k_max + 1, kMaxParts]
    FeatPart* feat;   // [n, k_max, kMaxParts] (draft rows)
    int32_t* out_tokens;
    int32_t* out_accepted;
    float* out_p;
    float* out_q;
    float* out_resid;
    float* out_qh;    // draft-row entropy (bits), or null
    float* out_qm;    // draft-row largest probability, or null
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
// The sweep reads each id once, so its loads are non-temporal like pass 1's
// (measured: pass 2 34.8 -> 32.6 us, and the rows no longer linger in the
// Infinity Cache).
template <sv_dtype DT>
struct Raw8 {
    typename Vec<DT>::raw_t w[8 / Vec<DT>::kElems];
    __device__ __forceinline__ void fetch(const char* row, int e) {
        const typename Vec<DT>::raw_t* vr = reinterpret_cast<const typename Vec<DT>::raw_t*>(row);
#pragma unroll
        for (int q = 0; q < 8 / Vec<DT>::kElems; ++q)
            w[q] = stream_load(vr + e / Vec<DT>::kElems + q);
    }
    __device__ __forceinline__ void unpack(float* x) const {
#pragma unroll
        for (int q = 0; q < 8 / Vec<DT>::kElems; ++q) Vec<DT>::unpack(w[q], x + q * Vec<DT>::kElems);
    }
};

// Weights of 8 ids, both in the scale of p's own sum S_p (the draw needs
// only their ratios): the residual S_p max(0, p - q) = max(0, p' - rq q') with
// p' = 2^(z_p c - ap), q' = 2^(z_q c - aq) and rq = S_p / S_q, one fused
// multiply-add and no normalising multiply; or the target mass p'.
template <bool RESID>
__device__ __forceinline__ void weights_from(const float* zp, const float* zq, float c, float ap,
                                             float aq, float rq, float* w) {
    if (RESID) {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float p = fast_exp2(fmaf(zp[k], c, -ap));
            const float q = fast_exp2(fmaf(zq[k], c, -aq));
            w[k] = fmaxf(0.0f, fmaf(-q, rq, p));
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) w[k] = fast_exp2(fmaf(zp[k], c, -ap));
    }
}

// Draw geometry: a super-group is Geom<DT, RESID>::kIds consecutive ids, one
// wave's unit of work in the sweep (lane l takes the 8-id groups at 8 l + 512 u,
// u < U).  A residual draw reads two rows per id, a bonus draw one: bf16 bonus
// rows take two groups per lane (the loads in flight of a residual draw's
// one), fp32 rows one either way (twice the registers per group).
template <sv_dtype DT, bool RESID>
struct Geom {
    static constexpr int kU = DT == SV_BF16 ? (RESID ? kDrawUnroll : 2 * kDrawUnroll)
                                            : (kDrawUnroll + 1) / 2;
    static constexpr int kIds = kWave * 8 * kU;
    static constexpr int kMaxGroups = (SV_MAX_VOCAB + kIds - 1) / kIds;
    static constexpr int kIdsPerLane = kIds / kWave;  // second look: one lane's ids
};
constexpr int kMaxGroupsAny = Geom<SV_F32, true>::kMaxGroups > Geom<SV_BF16, true>::kMaxGroups
                                  ? Geom<SV_F32, true>::kMaxGroups
                                  : Geom<SV_BF16, true>::kMaxGroups;
// the early stop of a draw with a known total takes its margin from at most
// 2^11 super-groups a row
static_assert(Geom<SV_F32, false>::kMaxGroups <= 2048 && Geom<SV_BF16, false>::kMaxGroups <= 2048,
              "the early stop's rounding margin assumes at most 2^11 super-groups");

struct DrawSmem {
    float gsum[kMaxGroupsAny];  // per super-group weight sums
    int next;                // next unclaimed super-group
    int tok;                 // the drawn id
    float total;             // W
    float done;              // known W: the sum of the super-groups finished so far
};

// Per-thread sum of 8 weights, in id order.
__device__ __forceinline__ float sum8(const float* w) {
    float s = w[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) s += w[k];
    return s;
}

struct DrawRow {
    const char* prow;
    const char* qrow;
    int vocab;
    bool aligned;  // both rows 16-byte aligned
    float c, ap, aq, rq;
};

// A super-group's raw words for one lane: U 8-id groups of each row.
template <sv_dtype DT, bool RESID>
struct GroupRaw {
    Raw8<DT> p[Geom<DT, RESID>::kU], q[Geom<DT, RESID>::kU];
};

template <sv_dtype DT, bool RESID>
__device__ __forceinline__ void group_fetch(const DrawRow& d, int g, int lane,
                                            GroupRaw<DT, RESID>& r) {
    const int e = g * Geom<DT, RESID>::kIds + lane * 8;
#pragma unroll
    for (int u = 0; u < Geom<DT, RESID>::kU; ++u) {
        r.p[u].fetch(d.prow, e + u * kWave * 8);
        if (RESID) r.q[u].fetch(d.qrow, e + u * kWave * 8);
    }
}

// This lane's share of super-group g: its U groups' weights summed in
// increasing id order.  `raw` holds the words when the group is fast.
template <sv_dtype DT, bool RESID>
__device__ __forceinline__ float group_lane_sum(const DrawRow& d, int g, int lane, bool fast,
                                                const GroupRaw<DT, RESID>& raw) {
    const int e = g * Geom<DT, RESID>::kIds + lane * 8;
    float acc = 0.0f;
#pragma unroll
    for (int u = 0; u < Geom<DT, RESID>::kU; ++u) {
        float zp[8], zq[8], w[8];
        if (fast) {
            raw.p[u].unpack(zp);
            if (RESID) raw.q[u].unpack(zq);
        } else {
            load8<DT>(d.prow, d.vocab, e + u * kWave * 8, d.aligned, zp);
            if (RESID) load8<DT>(d.qrow, d.vocab, e + u * kWave * 8, d.aligned, zq);
        }
        weights_from<RESID>(zp, zq, d.c, d.ap, d.aq, d.rq, w);
        acc += sum8(w);
    }
    return acc;
}

// Inverse-CDF draw over one row's weights (RESID: residual of two rows).
//  1. Sweep: the row is cut into super-groups of Geom::kIds ids; waves claim
//     them in turn from an LDS counter (the next one's loads in flight while
//     the current one is summed) and store each super-group's sum, a fixed
//     reduction order, in LDS.  No barrier inside the stream.
//  2. Wave 0 walks the sums in id order (a wave scan), W is their total and
//     the super-group where the running sum passes v * W is read once more,
//     Geom::kIdsPerLane consecutive ids per lane, to find the id.
// If rounding leaves v * W at or above the running total, the last id of
// positive weight is taken.  Only ids of positive weight are ever drawn.
// *mass gets W; returns -2 if W is not positive.
// w_known > 0 (a draw from one row whose total pass 1 has summed): W is
// w_known, so v * W is known before the sweep, and the waves stop claiming
// once the super-groups already finished sum past it with a margin that
// covers every rounding of both sums (claims go out in id order, so the
// crossing then lies among the claimed ones); the walk covers those.
template <sv_dtype DT, bool RESID>
__device__ int draw_row(const char* prow, const char* qrow, int vocab, float c, float ap,
                        float aq, float rq, float v, DrawSmem& sm, float* mass,
                        bool claims_ready = false, float w_known = 0.0f) {
    using G = Geom<DT, RESID>;
    constexpr int kGroupIds = G::kIds;
    constexpr int kIdsPerLane = G::kIdsPerLane;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    DrawRow d;
    d.prow = prow;
    d.qrow = qrow;
    d.vocab = vocab;
    d.aligned = ((reinterpret_cast<uintptr_t>(prow) | reinterpret_cast<uintptr_t>(qrow)) & 15) == 0;
    d.c = c;
    d.ap = ap;
    d.aq = aq;
    d.rq = rq;
    const int n_groups = (vocab + kGroupIds - 1) / kGroupIds;

    // ---- 1. sweep (claims_ready: sm.next and sm.done were set before a
    // barrier the caller has passed)
    const bool early = !RESID && w_known > 0.0f;
    // the finished super-groups' sum (in any order) and the walk's (in id
    // order) each lie within n_groups * 2^-24 of their exact sums, n_groups
    // <= 2^11: a finished sum above v W (1 + 2^-10) puts the walk's
    // running sum over the claimed super-groups above v W
    const float stop_at = v * w_known * (1.0f + 0x1p-10f);
    if (!claims_ready) {
        if (tid == 0) {
            sm.next = kP2Waves;
            sm.done = 0.0f;
        }
        __syncthreads();
    }
    {
        // super-groups [0, n_fast) lie wholly inside an aligned row: a tight
        // loop with two register buffers in turn; the rest (the row's last,
        // partial super-group, or every one of an unaligned row) element-wise
        const int n_fast = d.aligned ? (d.vocab & ~7) / kGroupIds : 0;
        auto claim = [&]() {
            int g2 = n_groups;  // no further claim
            if (lane == 0 &&
                (!early || __hip_atomic_load(&sm.done, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_WORKGROUP) <= stop_at))
                g2 = atomicAdd(&sm.next, 1);
            return __builtin_amdgcn_readfirstlane(g2);
        };
        auto publish = [&](int g, float gs) {
            if (lane == 0) {
                sm.gsum[g] = gs;
                if (early) atomicAdd(&sm.done, gs);
            }
        };
        int g = wave;  // the first claim of each wave is implicit
        GroupRaw<DT, RESID> ba, bb;
        if (g < n_fast) group_fetch<DT, RESID>(d, g, lane, ba);
        while (g < n_fast) {
            int g2 = claim();
            if (g2 < n_fast) group_fetch<DT, RESID>(d, g2, lane, bb);
            float gs = wave_sum_dpp(group_lane_sum<DT, RESID>(d, g, lane, true, ba), lane);
            publish(g, gs);
            g = g2;
            if (g >= n_fast) break;
            g2 = claim();
            if (g2 < n_fast) group_fetch<DT, RESID>(d, g2, lane, ba);
            gs = wave_sum_dpp(group_lane_sum<DT, RESID>(d, g, lane, true, bb), lane);
            publish(g, gs);
            g = g2;
        }
        while (g < n_groups) {
            const float gs = wave_sum_dpp(group_lane_sum<DT, RESID>(d, g, lane, false, ba), lane);
            publish(g, gs);
            g = claim();
        }
    }
    __syncthreads();

    // ---- 2. walk and second look (wave 0)
    if (wave == 0) {
        // the super-groups swept: every one below the claim counter (all of
        // them unless the sweep stopped early)
        const int n_swept = min(sm.next, n_groups);
        // lane l owns super-groups [l G, (l + 1) G), G = ceil(n_groups / 64)
        // (every lane a few, however long the row).  The running sum at a
        // super-group is its lane's base (an exclusive wave scan of the lane
        // sums) plus the lane's own super-groups up to it, in order: it
        // depends only on the super-groups at or before it, so an early stop
        // past the crossing changes nothing.
        const int gpl = (n_groups + kWave - 1) / kWave;
        const int g_lo = lane * gpl, g_hi = min(g_lo + gpl, n_swept);
        float lsum = 0.0f;
        int lastg = -1;  // the lane's last positive super-group
        for (int g = g_lo; g < g_hi; ++g) {
            const float x = sm.gsum[g];
            lsum += x;
            if (x > 0.0f) lastg = g;
        }
        const float incl = wave_incl_sum_dpp(lsum, lane);
        // the lane below's inclusive sum (DPP wave_shr:1; lane 0 reads 0)
        const float excl = __int_as_float(
            __builtin_amdgcn_update_dpp(0, __float_as_int(incl), 0x138, 0xf, 0xf, false));
        const float swept = lane63(incl);
        const float W = early ? w_known : swept;
        int tok = -2;
        if (W > 0.0f && swept > 0.0f) {
            const float tgt = v * W;
            // the first positive super-group whose running sum passes tgt
            float run = excl, fbase = 0.0f;
            int found = -1;
            for (int g = g_lo; g < g_hi; ++g) {
                const float x = sm.gsum[g];
                const float nr = run + x;
                if (found < 0 && x > 0.0f && nr > tgt) {
                    found = g;
                    fbase = run;
                }
                run = nr;
            }
            const uint64_t fm = __ballot(found >= 0);
            bool crossing = fm != 0;
            int hit;
            float hit_base = 0.0f;
            if (crossing) {
                const int hl = __builtin_ctzll(fm);
                hit = __builtin_amdgcn_readlane(found, hl);
                hit_base = readlane_t(fbase, hl);
            } else {  // rounding: the last positive id of the last positive super-group
                const uint64_t pm = __ballot(lastg >= 0);
                hit = __builtin_amdgcn_readlane(lastg, 63 - __builtin_clzll(pm));
            }
            // second look: lane l takes ids [g0 + l n, g0 + (l + 1) n), n = kIdsPerLane
            const int e0 = hit * kGroupIds + lane * kIdsPerLane;
            float wts[kIdsPerLane];
            float ls = 0.0f;
#pragma unroll
            for (int k8 = 0; k8 < kIdsPerLane / 8; ++k8) {
                float zp[8], zq[8];
                const int e = e0 + k8 * 8;
                if (e < vocab) {
                    load8<DT>(prow, vocab, e, d.aligned, zp);
                    if (RESID) load8<DT>(qrow, vocab, e, d.aligned, zq);
                    weights_from<RESID>(zp, zq, c, ap, aq, rq, wts + k8 * 8);
                } else {
#pragma unroll
                    for (int k = 0; k < 8; ++k) wts[k8 * 8 + k] = 0.0f;
                }
            }
#pragma unroll
            for (int k = 0; k < kIdsPerLane; ++k) ls += wts[k];
            const float li = wave_incl_sum_dpp(ls, lane);
            float r2 = hit_base + (li - ls);
            int cand = 0x7fffffff, lastpos = -1;
#pragma unroll
            for (int k = 0; k < kIdsPerLane; ++k) {
                r2 += wts[k];
                // Only an id of positive weight can be drawn: the second look and
                // the sweep round differently, so a lane may start above v * W;
                // its first positive id is then the crossing.
                const bool positive = wts[k] > 0.0f;
                if (crossing && positive && r2 > tgt && cand == 0x7fffffff) cand = e0 + k;
                if (positive) lastpos = e0 + k;
            }
            const uint64_t mc = __ballot(cand != 0x7fffffff);
            const uint64_t ml = __ballot(lastpos >= 0);
            if (mc)
                tok = __builtin_amdgcn_readlane(cand, __builtin_ctzll(mc));
            else if (ml)
                tok = __builtin_amdgcn_readlane(lastpos, 63 - __builtin_clzll(ml));
            else
                tok = -1;  // unreachable: the group's sum was positive
        }
        if (lane == 0) {
            sm.tok = tok;
            sm.total = W;
        }
    }
    __syncthreads();
    const int tok = sm.tok;
    *mass = sm.total;
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
        if (a.out_qh) a.out_qh[(int64_t)r * a.k_max + j] = -1.0f;
        if (a.out_qm) a.out_qm[(int64_t)r * a.k_max + j] = -1.0f;
    }
    if (tid == 0) {
        a.out_accepted[r] = -1;
        if (a.out_resid) a.out_resid[r] = -1.0f;
        raise_error(a.dev_error, bits);
    }
}

// Statistics of one row, merged from its parts.
struct RowMerged {
    float A, S;      // stochastic: offset and sum over the row
    float pd, lpd;   // stochastic: p(d) and log2 p(d) of the position's draft id
    float mx;        // greedy: the row's max logit
    int idx;         // greedy: lowest id reaching it
    float ent, pmax; // stochastic draft row with features: entropy (bits), largest probability
    bool fault;      // NaN or +inf somewhere, or no finite mass
};

// One row's part records, loaded into registers (parts of them).
struct RowParts {
    PartStat p[kMaxParts];
    __device__ __forceinline__ void load(const PartStat* ps, int parts) {
#pragma unroll
        for (int h = 0; h < kMaxParts; ++h)
            if (h < parts) p[h] = ps[h];
    }
};
struct RowFeats {
    FeatPart f[kMaxParts];
    __device__ __forceinline__ void load(const FeatPart* fs, int parts) {
#pragma unroll
        for (int h = 0; h < kMaxParts; ++h)
            if (h < parts) f[h] = fs[h];
    }
};

// Merge the parts of one row in part order (deterministic).  d: the draft id
// whose probability is wanted, or -1.  feat: also the draft-row features, from
// the row's feature records fs.
template <bool GREEDY>
__device__ __forceinline__ RowMerged merge_parts(const RowParts& rp, int parts, int plen, int d,
                                                 float c, bool feat = false,
                                                 const RowFeats& fs = RowFeats{}) {
    const PartStat* p = rp.p;
    RowMerged m;
    m.A = -kInf;
    m.S = 0.0f;
    m.pd = -1.0f;
    m.lpd = -kInf;
    m.mx = -kInf;
    m.idx = 0x7fffffff;
    m.ent = -1.0f;
    m.pmax = -1.0f;
    m.fault = false;
    if (GREEDY) {
#pragma unroll
        for (int h = 0; h < kMaxParts; ++h) {
            if (h >= parts) break;
            if (p[h].idx < 0) m.fault = true;                   // a NaN in the part
            if (p[h].a > m.mx) {                                 // first part wins ties
                m.mx = p[h].a;
                m.idx = p[h].idx;
            }
        }
        if (m.mx == kInf || m.mx == -kInf) m.fault = true;
        return m;
    }
#pragma unroll
    for (int h = 0; h < kMaxParts; ++h) {
        if (h >= parts) break;
        if (!(p[h].s >= 0.0f)) {
            m.fault = true;  // NaN or +inf in the part
        } else if (p[h].s > 0.0f) {
            if (m.S == 0.0f) {
                m.A = p[h].a;
                m.S = p[h].s;
            } else {
                merge_as(m.A, m.S, p[h].a, p[h].s);
            }
        }
    }
    if (!(m.S > 0.0f) || !is_finite_bits(m.S) || !is_finite_bits(m.A)) m.fault = true;
    if (d >= 0 && !m.fault) {
        // part d / plen holds d's logit; its scaled log-probability is finite
        // even where p(d) is an fp32 subnormal or zero
        const int hd = d / plen;
        float zd = 0.0f;
#pragma unroll
        for (int h = 0; h < kMaxParts; ++h)
            if (h == hd) zd = p[h].zd;
        const float y = fmaf(zd, c, -m.A);
        m.pd = exp2f(y) / m.S;
        m.lpd = y - log2f(m.S);
    }
    if (feat && !m.fault) {
        // entropy = log2 S - E / S with E = sum_x 2^(y_x - A) (y_x - A): each
        // part's e moved to the row's offset A (parts without mass add nothing)
        float e = 0.0f, mx = -kInf;
#pragma unroll
        for (int h = 0; h < kMaxParts; ++h) {
            if (h >= parts) break;
            if (p[h].s > 0.0f) {
                const FeatPart f = fs.f[h];
                e += scale_exp2(fmaf(p[h].a - m.A, p[h].s, f.e), p[h].a - m.A);
                mx = fmaxf(mx, f.mx);
            }
        }
        m.ent = fmaxf(0.0f, log2f(m.S) - e / m.S);
        m.pmax = exp2f(fmaf(mx, c, -m.A)) / m.S;
    }
    return m;
}

struct FinishSmem {
    DrawSmem draw;
    float ta[kWave], ts[kWave], qa[kWave], qs[kWave];  // merged rows of position j
    float tpd[kWave], qpd[kWave];                      // p(d_j), q(d_j)
    float qh[kWave], qm[kWave];                        // draft row j's features
    int gidx[kWave];                                   // greedy: argmax of target row j
    float ba, bs;                                      // bonus row b (stochastic)
    int bidx;                                          // bonus row b (greedy)
    float v;                                           // the draw's uniform (position L)
    int L, b, lo, fault;
};

template <sv_dtype DT, bool GREEDY>
__device__ void finish_request(const Args& a, int r, FinishSmem& sm) {
    const int tid = threadIdx.x;
    const int k_max = a.k_max;
    const int parts = a.parts, plen = part_len(a.vocab, parts);
    const PartStat* st = a.stats + (int64_t)r * (2 * k_max + 1) * kMaxParts;
    if (tid < kWave) {
        // lane j: position j (target row j and draft row j); lane b also
        // merges the bonus row (target row b).  Every load this wave needs is
        // issued before the offsets are checked: the draft id and the part
        // records of target row j and draft row j do not depend on them.
        const int lane = tid, j = lane;
        const bool feat = !GREEDY && (a.out_qh != nullptr || a.out_qm != nullptr);
        const int lo = a.cu_rows[r], hi = a.cu_rows[r + 1];
        const int d = j < k_max ? a.draft_tokens[(int64_t)r * k_max + j] : -1;
        RowParts tp, qp;
        RowFeats fq;
        if (j <= k_max) tp.load(st + (int64_t)j * kMaxParts, parts);
        if (!GREEDY && j < k_max) qp.load(st + (int64_t)(k_max + 1 + j) * kMaxParts, parts);
        if (feat && j < k_max) fq.load(a.feat + ((int64_t)r * k_max + j) * kMaxParts, parts);
        float u = 0.0f, v = 0.0f;
        if (!GREEDY) draw_uniforms(a.seed, a.step, (uint32_t)r, (uint32_t)j, &u, &v);
        const int b = hi - lo - 1;
        int fault = 0;
        bool acc = true;
        if (lo < 0 || b < 0 || b > k_max || (int64_t)hi > a.target_rows) {
            fault = SV_DEV_BAD_CU_ROWS;
        } else {
            if (j < b) {
                const bool d_ok = d >= 0 && d < a.vocab;
                if (!d_ok) fault |= SV_DEV_BAD_TOKEN;
                const RowMerged t = merge_parts<GREEDY>(tp, parts, plen, d_ok ? d : -1, a.c);
                if (t.fault) fault |= SV_DEV_NONFINITE;
                if (GREEDY) {
                    acc = t.idx == d;
                    sm.gidx[j] = t.idx;
                } else {
                    const RowMerged q =
                        merge_parts<false>(qp, parts, plen, d_ok ? d : -1, a.c, feat, fq);
                    if (q.fault) fault |= SV_DEV_NONFINITE;
                    // u < min(1, p/q), the ratio taken from log2 p - log2 q so that
                    // probabilities below fp32's normal range do not decide it
                    acc = u < exp2f(t.lpd - q.lpd);
                    sm.ta[j] = t.A;
                    sm.ts[j] = t.S;
                    sm.qa[j] = q.A;
                    sm.qs[j] = q.S;
                    sm.tpd[j] = t.pd;
                    sm.qpd[j] = q.pd;
                    sm.qh[j] = q.ent;
                    sm.qm[j] = q.pmax;
                }
            }
            // the bonus row b: lane b's own target records (a wave has 64
            // lanes, so b = 64 is loaded here by lane 0)
            const bool bonus_lane = b < kWave ? j == b : j == 0;
            if (bonus_lane) {
                if (b >= kWave) tp.load(st + (int64_t)b * kMaxParts, parts);
                const RowMerged t = merge_parts<GREEDY>(tp, parts, plen, -1, a.c);
                if (t.fault) fault |= SV_DEV_NONFINITE;
                sm.ba = t.A;
                sm.bs = t.S;
                sm.bidx = t.idx;
            }
        }
        fault = wave_or_int(fault);
        const uint64_t rej = __ballot(!acc);
        const int L = rej ? __builtin_ctzll(rej) : b;
        if (!GREEDY && j == L) sm.v = v;  // L = 64 (every draft of 64 kept) draws it below
        if (lane == 0) {
            sm.L = L;
            sm.b = b;
            sm.lo = lo;
            sm.fault = fault;
            if (!GREEDY) {
                sm.draw.next = kP2Waves;  // the draw's first claims are implicit
                sm.draw.done = 0.0f;
            }
        }
        // Every output the draw does not decide is written now, by the lane of
        // its position: the accepted drafts, the -1 after L, the per-position
        // probabilities and features, and L.  The token at L follows the draw
        // (a fault found later overwrites all of them).
        if (!fault) {
            int32_t* tok_out = a.out_tokens + (int64_t)r * (k_max + 1);
            if (j <= k_max && j != L) tok_out[j] = j < L ? d : -1;
            if (j == 0 && k_max == kWave && L != kWave) tok_out[kWave] = -1;
            if (j < k_max) {
                const bool has = !GREEDY && j < b;
                const int64_t o = (int64_t)r * k_max + j;
                if (a.out_p) a.out_p[o] = has ? sm.tpd[j] : -1.0f;
                if (a.out_q) a.out_q[o] = has ? sm.qpd[j] : -1.0f;
                if (a.out_qh) a.out_qh[o] = has ? sm.qh[j] : -1.0f;
                if (a.out_qm) a.out_qm[o] = has ? sm.qm[j] : -1.0f;
            }
            if (j == 0) a.out_accepted[r] = L;
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
        token = L < b ? sm.gidx[L] : sm.bidx;
    } else {
        float v = sm.v;
        if (L >= kWave) {
            float u;
            draw_uniforms(a.seed, a.step, (uint32_t)r, (uint32_t)L, &u, &v);
        }
        const char* prow = a.target + ((int64_t)lo + L) * a.target_ld_bytes;
        if (L < b) {
            const float tA = sm.ta[L], tS = sm.ts[L];
            const char* qrow = a.draft + ((int64_t)r * k_max + L) * a.draft_ld_bytes;
            token = draw_row<DT, true>(prow, qrow, a.vocab, a.c, tA, sm.qa[L], tS / sm.qs[L], v,
                                       sm.draw, &mass, true);
            mass /= tS;  // the residual's weights are in units of 1 / S_p
            if (token == -2) {  // zero residual mass: draw from p instead
                float unused;
                token = draw_row<DT, false>(prow, prow, a.vocab, a.c, tA, 0.0f, 1.0f, v, sm.draw,
                                            &unused, false, tS);
            }
        } else {
            float unused;
            token = draw_row<DT, false>(prow, prow, a.vocab, a.c, sm.ba, 0.0f, 1.0f, v, sm.draw,
                                        &unused, true, sm.bs);
        }
    }
    if (token < 0) {  // no id carries weight: only reachable through a numeric fault
        emit_fault(a, r, SV_DEV_NONFINITE);
        return;
    }
    if (tid == 0) {
        a.out_tokens[(int64_t)r * (k_max + 1) + L] = token;
        if (a.out_resid) a.out_resid[r] = (!GREEDY && L < b) ? mass : -1.0f;
    }
}

// ------------------------------------------------------------------ kernels

// Pass-1 workgroup g -> (request, slot).  Groups of n workgroups run the same
// row kind for every request.  Slots: target j = j, draft j = k_max + 1 + j.
#ifndef SV_PASS1_ASCENDING
#define SV_PASS1_ASCENDING 1
#endif
__device__ __forceinline__ void pass1_slot(int g, int n_req, int k_max, bool greedy, int* r,
                                           int* slot) {
    const int grp = g / n_req;
    *r = g - grp * n_req;
#if SV_PASS1_ASCENDING
    // position 0 first: every request verifies its low positions, so the
    // workgroups that find no row (positions past a request's budget) come
    // last, where they overlap the tail instead of delaying the stream
    if (greedy) {
        *slot = grp;
        return;
    }
    const int j = grp >> 1;
    *slot = (grp & 1) == 0 ? j : k_max + 1 + j;
#else
    // target K first, then for j = K-1 .. 0 draft row j and target row j
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
#endif
}

// Dense pass-1 order: with well-formed row offsets (cu_rows[0] = 0, every
// kept count in [0, k_max], the last offset within target_rows) workgroup u
// takes the u-th existing row part — target rows in packed order, then draft
// rows request by request — found by a binary search of the offsets staged in
// LDS, so every workgroup past the kept rows sits at the end of the grid.
// Other offsets (and batches above kDenseMaxReq requests) keep the
// (position, request) order of pass1_slot, whose checks reject bad offsets
// request by request.
#ifndef SV_PASS1_DENSE
#define SV_PASS1_DENSE 1
#endif
constexpr int kDenseMaxReq = 512;  // each workgroup stages n + 1 offsets

// Largest i in [0, n] with key(i) <= x, key non-decreasing and key(0) <= x:
// two wave-wide steps (each lane tests one candidate, a ballot counts).
template <typename Key>
__device__ __forceinline__ int last_at_most(int n, int x, Key key) {
    const int lane = threadIdx.x & (kWave - 1);
    const int step = (n + kWave) / kWave;  // 64 * step > n
    int i1 = lane * step;
    const uint64_t m1 = __ballot(i1 <= n && key(i1 <= n ? i1 : n) <= x);
    const int base = (__popcll(m1) - 1) * step;  // key(base) <= x < key(base + step)
    const int i2 = base + lane;
    const uint64_t m2 = __ballot(lane < step && i2 <= n && key(i2 <= n ? i2 : n) <= x);
    return base + __popcll(m2) - 1;
}

template <sv_dtype DT, bool GREEDY, bool FEAT>
__global__ __launch_bounds__(pass1_threads<GREEDY>()) void rowstats_kernel(Args a, int n_req,
                                                                          int parts) {
    constexpr int T = pass1_threads<GREEDY>();
    __shared__ float redf[4 * (T / kWave)];
    __shared__ int redi[2 * (T / kWave)];
    __shared__ int32_t cu_s[SV_PASS1_DENSE ? kDenseMaxReq + 1 : 1];
    const int h = blockIdx.x % parts;
    int r, slot, lo, hi;
    bool dense = false;
    if (SV_PASS1_DENSE && n_req <= kDenseMaxReq) {
        // one barrier: each thread checks the offsets it stages
        int bad = 0;
        for (int i = threadIdx.x; i <= n_req; i += T) {
            const int v = a.cu_rows[i];
            cu_s[i] = v;
            if (i == 0) bad |= v != 0;
            if (i == n_req) bad |= (int64_t)v > a.target_rows;
            if (i < n_req) {
                const int b = a.cu_rows[i + 1] - v - 1;
                bad |= b < 0 || b > a.k_max;
            }
        }
        dense = !__syncthreads_or(bad);
    }
    if (dense) {
        const int unit = blockIdx.x / parts;
        const int rows_t = cu_s[n_req], rows_d = rows_t - n_req;
        if (unit < rows_t) {  // target row `unit`
            r = last_at_most(n_req, unit, [&](int i) { return cu_s[i]; });
            slot = unit - cu_s[r];
        } else if (!GREEDY && unit < rows_t + rows_d) {  // draft row `unit - rows_t`
            const int d = unit - rows_t;
            r = last_at_most(n_req, d, [&](int i) { return cu_s[i] - i; });
            slot = a.k_max + 1 + (d - (cu_s[r] - r));
        } else {
            return;
        }
        lo = cu_s[r];
        hi = cu_s[r + 1];
    } else {
        pass1_slot(blockIdx.x / parts, n_req, a.k_max, GREEDY, &r, &slot);
        lo = a.cu_rows[r];
        hi = a.cu_rows[r + 1];
    }
    const int b = hi - lo - 1;
    if (lo < 0 || b < 0 || b > a.k_max || (int64_t)hi > a.target_rows) return;
    const bool is_draft = slot > a.k_max;
    const int j = is_draft ? slot - a.k_max - 1 : slot;
    if (is_draft ? (j >= b) : (j > b)) return;
    const char* row = is_draft ? a.draft + ((int64_t)r * a.k_max + j) * a.draft_ld_bytes
                               : a.target + ((int64_t)lo + j) * a.target_ld_bytes;
    // this workgroup's part of the row: ids [p0, p1)
    const int plen = part_len(a.vocab, parts);
    const int p0 = min(a.vocab, h * plen), p1 = min(a.vocab, p0 + plen);
    const char* prow = row + (int64_t)p0 * Vec<DT>::kBytes;
    PartStat* out = a.stats + ((int64_t)r * (2 * a.k_max + 1) + slot) * kMaxParts + h;
    if (GREEDY) {
        float mx;
        int idx;
        bool nan;
        row_argmax<DT, kGreedyThreads, kGreedyUnroll>(prow, p1 - p0, redf, redi, &mx, &idx, &nan);
        if (threadIdx.x == 0) {
            PartStat st{};
            st.a = mx;
            st.idx = nan ? -1 : (idx == 0x7fffffff ? idx : p0 + idx);
            *out = st;
        }
        return;
    }
    // the draft id's logit: fetched by thread 0 inside the stream (ids are
    // checked in pass 2; one outside [0, vocab) is never in a part)
    const int32_t* dtok = j < b ? a.draft_tokens + (int64_t)r * a.k_max + j : nullptr;
    float zd = 0.0f;  // in thread 0, and only if the id lies in [p0, p1)
    float A, S;
    FeatAcc fa;
    if (FEAT && is_draft)
        row_stats_stochastic<DT, true>(prow, p1 - p0, a.c, redf, &A, &S, &fa, dtok, &zd,
                                       p0);
    else
        row_stats_stochastic<DT>(prow, p1 - p0, a.c, redf, &A, &S, nullptr, dtok, &zd,
                                 p0);
    if (FEAT && is_draft && threadIdx.x == 0) {
        FeatPart f;
        f.e = fa.e;
        f.mx = fa.mx;
        a.feat[((int64_t)r * a.k_max + j) * kMaxParts + h] = f;
    }
    if (threadIdx.x == 0) {
        // S is NaN or +inf for a faulty part, 0 (A = -inf) for one without mass
        const bool fault = !(S >= 0.0f) || !is_finite_bits(S) || (S > 0.0f && !is_finite_bits(A));
        PartStat st;
        st.a = fault ? 0.0f : A;
        st.s = fault ? -1.0f : S;
        st.zd = zd;
        st.idx = 0;
        *out = st;
    }
}

template <sv_dtype DT, bool GREEDY>
__global__ __launch_bounds__(GREEDY ? kWave : kP2Threads) void decide_kernel(Args a) {
    __shared__ FinishSmem fin;
    finish_request<DT, GREEDY>(a, blockIdx.x, fin);
}

size_t stats_bytes(int n_req, int k_max) {
    return (size_t)n_req * (size_t)(2 * k_max + 1) * kMaxParts * sizeof(PartStat);
}

int host_row_parts(int vocab, bool greedy) {
    const int ids = greedy ? kGreedyPartIds : kPartIds;
    const int h = (vocab + ids - 1) / ids;
    return h < 1 ? 1 : (h > kMaxParts ? kMaxParts : h);
}

template <sv_dtype DT, bool GREEDY>
hipError_t launch_typed(const VerifyArgs& v, hipStream_t stream) {
    const int esize = Vec<DT>::kBytes;
    // draft-row features exist only where draft rows are read (stochastic)
    const bool feat = !GREEDY && (v.out_q_entropy != nullptr || v.out_q_max != nullptr);
    const int parts = host_row_parts(v.vocab, GREEDY);
    Args a{static_cast<const char*>(v.target), v.target_ld * esize, v.target_rows,
           static_cast<const char*>(v.draft), v.draft_ld * esize, v.vocab, v.draft_tokens,
           v.cu_rows, v.k_max, parts, kLog2e / v.temperature, v.seed, v.step,
           static_cast<PartStat*>(v.ws),
           reinterpret_cast<FeatPart*>(static_cast<char*>(v.ws) + stats_bytes(v.n_req, v.k_max)),
           v.out_tokens, v.out_accepted, v.out_p_draft, v.out_q_draft, v.out_residual_mass,
           v.out_q_entropy, v.out_q_max, v.dev_error};  // greedy: -1 written there
    const int slots = GREEDY ? v.k_max + 1 : 2 * v.k_max + 1;
    if (v.stages & 1) {
        const dim3 grid((unsigned)((int64_t)v.n_req * slots * parts));  // < 2^23 (host-checked)
        if constexpr (GREEDY)
            hipLaunchKernelGGL((rowstats_kernel<DT, true, false>), grid, dim3(kGreedyThreads), 0, stream,
                               a, v.n_req, parts);
        else if (feat)
            hipLaunchKernelGGL((rowstats_kernel<DT, false, true>), grid, dim3(kThreads), 0, stream,
                               a, v.n_req, parts);
        else
            hipLaunchKernelGGL((rowstats_kernel<DT, false, false>), grid, dim3(kThreads), 0,
                               stream, a, v.n_req, parts);
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
    return stats_bytes(n_req, k_max) + (size_t)n_req * (size_t)k_max * kMaxParts * sizeof(FeatPart);
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
