// Device-side helpers shared by the libspecverify kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "libspecverify.h"

namespace sv {

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw v_exp_f32: 2^x, 1 ulp, flushes results below 2^-126 (terms that small
// do not change an fp32 sum that holds a term >= 1).
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Bit-level classification (independent of any fast-math assumptions).
__device__ __forceinline__ bool is_nan_bits(float x) {
    return (__float_as_uint(x) & 0x7fffffffu) > 0x7f800000u;
}
__device__ __forceinline__ bool is_finite_bits(float x) {
    return (__float_as_uint(x) & 0x7fffffffu) < 0x7f800000u;
}

// Whole-wave reductions, every lane gets the result.  They go through the DPP
// scan below (a few cycles a step) rather than LDS permutes (hundreds of
// cycles a dependent step when the waves of a workgroup all reduce at once).
template <typename T>
__device__ __forceinline__ T wave_sum(T v);
__device__ __forceinline__ float wave_max(float v);
__device__ __forceinline__ int wave_or_int(int v);

// ------------------------------------------------------------ DPP lane moves
// Cross-lane moves through the VALU's data-parallel-primitive path (a few
// cycles) instead of LDS permutes.  gfx9 DPP controls: row_shr:n = 0x110 + n
// (lane i of each 16-lane row reads lane i - n of that row), row_bcast:15 =
// 0x142 (lane 15 of each row feeds the next row), row_bcast:31 = 0x143
// (lane 31 feeds rows 2 and 3).  Lanes whose source is outside the row, or
// whose row is masked off, read 0; every caller below ignores those lanes.
// All 64 lanes must be active.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK, typename T>
__device__ __forceinline__ T dpp_move_t(T v) {
    static_assert(sizeof(T) % 4 == 0, "32-bit words");
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) w[i] = dpp_move<CTRL, ROW_MASK>(w[i]);
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}

// Value of lane 63, in every lane.
template <typename T>
__device__ __forceinline__ T lane63(T v) {
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) w[i] = __builtin_amdgcn_readlane(w[i], 63);
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}

// Value of lane `src` (the same in every lane), in every lane.
template <typename T>
__device__ __forceinline__ T readlane_t(T v, int src) {
    uint32_t w[sizeof(T) / 4];
    __builtin_memcpy(w, &v, sizeof(T));
    const int l = __builtin_amdgcn_readfirstlane(src);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) w[i] = __builtin_amdgcn_readlane(w[i], l);
    T r;
    __builtin_memcpy(&r, w, sizeof(T));
    return r;
}

// Inclusive scan over the 64 lanes, op(earlier, later) associative; a fixed
// combination order (deterministic).  Lane 63 ends with the whole-wave value.
template <typename T, typename Op>
__device__ __forceinline__ T wave_scan_dpp(T v, int lane, Op op) {
    const int rl = lane & 15;
    T t;
    t = dpp_move_t<0x111, 0xf>(v);
    if (rl >= 1) v = op(t, v);
    t = dpp_move_t<0x112, 0xf>(v);
    if (rl >= 2) v = op(t, v);
    t = dpp_move_t<0x114, 0xf>(v);
    if (rl >= 4) v = op(t, v);
    t = dpp_move_t<0x118, 0xf>(v);
    if (rl >= 8) v = op(t, v);
    t = dpp_move_t<0x142, 0xa>(v);
    if (lane & 16) v = op(t, v);
    t = dpp_move_t<0x143, 0xc>(v);
    if (lane & 32) v = op(t, v);
    return v;
}

struct AddOp {
    template <typename T>
    __device__ __forceinline__ T operator()(T a, T b) const { return a + b; }
};

template <typename T>
__device__ __forceinline__ T wave_incl_sum_dpp(T v, int lane) {
    return wave_scan_dpp(v, lane, AddOp{});
}

// Whole-wave sum, in every lane.
template <typename T>
__device__ __forceinline__ T wave_sum_dpp(T v, int lane) {
    return lane63(wave_scan_dpp(v, lane, AddOp{}));
}

struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct OrOp {
    __device__ __forceinline__ int operator()(int a, int b) const { return a | b; }
};

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
    return wave_sum_dpp(v, (int)__lane_id());
}

__device__ __forceinline__ float wave_max(float v) {
    return lane63(wave_scan_dpp(v, (int)__lane_id(), MaxOp{}));
}

__device__ __forceinline__ int wave_or_int(int v) {
    return lane63(wave_scan_dpp(v, (int)__lane_id(), OrOp{}));
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC'11, section 3): per round the products of the two
// multipliers with counter words 0 and 2 are split in high and low halves,
// the new counter is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0), and the key
// advances by the Weyl constants.
struct Philox4 {
    uint32_t x0, x1, x2, x3;
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
    constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        const uint32_t hi0 = __umulhi(kMul0, c0), lo0 = kMul0 * c0;
        const uint32_t hi1 = __umulhi(kMul1, c2), lo1 = kMul1 * c2;
        const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
        c0 = n0;
        c1 = lo1;
        c2 = n2;
        c3 = lo0;
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    return {c0, c1, c2, c3};
}

// Uniforms of (request, position, step): u from word 0, v from word 1, each
// the top 24 bits scaled by 2^-24 (exact in fp32).
__device__ __forceinline__ void draw_uniforms(uint64_t seed, uint64_t step, uint32_t req,
                                              uint32_t pos, float* u, float* v) {
    const Philox4 w = philox4x32_10(req, pos, (uint32_t)step, (uint32_t)(step >> 32),
                                    (uint32_t)seed, (uint32_t)(seed >> 32));
    *u = (float)(w.x0 >> 8) * 0x1p-24f;
    *v = (float)(w.x1 >> 8) * 0x1p-24f;
}

__device__ __forceinline__ void raise_error(int32_t* dev_error, int bits) {
    if (dev_error != nullptr && bits) atomicOr(dev_error, bits);
}

}  // namespace sv
