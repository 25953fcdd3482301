// sq_device.h -- device helpers shared by the library's HIP kernels (gfx950).
//
// Element types, 16-byte vector loads, the symmetric 8-bit quantiser and
// wavefront/workgroup max reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- dtypes

struct F32 {
    typedef float T;
    static constexpr int VEC = 4;  // elements per 16 bytes
    __device__ static float to_f32(T v) { return v; }
    __device__ static T from_f32(float f) { return f; }
};

struct F16 {
    typedef _Float16 T;
    static constexpr int VEC = 8;
    __device__ static float to_f32(T v) { return (float)v; }         // exact
    __device__ static T from_f32(float f) { return (_Float16)f; }    // round to nearest even
};

struct BF16 {
    typedef uint16_t T;  // raw bits
    static constexpr int VEC = 8;
    __device__ static float to_f32(T v) { return __uint_as_float((uint32_t)v << 16); }  // exact
    // Round to nearest, ties to even, on the bit pattern (finite inputs).
    __device__ static T from_f32(float f) {
        uint32_t u = __float_as_uint(f);
        u += 0x7FFFu + ((u >> 16) & 1u);
        return (T)(u >> 16);
    }
};

// Load VEC consecutive elements (16 bytes, 16-byte aligned) widened to fp32.
template <class D>
__device__ inline void load_vec(const typename D::T* p, float (&out)[D::VEC]) {
    const uint4 raw = *reinterpret_cast<const uint4*>(p);
    const typename D::T* e = reinterpret_cast<const typename D::T*>(&raw);
#pragma unroll
    for (int i = 0; i < D::VEC; ++i) out[i] = D::to_f32(e[i]);
}

// Keeps v's fp32 rounding: without it the compiler merges a multiply, add or
// FMA with a following fp16 conversion into one mixed-precision FMA that
// rounds the exact value once to fp16 (a different result at fp16 ties).
__device__ inline void pin_f32(float& v) { __asm__("" : "+v"(v)); }

// ------------------------------------------------------------- quantiser
// step = absmax / 127 (fp32 IEEE division); code = clamp(round half away
// from zero (v / step), -127, 127); a zero step gives code 0.  These helpers
// are also built for the host, where a CPU test replays them against the
// IEEE quotient.
__host__ __device__ inline float quant_step(float absmax) { return absmax / 127.0f; }

// Rounding half away from zero as one addition and the truncating
// conversion: t + copysign(0.5 - 2^-25, t), rounded to nearest in fp32, has
// round(t) as its integer part for every fp32 t (the constant, not 0.5, keeps
// t = 0.5 - 2^-25 from rounding up to 1; beyond 127 the clamp decides, and
// NaN gives -127 as fmax(NaN, -127) does).  Four vector instructions
// (bit-insert, add, med3, convert) against eight for roundf and the clamp;
// the host test checks every fp32 bit pattern against roundf.
__host__ __device__ inline int code_from_quotient(float t) {
    float r = t + __builtin_copysignf(0.5f - 0x1p-25f, t);
    r = __builtin_fminf(__builtin_fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

__host__ __device__ inline int quant_code(float v, float step) {
    if (step == 0.0f) return 0;
    return code_from_quotient(v / step);
}

// One step shared by a whole row: the quotient v / step is needed for every
// element, so the correctly rounded reciprocal y = 1 / step is computed once
// and each quotient is formed by Markstein's correction
//   q0 = RN(v * y),  r = v - q0 * step (exact, one FMA),  q = RN(q0 + r * y),
// which equals the IEEE quotient RN(v / step) when y = RN(1 / step) and no
// intermediate leaves the normal range (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990; correctness proofs by Cornea-Hasegan, Golliver and
// Markstein, ARITH-14, 1999).  Steps outside [2^-96, 2^96] use the plain
// IEEE division instead.
//
// A step fixed in advance (the static per-tensor step) meets values far
// beyond 127 steps, and v * y may then overflow to infinity, which turns the
// correction into inf - inf = NaN.  Such callers saturate v to +-128 steps
// first (lim = 128 * step, exact: a power-of-two multiple of a step in
// [2^-96, 2^96]): a value beyond it has the code +-127 either way, and the
// quotient of the saturated value is exactly +-128, so the sign survives.
struct RowStep {
    float step, rcp, lim;
    bool fast;
};

// Quantiser parameters for a given step.
__host__ __device__ inline RowStep given_step(float step) {
    RowStep q;
    q.step = step;
    q.fast = step >= 0x1p-96f && step <= 0x1p96f;
    q.rcp = q.fast ? 1.0f / step : 0.0f;
    q.lim = q.fast ? 128.0f * step : 0.0f;
    return q;
}

// ... and for the step absmax / 127 of a row's maximum.
__host__ __device__ inline RowStep row_step(float absmax) { return given_step(quant_step(absmax)); }

// FAST: the caller has checked q.fast (a row-uniform branch taken once).
// SAT: v may lie beyond 128 steps (a step not taken from v's own row).
template <bool FAST, bool SAT = false>
__host__ __device__ inline int quant_code(float v, const RowStep& q) {
    if (q.step == 0.0f) return 0;
    float t;
    if constexpr (FAST) {
        if constexpr (SAT) v = __builtin_fminf(__builtin_fmaxf(v, -q.lim), q.lim);
        const float q0 = v * q.rcp;
        const float r = __builtin_fmaf(-q0, q.step, v);
        t = __builtin_fmaf(r, q.rcp, q0);
    } else {
        t = v / q.step;
    }
    return code_from_quotient(t);
}

// ------------------------------------------------------------ reductions
// Max over the 64 lanes, the same value in every lane: DPP rotations within
// each row of 16 lanes, then the four row results through scalar registers
// (no LDS round trips, unlike a shuffle).
__device__ inline float wave_max_dpp(float v) {
    int x = __float_as_int(v);
    v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x128, 0xF, 0xF, false)));
    x = __float_as_int(v);
    v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x124, 0xF, 0xF, false)));
    x = __float_as_int(v);
    v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x122, 0xF, 0xF, false)));
    x = __float_as_int(v);
    v = __builtin_fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(x, x, 0x121, 0xF, 0xF, false)));
    x = __float_as_int(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(x, 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(x, 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(x, 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(x, 48));
    return __builtin_fmaxf(__builtin_fmaxf(a, b), __builtin_fmaxf(c, d));
}

__device__ inline float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// Max over the workgroup; every thread gets the result.  `red` holds one
// float per wave.  Contains __syncthreads().
template <int NT>
__device__ inline float block_max(float v, float* red) {
    constexpr int NW = NT / 64;
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = __builtin_fmaxf(r, red[w]);
    __syncthreads();
    return r;
}

// Non-negative floats order like their bit patterns as unsigned integers, so
// an unsigned atomic max is an exact, order-independent float max for them.
__device__ inline void atomic_max_nonneg(float* addr, float v) {
    atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

}  // namespace sq
