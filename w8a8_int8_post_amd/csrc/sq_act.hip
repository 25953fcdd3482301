// sq_act.hip -- per-token dynamic activation quantisation on gfx950.
//
// P1 = abeam.tech explainer of "SmoothQuant: Accurate and Efficient
// Post-Training Quantization for Large Language Models", section 推論方法
// (O1: activations quantised per token, dynamically) and section
// 数学的に何をしているのか (X diag(s)^-1 when the scale is not folded).
//
// One or more wavefronts per token row.  Each lane keeps its slice of the row
// in registers between the absmax reduction and the quantisation, so the row
// is read from HBM once; loads are 16 bytes per lane and consecutive lanes
// read consecutive 16-byte pieces of the row.  Many rows (prefill) take one
// wavefront each, or share one when a row has at most 64 pieces (the
// head_dim-long rows of attention), reduced without LDS; few rows (decode)
// are spread over up to 16 wavefronts.  Rows whose length is not a multiple of 16 bytes, or
// longer than the register budget, take a two-pass variant (the second pass
// re-reads the row).
#include <type_traits>

#include "sq_device.h"
#include "sq_launch.h"

namespace sq {
namespace {

template <class D, bool SMOOTH>
__device__ inline void load_smoothed(const typename D::T* p, const float* smooth, int64_t k,
                                     float (&v)[D::VEC]) {
    load_vec<D>(p, v);
    if constexpr (SMOOTH) {
#pragma unroll
        for (int e = 0; e < D::VEC; e += 4) {
            const float4 s4 = *reinterpret_cast<const float4*>(smooth + k + e);
            v[e] = v[e] / s4.x;
            v[e + 1] = v[e + 1] / s4.y;
            v[e + 2] = v[e + 2] / s4.z;
            v[e + 3] = v[e + 3] / s4.w;
        }
    }
}

// dst2 (nullable): a second place for the same codes (the fragment-packed copy).
template <bool FAST, int V, bool SAT = false>
__device__ inline void store_codes(int8_t* dst, const float (&v)[V], const RowStep& step,
                                   int8_t* dst2 = nullptr) {
    if constexpr (V == 8) {
        uint32_t lo = 0, hi = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) lo |= (uint32_t)(uint8_t)quant_code<FAST, SAT>(v[e], step) << (8 * e);
#pragma unroll
        for (int e = 0; e < 4; ++e) hi |= (uint32_t)(uint8_t)quant_code<FAST, SAT>(v[4 + e], step) << (8 * e);
        *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
        if (dst2) *reinterpret_cast<uint2*>(dst2) = make_uint2(lo, hi);
    } else {
        uint32_t w = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) w |= (uint32_t)(uint8_t)quant_code<FAST, SAT>(v[e], step) << (8 * e);
        *reinterpret_cast<uint32_t*>(dst) = w;
        if (dst2) *reinterpret_cast<uint32_t*>(dst2) = w;
    }
}

// Byte offset of code k of token row m (m < 16) in the fragment-packed copy:
// 64-byte k-group c is one 1 KB block whose 16-byte piece g * 16 + m holds
// row m, inputs 64c + 16g .. +15 (the weights' packed layout for one block of
// 16 rows, so that a few-token GEMM reads each activation fragment as one
// contiguous kilobyte).
__device__ inline int64_t packed_code_offset(int64_t m, int64_t k) {
    return (k >> 6) * 1024 + ((((k & 63) >> 4) << 4) + m) * 16 + (k & 15);
}

// Max over aligned groups of G lanes (G a power of two, at most 64).
template <int G>
__device__ inline float group_max(float v) {
    if constexpr (G == 64) {
        return wave_max_dpp(v);
    } else {
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
        return v;
    }
}

// Register-resident variant: WPR waves per token row, each lane holding up to
// NCH 16-byte pieces of the row (K / VEC <= LPR * WPR * NCH).  Short rows take
// LPR < 64 lanes each (64 / LPR rows per wave, WPR == 1), so that a wave load
// still covers 1 KB of consecutive rows.  A workgroup of NT threads handles
// NT / (64 * WPR) * (64 / LPR) rows; with WPR == 1 the reduction is a
// wavefront reduction only (no LDS, no barrier).
template <class D, int NT, int WPR, int NCH, bool SMOOTH, int LPR = 64>
__global__ __launch_bounds__(NT) void act_quant_reg_kernel(const typename D::T* __restrict__ x,
                                                           const float* __restrict__ smooth,
                                                           int64_t M, int64_t K,
                                                           int8_t* __restrict__ xq,
                                                           float* __restrict__ sx,
                                                           int8_t* __restrict__ xp) {
    static_assert(LPR == 64 || WPR == 1, "rows shorter than a wave take one wave part");
    constexpr int V = D::VEC;
    constexpr int RPV = 64 / LPR;               // rows per wave
    constexpr int RPW = NT / (64 * WPR) * RPV;  // rows per workgroup
    __shared__ float red[NT / 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int sub = lane % LPR;  // the lane's place in its row's lane group
    const int64_t m = (int64_t)blockIdx.x * RPW + (wave / WPR) * RPV + lane / LPR;
    const int part = wave % WPR;  // which of the row's waves
    const bool live = m < M;
    const typename D::T* row = x + (live ? m : 0) * K;
    const int64_t nch = K / V;
    // All of the lane's loads are issued before any is used, as straight-line
    // code from clamped addresses (a conditional load would make the compiler
    // wait for each load before the next is issued); pieces past the row end
    // are left out of the maximum and are not stored.
    uint4 raw[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t ci = ((int64_t)c * WPR + part) * LPR + sub;
        raw[c] = *reinterpret_cast<const uint4*>(row + (ci < nch ? ci : nch - 1) * V);
    }
    float4 sm[NCH][V / 4];
    if constexpr (SMOOTH) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t ci = ((int64_t)c * WPR + part) * LPR + sub;
            const float* sp = smooth + (ci < nch ? ci : nch - 1) * V;
#pragma unroll
            for (int q = 0; q < V / 4; ++q) sm[c][q] = *reinterpret_cast<const float4*>(sp + 4 * q);
        }
    }
    float v[NCH][V];
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t ci = ((int64_t)c * WPR + part) * LPR + sub;
        const typename D::T* e = reinterpret_cast<const typename D::T*>(&raw[c]);
#pragma unroll
        for (int q = 0; q < V; ++q) {
            v[c][q] = D::to_f32(e[q]);
            if constexpr (SMOOTH) {
                const float4 s4 = sm[c][q / 4];
                const float sq = (q & 3) == 0 ? s4.x : (q & 3) == 1 ? s4.y : (q & 3) == 2 ? s4.z : s4.w;
                v[c][q] = v[c][q] / sq;
            }
        }
        if (ci < nch) {
#pragma unroll
            for (int q = 0; q < V; ++q) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[c][q]));
        }
    }
    amax = group_max<LPR>(amax);
    if constexpr (WPR > 1) {
        if (lane == 0) red[wave] = amax;
        __syncthreads();
        const int w0 = wave - part;
#pragma unroll
        for (int w = 0; w < WPR; ++w) amax = __builtin_fmaxf(amax, red[w0 + w]);
    }
    if (!live) return;
    const RowStep step = row_step(amax);
    if (part == 0 && sub == 0) sx[m] = step.step;
    int8_t* qrow = xq + m * K;
    // xp (nullable, fewer than 16 rows): the fragment-packed copy as well
    auto pk = [&](int64_t ci) { return xp ? xp + packed_code_offset(m, ci * V) : nullptr; };
    if (step.fast) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t ci = ((int64_t)c * WPR + part) * LPR + sub;
            if (ci < nch) store_codes<true, V>(qrow + ci * V, v[c], step, pk(ci));
        }
    } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int64_t ci = ((int64_t)c * WPR + part) * LPR + sub;
            if (ci < nch) store_codes<false, V>(qrow + ci * V, v[c], step, pk(ci));
        }
    }
}

// Two-pass variant for any K (element-wise when K is not a multiple of VEC).
template <class D, int NT, bool SMOOTH>
__global__ __launch_bounds__(NT) void act_quant_2pass_kernel(const typename D::T* __restrict__ x,
                                                             const float* __restrict__ smooth,
                                                             int64_t K, int8_t* __restrict__ xq,
                                                             float* __restrict__ sx) {
    __shared__ float red[NT / 64];
    const int64_t m = blockIdx.x;
    const typename D::T* row = x + m * K;
    float amax = 0.0f;
    for (int64_t k = threadIdx.x; k < K; k += NT) {
        float v = D::to_f32(row[k]);
        if constexpr (SMOOTH) v = v / smooth[k];
        amax = __builtin_fmaxf(amax, __builtin_fabsf(v));
    }
    amax = block_max<NT>(amax, red);
    const RowStep step = row_step(amax);
    if (threadIdx.x == 0) sx[m] = step.step;
    int8_t* qrow = xq + m * K;
    for (int64_t k = threadIdx.x; k < K; k += NT) {
        float v = D::to_f32(row[k]);
        if constexpr (SMOOTH) v = v / smooth[k];
        qrow[k] = (int8_t)(step.fast ? quant_code<true>(v, step) : quant_code<false>(v, step));
    }
}

template <class D, bool SMOOTH>
hipError_t act_quant_typed(const void* xv, int64_t M, int64_t K, const float* smooth, int8_t* xq,
                           float* sx, hipStream_t s, int8_t* xp) {
    const typename D::T* x = static_cast<const typename D::T*>(xv);
    const int64_t nch = K / D::VEC;  // 16-byte pieces per row
    auto grid = [&](int rows_per_wg) { return dim3((unsigned)((M + rows_per_wg - 1) / rows_per_wg)); };
    if (K % D::VEC != 0 || nch > 16 * 64 * 8) {
        hipLaunchKernelGGL((act_quant_2pass_kernel<D, 512, SMOOTH>), dim3((unsigned)M), dim3(512), 0,
                           s, x, smooth, K, xq, sx);
    } else if (M >= 512) {
        // Many rows: short rows share a wave (4, 8 or 16 lanes per row, up to
        // 4 pieces per lane: 65536 rows of 128 fp16 take 6.0 us against 6.8 us
        // at one piece per lane); rows of 257-512 pieces take two waves of
        // 4 pieces (2048 x 4096 fp16: 8.6 -> 8.0 us); longer rows take
        // 4, 8 or 16 waves with as few pieces per lane as cover the row, so
        // that no lane idles on the common widths (8192 x 12288: 55.0 -> 53.7
        // us with 8 waves x 3; 2048 x 16384: 21.7 -> 20.5 us with 8 x 4;
        // 8192 x 49152: 233.7 -> 214.9 us with 16 x 6; rows rotated past the
        // Infinity Cache, same box).
        if (nch <= 8)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 2, SMOOTH, 4>), grid(64), dim3(256),
                               0, s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 16)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 4, SMOOTH, 4>), grid(64), dim3(256),
                               0, s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 32)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 4, SMOOTH, 8>), grid(32), dim3(256),
                               0, s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 64)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 4, SMOOTH, 16>), grid(16), dim3(256),
                               0, s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 64 * 2)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 2, SMOOTH>), grid(4), dim3(256), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 64 * 4)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 1, 4, SMOOTH>), grid(4), dim3(256), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 128 * 4)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 2, 4, SMOOTH>), grid(2), dim3(256), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 128 * 8)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 2, 8, SMOOTH>), grid(2), dim3(256), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 512 * 3)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 512, 8, 3, SMOOTH>), grid(1), dim3(512), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 512 * 4)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 512, 8, 4, SMOOTH>), grid(1), dim3(512), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else if (nch <= 1024 * 6)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 1024, 16, 6, SMOOTH>), grid(1), dim3(1024),
                               0, s, x, smooth, M, K, xq, sx, xp);
        else
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 1024, 16, 8, SMOOTH>), grid(1), dim3(1024),
                               0, s, x, smooth, M, K, xq, sx, xp);
    } else {
        // Few rows (decode): spread each row over up to 16 waves.
        if (nch <= 256 * 4)
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 256, 4, 4, SMOOTH>), grid(1), dim3(256), 0,
                               s, x, smooth, M, K, xq, sx, xp);
        else
            hipLaunchKernelGGL((act_quant_reg_kernel<D, 1024, 16, 8, SMOOTH>), grid(1), dim3(1024),
                               0, s, x, smooth, M, K, xq, sx, xp);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// x_hat = dt(fp32(x) / s[k]), element-wise with 16-byte accesses.
template <class D, bool VECT>
__global__ __launch_bounds__(256) void smooth_act_kernel(const typename D::T* __restrict__ x,
                                                         const float* __restrict__ smooth,
                                                         int64_t M, int64_t K,
                                                         typename D::T* __restrict__ out) {
    constexpr int V = VECT ? D::VEC : 1;
    const int64_t total = M * K / V;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t e0 = i * V;
        const int64_t k = e0 % K;
        if constexpr (VECT) {
            float v[V];
            load_smoothed<D, true>(x + e0, smooth, k, v);
            typename D::T o[V];
#pragma unroll
            for (int e = 0; e < V; ++e) o[e] = D::from_f32(v[e]);
            *reinterpret_cast<uint4*>(out + e0) = *reinterpret_cast<const uint4*>(o);
        } else {
            out[e0] = D::from_f32(D::to_f32(x[e0]) / smooth[k]);
        }
    }
}

template <class D>
hipError_t smooth_act_typed(const void* xv, int64_t M, int64_t K, const float* smooth, void* ov,
                            hipStream_t s) {
    const typename D::T* x = static_cast<const typename D::T*>(xv);
    typename D::T* o = static_cast<typename D::T*>(ov);
    const bool vect = K % D::VEC == 0;
    const int64_t items = vect ? M * K / D::VEC : M * K;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (vect)
        hipLaunchKernelGGL((smooth_act_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, s, x,
                           smooth, M, K, o);
    else
        hipLaunchKernelGGL((smooth_act_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, s,
                           x, smooth, M, K, o);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Per-tensor activation quantisation [P1 推論方法: O2 per tensor, dynamic;
// O3 per tensor, static].  The tensor is treated as M * K contiguous values
// (rows are contiguous), in 16-byte chunks when K is a multiple of the
// vector width (a chunk then never crosses a row), else element by element.

constexpr int kTensorThreads = 256;
constexpr int kTensorUnroll = 4;  // chunks in flight per thread

// Chunk c of the flat tensor (V values), widened to fp32 and optionally
// divided by the smoothing factors of its channels.
template <class D, bool SMOOTH, int V>
__device__ inline void load_chunk_f32(const typename D::T* x, const float* smooth, int64_t c,
                                      int64_t K, float (&v)[V]) {
    if constexpr (V == D::VEC) {
        load_vec<D>(x + c * V, v);
    } else {
        v[0] = D::to_f32(x[c]);
    }
    if constexpr (SMOOTH) {
        const int64_t k0 = (c * V) % K;
        if constexpr (V % 4 == 0) {
#pragma unroll
            for (int e = 0; e < V; e += 4) {
                const float4 s4 = *reinterpret_cast<const float4*>(smooth + k0 + e);
                v[e] = v[e] / s4.x;
                v[e + 1] = v[e + 1] / s4.y;
                v[e + 2] = v[e + 2] / s4.z;
                v[e + 3] = v[e + 3] / s4.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < V; ++e) v[e] = v[e] / smooth[k0 + e];
        }
    }
}

// Partial maxima of |x_hat|: workgroup b writes the largest value of its
// grid-stride share to part[b] (the tensor's maximum is that of the parts).
template <class D, bool SMOOTH, int V>
__global__ __launch_bounds__(kTensorThreads) void tensor_absmax_kernel(
    const typename D::T* __restrict__ x, const float* __restrict__ smooth, int64_t M, int64_t K,
    float* __restrict__ part) {
    __shared__ float red[kTensorThreads / 64];
    const int64_t total = M * K / V;
    const int64_t stride = (int64_t)gridDim.x * kTensorThreads;
    float m = 0.0f;
    for (int64_t i0 = (int64_t)blockIdx.x * kTensorThreads + threadIdx.x; i0 < total;
         i0 += stride * kTensorUnroll) {
        float v[kTensorUnroll][V];
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u) {
            const int64_t i = i0 + u * stride;
            load_chunk_f32<D, SMOOTH, V>(x, smooth, i < total ? i : total - 1, K, v[u]);
        }
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u)
            if (i0 + u * stride < total) {
#pragma unroll
                for (int e = 0; e < V; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[u][e]));
            }
    }
    m = block_max<kTensorThreads>(m, red);
    if (threadIdx.x == 0) part[blockIdx.x] = m;
}

// One workgroup: the tensor's absmax from the nb partial maxima held in
// x_scale[0..nb), then x_scale[0..M) <- absmax / 127.  Every read happens
// before the barriers inside block_max, every write after them.
__global__ __launch_bounds__(1024) void reduce_fill_kernel(float* x_scale, int nb, int64_t M) {
    __shared__ float red[16];
    float m = 0.0f;
    for (int i = threadIdx.x; i < nb; i += 1024) m = __builtin_fmaxf(m, x_scale[i]);
    m = block_max<1024>(m, red);
    const float st = quant_step(m);
    for (int64_t i = threadIdx.x; i < M; i += 1024) x_scale[i] = st;
}

// Codes with the step src[0]; with FILL, workgroup 0 also writes the step
// to x_scale[0..M) (src must not lie in x_scale then).
template <class D, bool SMOOTH, int V, bool FILL>
__global__ __launch_bounds__(kTensorThreads) void tensor_quant_kernel(
    const typename D::T* __restrict__ x, const float* __restrict__ smooth, int64_t M, int64_t K,
    const float* src, int8_t* __restrict__ xq, float* x_scale) {
    const RowStep q = given_step(src[0]);
    if (FILL && blockIdx.x == 0)
        for (int64_t m = threadIdx.x; m < M; m += kTensorThreads) x_scale[m] = q.step;
    const int64_t total = M * K / V;
    const int64_t stride = (int64_t)gridDim.x * kTensorThreads;
    for (int64_t i0 = (int64_t)blockIdx.x * kTensorThreads + threadIdx.x; i0 < total;
         i0 += stride * kTensorUnroll) {
        float v[kTensorUnroll][V];
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u) {
            const int64_t i = i0 + u * stride;
            load_chunk_f32<D, SMOOTH, V>(x, smooth, i < total ? i : total - 1, K, v[u]);
        }
#pragma unroll
        for (int u = 0; u < kTensorUnroll; ++u) {
            const int64_t i = i0 + u * stride;
            if (i >= total) continue;
            // the step may be a static one: values beyond 128 steps saturate
            if constexpr (V == 1) {
                xq[i] = (int8_t)(q.fast ? quant_code<true, true>(v[u][0], q)
                                        : quant_code<false>(v[u][0], q));
            } else if (q.fast) {
                store_codes<true, V, true>(xq + i * V, v[u], q);
            } else {
                store_codes<false, V>(xq + i * V, v[u], q);
            }
        }
    }
}

// Dynamic: partial maxima (at most min(M, 1024) workgroups, into x_scale),
// their maximum and the step (one workgroup, into every x_scale entry), the
// codes.  Static: the codes, workgroup 0 writing x_scale.
template <class D, bool SMOOTH, int V>
hipError_t pertensor_typed(const void* xv, int64_t M, int64_t K, const float* smooth,
                           const float* step, int8_t* xq, float* x_scale, hipStream_t s) {
    const typename D::T* x = static_cast<const typename D::T*>(xv);
    const int64_t total = M * K / V;
    const int64_t per_block = kTensorThreads * kTensorUnroll;
    int64_t blocks = (total + per_block - 1) / per_block;
    if (blocks > 256 * 16) blocks = 256 * 16;
    if (!step) {
        int64_t nb = blocks < M ? blocks : M;
        if (nb > 1024) nb = 1024;
        hipLaunchKernelGGL((tensor_absmax_kernel<D, SMOOTH, V>), dim3((unsigned)nb),
                           dim3(kTensorThreads), 0, s, x, smooth, M, K, x_scale);
        hipLaunchKernelGGL(reduce_fill_kernel, dim3(1), dim3(1024), 0, s, x_scale, (int)nb, M);
        hipLaunchKernelGGL((tensor_quant_kernel<D, SMOOTH, V, false>), dim3((unsigned)blocks),
                           dim3(kTensorThreads), 0, s, x, smooth, M, K, x_scale, xq, x_scale);
    } else {
        hipLaunchKernelGGL((tensor_quant_kernel<D, SMOOTH, V, true>), dim3((unsigned)blocks),
                           dim3(kTensorThreads), 0, s, x, smooth, M, K, step, xq, x_scale);
    }
    return hipGetLastError();
}

template <class D>
hipError_t pertensor_dispatch(const void* x, int64_t M, int64_t K, const float* smooth,
                              const float* step, int8_t* xq, float* x_scale, hipStream_t s) {
    const bool vect = K % D::VEC == 0;
    if (smooth) {
        return vect ? pertensor_typed<D, true, D::VEC>(x, M, K, smooth, step, xq, x_scale, s)
                    : pertensor_typed<D, true, 1>(x, M, K, smooth, step, xq, x_scale, s);
    }
    return vect ? pertensor_typed<D, false, D::VEC>(x, M, K, smooth, step, xq, x_scale, s)
                : pertensor_typed<D, false, 1>(x, M, K, smooth, step, xq, x_scale, s);
}

// O3's step from calibration: the largest a_j / s_j (fp32 division), over
// 127.  One workgroup.
__global__ __launch_bounds__(1024) void static_step_kernel(const float* __restrict__ a,
                                                           const float* __restrict__ sm, int64_t K,
                                                           float* __restrict__ out) {
    __shared__ float red[16];
    float m = 0.0f;
    for (int64_t j = threadIdx.x; j < K; j += 1024) m = __builtin_fmaxf(m, a[j] / sm[j]);
    m = block_max<1024>(m, red);
    if (threadIdx.x == 0) out[0] = quant_step(m);
}


// ---------------------------------------------------------------------------
// LayerNorm carrying the folded smoothing factors, fused with per-token
// quantisation [P1 数学的に何をしているのか: diag(s)^-1 is folded into the
// LayerNorm's scale and shift, so the LayerNorm emits X_hat; P1 推論方法: O1
// quantises X_hat per token].  The LayerNorm is the standard one (Ba, Kiros
// and Hinton 2016): (x - mean) / sqrt(var + eps) * gamma + beta, biased
// variance.  One workgroup per row; the row stays in registers from the load
// to the code store, so x is read once and X_hat never goes to memory unless
// asked for.  Statistics: double sums (each lane over its pieces, then across
// the workgroup), mean = S / K, var = sum((x - mean)^2) / K, rstd =
// 1 / sqrt(var + eps), all in double, each rounded once to fp32.  Element-wise:
// ((x - mean) * rstd) * gamma + beta in fp32, one rounding per operation,
// then the store in the activation dtype; the stored values are quantised
// like sq_quant_act_pertoken's.
// Sum over the WPR waves of each row (WPR > 1: through LDS; every wave of the
// workgroup takes part, so the barrier is reached by all).
template <int NT, int WPR, class T>
__device__ inline T row_sum(T v, T* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if constexpr (WPR > 1) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) red[wave] = v;
        __syncthreads();
        const int w0 = wave - wave % WPR;
        v = red[w0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) v += red[w0 + w];
        __syncthreads();
    }
    return v;
}

template <int NT, int WPR>
__device__ inline float row_max(float v, float* red) {
    v = wave_max(v);
    if constexpr (WPR > 1) {
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) red[wave] = v;
        __syncthreads();
        const int w0 = wave - wave % WPR;
        v = red[w0];
#pragma unroll
        for (int w = 1; w < WPR; ++w) v = __builtin_fmaxf(v, red[w0 + w]);
    }
    return v;
}

// WPR waves per row, NT / (64 * WPR) rows per workgroup; each lane holds NCH
// pieces of its row (piece (c * WPR + part) * 64 + lane: consecutive lanes,
// consecutive pieces).  VECT: pieces of 16 bytes (K % VEC == 0), else single
// elements.  With WPR == 1 the reductions are wavefront shuffles only.
template <class D, int NT, int WPR, int NCH, bool VECT, bool HAT>
__global__ __launch_bounds__(NT) void ln_quant_kernel(const typename D::T* __restrict__ x,
                                                      const float* __restrict__ gamma,
                                                      const float* __restrict__ beta, double eps,
                                                      int64_t M, int64_t K,
                                                      int8_t* __restrict__ xq,
                                                      float* __restrict__ sx,
                                                      typename D::T* __restrict__ xhat) {
    typedef typename D::T T;
    constexpr int W = VECT ? D::VEC : 1;  // elements per piece
    constexpr int RPW = NT / (64 * WPR);  // rows per workgroup
    // The row stays in registers from load to code store.  1024-thread
    // workgroups (a register budget of 128 per lane) with 16-bit rows hold
    // it packed, two elements per 32-bit register, and widen each element
    // when it is used (exact), so that rows of up to 8 pieces per lane fit
    // without spilling; the others hold it widened to fp32.
    constexpr bool RAW = NT == 1024 && VECT && sizeof(T) == 2;
    constexpr int WS = RAW ? W / 2 : W;  // storage slots per piece
    typedef typename std::conditional<RAW, uint32_t, float>::type S;
    auto get = [](const S (&p)[WS], int e) -> float {
        if constexpr (RAW) {
            const uint32_t h = (e & 1) ? (p[e >> 1] >> 16) : (p[e >> 1] & 0xFFFFu);
            return D::to_f32(__builtin_bit_cast(T, (uint16_t)h));
        } else {
            return p[e];
        }
    };
    auto put = [](S (&p)[WS], int e, float f) {  // f is exactly representable in T
        if constexpr (RAW) {
            const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, D::from_f32(f));
            p[e >> 1] = (e & 1) ? ((p[e >> 1] & 0xFFFFu) | (h << 16)) : ((p[e >> 1] & 0xFFFF0000u) | h);
        } else {
            p[e] = f;
        }
    };
    __shared__ double dred[NT / 64];
    __shared__ float fred[NT / 64];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t m = (int64_t)blockIdx.x * RPW + wave / WPR;
    const int part = wave % WPR;
    const bool live = m < M;
    const T* row = x + (live ? m : 0) * K;
    const int64_t npc = K / W;  // pieces in the row
    S v[NCH][WS];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t pc = ((int64_t)c * WPR + part) * 64 + lane;
        const int64_t pcl = pc < npc ? pc : npc - 1;  // clamped: loads stay straight-line
        if constexpr (RAW)
            *reinterpret_cast<uint4*>(v[c]) = *reinterpret_cast<const uint4*>(row + pcl * W);
        else if constexpr (VECT)
            load_vec<D>(row + pcl * W, v[c]);
        else
            v[c][0] = D::to_f32(row[pcl]);
    }
    double s = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (((int64_t)c * WPR + part) * 64 + lane < npc)
#pragma unroll
            for (int e = 0; e < W; ++e) s += (double)get(v[c], e);
    const double mu_d = row_sum<NT, WPR>(s, dred) / (double)K;
    double q = 0.0;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (((int64_t)c * WPR + part) * 64 + lane < npc)
#pragma unroll
            for (int e = 0; e < W; ++e) {
                const double d = (double)get(v[c], e) - mu_d;
                q += d * d;
            }
    const double var_d = row_sum<NT, WPR>(q, dred) / (double)K;
    const float mu = (float)mu_d;
    const float rstd = (float)(1.0 / __builtin_sqrt(var_d + eps));
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t pc = ((int64_t)c * WPR + part) * 64 + lane;
        const int64_t k0 = (pc < npc ? pc : npc - 1) * W;
        float g[W], b[W];
        if constexpr (W % 4 == 0) {
#pragma unroll
            for (int e = 0; e < W; e += 4) {
                const float4 g4 = *reinterpret_cast<const float4*>(gamma + k0 + e);
                const float4 b4 = *reinterpret_cast<const float4*>(beta + k0 + e);
                g[e] = g4.x; g[e + 1] = g4.y; g[e + 2] = g4.z; g[e + 3] = g4.w;
                b[e] = b4.x; b[e + 1] = b4.y; b[e + 2] = b4.z; b[e + 3] = b4.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < W; ++e) {
                g[e] = gamma[k0 + e];
                b[e] = beta[k0 + e];
            }
        }
#pragma unroll
        for (int e = 0; e < W; ++e) {
            float t = get(v[c], e) - mu;
            t = t * rstd;
            t = t * g[e];
            t = t + b[e];
            pin_f32(t);
            put(v[c], e, D::to_f32(D::from_f32(t)));  // the value as stored in the activation dtype
        }
        if (pc < npc)
#pragma unroll
            for (int e = 0; e < W; ++e) amax = __builtin_fmaxf(amax, __builtin_fabsf(get(v[c], e)));
    }
    amax = row_max<NT, WPR>(amax, fred);
    if (!live) return;
    const RowStep step = row_step(amax);
    if (part == 0 && lane == 0) sx[m] = step.step;
    int8_t* qrow = xq + m * K;
    T* hrow = HAT ? xhat + m * K : nullptr;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int64_t pc = ((int64_t)c * WPR + part) * 64 + lane;
        if (pc >= npc) continue;
        if constexpr (HAT) {
            T h[W];
#pragma unroll
            for (int e = 0; e < W; ++e) h[e] = D::from_f32(get(v[c], e));  // exact: already in T
            if constexpr (VECT)
                *reinterpret_cast<uint4*>(hrow + pc * W) = *reinterpret_cast<const uint4*>(h);
            else
                hrow[pc] = h[0];
        }
        float f[W];
#pragma unroll
        for (int e = 0; e < W; ++e) f[e] = get(v[c], e);
        if constexpr (VECT) {
            if (step.fast)
                store_codes<true, W>(qrow + pc * W, f, step);
            else
                store_codes<false, W>(qrow + pc * W, f, step);
        } else {
            qrow[pc] = (int8_t)(step.fast ? quant_code<true>(f[0], step)
                                          : quant_code<false>(f[0], step));
        }
    }
}

template <class D, int NT, int WPR, int NCH, bool VECT>
void ln_launch(const void* x, int64_t M, int64_t K, const float* g, const float* b, double eps,
               int8_t* xq, float* sx, void* xhat, hipStream_t s) {
    typedef typename D::T T;
    constexpr int RPW = NT / (64 * WPR);
    const dim3 grid((unsigned)((M + RPW - 1) / RPW));
    if (xhat)
        hipLaunchKernelGGL((ln_quant_kernel<D, NT, WPR, NCH, VECT, true>), grid, dim3(NT), 0, s,
                           static_cast<const T*>(x), g, b, eps, M, K, xq, sx, static_cast<T*>(xhat));
    else
        hipLaunchKernelGGL((ln_quant_kernel<D, NT, WPR, NCH, VECT, false>), grid, dim3(NT), 0, s,
                           static_cast<const T*>(x), g, b, eps, M, K, xq, sx, nullptr);
}

// Pieces per row npc: one wave per row while it holds the row in 8 pieces per
// lane (many rows: no barrier at all); longer rows, or few rows (decode, where
// one wave per row would leave most of the GPU idle), spread over 4 or 16 waves.
template <class D>
hipError_t ln_typed(const void* x, int64_t M, int64_t K, const float* g, const float* b,
                    double eps, int8_t* xq, float* sx, void* xhat, hipStream_t s) {
    const bool few = M < 1024;
    if (K % D::VEC == 0) {
        const int64_t npc = K / D::VEC;
        if (npc <= 64 * 2 && !few)
            ln_launch<D, 256, 1, 2, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 64 * 4 && !few)
            ln_launch<D, 256, 1, 4, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 64 * 8 && !few)
            ln_launch<D, 256, 1, 8, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 256 * 2)
            ln_launch<D, 256, 4, 2, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 256 * 8)
            ln_launch<D, 256, 4, 8, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 1024 * 4)
            ln_launch<D, 1024, 16, 4, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (npc <= 1024 * 8)
            ln_launch<D, 1024, 16, 8, true>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else
            return hipErrorInvalidValue;
    } else {
        if (K <= 256 * 4)
            ln_launch<D, 256, 4, 4, false>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (K <= 1024 * 8)
            ln_launch<D, 1024, 16, 8, false>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else if (K <= 1024 * 16)
            ln_launch<D, 1024, 16, 16, false>(x, M, K, g, b, eps, xq, sx, xhat, s);
        else
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_act_quant_pertensor(const void* x, Dt dt, int64_t M, int64_t K,
                                      const float* smooth, const float* step, int8_t* xq,
                                      float* x_scale, hipStream_t s) {
    switch (dt) {
        case Dt::F32: return pertensor_dispatch<F32>(x, M, K, smooth, step, xq, x_scale, s);
        case Dt::F16: return pertensor_dispatch<F16>(x, M, K, smooth, step, xq, x_scale, s);
        case Dt::BF16: return pertensor_dispatch<BF16>(x, M, K, smooth, step, xq, x_scale, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_static_act_step(const float* a, const float* smooth, int64_t K, float* step_out,
                                  hipStream_t s) {
    hipLaunchKernelGGL(static_step_kernel, dim3(1), dim3(1024), 0, s, a, smooth, K, step_out);
    return hipGetLastError();
}

hipError_t launch_act_quant(const void* x, Dt dt, int64_t M, int64_t K, const float* smooth,
                            int8_t* xq, float* x_scale, hipStream_t s, int8_t* xp) {
    const bool sm = smooth != nullptr;
    if (xp && !act_quant_packs(dt, M, K)) return hipErrorInvalidValue;
    switch (dt) {
        case Dt::F32:
            return sm ? act_quant_typed<F32, true>(x, M, K, smooth, xq, x_scale, s, xp)
                      : act_quant_typed<F32, false>(x, M, K, smooth, xq, x_scale, s, xp);
        case Dt::F16:
            return sm ? act_quant_typed<F16, true>(x, M, K, smooth, xq, x_scale, s, xp)
                      : act_quant_typed<F16, false>(x, M, K, smooth, xq, x_scale, s, xp);
        case Dt::BF16:
            return sm ? act_quant_typed<BF16, true>(x, M, K, smooth, xq, x_scale, s, xp)
                      : act_quant_typed<BF16, false>(x, M, K, smooth, xq, x_scale, s, xp);
    }
    return hipErrorInvalidValue;
}

// The register-resident kernel (which alone writes the fragment-packed copy)
// takes the rows: at most 16 rows (the copy's block), K a multiple of the
// 16-byte piece and at most 8192 pieces.
bool act_quant_packs(Dt dt, int64_t M, int64_t K) {
    const int64_t vec = dt == Dt::F32 ? 4 : 8;
    return M >= 1 && M <= 16 && K % vec == 0 && K / vec <= 16 * 64 * 8;
}

hipError_t launch_smooth_act(const void* x, Dt dt, int64_t M, int64_t K, const float* smooth,
                             void* x_hat, hipStream_t s) {
    switch (dt) {
        case Dt::F32: return smooth_act_typed<F32>(x, M, K, smooth, x_hat, s);
        case Dt::F16: return smooth_act_typed<F16>(x, M, K, smooth, x_hat, s);
        case Dt::BF16: return smooth_act_typed<BF16>(x, M, K, smooth, x_hat, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_ln_quant(const void* x, Dt dt, int64_t M, int64_t K, const float* gamma,
                           const float* beta, double eps, int8_t* xq, float* x_scale, void* x_hat,
                           hipStream_t s) {
    switch (dt) {
        case Dt::F32: return ln_typed<F32>(x, M, K, gamma, beta, eps, xq, x_scale, x_hat, s);
        case Dt::F16: return ln_typed<F16>(x, M, K, gamma, beta, eps, xq, x_scale, x_hat, s);
        case Dt::BF16: return ln_typed<BF16>(x, M, K, gamma, beta, eps, xq, x_scale, x_hat, s);
    }
    return hipErrorInvalidValue;
}

int64_t ln_max_k(Dt dt, int64_t K) {
    const int64_t vec = dt == Dt::F32 ? 4 : 8;
    return K % vec == 0 ? 1024 * 8 * vec : 1024 * 16;
}

}  // namespace sq
