// sq_gemm_common.h -- device helpers shared by the GEMM kernels (internal):
// the scale-back epilogue and masked 16-byte operand loads.
#pragma once

#include "sq_device.h"
#include "sq_launch.h"

namespace sq {

// Tile counters at the start of a split-K workspace (the split form is taken
// only while the output has at most this many tiles).
constexpr int kSplitkCounters = 4096;

// Entry blockIdx.y of a batched product whose operands, scales and outputs
// lie back to back (entry z: A + z*M*K, B + z*b_stride, sx + z*M, sw + z*N,
// Y + z*M*N elements).  Entry 0 is the unbatched call.
template <Out O, class PA, class PB, class PX, class PW, class PY>
__device__ inline void batch_entry(PA& A, PB& B, PX& sx, PW& sw, PY& Y, int M, int N, int K,
                                   int64_t b_stride) {
    const int64_t z = blockIdx.y;
    if (z == 0) return;
    A += z * (int64_t)M * K;
    B += z * b_stride;
    if (sx) sx += z * M;
    if (sw) sw += z * N;
    constexpr int ES = (O == Out::F16 || O == Out::BF16) ? 2 : 4;
    Y = static_cast<void*>(static_cast<char*>(Y) + z * (int64_t)M * N * ES);
}

__device__ inline float dequant(int acc, float sxm, float swn) {
    float f = (float)acc;  // round to nearest even
    f = f * sxm;
    f = f * swn;
    pin_f32(f);
    return f;
}

template <Out O>
__device__ inline void store_out(void* y, int64_t idx, int acc, float sxm, float swn) {
    if constexpr (O == Out::I32) {
        static_cast<int*>(y)[idx] = acc;
    } else if constexpr (O == Out::F32) {
        static_cast<float*>(y)[idx] = dequant(acc, sxm, swn);
    } else if constexpr (O == Out::F16) {
        static_cast<_Float16*>(y)[idx] = (_Float16)dequant(acc, sxm, swn);
    } else {
        static_cast<uint16_t*>(y)[idx] = BF16::from_f32(dequant(acc, sxm, swn));
    }
}

// Scale back followed by the rest of the layer: RN(RN(acc * sx) * sw + bias)
// (the channel scale and the bias in one fp32 FMA), then ReLU as v > 0 ? v : +0.
__device__ inline float dequant_ext(int acc, float sxm, float swn, float bn, int relu) {
    float f = (float)acc;
    f = f * sxm;
    f = __builtin_fmaf(f, swn, bn);
    pin_f32(f);
    return (relu && !(f > 0.0f)) ? 0.0f : f;
}

template <Out O>
__device__ inline void store_val(void* y, int64_t idx, float v) {
    if constexpr (O == Out::F32) {
        static_cast<float*>(y)[idx] = v;
    } else if constexpr (O == Out::F16) {
        static_cast<_Float16*>(y)[idx] = (_Float16)v;
    } else {
        static_cast<uint16_t*>(y)[idx] = BF16::from_f32(v);
    }
}

// store_out, or with EXT the scale back extended by e (output channel n).
template <Out O, bool EXT>
__device__ inline void store_out_ext(void* y, int64_t idx, int acc, float sxm, float swn,
                                     const Epi& e, int n) {
    if constexpr (EXT) {
        static_assert(O != Out::I32, "no epilogue on raw accumulators");
        store_val<O>(y, idx, dequant_ext(acc, sxm, swn, e.bias ? e.bias[n] : 0.0f, e.relu));
    } else {
        store_out<O>(y, idx, acc, sxm, swn);
    }
}

// 16 bytes of row r starting at column k of a row-major [R x K] int8 matrix;
// zero outside the matrix.  KVEC: K % 16 == 0, so a chunk is wholly inside or
// wholly outside and is one aligned 16-byte load.
template <bool KVEC>
__device__ inline v4i load_chunk(const int8_t* __restrict__ base, int r, int R, int k, int K) {
    v4i z = {0, 0, 0, 0};
    if (r >= R || k >= K) return z;
    const int8_t* p = base + (int64_t)r * K + k;
    if constexpr (KVEC) {
        return *reinterpret_cast<const v4i*>(p);
    } else {
        uint32_t w[4] = {0u, 0u, 0u, 0u};
        for (int b = 0; b < 16; ++b)
            if (k + b < K) w[b >> 2] |= (uint32_t)(uint8_t)p[b] << (8 * (b & 3));
        v4i v = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        return v;
    }
}

}  // namespace sq
