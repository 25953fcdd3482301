// sq_offline.hip -- offline steps of the SmoothQuant transform on gfx950.
//
// Pages (title, section):
//   P1 = abeam.tech explainer of "SmoothQuant: Accurate and Efficient
//        Post-Training Quantization for Large Language Models".
//
//   * column absmax   : calibration statistic max_t |X[t, j]| (P1 用語解説
//                       "Calibration", 学習方法) and the per-output-channel
//                       weight range max_j |W_hat[j, n]|;
//   * smooth + fold   : s_j = max|X_j|^alpha / max|W_j|^(1-alpha) (P1
//                       smoothing factor はどう決めるのか) and diag(s) W,
//                       gamma/s, beta/s (P1 数学的に何をしているのか);
//   * weight quantise : per-output-channel step, codes transposed to [N x K].
//
// All of these stream their input once or twice from HBM; the layouts keep
// every global access coalesced along the contiguous axis.
#include "sq_device.h"
#include "sq_launch.h"

namespace sq {
namespace {

constexpr int kColThreads = 256;

__global__ void fill_zero_kernel(float* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}

// out[c] = max(out[c], max_{r in this block's rows} |x[r, c]|) via atomic max.
// Vector path: each thread owns VEC consecutive columns (one 16-byte load per
// row); consecutive threads own consecutive 16-byte pieces of a row.
template <class D, bool VECT>
__global__ __launch_bounds__(kColThreads) void colmax_kernel(const typename D::T* __restrict__ x,
                                                             int64_t R, int64_t C,
                                                             int64_t rows_per_block,
                                                             float* __restrict__ out) {
    constexpr int V = VECT ? D::VEC : 1;
    x += (int64_t)blockIdx.z * R * C;  // batch entry (0 unbatched)
    out += (int64_t)blockIdx.z * C;
    const int64_t c0 = ((int64_t)blockIdx.x * kColThreads + threadIdx.x) * V;
    if (c0 >= C) return;
    const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
    const int64_t r1 = r0 + rows_per_block < R ? r0 + rows_per_block : R;
    float m[V];
#pragma unroll
    for (int i = 0; i < V; ++i) m[i] = 0.0f;
    if constexpr (VECT) {
        int64_t r = r0;
        for (; r + 4 <= r1; r += 4) {
            float v[4][V];
#pragma unroll
            for (int u = 0; u < 4; ++u) load_vec<D>(x + (r + u) * C + c0, v[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < V; ++i) m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[u][i]));
        }
        for (; r < r1; ++r) {
            float v[V];
            load_vec<D>(x + r * C + c0, v);
#pragma unroll
            for (int i = 0; i < V; ++i) m[i] = __builtin_fmaxf(m[i], __builtin_fabsf(v[i]));
        }
    } else {
        for (int64_t r = r0; r < r1; ++r)
            m[0] = __builtin_fmaxf(m[0], __builtin_fabsf(D::to_f32(x[r * C + c0])));
    }
#pragma unroll
    for (int i = 0; i < V; ++i) atomic_max_nonneg(out + c0 + i, m[i]);
}

template <class D>
hipError_t colmax_typed(const void* xv, int64_t R, int64_t C, float* out, hipStream_t s,
                        int64_t batch = 1) {
    const typename D::T* x = static_cast<const typename D::T*>(xv);
    const bool vect = (C % D::VEC) == 0;
    const int64_t per_thread = vect ? D::VEC : 1;
    const int64_t col_blocks = (C + kColThreads * per_thread - 1) / (kColThreads * per_thread);
    // Split rows so that the grid has a few thousand workgroups.
    int64_t splits = (4096 + col_blocks * batch - 1) / (col_blocks * batch);
    if (splits > R) splits = R;
    if (splits > 65535) splits = 65535;
    if (splits < 1) splits = 1;
    const int64_t rows_per_block = (R + splits - 1) / splits;
    splits = (R + rows_per_block - 1) / rows_per_block;
    dim3 grid((unsigned)col_blocks, (unsigned)splits, (unsigned)batch);
    if (vect)
        hipLaunchKernelGGL((colmax_kernel<D, true>), grid, dim3(kColThreads), 0, s, x, R, C,
                           rows_per_block, out);
    else
        hipLaunchKernelGGL((colmax_kernel<D, false>), grid, dim3(kColThreads), 0, s, x, R, C,
                           rows_per_block, out);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// One workgroup per row j of W [K x N]:
//   b_j = max_n |w[j, n]|;  s_j = pow(a_j, alpha) / pow(b_j, 1 - alpha) in
//   double, rounded once to fp32 (1 for an all-zero channel);
//   w_out[j, :] = s_j * w[j, :];  gamma_j /= s_j;  beta_j /= s_j.
constexpr int kFoldThreads = 256;

template <class D, bool VECT>
__global__ __launch_bounds__(kFoldThreads) void smooth_fold_kernel(
    const float* __restrict__ a, const typename D::T* __restrict__ w, int64_t N, double alpha,
    float* __restrict__ s_out, float* __restrict__ w_out, float* __restrict__ gamma,
    float* __restrict__ beta) {
    __shared__ float red[kFoldThreads / 64];
    __shared__ float s_shared;
    const int64_t j = blockIdx.x;
    const typename D::T* row = w + j * N;
    float* orow = w_out + j * N;
    constexpr int V = VECT ? D::VEC : 1;
    const int64_t nvec = N / V;

    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < nvec; i += kFoldThreads) {
        if constexpr (VECT) {
            float v[V];
            load_vec<D>(row + i * V, v);
#pragma unroll
            for (int e = 0; e < V; ++e) m = __builtin_fmaxf(m, __builtin_fabsf(v[e]));
        } else {
            m = __builtin_fmaxf(m, __builtin_fabsf(D::to_f32(row[i])));
        }
    }
    const float b = block_max<kFoldThreads>(m, red);

    if (threadIdx.x == 0) {
        const float aj = a[j];
        float sj = 1.0f;
        if (aj != 0.0f && b != 0.0f)
            sj = (float)(pow((double)aj, alpha) / pow((double)b, 1.0 - alpha));
        s_out[j] = sj;
        if (gamma) gamma[j] = gamma[j] / sj;
        if (beta) beta[j] = beta[j] / sj;
        s_shared = sj;
    }
    __syncthreads();
    const float sj = s_shared;

    for (int64_t i = threadIdx.x; i < nvec; i += kFoldThreads) {
        if constexpr (VECT) {
            float v[V];
            load_vec<D>(row + i * V, v);
#pragma unroll
            for (int e = 0; e < V; e += 4) {
                float4 o = make_float4(sj * v[e], sj * v[e + 1], sj * v[e + 2], sj * v[e + 3]);
                *reinterpret_cast<float4*>(orow + i * V + e) = o;
            }
        } else {
            orow[i] = sj * D::to_f32(row[i]);
        }
    }
}

template <class D>
hipError_t smooth_fold_typed(const float* a, const void* wv, int64_t K, int64_t N, double alpha,
                             float* s_out, float* w_out, float* gamma, float* beta,
                             hipStream_t s) {
    const typename D::T* w = static_cast<const typename D::T*>(wv);
    if (N % D::VEC == 0)
        hipLaunchKernelGGL((smooth_fold_kernel<D, true>), dim3((unsigned)K), dim3(kFoldThreads), 0,
                           s, a, w, N, alpha, s_out, w_out, gamma, beta);
    else
        hipLaunchKernelGGL((smooth_fold_kernel<D, false>), dim3((unsigned)K), dim3(kFoldThreads),
                           0, s, a, w, N, alpha, s_out, w_out, gamma, beta);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Weight quantisation, transposing [K x N] -> [N x K] through a 64 x 64 LDS
// tile.  `absmax[n]` holds max_j |w[j, n]| when this kernel runs; the step
// absmax/127 is recomputed per element (the same fp32 division every time).
constexpr int kTile = 64;
constexpr int kTileThreads = 256;

template <class D>
__global__ __launch_bounds__(kTileThreads) void quant_transpose_kernel(
    const typename D::T* __restrict__ w, int64_t K, int64_t N, const float* __restrict__ absmax,
    int8_t* __restrict__ wq) {
    __shared__ int8_t tile[kTile][kTile + 4];
    w += (int64_t)blockIdx.z * K * N;  // batch entry (0 unbatched)
    absmax += (int64_t)blockIdx.z * N;
    wq += (int64_t)blockIdx.z * N * K;
    const int64_t j0 = (int64_t)blockIdx.y * kTile;
    const int64_t n0 = (int64_t)blockIdx.x * kTile;
    const int t = threadIdx.x;
    const int nn = t & (kTile - 1);
    const float step = (n0 + nn < N) ? quant_step(absmax[n0 + nn]) : 0.0f;
#pragma unroll 4
    for (int i = 0; i < kTile * kTile / kTileThreads; ++i) {
        const int jj = (i * kTileThreads + t) >> 6;
        int8_t q = 0;
        if (j0 + jj < K && n0 + nn < N)
            q = (int8_t)quant_code(D::to_f32(w[(j0 + jj) * N + n0 + nn]), step);
        tile[nn][jj] = q;
    }
    __syncthreads();
    // Write: 16 threads cover one output row n (64 bytes of j), 4 bytes each.
    for (int i = 0; i < kTile * kTile / (4 * kTileThreads); ++i) {
        const int idx = i * kTileThreads + t;
        const int rn = idx >> 4;       // 0..63
        const int cj = (idx & 15) * 4; // 0..60
        const int64_t n = n0 + rn;
        if (n >= N) continue;
        const int64_t jb = j0 + cj;
        if (jb + 4 <= K && (K % 4) == 0) {
            uint32_t packed = (uint32_t)(uint8_t)tile[rn][cj] |
                              ((uint32_t)(uint8_t)tile[rn][cj + 1] << 8) |
                              ((uint32_t)(uint8_t)tile[rn][cj + 2] << 16) |
                              ((uint32_t)(uint8_t)tile[rn][cj + 3] << 24);
            *reinterpret_cast<uint32_t*>(wq + n * K + jb) = packed;
        } else {
            for (int e = 0; e < 4; ++e)
                if (jb + e < K) wq[n * K + jb + e] = tile[rn][cj + e];
        }
    }
}

// One-pass per-column quantisation of [K x N] matrices (K a multiple of 16,
// at most 4 * NT / PPR * NR rows; N a multiple of CB = PPR * VEC columns).
// Workgroup (column block, entry): each thread keeps 4 consecutive rows x one
// 16-byte piece per pass in registers (raw, NR passes), so the block is read
// from HBM once; the column maxima are reduced across the workgroup; the codes
// of the CB output rows, a contiguous [CB x K] block of wq, are assembled in
// LDS and written with 16-byte stores.  Blocks of neighbouring columns (which
// share the 128-byte lines of each input row) are mapped to one XCD.  Codes
// are the IEEE quotient v / step, formed as in the per-token quantiser
// (Markstein's correction from RN(1 / step)) when the step is in range.
template <class D, int NT, int NR, int PPR>
__global__ __launch_bounds__(NT) void colquant_kernel(const typename D::T* __restrict__ w,
                                                      int64_t K, int64_t N, int64_t batch,
                                                      int8_t* __restrict__ wq,
                                                      float* __restrict__ w_scale) {
    constexpr int V = D::VEC, CB = PPR * V, NWV = NT / 64;
    constexpr int ROWS = NT / PPR * 4;      // rows per pass
    constexpr int PITCH = ROWS * NR + 16;   // LDS row pitch (bytes): 16-byte aligned, banks shifted
    static_assert(PPR == 1 || PPR == 2, "one or two pieces per row");
    __shared__ __attribute__((aligned(16))) int8_t tile[CB * PITCH];
    __shared__ float red[NWV][CB];
    __shared__ float steps[CB];
    // XCD-aware order: hardware block b runs on XCD b % 8; logical blocks
    // ceil(T / 8) apart go to one XCD, consecutive ones to the same XCD.
    const int64_t nb = N / CB, T = nb * batch, per = (T + 7) / 8;
    const int64_t b = blockIdx.x, xcd = b & 7, slot = b >> 3;
    const int64_t full = T - 8 * (per - 1);  // XCDs that hold `per` blocks (the rest per - 1)
    const int64_t L = xcd < full ? xcd * per + slot : full * per + (xcd - full) * (per - 1) + slot;
    const int64_t entry = L / nb, n0 = (L % nb) * CB;
    w += entry * K * N;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int p = t % PPR;        // which 16-byte piece of the CB columns
    const int g = t / PPR;        // row group (4 rows) within a pass
    uint4 raw[NR][4];
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = (int64_t)q * ROWS + g * 4 + i;
            raw[q][i] = *reinterpret_cast<const uint4*>(w + (r < K ? r : K - 1) * N + n0 + p * V);
        }
    float m[V];
#pragma unroll
    for (int e = 0; e < V; ++e) m[e] = 0.0f;
#pragma unroll
    for (int q = 0; q < NR; ++q)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if ((int64_t)q * ROWS + g * 4 + i < K) {
                const typename D::T* v = reinterpret_cast<const typename D::T*>(&raw[q][i]);
#pragma unroll
                for (int e = 0; e < V; ++e) m[e] = __builtin_fmaxf(m[e], __builtin_fabsf(D::to_f32(v[e])));
            }
#pragma unroll
    for (int e = 0; e < V; ++e) {
#pragma unroll
        for (int off = 32; off >= PPR; off >>= 1) m[e] = __builtin_fmaxf(m[e], __shfl_xor(m[e], off, 64));
    }
    if (lane < PPR) {
#pragma unroll
        for (int e = 0; e < V; ++e) red[wave][lane * V + e] = m[e];
    }
    __syncthreads();
    if (t < CB) {
        float a = red[0][t];
#pragma unroll
        for (int v = 1; v < NWV; ++v) a = __builtin_fmaxf(a, red[v][t]);
        const float st = quant_step(a);
        steps[t] = st;
        w_scale[entry * N + n0 + t] = st;
    }
    __syncthreads();
    RowStep st[V];
#pragma unroll
    for (int e = 0; e < V; ++e) st[e] = given_step(steps[p * V + e]);
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        if ((int64_t)q * ROWS + g * 4 >= K) continue;  // K % 4 == 0: whole groups
#pragma unroll
        for (int e = 0; e < V; ++e) {
            uint32_t word = 0;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const typename D::T* v = reinterpret_cast<const typename D::T*>(&raw[q][i]);
                const float x = D::to_f32(v[e]);
                const int c = st[e].fast ? quant_code<true>(x, st[e]) : quant_code<false>(x, st[e]);
                word |= (uint32_t)(uint8_t)c << (8 * i);
            }
            *reinterpret_cast<uint32_t*>(tile + (p * V + e) * PITCH + q * ROWS + g * 4) = word;
        }
    }
    __syncthreads();
    int8_t* dst = wq + (entry * N + n0) * K;
    const int64_t per_row = K / 16, pieces = CB * per_row;
    for (int64_t i = t; i < pieces; i += NT) {
        const int64_t c = i / per_row, k = (i - c * per_row) * 16;
        *reinterpret_cast<uint4*>(dst + c * K + k) =
            *reinterpret_cast<const uint4*>(tile + c * PITCH + k);
    }
}

// The one-pass kernel when the shape and alignment allow it (returns false
// when they do not, and nothing was launched).
template <class D>
bool colquant_typed(const void* wv, int64_t batch, int64_t K, int64_t N, int8_t* wq,
                    float* w_scale, hipStream_t s, hipError_t* err) {
    constexpr int CB = 2 * D::VEC;  // two pieces per row and workgroup
    const auto al = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15) == 0; };
    if (K <= 0 || K % 16 != 0 || K > 8192 || N % CB != 0 || batch > 65535 || !al(wv) || !al(wq))
        return false;
    const int64_t T = (N / CB) * batch;
    if (T > 0x7fffffff) return false;
    const typename D::T* w = static_cast<const typename D::T*>(wv);
    const dim3 grid((unsigned)T);
    if (K <= 512)
        hipLaunchKernelGGL((colquant_kernel<D, 256, 1, 2>), grid, dim3(256), 0, s, w, K, N, batch, wq, w_scale);
    else if (K <= 2048)
        hipLaunchKernelGGL((colquant_kernel<D, 1024, 1, 2>), grid, dim3(1024), 0, s, w, K, N, batch, wq, w_scale);
    else if (K <= 4096)
        hipLaunchKernelGGL((colquant_kernel<D, 1024, 2, 2>), grid, dim3(1024), 0, s, w, K, N, batch, wq, w_scale);
    else
        hipLaunchKernelGGL((colquant_kernel<D, 1024, 4, 2>), grid, dim3(1024), 0, s, w, K, N, batch, wq, w_scale);
    *err = hipGetLastError();
    return true;
}

bool colquant(const void* w, Dt dt, int64_t batch, int64_t K, int64_t N, int8_t* wq,
              float* w_scale, hipStream_t s, hipError_t* err) {
    switch (dt) {
        case Dt::F32: return colquant_typed<F32>(w, batch, K, N, wq, w_scale, s, err);
        case Dt::F16: return colquant_typed<F16>(w, batch, K, N, wq, w_scale, s, err);
        case Dt::BF16: return colquant_typed<BF16>(w, batch, K, N, wq, w_scale, s, err);
    }
    return false;
}

// p[0..n) <- max of p[0..n) (non-negative values).  One workgroup: every
// read happens before the barriers in block_max, every write after them.
__global__ __launch_bounds__(1024) void max_fill_kernel(float* p, int64_t n) {
    __shared__ float red[16];
    float m = 0.0f;
    for (int64_t i = threadIdx.x; i < n; i += 1024) m = __builtin_fmaxf(m, p[i]);
    m = block_max<1024>(m, red);
    for (int64_t i = threadIdx.x; i < n; i += 1024) p[i] = m;
}

__global__ void absmax_to_step_kernel(float* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = quant_step(p[i]);
}

// Fold of the next layer's smoothing into a preceding linear layer [P1
// 数学的に何をしているのか: the scales may be absorbed by the preceding linear
// layer]: w_out[i, j] = fp32(w[i, j]) / s[j] over its output columns j, 16
// bytes of w per thread step when K is a multiple of the vector width.
template <class D, bool VECT>
__global__ __launch_bounds__(256) void fold_prev_kernel(const typename D::T* __restrict__ w,
                                                        const float* __restrict__ sm, int64_t Kp,
                                                        int64_t K, float* __restrict__ out) {
    constexpr int V = VECT ? D::VEC : 1;
    const int64_t total = Kp * K / V;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * 256) {
        const int64_t e0 = i * V;
        const int64_t j = e0 % K;
        if constexpr (VECT) {
            float v[V];
            load_vec<D>(w + e0, v);
#pragma unroll
            for (int e = 0; e < V; e += 4) {
                const float4 s4 = *reinterpret_cast<const float4*>(sm + j + e);
                float4 o;
                o.x = v[e] / s4.x;
                o.y = v[e + 1] / s4.y;
                o.z = v[e + 2] / s4.z;
                o.w = v[e + 3] / s4.w;
                *reinterpret_cast<float4*>(out + e0 + e) = o;
            }
        } else {
            out[e0] = D::to_f32(w[e0]) / sm[j];
        }
    }
}

__global__ __launch_bounds__(256) void div_inplace_kernel(float* __restrict__ b,
                                                          const float* __restrict__ sm, int64_t K) {
    for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < K; j += (int64_t)gridDim.x * 256)
        b[j] = b[j] / sm[j];
}

template <class D>
hipError_t fold_prev_typed(const void* wv, int64_t Kp, int64_t K, const float* sm, float* out,
                           hipStream_t s) {
    const typename D::T* w = static_cast<const typename D::T*>(wv);
    const bool vect = K % D::VEC == 0;
    const int64_t items = vect ? Kp * K / D::VEC : Kp * K;
    int64_t blocks = (items + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    if (vect)
        hipLaunchKernelGGL((fold_prev_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, s, w,
                           sm, Kp, K, out);
    else
        hipLaunchKernelGGL((fold_prev_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, s,
                           w, sm, Kp, K, out);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_colmax(const void* x, Dt dt, int64_t R, int64_t C, float* out, bool zero_first,
                         hipStream_t s) {
    if (zero_first) {
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((C + 255) / 256)), dim3(256), 0, s,
                           out, C);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    switch (dt) {
        case Dt::F32: return colmax_typed<F32>(x, R, C, out, s);
        case Dt::F16: return colmax_typed<F16>(x, R, C, out, s);
        case Dt::BF16: return colmax_typed<BF16>(x, R, C, out, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_smooth_fold(const float* a, const void* w, Dt dt, int64_t K, int64_t N,
                              double alpha, float* s_out, float* w_out, float* gamma, float* beta,
                              hipStream_t s) {
    switch (dt) {
        case Dt::F32: return smooth_fold_typed<F32>(a, w, K, N, alpha, s_out, w_out, gamma, beta, s);
        case Dt::F16: return smooth_fold_typed<F16>(a, w, K, N, alpha, s_out, w_out, gamma, beta, s);
        case Dt::BF16:
            return smooth_fold_typed<BF16>(a, w, K, N, alpha, s_out, w_out, gamma, beta, s);
    }
    return hipErrorInvalidValue;
}

template <class D>
static hipError_t quant_transpose_typed(const void* wv, int64_t K, int64_t N, const float* absmax,
                                        int8_t* wq, hipStream_t s, int64_t batch = 1) {
    dim3 grid((unsigned)((N + kTile - 1) / kTile), (unsigned)((K + kTile - 1) / kTile),
              (unsigned)batch);
    hipLaunchKernelGGL((quant_transpose_kernel<D>), grid, dim3(kTileThreads), 0, s,
                       static_cast<const typename D::T*>(wv), K, N, absmax, wq);
    return hipGetLastError();
}

hipError_t launch_quant_weight_pertensor(const void* w, Dt dt, int64_t K, int64_t N, int8_t* wq,
                                         float* w_scale, hipStream_t s) {
    // per-column absmax, then every column takes the tensor's maximum; the
    // per-channel steps and codes that follow are then those of one step
    hipError_t e = launch_colmax(w, dt, K, N, w_scale, true, s);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(max_fill_kernel, dim3(1), dim3(1024), 0, s, w_scale, N);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (dt) {
        case Dt::F32: e = quant_transpose_typed<F32>(w, K, N, w_scale, wq, s); break;
        case Dt::F16: e = quant_transpose_typed<F16>(w, K, N, w_scale, wq, s); break;
        case Dt::BF16: e = quant_transpose_typed<BF16>(w, K, N, w_scale, wq, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(absmax_to_step_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                       w_scale, N);
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, Dt dt, int64_t K, int64_t N, int8_t* wq,
                               float* w_scale, hipStream_t s) {
    hipError_t e1 = hipSuccess;
    if (colquant(w, dt, 1, K, N, wq, w_scale, s, &e1)) return e1;
    // 1) w_scale <- per-column absmax (zeroed first)
    hipError_t e = launch_colmax(w, dt, K, N, w_scale, true, s);
    if (e != hipSuccess) return e;
    // 2) codes, transposed
    switch (dt) {
        case Dt::F32: e = quant_transpose_typed<F32>(w, K, N, w_scale, wq, s); break;
        case Dt::F16: e = quant_transpose_typed<F16>(w, K, N, w_scale, wq, s); break;
        case Dt::BF16: e = quant_transpose_typed<BF16>(w, K, N, w_scale, wq, s); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    // 3) w_scale <- absmax / 127
    hipLaunchKernelGGL(absmax_to_step_kernel, dim3((unsigned)((N + 255) / 256)), dim3(256), 0, s,
                       w_scale, N);
    return hipGetLastError();
}

hipError_t launch_fold_prev_linear(const float* sm, const void* w, Dt dt, int64_t Kp, int64_t K,
                                  float* w_out, float* bias, hipStream_t s) {
    hipError_t e = hipErrorInvalidValue;
    switch (dt) {
        case Dt::F32: e = fold_prev_typed<F32>(w, Kp, K, sm, w_out, s); break;
        case Dt::F16: e = fold_prev_typed<F16>(w, Kp, K, sm, w_out, s); break;
        case Dt::BF16: e = fold_prev_typed<BF16>(w, Kp, K, sm, w_out, s); break;
    }
    if (e != hipSuccess || !bias) return e;
    hipLaunchKernelGGL(div_inplace_kernel, dim3((unsigned)((K + 255) / 256 < 1024 ? (K + 255) / 256 : 1024)),
                       dim3(256), 0, s, bias, sm, K);
    return hipGetLastError();
}

// Per-column quantisation of `batch` matrices [K x N] lying back to back
// (each column n of entry b gets its own step; codes transposed to [N x K]).
hipError_t launch_quant_weight_batched(const void* w, Dt dt, int64_t batch, int64_t K, int64_t N,
                                       int8_t* wq, float* w_scale, hipStream_t s) {
    hipError_t e1 = hipSuccess;
    if (colquant(w, dt, batch, K, N, wq, w_scale, s, &e1)) return e1;
    const int64_t n = batch * N;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       w_scale, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    switch (dt) {
        case Dt::F32: e = colmax_typed<F32>(w, K, N, w_scale, s, batch); break;
        case Dt::F16: e = colmax_typed<F16>(w, K, N, w_scale, s, batch); break;
        case Dt::BF16: e = colmax_typed<BF16>(w, K, N, w_scale, s, batch); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    switch (dt) {
        case Dt::F32: e = quant_transpose_typed<F32>(w, K, N, w_scale, wq, s, batch); break;
        case Dt::F16: e = quant_transpose_typed<F16>(w, K, N, w_scale, wq, s, batch); break;
        case Dt::BF16: e = quant_transpose_typed<BF16>(w, K, N, w_scale, wq, s, batch); break;
        default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(absmax_to_step_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       w_scale, n);
    return hipGetLastError();
}

}  // namespace sq
