// sq_decode.hip -- the few-token (decode) regime of the W8A8 linear layer, gfx950.
//
// P1 = abeam.tech explainer of "SmoothQuant: Accurate and Efficient
// Post-Training Quantization for Large Language Models": 推論方法 (per-token
// activation quantisation, then the INT8 GEMM); P4 = blogs.itmedia.co.jp
// 量子化 blog, section 3 (multiply the scale factor back at inference).
//
// With at most 64 tokens the layer is bound by streaming the weight matrix
// from HBM once.  The weights go from global memory straight into MFMA
// fragments (no LDS staging): one workgroup per 16 output channels; its
// waves interleave over K in 256-byte steps (4 k-groups of 64 bytes), each
// wave keeping two steps of weight loads in flight (the next is issued before
// the MFMAs of the current); v_mfma_i32_16x16x64_i8 takes the weights as the
// 16-row operand and up to four 16-token blocks of activations as the other;
// the waves' partial sums are added in LDS before the epilogue.
//
// Loads in the stream are straight-line code from clamped addresses (a
// fragment past K meets a zero activation fragment; a row past N is never
// stored), the wave index is made wave-uniform, and activation fragments
// are read before the next weight loads are issued: loads complete in order,
// so the MFMAs then wait only for their own operands, not for the loads in
// flight behind them.
//
// Row-major weights of a multiple-of-16 KB row length put the 16 rows of one
// fragment on one HBM channel; the fragment-packed layout (one contiguous
// kilobyte per fragment) avoids that.
#include "sq_gemm_common.h"

namespace sq {
namespace {

constexpr int kNW = 8;  // waves per workgroup
constexpr int kU = 1;   // 256-byte K steps per stage

// A stage: this wave's k-groups c = (st + u * NW) * 4 + t, u < U, t < 4.
template <int NW, int U, class WF>
__device__ inline void load_stage(v4i (&w)[U][4], int st, int KG, const WF& wfrag) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int c = (st + u * NW) * 4 + t;
            w[u][t] = wfrag(c < KG ? c : KG - 1);
        }
}

template <int TB, int NW, int U, class XF>
__device__ inline void load_x(v4i (&x)[U][TB][4], int st, const XF& xfrag) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t) x[u][b][t] = xfrag(b, (st + u * NW) * 4 + t);
}

template <int TB, int U>
__device__ inline void mfma_stage(v4i (&acc)[TB], const v4i (&w)[U][4], const v4i (&x)[U][TB][4]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u][t], x[u][b][t], acc[b], 0, 0, 0);
}

// The wave's steps st = wave, wave + S, ... (S = NW * U), double-buffered.
// w0 must hold the stage at st = wave on entry (if wave < nsteps).
// wfrag(c): weight fragment of k-group c < KG.  xfrag(b, c): activation
// fragment of token block b, k-group c (zero past K or past the tokens).
template <int TB, int NW, int U, class WF, class XF>
__device__ inline void stream_k(v4i (&acc)[TB], v4i (&w0)[U][4], v4i (&w1)[U][4], int wave,
                                int nsteps, int KG, const WF& wfrag, const XF& xfrag) {
    constexpr int S = NW * U;
    int st = wave;
    if (st >= nsteps) return;
    while (true) {
        v4i x[U][TB][4];
        load_x<TB, NW, U>(x, st, xfrag);
        if (st + S >= nsteps) {
            mfma_stage<TB, U>(acc, w0, x);
            return;
        }
        load_stage<NW, U>(w1, st + S, KG, wfrag);
        mfma_stage<TB, U>(acc, w0, x);
        st += S;
        load_x<TB, NW, U>(x, st, xfrag);
        if (st + S >= nsteps) {
            mfma_stage<TB, U>(acc, w1, x);
            return;
        }
        load_stage<NW, U>(w0, st + S, KG, wfrag);
        mfma_stage<TB, U>(acc, w1, x);
        st += S;
    }
}

// Cross-wave sum of the accumulators and the scaled store.  16 x 16
// accumulator layout: lane l, element q holds row 4*(l/16) + q (output
// channel) and column l%16 (token).  sxf(tok) gives the token's step.
template <int TB, int NW, Out O, class SX, bool EXT = false>
__device__ inline void reduce_store(v4i (*red)[TB][64], const v4i (&acc)[TB], int wave, int lane,
                                    int n0, int M, int N, const float* __restrict__ sw, void* Y,
                                    const SX& sxf, const Epi& epi = Epi()) {
#pragma unroll
    for (int b = 0; b < TB; ++b) red[wave][b][lane] = acc[b];
    __syncthreads();
    if (wave < TB) {
        const int b = wave;
        v4i tot = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) tot += red[w][b][lane];
        const int g = lane >> 4;
        const int tok = b * 16 + (lane & 15);
        if (tok < M) {
            const float sxm = (O != Out::I32) ? sxf(tok) : 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = n0 + 4 * g + qq;
                if (n < N) {
                    const float swn = (O != Out::I32) ? sw[n] : 0.0f;
                    store_out_ext<O, EXT>(Y, (int64_t)tok * N + n, tot[qq], sxm, swn, epi, n);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Row-major weights [N x K] (M <= 16 * TB).  KVEC: K % 16 == 0, so each
// 16-byte chunk is wholly inside or outside a row and loads from a clamped
// address; otherwise chunks are assembled byte by byte with masking.
template <int TB, int NW, int U, Out O, bool KVEC, bool EXT>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    __shared__ v4i red[NW][TB][64];
    batch_entry<O>(X, W, sx, sw, Y, M, N, K, (int64_t)N * K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const int r = lane & 15, g = lane >> 4;
    const int KG = (K + 63) / 64, nsteps = (KG + 3) / 4;
    const int wrow = n0 + r < N ? n0 + r : N - 1;

    auto wfrag = [&](int c) -> v4i {
        const int k = c * 64 + g * 16;
        if constexpr (KVEC) {
            const v4i v = *reinterpret_cast<const v4i*>(W + (int64_t)wrow * K + (k < K ? k : K - 16));
            return k < K ? v : v4i{0, 0, 0, 0};
        } else {
            return load_chunk<false>(W, wrow, N, k, K);
        }
    };
    auto xfrag = [&](int b, int c) -> v4i {
        const int tok = b * 16 + r, k = c * 64 + g * 16;
        if constexpr (KVEC) {
            const int t = tok < M ? tok : M - 1;
            const v4i v = *reinterpret_cast<const v4i*>(X + (int64_t)t * K + (k < K ? k : K - 16));
            return (tok < M && k < K) ? v : v4i{0, 0, 0, 0};
        } else {
            return load_chunk<false>(X, tok, M, k, K);
        }
    };

    v4i acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = v4i{0, 0, 0, 0};
    v4i w0[U][4], w1[U][4];
    load_stage<NW, U>(w0, wave, KG, wfrag);  // clamped: valid for any wave
    stream_k<TB, NW, U>(acc, w0, w1, wave, nsteps, KG, wfrag, xfrag);
    auto sxf = [&](int tok) { return sx[tok]; };
    reduce_store<TB, NW, O, decltype(sxf), EXT>(red, acc, wave, lane, n0, M, N, sw, Y, sxf, epi);
}

// Fragment-packed weights (K % 64 == 0): each weight fragment is one
// contiguous, non-temporal 1 KB wave load.
template <int TB, int NW, int U, Out O, bool EXT>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_packed_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ Wp, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    __shared__ v4i red[NW][TB][64];
    batch_entry<O>(X, Wp, sx, sw, Y, M, N, K, (int64_t)((N + 15) / 16) * 16 * K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b0 = blockIdx.x, n0 = b0 * 16;
    const int r = lane & 15, g = lane >> 4;
    const int KG = K / 64, nsteps = (KG + 3) / 4;
    const int8_t* wblk = Wp + (int64_t)b0 * KG * 1024 + lane * 16;

    auto wfrag = [&](int c) -> v4i {
        return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wblk + (int64_t)c * 1024));
    };
    auto xfrag = [&](int b, int c) -> v4i {
        const int tok = b * 16 + r;
        const int t = tok < M ? tok : M - 1, cc = c < KG ? c : KG - 1;
        const v4i v = *reinterpret_cast<const v4i*>(X + (int64_t)t * K + cc * 64 + g * 16);
        return (tok < M && c < KG) ? v : v4i{0, 0, 0, 0};
    };

    v4i acc[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[b] = v4i{0, 0, 0, 0};
    v4i w0[U][4], w1[U][4];
    load_stage<NW, U>(w0, wave, KG, wfrag);  // clamped: valid for any wave
    stream_k<TB, NW, U>(acc, w0, w1, wave, nsteps, KG, wfrag, xfrag);
    auto sxf = [&](int tok) { return sx[tok]; };
    reduce_store<TB, NW, O, decltype(sxf), EXT>(red, acc, wave, lane, n0, M, N, sw, Y, sxf, epi);
}

// Fragment-packed weights, up to 16 tokens, one 16-channel block per
// workgroup, no double buffering: each iteration issues the wave's U steps
// of weight fragments and their activation fragments together, waits once,
// then runs the MFMAs.  With the next stage's loads issued only after the
// current MFMAs the wave keeps U steps in flight, but the code has no
// wait that counts a later load, fewer registers (44 at U = 1: eight waves
// per SIMD, so up to four workgroups share a CU) and a shorter tail.
// Measured on one box against the double-buffered kernel (1 token, packed
// weights streamed from HBM): 12288 x 4096 11.35 -> 9.76 us, 4096 x 16384
// 13.27 -> 11.93 us, 28672 x 8192 38.7 -> 35.9 us, 8192 x 28672 37.1 -> 36.2
// us (U = 2); 4 tokens x 28672 x 8192 40.0 -> 35.5 us (against four blocks
// per workgroup).
// PX: X is the fragment-packed copy of the codes (as in the RB-block kernel
// below): each activation fragment is one contiguous kilobyte.
template <int U, Out O, bool EXT, bool PX = false>
__global__ __launch_bounds__(kNW * 64) void gemm_skinny_lean_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ Wp, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    constexpr int NW = kNW;
    __shared__ v4i red[NW][1][64];
    batch_entry<O>(X, Wp, sx, sw, Y, M, N, K, (int64_t)((N + 15) / 16) * 16 * K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int b0 = blockIdx.x, n0 = b0 * 16;
    const int r = lane & 15, g = lane >> 4;
    const int KG = K / 64, nsteps = (KG + 3) / 4;
    const int8_t* wblk = Wp + (int64_t)b0 * KG * 1024 + lane * 16;
    const int8_t* xrow = X + (int64_t)(r < M ? r : M - 1) * K + g * 16;
    v4i acc[1] = {v4i{0, 0, 0, 0}};
    for (int st = wave; st < nsteps; st += NW * U) {
        v4i w[U][4], x[U][1][4];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = (st + u * NW) * 4 + t;
                w[u][t] = __builtin_nontemporal_load(
                    reinterpret_cast<const v4i*>(wblk + (int64_t)(c < KG ? c : KG - 1) * 1024));
            }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = (st + u * NW) * 4 + t;
                const int cc = c < KG ? c : KG - 1;
                const v4i v = PX ? *reinterpret_cast<const v4i*>(X + (int64_t)cc * 1024 + lane * 16)
                                 : *reinterpret_cast<const v4i*>(xrow + cc * 64);
                x[u][0][t] = (r < M && c < KG) ? v : v4i{0, 0, 0, 0};
            }
        mfma_stage<1, U>(acc, w, x);
    }
    auto sxf = [&](int tok) { return sx[tok]; };
    reduce_store<1, NW, O, decltype(sxf), EXT>(red, acc, wave, lane, n0, M, N, sw, Y, sxf, epi);
}

// ---------------------------------------------------------------------------
// Whole decode layer in one launch (M <= 16 tokens, packed weights).  Every
// workgroup
//  1) loads the activations (CPT 16-byte chunks per thread, into registers),
//     then issues its first weight stage, so that waiting for the
//     activations does not wait for the weights;
//  2) takes each token's absmax (DPP row reduction, then across waves in
//     LDS; MM = 4 or 16 token slots) -- the same maximum and the same
//     quantiser as the standalone per-token kernel, so codes and steps are
//     identical;
//  3) writes the codes into LDS (workgroup 0 also stores xq and x_scale);
//  4) streams its 16 output channels with the activation fragments read
//     from LDS, one stage of two 256-byte steps per wave in flight.
// LDS: M * K bytes of codes.  STATIC (O3, one step for the whole tensor,
// given in step_in[0]): step 2 disappears and every token takes that step.
// Fragment-packed weights, up to 16 tokens, RB 16-channel blocks per
// workgroup: each activation fragment a wave loads serves RB weight
// fragments (RB MFMAs), so with many tokens the activation reads (one
// kilobyte per fragment, 16 distinct rows) stop doubling the bytes each CU
// loads per weight byte.
// PX: X is the fragment-packed copy of the codes (one 16-row block, 1 KB per
// 64-byte k-group, as the quantiser's packed output), so each activation
// fragment is one contiguous kilobyte instead of 16 row pieces K bytes apart.
template <int RB, int NW, int U, Out O, bool EXT, bool PX = false>
__global__ __launch_bounds__(NW * 64) void gemm_skinny_packed_rb_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ Wp, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    static_assert(RB <= NW, "wave i sums and stores block i");
    __shared__ v4i red[NW][RB][64];
    batch_entry<O>(X, Wp, sx, sw, Y, M, N, K, (int64_t)((N + 15) / 16) * 16 * K);
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nb = (N + 15) / 16;
    const int b0 = blockIdx.x * RB, n0 = b0 * 16;
    const int r = lane & 15, g = lane >> 4;
    const int KG = K / 64, nsteps = (KG + 3) / 4;
    const int8_t* wblk[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) {
        const int rb = b0 + i < nb ? b0 + i : nb - 1;  // clamped: never stored
        wblk[i] = Wp + (int64_t)rb * KG * 1024 + lane * 16;
    }
    auto load_w = [&](v4i(&w)[U][RB][4], int st) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const int c = (st + u * NW) * 4 + t;
                    w[u][i][t] = __builtin_nontemporal_load(
                        reinterpret_cast<const v4i*>(wblk[i] + (int64_t)(c < KG ? c : KG - 1) * 1024));
                }
    };
    auto load_x = [&](v4i(&x)[U][4], int st) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int c = (st + u * NW) * 4 + t;
                const int tt = r < M ? r : M - 1, cc = c < KG ? c : KG - 1;
                const v4i v = PX ? *reinterpret_cast<const v4i*>(X + (int64_t)cc * 1024 + lane * 16)
                                 : *reinterpret_cast<const v4i*>(X + (int64_t)tt * K + cc * 64 + g * 16);
                x[u][t] = (r < M && c < KG) ? v : v4i{0, 0, 0, 0};
            }
    };
    v4i acc[RB];
#pragma unroll
    for (int i = 0; i < RB; ++i) acc[i] = v4i{0, 0, 0, 0};
    auto mf = [&](const v4i(&w)[U][RB][4], const v4i(&x)[U][4]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(w[u][i][t], x[u][t], acc[i], 0, 0, 0);
    };
    // the wave's steps st = wave, wave + S, ..., double-buffered as stream_k
    constexpr int S = NW * U;
    v4i w0[U][RB][4], w1[U][RB][4];
    load_w(w0, wave);  // clamped: valid for any wave
    int st = wave;
    if (st < nsteps) {
        while (true) {
            v4i x[U][4];
            load_x(x, st);
            if (st + S >= nsteps) {
                mf(w0, x);
                break;
            }
            load_w(w1, st + S);
            mf(w0, x);
            st += S;
            load_x(x, st);
            if (st + S >= nsteps) {
                mf(w1, x);
                break;
            }
            load_w(w0, st + S);
            mf(w1, x);
            st += S;
        }
    }
    // cross-wave sums: wave i adds up block i (accumulator layout as reduce_store)
#pragma unroll
    for (int i = 0; i < RB; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave < RB) {
        const int i = wave;
        v4i tot = red[0][i][lane];
#pragma unroll
        for (int w = 1; w < NW; ++w) tot += red[w][i][lane];
        const int tok = lane & 15;
        if (tok < M) {
            const float sxm = (O != Out::I32) ? sx[tok] : 0.0f;
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) {
                const int n = n0 + i * 16 + 4 * g + qq;
                if (n < N) {
                    const float swn = (O != Out::I32) ? sw[n] : 0.0f;
                    store_out_ext<O, EXT>(Y, (int64_t)tok * N + n, tot[qq], sxm, swn, epi, n);
                }
            }
        }
    }
}

// Every workgroup quantises all M x K activations itself, which pays off
// only while that work is small next to streaming the workgroup's weights.
// Measured on one box against quantiser + packed GEMM (two launches):
// faster fused for 1 token with K = 4096, 8192 and 16384 (10.6 / 39.5 / 15.0
// us against 13.9 / 42.3 / 17.9); slower for 1 x 28672 (46.9 against 43.9)
// and for 4 and 8 tokens (4 x 4096: 16.4 against 14.6; 8 x 4096: 38.4
// against 15.1), where the redundant quantisation dominates.
constexpr int kFusedMaxM = 2;
constexpr int kFusedMaxElems = 16384;  // M * K
constexpr int kFusedMaxLds = 32 * 1024;
constexpr int kXsPad = 16;  // bytes after each token row of codes in LDS
constexpr int kFusedMaxCpt = 16;
constexpr int kFusedU = 2;  // 256-byte K steps per stage in the one-call layer

template <class D, int NW, int U, Out O, int CPT, int MM, bool STATIC>
__global__ __launch_bounds__(NW * 64) void linear_decode_fused_kernel(
    const typename D::T* __restrict__ X, const int8_t* __restrict__ Wp,
    const float* __restrict__ sw, const float* __restrict__ step_in, int8_t* __restrict__ xq_out,
    float* __restrict__ sx_out, void* __restrict__ Y, int M, int N, int K) {
    constexpr int NT = NW * 64, V = D::VEC;
    // [M][K + kXsPad] codes: the pad puts the rows of one MFMA fragment
    // (16 tokens, same k) on distinct LDS banks; a row pitch of K bytes (a
    // multiple of 256) would put them all on the same ones
    extern __shared__ __attribute__((aligned(16))) int8_t xs[];
    const int XP = K + kXsPad;
    __shared__ v4i red[NW][1][64];
    __shared__ float rmax[MM][NW];
    __shared__ float smax[MM];  // per-token absmax
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int nblk = (N + 15) / 16;
    int blk = blockIdx.x;  // this workgroup's 16-channel blocks: blk, blk + gridDim.x, ...
    const bool wg0 = blockIdx.x == 0;
    const int r = lane & 15, g = lane >> 4;
    const int KG = K / 64, nsteps = (KG + 3) / 4;
    const int nch = K / V, TC = M * nch;  // 16-byte chunks of x
    const int8_t* wblk = Wp + (int64_t)blk * KG * 1024 + lane * 16;

    // 1) activations first, then the first weight stage
    uint4 xr[CPT];
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = i * NT + tid;
        xr[i] = j < TC ? *reinterpret_cast<const uint4*>(X + (int64_t)j * V) : make_uint4(0, 0, 0, 0);
    }
    auto wfrag = [&](int c) -> v4i {
        return __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wblk + (int64_t)c * 1024));
    };
    // unconditional (clamped) so that the wait for x below counts only x
    v4i w[U][4];
    load_stage<NW, U>(w, wave, KG, wfrag);

    // 2) per-token absmax (x rows are contiguous: chunk j belongs to token j / nch)
    // a token's step (per-token maxima from LDS: a runtime index into a
    // register array would put the array in scratch memory)
    float sstep = 0.0f;
    auto step_of = [&](int m) -> float {
        if constexpr (STATIC) return sstep;
        else return quant_step(smax[m]);
    };
    if constexpr (STATIC) {
        sstep = step_in[0];
    } else {
    float am[MM];
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) am[mm] = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = i * NT + tid;
        const int m = j < TC ? j / nch : MM;
        const typename D::T* e = reinterpret_cast<const typename D::T*>(&xr[i]);
        float a = 0.0f;
#pragma unroll
        for (int q = 0; q < V; ++q) a = __builtin_fmaxf(a, __builtin_fabsf(D::to_f32(e[q])));
#pragma unroll
        for (int mm = 0; mm < MM; ++mm)
            if (m == mm) am[mm] = __builtin_fmaxf(am[mm], a);
    }
#pragma unroll
    for (int mm = 0; mm < MM; ++mm) {
        const float w = wave_max_dpp(am[mm]);
        if (lane == 0) rmax[mm][wave] = w;
    }
    __syncthreads();
    if (tid < MM) {
        float a = rmax[tid][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) a = __builtin_fmaxf(a, rmax[tid][w]);
        smax[tid] = a;
    }
    __syncthreads();
    }  // !STATIC

    // 3) codes into LDS (and xq, x_scale from workgroup 0)
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int j = i * NT + tid;
        if (j < TC) {
            const RowStep st = given_step(step_of(j / nch));
            const typename D::T* e = reinterpret_cast<const typename D::T*>(&xr[i]);
            int8_t q[V];
            if (st.fast) {
#pragma unroll
                for (int k = 0; k < V; ++k) q[k] = (int8_t)quant_code<true, STATIC>(D::to_f32(e[k]), st);
            } else {
#pragma unroll
                for (int k = 0; k < V; ++k) q[k] = (int8_t)quant_code<false>(D::to_f32(e[k]), st);
            }
            if constexpr (V == 8) {
                const uint2 p = *reinterpret_cast<const uint2*>(q);
                *reinterpret_cast<uint2*>(xs + (j / nch) * XP + (j % nch) * V) = p;
                if (wg0) *reinterpret_cast<uint2*>(xq_out + (int64_t)j * V) = p;
            } else {
                const uint32_t p = *reinterpret_cast<const uint32_t*>(q);
                *reinterpret_cast<uint32_t*>(xs + (j / nch) * XP + (j % nch) * V) = p;
                if (wg0) *reinterpret_cast<uint32_t*>(xq_out + (int64_t)j * V) = p;
            }
        }
    }
    if (wg0 && tid < M) sx_out[tid] = step_of(tid);
    __syncthreads();

    // 4) the weight stream
    auto xfrag = [&](int, int c) -> v4i {
        const int t = r < M ? r : M - 1, cc = c < KG ? c : KG - 1;
        const v4i v = *reinterpret_cast<const v4i*>(xs + t * XP + cc * 64 + g * 16);
        return (r < M && c < KG) ? v : v4i{0, 0, 0, 0};
    };
    // One stage of U steps in flight per wave, the next issued after the
    // MFMAs of the current one: the first stage (all of a short K) was in
    // flight during the quantisation, and the stage registers stay few.  The
    // workgroup then moves on to its next block (the codes stay in LDS), whose
    // first stage is issued before this block's cross-wave sum.
    const int tok = lane & 15;  // this lane's token (stored only if < M)
    const float sx_lane = step_of(tok < MM ? tok : 0);
    constexpr int S = NW * U;
    while (true) {
        v4i acc[1] = {v4i{0, 0, 0, 0}};
        for (int st = wave; st < nsteps; st += S) {
            v4i x[U][1][4];
            load_x<1, NW, U>(x, st, xfrag);
            mfma_stage<1, U>(acc, w, x);
            if (st + S < nsteps) load_stage<NW, U>(w, st + S, KG, wfrag);
        }
        const int n0 = blk * 16;
        const int nxt = blk + (int)gridDim.x;
        if (nxt < nblk) {
            wblk = Wp + (int64_t)nxt * KG * 1024 + lane * 16;
            load_stage<NW, U>(w, wave, KG, wfrag);
        }
        reduce_store<1, NW, O>(red, acc, wave, lane, n0, M, N, sw, Y,
                               [sx_lane](int) { return sx_lane; });
        if (nxt >= nblk) break;
        __syncthreads();  // every wave has read `red` before the next block writes it
        blk = nxt;
    }
}

template <class D, Out O, int NW, int U, int CPT, int MM, bool STATIC>
hipError_t launch_fused_cpt(const void* x, const int8_t* wp, const float* sw, const float* step,
                            int8_t* xq, float* sx, void* y, int M, int N, int K, hipStream_t s) {
    // Persistent workgroups: as many as fit on the GPU at once (LDS holds the
    // codes, M * K bytes, next to the reduction buffer; at most 32 waves per
    // CU), each taking an equal share of the 16-channel blocks, so that the
    // quantisation is done once per workgroup rather than once per block.
    const int nblk = (N + 15) / 16;
    int per_cu = 163840 / (M * (K + kXsPad) + NW * 1024 + 1024);
    per_cu = per_cu < 1 ? 1 : (per_cu > 32 / NW ? 32 / NW : per_cu);
    const int slots = device_cu_count() * per_cu;
    const int per = (nblk + slots - 1) / slots;
    const int G = (nblk + per - 1) / per;
    hipLaunchKernelGGL((linear_decode_fused_kernel<D, NW, U, O, CPT, MM, STATIC>),
                       dim3((unsigned)G), dim3(NW * 64), (size_t)M * (K + kXsPad), s,
                       static_cast<const typename D::T*>(x), wp, sw, step, xq, sx, y, M, N, K);
    return hipGetLastError();
}

// CPT: 16-byte chunks of x per thread; MM: token slots of the absmax (the
// static variant has none and always takes MM = 4).
template <class D, Out O, int NW, int U, bool STATIC>
hipError_t launch_fused_nw(const void* x, const int8_t* wp, const float* sw, const float* step,
                           int8_t* xq, float* sx, void* y, int M, int N, int K, hipStream_t s) {
    const int cpt = (M * (K / D::VEC) + NW * 64 - 1) / (NW * 64);
#define SQ_FUSED(C, MMV) \
    return launch_fused_cpt<D, O, NW, U, C, MMV, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s)
    if (cpt <= 1) SQ_FUSED(1, 4);
    if (cpt <= 2) SQ_FUSED(2, 4);
    if (cpt <= 4) SQ_FUSED(4, 4);
    if (cpt <= 8) SQ_FUSED(8, 4);
    SQ_FUSED(16, 4);
#undef SQ_FUSED
}

// Wide layers (at least 768 channel blocks) take 4-wave workgroups with 2
// steps per stage (twice as many workgroups resident per CU as with 8
// waves); narrow layers keep 8 waves x 2 steps.  Measured on one box, medians
// of interleaved rounds, 1 token: 12288 x 4096 10.82 -> 10.59 us, 16384 x
// 4096 13.10 -> 12.96 us, 28672 x 8192 37.34 (4 waves x 4 steps) -> 37.09 us;
// 4096 x 16384 stays at 14.25 us (4 waves: 16.17).
template <class D, Out O, bool STATIC>
hipError_t launch_fused(const void* x, const int8_t* wp, const float* sw, const float* step,
                        int8_t* xq, float* sx, void* y, int M, int N, int K, hipStream_t s) {
    if ((N + 15) / 16 >= 768)
        return launch_fused_nw<D, O, 4, 2, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s);
    return launch_fused_nw<D, O, kNW, kFusedU, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s);
}

// The one-kernel path applies: few tokens, M * K within the redundant-work
// (and LDS) budget, x within the per-thread register budget.
bool fused_fits(Dt xdt, int64_t M, int64_t K) {
    const int64_t vec = xdt == Dt::F32 ? 4 : 8;
    return M <= kFusedMaxM && M * K <= kFusedMaxElems && M * K <= kFusedMaxLds &&
           M * (K / vec) <= (int64_t)kFusedMaxCpt * kNW * 64;
}

template <class D, bool STATIC>
hipError_t fused_out(const void* x, const int8_t* wp, const float* sw, const float* step,
                     int8_t* xq, float* sx, void* y, Out out, int M, int N, int K, hipStream_t s) {
    switch (out) {
        case Out::F16:
            return launch_fused<D, Out::F16, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s);
        case Out::BF16:
            return launch_fused<D, Out::BF16, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s);
        case Out::F32:
            return launch_fused<D, Out::F32, STATIC>(x, wp, sw, step, xq, sx, y, M, N, K, s);
        default: break;
    }
    return hipErrorInvalidValue;
}

template <bool STATIC>
hipError_t fused_dt(const void* x, Dt xdt, const int8_t* wp, const float* sw, const float* step,
                    int8_t* xq, float* sx, void* y, Out out, int M, int N, int K, hipStream_t s) {
    switch (xdt) {
        case Dt::F32: return fused_out<F32, STATIC>(x, wp, sw, step, xq, sx, y, out, M, N, K, s);
        case Dt::F16: return fused_out<F16, STATIC>(x, wp, sw, step, xq, sx, y, out, M, N, K, s);
        case Dt::BF16: return fused_out<BF16, STATIC>(x, wp, sw, step, xq, sx, y, out, M, N, K, s);
    }
    return hipErrorInvalidValue;
}

template <int TB, Out O, bool EXT>
hipError_t skinny_tb(const int8_t* xq, const float* sx, const int8_t* w, const float* sw, int M,
                     int N, int K, void* y, bool packed, Epi epi, hipStream_t s, int batch) {
    const int nb = (N + 15) / 16;
    const dim3 grid((unsigned)nb, (unsigned)batch), block(kNW * 64);
    // Packed weights, up to 16 tokens: the lean kernel (U = 2 for K >= 24576)
    // at one or two tokens, and up to 8 tokens on wide layers (>= 768
    // channel blocks: 8 tokens x 28672 x 8192 40.4 -> 38.4 us); else, from 4
    // tokens on >= 512 blocks, RB blocks per workgroup share each activation
    // fragment, as long as the grid keeps >= 192 workgroups (fewer starve the
    // HBM stream).  Measured on one box, 16 tokens: 28672 x 8192 48.6 -> 40.9
    // us (RB 4), 8192 x 28672 52.6 -> 40.9 us (RB 2), 12288 x 4096 14.7 ->
    // 12.1 us (RB 4); narrower layers take the lean kernel (4096 x 16384 at 16
    // tokens 15.3 us either way).  The RB 4 kernel holds 229 registers, so
    // one 8-wave workgroup fits a CU; where its grid would take more than one
    // round, 4-wave workgroups (two per CU) run it in one (28672 x 8192 at 16 /
    // 12 tokens 41.2 / 41.7 -> 39.6 / 38.6 us; on layers of at most 1024
    // blocks the 8-wave form stays ahead: 16384 x 4096 at 16 tokens 13.7
    // against 14.2 us).
    const bool lean = packed && TB == 1 &&
                      (M <= 2 || (M <= 8 && nb >= 768) || nb < 512 || M < 4);
    if (lean) {
        if (M <= 2 && K >= 24576)
            hipLaunchKernelGGL((gemm_skinny_lean_kernel<2, O, EXT>), grid, block, 0, s, xq, w, sx,
                               sw, y, M, N, K, epi);
        else
            hipLaunchKernelGGL((gemm_skinny_lean_kernel<1, O, EXT>), grid, block, 0, s, xq, w, sx,
                               sw, y, M, N, K, epi);
    } else if (packed && TB == 1 && M >= 4 && nb >= 512) {
        if (nb >= 768 && (int64_t)((nb + 3) / 4) * batch > device_cu_count())
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<4, 4, kU, O, EXT>),
                               dim3((unsigned)((nb + 3) / 4), (unsigned)batch), dim3(256), 0, s, xq,
                               w, sx, sw, y, M, N, K, epi);
        else if (nb >= 768)
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<4, kNW, kU, O, EXT>),
                               dim3((unsigned)((nb + 3) / 4), (unsigned)batch), block, 0, s, xq, w,
                               sx, sw, y, M, N, K, epi);
        else
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<2, kNW, kU, O, EXT>),
                               dim3((unsigned)((nb + 1) / 2), (unsigned)batch), block, 0, s, xq, w,
                               sx, sw, y, M, N, K, epi);
    } else if (packed)
        hipLaunchKernelGGL((gemm_skinny_packed_kernel<TB, kNW, kU, O, EXT>), grid, block, 0, s, xq,
                           w, sx, sw, y, M, N, K, epi);
    else if (K % 16 == 0)
        hipLaunchKernelGGL((gemm_skinny_kernel<TB, kNW, kU, O, true, EXT>), grid, block, 0, s, xq,
                           w, sx, sw, y, M, N, K, epi);
    else
        hipLaunchKernelGGL((gemm_skinny_kernel<TB, kNW, kU, O, false, EXT>), grid, block, 0, s, xq,
                           w, sx, sw, y, M, N, K, epi);
    return hipGetLastError();
}

template <Out O, bool EXT>
hipError_t skinny_out(const int8_t* xq, const float* sx, const int8_t* w, const float* sw, int M,
                      int N, int K, void* y, bool packed, Epi epi, hipStream_t s, int batch) {
    if (M <= 16) return skinny_tb<1, O, EXT>(xq, sx, w, sw, M, N, K, y, packed, epi, s, batch);
    if (M <= 32) return skinny_tb<2, O, EXT>(xq, sx, w, sw, M, N, K, y, packed, epi, s, batch);
    if (M <= 48) return skinny_tb<3, O, EXT>(xq, sx, w, sw, M, N, K, y, packed, epi, s, batch);
    return skinny_tb<4, O, EXT>(xq, sx, w, sw, M, N, K, y, packed, epi, s, batch);
}

}  // namespace

// The packed-activation GEMM applies where the two-launch layer runs the
// RB-block kernel at 13-16 tokens (and on deep narrow layers, below): there
// each activation fragment spans 16
// token rows, and reading it as one kilobyte of the packed copy saves 1-2 us
// per layer on the Llama-70B-like layers (28672 x 8192 at 16 tokens 40.1 ->
// 38.0 us, 8192 x 28672 42.2 -> 41.2 us; at 4-12 tokens no gain).
// Narrower layers (< 512 blocks) run the lean kernel on the packed copy where
// K >= 16384, where each workgroup's 16 x K codes are as many bytes as its
// weights.  Measured on one box (quantiser + GEMM per call, fp16, medians of
// interleaved rounds, weights past the Infinity Cache; row-major codes ->
// packed copy): 16 x 4096 x 16384 (M x N x K) 19.9 -> 18.2 us, 16 x 2048 x
// 16384 18.3 -> 17.1 us, 13 x 4096 x 16384 18.3 -> 18.2 us; shallower layers
// lose (16 x 4096 x 4096 12.5 -> 13.0 us, 16 x 1024 x 8192 13.4 -> 13.8 us).
bool packed_x_applies(int64_t M, int64_t N, int64_t K) {
    return M >= 13 && M <= 16 && ((N + 15) / 16 >= 512 || K >= 16384);
}

hipError_t launch_skinny_px(const int8_t* xp, const float* sx, const int8_t* wp, const float* sw,
                            int64_t M, int64_t N, int64_t K, void* y, Out out, hipStream_t s) {
    if (!packed_x_applies(M, N, K)) return hipErrorInvalidValue;
    const int nb = (int)((N + 15) / 16), m = (int)M, n = (int)N, k = (int)K;
    const Epi epi;
#define SQ_PX(O)                                                                                   \
    do {                                                                                           \
        if (nb < 512)                                                                              \
            hipLaunchKernelGGL((gemm_skinny_lean_kernel<1, O, false, true>), dim3((unsigned)nb),   \
                               dim3(kNW * 64), 0, s, xp, wp, sx, sw, y, m, n, k, epi);             \
        else if (nb >= 768 && (nb + 3) / 4 > device_cu_count())                                    \
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<4, 4, kU, O, false, true>),           \
                               dim3((unsigned)((nb + 3) / 4)), dim3(256), 0, s, xp, wp, sx, sw, y, \
                               m, n, k, epi);                                                      \
        else if (nb >= 768)                                                                        \
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<4, kNW, kU, O, false, true>),         \
                               dim3((unsigned)((nb + 3) / 4)), dim3(kNW * 64), 0, s, xp, wp, sx,   \
                               sw, y, m, n, k, epi);                                               \
        else                                                                                       \
            hipLaunchKernelGGL((gemm_skinny_packed_rb_kernel<2, kNW, kU, O, false, true>),         \
                               dim3((unsigned)((nb + 1) / 2)), dim3(kNW * 64), 0, s, xp, wp, sx,   \
                               sw, y, m, n, k, epi);                                               \
        return hipGetLastError();                                                                  \
    } while (0)
    switch (out) {
        case Out::F16: SQ_PX(Out::F16);
        case Out::BF16: SQ_PX(Out::BF16);
        case Out::F32: SQ_PX(Out::F32);
        default: break;
    }
#undef SQ_PX
    return hipErrorInvalidValue;
}

hipError_t launch_skinny(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                         int M, int N, int K, void* y, Out out, bool packed, hipStream_t s,
                         Epi epi, int batch) {
#define SQ_SK(O, E) return skinny_out<O, E>(xq, sx, w, sw, M, N, K, y, packed, epi, s, batch)
    const bool ext = epi.on();
    switch (out) {
        case Out::I32: SQ_SK(Out::I32, false);
        case Out::F16: if (ext) SQ_SK(Out::F16, true); SQ_SK(Out::F16, false);
        case Out::BF16: if (ext) SQ_SK(Out::BF16, true); SQ_SK(Out::BF16, false);
        case Out::F32: if (ext) SQ_SK(Out::F32, true); SQ_SK(Out::F32, false);
    }
#undef SQ_SK
    return hipErrorInvalidValue;
}

hipError_t launch_linear_packed(const void* x, Dt xdt, int64_t M, int64_t K, const int8_t* wp,
                                const float* w_scale, int64_t N, int8_t* xq, float* x_scale,
                                void* y, Out out, hipStream_t s) {
    if (fused_fits(xdt, M, K))
        return fused_dt<false>(x, xdt, wp, w_scale, nullptr, xq, x_scale, y, out, (int)M, (int)N,
                               (int)K, s);
    hipError_t e = launch_act_quant(x, xdt, M, K, nullptr, xq, x_scale, s);
    if (e != hipSuccess) return e;
    return launch_gemm_packed(xq, x_scale, wp, w_scale, M, N, K, y, out, s);
}

int64_t linear_workspace_bytes(Dt xdt, int64_t M, int64_t N, int64_t K) {
    if (fused_fits(xdt, M, K) || !packed_x_applies(M, N, K) || !act_quant_packs(xdt, M, K)) return 0;
    return 16 * K;
}

// As launch_linear_packed; at 13-16 tokens on layers of >= 512 channel
// blocks the quantiser also writes the fragment-packed copy of the codes
// into xp, which the GEMM then reads.
hipError_t launch_linear_packed_ws(const void* x, Dt xdt, int64_t M, int64_t K, const int8_t* wp,
                                   const float* w_scale, int64_t N, int8_t* xq, float* x_scale,
                                   void* y, Out out, int8_t* xp, hipStream_t s) {
    if (linear_workspace_bytes(xdt, M, N, K) == 0)
        return launch_linear_packed(x, xdt, M, K, wp, w_scale, N, xq, x_scale, y, out, s);
    hipError_t e = launch_act_quant(x, xdt, M, K, nullptr, xq, x_scale, s, xp);
    if (e != hipSuccess) return e;
    return launch_skinny_px(xp, x_scale, wp, w_scale, M, N, K, y, out, s);
}

hipError_t launch_linear_packed_static(const void* x, Dt xdt, int64_t M, int64_t K,
                                       const int8_t* wp, const float* w_scale, int64_t N,
                                       const float* step, int8_t* xq, float* x_scale, void* y,
                                       Out out, hipStream_t s) {
    if (fused_fits(xdt, M, K))
        return fused_dt<true>(x, xdt, wp, w_scale, step, xq, x_scale, y, out, (int)M, (int)N,
                              (int)K, s);
    hipError_t e = launch_act_quant_pertensor(x, xdt, M, K, nullptr, step, xq, x_scale, s);
    if (e != hipSuccess) return e;
    return launch_gemm_packed(xq, x_scale, wp, w_scale, M, N, K, y, out, s);
}

}  // namespace sq
