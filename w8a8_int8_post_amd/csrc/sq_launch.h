// sq_launch.h -- host-side launchers of the library's kernels (internal).
// Each enqueues its kernels on `s` and returns the launch status; argument
// validation happens in sq_api.hip before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

enum class Dt : int { F32 = 0, F16 = 1, BF16 = 2 };
enum class Out : int { I32 = 0, F16 = 1, BF16 = 2, F32 = 3 };

// Optional rest of a linear layer after the scale back:
// y = relu?(scaled + bias[n]).  Off (the plain scale back) by default.
struct Epi {
    const float* bias = nullptr;  // fp32 [N] or null
    int relu = 0;
    bool on() const { return bias != nullptr || relu != 0; }
    // split-K launches only: int32 workspace (splits slices of [M x N], then
    // one counter per output tile) and the number of splits of K
    int32_t* ws = nullptr;
    int splits = 1;
};

hipError_t launch_colmax(const void* x, Dt dt, int64_t R, int64_t C, float* out, bool zero_first,
                         hipStream_t s);
hipError_t launch_smooth_fold(const float* a, const void* w, Dt dt, int64_t K, int64_t N,
                              double alpha, float* s_out, float* w_out, float* gamma, float* beta,
                              hipStream_t s);
hipError_t launch_quant_weight(const void* w, Dt dt, int64_t K, int64_t N, int8_t* wq,
                               float* w_scale, hipStream_t s);
// xp (nullable): also write the codes in the fragment-packed layout of one
// 16-row block (act_quant_packs must hold).
hipError_t launch_act_quant(const void* x, Dt dt, int64_t M, int64_t K, const float* smooth,
                            int8_t* xq, float* x_scale, hipStream_t s, int8_t* xp = nullptr);
bool act_quant_packs(Dt dt, int64_t M, int64_t K);
hipError_t launch_act_quant_pertensor(const void* x, Dt dt, int64_t M, int64_t K,
                                      const float* smooth, const float* step, int8_t* xq,
                                      float* x_scale, hipStream_t s);
hipError_t launch_static_act_step(const float* a, const float* smooth, int64_t K, float* step_out,
                                  hipStream_t s);
hipError_t launch_quant_weight_pertensor(const void* w, Dt dt, int64_t K, int64_t N, int8_t* wq,
                                         float* w_scale, hipStream_t s);
hipError_t launch_quant_weight_batched(const void* w, Dt dt, int64_t batch, int64_t K, int64_t N,
                                       int8_t* wq, float* w_scale, hipStream_t s);
hipError_t launch_fold_prev_linear(const float* sm, const void* w, Dt dt, int64_t Kp, int64_t K,
                                  float* w_out, float* bias, hipStream_t s);
hipError_t launch_ln_quant(const void* x, Dt dt, int64_t M, int64_t K, const float* gamma,
                           const float* beta, double eps, int8_t* xq, float* x_scale, void* x_hat,
                           hipStream_t s);
// Largest K the fused LayerNorm kernels hold in registers for this dtype and K.
int64_t ln_max_k(Dt dt, int64_t K);
hipError_t launch_smooth_act(const void* x, Dt dt, int64_t M, int64_t K, const float* smooth,
                             void* x_hat, hipStream_t s);
// batch > 1: `batch` products back to back (see batch_entry), blockIdx.y
// selecting the entry.
hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, Out out,
                       hipStream_t s, Epi epi = Epi(), int batch = 1);

// Compute units of the current device (cached per device).
int device_cu_count();
int64_t packed_weight_bytes(int64_t N, int64_t K);
hipError_t launch_pack_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* wp, hipStream_t s);
hipError_t launch_gemm_packed(const int8_t* xq, const float* x_scale, const int8_t* wp,
                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                              Out out, hipStream_t s, Epi epi = Epi());

// Split-K form of the GEMM with scale back (packed or row-major weights) for
// shapes whose output tiles alone would leave most CUs idle.  splitk_splits
// gives the number of splits the library takes for a shape (1: none; the
// call then runs the plain GEMM), splitk_workspace_bytes the workspace it
// needs (0 when there is no split).
int splitk_splits(int64_t M, int64_t N, int64_t K);
int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K);
// The split-K form on packed weights with the library's static scratch
// instead of a caller workspace (noalloc_scratch_bytes: its size; shapes
// whose split needs more are rejected by the entry point).
int64_t noalloc_scratch_bytes();
hipError_t launch_gemm_splitk_noalloc(const int8_t* xq, const float* x_scale, const int8_t* wp,
                                      const float* w_scale, int64_t M, int64_t N, int64_t K,
                                      void* y, Out out, hipStream_t s);
hipError_t launch_gemm_splitk(const int8_t* xq, const float* x_scale, const int8_t* w,
                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                              Out out, bool packed, int32_t* ws, hipStream_t s);

// Few-token GEMM (M <= 64): row-major or fragment-packed weights.
hipError_t launch_skinny(const int8_t* xq, const float* sx, const int8_t* w, const float* sw,
                         int M, int N, int K, void* y, Out out, bool packed, hipStream_t s,
                         Epi epi = Epi(), int batch = 1);

hipError_t launch_linear_packed(const void* x, Dt xdt, int64_t M, int64_t K, const int8_t* wp,
                                const float* w_scale, int64_t N, int8_t* xq, float* x_scale,
                                void* y, Out out, hipStream_t s);
int64_t linear_workspace_bytes(Dt xdt, int64_t M, int64_t N, int64_t K);
hipError_t launch_linear_packed_ws(const void* x, Dt xdt, int64_t M, int64_t K, const int8_t* wp,
                                   const float* w_scale, int64_t N, int8_t* xq, float* x_scale,
                                   void* y, Out out, int8_t* xp, hipStream_t s);
hipError_t launch_linear_packed_static(const void* x, Dt xdt, int64_t M, int64_t K,
                                       const int8_t* wp, const float* w_scale, int64_t N,
                                       const float* step, int8_t* xq, float* x_scale, void* y,
                                       Out out, hipStream_t s);

}  // namespace sq
