// sq_api.hip -- the library's extern "C" entry points (declared in include/sq.h).
//
// Each entry point validates its arguments on the host, before any HIP call,
// then enqueues its kernels on the caller's stream and returns.  No device
// memory is allocated and no state is kept between calls.
#include "sq.h"
#include "sq_launch.h"

namespace {

constexpr int64_t kMaxDim = SQ_MAX_DIM;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dt_ok(sq_dtype d) { return d == SQ_F32 || d == SQ_F16 || d == SQ_BF16; }

sq::Dt to_dt(sq_dtype d) { return static_cast<sq::Dt>(static_cast<int>(d)); }

bool dims_ok(int64_t a, int64_t b) { return a >= 1 && b >= 1 && a <= kMaxDim && b <= kMaxDim; }

sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// [a, a + na) and [b, b + nb) share a byte (either may be null: no overlap).
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
    if (!a || !b) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + (uintptr_t)nb && y < x + (uintptr_t)na;
}

int64_t dt_bytes(sq_dtype d) { return d == SQ_F32 ? 4 : 2; }

}  // namespace

extern "C" {

const char* sq_version(void) { return "sq-mi355x 0.1 (gfx950)"; }

sq_status sq_calibrate_absmax(const void* x, sq_dtype xdt, int64_t T, int64_t K, float* a,
                              int accumulate, void* stream) {
    if (!x || !a) return SQ_ERR_NULL;
    if (!dims_ok(T, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(xdt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(a)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_colmax(x, to_dt(xdt), T, K, a, accumulate == 0, as_stream(stream)));
}

sq_status sq_smooth_fold(const float* a, const void* w, sq_dtype wdt, int64_t K, int64_t N,
                         double alpha, float* s_out, float* w_out, float* gamma, float* beta,
                         void* stream) {
    if (!a || !w || !s_out || !w_out) return SQ_ERR_NULL;
    if (!dims_ok(K, N)) return SQ_ERR_SHAPE;
    if (!dt_ok(wdt)) return SQ_ERR_DTYPE;
    if (!(alpha >= 0.0 && alpha <= 1.0)) return SQ_ERR_ALPHA;  // also rejects NaN
    if (!aligned16(a) || !aligned16(w) || !aligned16(s_out) || !aligned16(w_out) ||
        (gamma && !aligned16(gamma)) || (beta && !aligned16(beta)))
        return SQ_ERR_ALIGN;
    return hip_status(sq::launch_smooth_fold(a, w, to_dt(wdt), K, N, alpha, s_out, w_out, gamma,
                                             beta, as_stream(stream)));
}

sq_status sq_quant_weight_perchannel(const void* w, sq_dtype wdt, int64_t K, int64_t N,
                                     int8_t* wq, float* w_scale, void* stream) {
    if (!w || !wq || !w_scale) return SQ_ERR_NULL;
    if (!dims_ok(K, N)) return SQ_ERR_SHAPE;
    if (!dt_ok(wdt)) return SQ_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_quant_weight(w, to_dt(wdt), K, N, wq, w_scale, as_stream(stream)));
}

sq_status sq_quant_act_pertoken(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                const float* smooth, int8_t* xq, float* x_scale, void* stream) {
    if (!x || !xq || !x_scale) return SQ_ERR_NULL;
    if (!dims_ok(M, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(xdt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || (smooth && !aligned16(smooth)))
        return SQ_ERR_ALIGN;
    return hip_status(
        sq::launch_act_quant(x, to_dt(xdt), M, K, smooth, xq, x_scale, as_stream(stream)));
}

sq_status sq_layernorm_quant_pertoken(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                      const float* gamma, const float* beta, double eps,
                                      int8_t* xq, float* x_scale, void* x_hat, void* stream) {
    if (!x || !gamma || !beta || !xq || !x_scale) return SQ_ERR_NULL;
    if (!dims_ok(M, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(xdt)) return SQ_ERR_DTYPE;
    if (K > sq::ln_max_k(to_dt(xdt), K)) return SQ_ERR_SHAPE;
    if (!(eps >= 0.0 && eps <= 1e300)) return SQ_ERR_EPS;  // also rejects NaN and inf
    if (!aligned16(x) || !aligned16(gamma) || !aligned16(beta) || !aligned16(xq) ||
        !aligned16(x_scale) || (x_hat && !aligned16(x_hat)))
        return SQ_ERR_ALIGN;
    const int64_t xb = M * K * dt_bytes(xdt);
    const void* outs[3] = {xq, x_scale, x_hat};
    const int64_t outn[3] = {M * K, M * 4, x_hat ? xb : 0};
    const void* ins[3] = {x, gamma, beta};
    const int64_t inn[3] = {xb, K * 4, K * 4};
    for (int o = 0; o < 3; ++o) {
        for (int i = 0; i < 3; ++i)
            if (overlaps(outs[o], outn[o], ins[i], inn[i])) return SQ_ERR_ALIAS;
        for (int p = o + 1; p < 3; ++p)
            if (overlaps(outs[o], outn[o], outs[p], outn[p])) return SQ_ERR_ALIAS;
    }
    return hip_status(sq::launch_ln_quant(x, to_dt(xdt), M, K, gamma, beta, eps, xq, x_scale,
                                          x_hat, as_stream(stream)));
}

sq_status sq_fold_prev_linear(const float* s, const void* w_prev, sq_dtype wdt, int64_t Kp,
                              int64_t K, float* w_out, float* bias, void* stream) {
    if (!s || !w_prev || !w_out) return SQ_ERR_NULL;
    if (!dims_ok(Kp, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(wdt)) return SQ_ERR_DTYPE;
    if (!aligned16(s) || !aligned16(w_prev) || !aligned16(w_out) || (bias && !aligned16(bias)))
        return SQ_ERR_ALIGN;
    return hip_status(sq::launch_fold_prev_linear(s, w_prev, to_dt(wdt), Kp, K, w_out, bias,
                                                  as_stream(stream)));
}

sq_status sq_quant_weight_pertensor(const void* w, sq_dtype wdt, int64_t K, int64_t N,
                                    int8_t* wq, float* w_scale, void* stream) {
    if (!w || !wq || !w_scale) return SQ_ERR_NULL;
    if (!dims_ok(K, N)) return SQ_ERR_SHAPE;
    if (!dt_ok(wdt)) return SQ_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)) return SQ_ERR_ALIGN;
    return hip_status(
        sq::launch_quant_weight_pertensor(w, to_dt(wdt), K, N, wq, w_scale, as_stream(stream)));
}

sq_status sq_quant_act_pertensor(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                 const float* smooth, const float* step_in, int8_t* xq,
                                 float* x_scale, void* stream) {
    if (!x || !xq || !x_scale) return SQ_ERR_NULL;
    if (!dims_ok(M, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(xdt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(x_scale) || (smooth && !aligned16(smooth)))
        return SQ_ERR_ALIGN;
    if (step_in && step_in >= x_scale && step_in < x_scale + M) return SQ_ERR_ALIAS;
    return hip_status(sq::launch_act_quant_pertensor(x, to_dt(xdt), M, K, smooth, step_in, xq,
                                                     x_scale, as_stream(stream)));
}

sq_status sq_static_act_step(const float* a, const float* s, int64_t K, float* step_out,
                             void* stream) {
    if (!a || !s || !step_out) return SQ_ERR_NULL;
    if (!dims_ok(1, K)) return SQ_ERR_SHAPE;
    return hip_status(sq::launch_static_act_step(a, s, K, step_out, as_stream(stream)));
}

sq_status sq_w8a8_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                               sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq) || !aligned16(w_scale) ||
        !aligned16(y))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(
        sq::launch_gemm(xq, x_scale, wq, w_scale, M, N, K, y, out, as_stream(stream)));
}

sq_status sq_w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                           int32_t* acc, void* stream) {
    if (!xq || !wq || !acc) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(acc)) return SQ_ERR_ALIGN;
    return hip_status(
        sq::launch_gemm(xq, nullptr, wq, nullptr, M, N, K, acc, sq::Out::I32, as_stream(stream)));
}

sq_status sq_smooth_activation(const void* x, sq_dtype dt, int64_t M, int64_t K, const float* s,
                               void* x_hat, void* stream) {
    if (!x || !s || !x_hat) return SQ_ERR_NULL;
    if (!dims_ok(M, K)) return SQ_ERR_SHAPE;
    if (!dt_ok(dt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(s) || !aligned16(x_hat)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_smooth_act(x, to_dt(dt), M, K, s, x_hat, as_stream(stream)));
}

int64_t sq_packed_weight_bytes(int64_t N, int64_t K) {
    if (!dims_ok(N, K) || K % 128 != 0) return -1;
    return sq::packed_weight_bytes(N, K);
}

sq_status sq_pack_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* wq_packed, void* stream) {
    if (!wq || !wq_packed) return SQ_ERR_NULL;
    if (!dims_ok(N, K) || K % 128 != 0) return SQ_ERR_SHAPE;
    if (!aligned16(wq) || !aligned16(wq_packed)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_pack_weight(wq, N, K, wq_packed, as_stream(stream)));
}

sq_status sq_w8a8_gemm_dequant_packed(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_packed, const float* w_scale, int64_t M,
                                      int64_t N, int64_t K, void* y, sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq_packed || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq_packed) || !aligned16(w_scale) ||
        !aligned16(y))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_gemm_packed(xq, x_scale, wq_packed, w_scale, M, N, K, y, out,
                                             as_stream(stream)));
}

int64_t sq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    if (!dims_ok(M, N) || K < 1 || K > SQ_MAX_K) return -1;
    return sq::splitk_workspace_bytes(M, N, K);
}

}  // extern "C"

namespace {
sq_status gemm_ws(const int8_t* xq, const float* x_scale, const int8_t* w, const float* w_scale,
                  int64_t M, int64_t N, int64_t K, void* y, sq_dtype ydt, void* workspace,
                  int64_t workspace_bytes, bool packed, void* stream) {
    if (!xq || !x_scale || !w || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || (packed && K % 128 != 0)) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(w) || !aligned16(w_scale) ||
        !aligned16(y))
        return SQ_ERR_ALIGN;
    const int64_t need = sq::splitk_workspace_bytes(M, N, K);
    if (need > 0) {
        if (!workspace || !aligned16(workspace) || workspace_bytes < need) return SQ_ERR_WORKSPACE;
        const int64_t wbytes = packed ? sq::packed_weight_bytes(N, K) : N * K;
        if (overlaps(workspace, need, y, M * N * dt_bytes(ydt)) ||
            overlaps(workspace, need, xq, M * K) || overlaps(workspace, need, w, wbytes) ||
            overlaps(workspace, need, x_scale, 4 * M) || overlaps(workspace, need, w_scale, 4 * N))
            return SQ_ERR_ALIAS;
    }
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_gemm_splitk(xq, x_scale, w, w_scale, M, N, K, y, out, packed,
                                             static_cast<int32_t*>(workspace), as_stream(stream)));
}
}  // namespace

extern "C" {

sq_status sq_w8a8_gemm_dequant_ws(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                                  sq_dtype ydt, void* workspace, int64_t workspace_bytes,
                                  void* stream) {
    return gemm_ws(xq, x_scale, wq, w_scale, M, N, K, y, ydt, workspace, workspace_bytes, false,
                   stream);
}

sq_status sq_w8a8_gemm_dequant_packed_ws(const int8_t* xq, const float* x_scale,
                                         const int8_t* wq_packed, const float* w_scale, int64_t M,
                                         int64_t N, int64_t K, void* y, sq_dtype ydt,
                                         void* workspace, int64_t workspace_bytes, void* stream) {
    return gemm_ws(xq, x_scale, wq_packed, w_scale, M, N, K, y, ydt, workspace, workspace_bytes,
                   true, stream);
}

sq_status sq_w8a8_gemm_dequant_packed_noalloc(const int8_t* xq, const float* x_scale,
                                              const int8_t* wq_packed, const float* w_scale,
                                              int64_t M, int64_t N, int64_t K, void* y,
                                              sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq_packed || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq_packed) || !aligned16(w_scale) ||
        !aligned16(y))
        return SQ_ERR_ALIGN;
    if (sq::splitk_workspace_bytes(M, N, K) > sq::noalloc_scratch_bytes()) return SQ_ERR_WORKSPACE;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_gemm_splitk_noalloc(xq, x_scale, wq_packed, w_scale, M, N, K, y,
                                                     out, as_stream(stream)));
}

int64_t sq_noalloc_scratch_bytes(void) { return sq::noalloc_scratch_bytes(); }

sq_status sq_w8a8_gemm_dequant_ex(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, const float* bias, int act, int64_t M,
                                  int64_t N, int64_t K, void* y, sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (act != SQ_ACT_NONE && act != SQ_ACT_RELU) return SQ_ERR_ACT;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq) || !aligned16(w_scale) ||
        !aligned16(y) || (bias && !aligned16(bias)))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    sq::Epi epi;
    epi.bias = bias;
    epi.relu = act == SQ_ACT_RELU;
    return hip_status(
        sq::launch_gemm(xq, x_scale, wq, w_scale, M, N, K, y, out, as_stream(stream), epi));
}

sq_status sq_w8a8_gemm_dequant_packed_ex(const int8_t* xq, const float* x_scale,
                                         const int8_t* wq_packed, const float* w_scale,
                                         const float* bias, int act, int64_t M, int64_t N,
                                         int64_t K, void* y, sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq_packed || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (act != SQ_ACT_NONE && act != SQ_ACT_RELU) return SQ_ERR_ACT;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq_packed) || !aligned16(w_scale) ||
        !aligned16(y) || (bias && !aligned16(bias)))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    sq::Epi epi;
    epi.bias = bias;
    epi.relu = act == SQ_ACT_RELU;
    return hip_status(sq::launch_gemm_packed(xq, x_scale, wq_packed, w_scale, M, N, K, y, out,
                                             as_stream(stream), epi));
}

sq_status sq_w8a8_bmm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                              const float* w_scale, int64_t batch, int64_t M, int64_t N,
                              int64_t K, void* y, sq_dtype ydt, void* stream) {
    if (!xq || !x_scale || !wq || !w_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || batch < 1 || batch > 65535) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(xq) || !aligned16(x_scale) || !aligned16(wq) || !aligned16(w_scale) ||
        !aligned16(y))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_gemm(xq, x_scale, wq, w_scale, M, N, K, y, out, as_stream(stream),
                                      sq::Epi(), (int)batch));
}

sq_status sq_w8a8_bmm_i32(const int8_t* xq, const int8_t* wq, int64_t batch, int64_t M, int64_t N,
                          int64_t K, int32_t* acc, void* stream) {
    if (!xq || !wq || !acc) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || batch < 1 || batch > 65535) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(acc)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_gemm(xq, nullptr, wq, nullptr, M, N, K, acc, sq::Out::I32,
                                      as_stream(stream), sq::Epi(), (int)batch));
}

sq_status sq_quant_weight_perchannel_batched(const void* w, sq_dtype wdt, int64_t batch,
                                             int64_t K, int64_t N, int8_t* wq, float* w_scale,
                                             void* stream) {
    if (!w || !wq || !w_scale) return SQ_ERR_NULL;
    if (!dims_ok(K, N) || batch < 1 || batch > 65535) return SQ_ERR_SHAPE;
    if (!dt_ok(wdt)) return SQ_ERR_DTYPE;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(w_scale)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_quant_weight_batched(w, to_dt(wdt), batch, K, N, wq, w_scale,
                                                      as_stream(stream)));
}

sq_status sq_w8a8_gemm_i32_packed(const int8_t* xq, const int8_t* wq_packed, int64_t M, int64_t N,
                                  int64_t K, int32_t* acc, void* stream) {
    if (!xq || !wq_packed || !acc) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || K < 1 || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!aligned16(xq) || !aligned16(wq_packed) || !aligned16(acc)) return SQ_ERR_ALIGN;
    return hip_status(sq::launch_gemm_packed(xq, nullptr, wq_packed, nullptr, M, N, K, acc,
                                             sq::Out::I32, as_stream(stream)));
}

sq_status sq_w8a8_linear_packed(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                const int8_t* wq_packed, const float* w_scale, int64_t N,
                                int8_t* xq, float* x_scale, void* y, sq_dtype ydt, void* stream) {
    if (!x || !wq_packed || !w_scale || !xq || !x_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || !dims_ok(K, 1) || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(xdt) || !dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(wq_packed) || !aligned16(w_scale) || !aligned16(xq) ||
        !aligned16(x_scale) || !aligned16(y))
        return SQ_ERR_ALIGN;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_linear_packed(x, to_dt(xdt), M, K, wq_packed, w_scale, N, xq,
                                               x_scale, y, out, as_stream(stream)));
}

sq_status sq_w8a8_linear_packed_static(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                       const int8_t* wq_packed, const float* w_scale, int64_t N,
                                       const float* step_in, int8_t* xq, float* x_scale, void* y,
                                       sq_dtype ydt, void* stream) {
    if (!x || !wq_packed || !w_scale || !step_in || !xq || !x_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || !dims_ok(K, 1) || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(xdt) || !dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(wq_packed) || !aligned16(w_scale) || !aligned16(xq) ||
        !aligned16(x_scale) || !aligned16(y))
        return SQ_ERR_ALIGN;
    if (step_in >= x_scale && step_in < x_scale + M) return SQ_ERR_ALIAS;
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_linear_packed_static(x, to_dt(xdt), M, K, wq_packed, w_scale, N,
                                                      step_in, xq, x_scale, y, out,
                                                      as_stream(stream)));
}

int64_t sq_linear_workspace_bytes(sq_dtype xdt, int64_t M, int64_t N, int64_t K) {
    if (!dims_ok(M, N) || !dims_ok(K, 1) || K % 128 != 0 || K > SQ_MAX_K || !dt_ok(xdt)) return -1;
    return sq::linear_workspace_bytes(to_dt(xdt), M, N, K);
}

sq_status sq_w8a8_linear_packed_ws(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                   const int8_t* wq_packed, const float* w_scale, int64_t N,
                                   int8_t* xq, float* x_scale, void* y, sq_dtype ydt,
                                   void* workspace, int64_t workspace_bytes, void* stream) {
    if (!x || !wq_packed || !w_scale || !xq || !x_scale || !y) return SQ_ERR_NULL;
    if (!dims_ok(M, N) || !dims_ok(K, 1) || K % 128 != 0) return SQ_ERR_SHAPE;
    if (K > SQ_MAX_K) return SQ_ERR_K_OVERFLOW;
    if (!dt_ok(xdt) || !dt_ok(ydt)) return SQ_ERR_DTYPE;
    if (!aligned16(x) || !aligned16(wq_packed) || !aligned16(w_scale) || !aligned16(xq) ||
        !aligned16(x_scale) || !aligned16(y))
        return SQ_ERR_ALIGN;
    const int64_t need = sq::linear_workspace_bytes(to_dt(xdt), M, N, K);
    if (need > 0) {
        if (!workspace || !aligned16(workspace) || workspace_bytes < need) return SQ_ERR_WORKSPACE;
        const void* ins[] = {x, wq_packed, w_scale};
        const int64_t inn[] = {M * K * dt_bytes(xdt), sq::packed_weight_bytes(N, K), 4 * N};
        const void* outs[] = {workspace, xq, x_scale, y};
        const int64_t outn[] = {need, M * K, 4 * M, M * N * dt_bytes(ydt)};
        for (int o = 0; o < 4; ++o) {
            for (int i = 0; i < 3; ++i)
                if (overlaps(outs[o], outn[o], ins[i], inn[i])) return SQ_ERR_ALIAS;
            for (int p = o + 1; p < 4; ++p)
                if (overlaps(outs[o], outn[o], outs[p], outn[p])) return SQ_ERR_ALIAS;
        }
    }
    sq::Out out = ydt == SQ_F16 ? sq::Out::F16 : (ydt == SQ_BF16 ? sq::Out::BF16 : sq::Out::F32);
    return hip_status(sq::launch_linear_packed_ws(
        x, to_dt(xdt), M, K, wq_packed, w_scale, N, xq, x_scale, y, out,
        need > 0 ? static_cast<int8_t*>(workspace) : nullptr, as_stream(stream)));
}

}  // extern "C"
