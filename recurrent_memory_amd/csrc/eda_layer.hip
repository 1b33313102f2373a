// eda_layer.hip -- the layer prologue as a pass of its own, for the fp32
// chunked path (the bf16 chunked path and decode fuse it into their kernels).
//
// Per token and value head h (key head h / (H / Hk)):
//   q, k, e <- x / max(||x||_2, 1e-6)                 (EDA paper Fig. 1: normalised q, k, e)
//   alpha   <- exp(l + (-l) exp(-(A / |l|) softplus(a + b_Delta))),  A = exp(A_log), l = -5
//              (EDA paper Eqs. (14)-(15); slides frame on the safe decay parameterization)
// written per value head (fp32) into the caller's workspace, then the
// chunked forward runs on them.
#include "eda_common.h"

namespace eda {

constexpr float LY_L2E = 1.4426950408889634f, LY_LN2 = 0.6931471805599453f;
constexpr float LY_FLOOR = -5.f, LY_EPS = 1e-6f;

template <typename Tin>
__global__ void __launch_bounds__(128)
eda_layer_prep(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ e,
               const Tin *__restrict__ a, const float *__restrict__ A_log,
               const float *__restrict__ dt_bias, float *__restrict__ qo, float *__restrict__ ko,
               float *__restrict__ eo, float *__restrict__ ao, int H, int Hk, int dk) {
    __shared__ float part[2][3];
    const long row = blockIdx.x;                      // (b, t, h) value-head row
    const int h = (int)(row % H), hk = h / (H / Hk);
    const long krow = (row / H) * Hk + hk;            // (b, t, hk) key-head row
    const int c = threadIdx.x, lane = c & 63, wave = c >> 6;
    const bool ok = c < dk;
    const float xq = ok ? to_f32(q[krow * dk + c]) : 0.f;
    const float xk = ok ? to_f32(k[krow * dk + c]) : 0.f;
    const float xe = ok ? to_f32(e[krow * dk + c]) : 0.f;
    const float s0 = wave_sum(xq * xq), s1 = wave_sum(xk * xk), s2 = wave_sum(xe * xe);
    if (lane == 0) {
        part[wave][0] = s0;
        part[wave][1] = s1;
        part[wave][2] = s2;
    }
    __syncthreads();
    if (!ok) return;
    auto inv = [](float ss) { return ss > LY_EPS * LY_EPS ? 1.f / sqrtf(ss) : 1.f / LY_EPS; };
    qo[row * dk + c] = xq * inv(part[0][0] + part[1][0]);
    ko[row * dk + c] = xk * inv(part[0][1] + part[1][1]);
    eo[row * dk + c] = xe * inv(part[0][2] + part[1][2]);
    const float x = to_f32(a[krow * dk + c]) + dt_bias[hk * dk + c];
    const float sp = fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)));
    const float A = expf(A_log[hk * dk + c]);
    ao[row * dk + c] = expf(LY_FLOOR - LY_FLOOR * expf(-(A / -LY_FLOOR) * sp));
}

template <typename Tin>
hipError_t launch_layer_prep(const void *q, const void *k, const void *e, const void *a,
                             const float *A_log, const float *dt_bias, float *qo, float *ko,
                             float *eo, float *ao, int B, int T, int H, int Hk, int dk,
                             hipStream_t stream) {
    const long rows = (long)B * T * H;
    hipLaunchKernelGGL(eda_layer_prep<Tin>, dim3((unsigned)rows), dim3(128), 0, stream, (const Tin *)q,
                       (const Tin *)k, (const Tin *)e, (const Tin *)a, A_log, dt_bias, qo, ko, eo, ao, H,
                       Hk, dk);
    return hipGetLastError();
}

template hipError_t launch_layer_prep<float>(const void *, const void *, const void *, const void *,
                                             const float *, const float *, float *, float *, float *,
                                             float *, int, int, int, int, int, hipStream_t);

}  // namespace eda
