// eda_decode.hip -- one-token EDA step for many independent (sequence, head)
// states: the decode path.
//
// Per (n, h) with state S (d_k x d_v, fp32, rows = key channels) and one
// token (q, k, e, v, alpha, beta, gamma), the paper's three ordered stages
// (EDA paper Sec. 3.3, Eqs. (9), (11), (13)) and the read o = S_new^T q are
// rewritten so that S is read from HBM once and written once:
//
//   Sh  = Diag(alpha) S                                   (decay)
//   r_e = Sh^T e,  rh_k = Sh^T k,  rh_q = Sh^T q          (one pass over S)
//   r_k = rh_k - gamma (k.e) r_e                          (= St^T k after erase)
//   u   = beta (v - r_k)                                  (corrected write value)
//   S_new = Sh - gamma e r_e^T + k u^T
//   o   = rh_q - gamma (q.e) r_e + (q.k) u                (= S_new^T q)
//
// This is an exact algebraic restatement of Eqs. (11) and (13) (substitute
// St = Sh - gamma e r_e^T into St^T k and S_new^T q).  The paper's Sec. 3.5
// notes the decode cost is dominated by reading and writing the state; the
// kernel is therefore laid out for HBM streaming.  A persistent grid of
// 512-thread workgroups (four per compute unit launched, one or two resident
// at a time by register use) walks the states; per state
// each thread owns a 4-column strip of 8 rows (rows rg + 16m), so every
// wavefront load/store instruction touches 1 KB of contiguous memory and all
// 8 loads of a thread are in flight together.  The state is touched exactly
// once per step, so its loads and stores carry the non-temporal hint (no
// reuse is expected from the caches; measured ~15% faster than plain
// accesses at 8192 states of 64 KB).
//
// LAYER variant (the layer prologue fused in): q, k, e and the safe gate's
// input a come per key head (Hk heads shared by groups of H / Hk value
// heads), alpha = exp(l + (-l) exp(-(A / |l|) softplus(a + b))) with l = -5
// (EDA paper Eqs. (14)-(15)), and q, k, e are L2-normalised here; the
// normalisation scales are applied to the reductions and the update terms.
//
// DPLR variant: the rank-1 DPLR update of GDN-2 and QED (QED slides, frame
// "GDN-2 separates decay, erase, and write"), Sh = Diag(alpha) S,
// S_new = Sh + k (v - Sh^T a)^T, o = S_new^T q = Sh^T q + (q.k)(v - Sh^T a),
// with the erase vector a passed as `e` and no beta or gamma: the same pass
// with gamma = 0, beta = 1 and Sh^T a in place of the corrected read.
#include "eda_common.h"

namespace eda {

constexpr float DEC_L2E = 1.4426950408889634f, DEC_LN2 = 0.6931471805599453f;
constexpr float DEC_FLOOR = -5.f, DEC_EPS = 1e-6f;

// natural-log-free safe gate: alpha from a, A_log, dt_bias (fp32)
__device__ __forceinline__ float dec_safe_gate(float a, float A_log, float b) {
    const float x = a + b;
    const float sp = fmaxf(x, 0.f) + DEC_LN2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * DEC_L2E));
    const float A = __builtin_amdgcn_exp2f(A_log * DEC_L2E);
    const float gl = DEC_FLOOR - DEC_FLOOR * __builtin_amdgcn_exp2f(-(A / -DEC_FLOOR) * sp * DEC_L2E);
    return __builtin_amdgcn_exp2f(gl * DEC_L2E);
}
__device__ __forceinline__ float dec_inv_norm(float ss) {
    return ss > DEC_EPS * DEC_EPS ? __builtin_amdgcn_rsqf(ss) : 1.f / DEC_EPS;
}

constexpr int DEC_NT = 512;           // threads per workgroup
constexpr int DEC_RG = DEC_NT / 32;   // row groups (32 column quads per row)
constexpr int DEC_R = 128 / DEC_RG;   // rows per thread
constexpr int DEC_NW = DEC_NT / 64;   // wavefronts

constexpr int DEC_PLAIN = 0, DEC_LAYER = 1, DEC_DPLR = 2;

// The 128-square plain and DPLR variants fit in 128 VGPRs, which lets two
// workgroups share a CU so that one streams while the other reduces (about 2%
// faster than one per CU); the others would spill at that limit.
template <typename Tin, bool FULL, int MODE>
__global__ void __launch_bounds__(DEC_NT) __attribute__((amdgpu_waves_per_eu(FULL && MODE != 1 ? 4 : 1)))
eda_decode_kernel(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ e,
                  const Tin *__restrict__ v, const void *__restrict__ decay,
                  const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                  const float *__restrict__ beta, const float *__restrict__ gamma,
                  const float *S_in, float *S_out, Tin *__restrict__ o, long NH, int H, int Hk,
                  int dk, int dv) {
    constexpr int R = DEC_R, RG = DEC_RG;
    constexpr bool LAYER = MODE == DEC_LAYER, DPLR = MODE == DEC_DPLR;
    __shared__ float sq[128], sk[128], se[128], sa[128];
    __shared__ float red[DEC_NW][3][128];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cq = tid & 31, rg = tid >> 5;  // column quad, row group
    if (FULL) { dk = 128; dv = 128; }

    const int grp = H / Hk;
    for (long nh = blockIdx.x; nh < NH; nh += gridDim.x) {
        // key row of this (sequence, value head)
        const long hk = (nh % H) / grp, nk = (nh / H) * Hk + hk;
        if (tid < 128) {
            const bool ok = tid < dk;
            sq[tid] = ok ? to_f32(q[nk * dk + tid]) : 0.f;
            sk[tid] = ok ? to_f32(k[nk * dk + tid]) : 0.f;
            se[tid] = ok ? to_f32(e[nk * dk + tid]) : 0.f;
            if constexpr (LAYER)
                sa[tid] = ok ? dec_safe_gate(to_f32(((const Tin *)decay)[nk * dk + tid]), A_log[hk * dk + tid],
                                             dt_bias[hk * dk + tid])
                             : 0.f;
            else
                sa[tid] = ok ? ((const float *)decay)[nk * dk + tid] : 0.f;
        }

        // Read the whole state strip first (independent of the vectors above).
        float s[R][4];
        const long sbase = nh * (long)dk * dv;
        if (S_in) {
            if (FULL) {
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    const f32x4 x = __builtin_nontemporal_load(
                        reinterpret_cast<const f32x4 *>(S_in + sbase + (rg + RG * m) * 128 + 4 * cq));
                    s[m][0] = x[0]; s[m][1] = x[1]; s[m][2] = x[2]; s[m][3] = x[3];
                }
            } else {
#pragma unroll
                for (int m = 0; m < R; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int i = rg + RG * m, j = 4 * cq + c;
                        s[m][c] = (i < dk && j < dv) ? S_in[sbase + (long)i * dv + j] : 0.f;
                    }
            }
        } else {
#pragma unroll
            for (int m = 0; m < R; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) s[m][c] = 0.f;
        }
        __syncthreads();

        // Address overlaps (k.e, q.e, q.k); every wave reduces them itself.
        const float x0 = sk[lane] * se[lane] + sk[lane + 64] * se[lane + 64];
        const float x1 = sq[lane] * se[lane] + sq[lane + 64] * se[lane + 64];
        const float x2 = sq[lane] * sk[lane] + sq[lane + 64] * sk[lane + 64];
        float ke = wave_sum(x0), qe = wave_sum(x1), qk = wave_sum(x2);
        // LAYER: inverse norms of q, k, e (uniform), applied to every term below
        float inq = 1.f, ink = 1.f, ine = 1.f;
        if constexpr (LAYER) {
            inq = dec_inv_norm(wave_sum(sq[lane] * sq[lane] + sq[lane + 64] * sq[lane + 64]));
            ink = dec_inv_norm(wave_sum(sk[lane] * sk[lane] + sk[lane + 64] * sk[lane + 64]));
            ine = dec_inv_norm(wave_sum(se[lane] * se[lane] + se[lane + 64] * se[lane + 64]));
            ke *= ink * ine;
            qe *= inq * ine;
            qk *= inq * ink;
        }

        // Decay folded into the reductions: Sh[i][j] = a_i S[i][j].
        float pe[4] = {0, 0, 0, 0}, pk[4] = {0, 0, 0, 0}, pq[4] = {0, 0, 0, 0};
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int i = rg + RG * m;
            const float a = sa[i], ae = a * se[i], ak = a * sk[i], aq = a * sq[i];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                pe[c] += ae * s[m][c];
                pk[c] += ak * s[m][c];
                pq[c] += aq * s[m][c];
            }
        }
        // Sum over the row groups: two per wave (lane and lane^32), then the waves.
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            pe[c] += __shfl_xor(pe[c], 32, 64);
            pk[c] += __shfl_xor(pk[c], 32, 64);
            pq[c] += __shfl_xor(pq[c], 32, 64);
        }
        if (lane < 32) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                red[wave][0][4 * cq + c] = pe[c];
                red[wave][1][4 * cq + c] = pk[c];
                red[wave][2][4 * cq + c] = pq[c];
            }
        }
        __syncthreads();

        const float b = DPLR ? 1.f : beta[nh], g = DPLR ? 0.f : gamma[nh];
        float re[4], u[4], ov[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * cq + c;
            float r0 = 0.f, r1 = 0.f, r2 = 0.f;
#pragma unroll
            for (int w = 0; w < DEC_NW; ++w) {
                r0 += red[w][0][j];
                r1 += red[w][1][j];
                r2 += red[w][2][j];
            }
            r0 *= ine;
            r1 *= ink;
            r2 *= inq;
            re[c] = r0;
            const float vj = (j < dv) ? to_f32(v[nh * dv + j]) : 0.f;
            const float rk = DPLR ? r0 : r1 - g * ke * r0;   // DPLR: the read along a
            u[c] = b * (vj - rk);
            ov[c] = r2 - g * qe * r0 + qk * u[c];
        }
        if (rg == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * cq + c;
                if (j < dv) o[nh * dv + j] = from_f32<Tin>(ov[c]);
            }
        }

        // S_new = Sh - gamma e r_e^T + k u^T, written once.
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int i = rg + RG * m;
            const float a = sa[i], ge = g * se[i] * ine, kk = sk[i] * ink;
            float w[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) w[c] = a * s[m][c] - ge * re[c] + kk * u[c];
            if (FULL) {
                __builtin_nontemporal_store(f32x4{w[0], w[1], w[2], w[3]},
                                            reinterpret_cast<f32x4 *>(S_out + sbase + i * 128 + 4 * cq));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int j = 4 * cq + c;
                    if (i < dk && j < dv) S_out[sbase + (long)i * dv + j] = w[c];
                }
            }
        }
        __syncthreads();   // the shared vectors and partial sums are refilled next
    }
}

// decay: alpha (fp32, [N, H, d_k]), or with A_log != NULL the safe gate's
// input a (Tin, [N, Hk, d_k]) of the fused layer prologue; Hk == H otherwise.
// beta == NULL (and A_log == NULL) selects the DPLR update, erase vector in `e`.
template <typename Tin>
hipError_t launch_decode(const void *q, const void *k, const void *e, const void *v,
                         const void *decay, const float *A_log, const float *dt_bias,
                         const float *beta, const float *gamma, const float *S_in, float *S_out,
                         void *o, int N, int H, int Hk, int dk, int dv, hipStream_t stream) {
    int dev = 0, ncu = 256;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const long NH = (long)N * H;
    const dim3 grid((unsigned)(NH < 4L * ncu ? NH : 4L * ncu)), block(DEC_NT);   // four per compute unit
    const bool full = dk == 128 && dv == 128;
    const int mode = A_log ? DEC_LAYER : (beta ? DEC_PLAIN : DEC_DPLR);
    auto kern = full ? (mode == DEC_LAYER  ? eda_decode_kernel<Tin, true, DEC_LAYER>
                        : mode == DEC_DPLR ? eda_decode_kernel<Tin, true, DEC_DPLR>
                                           : eda_decode_kernel<Tin, true, DEC_PLAIN>)
                     : (mode == DEC_LAYER  ? eda_decode_kernel<Tin, false, DEC_LAYER>
                        : mode == DEC_DPLR ? eda_decode_kernel<Tin, false, DEC_DPLR>
                                           : eda_decode_kernel<Tin, false, DEC_PLAIN>);
    hipLaunchKernelGGL(kern, grid, block, 0, stream, (const Tin *)q, (const Tin *)k, (const Tin *)e,
                       (const Tin *)v, decay, A_log, dt_bias, beta, gamma, S_in, S_out, (Tin *)o, NH, H,
                       Hk, dk, dv);
    return hipGetLastError();
}

template hipError_t launch_decode<float>(const void *, const void *, const void *, const void *,
                                         const void *, const float *, const float *, const float *,
                                         const float *, const float *, float *, void *, int, int, int,
                                         int, int, hipStream_t);
template hipError_t launch_decode<bf16>(const void *, const void *, const void *, const void *,
                                        const void *, const float *, const float *, const float *,
                                        const float *, const float *, float *, void *, int, int, int,
                                        int, int, hipStream_t);

}  // namespace eda
