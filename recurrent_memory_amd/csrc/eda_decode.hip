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
// kernel is therefore laid out for HBM streaming.  A persistent grid walks
// the states; per state each thread owns a 4-column strip of R rows (rows
// rg + RG m), so every wavefront load/store instruction touches 1 KB of
// contiguous memory, and the loop is software-pipelined (below) so that the
// next state's loads are in flight while this one is reduced and written.
// The state is touched exactly once per step, so its loads and stores carry
// the non-temporal hint (no reuse is expected from the caches; measured ~15%
// faster than plain accesses at 8192 states of 64 KB).
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
#include <type_traits>

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

constexpr int DEC_PLAIN = 0, DEC_LAYER = 1, DEC_DPLR = 2;

// Workgroup shape.  The 128-square plain and DPLR variants run 1024 threads
// (4 rows per thread, one workgroup per CU): the strips of the state in hand
// and of the next one both fit in the 128 VGPRs a 1024-thread workgroup
// allows.  The layer and ragged variants need more registers than that and
// keep 512 threads (8 rows per thread).
template <bool FULL, int MODE>
struct DecShape {
    static constexpr int NT = FULL && MODE != DEC_LAYER ? 1024 : 512;   // threads per workgroup
    static constexpr int RG = NT / 32;                                   // row groups (32 column quads per row)
    static constexpr int R = 128 / RG;                                   // rows per thread
    static constexpr int NW = NT / 64;                                   // wavefronts
};

// Software pipelining: every input of state n + 1 (its token vectors, gates,
// value and state strip) is fetched at the start of state n, before its
// reductions and its stores.  Vector
// loads and stores share one in-order counter, so a wait for a load issued
// after those stores would also wait for them; issued before, the loads are
// waited for at the top of the next state while the stores stay in flight.
// States never overlap in memory, so fetching state n + 1 before writing state
// n is exact also when S_out == S_in.
template <typename Tin, bool FULL, int MODE>
__global__ void __launch_bounds__((DecShape<FULL, MODE>::NT))
    __attribute__((amdgpu_waves_per_eu(DecShape<FULL, MODE>::NT == 1024 ? 4 : 1)))
eda_decode_kernel(const Tin *__restrict__ q, const Tin *__restrict__ k, const Tin *__restrict__ e,
                  const Tin *__restrict__ v, const void *__restrict__ decay,
                  const float *__restrict__ A_log, const float *__restrict__ dt_bias,
                  const float *__restrict__ beta, const float *__restrict__ gamma,
                  const float *S_in, float *S_out, Tin *__restrict__ o, long NH, int H, int Hk,
                  int dk, int dv) {
    using SH = DecShape<FULL, MODE>;
    constexpr int R = SH::R, RG = SH::RG, NW = SH::NW;
    constexpr bool LAYER = MODE == DEC_LAYER, DPLR = MODE == DEC_DPLR;
    __shared__ float sq[128], sk[128], se[128], sa[128];
    __shared__ float red[NW][3][128];
    __shared__ float fin[3][128];   // the three reductions, summed over the waves

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cq = tid & 31, rg = tid >> 5;  // column quad, row group
    if (FULL) { dk = 128; dv = 128; }
    const int grp = H / Hk;

    // inputs of one state, in registers from the fetch to their use; the token
    // values stay raw (loaded from clamped, always valid addresses) and are
    // converted and masked where they are used, so nothing waits for them
    // before the previous state's stores are issued
    using DT = typename std::conditional<LAYER, Tin, float>::type;   // decay input
    Tin rq = Tin(0), rk = Tin(0), rce = Tin(0), rv[4] = {Tin(0), Tin(0), Tin(0), Tin(0)};
    DT ra = DT(0);
    float rA = 0.f, rB = 0.f, xb = 0.f, xg = 0.f;
    float s[R][4], sn[R][4];   // the strip of the state in hand and of the next one
    auto fetch = [&](long nh, float (&st)[R][4]) __attribute__((always_inline)) {
        const long hk = (nh % H) / grp, nk = (nh / H) * Hk + hk;
        if (tid < 128) {
            const long ch = nk * dk + (tid < dk ? tid : 0);
            rq = q[ch];
            rk = k[ch];
            rce = e[ch];
            ra = ((const DT *)decay)[ch];
            if constexpr (LAYER) {
                rA = A_log[hk * dk + (tid < dk ? tid : 0)];
                rB = dt_bias[hk * dk + (tid < dk ? tid : 0)];
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * cq + c;
            rv[c] = v[nh * dv + (j < dv ? j : 0)];
        }
        xb = DPLR ? 1.f : beta[nh];
        xg = DPLR ? 0.f : gamma[nh];
        const long sbase = nh * (long)dk * dv;
        if (S_in) {
            if (FULL) {
#pragma unroll
                for (int m = 0; m < R; ++m) {
                    const f32x4 x = __builtin_nontemporal_load(
                        reinterpret_cast<const f32x4 *>(S_in + sbase + (rg + RG * m) * 128 + 4 * cq));
                    st[m][0] = x[0]; st[m][1] = x[1]; st[m][2] = x[2]; st[m][3] = x[3];
                }
            } else {
#pragma unroll
                for (int m = 0; m < R; ++m)
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const int i = rg + RG * m, j = 4 * cq + c;
                        st[m][c] = (i < dk && j < dv) ? S_in[sbase + (long)i * dv + j] : 0.f;
                    }
            }
        } else {
#pragma unroll
            for (int m = 0; m < R; ++m)
#pragma unroll
                for (int c = 0; c < 4; ++c) st[m][c] = 0.f;
        }
    };

    long nh = blockIdx.x;
    if (nh < NH) {
        fetch(nh, s);
        // The first state's inputs are consumed (unused) here, so the compiler
        // waits for them once, before the loop; the waits at the top of the loop
        // are then counted for the loop path alone, where the previous state's
        // stores follow the fetch and stay in flight.
        asm volatile("" ::"v"((uint32_t)rq), "v"((uint32_t)rk), "v"((uint32_t)rce), "v"(ra), "v"(rA), "v"(rB),
                     "v"(xb), "v"(xg));
        asm volatile("" ::"v"((uint32_t)rv[0]), "v"((uint32_t)rv[1]), "v"((uint32_t)rv[2]), "v"((uint32_t)rv[3]));
#pragma unroll
        for (int m = 0; m < R; ++m) asm volatile("" ::"v"(s[m][0]), "v"(s[m][1]), "v"(s[m][2]), "v"(s[m][3]));
    }
    for (; nh < NH; nh += gridDim.x) {
        if (tid < 128) {
            const bool ok = tid < dk;
            sq[tid] = ok ? to_f32(rq) : 0.f;
            sk[tid] = ok ? to_f32(rk) : 0.f;
            se[tid] = ok ? to_f32(rce) : 0.f;
            if constexpr (LAYER) sa[tid] = ok ? dec_safe_gate(to_f32(ra), rA, rB) : 0.f;
            else sa[tid] = ok ? ra : 0.f;
        }
        const float b = xb, g = xg;
        float vv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) vv[c] = (4 * cq + c < dv) ? to_f32(rv[c]) : 0.f;
        // the next state's inputs, fetched now: they arrive while this state is
        // reduced and updated, and they precede this state's stores
        const long cur = nh, nxt = nh + gridDim.x;
        if (nxt < NH) fetch(nxt, sn);
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
        // each of 384 threads adds one (reduction, column) over the waves, in wave order
        if (tid < 384) {
            const int ty = tid >> 7, j = tid & 127;
            float acc = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) acc += red[w][ty][j];
            fin[ty][j] = acc;
        }
        __syncthreads();

        float re[4], u[4], ov[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int j = 4 * cq + c;
            float r0 = fin[0][j], r1 = fin[1][j], r2 = fin[2][j];
            r0 *= ine;
            r1 *= ink;
            r2 *= inq;
            re[c] = r0;
            const float rk = DPLR ? r0 : r1 - g * ke * r0;   // DPLR: the read along a
            u[c] = b * (vv[c] - rk);
            ov[c] = r2 - g * qe * r0 + qk * u[c];
        }

        // S_new = Sh - gamma e r_e^T + k u^T
        float w[R][4];
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int i = rg + RG * m;
            const float a = sa[i], ge = g * se[i] * ine, kk = sk[i] * ink;
#pragma unroll
            for (int c = 0; c < 4; ++c) w[m][c] = a * s[m][c] - ge * re[c] + kk * u[c];
        }
        // the shared vectors and partial sums are refilled by the next state
        __syncthreads();

        const long sbase = cur * (long)dk * dv;
#pragma unroll
        for (int m = 0; m < R; ++m) {
            const int i = rg + RG * m;
            if (FULL) {
                __builtin_nontemporal_store(f32x4{w[m][0], w[m][1], w[m][2], w[m][3]},
                                            reinterpret_cast<f32x4 *>(S_out + sbase + i * 128 + 4 * cq));
            } else {
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const int j = 4 * cq + c;
                    if (i < dk && j < dv) S_out[sbase + (long)i * dv + j] = w[m][c];
                }
            }
        }
        if (rg == 0) {
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int j = 4 * cq + c;
                if (j < dv) o[cur * dv + j] = from_f32<Tin>(ov[c]);
            }
        }
#pragma unroll
        for (int m = 0; m < R; ++m)
#pragma unroll
            for (int c = 0; c < 4; ++c) s[m][c] = sn[m][c];
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
    const bool full = dk == 128 && dv == 128;
    const int mode = A_log ? DEC_LAYER : (beta ? DEC_PLAIN : DEC_DPLR);
    // a persistent grid: one 1024-thread workgroup per compute unit, or four
    // 512-thread workgroups launched per compute unit (one or two resident)
    const bool wide = full && mode != DEC_LAYER;
    const long per = wide ? (long)ncu : 4L * ncu;
    const dim3 grid((unsigned)(NH < per ? NH : per)), block(wide ? 1024 : 512);
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
