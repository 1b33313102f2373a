// eda_bwd.hip -- backward pass of the EDA recurrence (gradients of
// L = <o, dO> + <S_T, dS_T> with respect to every input), token by token.
//
// Forward, per token (EDA paper Sec. 3.3, Eqs. (9)-(13)):
//   Sh = Diag(alpha) S,  r_e = Sh^T e,  St = Sh - gamma e r_e^T,
//   r_k = St^T k = Sh^T k - gamma (k.e) r_e,  u = v - r_k,  S' = St + beta k u^T,  o = S'^T q.
// Reverse, with G = dL/dS' (carried from the next token) plus q dO^T:
//   dq = S' dO,  w = G^T k,  dv = beta w,  dbeta = w.u,
//   dk = beta (G u - St w),  dSt = G - beta k w^T,
//   z = dSt^T e = G^T e - beta (k.e) w,  dSh = dSt - gamma e z^T,
//   de = -gamma (dSt r_e + Sh z),  dgamma = -z.r_e,
//   dalpha = rowsum(dSh o S),  dL/dS = Diag(alpha) dSh.
// (the adjoint of each stage, written out; checked against the fp64 oracle's
// automatic differentiation of the same stages).
//
// Layout: one workgroup per (sequence, head, 16-column slice of the values),
// 128 threads, thread i owns key row i of the state slice and of G in
// registers.  Column sums (over key rows) are butterflies within a wave plus
// one exchange between the two waves; row sums (over the slice's columns)
// stay in the thread, so dq, dk, de, dalpha leave as per-slice partials
// that a second kernel adds up (deterministically).  The states are not
// stored per token: a first sweep writes fp32 checkpoints every CB tokens to
// the workspace, and the reverse sweep recomputes each CB-token segment's
// states (and their column sums) into LDS before walking it backwards.
#include "eda_common.h"

namespace eda {

constexpr int BW_NT = 128;   // threads: one key row each (d_k <= 128)
constexpr int BW_NC = 16;    // value columns per workgroup
constexpr int BW_CB = 4;     // tokens between state checkpoints (LDS: four workgroups per CU)
constexpr int BW_SP = BW_NC;            // LDS row of a state slice
constexpr int BW_RW = 2 * BW_NC + 4;    // recorded column sums per token: r_e, r_k, k.e

struct BwdArgs {
    const void *q, *k, *e, *v, *dO;
    const float *alpha, *beta, *gamma, *S0, *dSf;
    float *dv, *dS0;
    float *ckpt;                          // [NS][BH][NCK][128][16]
    float *pq, *pk, *pe, *pa;             // [NS][B*T*H][128] partial row sums
    float *pb, *pg;                       // [NS][B*T*H]
    int B, T, H, dk, dvd, NS, NCK;
};

// Sum over the 64 lanes of a wave, returned to every lane: prefix sums
// inside each row of 16 lanes with DPP row shifts, the rows combined with
// the row broadcasts, then lane 63 (which now holds the total) read back.
#define EDA_BW_DPP(v, ctrl, rmask) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), ctrl, rmask, 0xf, false))
__device__ __forceinline__ float wave_total(float x) {
    x += EDA_BW_DPP(x, 0x111, 0xf);   // row_shr:1
    x += EDA_BW_DPP(x, 0x112, 0xf);   // row_shr:2
    x += EDA_BW_DPP(x, 0x114, 0xf);   // row_shr:4
    x += EDA_BW_DPP(x, 0x118, 0xf);   // row_shr:8 (lane 15 of each row: the row's sum)
    x += EDA_BW_DPP(x, 0x142, 0xa);   // row_bcast:15 into rows 1 and 3
    x += EDA_BW_DPP(x, 0x143, 0xc);   // row_bcast:31 into rows 2 and 3
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
#undef EDA_BW_DPP

// Sum of x over the 128 threads of the workgroup (both waves), returned to
// every thread.  `xw` is a two-buffer exchange area [2][2][N]; `par` flips
// between calls so that a fast wave never overwrites values still being read.
template <int N>
__device__ __forceinline__ void wg_colsum(float (&x)[N], float *xw, int &par, int lane, int wave) {
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] = wave_total(x[n]);
    float *mine = xw + (par * 2 + wave) * N, *other = xw + (par * 2 + (wave ^ 1)) * N;
    if (lane == 0) {
#pragma unroll
        for (int n = 0; n < N; ++n) mine[n] = x[n];
    }
    __syncthreads();
#pragma unroll
    for (int n = 0; n < N; ++n) x[n] += other[n];
    par ^= 1;
}

template <typename Tin>
__global__ void __launch_bounds__(BW_NT) eda_bwd_kernel(BwdArgs a) {
    constexpr int NC = BW_NC, CB = BW_CB;
    __shared__ __attribute__((aligned(16))) float Sbuf[CB][BW_NT][BW_SP];   // states before each token
    __shared__ float rec[CB][BW_RW];                                         // their column sums
    __shared__ float xw[2 * 2 * (2 * NC + 1)];

    const int i = threadIdx.x, lane = i & 63, wave = i >> 6;
    const int s = blockIdx.x % a.NS, bh = blockIdx.x / a.NS;
    const int b = bh / a.H, h = bh % a.H, n0 = s * NC;
    const int BH = a.B * a.H;
    const long BTH = (long)a.B * a.T * a.H;
    const bool rok = i < a.dk;
    int par = 0;
    auto tokrow = [&](int t) { return ((long)b * a.T + t) * a.H + h; };
    auto ld = [](const void *p, long idx) { return to_f32(((const Tin *)p)[idx]); };

    float S[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
        S[j] = (a.S0 && rok && n0 + j < a.dvd) ? a.S0[((long)bh * a.dk + i) * a.dvd + n0 + j] : 0.f;

    // the inputs of one token for this thread's row and the slice's columns,
    // loaded one token ahead of their use
    struct Tok {
        float q, k, e, a, bt, gm, v[NC], dO[NC];
    };
    auto load_tok = [&](int t, bool with_out) {
        Tok x;
        const long row = tokrow(t);
        x.q = rok && with_out ? ld(a.q, row * a.dk + i) : 0.f;
        x.k = rok ? ld(a.k, row * a.dk + i) : 0.f;
        x.e = rok ? ld(a.e, row * a.dk + i) : 0.f;
        x.a = rok ? a.alpha[row * a.dk + i] : 1.f;
        x.bt = a.beta[row];
        x.gm = a.gamma[row];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            const bool cj = n0 + j < a.dvd;
            x.v[j] = cj ? ld(a.v, row * a.dvd + n0 + j) : 0.f;
            x.dO[j] = cj && with_out ? ld(a.dO, row * a.dvd + n0 + j) : 0.f;
        }
        return x;
    };

    // one token forward from S (the state before the token); the column sums
    // are returned in r (r_e, r_k, k.e)
    auto fwd_step = [&](float (&St)[NC], const Tok &x, float (&r)[2 * NC + 1]) {
        const float ki = x.k, ei = x.e, ai = x.a, bt = x.bt, gm = x.gm;
        float Sh[NC];
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            Sh[j] = ai * St[j];
            r[j] = ei * Sh[j];
            r[NC + j] = ki * Sh[j];
        }
        r[2 * NC] = ki * ei;
        wg_colsum<2 * NC + 1>(r, xw, par, lane, wave);
#pragma unroll
        for (int j = 0; j < NC; ++j) {
            r[NC + j] -= gm * r[2 * NC] * r[j];                        // r_k = Sh^T k - gamma (k.e) r_e
            St[j] = Sh[j] - gm * ei * r[j] + bt * ki * (x.v[j] - r[NC + j]);
        }
    };

    // ---- sweep 1: checkpoints of the state before tokens 0, CB, 2 CB, ...
    float *ck = a.ckpt + ((long)s * BH + bh) * a.NCK * (BW_NT * NC);
    {
        Tok cur = load_tok(0, false);
        for (int t = 0; t < a.T; ++t) {
            const Tok nxt = load_tok(t + 1 < a.T ? t + 1 : t, false);
            if (t % CB == 0) {
                float4 *dst = (float4 *)(ck + ((long)(t / CB) * BW_NT + i) * NC);
#pragma unroll
                for (int j = 0; j < NC; j += 4) dst[j / 4] = make_float4(S[j], S[j + 1], S[j + 2], S[j + 3]);
            }
            float r[2 * NC + 1];
            fwd_step(S, cur, r);
            cur = nxt;
        }
    }

    // ---- sweep 2: backwards over the segments
    float G[NC];
#pragma unroll
    for (int j = 0; j < NC; ++j)
        G[j] = (a.dSf && rok && n0 + j < a.dvd) ? a.dSf[((long)bh * a.dk + i) * a.dvd + n0 + j] : 0.f;
    for (int c = a.NCK - 1; c >= 0; --c) {
        const int t0 = c * CB, nt = min(CB, a.T - t0);
        {
            const float4 *src = (const float4 *)(ck + ((long)c * BW_NT + i) * NC);
#pragma unroll
            for (int j = 0; j < NC; j += 4) {
                const float4 x = src[j / 4];
                S[j] = x.x; S[j + 1] = x.y; S[j + 2] = x.z; S[j + 3] = x.w;
            }
        }
        {
            Tok cur = load_tok(t0, false);
            for (int tau = 0; tau < nt; ++tau) {
                const Tok nxt = load_tok(tau + 1 < nt ? t0 + tau + 1 : t0 + tau, false);
#pragma unroll
                for (int j = 0; j < NC; ++j) Sbuf[tau][i][j] = S[j];
                float r[2 * NC + 1];
                fwd_step(S, cur, r);
                if (i == 0) {
#pragma unroll
                    for (int n = 0; n < 2 * NC + 1; ++n) rec[tau][n] = r[n];
                }
                cur = nxt;
            }
        }
        __syncthreads();
        Tok cur = load_tok(t0 + nt - 1, true);
        for (int tau = nt - 1; tau >= 0; --tau) {
            const int t = t0 + tau;
            const long row = tokrow(t);
            const Tok nxt = load_tok(tau > 0 ? t - 1 : t, true);
            const float qi = cur.q, ki = cur.k, ei = cur.e, ai = cur.a, bt = cur.bt, gm = cur.gm;
            const float ke = rec[tau][2 * NC];
            float Sp[NC], Sh[NC], St[NC], up[NC], dO[NC], re[NC];
            float dq = 0.f;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                Sp[j] = Sbuf[tau][i][j];
                re[j] = rec[tau][j];
                const float vj = cur.v[j];
                dO[j] = cur.dO[j];
                Sh[j] = ai * Sp[j];
                St[j] = Sh[j] - gm * ei * re[j];
                up[j] = vj - rec[tau][NC + j];
                const float Sn = St[j] + bt * ki * up[j];
                G[j] += qi * dO[j];                                      // dL/dS' includes q dO^T
                dq += Sn * dO[j];
            }
            float wz[2 * NC + 1];
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                wz[j] = G[j] * ki;                                       // -> w = G^T k
                wz[NC + j] = G[j] * ei;                                  // -> G^T e
            }
            wz[2 * NC] = 0.f;
            wg_colsum<2 * NC + 1>(wz, xw, par, lane, wave);
            float dkp = 0.f, dep = 0.f, dap = 0.f, dbp = 0.f, dgp = 0.f;
#pragma unroll
            for (int j = 0; j < NC; ++j) {
                const float w = wz[j];
                const float z = wz[NC + j] - bt * ke * w;
                const float dSt = G[j] - bt * ki * w;
                const float dSh = dSt - gm * ei * z;
                dkp += G[j] * up[j] - St[j] * w;
                dep += dSt * re[j] + Sh[j] * z;
                dap += dSh * Sp[j];
                dbp += w * up[j];
                dgp += z * re[j];
                G[j] = ai * dSh;
            }
            const long pr = (long)s * BTH + row;
            if (i == 0) {
#pragma unroll
                for (int j = 0; j < NC; ++j)
                    if (n0 + j < a.dvd) a.dv[row * a.dvd + n0 + j] = bt * wz[j];
                a.pb[pr] = dbp;
                a.pg[pr] = -dgp;
            }
            a.pq[pr * BW_NT + i] = dq;
            a.pk[pr * BW_NT + i] = bt * dkp;
            a.pe[pr * BW_NT + i] = -gm * dep;
            a.pa[pr * BW_NT + i] = dap;
            cur = nxt;
        }
        __syncthreads();   // Sbuf and rec are refilled by the next segment
    }
    if (a.dS0 && rok) {
#pragma unroll
        for (int j = 0; j < NC; ++j)
            if (n0 + j < a.dvd) a.dS0[((long)bh * a.dk + i) * a.dvd + n0 + j] = G[j];
    }
}

// Sum the per-slice partials: dq, dk, de, dalpha over (B*T*H, d_k), dbeta,
// dgamma over B*T*H.
__global__ void __launch_bounds__(256) eda_bwd_reduce(const float *pq, const float *pk, const float *pe,
                                                     const float *pa, const float *pb, const float *pg,
                                                     float *dq, float *dk, float *de, float *dalpha,
                                                     float *dbeta, float *dgamma, long BTH, int dkk, int NS) {
    const long n = BTH * dkk;
    for (long idx = blockIdx.x * 256L + threadIdx.x; idx < n + BTH; idx += (long)gridDim.x * 256) {
        if (idx < n) {
            const long r = idx / dkk, i = idx % dkk;
            float sq = 0.f, sk = 0.f, se = 0.f, sa = 0.f;
            for (int s = 0; s < NS; ++s) {
                const long p = ((long)s * BTH + r) * BW_NT + i;
                sq += pq[p]; sk += pk[p]; se += pe[p]; sa += pa[p];
            }
            dq[idx] = sq; dk[idx] = sk; de[idx] = se; dalpha[idx] = sa;
        } else {
            const long r = idx - n;
            float sb = 0.f, sg = 0.f;
            for (int s = 0; s < NS; ++s) {
                sb += pb[(long)s * BTH + r];
                sg += pg[(long)s * BTH + r];
            }
            dbeta[r] = sb; dgamma[r] = sg;
        }
    }
}

size_t bwd_ws_bytes(int B, int T, int H, int dk, int dv) {
    (void)dk;
    const long NS = (dv + BW_NC - 1) / BW_NC, NCK = (T + BW_CB - 1) / BW_CB, BTH = (long)B * T * H;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    return al((size_t)NS * B * H * NCK * BW_NT * BW_NC * 4) + 4 * al((size_t)NS * BTH * BW_NT * 4) +
           2 * al((size_t)NS * BTH * 4);
}

template <typename Tin>
hipError_t launch_bwd(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                      const float *beta, const float *gamma, const float *S0, const void *dO,
                      const float *dSf, float *dq, float *dk, float *de, float *dv, float *dalpha,
                      float *dbeta, float *dgamma, float *dS0, int B, int T, int H, int dkk, int dvd,
                      void *ws, hipStream_t stream) {
    const int NS = (dvd + BW_NC - 1) / BW_NC, NCK = (T + BW_CB - 1) / BW_CB;
    const long BTH = (long)B * T * H;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    char *w = (char *)ws;
    BwdArgs a;
    a.q = q; a.k = k; a.e = e; a.v = v; a.dO = dO;
    a.alpha = alpha; a.beta = beta; a.gamma = gamma; a.S0 = S0; a.dSf = dSf;
    a.dv = dv; a.dS0 = dS0;
    a.ckpt = (float *)w;
    w += al((size_t)NS * B * H * NCK * BW_NT * BW_NC * 4);
    float **parts[4] = {&a.pq, &a.pk, &a.pe, &a.pa};
    for (float **p : parts) {
        *p = (float *)w;
        w += al((size_t)NS * BTH * BW_NT * 4);
    }
    a.pb = (float *)w;
    w += al((size_t)NS * BTH * 4);
    a.pg = (float *)w;
    a.B = B; a.T = T; a.H = H; a.dk = dkk; a.dvd = dvd; a.NS = NS; a.NCK = NCK;
    hipLaunchKernelGGL(eda_bwd_kernel<Tin>, dim3((unsigned)((long)B * H * NS)), dim3(BW_NT), 0, stream, a);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const long n = BTH * dkk + BTH;
    const unsigned grid = (unsigned)((n + 255) / 256 < 8192 ? (n + 255) / 256 : 8192);
    hipLaunchKernelGGL(eda_bwd_reduce, dim3(grid), dim3(256), 0, stream, a.pq, a.pk, a.pe, a.pa, a.pb, a.pg,
                       dq, dk, de, dalpha, dbeta, dgamma, BTH, dkk, NS);
    return hipGetLastError();
}

template hipError_t launch_bwd<float>(const void *, const void *, const void *, const void *, const float *,
                                      const float *, const float *, const float *, const void *, const float *,
                                      float *, float *, float *, float *, float *, float *, float *, float *,
                                      int, int, int, int, int, void *, hipStream_t);
template hipError_t launch_bwd<bf16>(const void *, const void *, const void *, const void *, const float *,
                                     const float *, const float *, const float *, const void *, const float *,
                                     float *, float *, float *, float *, float *, float *, float *, float *,
                                     int, int, int, int, int, void *, hipStream_t);

}  // namespace eda
