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
// 256 threads: the two adjacent lanes 2i and 2i + 1 own key row i of the
// state slice and of G in registers, 8 columns each (two waves per SIMD
// with two workgroups per CU).  Column sums (over key rows) go through LDS:
// adjacent rows are paired within the wave, the 64 x 32 pair sums are
// transposed through LDS, eight threads add up each column, and the totals
// come back to the threads that need them.  Row sums (over the slice's
// columns) take one lane swap, so dq, dk, de, dalpha leave as per-slice
// partials that a second kernel adds up (deterministically).  The states are not stored per token: a first sweep
// writes fp32 checkpoints every CB tokens and each token's column sums to
// the workspace, and the reverse sweep recomputes each CB-token segment's
// states from them (no reductions) into LDS before walking it backwards.
// Every input of a segment is fetched a whole segment ahead of its use.
#include <type_traits>

#include "eda_common.h"

namespace eda {

constexpr int BW_ROWS = 128;  // key rows (d_k <= 128)
constexpr int BW_NT = 256;    // threads: two per key row
constexpr int BW_NC = 16;     // value columns per workgroup
constexpr int BW_HC = 8;      // value columns per thread
constexpr int BW_CB = 8;     // tokens per segment: between state checkpoints, and per input fetch
constexpr int BW_SP = BW_NC;            // LDS row of a state slice
constexpr int BW_NR = 2 * BW_NC + 1;    // recorded column sums per token: r_e, r_k, k.e
constexpr int BW_RW = 2 * BW_NC + 4;    // their LDS row (16-byte multiple)

struct BwdArgs {
    const void *q, *k, *e, *v, *dO;
    const float *alpha, *beta, *gamma, *S0, *dSf;
    float *dv, *dS0;
    float *ckpt;                          // [NS][BH][NCK][128][16]
    float *recg;                          // [NS][BH][T][NR] column sums of each token
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

// Sum of one lane with its neighbour (lanes 2i, 2i + 1): the two halves of a
// key row.  Both lanes get the same bits.
__device__ __forceinline__ float pair_sum(float x) {
    return x + __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xb1, 0xf, 0xf,
                                                                     false));   // quad_perm [1,0,3,2]
}

// Column sums over the 128 key rows of the two quantities a and b, 16
// columns each; thread t holds row t/2, columns 8 (t & 1) .. + 7 of both in
// x[0..7] (a) and x[8..15] (b), and gets back the totals of those columns.
// Steps: rows 2m and 2m + 1 (lanes t and t ^ 2) add up with a DPP quad swap;
// of the four lanes of a row pair, those with bit 1 clear write their a
// values and the others their b values to row m of Xs [64][33]; after a
// barrier thread t adds column t % 32 over 8 of those rows, the two such
// partials of a wave meet with a lane swap, and the four waves' sums go
// through Ps [4][36], added up in wave order.  With EXTRA, `extra` (a
// per-row value counted once per row) is summed too.  Xs and Ps are read
// only between this call's two barriers and after the second, so
// consecutive calls need no further synchronisation.
constexpr int BW_XS = 33, BW_PS = 36;
template <bool EXTRA>
__device__ __forceinline__ void wg_colsum(float (&x)[16], float &extra, float *Xs, float *Ps, int t, int lane,
                                          int wave) {
#pragma unroll
    for (int n = 0; n < 16; ++n)
        x[n] += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x[n]), 0x4e, 0xf,
                                                                      0xf, false));   // quad_perm [2,3,0,1]
    {
        // (a bit-mask select: a conditional choice between the two groups
        // would be compiled into an indexed access to a stack copy of x)
        const int sel = (t >> 1) & 1, msk = -sel;
        float *row = Xs + (t >> 2) * BW_XS + 16 * sel + 8 * (t & 1);
#pragma unroll
        for (int n = 0; n < 8; ++n) {
            const int lo = __builtin_bit_cast(int, x[n]), hi = __builtin_bit_cast(int, x[8 + n]);
            row[n] = __builtin_bit_cast(float, (lo & ~msk) | (hi & msk));
        }
    }
    if (EXTRA) extra = wave_total(extra);
    __syncthreads();
    {
        const int j = t & 31, p = t >> 5;
        const float *col = Xs + 8 * p * BW_XS + j;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int r = 0; r < 8; r += 2) {
            s0 += col[r * BW_XS];
            s1 += col[(r + 1) * BW_XS];
        }
        float s = s0 + s1;
        s += __shfl_xor(s, 32, 64);
        if (lane < 32) Ps[wave * BW_PS + j] = s;
        if (EXTRA && lane == 0) Ps[wave * BW_PS + 32] = extra;
    }
    __syncthreads();
    const int c0 = 8 * (t & 1);
#pragma unroll
    for (int g = 0; g < 2; ++g) {
#pragma unroll
        for (int n = 0; n < 8; n += 4) {
            const int o = 16 * g + c0 + n;
            float4 acc = *(const float4 *)(Ps + o);
#pragma unroll
            for (int w = 1; w < 4; ++w) {
                const float4 u = *(const float4 *)(Ps + w * BW_PS + o);
                acc.x += u.x; acc.y += u.y; acc.z += u.z; acc.w += u.w;
            }
            x[8 * g + n] = acc.x; x[8 * g + n + 1] = acc.y; x[8 * g + n + 2] = acc.z; x[8 * g + n + 3] = acc.w;
        }
    }
    if (EXTRA) extra = ((Ps[32] + Ps[BW_PS + 32]) + Ps[2 * BW_PS + 32]) + Ps[3 * BW_PS + 32];
}
// Total number n (0..31) of the last column sum, read back from Ps in the
// same order of addition.
__device__ __forceinline__ float colsum_total(const float *Ps, int n) {
    return ((Ps[n] + Ps[BW_PS + n]) + Ps[2 * BW_PS + n]) + Ps[3 * BW_PS + n];
}

template <typename Tin>
__global__ void __launch_bounds__(BW_NT) eda_bwd_kernel(BwdArgs a) {
    constexpr int NC = BW_NC, HC = BW_HC, CB = BW_CB, NR = BW_NR, RW = BW_RW, ROWS = BW_ROWS;
    constexpr int NCOL = CB * 2 * NC, CPT = NCOL / BW_NT;          // slice entries per thread
    constexpr int NREC = CB * NR, RPT = (NREC + BW_NT - 1) / BW_NT;  // recorded sums per thread
    static_assert(NCOL % BW_NT == 0 && 2 * CB <= BW_NT && 2 * HC == NC && NC == 16, "segment staging split");
    __shared__ __attribute__((aligned(16))) float Sbuf[CB][ROWS][BW_SP];    // states before each token
    __shared__ __attribute__((aligned(16))) float rec[2][CB][RW];           // their column sums, two segments
    __shared__ __attribute__((aligned(16))) float colb[2][CB][2][NC];       // v and dO slices, two segments
    __shared__ float unib[2][CB][2];                                        // beta and gamma, two segments
    __shared__ __attribute__((aligned(16))) float Xs[64 * BW_XS];
    __shared__ __attribute__((aligned(16))) float Ps[4 * BW_PS];

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int i = t >> 1, hf = t & 1, c0 = HC * hf;   // key row, column half, its first column
    const int s = blockIdx.x % a.NS, bh = blockIdx.x / a.NS;
    const int b = bh / a.H, h = bh % a.H, n0 = s * NC;
    const int BH = a.B * a.H;
    const long BTH = (long)a.B * a.T * a.H;
    const bool rok = i < a.dk;
    const int ri = rok ? i : a.dk - 1;   // a valid row to read for padded rows
    auto tokrow = [&](int tk) { return ((long)b * a.T + tk) * a.H + h; };
    auto tclamp = [&](int tk) { return tk < a.T ? tk : a.T - 1; };

    float S[HC];
#pragma unroll
    for (int n = 0; n < HC; ++n) {
        const int col = n0 + c0 + n;
        S[n] = (a.S0 && rok && col < a.dvd) ? a.S0[((long)bh * a.dk + i) * a.dvd + col] : 0.f;
    }

    float *ck = a.ckpt + ((long)s * BH + bh) * a.NCK * (ROWS * NC);
    float *rg = a.recg + ((long)s * BH + bh) * a.T * NR;

    // The inputs of one segment of CB tokens, fetched a whole segment ahead
    // of their use, raw and from clamped (always valid) addresses so that no
    // load waits before the next segment: this thread's key row of every
    // token; CPT entries of the segment's value / output-gradient slice and
    // one beta or gamma (threads below 2 CB), which go to LDS for everyone;
    // in the reverse sweep also the checkpoint row half and RPT recorded
    // sums.  Padding (rows past d_k, columns past d_v) is zeroed when
    // committed; tokens past the end are never used.
    struct Seg {
        Tin q[CB], k[CB], e[CB];
        float al[CB];
        Tin cv[CPT];
        float u;
        float ckp[HC];
        float rc[RPT];
    };
    auto load_seg = [&](int c, auto rev_c) __attribute__((always_inline)) {
        constexpr bool REV = decltype(rev_c)::value;
        Seg x;
        const int t0 = c * CB;
#pragma unroll
        for (int tau = 0; tau < CB; ++tau) {
            const long ro = tokrow(tclamp(t0 + tau)) * a.dk + ri;
            if (REV) x.q[tau] = ((const Tin *)a.q)[ro];
            x.k[tau] = ((const Tin *)a.k)[ro];
            x.e[tau] = ((const Tin *)a.e)[ro];
            x.al[tau] = a.alpha[ro];
        }
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const int f = t + BW_NT * m, tau = f / (2 * NC), which = (f / NC) & 1, j = f % NC;
            const int col = n0 + j < a.dvd ? n0 + j : a.dvd - 1;
            const Tin *src = (REV && which) ? (const Tin *)a.dO : (const Tin *)a.v;
            x.cv[m] = src[tokrow(tclamp(t0 + tau)) * a.dvd + col];
        }
        x.u = ((t & 1) ? a.gamma : a.beta)[tokrow(tclamp(t0 + ((t >> 1) % CB)))];
        if (REV) {
            const float4 *src = (const float4 *)(ck + ((long)c * ROWS + i) * NC + c0);
#pragma unroll
            for (int n = 0; n < HC; n += 4) {
                const float4 y = src[n / 4];
                x.ckp[n] = y.x; x.ckp[n + 1] = y.y; x.ckp[n + 2] = y.z; x.ckp[n + 3] = y.w;
            }
            const long last = (long)a.T * NR - 1;
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const long f = (long)t0 * NR + t + BW_NT * m;
                x.rc[m] = rg[f < last ? f : last];
            }
        }
        return x;
    };
    // the shared part of a fetched segment -> LDS buffers `buf`; the row part
    // -> the token queues
    float qr[CB], kr[CB], er[CB], ar[CB];
    auto commit = [&](const Seg &x, int buf, auto rev_c) __attribute__((always_inline)) {
        constexpr bool REV = decltype(rev_c)::value;
#pragma unroll
        for (int m = 0; m < CPT; ++m) {
            const int f = t + BW_NT * m, which = (f / NC) & 1, j = f % NC;
            const bool ok = n0 + j < a.dvd && (REV || which == 0);
            (&colb[buf][0][0][0])[f] = ok ? to_f32(x.cv[m]) : 0.f;
        }
        if (t < 2 * CB) (&unib[buf][0][0])[t] = x.u;
        if (REV) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int f = t + BW_NT * m;
                if (f < NREC) rec[buf][f / NR][f % NR] = x.rc[m];
            }
        }
#pragma unroll
        for (int tau = 0; tau < CB; ++tau) {
            qr[tau] = REV && rok ? to_f32(x.q[tau]) : 0.f;
            kr[tau] = rok ? to_f32(x.k[tau]) : 0.f;
            er[tau] = rok ? to_f32(x.e[tau]) : 0.f;
            ar[tau] = rok ? x.al[tau] : 1.f;
        }
    };
    // The token loops stay rolled (the kernel's code must fit the instruction
    // cache), so the per-token row inputs are queues rotated by one token per
    // step: the forward walk reads slot 0 and rotates left, which leaves token
    // nt - 1 in slot CB - 1 for the backward walk, which rotates right.
    auto rotl = [](float (&x)[CB]) {
        const float f = x[0];
#pragma unroll
        for (int j = 0; j + 1 < CB; ++j) x[j] = x[j + 1];
        x[CB - 1] = f;
    };
    auto rotr = [](float (&x)[CB]) {
        const float l = x[CB - 1];
#pragma unroll
        for (int j = CB - 1; j > 0; --j) x[j] = x[j - 1];
        x[0] = l;
    };
    using Fwd = std::integral_constant<bool, false>;
    using Rev = std::integral_constant<bool, true>;

    // ---- sweep 1: checkpoints of the state before tokens 0, CB, 2 CB, ...,
    // and every token's column sums r_e, r_k (after the erase), k.e
    {
        Seg nxt = load_seg(0, Fwd{});
        for (int c = 0; c < a.NCK; ++c) {
            const int t0 = c * CB, nt = min(CB, a.T - t0), buf = c & 1;
            commit(nxt, buf, Fwd{});
            __syncthreads();   // this segment's slice is in LDS; the previous one is no longer read
            if (c + 1 < a.NCK) nxt = load_seg(c + 1, Fwd{});
            float4 *dst = (float4 *)(ck + ((long)c * ROWS + i) * NC + c0);
#pragma unroll
            for (int n = 0; n < HC; n += 4) dst[n / 4] = make_float4(S[n], S[n + 1], S[n + 2], S[n + 3]);
#pragma unroll 1
            for (int tau = 0; tau < nt; ++tau) {
                const float ki = kr[0], ei = er[0], ai = ar[0];
                const float bt = unib[buf][tau][0], gm = unib[buf][tau][1];
                const float *vs = colb[buf][tau][0] + c0;
                float Sh[HC], r[2 * HC];
#pragma unroll
                for (int n = 0; n < HC; ++n) {
                    Sh[n] = ai * S[n];
                    r[n] = ei * Sh[n];
                    r[HC + n] = ki * Sh[n];
                }
                float ke = hf ? 0.f : ki * ei;
                wg_colsum<true>(r, ke, Xs, Ps, t, lane, wave);
#pragma unroll
                for (int n = 0; n < HC; ++n) {
                    r[HC + n] -= gm * ke * r[n];                          // r_k = Sh^T k - gamma (k.e) r_e
                    S[n] = Sh[n] - gm * ei * r[n] + bt * ki * (vs[n] - r[HC + n]);
                }
                // thread n < 33 records sum n (the same additions, in the same order)
                if (t < NR) {
                    float x = ke;
                    if (t < NC) x = colsum_total(Ps, t);
                    else if (t < 2 * NC) x = colsum_total(Ps, t) - gm * ke * colsum_total(Ps, t - NC);
                    rg[(long)(t0 + tau) * NR + t] = x;
                }
                rotl(kr); rotl(er); rotl(ar);
            }
        }
    }

    // ---- sweep 2: backwards over the segments
    float G[HC];
#pragma unroll
    for (int n = 0; n < HC; ++n) {
        const int col = n0 + c0 + n;
        G[n] = (a.dSf && rok && col < a.dvd) ? a.dSf[((long)bh * a.dk + i) * a.dvd + col] : 0.f;
    }
    // (sweep 1's stores of the checkpoints and sums are complete: the
    // workgroup barriers since then wait for every wave's memory operations)
    __syncthreads();
    Seg nxt = load_seg(a.NCK - 1, Rev{});
    for (int c = a.NCK - 1; c >= 0; --c) {
        const int t0 = c * CB, nt = min(CB, a.T - t0), buf = c & 1;
        commit(nxt, buf, Rev{});
#pragma unroll
        for (int n = 0; n < HC; ++n) S[n] = nxt.ckp[n];
        __syncthreads();   // slice and sums in LDS; the previous segment's buffers no longer read
        if (c > 0) nxt = load_seg(c - 1, Rev{});
        // recompute the segment's states into this thread's part of Sbuf
#pragma unroll 1
        for (int tau = 0; tau < nt; ++tau) {
#pragma unroll
            for (int n = 0; n < HC; n += 4)
                *(float4 *)&Sbuf[tau][i][c0 + n] = make_float4(S[n], S[n + 1], S[n + 2], S[n + 3]);
            const float ki = kr[0], ei = er[0], ai = ar[0];
            const float bt = unib[buf][tau][0], gm = unib[buf][tau][1];
            const float *vs = colb[buf][tau][0] + c0, *rr = rec[buf][tau] + c0;
#pragma unroll
            for (int n = 0; n < HC; ++n) S[n] = ai * S[n] - gm * ei * rr[n] + bt * ki * (vs[n] - rr[NC + n]);
            rotl(qr); rotl(kr); rotl(er); rotl(ar);
        }
#pragma unroll 1
        for (int tau = nt - 1; tau >= 0; --tau) {
            const long row = tokrow(t0 + tau);
            const float qi = qr[CB - 1], ki = kr[CB - 1], ei = er[CB - 1], ai = ar[CB - 1];
            rotr(qr); rotr(kr); rotr(er); rotr(ar);
            const float bt = unib[buf][tau][0], gm = unib[buf][tau][1];
            const float *vs = colb[buf][tau][0] + c0, *dOs = colb[buf][tau][1] + c0, *rr = rec[buf][tau] + c0;
            const float ke = rec[buf][tau][2 * NC];
            float Sp[HC], Sh[HC], St[HC], up[HC], re[HC];
            float dq = 0.f;
#pragma unroll
            for (int n = 0; n < HC; ++n) {
                Sp[n] = Sbuf[tau][i][c0 + n];
                re[n] = rr[n];
                Sh[n] = ai * Sp[n];
                St[n] = Sh[n] - gm * ei * re[n];
                up[n] = vs[n] - rr[NC + n];
                const float Sn = St[n] + bt * ki * up[n];
                G[n] += qi * dOs[n];                                     // dL/dS' includes q dO^T
                dq += Sn * dOs[n];
            }
            float wz[2 * HC], unused = 0.f;
#pragma unroll
            for (int n = 0; n < HC; ++n) {
                wz[n] = G[n] * ki;                                       // -> w = G^T k
                wz[HC + n] = G[n] * ei;                                  // -> G^T e
            }
            wg_colsum<false>(wz, unused, Xs, Ps, t, lane, wave);
            float dkp = 0.f, dep = 0.f, dap = 0.f, dbp = 0.f, dgp = 0.f, dvj = 0.f;
#pragma unroll
            for (int n = 0; n < HC; ++n) {
                const float w = wz[n];
                const float z = wz[HC + n] - bt * ke * w;
                const float dSt = G[n] - bt * ki * w;
                const float dSh = dSt - gm * ei * z;
                dkp += G[n] * up[n] - St[n] * w;
                dep += dSt * re[n] + Sh[n] * z;
                dap += dSh * Sp[n];
                dbp += w * up[n];
                dgp += z * re[n];
                G[n] = ai * dSh;
                dvj = (t >> 1) == n ? w : dvj;   // threads t < 16: column 8 (t & 1) + t / 2
            }
            dq = pair_sum(dq);
            dkp = pair_sum(dkp);
            dep = pair_sum(dep);
            dap = pair_sum(dap);
            dbp = pair_sum(dbp);
            dgp = pair_sum(dgp);
            const long pr = (long)s * BTH + row;
            if (t < NC) {
                const int col = n0 + c0 + (t >> 1);
                if (col < a.dvd) a.dv[row * a.dvd + col] = bt * dvj;
            }
            if (t == NC) a.pb[pr] = dbp;
            if (t == NC + 2) a.pg[pr] = -dgp;
            if (hf == 0) {
                a.pq[pr * ROWS + i] = dq;
                a.pk[pr * ROWS + i] = bt * dkp;
            } else {
                a.pe[pr * ROWS + i] = -gm * dep;
                a.pa[pr * ROWS + i] = dap;
            }
        }
    }
    if (a.dS0 && rok) {
#pragma unroll
        for (int n = 0; n < HC; ++n) {
            const int col = n0 + c0 + n;
            if (col < a.dvd) a.dS0[((long)bh * a.dk + i) * a.dvd + col] = G[n];
        }
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
                const long p = ((long)s * BTH + r) * BW_ROWS + i;
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
    return al((size_t)NS * B * H * NCK * BW_ROWS * BW_NC * 4) + al((size_t)NS * BTH * BW_NR * 4) +
           4 * al((size_t)NS * BTH * BW_ROWS * 4) + 2 * al((size_t)NS * BTH * 4);
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
    w += al((size_t)NS * B * H * NCK * BW_ROWS * BW_NC * 4);
    a.recg = (float *)w;
    w += al((size_t)NS * BTH * BW_NR * 4);
    float **parts[4] = {&a.pq, &a.pk, &a.pe, &a.pa};
    for (float **p : parts) {
        *p = (float *)w;
        w += al((size_t)NS * BTH * BW_ROWS * 4);
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
