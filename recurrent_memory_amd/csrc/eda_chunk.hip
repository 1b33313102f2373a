// eda_chunk.hip -- chunk-parallel EDA forward (prefill) in two kernels: an
// intra-chunk kernel writes each chunk's state-independent factors to a
// workspace, then a state-pass kernel carries the state through the chunks.
// This is the fp32-input path (fp32 matrix-core products throughout); bf16
// inputs take the two kernels of eda_bf16.hip.
//
// Sub-step form.  Each token t becomes two rank-1 sub-steps of the gated
// delta recurrence S_j = (I - b'_j kap_j kap_j^T) D_j S_{j-1} + b'_j kap_j nu_j^T
// (EDA paper Sec. 3.4, Eqs. (17)-(18); slides frame "Two virtual steps
// recover a standard delta recurrence"):
//   erase sub-step 2t  : kap = e_t, b' = gamma_t, nu = 0,   D = Diag(alpha_t)
//   delta sub-step 2t+1: kap = k_t, b' = beta_t,  nu = v_t, D = I, output S^T q_t
// Writing S_j = D_j S_{j-1} + kap_j u_j^T with u_j = b'_j (nu_j - (D_j S_{j-1})^T kap_j)
// and unrolling over a chunk of C tokens (L = 2C sub-steps) from the state S
// at the chunk start gives (G_t = sum_{s<=t} log alpha_s inside the chunk,
// Gam_j = exp(G_{t(j)}), products and ratios per key channel):
//   (I + A) U = Diag(b') (N - (kap o Gam) S),   A_ji = b'_j sum_c kap_jc kap_ic Gam_jc/Gam_ic  (i < j)
//   o_t   = (q_t o Gam_t)^T S + sum_{i <= 2t+1} P_ti u_i,   P_ti = sum_c q_tc kap_ic Gam_tc/Gam_ic
//   S_next = Diag(Gam_C) S + Khat^T U,                      Khat_i = kap_i o Gam_C / Gam_i
// which is the WY/UT chunk form the paper sketches in Sec. 3.4 (Eqs. (19)-(22),
// whose printed form the reading notes flag as inconsistent; this form is
// re-derived from Eqs. (17)-(18) and checked against the token recurrence).
// With Minv = (I + A)^{-1} (unit lower triangular):
//   U = Diag(b') N + Mb V + Wn S,   Mb = (Minv - I)[:, delta cols] Diag(beta),
//   Wn = -Minv Diag(b') (kap o Gam).
//
// Kernel 1 (one workgroup per chunk and head, fully parallel) computes the
// S-independent factors Wn, Qt = q o Gam, P, Khat^T, Mb and Gam_C.  Kernel 2
// (one workgroup per head and 32-column slice of d_v, serial over chunks)
// keeps its fp32 state slice in registers and per chunk forms U, the
// outputs and the next state with matrix-core products.  The identity part
// of U (beta_t v_t on delta rows) is added in fp32 and v enters the products
// unrounded, so no rounded copy of U' = Minv Diag(b') N is ever stored.
//
// Range safety of the decay ratios: Gam_j/Gam_i = exp(G_j - G_i) is split as
// exp(G_j - r) * exp(r - G_i) with a per-channel reference r = G_last/2, so
// both factors lie in [exp(-|G_last|/2), exp(|G_last|/2)].  When some channel
// decays by more than exp(-GLIM) inside one chunk (possible near the safe
// gate's floor alpha ~ e^-5, which the reading notes warn can underflow long
// products), the chunk takes an exact element-wise path for A and P instead.
#include "eda_common.h"

namespace eda {

constexpr float GLIM = 100.f;

__host__ __device__ constexpr int cmax(int a, int b) { return a > b ? a : b; }

template <typename T, int C, int D>
struct ChunkGeom {
    static constexpr int L = 2 * C;             // sub-steps per chunk
    static constexpr int NB = L / 16;           // 16-row blocks of sub-steps
    static constexpr int PAD = 16 / (int)sizeof(T);
    static constexpr int LDA = D + PAD;         // LDS row stride, rows of length D
    static constexpr int LDL = L + PAD;         // LDS row stride, rows of length L
    static constexpr int ZLD = L / 2 + PAD;
    static constexpr int NT = 256;
    static constexpr int TPC = NT / D;          // threads per key channel
    static constexpr int TPT = C / TPC;         // tokens per thread
    static_assert(TPC >= 1 && TPT >= 1 && C % TPC == 0, "bad thread split");
    // LDS regions (bytes)
    static constexpr int szKl = L * LDA * (int)sizeof(T);
    static constexpr int szAbf = L * LDL * (int)sizeof(T);
    static constexpr int szAd = NB * 16 * 17 * 4;
    static constexpr int R1 = cmax(szKl, szAbf + szAd);
    static constexpr int szKr = L * LDA * (int)sizeof(T);
    static constexpr int szQl = C * LDA * (int)sizeof(T);
    static constexpr int szMI = L * LDL * (int)sizeof(T);
    static constexpr int szZ = (L / 2) * ZLD * (int)sizeof(T);
    static constexpr int R23 = cmax(cmax(szKr + szQl, 2 * szMI + szZ), C * D * 4 + szQl);
    static constexpr int szKlT = D * LDL * (int)sizeof(T);
    static constexpr int szMisc = (L + 2 * C + D + TPC * D) * 4;
    static constexpr int LDS = R1 + R23 + szKlT + szMisc;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
    // workspace element offsets per chunk-head (units of T), then Gam_C as fp32
    static constexpr long oW = 0;                 // Wn   [L][D]
    static constexpr long oQ = oW + (long)L * D;  // Qt   [C][D]
    static constexpr long oP = oQ + (long)C * D;  // P    [C][L]
    static constexpr long oK = oP + (long)C * L;  // Kh^T [D][L]
    static constexpr long oM = oK + (long)D * L;  // Mb   [L][C]
    static constexpr long nT = oM + (long)L * C;
    static constexpr long lamByte = (nT * (long)sizeof(T) + 255) / 256 * 256;
    static constexpr long stride = (lamByte + D * 4 + 255) / 256 * 256;  // bytes per chunk-head
};

template <typename T, int C, int D>
size_t chunk_workspace_bytes(int B, int T_, int H) {
    const long NC = (T_ + C - 1) / C;
    return (size_t)((long)B * H * NC * ChunkGeom<T, C, D>::stride);
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-chunk factors.  grid = B*H*NC, block = 256.
// ---------------------------------------------------------------------------
// DPLR: the rank-1 DPLR update S_t = (I - k_t a_t^T) Diag(alpha_t) S_{t-1} + k_t v_t^T
// (GDN-2 and QED) in the same sub-step form: erase sub-steps only decay
// (kap = 0, b' = 0), delta sub-steps read along a (passed as `e`) and write
// along k with b' = 1; beta and gamma are not read.
template <typename T, int C, int D, bool DPLR>
__global__ void __launch_bounds__(256)
eda_chunk_intra(const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ e,
                const float *__restrict__ alpha, const float *__restrict__ beta,
                const float *__restrict__ gamma, char *__restrict__ ws, int Tlen, int H, int dk,
                int NC) {
    using G = ChunkGeom<T, C, D>;
    constexpr int L = G::L, NB = G::NB, LDA = G::LDA, LDL = G::LDL, ZLD = G::ZLD;
    constexpr int TPC = G::TPC, TPT = G::TPT;
    __shared__ __attribute__((aligned(16))) char smem[G::LDS];
    char *R1 = smem, *R23 = smem + G::R1, *R4 = R23 + G::R23, *RM = R4 + G::szKlT;
    T *Kl = (T *)R1;                                   // kap o exp(G - r)      [L][LDA]
    T *Abf = (T *)R1;                                  // strictly lower A      [L][LDL]
    float *Ad = (float *)(R1 + G::szAbf);              // diagonal 16-blocks    [NB][16][17]
    T *Kr = (T *)R23;                                  // kap o exp(r - G)      [L][LDA]
    T *Ql = (T *)(R23 + G::szKr);                      // q o exp(G - r)        [C][LDA]
    float *Gs = (float *)R23;                          // G (wide-decay path)   [C][D]
    T *Qraw = (T *)(R23 + C * D * 4);                  // q (wide-decay path)   [C][LDA]
    T *MI = (T *)R23;                                  // Minv                  [L][LDL]
    T *MT = (T *)(R23 + G::szMI);                      // Minv^T                [L][LDL]
    T *Zt = (T *)(R23 + 2 * G::szMI);                  // scratch               [L/2][ZLD]
    T *KlT = (T *)R4;                                  // Diag(b') kap o exp(G-r), transposed [D][LDL]
    float *bp = (float *)RM;                           // b' per sub-step       [L]
    float *sb = bp + L, *sgm = sb + C;                 // beta, gamma           [C]
    float *er = sgm + C;                               // exp(r)                [D]
    float *gsum = er + D;                              // scan partials         [TPC][D]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ch = blockIdx.x;                  // ((b*H + h)*NC + chunk)
    const int chunk = ch % NC, bh = ch / NC;
    const int b = bh / H, h = bh % H;
    const int t0 = chunk * C;
    const int nvalid = min(C, Tlen - t0);
    char *wsc = ws + (long)ch * G::stride;
    T *gW = (T *)wsc + G::oW, *gQ = (T *)wsc + G::oQ, *gP = (T *)wsc + G::oP;
    T *gK = (T *)wsc + G::oK, *gM = (T *)wsc + G::oM;
    float *gLam = (float *)(wsc + G::lamByte);
    auto row = [&](int tau) -> long { return ((long)b * Tlen + t0 + tau) * H + h; };

    // ---- phase A: gates and cumulative log-decay ------------------------------
    if (tid < C) {
        const bool ok = tid < nvalid;
        sb[tid] = ok ? (DPLR ? 1.f : beta[row(tid)]) : 0.f;
        sgm[tid] = ok && !DPLR ? gamma[row(tid)] : 0.f;
    }
    const int c = tid % D, seg = tid / D;
    const bool cok = c < dk;
    float g[TPT];
    {
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int tau = seg * TPT + i;
            const float a = (cok && tau < nvalid) ? alpha[row(tau) * dk + c] : 1.f;
            acc += __logf(a);
            g[i] = acc;
        }
        gsum[seg * D + c] = acc;
    }
    __syncthreads();
    if (tid < L) bp[tid] = (tid & 1) ? sb[tid >> 1] : sgm[tid >> 1];
    float pre = 0.f, glast = 0.f;
#pragma unroll
    for (int s = 0; s < TPC; ++s) {
        const float x = gsum[s * D + c];
        if (s < seg) pre += x;
        glast += x;
    }
#pragma unroll
    for (int i = 0; i < TPT; ++i) g[i] += pre;
    const bool wide = __syncthreads_or(glast < -GLIM) != 0;
    const float r = wide ? 0.f : 0.5f * glast;
    if (seg == 0) {
        er[c] = __expf(r);
        gLam[c] = __expf(glast);
    }

    // ---- phase B: scaled operands (LDS) and S-independent outputs (global) ----
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
        const int tau = seg * TPT + i;
        const bool ok = cok && tau < nvalid;
        const float ev = ok ? to_f32(e[row(tau) * dk + c]) : 0.f;
        const float kv = ok ? to_f32(k[row(tau) * dk + c]) : 0.f;
        const float qv = ok ? to_f32(q[row(tau) * dk + c]) : 0.f;
        const float Gt = g[i];
        float fw;
        if (!wide) {
            const float f = __expf(Gt - r), fi = __expf(r - Gt);
            Kl[(2 * tau) * LDA + c] = from_f32<T>(ev * f);
            Kl[(2 * tau + 1) * LDA + c] = from_f32<T>((DPLR ? ev : kv) * f);   // DPLR: reads along a
            Kr[(2 * tau) * LDA + c] = from_f32<T>(DPLR ? 0.f : ev * fi);        // DPLR: no erase key
            Kr[(2 * tau + 1) * LDA + c] = from_f32<T>(kv * fi);
            Ql[tau * LDA + c] = from_f32<T>(qv * f);
            fw = f;
        } else {
            Kl[(2 * tau) * LDA + c] = from_f32<T>(ev);
            Kl[(2 * tau + 1) * LDA + c] = from_f32<T>(kv);
            Qraw[tau * LDA + c] = from_f32<T>(qv);
            Gs[tau * D + c] = Gt;
            fw = __expf(Gt);
        }
        // b'-scaled, transposed copy for W (gates are zero past the tail).
        KlT[c * LDL + 2 * tau] = from_f32<T>(sgm[tau] * ev * fw);
        KlT[c * LDL + 2 * tau + 1] = from_f32<T>(sb[tau] * (DPLR ? ev : kv) * fw);
        gQ[tau * D + c] = from_f32<T>(qv * __expf(Gt));
        const float fk = __expf(glast - Gt);
        gK[(long)c * L + 2 * tau] = from_f32<T>(DPLR ? 0.f : ev * fk);
        gK[(long)c * L + 2 * tau + 1] = from_f32<T>(kv * fk);
    }
    __syncthreads();

    // ---- phase C: decayed Gram A (strictly lower) and query products P -------
    constexpr int NGT = NB * (NB + 1) / 2;             // lower-triangle tiles incl. diagonal
    constexpr int GPW = (NGT + 3) / 4;                 // per wave
    constexpr int NAE = (L * L + 255) / 256;           // wide path: entries per thread
    float aval[(GPW * 4 > NAE) ? GPW * 4 : NAE];
    if (!wide) {
        int idx = 0;
#pragma unroll
        for (int J = 0; J < NB; ++J)
#pragma unroll
            for (int I = 0; I <= J; ++I, ++idx) {
                if ((idx & 3) != wave) continue;
                f32x4 acc = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * I * LDA, LDA, zero4(), lane);
                const int m = idx >> 2;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * J + 4 * (lane >> 4) + rr, ii = 16 * I + (lane & 15);
                    aval[4 * m + rr] = (j > ii) ? bp[j] * acc[rr] : 0.f;
                }
            }
        // P^T tiles: P^T[i][t] = sum_c Kr[i][c] Ql[t][c], kept for i <= 2t+1.
        constexpr int NPT = NB * (C / 16);
        for (int pidx = wave; pidx < NPT; pidx += 4) {
            const int I = pidx / (C / 16), Tb = pidx % (C / 16);
            const int tcol = 16 * Tb + (lane & 15);
            const int i0 = 16 * I + 4 * (lane >> 4);
            f32x4 acc = zero4();
            if (16 * I <= 2 * (16 * Tb + 15) + 1)
                acc = tile_nt<T, D>(Kr + 16 * I * LDA, LDA, Ql + 16 * Tb * LDA, LDA, acc, lane);
            float w4[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) w4[rr] = (i0 + rr <= 2 * tcol + 1) ? acc[rr] : 0.f;
            store4<T>(gP + (long)tcol * L + i0, w4[0], w4[1], w4[2], w4[3]);
        }
    } else {
        // Exact element-wise path for chunks with extreme decay.
#pragma unroll
        for (int m = 0; m < NAE; ++m) {
            const int idx = tid + 256 * m;
            float s = 0.f;
            if (idx < L * L) {
                const int j = idx / L, ii = idx % L;
                // (DPLR: delta rows and columns only; row j reads along a, raw in row j - 1)
                if (ii < j && (!DPLR || ((j & 1) && (ii & 1)))) {
                    const int tj = j >> 1, ti = ii >> 1, jr = DPLR ? j - 1 : j;
                    for (int cc = 0; cc < D; ++cc)
                        s += to_f32(Kl[jr * LDA + cc]) * to_f32(Kl[ii * LDA + cc]) *
                             __expf(Gs[tj * D + cc] - Gs[ti * D + cc]);
                    s *= bp[j];
                }
            }
            aval[m] = s;
        }
        for (int idx = tid; idx < C * L; idx += 256) {
            const int tau = idx / L, ii = idx % L;
            float s = 0.f;
            if (ii <= 2 * tau + 1 && (!DPLR || (ii & 1))) {
                const int ti = ii >> 1;
                for (int cc = 0; cc < D; ++cc)
                    s += to_f32(Qraw[tau * LDA + cc]) * to_f32(Kl[ii * LDA + cc]) *
                         __expf(Gs[tau * D + cc] - Gs[ti * D + cc]);
            }
            gP[(long)tau * L + ii] = from_f32<T>(s);
        }
    }
    __syncthreads();

    // Scatter A: off-diagonal blocks as T (matrix-core operands), diagonal
    // blocks in fp32 (substitution); clear Minv and Minv^T.
    if (!wide) {
        int idx = 0;
#pragma unroll
        for (int J = 0; J < NB; ++J)
#pragma unroll
            for (int I = 0; I <= J; ++I, ++idx) {
                if ((idx & 3) != wave) continue;
                const int m = idx >> 2;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int jl = 4 * (lane >> 4) + rr, il = lane & 15;
                    if (J == I) Ad[(J * 16 + jl) * 17 + il] = aval[4 * m + rr];
                    else Abf[(16 * J + jl) * LDL + 16 * I + il] = from_f32<T>(aval[4 * m + rr]);
                }
            }
    } else {
#pragma unroll
        for (int m = 0; m < NAE; ++m) {
            const int idx = tid + 256 * m;
            if (idx < L * L) {
                const int j = idx / L, ii = idx % L;
                if ((j >> 4) == (ii >> 4)) Ad[((j >> 4) * 16 + (j & 15)) * 17 + (ii & 15)] = aval[m];
                else if (ii < j) Abf[j * LDL + ii] = from_f32<T>(aval[m]);
            }
        }
    }
    for (int idx = tid; idx < 2 * L * LDL; idx += 256) MI[idx] = from_f32<T>(0.f);  // MI and MT are adjacent
    __syncthreads();

    // ---- phase D: inverse of the diagonal blocks (fp32 forward substitution) --
    if (tid < L) {
        const int J = tid >> 4, col = tid & 15;
        float x[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float s = (i == col) ? 1.f : 0.f;
#pragma unroll
            for (int p = 0; p < i; ++p) s -= Ad[(J * 16 + i) * 17 + p] * x[p];
            x[i] = s;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            MI[(16 * J + i) * LDL + 16 * J + col] = from_f32<T>(x[i]);
            MT[(16 * J + col) * LDL + 16 * J + i] = from_f32<T>(x[i]);
        }
    }
    __syncthreads();

    // ---- phase E: recursive doubling, X21 = -X22 (A21 X11) ----------------------
#pragma unroll
    for (int s = 16; s < L; s *= 2) {
        const int ns = s / 16, npairs = L / (2 * s), ntl = npairs * ns * ns;
        for (int t = wave; t < ntl; t += 4) {
            const int p = t / (ns * ns), ab = (t / ns) % ns, nb = t % ns;
            const int m = (2 * p + 1) * s;
            f32x4 acc = tile_nt_dyn<T>(Abf + (m + 16 * ab) * LDL + (m - s), LDL,
                                       MT + (m - s + 16 * nb) * LDL + (m - s), LDL, s, zero4(), lane);
            // Z[a][n] -> Zt[p*s + n][a]
            store4<T>(Zt + (p * s + 16 * nb + (lane & 15)) * ZLD + 16 * ab + 4 * (lane >> 4),
                      acc[0], acc[1], acc[2], acc[3]);
        }
        __syncthreads();
        for (int t = wave; t < ntl; t += 4) {
            const int p = t / (ns * ns), ab = (t / ns) % ns, nb = t % ns;
            const int m = (2 * p + 1) * s;
            f32x4 acc = tile_nt_dyn<T>(MI + (m + 16 * ab) * LDL + m, LDL,
                                       Zt + (p * s + 16 * nb) * ZLD, ZLD, s, zero4(), lane);
            const int a0 = m + 16 * ab + 4 * (lane >> 4), jcol = m - s + 16 * nb + (lane & 15);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) MI[(a0 + rr) * LDL + jcol] = from_f32<T>(-acc[rr]);
            store4<T>(MT + jcol * LDL + a0, -acc[0], -acc[1], -acc[2], -acc[3]);
        }
        __syncthreads();
    }

    // ---- phase F: Wn = -Minv Diag(b') (kap o Gam)  and  Mb ----------------------
    constexpr int NWT = (D / 16) * NB;
    for (int t = wave; t < NWT; t += 4) {
        const int cb = t / NB, ib = t % NB;
        f32x4 acc = tile_nt<T, L>(KlT + 16 * cb * LDL, LDL, MI + 16 * ib * LDL, LDL, zero4(), lane);
        const int c0 = 16 * cb + 4 * (lane >> 4), i = 16 * ib + (lane & 15);
        store4<T>(gW + (long)i * D + c0, -acc[0] * er[c0], -acc[1] * er[c0 + 1],
                  -acc[2] * er[c0 + 2], -acc[3] * er[c0 + 3]);
    }
    for (int idx = tid; idx < L * C; idx += 256) {
        const int i = idx / C, tau = idx % C;
        const float val = (i > 2 * tau + 1) ? to_f32(MI[i * LDL + 2 * tau + 1]) * sb[tau] : 0.f;
        gM[idx] = from_f32<T>(val);
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state pass.  One workgroup per (head, BV-column slice); the
// slices of one head get workgroup ids congruent mod 8 so they run on the
// same XCD and share its L2 for the per-chunk factors.
// ---------------------------------------------------------------------------
template <typename T, int C, int D, int BV>
__global__ void __launch_bounds__(256)
eda_chunk_state(const T *__restrict__ v, const float *__restrict__ beta,
                const float *__restrict__ S0, float *S_final, T *__restrict__ o,
                const char *__restrict__ ws, int Tlen, int H, int BH, int dk, int dv, int NC,
                int NSv) {
    using G = ChunkGeom<T, C, D>;
    constexpr int L = G::L, PAD = G::PAD;
    constexpr int LDS_S = D + PAD, LDS_U = L + PAD, LDS_V = C + PAD;
    constexpr int NST = (D / 16) * (BV / 16);       // state tiles
    constexpr int SPW = (NST + 3) / 4;
    constexpr int NUT = (L / 16) * (BV / 16);       // U tiles
    constexpr int UPW = (NUT + 3) / 4;
    constexpr int NOT = (BV / 16) * (C / 16);       // output tiles
    __shared__ __attribute__((aligned(16))) T St[2][BV * LDS_S];
    __shared__ __attribute__((aligned(16))) T Ut[2][BV * LDS_U];
    __shared__ __attribute__((aligned(16))) T Vt[2][BV * LDS_V];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / NSv) * 8 + xcd, slice = slot % NSv;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H, n0 = slice * BV;
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;
    const long sbase = (long)bh * dk * dv;

    f32x4 S[SPW];
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        S[m] = zero4();
        const int t = wave + 4 * m;
        if (t < NST && S0) {
            const int rb = t / (BV / 16), cb = t % (BV / 16);
            const int col = n0 + 16 * cb + l16;
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int rw = 16 * rb + g4 + rr;
                if (rw < dk && col < dv) S[m][rr] = S0[sbase + (long)rw * dv + col];
            }
        }
    }

    for (int cidx = 0; cidx < NC; ++cidx) {
        const int buf = cidx & 1, t0 = cidx * C, nvalid = min(C, Tlen - t0);
        const char *wsc = ws + ((long)bh * NC + cidx) * G::stride;
        const T *gW = (const T *)wsc + G::oW, *gQ = (const T *)wsc + G::oQ;
        const T *gP = (const T *)wsc + G::oP, *gK = (const T *)wsc + G::oK;
        const T *gM = (const T *)wsc + G::oM;
        const float *gLam = (const float *)(wsc + G::lamByte);
        T *st = St[buf], *ut = Ut[buf], *vt = Vt[buf];

        // state snapshot (operand copy) and value slice, both transposed
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + 4 * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                store4<T>(st + (16 * cb + l16) * LDS_S + 16 * rb + g4, S[m][0], S[m][1], S[m][2], S[m][3]);
            }
        }
        for (int idx = tid; idx < C * BV; idx += 256) {
            const int tau = idx / BV, n = idx % BV;
            float x = 0.f;
            if (tau < nvalid && n0 + n < dv) x = to_f32(v[(((long)b * Tlen + t0 + tau) * H + h) * dv + n0 + n]);
            vt[n * LDS_V + tau] = from_f32<T>(x);
        }
        __syncthreads();

        // U = Diag(b') N + Mb V + Wn S
#pragma unroll
        for (int m = 0; m < UPW; ++m) {
            const int t = wave + 4 * m;
            if (t < NUT) {
                const int jb = t / (BV / 16), nb = t % (BV / 16);
                f32x4 acc;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * jb + g4 + rr, tau = j >> 1;
                    acc[rr] = 0.f;
                    if ((j & 1) && tau < nvalid)   // (no beta: the DPLR update writes v itself)
                        acc[rr] = (beta ? beta[((long)b * Tlen + t0 + tau) * H + h] : 1.f) *
                                  to_f32(vt[(16 * nb + l16) * LDS_V + tau]);
                }
                acc = tile_nt<T, D>(gW + (long)16 * jb * D, D, st + 16 * nb * LDS_S, LDS_S, acc, lane);
                acc = tile_nt<T, C>(gM + (long)16 * jb * C, C, vt + 16 * nb * LDS_V, LDS_V, acc, lane);
                store4<T>(ut + (16 * nb + l16) * LDS_U + 16 * jb + g4, acc[0], acc[1], acc[2], acc[3]);
            }
        }
        __syncthreads();

        // o^T = S^T Qt^T + U^T P^T  (outputs of the chunk's tokens)
        for (int t = wave; t < NOT; t += 4) {
            const int nb = t / (C / 16), tb = t % (C / 16);
            f32x4 acc = tile_nt<T, D>(st + 16 * nb * LDS_S, LDS_S, gQ + (long)16 * tb * D, D, zero4(), lane);
            acc = tile_nt<T, L>(ut + 16 * nb * LDS_U, LDS_U, gP + (long)16 * tb * L, L, acc, lane);
            const int tau = 16 * tb + l16, n = n0 + 16 * nb + g4;
            if (tau < nvalid) {
                T *op = o + (((long)b * Tlen + t0 + tau) * H + h) * dv;
                if (n + 3 < dv && (dv & 3) == 0) {
                    store4<T>(op + n, acc[0], acc[1], acc[2], acc[3]);
                } else {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        if (n + rr < dv) op[n + rr] = from_f32<T>(acc[rr]);
                }
            }
        }

        // S <- Diag(Gam_C) S + Khat^T U
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + 4 * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                f32x4 acc;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) acc[rr] = gLam[16 * rb + g4 + rr] * S[m][rr];
                S[m] = tile_nt<T, L>(gK + (long)16 * rb * L, L, ut + 16 * cb * LDS_U, LDS_U, acc, lane);
            }
        }
    }

    if (S_final) {
        // All reads of S0 happened before the chunk loop; S_final may alias S0.
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + 4 * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                const int col = n0 + 16 * cb + l16;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int rw = 16 * rb + g4 + rr;
                    if (rw < dk && col < dv) S_final[sbase + (long)rw * dv + col] = S[m][rr];
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch (called by the C ABI after argument checks).
// ---------------------------------------------------------------------------
template <typename T, int C, int D>
hipError_t launch_chunked_t(int phase, const void *q, const void *k, const void *e, const void *v,
                            const float *alpha, const float *beta, const float *gamma,
                            const float *S0, void *o, float *S_final, int B, int Tlen, int H,
                            int dk, int dv, void *ws, hipStream_t stream, hipEvent_t const *ev) {
    constexpr int BV = 32;
    const int NC = (Tlen + C - 1) / C;
    const int BH = B * H;
    hipError_t err;
    if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    if (phase & 1) {
        // beta == NULL selects the rank-1 DPLR update (erase vector a in `e`)
        auto k1 = beta ? eda_chunk_intra<T, C, D, false> : eda_chunk_intra<T, C, D, true>;
        hipLaunchKernelGGL(k1, dim3((unsigned)(BH * NC)), dim3(256), 0, stream, (const T *)q,
                           (const T *)k, (const T *)e, alpha, beta, gamma, (char *)ws, Tlen, H, dk, NC);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    if (phase & 2) {
        const int NSv = (dv + BV - 1) / BV;
        const int grid = 8 * ((BH + 7) / 8) * NSv;
        hipLaunchKernelGGL((eda_chunk_state<T, C, D, BV>), dim3((unsigned)grid), dim3(256), 0,
                           stream, (const T *)v, beta, S0, S_final, (T *)o, (const char *)ws, Tlen,
                           H, BH, dk, dv, NC, NSv);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return ev ? hipEventRecord(ev[2], stream) : hipSuccess;
}

static int pad_dim(int dk, int dv) {
    const int p = dk > dv ? dk : dv;
    return p <= 32 ? 32 : (p <= 64 ? 64 : 128);
}

template <typename T>
size_t chunked_ws_t(int B, int Tlen, int H, int dk, int dv, int chunk) {
    const int D = pad_dim(dk, dv);
#define EDA_WS(CC, DD) if (chunk == CC && D == DD) return chunk_workspace_bytes<T, CC, DD>(B, Tlen, H);
    EDA_WS(16, 32) EDA_WS(16, 64) EDA_WS(16, 128)
    EDA_WS(32, 32) EDA_WS(32, 64) EDA_WS(32, 128)
#undef EDA_WS
    return 0;
}

// phase: 1 = intra-chunk factors only, 2 = state pass only, 3 = both.
template <typename T>
hipError_t launch_chunked(int phase, const void *q, const void *k, const void *e, const void *v,
                          const float *alpha, const float *beta, const float *gamma,
                          const float *S0, void *o, float *S_final, int B, int Tlen, int H, int dk,
                          int dv, int chunk, void *ws, hipStream_t stream, hipEvent_t const *ev) {
    const int D = pad_dim(dk, dv);
#define EDA_GO(CC, DD)                                                                          \
    if (chunk == CC && D == DD)                                                                 \
        return launch_chunked_t<T, CC, DD>(phase, q, k, e, v, alpha, beta, gamma, S0, o,        \
                                           S_final, B, Tlen, H, dk, dv, ws, stream, ev);
    EDA_GO(16, 32) EDA_GO(16, 64) EDA_GO(16, 128)
    EDA_GO(32, 32) EDA_GO(32, 64) EDA_GO(32, 128)
#undef EDA_GO
    return hipErrorInvalidValue;
}

template size_t chunked_ws_t<float>(int, int, int, int, int, int);
template hipError_t launch_chunked<float>(int, const void *, const void *, const void *,
                                          const void *, const float *, const float *, const float *,
                                          const float *, void *, float *, int, int, int, int, int,
                                          int, void *, hipStream_t, hipEvent_t const *);

}  // namespace eda
