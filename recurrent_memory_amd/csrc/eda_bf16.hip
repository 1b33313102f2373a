// eda_bf16.hip -- chunked EDA forward for bf16 inputs, in two kernels.
//
// Sub-step form (EDA paper, Sec. 3.4, Eqs. (17)-(18); reading slides, frame
// "Two virtual steps recover a standard delta recurrence"): token t is an
// erase sub-step (key e_t, gate gamma_t, decay alpha_t, no value) followed by
// a delta sub-step (key k_t, gate beta_t, value v_t, no decay).  Writing sub-
// step j as S_j = D_j S_{j-1} + kap_j u_j^T, u_j = b'_j (nu_j - (D_j S_{j-1})^T kap_j),
// and unrolling over a chunk of C tokens (L = 2C sub-steps) from the state S
// at the chunk start (G = cumulative log-decay inside the chunk, per key
// channel; t(j) = token of sub-step j):
//
//   (I + A) U = Diag(b') (N - (kap o e^G) S),  A_ji = b'_j sum_c kap_jc kap_ic e^{G_t(j)c - G_t(i)c}  (i < j)
//   o_t       = (q_t o e^{G_t})^T S + sum_{i <= 2t+1} P_ti u_i,   P_ti = sum_c q_tc kap_ic e^{G_tc - G_t(i)c}
//   S_next    = Diag(e^{G_C}) S + Khat^T U,                        Khat_ic = kap_ic e^{G_Cc - G_t(i)c}
//
// (N holds v_t on delta rows and 0 on erase rows; our own derivation of the
// chunk form the paper outlines -- its WY/UT equations are not legible on
// the pages -- checked against the token recurrence).  Decay ratios are split
// per channel around r = G_C / 2:
//   Kl = kap o e^{G - r},  Kr = kap o e^{r - G},  Ql = q o e^{G - r},
// so A = Diag(b') strict_lower(Kl Kr^T), P = causal(Ql Kr^T), and with the
// scaled state S' = Diag(e^r) S:
//   Z = Diag(b') (N - Kl S'),  U = (I + A)^{-1} Z,  o = Ql S' + P U,
//   S_next = Diag(e^r) (Diag(e^r) S + Kr^T U)            (e^{G_C} = e^{2r}).
// Every factor stays within e^{+-|G_C|/2}; a chunk in which some channel
// decays by more than e^-120 (only possible below the safe gate's floor
// alpha = e^-5) computes A and P element-wise from e^{G_j - G_i} and stores
// the unsplit factors kap o e^G, q o e^G and Khat instead.
//
// Kernel 1 (eda_bf16_factors): one workgroup per (head, chunk), all chunks in
//   parallel.  Computes the state-independent factors -- Kl, Kr, Ql, the
//   causal P, (I + A)^{-1} and the per-channel scales -- and writes them to the
//   workspace.  The unit lower-triangular inverse: fp32 substitution on the
//   16x16 diagonal blocks, then one column block of the off-diagonal part per
//   wave, with the blocks held in registers.
// Kernel 2 (eda_bf16_state): one workgroup per (head, slice of value columns),
//   serial over chunks.  Keeps the fp32 state in registers and per chunk
//   forms Z, U, the outputs and the next state on the matrix cores (three
//   barriers per chunk), while the next chunk's factor block is fetched into
//   the other half of a double buffer.
//
// Workspace: one block of FacLayout<C, D>::bytes per chunk and head, rows
// padded exactly like the LDS copies, so kernel 2 fetches a block as one
// contiguous copy.
#include <type_traits>

#include "eda_common.h"

namespace eda {
namespace b16 {

// wide-chunk threshold on a chunk's log2-decay (e^-120 = 2^-173)
constexpr float WIDE_G2 = 173.f;

__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }
__host__ __device__ constexpr int align256(int x) { return (x + 255) / 256 * 256; }

__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

// Make this wave's earlier LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Inclusive prefix sum over groups of N consecutive lanes (N a power of two);
// `seg` is the lane's index in its group.  Groups of 16 use DPP row shifts.
template <int N>
__device__ __forceinline__ float scan_group(float x, int seg) {
    if constexpr (N == 16) {
#define EDA_ROW_SHR(n) \
        x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + (n), 0xf, 0xf, true))
        EDA_ROW_SHR(1); EDA_ROW_SHR(2); EDA_ROW_SHR(4); EDA_ROW_SHR(8);
#undef EDA_ROW_SHR
    } else {
#pragma unroll
        for (int off = 1; off < N; off <<= 1) {
            const float y = __shfl_up(x, off, N);
            if (seg >= off) x += y;
        }
    }
    return x;
}

// Value of the last lane of each group of N consecutive lanes.
template <int N>
__device__ __forceinline__ float group_last(float x) {
    if constexpr (N == 16) {
        // ds_swizzle bit mode: lane' = (lane & 0x10) | 0xF within each 32 lanes
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F0));
    } else {
        return __shfl(x, N - 1, N);
    }
}

// ---------------------------------------------------------------------------
// Workspace block of one chunk and head (byte offsets).
// ---------------------------------------------------------------------------
template <int C, int D>
struct FacLayout {
    static constexpr int L = 2 * C, LDA = D + 8, LDL = L + 8;
    static constexpr int oKl = 0;                          // Kl    [L][LDA] bf16
    static constexpr int oKr = oKl + L * LDA * 2;          // Kr    [L][LDA] bf16 (wide: Khat)
    static constexpr int oQl = oKr + L * LDA * 2;          // Ql    [C][LDA] bf16
    static constexpr int oMI = oQl + C * LDA * 2;          // (I+A)^-1 [L][LDL] bf16, lower blocks
    static constexpr int oP = oMI + L * LDL * 2;           // P     [C][LDL] bf16, causal part
    static constexpr int oErS = oP + C * LDL * 2;          // e^r (1 if wide)      [D] fp32
    static constexpr int oLam = oErS + D * 4;              // e^r (e^{G_C} if wide) [D] fp32
    static constexpr int oSK = oLam + D * 4;               // e^r (1 if wide)      [D] fp32
    static constexpr int oBp = oSK + D * 4;                // b' per sub-step      [L] fp32
    static constexpr int bytes = align256(oBp + L * 4);
    static_assert(oKr % 16 == 0 && oQl % 16 == 0 && oMI % 16 == 0 && oP % 16 == 0 && oErS % 16 == 0,
                  "16-byte sections");
};

// ---------------------------------------------------------------------------
// Kernel 1: chunk factors.  grid = B*H*NC, block = 64*NW.
// ---------------------------------------------------------------------------
template <int C, int D, int NW>
struct K1Geom {
    static constexpr int L = 2 * C, NB = L / 16, NT = 64 * NW;
    static constexpr int LDA = D + 8, LDL = L + 8, ADS = 20, ASD = D + 8, MTW = 24;
    static constexpr int NQ = D / 4;
    static constexpr int TPC = imin(NT / NQ, C);       // threads per channel quad
    static constexpr int TPT = C / TPC;                // tokens per thread
    static constexpr int ACT = NQ * TPC;               // threads with an element-wise role
    static_assert((TPC & (TPC - 1)) == 0 && TPC <= 64 && C % TPC == 0 && ACT <= NT, "split");
    static_assert(TPT == 1 || TPT == 2, "token run");
    static constexpr int NZW = NW - NB;                // matrix waves (A and P tiles)
    static_assert(NZW >= 1, "too few waves");
    static constexpr int LPR = D / 8, RPP = NT / LPR, PQ = (C + RPP - 1) / RPP;   // 16-byte row loads
    static constexpr int LPA = D / 4, RPA = NT / LPA, PA = (C + RPA - 1) / RPA;
    // LDS (bytes).  Before the operands are formed, Kl holds the raw alpha
    // rows (fp32 [C][ASD]), Kr the raw e and k rows, Ql the raw q rows; in a
    // wide chunk Kl then holds G (fp32 [C][D]) and Kr, Ql keep the raw keys.
    static constexpr int szKl = align16(L * LDA * 2), szQl = align16(C * LDA * 2);
    static_assert(C * ASD * 4 <= szKl && C * D * 4 <= szKl, "Kl region reuse");
    static constexpr int szAbf = align16(L * LDL * 2), szAd = NB * 16 * ADS * 4;
    static constexpr int szMI = align16(L * LDL * 2), szMT = NB * 16 * MTW * 2;
    static constexpr int szMisc = (L + 2 * C + D) * 4;
    static constexpr int oKl = 0, oKr = oKl + szKl, oQl = oKr + szKl, oAbf = oQl + szQl;
    static constexpr int oAd = oAbf + szAbf, oMI = oAd + szAd, oMT = oMI + szMI, oMisc = oMT + szMT;
    static constexpr int LDS = oMisc + szMisc;
    static_assert(LDS <= 80 * 1024, "two workgroups per compute unit");
};

template <int C, int D, int NW>
__global__ void __launch_bounds__(64 * NW)
eda_bf16_factors(const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ e,
                 const float *__restrict__ alpha, const float *__restrict__ beta,
                 const float *__restrict__ gamma, char *__restrict__ ws, int Tlen, int H, int dk,
                 int NC, int vec) {
    using G = K1Geom<C, D, NW>;
    using F = FacLayout<C, D>;
    using T = bf16;
    constexpr int L = G::L, NB = G::NB, NT = G::NT, LDA = G::LDA, LDL = G::LDL, ADS = G::ADS;
    constexpr int ASD = G::ASD, MTW = G::MTW, TPC = G::TPC, TPT = G::TPT, NZW = G::NZW;
    constexpr int LPR = G::LPR, RPP = G::RPP, PQ = G::PQ, LPA = G::LPA, RPA = G::RPA, PA = G::PA;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Kl = (T *)(smem + G::oKl);
    float *As = (float *)(smem + G::oKl);   // raw alpha [C][ASD] (before the operands)
    float *Gs = (float *)(smem + G::oKl);   // wide chunk: G (log2) [C][D]
    T *Kr = (T *)(smem + G::oKr);
    T *Ql = (T *)(smem + G::oQl);
    T *Abf = (T *)(smem + G::oAbf);          // A, off-diagonal 16-blocks   [L][LDL]
    float *Ad = (float *)(smem + G::oAd);    // A, diagonal 16-blocks      [NB][16][ADS]
    T *MI = (T *)(smem + G::oMI);            // (I + A)^{-1}               [L][LDL]
    T *MT = (T *)(smem + G::oMT);            // its diagonal blocks, transposed [NB][16][MTW]
    float *bp = (float *)(smem + G::oMisc);  // b' per sub-step            [L]
    float *sb = bp + L, *sg = sb + C;        // beta, gamma per token      [C]
    float *glc = sg + C;                     // G_C per channel (log2)     [D]

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;
    const int bh = blockIdx.x / NC, cidx = blockIdx.x % NC;
    const int b = bh / H, h = bh % H;
    const int t0 = cidx * C, nval = min(C, Tlen - t0);
    const long hrow = (long)b * Tlen * H + h;
    const int HK = H * dk;
    const bf16 *qh = q + hrow * dk, *kh = k + hrow * dk, *eh = e + hrow * dk;
    const float *ah = alpha + hrow * dk;
    char *wsb = ws + ((long)bh * NC + cidx) * F::bytes;
    T *gKl = (T *)(wsb + F::oKl), *gKr = (T *)(wsb + F::oKr), *gQl = (T *)(wsb + F::oQl);
    T *gMI = (T *)(wsb + F::oMI), *gP = (T *)(wsb + F::oP);
    float *gErS = (float *)(wsb + F::oErS), *gLam = (float *)(wsb + F::oLam);
    float *gSK = (float *)(wsb + F::oSK), *gBp = (float *)(wsb + F::oBp);

    // ---- raw chunk rows -> LDS (whole-row 16-byte loads) -------------------------
    if (vec && nval == C) {
#pragma unroll
        for (int p = 0; p < PQ; ++p) {
            const int r = tid / LPR + RPP * p, blk = tid % LPR;
            if (RPP * PQ == C || r < C) {
                const int off = (t0 + r) * HK + 8 * blk;
                *(uint4 *)(Ql + r * LDA + 8 * blk) = *(const uint4 *)(qh + off);
                *(uint4 *)(Kr + (2 * r) * LDA + 8 * blk) = *(const uint4 *)(eh + off);
                *(uint4 *)(Kr + (2 * r + 1) * LDA + 8 * blk) = *(const uint4 *)(kh + off);
            }
        }
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            const int r = tid / LPA + RPA * p, blk = tid % LPA;
            if (RPA * PA == C || r < C)
                *(f32x4 *)(As + r * ASD + 4 * blk) = *(const f32x4 *)(ah + (t0 + r) * HK + 4 * blk);
        }
    } else {
        for (int idx = tid; idx < C * D; idx += NT) {
            const int r = idx / D, c = idx % D;
            const bool ok = r < nval && c < dk;
            const int off = (t0 + r) * HK + c;
            Ql[r * LDA + c] = ok ? q[hrow * dk + off] : (T)0;
            Kr[(2 * r) * LDA + c] = ok ? e[hrow * dk + off] : (T)0;
            Kr[(2 * r + 1) * LDA + c] = ok ? k[hrow * dk + off] : (T)0;
            As[r * ASD + c] = ok ? alpha[hrow * dk + off] : 1.f;
        }
    }
    if (tid < C) {
        const bool ok = tid < nval;
        const float bv = ok ? beta[hrow + (long)(t0 + tid) * H] : 0.f;
        const float gv = ok ? gamma[hrow + (long)(t0 + tid) * H] : 0.f;
        sb[tid] = bv;
        sg[tid] = gv;
        bp[2 * tid] = gv;
        bp[2 * tid + 1] = bv;
        *(f32x2 *)(gBp + 2 * tid) = f32x2{gv, bv};
    }
    __syncthreads();

    // ---- cumulative log2-decay per channel; wide-chunk vote ----------------------
    const bool act = tid < G::ACT;
    const int seg = tid % TPC, c0 = 4 * (tid / TPC);
    float g[TPT][4];
    bool wide_here = false;
    {
        float base[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            // tokens seg + TPC i: one group scan per run, offset by the earlier runs' totals
            const f32x4 pa = act ? *(const f32x4 *)(As + (seg + TPC * i) * ASD + c0) : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                g[i][j] = base[j] + scan_group<TPC>(__builtin_amdgcn_logf(pa[j]), seg);
                base[j] = group_last<TPC>(g[i][j]);
            }
        }
        if (act && seg == TPC - 1) {
            *(f32x4 *)(glc + c0) = f32x4{base[0], base[1], base[2], base[3]};
#pragma unroll
            for (int j = 0; j < 4; ++j) wide_here |= base[j] < -WIDE_G2;
        }
    }
    const bool wide = __syncthreads_or(wide_here) != 0;

    // ---- scaled operands (LDS and workspace) and per-channel scales --------------
    if (act) {
        const f32x4 gl = *(const f32x4 *)(glc + c0);
        float r[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = wide ? 0.f : 0.5f * gl[j];
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int tau = seg + TPC * i;
            const uint2 pq = *(const uint2 *)(Ql + tau * LDA + c0);
            const uint2 pe = *(const uint2 *)(Kr + (2 * tau) * LDA + c0);
            const uint2 pk = *(const uint2 *)(Kr + (2 * tau + 1) * LDA + c0);
            const float ev[4] = {lo_bf16(pe.x), hi_bf16(pe.x), lo_bf16(pe.y), hi_bf16(pe.y)};
            const float kv[4] = {lo_bf16(pk.x), hi_bf16(pk.x), lo_bf16(pk.y), hi_bf16(pk.y)};
            const float qv[4] = {lo_bf16(pq.x), hi_bf16(pq.x), lo_bf16(pq.y), hi_bf16(pq.y)};
            float f[4], fi[4];
            if (!wide) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f[j] = exp2f_(g[i][j] - r[j]);
                    fi[j] = exp2f_(r[j] - g[i][j]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f[j] = exp2f_(g[i][j]);
                    fi[j] = exp2f_(gl[j] - g[i][j]);   // Khat factor, <= 1
                }
            }
            const uint2 kl0 = make_uint2(pack_bf16(ev[0] * f[0], ev[1] * f[1]), pack_bf16(ev[2] * f[2], ev[3] * f[3]));
            const uint2 kl1 = make_uint2(pack_bf16(kv[0] * f[0], kv[1] * f[1]), pack_bf16(kv[2] * f[2], kv[3] * f[3]));
            const uint2 kr0 = make_uint2(pack_bf16(ev[0] * fi[0], ev[1] * fi[1]), pack_bf16(ev[2] * fi[2], ev[3] * fi[3]));
            const uint2 kr1 = make_uint2(pack_bf16(kv[0] * fi[0], kv[1] * fi[1]), pack_bf16(kv[2] * fi[2], kv[3] * fi[3]));
            const uint2 ql = make_uint2(pack_bf16(qv[0] * f[0], qv[1] * f[1]), pack_bf16(qv[2] * f[2], qv[3] * f[3]));
            *(uint2 *)(gKl + (2 * tau) * LDA + c0) = kl0;
            *(uint2 *)(gKl + (2 * tau + 1) * LDA + c0) = kl1;
            *(uint2 *)(gKr + (2 * tau) * LDA + c0) = kr0;
            *(uint2 *)(gKr + (2 * tau + 1) * LDA + c0) = kr1;
            *(uint2 *)(gQl + tau * LDA + c0) = ql;
            if (!wide) {
                // Kl overwrites the raw alpha rows, which were last read before the vote
                *(uint2 *)(Kl + (2 * tau) * LDA + c0) = kl0;
                *(uint2 *)(Kl + (2 * tau + 1) * LDA + c0) = kl1;
                *(uint2 *)(Kr + (2 * tau) * LDA + c0) = kr0;
                *(uint2 *)(Kr + (2 * tau + 1) * LDA + c0) = kr1;
                *(uint2 *)(Ql + tau * LDA + c0) = ql;
            } else {
                *(f32x4 *)(Gs + tau * D + c0) = f32x4{g[i][0], g[i][1], g[i][2], g[i][3]};
            }
        }
        if (seg == 0) {
            f32x4 er, lam, skk;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float x = exp2f_(r[j]);
                er[j] = wide ? 1.f : x;
                lam[j] = wide ? exp2f_(gl[j]) : x;
                skk[j] = wide ? 1.f : x;
            }
            *(f32x4 *)(gErS + c0) = er;
            *(f32x4 *)(gLam + c0) = lam;
            *(f32x4 *)(gSK + c0) = skk;
        }
    }
    __syncthreads();

    // ---- A (strictly lower, b'-scaled) and P (causal); diagonal blocks inverted --
    auto invert_diag = [&](int J) {
        if (lane < 16) {
            const int col = lane;
            float x[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const f32x4 *arow = (const f32x4 *)(Ad + (J * 16 + i) * ADS);
                f32x4 av[4];
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                    if (4 * v4 < i) av[v4] = arow[v4];
                float sum = (i == col) ? 1.f : 0.f;
#pragma unroll
                for (int p = 0; p < i; ++p) sum -= av[p >> 2][p & 3] * x[p];
                x[i] = sum;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) MI[(16 * J + i) * LDL + 16 * J + col] = from_f32<T>(x[i]);
            uint4 *mt = (uint4 *)(MT + (16 * J + col) * MTW);
            mt[0] = make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                               pack_bf16(x[6], x[7]));
            mt[1] = make_uint4(pack_bf16(x[8], x[9]), pack_bf16(x[10], x[11]), pack_bf16(x[12], x[13]),
                               pack_bf16(x[14], x[15]));
        }
    };
    const int mw = wave - NB;   // matrix-wave index (< 0 on the inverse waves)
    if (!wide) {
        if (wave < NB) {
            const int J = wave;
            const f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * J * LDA, LDA, zero4(), lane);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int jl = g4 + rr;
                Ad[(J * 16 + jl) * ADS + l16] = (jl > l16) ? bp[16 * J + jl] * a[rr] : 0.f;
            }
            wave_lds_sync();
            invert_diag(J);
        }
        constexpr int NOD = NB * (NB - 1) / 2;
        constexpr int NPT = NB * (C / 16);
        for (int t = mw; mw >= 0 && t < NOD + NPT; t += NZW) {
            if (t < NOD) {
                int J = 1, I = t;
                while (I >= J) { I -= J; ++J; }
                const f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * I * LDA, LDA, zero4(), lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * J + g4 + rr;
                    Abf[j * LDL + 16 * I + l16] = from_f32<T>(bp[j] * a[rr]);
                }
            } else {
                // P^T tile: rows = sub-steps i, cols = tokens; kept for i <= 2 tau + 1
                const int I = (t - NOD) / (C / 16), Tb = (t - NOD) % (C / 16);
                if (16 * I > 32 * Tb + 31) continue;   // beyond every token's causal range
                const f32x4 a = tile_nt<T, D>(Kr + 16 * I * LDA, LDA, Ql + 16 * Tb * LDA, LDA, zero4(), lane);
                const int tau = 16 * Tb + l16, i0 = 16 * I + g4;
                float w4[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) w4[rr] = (i0 + rr <= 2 * tau + 1) ? a[rr] : 0.f;
                store4<T>(gP + tau * LDL + i0, w4[0], w4[1], w4[2], w4[3]);
            }
        }
    } else {
        // exact element-wise path: e^{G_j - G_i} is never split (Kr, Ql hold raw keys)
        for (int idx = tid; idx < L * L; idx += NT) {
            const int j = idx / L, ii = idx % L;
            float s = 0.f;
            if (ii < j) {
                const int tj = j >> 1, ti = ii >> 1;
#pragma unroll 2
                for (int cc = 0; cc < D; ++cc)
                    s += to_f32(Kr[j * LDA + cc]) * to_f32(Kr[ii * LDA + cc]) *
                         exp2f_(Gs[tj * D + cc] - Gs[ti * D + cc]);
                s *= bp[j];
            }
            if ((j >> 4) == (ii >> 4)) Ad[((j >> 4) * 16 + (j & 15)) * ADS + (ii & 15)] = s;
            else if (ii < j) Abf[j * LDL + ii] = from_f32<T>(s);
        }
        for (int idx = tid; idx < C * L; idx += NT) {
            const int tau = idx / L, ii = idx % L;
            float s = 0.f;
            if (ii <= 2 * tau + 1) {
                const int ti = ii >> 1;
#pragma unroll 2
                for (int cc = 0; cc < D; ++cc)
                    s += to_f32(Ql[tau * LDA + cc]) * to_f32(Kr[ii * LDA + cc]) *
                         exp2f_(Gs[tau * D + cc] - Gs[ti * D + cc]);
            }
            gP[tau * LDL + ii] = from_f32<T>(s);
        }
        __syncthreads();
        if (wave < NB) invert_diag(wave);
    }
    __syncthreads();

    // ---- off-diagonal blocks of (I + A)^{-1}, one column block per wave:
    //      X_JI = -X_JJ sum_{I <= K < J} A_JK X_KI, for J = I+1, I+2, ...
    // A 16x16 accumulator (lane: rows 4g..4g+3 of column l%16) is exactly the
    // B operand of the 16x16x16 instruction, so the X_KI stay in registers.
    if (wave < NB - 1) {
        const int I = wave;
        s16x4 xb[NB];   // X_KI as bf16 B operands (K >= I)
#pragma unroll
        for (int K = 0; K < NB - 1; ++K)
            if (K == I) xb[K] = *(const s16x4 *)(MT + (16 * K + l16) * MTW + g4);
#pragma unroll
        for (int J = 1; J < NB; ++J) {
            if (J <= I) continue;
            f32x4 t = zero4();
#pragma unroll
            for (int K = 0; K < J; ++K) {
                if (K < I) continue;
                const s16x4 a = *(const s16x4 *)(Abf + (16 * J + l16) * LDL + 16 * K + g4);
                t = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, xb[K], t, 0, 0, 0);
            }
            const s16x4 tb = __builtin_bit_cast(s16x4, make_uint2(pack_bf16(t[0], t[1]), pack_bf16(t[2], t[3])));
            const s16x4 m = *(const s16x4 *)(MI + (16 * J + l16) * LDL + 16 * J + g4);
            const f32x4 x = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(m, tb, zero4(), 0, 0, 0);
            const uint32_t x01 = pack_bf16(-x[0], -x[1]), x23 = pack_bf16(-x[2], -x[3]);
            xb[J] = __builtin_bit_cast(s16x4, make_uint2(x01, x23));
            const int a0 = 16 * J + g4, ncol = 16 * I + l16;
            MI[(a0 + 0) * LDL + ncol] = (T)(x01 & 0xffffu);
            MI[(a0 + 1) * LDL + ncol] = (T)(x01 >> 16);
            MI[(a0 + 2) * LDL + ncol] = (T)(x23 & 0xffffu);
            MI[(a0 + 3) * LDL + ncol] = (T)(x23 >> 16);
        }
    }
    __syncthreads();

    // ---- (I + A)^{-1} -> workspace (only its lower blocks are ever read) --------
    for (int idx = tid; idx < L * LDL / 8; idx += NT)
        ((uint4 *)gMI)[idx] = ((const uint4 *)MI)[idx];
}

// ---------------------------------------------------------------------------
// Kernel 2: state pass.  One workgroup per (head, BV-column slice); the
// slices of one head get workgroup ids congruent mod 8 (same XCD, one L2 for
// the shared factor blocks).
// ---------------------------------------------------------------------------
template <int C, int D, int BV, int NW>
struct K2Geom {
    using F = FacLayout<C, D>;
    static constexpr int L = 2 * C, NB = L / 16, NT = 64 * NW;
    static constexpr int LDA = D + 8, LDL = L + 8, LDO = BV + 8;
    static constexpr int FB = F::bytes;                       // factor block
    static constexpr int NFU = FB / 16;                       // its 16-byte units
    static constexpr int VB = C * BV * 2, NVU = VB / 16;      // value slice of a chunk
    static constexpr int NU = NFU + NVU, UPT = (NU + NT - 1) / NT;   // prefetch units per thread
    static constexpr int NYT = NB * (BV / 16), YPW = (NYT + NW - 1) / NW;   // Z / U tiles
    static constexpr int NOT = (BV / 16) * (C / 16), OPW = (NOT + NW - 1) / NW;  // output tiles
    static constexpr int NST = (D / 16) * (BV / 16), SPW = (NST + NW - 1) / NW;  // state tiles
    static constexpr int szSt = align16(BV * LDA * 2), szVs = align16(VB);
    static constexpr int szZt = align16(BV * LDL * 2), szOs = align16(C * LDO * 2);
    static constexpr int oBuf = 0, oSt = 2 * FB, oVs = oSt + szSt, oZt = oVs + 2 * szVs;
    static constexpr int oUt = oZt + szZt, oOs = oUt + szZt;
    static constexpr int LDS = oOs + szOs;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
    static_assert(VB % 16 == 0, "value slice in 16-byte units");
};

template <int C, int D, int BV, int NW>
__global__ void __launch_bounds__(64 * NW)
eda_bf16_state(const bf16 *__restrict__ v, const float *S0, float *S_final, bf16 *__restrict__ o,
               const char *__restrict__ ws, int Tlen, int H, int BH, int dk, int dv, int NC, int R,
               int vvec) {
    using G = K2Geom<C, D, BV, NW>;
    using F = FacLayout<C, D>;
    using T = bf16;
    constexpr int L = G::L, NT = G::NT, LDA = G::LDA, LDL = G::LDL, LDO = G::LDO, FB = G::FB;
    constexpr int NFU = G::NFU, NU = G::NU, UPT = G::UPT;
    constexpr int NYT = G::NYT, YPW = G::YPW, NOT = G::NOT, OPW = G::OPW, NST = G::NST, SPW = G::SPW;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *St = (T *)(smem + G::oSt);   // S'^T (bf16 operand) [BV][LDA]
    T *Zt = (T *)(smem + G::oZt);   // Z^T (bf16)          [BV][LDL]
    T *Ut = (T *)(smem + G::oUt);   // U^T (bf16)          [BV][LDL]
    T *Os = (T *)(smem + G::oOs);   // outputs awaiting their store [C][LDO]

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / R) * 8 + xcd, slice = slot % R;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H, n0 = slice * BV;
    const long sbase = (long)bh * dk * dv;
    const long hrow = (long)b * Tlen * H + h;
    const int HV = H * dv;
    const bf16 *vh = v + hrow * dv + n0;
    const char *wsh = ws + (long)bh * NC * FB;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;

    // ---- prefetch of one chunk: factor block + value slice, 16-byte units -----
    uint4 pre[UPT];
    auto load_chunk = [&](int cidx) {
        const uint4 *src = (const uint4 *)(wsh + (long)cidx * FB);
        const int t0 = cidx * C, nval = min(C, Tlen - t0);
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = tid + NT * m;
            if (u < NFU) {
                pre[m] = src[u];
            } else if (u < NU) {
                const int vu = u - NFU, tau = vu / (BV / 8), n = 8 * (vu % (BV / 8));
                if (vvec && tau < nval && n0 + n + 8 <= dv) {
                    pre[m] = *(const uint4 *)(vh + (t0 + tau) * HV + n);
                } else {
                    uint32_t x[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        x[j] = (tau < nval && n0 + n + j < dv) ? vh[(t0 + tau) * HV + n + j] : 0u;
                    pre[m] = make_uint4(x[0] | (x[1] << 16), x[2] | (x[3] << 16), x[4] | (x[5] << 16),
                                        x[6] | (x[7] << 16));
                }
            }
        }
    };
    auto store_chunk = [&](int cidx) {
        char *buf = smem + G::oBuf + (cidx & 1) * FB;
        char *vs = smem + G::oVs + (cidx & 1) * G::szVs;
#pragma unroll
        for (int m = 0; m < UPT; ++m) {
            const int u = tid + NT * m;
            if (u < NFU) ((uint4 *)buf)[u] = pre[m];
            else if (u < NU) ((uint4 *)vs)[u - NFU] = pre[m];
        }
    };
    auto flush_outputs = [&](int cprev) {
        const int tp0 = cprev * C, nv = min(C, Tlen - tp0);
        for (int idx = tid; idx < C * (BV / 4); idx += NT) {
            const int tau = idx / (BV / 4), n = 4 * (idx % (BV / 4));
            if (tau >= nv) continue;
            const uint2 val = *(const uint2 *)(Os + tau * LDO + n);
            T *op = o + (hrow + (long)(tp0 + tau) * H) * dv + n0 + n;
            if ((dv & 3) == 0 && n0 + n + 3 < dv) {
                *(uint2 *)op = val;
            } else {
                const T vv[4] = {(T)(val.x & 0xffffu), (T)(val.x >> 16), (T)(val.y & 0xffffu), (T)(val.y >> 16)};
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
                    if (n0 + n + rr < dv) op[rr] = vv[rr];
            }
        }
    };
    // S'^T = (Diag(e^r) S)^T for chunk cidx, the bf16 operand of its products
    f32x4 S[SPW];
    auto write_St = [&](int cidx) {
        const float *erS = (const float *)(smem + G::oBuf + (cidx & 1) * FB + F::oErS);
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + NW * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                const f32x4 sc = *(const f32x4 *)(erS + 16 * rb + g4);
                store4<T>(St + (16 * cb + l16) * LDA + 16 * rb + g4, sc[0] * S[m][0], sc[1] * S[m][1],
                          sc[2] * S[m][2], sc[3] * S[m][3]);
            }
        }
    };

    // ---- initial state (fp32, accumulator layout), first chunk -------------------
#pragma unroll
    for (int m = 0; m < SPW; ++m) {
        S[m] = zero4();
        const int t = wave + NW * m;
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
    load_chunk(0);
    store_chunk(0);
    if (NC > 1) load_chunk(1);
    __syncthreads();
    write_St(0);

    for (int cidx = 0; cidx < NC; ++cidx) {
        const char *buf = smem + G::oBuf + (cidx & 1) * FB;
        const T *Kl = (const T *)(buf + F::oKl), *Kr = (const T *)(buf + F::oKr);
        const T *Ql = (const T *)(buf + F::oQl), *MI = (const T *)(buf + F::oMI);
        const T *Pm = (const T *)(buf + F::oP);
        const float *lam1 = (const float *)(buf + F::oLam), *sK = (const float *)(buf + F::oSK);
        const float *bp = (const float *)(buf + F::oBp);
        const T *Vs = (const T *)(smem + G::oVs + (cidx & 1) * G::szVs);
        __syncthreads();   // S' of this chunk and its factor block are in place

        // ---- the next chunk's block goes to the other buffer (its previous
        //      readers finished before the barrier above); the previous chunk's
        //      outputs are stored before the loads are issued, so every later
        //      wait is on operations issued a whole chunk earlier
        if (cidx + 1 < NC) store_chunk(cidx + 1);
        if (cidx > 0) flush_outputs(cidx - 1);
        if (cidx + 2 < NC) load_chunk(cidx + 2);

        // ---- Z = Diag(b') (N - Kl S') ; the state-independent half of o, Ql S' ---
        f32x4 ZR[YPW];   // fp32 rounding residual of Z, added back in the U product
#pragma unroll
        for (int m = 0; m < YPW; ++m) {
            const int t = wave + NW * m;
            ZR[m] = zero4();
            if (t < NYT) {
                const int jb = t / (BV / 16), nb = t % (BV / 16);
                const f32x4 y = tile_nt<T, D>(Kl + 16 * jb * LDA, LDA, St + 16 * nb * LDA, LDA, zero4(), lane);
                float z[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * jb + g4 + rr;
                    const float nv = (j & 1) ? to_f32(Vs[(j >> 1) * BV + 16 * nb + l16]) : 0.f;
                    z[rr] = bp[j] * (nv - y[rr]);
                }
                const uint32_t z01 = pack_bf16(z[0], z[1]), z23 = pack_bf16(z[2], z[3]);
                *(uint2 *)(Zt + (16 * nb + l16) * LDL + 16 * jb + g4) = make_uint2(z01, z23);
                ZR[m] = f32x4{z[0] - lo_bf16(z01), z[1] - hi_bf16(z01), z[2] - lo_bf16(z23), z[3] - hi_bf16(z23)};
            }
        }
        f32x4 OA[OPW];
#pragma unroll
        for (int m = 0; m < OPW; ++m) {
            const int t = (NW - 1 - wave) + NW * m;   // start on the waves with the fewest Z tiles
            OA[m] = zero4();
            if (t < NOT) {
                const int nb = t / (C / 16), tb = t % (C / 16);
                OA[m] = tile_nt<T, D>(St + 16 * nb * LDA, LDA, Ql + 16 * tb * LDA, LDA, zero4(), lane);
            }
        }
        __syncthreads();

        // ---- U = (I + A)^{-1} Z ----------------------------------------------------
#pragma unroll
        for (int m = 0; m < YPW; ++m) {
            const int t = wave + NW * m;
            if (t < NYT) {
                const int jb = t / (BV / 16), nb = t % (BV / 16);
                const f32x4 u = tile_nt_dyn<T>(MI + 16 * jb * LDL, LDL, Zt + 16 * nb * LDL, LDL,
                                               16 * (jb + 1), ZR[m], lane);
                store4<T>(Ut + (16 * nb + l16) * LDL + 16 * jb + g4, u[0], u[1], u[2], u[3]);
            }
        }
        __syncthreads();

        // ---- o = Ql S' + P U ; S <- e^r (e^r S + Kr^T U) ; S' of the next chunk ------
#pragma unroll
        for (int m = 0; m < OPW; ++m) {
            const int t = (NW - 1 - wave) + NW * m;
            if (t < NOT) {
                const int nb = t / (C / 16), tb = t % (C / 16);
                const f32x4 a = tile_nt_dyn<T>(Ut + 16 * nb * LDL, LDL, Pm + 16 * tb * LDL, LDL,
                                               min(L, 32 * (tb + 1)), OA[m], lane);
                store4<T>(Os + (16 * tb + l16) * LDO + 16 * nb + g4, a[0], a[1], a[2], a[3]);
            }
        }
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + NW * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                const f32x4 lm = *(const f32x4 *)(lam1 + 16 * rb + g4);
                const f32x4 sk = *(const f32x4 *)(sK + 16 * rb + g4);
                f32x4 a;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) a[rr] = lm[rr] * S[m][rr];
                a = tile_tn_bf16<L>(Kr + 16 * rb, LDA, Ut + 16 * cb * LDL, LDL, a, lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[m][rr] = sk[rr] * a[rr];
            }
        }
        // St is read only by the Z and Ql S' products, before the previous barrier
        if (cidx + 1 < NC) write_St(cidx + 1);
    }

    __syncthreads();
    flush_outputs(NC - 1);
    if (S_final) {
        // every read of S0 happened before the chunk loop, so S_final may be S0
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + NW * m;
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
// host side
// ---------------------------------------------------------------------------
constexpr int NWAVES = 8;

static int pad_dim(int dk, int dv) {
    const int p = dk > dv ? dk : dv;
    return p <= 32 ? 32 : (p <= 64 ? 64 : 128);
}

// Value-column slice width of the state pass: the narrowest slice (>= 16
// columns) that still leaves at most one workgroup per compute unit (256 on
// MI355X).
static int slice_width(int BH, int D) {
    int bv = 16;
    while (bv < 32 && bv < D && (long)BH * (D / bv) > 256) bv *= 2;
    return bv;
}

template <int C, int D>
size_t ws_bytes(int B, int Tlen, int H) {
    return (size_t)B * H * ((Tlen + C - 1) / C) * FacLayout<C, D>::bytes;
}

template <int C, int D, int BV>
hipError_t launch_t(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                    const float *beta, const float *gamma, const float *S0, void *o, float *S_final,
                    int B, int Tlen, int H, int dk, int dv, void *ws, hipStream_t stream) {
    using G1 = K1Geom<C, D, NWAVES>;
    using G2 = K2Geom<C, D, BV, NWAVES>;
    const int NC = (Tlen + C - 1) / C, BH = B * H;
    // 16-byte loads of whole rows need d_k == D and 16-byte aligned bases
    // (D is a multiple of 8, so every row start stays aligned)
    const int vec = (dk == D) && ((uintptr_t)q % 16 == 0) && ((uintptr_t)k % 16 == 0) &&
                    ((uintptr_t)e % 16 == 0) && ((uintptr_t)alpha % 16 == 0);
    const int vvec = (dv % 8 == 0) && ((uintptr_t)v % 16 == 0);
    auto k1 = eda_bf16_factors<C, D, NWAVES>;
    auto k2 = eda_bf16_state<C, D, BV, NWAVES>;
    hipError_t err = hipFuncSetAttribute((const void *)k1, hipFuncAttributeMaxDynamicSharedMemorySize, G1::LDS);
    if (err != hipSuccess) return err;
    err = hipFuncSetAttribute((const void *)k2, hipFuncAttributeMaxDynamicSharedMemorySize, G2::LDS);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k1, dim3((unsigned)(BH * NC)), dim3(G1::NT), G1::LDS, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)e, alpha, beta, gamma, (char *)ws, Tlen, H, dk, NC, vec);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int R = (dv + BV - 1) / BV;
    const int grid = 8 * ((BH + 7) / 8) * R;
    hipLaunchKernelGGL(k2, dim3((unsigned)grid), dim3(G2::NT), G2::LDS, stream, (const bf16 *)v, S0,
                       S_final, (bf16 *)o, (const char *)ws, Tlen, H, BH, dk, dv, NC, R, vvec);
    return hipGetLastError();
}

}  // namespace b16

size_t bf16_ws_bytes(int B, int Tlen, int H, int dk, int dv, int chunk) {
    const int D = b16::pad_dim(dk, dv);
#define EDA_WS(CC, DD) if (chunk == CC && D == DD) return b16::ws_bytes<CC, DD>(B, Tlen, H);
    EDA_WS(16, 32) EDA_WS(16, 64) EDA_WS(16, 128)
    EDA_WS(32, 32) EDA_WS(32, 64) EDA_WS(32, 128)
#undef EDA_WS
    return 0;
}

hipError_t launch_bf16(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                       const float *beta, const float *gamma, const float *S0, void *o, float *S_final,
                       int B, int Tlen, int H, int dk, int dv, int chunk, void *ws, hipStream_t stream) {
    const int D = b16::pad_dim(dk, dv), BV = b16::slice_width(B * H, D);
#define EDA_GO(CC, DD, BB)                                                                        \
    if (chunk == CC && D == DD && BV == BB)                                                       \
        return b16::launch_t<CC, DD, BB>(q, k, e, v, alpha, beta, gamma, S0, o, S_final, B, Tlen, \
                                         H, dk, dv, ws, stream);
    EDA_GO(16, 32, 16) EDA_GO(16, 32, 32) EDA_GO(16, 64, 16) EDA_GO(16, 64, 32)
    EDA_GO(16, 128, 16) EDA_GO(16, 128, 32)
    EDA_GO(32, 32, 16) EDA_GO(32, 32, 32) EDA_GO(32, 64, 16) EDA_GO(32, 64, 32)
    EDA_GO(32, 128, 16) EDA_GO(32, 128, 32)
#undef EDA_GO
    return hipErrorInvalidValue;
}

}  // namespace eda
