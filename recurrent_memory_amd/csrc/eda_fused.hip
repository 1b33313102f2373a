// eda_fused.hip -- single-pass chunked EDA forward for bf16 inputs: one
// workgroup per (head, slice of value columns) walks the chunks in order and
// does all of a chunk's work on chip.
//
// Sub-step form (EDA paper, Sec. 3.4, Eqs. (17)-(18); reading slides, frame
// "Two virtual steps recover a standard delta recurrence"): token t is an
// erase sub-step (key e_t, gate gamma_t, decay alpha_t, no value) followed by
// a delta sub-step (key k_t, gate beta_t, value v_t, no decay).  Writing sub-
// step j as S_j = D_j S_{j-1} + kap_j u_j^T, u_j = b'_j (nu_j - (D_j S_{j-1})^T kap_j),
// and unrolling over a chunk of C tokens (L = 2C sub-steps) from the state S
// at the chunk start (G = cumulative log-decay inside the chunk, per key
// channel; Gam = exp(G); t(j) = token of sub-step j):
//
//   (I + A) U = Diag(b') (N - (kap o Gam) S),   A_ji = b'_j sum_c kap_jc kap_ic Gam_t(j)c / Gam_t(i)c   (i < j)
//   o_t       = (q_t o Gam_t)^T S + sum_{i <= 2t+1} P_ti u_i,   P_ti = sum_c q_tc kap_ic Gam_tc / Gam_t(i)c
//   S_next    = Diag(Gam_C) S + Khat^T U,                        Khat_ic = kap_ic Gam_Cc / Gam_t(i)c
//
// (N holds v_t on delta rows and 0 on erase rows).  This is our own
// derivation of the chunk form the paper outlines (its WY/UT equations are
// not legible on the pages), checked against the token recurrence.
//
// Decay ratios are split per channel around r = G_C / 2:
//   Kl = kap o exp(G - r),  Kr = kap o exp(r - G),  Ql = q o exp(G - r),
// so A = Diag(b') strict_lower(Kl Kr^T), P = causal(Ql Kr^T), and with the
// scaled state S' = Diag(exp r) S:
//   Z = Diag(b') (N - Kl S'),  U = (I + A)^{-1} Z,  o = Ql S' + P U,
//   S_next = Diag(exp r) (Diag(exp r) S + Kr^T U)       (Gam_C = exp(2r)).
// Every factor stays within exp(+-|G_C|/2); a chunk in which some channel
// decays by more than exp(-120) (only possible below the safe gate's
// floor alpha = e^-5) takes an exact element-wise path for A and P and the
// unsplit factors kap o Gam, q o Gam, Khat instead.
//
// Work split inside one chunk: the state-independent part (cumulative decay,
// A and P on the matrix cores, the unit lower-triangular inverse: fp32
// substitution on the 16x16 diagonal blocks, then one column block of the
// off-diagonal part per wave) is
// recomputed by every value slice of a head -- matrix-core work instead of
// memory traffic; the state-dependent part (Kl S', U, outputs, next state)
// uses the fp32 state held in registers, with a bf16 copy in LDS as the
// matrix-core operand.  Z enters the inverse product in bf16, and its fp32
// rounding residual is added back so the identity part of U stays exact.
//
// The workgroups of one head's slices get ids congruent mod 8, so they are
// dispatched to the same XCD and read the head's inputs through one L2.
#include <type_traits>

#include "eda_common.h"

namespace eda {

// wide-chunk threshold on the chunk's log2-decay (exp(-120) = 2^-173)
constexpr float WIDE_G2 = 173.f;

__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

// Make this wave's earlier LDS writes visible to its own later LDS reads
// (other lanes included); waves of one workgroup still need a barrier.
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

__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }

template <int C, int D, int BV, int NW>
struct FusedGeom {
    static constexpr int L = 2 * C, NB = L / 16, NT = 64 * NW;
    static constexpr int LDA = D + 8, LDL = L + 8;  // +16 bytes per row
    // element-wise role: 4 consecutive key channels x a run of TPT tokens
    static constexpr int NQ = D / 4;
    static constexpr int TPC = imin(NT / NQ, C);       // threads per channel quad
    static constexpr int TPT = C / TPC;                // tokens per thread
    static constexpr int ACT = NQ * TPC;               // active threads
    static_assert((TPC & (TPC - 1)) == 0 && TPC <= 64 && C % TPC == 0 && ACT <= NT, "split");
    static_assert(TPT == 1 || TPT == 2, "token run");
    static constexpr int VPT = (C * BV + NT - 1) / NT; // value elements per thread
    // waves 0..NB-1 invert the diagonal blocks of A and sweep the inverse; the
    // other NZW "matrix" waves own the Z/U tiles, A and P tiles and the
    // state-independent half of the outputs
    static constexpr int NZW = NW - NB;
    static_assert(NZW >= 1, "too few waves for this chunk size");
    static constexpr int NYT = NB * (BV / 16);         // Z / U tiles
    static constexpr int YPW = (NYT + NZW - 1) / NZW;
    static constexpr int NOT = (BV / 16) * (C / 16);   // output tiles
    static constexpr int OPW = (NOT + NZW - 1) / NZW;
    // LDS layout (bytes)
    static constexpr int szKl = align16(L * LDA * 2), szQl = align16(C * LDA * 2);
    static constexpr int szP = align16(C * LDL * 2);
    static constexpr int ADS = 20;                     // Ad row stride (floats): conflict-free writes, 16-byte rows
    static constexpr int szAbf = align16(L * LDL * 2), szAd = NB * 16 * ADS * 4;
    static constexpr int szMI = align16(L * LDL * 2);
    static constexpr int szGs = C * D * 4;             // element-wise path only, aliases MI, MT
    static constexpr int szInv = imax(2 * szMI, szGs);
    static constexpr int szSt = align16(BV * LDA * 2), szVs = align16(C * BV * 2);
    static constexpr int szZt = align16(BV * LDL * 2);
    static constexpr int LDO = BV + 8, szOs = align16(C * LDO * 2);   // output staging
    static constexpr int szMisc = (L + 2 * C + 4 * D) * 4;
    // staging of one chunk's raw inputs (written late in the previous chunk)
    static constexpr int ASD = D + 8;                  // alpha staging row stride (floats)
    static constexpr int szQs = align16(C * LDA * 2), szAs = align16(C * ASD * 4);
    static constexpr int LPR = D / 8, RPP = NT / LPR, PQ = (C + RPP - 1) / RPP;   // 16-byte loads of bf16 rows
    static constexpr int LPA = D / 4, RPA = NT / LPA, PA = (C + RPA - 1) / RPA;   // 16-byte loads of alpha rows
    static constexpr int oKl = 0, oKr = oKl + szKl, oQl = oKr + szKl, oQs = oQl + szQl;
    static constexpr int oKs = oQs + szQs, oEs = oKs + szQs, oAs = oEs + szQs;
    static constexpr int oP = oAs + szAs, oAbf = oP + szP;
    static constexpr int oAd = oAbf + szAbf, oInv = oAd + szAd, oSt = oInv + szInv;
    static constexpr int oVs = oSt + szSt, oZt = oVs + szVs, oUt = oZt + szZt;
    static constexpr int oOs = oUt + szZt, oMisc = oOs + szOs;
    static constexpr int LDS = oMisc + szMisc;
    static_assert(LDS <= 160 * 1024, "LDS budget exceeded");
};

template <int C, int D, int BV, int NW>
__global__ void __launch_bounds__(64 * NW)
eda_chunk_fused(const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ e,
                const bf16 *__restrict__ v, const float *__restrict__ alpha,
                const float *__restrict__ beta, const float *__restrict__ gamma,
                const float *S0, float *S_final, bf16 *__restrict__ o, int Tlen, int H, int BH,
                int dk, int dv, int NC, int R, int vec) {
    using G = FusedGeom<C, D, BV, NW>;
    using T = bf16;
    constexpr int L = G::L, NB = G::NB, NT = G::NT, LDA = G::LDA, LDL = G::LDL;
    constexpr int TPC = G::TPC, TPT = G::TPT, VPT = G::VPT, NYT = G::NYT, YPW = G::YPW;
    constexpr int NZW = G::NZW, NOT = G::NOT, OPW = G::OPW;
    constexpr int ADS = G::ADS, ASD = G::ASD;
    constexpr int LPR = G::LPR, RPP = G::RPP, PQ = G::PQ, LPA = G::LPA, RPA = G::RPA, PA = G::PA;
    constexpr int NST = (D / 16) * (BV / 16);          // state tiles
    constexpr int SPW = (NST + NW - 1) / NW;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Kl = (T *)(smem + G::oKl);       // kap o exp(G - r)                 [L][LDA]
    T *Kr = (T *)(smem + G::oKr);       // kap o exp(r - G); wide: raw kap, then Khat [L][LDA]
    T *Ql = (T *)(smem + G::oQl);       // q o exp(G - r)                   [C][LDA]
    T *Qs = (T *)(smem + G::oQs);       // raw q, k, e of the chunk          [C][LDA]
    T *Ks = (T *)(smem + G::oKs);
    T *Es = (T *)(smem + G::oEs);
    float *As = (float *)(smem + G::oAs);  // raw alpha of the chunk        [C][ASD]
    T *Pm = (T *)(smem + G::oP);        // P, causal                        [C][LDL]
    T *Abf = (T *)(smem + G::oAbf);     // A, off-diagonal 16-blocks        [L][LDL]
    float *Ad = (float *)(smem + G::oAd);  // A, diagonal 16-blocks (fp32)  [NB][16][ADS]
    T *MI = (T *)(smem + G::oInv);      // (I + A)^{-1}                     [L][LDL]
    T *MT = MI + L * LDL;               // its transpose (diagonal blocks)  [L][LDL]
    float *Gs = (float *)(smem + G::oInv);  // G (wide)                     [C][D]
    T *St = (T *)(smem + G::oSt);       // S'^T (bf16 operand)              [BV][LDA]
    T *Vs = (T *)(smem + G::oVs);       // values of the slice              [C][BV]
    T *Zt = (T *)(smem + G::oZt);       // Z^T (bf16)                       [BV][LDL]
    T *Ut = (T *)(smem + G::oUt);       // U^T (bf16)                       [BV][LDL]
    T *Os = (T *)(smem + G::oOs);       // previous chunk's outputs          [C][LDO]
    float *bp = (float *)(smem + G::oMisc);   // b' per sub-step            [L]
    float *sb = bp + L, *sg = sb + C;         // beta, gamma per token      [C]
    float *glc = sg + C;                      // G_C per channel (log2)     [D]
    float *erL = glc + D;                     // exp(r) = 2^(G_C/2)         [D]
    float *lam1 = erL + D, *sK = lam1 + D;    // state-update scales        [D]

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / R) * 8 + xcd, slice = slot % R;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H, n0 = slice * BV;
    const long sbase = (long)bh * dk * dv;
    auto row = [&](int t) -> long { return ((long)b * Tlen + t) * H + h; };
    // this head's first token; per-token strides H*d fit in 32 bits (the C ABI
    // bounds B*T*H*d below 2^31)
    const long hrow = (long)b * Tlen * H + h;
    const bf16 *qh = q + hrow * dk, *kh = k + hrow * dk, *eh = e + hrow * dk;
    const float *ah = alpha + hrow * dk, *bh_ = beta + hrow, *gh = gamma + hrow;
    const bf16 *vh = v + hrow * dv + n0;
    const int HK = H * dk, HV = H * dv;

    // ---- prefetch of one chunk: whole-row 16-byte loads into registers, ---------------
    // ---- written to the LDS staging buffers later (stage_chunk) ----------------------
    uint4 rq[PQ], rk[PQ], re[PQ];
    f32x4 ra[PA];
    bf16 pv[VPT];
    float pb = 0.f, pg = 0.f;
    auto load_chunk = [&](int cidx, int tid) {
        const int t0 = cidx * C, nval = min(C, Tlen - t0);
        if (vec && nval == C) {
            // whole chunk, d_k == D, aligned rows: no masking
#pragma unroll
            for (int p = 0; p < PQ; ++p) {
                const int r = tid / LPR + RPP * p, blk = tid % LPR;
                if (RPP * PQ == C || r < C) {
                    const int off = (t0 + r) * HK + 8 * blk;
                    rq[p] = *(const uint4 *)(qh + off);
                    rk[p] = *(const uint4 *)(kh + off);
                    re[p] = *(const uint4 *)(eh + off);
                }
            }
#pragma unroll
            for (int p = 0; p < PA; ++p) {
                const int r = tid / LPA + RPA * p, blk = tid % LPA;
                if (RPA * PA == C || r < C) ra[p] = *(const f32x4 *)(ah + (t0 + r) * HK + 4 * blk);
            }
        } else {
#pragma unroll
            for (int p = 0; p < PQ; ++p) {
                const int r = tid / LPR + RPP * p, c8 = 8 * (tid % LPR);
                uint32_t xq[8], xk[8], xe[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const bool ok = r < nval && c8 + j < dk;
                    const int off = (t0 + r) * HK + c8 + j;
                    xq[j] = ok ? qh[off] : 0u;
                    xk[j] = ok ? kh[off] : 0u;
                    xe[j] = ok ? eh[off] : 0u;
                }
                rq[p] = make_uint4(xq[0] | (xq[1] << 16), xq[2] | (xq[3] << 16), xq[4] | (xq[5] << 16), xq[6] | (xq[7] << 16));
                rk[p] = make_uint4(xk[0] | (xk[1] << 16), xk[2] | (xk[3] << 16), xk[4] | (xk[5] << 16), xk[6] | (xk[7] << 16));
                re[p] = make_uint4(xe[0] | (xe[1] << 16), xe[2] | (xe[3] << 16), xe[4] | (xe[5] << 16), xe[6] | (xe[7] << 16));
            }
#pragma unroll
            for (int p = 0; p < PA; ++p) {
                const int r = tid / LPA + RPA * p, c4 = 4 * (tid % LPA);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bool ok = r < nval && c4 + j < dk;
                    ra[p][j] = ok ? ah[(t0 + r) * HK + c4 + j] : 1.f;
                }
            }
        }
        if (nval == C && n0 + BV <= dv && C * BV == NT * VPT) {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                const int idx = tid + NT * m;
                pv[m] = vh[(t0 + idx / BV) * HV + idx % BV];
            }
        } else {
#pragma unroll
            for (int m = 0; m < VPT; ++m) {
                const int idx = tid + NT * m, tau = idx / BV, n = idx % BV;
                const bool ok = idx < C * BV && tau < nval && n0 + n < dv;
                pv[m] = ok ? vh[(t0 + tau) * HV + n] : (bf16)0;
            }
        }
        if (tid < C) {
            const bool ok = tid < nval;
            pb = ok ? bh_[(t0 + tid) * H] : 0.f;
            pg = ok ? gh[(t0 + tid) * H] : 0.f;
        }
    };
    auto stage_chunk = [&](int tid) {
#pragma unroll
        for (int p = 0; p < PQ; ++p) {
            const int r = tid / LPR + RPP * p, blk = tid % LPR;
            if (RPP * PQ == C || r < C) {
                *(uint4 *)(Qs + r * LDA + 8 * blk) = rq[p];
                *(uint4 *)(Ks + r * LDA + 8 * blk) = rk[p];
                *(uint4 *)(Es + r * LDA + 8 * blk) = re[p];
            }
        }
#pragma unroll
        for (int p = 0; p < PA; ++p) {
            const int r = tid / LPA + RPA * p, blk = tid % LPA;
            if (RPA * PA == C || r < C) *(f32x4 *)(As + r * ASD + 4 * blk) = ra[p];
        }
    };

    // ---- outputs: staged in LDS, written one chunk later ----------------------------
    // Loads and stores share one completion counter, so a wait for the next
    // chunk's inputs would also wait for stores issued just before it; writing
    // a chunk's outputs right before the following prefetch keeps every wait
    // on operations issued a whole chunk earlier.
    constexpr int LDO = G::LDO;
    auto flush_outputs = [&](int cprev, int tid) {
        const int tp0 = cprev * C, nv = min(C, Tlen - tp0);
        for (int idx = tid; idx < C * (BV / 4); idx += NT) {
            const int tau = idx / (BV / 4), n = 4 * (idx % (BV / 4));
            if (tau >= nv) continue;
            const uint2 val = *(const uint2 *)(Os + tau * LDO + n);
            T *op = o + row(tp0 + tau) * dv + n0 + n;
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

    // ---- initial state (fp32, accumulator layout) ----------------------------------
    f32x4 S[SPW];
    {
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int g4 = 4 * (lane >> 4), l16 = lane & 15;
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
        load_chunk(0, tid);
        stage_chunk(tid);
    }
    __syncthreads();

    for (int cidx = 0; cidx < NC; ++cidx) {
        const int t0 = cidx * C, nvalid = min(C, Tlen - t0);
        // Lane roles are re-derived inside the loop from an opaque copy of the
        // thread id; otherwise the compiler hoists every per-lane LDS address of
        // the unrolled body out of the loop and runs out of registers.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g4 = 4 * (lane >> 4), l16 = lane & 15;
        const bool act = tid < G::ACT;
        const int qd = tid / TPC, seg = tid % TPC, c0 = 4 * qd;

        // ---- 1a. gates; cumulative log-decay per channel ------------------------
        if (tid < C) {
            sb[tid] = pb;
            sg[tid] = pg;
            bp[2 * tid] = pg;
            bp[2 * tid + 1] = pb;
        }
        // g: cumulative log2-decay of this thread's tokens; G = g ln 2
        float g[TPT][4];
        bool wide_here = false;
        {
            // tokens seg + TPC i: one group scan per i, offset by the earlier runs' totals
            float base[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const f32x4 pa = act ? *(const f32x4 *)(As + (seg + TPC * i) * ASD + c0)
                                     : f32x4{1.f, 1.f, 1.f, 1.f};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    g[i][j] = base[j] + scan_group<TPC>(__builtin_amdgcn_logf(pa[j]), seg);
                    base[j] = group_last<TPC>(g[i][j]);
                }
            }
            if (act && seg == TPC - 1) {
                *(f32x4 *)(glc + c0) = f32x4{base[0], base[1], base[2], base[3]};
                *(f32x4 *)(erL + c0) = f32x4{exp2f_(0.5f * base[0]), exp2f_(0.5f * base[1]),
                                             exp2f_(0.5f * base[2]), exp2f_(0.5f * base[3])};
#pragma unroll
                for (int j = 0; j < 4; ++j) wide_here |= base[j] < -WIDE_G2;
            }
        }
        // also the barrier after the previous chunk's last reads
        const bool wide = __syncthreads_or(wide_here) != 0;
        const f32x4 gl = act ? *(const f32x4 *)(glc + c0) : zero4();

        // ---- 1b. scaled operands, scales, S' and V --------------------------------
        if (act) {
            float r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = wide ? 0.f : 0.5f * gl[j];
            auto token_ops = [&](auto WIDE) {
#pragma unroll
                for (int i = 0; i < TPT; ++i) {
                    const int tau = seg + TPC * i;
                    const uint2 pq = *(const uint2 *)(Qs + tau * LDA + c0);
                    const uint2 pk = *(const uint2 *)(Ks + tau * LDA + c0);
                    const uint2 pe = *(const uint2 *)(Es + tau * LDA + c0);
                    float ev[4], kv[4], qv[4];
                    ev[0] = lo_bf16(pe.x); ev[1] = hi_bf16(pe.x);
                    ev[2] = lo_bf16(pe.y); ev[3] = hi_bf16(pe.y);
                    kv[0] = lo_bf16(pk.x); kv[1] = hi_bf16(pk.x);
                    kv[2] = lo_bf16(pk.y); kv[3] = hi_bf16(pk.y);
                    qv[0] = lo_bf16(pq.x); qv[1] = hi_bf16(pq.x);
                    qv[2] = lo_bf16(pq.y); qv[3] = hi_bf16(pq.y);
                    float f[4];
                    if constexpr (!decltype(WIDE)::value) {
                        float fi[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            f[j] = exp2f_(g[i][j] - r[j]);
                            fi[j] = exp2f_(r[j] - g[i][j]);
                        }
                        *(uint2 *)(Kr + (2 * tau) * LDA + c0) =
                            make_uint2(pack_bf16(ev[0] * fi[0], ev[1] * fi[1]), pack_bf16(ev[2] * fi[2], ev[3] * fi[3]));
                        *(uint2 *)(Kr + (2 * tau + 1) * LDA + c0) =
                            make_uint2(pack_bf16(kv[0] * fi[0], kv[1] * fi[1]), pack_bf16(kv[2] * fi[2], kv[3] * fi[3]));
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            f[j] = exp2f_(g[i][j]);
                            Gs[tau * D + c0 + j] = g[i][j];
                        }
                        *(uint2 *)(Kr + (2 * tau) * LDA + c0) = pe;
                        *(uint2 *)(Kr + (2 * tau + 1) * LDA + c0) = pk;
                    }
                    *(uint2 *)(Kl + (2 * tau) * LDA + c0) =
                        make_uint2(pack_bf16(ev[0] * f[0], ev[1] * f[1]), pack_bf16(ev[2] * f[2], ev[3] * f[3]));
                    *(uint2 *)(Kl + (2 * tau + 1) * LDA + c0) =
                        make_uint2(pack_bf16(kv[0] * f[0], kv[1] * f[1]), pack_bf16(kv[2] * f[2], kv[3] * f[3]));
                    *(uint2 *)(Ql + tau * LDA + c0) =
                        make_uint2(pack_bf16(qv[0] * f[0], qv[1] * f[1]), pack_bf16(qv[2] * f[2], qv[3] * f[3]));
                }
            };
            if (!wide) token_ops(std::false_type{});
            else token_ops(std::true_type{});
            if (seg == 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float er = exp2f_(r[j]);
                    lam1[c0 + j] = wide ? exp2f_(gl[j]) : er;
                    sK[c0 + j] = wide ? 1.f : er;
                }
            }
        }
        // S' = Diag(exp r) S, stored transposed as the bf16 operand
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int t = wave + NW * m;
            if (t < NST) {
                const int rb = t / (BV / 16), cb = t % (BV / 16);
                float sc[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) sc[rr] = wide ? 1.f : erL[16 * rb + g4 + rr];
                store4<T>(St + (16 * cb + l16) * LDA + 16 * rb + g4, sc[0] * S[m][0], sc[1] * S[m][1],
                          sc[2] * S[m][2], sc[3] * S[m][3]);
            }
        }
#pragma unroll
        for (int m = 0; m < VPT; ++m) {
            const int idx = tid + NT * m;
            if (idx < C * BV) Vs[idx] = pv[m];
        }
        if (cidx > 0) flush_outputs(cidx - 1, tid);
        if (cidx + 1 < NC) load_chunk(cidx + 1, tid);
        __syncthreads();

        // ---- 1c. Z = Diag(b') (N - Kl S') ; A (strictly lower) ; P (causal) -------
        const int mw = wave - NB;  // matrix-wave index (< 0 on the inverse waves)
        f32x4 ZR[YPW];  // fp32 rounding residual of Z, kept for the U product
#pragma unroll
        for (int m = 0; m < YPW; ++m) {
            const int t = mw + NZW * m;
            ZR[m] = zero4();
            if (mw >= 0 && t < NYT) {
                const int jb = t / (BV / 16), nb = t % (BV / 16);
                f32x4 y = tile_nt<T, D>(Kl + 16 * jb * LDA, LDA, St + 16 * nb * LDA, LDA, zero4(), lane);
                float z[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int j = 16 * jb + g4 + rr;
                    const float nv = (j & 1) ? to_f32(Vs[(j >> 1) * BV + 16 * nb + l16]) : 0.f;
                    z[rr] = bp[j] * (nv - y[rr]);
                }
                const uint32_t z01 = pack_bf16(z[0], z[1]), z23 = pack_bf16(z[2], z[3]);
                *(uint2 *)(Zt + (16 * nb + l16) * LDL + 16 * jb + g4) = make_uint2(z01, z23);
                ZR[m] = f32x4{z[0] - lo_bf16(z01), z[1] - hi_bf16(z01), z[2] - lo_bf16(z23),
                              z[3] - hi_bf16(z23)};
            }
        }
        // Diagonal blocks of A: wave J computes block J, then inverts it by
        // fp32 substitution (lanes = columns) without leaving the wave.
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
                uint4 *mt = (uint4 *)(MT + (16 * J + col) * LDL + 16 * J);
                mt[0] = make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                                   pack_bf16(x[6], x[7]));
                mt[1] = make_uint4(pack_bf16(x[8], x[9]), pack_bf16(x[10], x[11]),
                                   pack_bf16(x[12], x[13]), pack_bf16(x[14], x[15]));
            }
        };
        if (!wide) {
            if (wave < NB) {
                const int J = wave;
                f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * J * LDA, LDA, zero4(), lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int jl = g4 + rr;
                    Ad[(J * 16 + jl) * ADS + l16] = (jl > l16) ? bp[16 * J + jl] * a[rr] : 0.f;
                }
                wave_lds_sync();
                invert_diag(J);
            }
            // off-diagonal A tiles, then P^T tiles, on the matrix waves
            constexpr int NOD = NB * (NB - 1) / 2;
            constexpr int NPT = NB * (C / 16);
            for (int t = mw; mw >= 0 && t < NOD + NPT; t += NZW) {
                if (t < NOD) {
                    int J = 1, I = t;
                    while (I >= J) { I -= J; ++J; }
                    f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * I * LDA, LDA, zero4(), lane);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int j = 16 * J + g4 + rr;
                        Abf[j * LDL + 16 * I + l16] = from_f32<T>(bp[j] * a[rr]);
                    }
                } else {
                    // P^T tile: rows = sub-steps i, cols = tokens; kept for i <= 2 tau + 1
                    const int I = (t - NOD) / (C / 16), Tb = (t - NOD) % (C / 16);
                    if (16 * I > 32 * Tb + 31) continue;   // beyond every token's causal range
                    f32x4 a = tile_nt<T, D>(Kr + 16 * I * LDA, LDA, Ql + 16 * Tb * LDA, LDA, zero4(), lane);
                    const int tau = 16 * Tb + l16, i0 = 16 * I + g4;
                    float w4[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) w4[rr] = (i0 + rr <= 2 * tau + 1) ? a[rr] : 0.f;
                    store4<T>(Pm + tau * LDL + i0, w4[0], w4[1], w4[2], w4[3]);
                }
            }
        } else {
            // exact element-wise path: exp(G_j - G_i) is never split
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
                        s += to_f32(Qs[tau * LDA + cc]) * to_f32(Kr[ii * LDA + cc]) *
                             exp2f_(Gs[tau * D + cc] - Gs[ti * D + cc]);
                }
                Pm[tau * LDL + ii] = from_f32<T>(s);
            }
            __syncthreads();
            // the state update reads Kr: turn the raw keys into Khat = kap 2^(G_C - G)
            for (int idx = tid; idx < L * D; idx += NT) {
                const int j = idx / D, cc = idx % D;
                Kr[j * LDA + cc] = from_f32<T>(to_f32(Kr[j * LDA + cc]) * exp2f_(glc[cc] - Gs[(j >> 1) * D + cc]));
            }
            __syncthreads();
            if (wave < NB) invert_diag(wave);
        }
        __syncthreads();

        // ---- 1d (matrix waves): the state-independent half of the outputs, Ql S'
        f32x4 OA[OPW];
#pragma unroll
        for (int m = 0; m < OPW; ++m) {
            const int t = mw + NZW * m;
            OA[m] = zero4();
            if (mw >= 0 && t < NOT) {
                const int nb = t / (C / 16), tb = t % (C / 16);
                OA[m] = tile_nt<T, D>(St + 16 * nb * LDA, LDA, Ql + 16 * tb * LDA, LDA, zero4(), lane);
            }
        }
        // ---- 1d. off-diagonal blocks of (I + A)^{-1}, one column block per wave:
        //      X_JI = -X_JJ sum_{I <= K < J} A_JK X_KI, for J = I+1, I+2, ...
        // A 16x16 accumulator (lane: rows 4g..4g+3 of column l%16) is exactly the
        // B operand of the 16x16x16 instruction, so the X_KI stay in registers.
        if (wave < NB - 1) {
            const int I = wave;
            s16x4 xb[NB];   // X_KI as bf16 B operands (K >= I)
#pragma unroll
            for (int K = 0; K < NB - 1; ++K)
                if (K == I) xb[K] = *(const s16x4 *)(MT + (16 * K + l16) * LDL + 16 * K + g4);
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
                const uint32_t t01 = pack_bf16(t[0], t[1]), t23 = pack_bf16(t[2], t[3]);
                const s16x4 tb = __builtin_bit_cast(s16x4, make_uint2(t01, t23));
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

        // ---- 2a. U = (I + A)^{-1} Z  (Z's rounding residual added in fp32) --------
        // First the next chunk's raw inputs go to the staging buffers: their last
        // readers in this chunk (1a, 1b, the element-wise path of 1c) are behind
        // the barriers above, and the barrier below orders them before the next
        // chunk's reads.
        if (cidx + 1 < NC) stage_chunk(tid);
#pragma unroll
        for (int m = 0; m < YPW; ++m) {
            const int t = mw + NZW * m;
            if (mw >= 0 && t < NYT) {
                const int jb = t / (BV / 16), nb = t % (BV / 16);
                f32x4 u = tile_nt_dyn<T>(MI + 16 * jb * LDL, LDL, Zt + 16 * nb * LDL, LDL,
                                         16 * (jb + 1), ZR[m], lane);
                store4<T>(Ut + (16 * nb + l16) * LDL + 16 * jb + g4, u[0], u[1], u[2], u[3]);
            }
        }
        __syncthreads();

        // ---- 2b. outputs o^T = S'^T Ql^T + U^T P^T ; S <- e^r (e^r S + Kr^T U) ------
#pragma unroll
        for (int m = 0; m < OPW; ++m) {
            const int t = mw + NZW * m;
            if (mw >= 0 && t < NOT) {
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
                f32x4 a;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) a[rr] = lam1[16 * rb + g4 + rr] * S[m][rr];
                a = tile_tn_bf16<L>(Kr + 16 * rb, LDA, Ut + 16 * cb * LDL, LDL, a, lane);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) S[m][rr] = sK[16 * rb + g4 + rr] * a[rr];
            }
        }
    }

    __syncthreads();
    flush_outputs(NC - 1, threadIdx.x);
    if (S_final) {
        // every read of S0 happened before the chunk loop, so S_final may be S0
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        const int g4 = 4 * (lane >> 4), l16 = lane & 15;
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
template <int C, int D, int BV, int NW>
hipError_t launch_fused_t(const void *q, const void *k, const void *e, const void *v,
                          const float *alpha, const float *beta, const float *gamma,
                          const float *S0, void *o, float *S_final, int B, int Tlen, int H, int dk,
                          int dv, hipStream_t stream) {
    using G = FusedGeom<C, D, BV, NW>;
    auto kern = eda_chunk_fused<C, D, BV, NW>;
    hipError_t err = hipFuncSetAttribute((const void *)kern,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, G::LDS);
    if (err != hipSuccess) return err;
    const int NC = (Tlen + C - 1) / C, BH = B * H;
    const int R = (dv + BV - 1) / BV;
    const int grid = 8 * ((BH + 7) / 8) * R;
    // 16-byte loads of whole token rows need d_k == D and 16-byte aligned
    // bases (D is a multiple of 8, so every row start stays aligned);
    // otherwise element loads are used
    const int vec = (dk == D) && ((uintptr_t)q % 16 == 0) && ((uintptr_t)k % 16 == 0) &&
                    ((uintptr_t)e % 16 == 0) && ((uintptr_t)alpha % 16 == 0);
    hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3(G::NT), G::LDS, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)e, (const bf16 *)v, alpha, beta, gamma, S0,
                       S_final, (bf16 *)o, Tlen, H, BH, dk, dv, NC, R, vec);
    return hipGetLastError();
}

static int fused_pad_dim(int dk, int dv) {
    const int p = dk > dv ? dk : dv;
    return p <= 32 ? 32 : (p <= 64 ? 64 : 128);
}

// Value-column slice width: the narrowest slice (>= 16 columns) that still
// leaves at most one workgroup per compute unit (256 on MI355X).
static int fused_slice(int BH, int D) {
    int bv = 16;
    while (bv < 32 && bv < D && (long)BH * (D / bv) > 256) bv *= 2;
    return bv;
}

hipError_t launch_fused(const void *q, const void *k, const void *e, const void *v,
                        const float *alpha, const float *beta, const float *gamma, const float *S0,
                        void *o, float *S_final, int B, int Tlen, int H, int dk, int dv, int chunk,
                        hipStream_t stream) {
    const int D = fused_pad_dim(dk, dv), BV = fused_slice(B * H, D);
#define EDA_FUSED(CC, DD, BB, WW)                                                               \
    if (chunk == CC && D == DD && BV == BB)                                                     \
        return launch_fused_t<CC, DD, BB, WW>(q, k, e, v, alpha, beta, gamma, S0, o, S_final, B, \
                                              Tlen, H, dk, dv, stream);
    EDA_FUSED(16, 32, 16, 8) EDA_FUSED(16, 32, 32, 8)
    EDA_FUSED(16, 64, 16, 8) EDA_FUSED(16, 64, 32, 8)
    EDA_FUSED(16, 128, 16, 8) EDA_FUSED(16, 128, 32, 8)
    EDA_FUSED(32, 32, 16, 8) EDA_FUSED(32, 32, 32, 8)
    EDA_FUSED(32, 64, 16, 8) EDA_FUSED(32, 64, 32, 8)
    EDA_FUSED(32, 128, 16, 8) EDA_FUSED(32, 128, 32, 8)
#undef EDA_FUSED
    return hipErrorInvalidValue;
}

}  // namespace eda
