// eda_bf16.hip -- chunked EDA forward for bf16 inputs, in two kernels.
//
// Sub-step form (EDA paper, Sec. 3.4, Eqs. (17)-(18); reading slides, frame
// "Two virtual steps recover a standard delta recurrence"): token t is an
// erase sub-step (key e_t, gate gamma_t, decay alpha_t, no value) followed by
// a delta sub-step (key k_t, gate beta_t, value v_t, no decay).  Writing sub-
// step j as S_j = D_j S_{j-1} + kap_j u_j^T, u_j = b'_j (nu_j - (D_j S_{j-1})^T lam_j)
// (lam = kap for EDA) and unrolling over a chunk of C tokens (L = 2C sub-
// steps) from the state S at the chunk start (G = cumulative log-decay inside
// the chunk, per key channel; t(j) = token of sub-step j) gives, with
// A_ji = b'_j sum_c lam_jc kap_ic e^{G_t(j)c - G_t(i)c} (i < j), M = (I + A)^{-1},
// P_ti = sum_c q_tc kap_ic e^{G_tc - G_t(i)c} (i <= 2t+1), Khat_i = kap_i o e^{G_C - G_t(i)}:
//
//   U = T' V - W S,   W = M Diag(b') (lam o e^G),   T'[:, t] = M[:, 2t+1] beta_t
//   o = (q o e^G) S + P U,      S_next = Diag(e^{G_C}) S + Khat^T U
//
// (our own derivation of the chunk form the paper outlines -- its WY/UT
// equations are not legible on the pages -- checked in fp64 against the
// token recurrence by the CPU tests).  Substituting U, the chunk is an affine
// map of the state with chunk-constant factors:
//
//   S_next = Diag(e^{G_C}) S + Phi S + Psi V,   O = Qhat S + Phat V
//   Phi = -Khat^T W  [d_k x d_k],  Psi = Khat^T T'  [d_k x C],
//   Qhat = (q o e^G) - P W  [C x d_k],  Phat = P T'  [C x C]
//
// so the serial pass over chunks needs one product per chunk on its chain.
// With Y = M^T Khat and Z = P M these are Phi = -Y^T Diag(b')(lam o e^G),
// Psi = Y[delta rows]^T Diag(beta), Qhat = q o e^G - Z Diag(b')(lam o e^G),
// Phat = Z[:, delta cols] Diag(beta): W and T' are never formed.
//
// Range safety: decay ratios are split per channel around r = G_C / 2,
//   Kl = Diag(b') lam o e^{G - r},  Kr = kap o e^{r - G},  Ql = q o e^{G - r},
// so A = strict_lower(Kl Kr^T) and P = causal(Ql Kr^T) only see factors
// within e^{+-|G_C|/2}; the exports carry the scale e^r of each key channel
// (lam o e^G = Kl e^r / b', Khat = Kr e^r, q o e^G = Ql e^r).  The split
// operands stay within e^{+-75} (inside the bf16 and fp32 ranges, with room
// for the sums of products that reach e^{75}); a chunk in which some channel
// decays by more than e^-150 forms A and P element-wise from e^{G_j - G_i}
// and uses unsplit operands (r = 0).
//
// Rounding: every matrix-core operand is bf16; products accumulate in fp32.
// Each exported factor is rounded once, from fp32 accumulators: beta and e^r
// are applied to the fp32 products, never to a rounded operand, so the
// rounded M enters W-like and T'-like terms identically (a write followed by
// an erase of the same address then cancels as in exact arithmetic).  P is
// kept as a bf16 pair P_hi + P_lo in Z = P M.
//
// Kernel 1 (eda_bf16_factors): persistent workgroups walk the (head, chunk)
//   items; each item's raw inputs are fetched into registers while the
//   previous item is processed.  Per item: cumulative decay, operands, A and
//   P on the matrix cores, (I + A)^{-1} (fp32 substitution on the 16 x 16
//   diagonal blocks, then one column block of the rest per wave), Y and Z,
//   then Phi and Qhat; Psi, Phat, Phi, Qhat and e^{G_C} go to the workspace.
// Kernel 2 (eda_bf16_state): one workgroup per (head, slice of value
//   columns), serial over chunks, fp32 state in registers, one barrier per
//   chunk.  The factors are stored in the per-lane order of the matrix-core
//   operands, so each wave fetches its own operands straight into registers
//   two chunks ahead.
//
// Workspace: one block of Fac<C, D>::bytes per chunk and head.  A "fragment"
// of a matrix X (rows x k, row-major view) is the 16 x 32 block at
// (16 rb, 32 ks): 64 lanes x 16 bytes, lane 16 g + r holding
// X[16 rb + r][32 ks + 8 g .. 32 ks + 8 g + 7] -- the operand layout of the
// 16x16x32 bf16 matrix instruction.
#include <type_traits>

#include "eda_common.h"

namespace eda {
namespace b16 {

// wide-chunk threshold on a chunk's log2-decay (e^-150 = 2^-216.4)
constexpr float WIDE_G2 = 216.4f;

__host__ __device__ constexpr int imax(int a, int b) { return a > b ? a : b; }
__host__ __device__ constexpr int imin(int a, int b) { return a < b ? a : b; }
__host__ __device__ constexpr int align16(int x) { return (x + 15) / 16 * 16; }
__host__ __device__ constexpr int align256(int x) { return (x + 255) / 256 * 256; }

__device__ __forceinline__ float exp2f_(float x) { return __builtin_amdgcn_exp2f(x); }

// Make this wave's earlier LDS writes visible to its own later LDS reads.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

typedef __attribute__((ext_vector_type(8))) short s16x8;

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Row fragment: lane 16 g + r gets p[r * ld + 8 g .. 8 g + 7] (any memory).
__device__ __forceinline__ bf16x8 frag_row(const bf16 *p, int ld, int lane) {
    return *reinterpret_cast<const bf16x8 *>(p + (lane & 15) * ld + 8 * (lane >> 4));
}
// Column fragment from LDS: lane 16 g + n gets p[(8 g + j) * ld + n], j = 0..7.
// The gfx950 transposing read: within a group of 16 lanes, lane i addresses
// row i/4, columns 4(i%4)..4(i%4)+3 of a 4 x 16 block, and lane n receives
// column n of the 4 rows.
__device__ __forceinline__ bf16x8 frag_col(const bf16 *p, int ld, int lane) {
    const int g = lane >> 4, i = lane & 15;
    const bf16 *mp = p + (8 * g + (i >> 2)) * ld + 4 * (i & 3);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)mp);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(mp + 4 * ld));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The same for a k = 16 operand of the 16x16x16 instruction: lane 16 g + n
// gets p[(4 g + j) * ld + n], j = 0..3.
__device__ __forceinline__ s16x4 frag_col4(const bf16 *p, int ld, int lane) {
    const int g = lane >> 4, i = lane & 15;
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(p + (4 * g + (i >> 2)) * ld + 4 * (i & 3)));
}

// Lane coordinates for 16x16 MFMA tiles (lane = 16 gq + l16, g4 = 4 gq), from
// an opaque copy of the lane id.  Each phase of a persistent kernel's item
// loop takes its own copy, so the lane-dependent LDS and workspace addresses
// are formed inside the phase instead of being hoisted out of the loop and
// held in registers across every phase.
struct LaneIds {
    int lane, g4, l16, gq;
};
__device__ __forceinline__ LaneIds lane_ids(int tid) {
    int x = tid & 63;
    asm volatile("" : "+v"(x));
    return {x, 4 * (x >> 4), x & 15, x >> 4};
}

// LDS byte address of a per-lane base, opaque to the compiler: the fixed
// offsets added to it stay in the instructions' immediate fields instead of
// being folded into the base (one register per offset, spilled under
// pressure).
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    uint32_t a = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char *)p;
    asm volatile("" : "+v"(a));
    return a;
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
// The bf16 pairs (-1, 0) and (0, -1), in scalar registers the compiler cannot
// see into: folded, this compiler encodes (-1, 0) as the inline constant -1.0,
// which the bf16 dot product reads as the 32-bit pattern 0xbf800000, i.e. (0, -1).
struct NegSel {
    uint32_t lo, hi;
};
__device__ __forceinline__ NegSel neg_sel() {
    NegSel m{0x0000bf80u, 0xbf800000u};
    asm volatile("" : "+s"(m.lo));
    asm volatile("" : "+s"(m.hi));
    return m;
}
// x - (element 0 or 1 of the bf16 pair h, by m = neg_sel's lo or hi), in one
// instruction (a bf16 dot product with an fp32 addend: the product is exact, so
// the only rounding is the sum's, and none when h is x rounded to bf16)
__device__ __forceinline__ float minus_bf16(uint32_t h, uint32_t m, float x) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, h), __builtin_bit_cast(bf16x2v, m), x, false);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 lds_ld2(uint32_t a) { return *(const __attribute__((address_space(3))) u32x2 *)(uintptr_t)a; }
__device__ __forceinline__ f32x2 lds_ldf2(uint32_t a) { return *(const __attribute__((address_space(3))) f32x2 *)(uintptr_t)a; }
__device__ __forceinline__ void lds_st2(uint32_t a, uint32_t x, uint32_t y) {
    *(__attribute__((address_space(3))) u32x2 *)(uintptr_t)a = u32x2{x, y};
}
__device__ __forceinline__ void lds_st16(uint32_t a, uint16_t x) { *(__attribute__((address_space(3))) uint16_t *)(uintptr_t)a = x; }
__device__ __forceinline__ s16x4 lds_ld_tr4(uint32_t a) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(uintptr_t)a);
}

__device__ __forceinline__ bf16x8 ld_frag(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ void st_frag(char *p, bf16x8 x) { *reinterpret_cast<bf16x8 *>(p) = x; }

constexpr float L2E = 1.4426950408889634f, LN2 = 0.6931471805599453f;
constexpr float GATE_FLOOR = -5.f;   // lower bound l of the safe gate's log-retention
constexpr float NORM_EPS = 1e-6f;    // x / max(||x||, eps)

// log2 of the safe gate's retention (EDA paper Eqs. (14)-(15)):
//   Delta = softplus(a + b),  g = l + (-l) exp(-(A / |l|) Delta),  log2 alpha = g log2 e,
// with Ap = (A / |l|) log2 e precomputed per channel; softplus(x) = max(x, 0) + ln(1 + e^-|x|).
__device__ __forceinline__ float safe_gate_log2(float a, float Ap, float b) {
    const float x = a + b;
    const float sp = fmaxf(x, 0.f) + LN2 * __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(-fabsf(x) * L2E));
    return -GATE_FLOOR * L2E * (__builtin_amdgcn_exp2f(-Ap * sp) - 1.f);
}

// Exchanges between the four 16-lane rows of a wave (gfx950 lane permutes),
// for x holding x0 .. x3 in rows 0 .. 3:
//   row_swap16(x) = {[x0 x0 x2 x2], [x1 x1 x3 x3]},
//   row_swap32(x) = {[x0 x1 x0 x1], [x2 x3 x2 x3]}.
__device__ __forceinline__ float2 row_swap16(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto p = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return make_float2(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float2 row_swap32(float x) {
    const uint32_t u = __builtin_bit_cast(uint32_t, x);
    const auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return make_float2(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}

// Value of lane S of each group of four lanes (DPP quad permutation).
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x55 * S, 0xf, 0xf, false));
}

// ---------------------------------------------------------------------------
// Workspace block of one chunk and head (byte offsets; fragments as above).
// Every factor is in natural units (the split scale e^r folded back in).
// ---------------------------------------------------------------------------
template <int C, int D>
struct Fac {
    static constexpr int L = 2 * C, NBL = L / 16, NBC = C / 16, NBD = D / 16;
    static constexpr int KSD = D / 32, KSC = (C + 31) / 32;   // k-steps over channels, over tokens
    static constexpr int FR = 1024;                            // one fragment
    static constexpr int oPhi = 0;                             // Phi  [NBD][KSD]  (rows, k: key channels)
    static constexpr int oPsi = oPhi + NBD * KSD * FR;         // Psi  [NBD][KSC]  (rows: channels, k: tokens; zero-padded)
    static constexpr int oQh = oPsi + NBD * KSC * FR;          // Qhat [NBC][KSD]  (rows: tokens, k: channels)
    static constexpr int oPh = oQh + NBC * KSD * FR;           // Phat [NBC][KSC]  (rows, k: tokens; zero-padded)
    static constexpr int oDec = oPh + NBC * KSC * FR;          // e^{G_C} [D] fp32
    static constexpr int bytes = align256(oDec + D * 4);
    static_assert(C == 16 || C == 32 || C == 64, "chunk");
    static_assert(D % 32 == 0 && D <= 128, "head dim");
};

// ---------------------------------------------------------------------------
// Kernel 1: chunk factors.  Persistent: workgroup w takes items w, w + grid,
// ...; item i is chunk NC - 1 - i / BH of head i % BH (last chunks first, so
// the earliest chunks, which the state pass reads first, were written last).
// ---------------------------------------------------------------------------
template <int C, int D>
struct K1G {
    using F = Fac<C, D>;
    static constexpr int L = 2 * C, NB = L / 16, NBC = C / 16, NBD = D / 16;
    // 64-token chunks: one 8-wave workgroup per compute unit (LDS); smaller
    // chunks: 4-wave workgroups, two per compute unit
    static constexpr int NW = C == 64 ? 8 : 4, NT = 64 * NW;
    static constexpr int LDA = D + 8, LDL = L + 8, ADS = 20, MTW = 24;
    // Decay scan and operand formation: lane (r, o) of wave w owns channels
    // 8 o .. 8 o + 7 of tokens w TPW + i TI + r (i < NI, r < RA).
    static constexpr int NO = D / 8;                   // 16-byte channel pieces per token row
    static constexpr int TI = 64 / NO;                 // token rows per wave instruction
    static constexpr int TPW = C / NW;                 // tokens per wave
    static constexpr int NI = imax(1, TPW / TI);       // token rows per lane
    static constexpr int RA = imin(TI, TPW);           // row groups of a wave holding tokens
    static_assert(TPW % TI == 0 || TPW < TI, "token split");
    // four 16-lane token rows per wave instruction, all holding tokens: the scan
    // moves between rows by lane permutes
    static constexpr bool ROWS4 = NO == 16 && RA == 4 && NW % 4 == 0;
    static_assert(NB <= NW, "one diagonal block per wave");
    static_assert(C <= 64, "beta/gamma staging by the first wave");
    // P (and later Z = P M) is stored packed: the rows of token block tb hold
    // sub-steps 0 .. 32 tb + 31 (P is zero beyond 2t + 1), row stride 32 tb + 40.
    static __host__ __device__ constexpr int pld(int tb) { return 32 * tb + 40; }
    static __host__ __device__ constexpr int poff(int tb) { return 16 * tb * (16 * tb + 24); }
    static constexpr int PSZ = poff(NBC);
    // LDS (bytes).  Kl holds G (fp32 [C][D]) in a wide chunk until the operands
    // are formed; Kr becomes Yhat = M^T Khat and P's high part becomes Z = P M;
    // the off-diagonal blocks of A are stored in the upper blocks of the L x L
    // region, block (J, I) at (I, J), which before the operands exist holds the
    // per-wave decay totals of the scan; MT holds the inverted diagonal blocks.
    static constexpr int szKl = align16(L * LDA * 2), szQl = align16(C * LDA * 2);
    static constexpr int szMI = align16(L * LDL * 2);
    static constexpr int szAd = NB * 16 * ADS * 4, szMT = NB * 16 * MTW * 2;
    static constexpr int szP = align16(PSZ * 2);
    static_assert(C * D * 4 <= szKl, "G in the Kl region");
    static_assert(NW * D * 4 <= szMI, "per-wave decay totals in the L x L region");
    static constexpr int oKl = 0, oKr = oKl + szKl, oQl = oKr + szKl, oMI = oQl + szQl;
    static constexpr int oAd = oMI + szMI, oMT = oAd + szAd, oPh = oMT + szMT, oPl = oPh + szP;
    static constexpr int oMisc = oPl + szP;
    static constexpr int LDS = oMisc + (L + 2 * C + D) * 4;
    static_assert(LDS <= (NW == 8 ? 160 : 80) * 1024, "LDS budget");
    // phase 4/5 work lists
    static constexpr int NZT = NBC * (NBC + 1);         // Z tiles (tb, J <= 2 tb + 1)
    // 8 waves and 128 channels: Phi as four 4 x 4-tile blocks on waves 0..3, Qhat
    // on waves 4..7 in pairs of column blocks sharing their Z fragments (fewer
    // LDS reads per product than one 2 x 4 block per wave and Qhat by column)
    static constexpr bool PQSPLIT = NW == 8 && NBD == 8;
    static constexpr int BM = PQSPLIT ? 4 : 2, BN = imin(4, NBD);   // Phi register block (tiles)
    static constexpr int NPB = (NBD / BM) * (NBD / BN); // Phi blocks
    static_assert(!PQSPLIT || NPB == 4, "Phi blocks on waves 0..3");
};

// VEC: d_k == D and 16-byte aligned q, k, e and decay input (each thread's
// 4-channel pieces move as single vector loads and are fetched one item
// ahead); otherwise, and for a ragged last chunk, the item is read
// element-wise with zero padding.
//
// LAYER: the layer prologue is fused -- `decay` holds the safe gate's input
// a (bf16, key heads) instead of alpha (fp32), A_log and dt_bias ([Hk][dk]
// fp32) give alpha per key channel, q, k, e are L2-normalised per token here,
// and the Hk key heads are shared by groups of H / Hk value heads (q, k, e, a
// per key head; beta, gamma, v per value head).  Otherwise Hk == H.
//
// DPLR: the rank-1 DPLR update S_t = (I - k_t a_t^T) Diag(alpha_t) S_{t-1} + k_t v_t^T
// (GDN-2 and QED; QED slides, frames on GDN-2's decay/erase/write split and
// on QED's erase vector) in the same sub-step form: the erase sub-step only
// decays (kap = 0, b' = 0) and the delta sub-step reads along a (the `e`
// input) and writes along k with b' = 1, so Kl's delta rows come from a and
// Kr's from k (a non-symmetric Gram); beta and gamma are not read.
constexpr int MODE_PLAIN = 0, MODE_LAYER = 1, MODE_DPLR = 2;

template <int C, int D, bool VEC, int MODE>
__global__ void __launch_bounds__((K1G<C, D>::NT)) __attribute__((amdgpu_waves_per_eu(2)))
eda_bf16_factors(const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ e,
                 const void *__restrict__ decay, const float *__restrict__ A_log,
                 const float *__restrict__ dt_bias, const float *__restrict__ beta,
                 const float *__restrict__ gamma, char *__restrict__ ws, int Tlen, int H, int Hk,
                 int dk, int NC, int BH) {
    using G = K1G<C, D>;
    using F = Fac<C, D>;
    using T = bf16;
    constexpr bool LAYER = MODE == MODE_LAYER, DPLR = MODE == MODE_DPLR;
    constexpr int L = G::L, NB = G::NB, NT = G::NT, NW = G::NW, LDA = G::LDA, LDL = G::LDL;
    constexpr int ADS = G::ADS, MTW = G::MTW, NO = G::NO, TI = G::TI, NI = G::NI, RA = G::RA;
    constexpr bool ROWS4 = G::ROWS4;
    constexpr int NBD = F::NBD, NBC = F::NBC, KSD = F::KSD, KSC = F::KSC;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Kl = (T *)(smem + G::oKl);            // Diag(b') Kl              [L][LDA]
    float *Gs = (float *)(smem + G::oKl);    // wide chunk: G (log2) [C][D]
    T *Kr = (T *)(smem + G::oKr);            // Kr, then Y = M^T Khat    [L][LDA]
    T *Ql = (T *)(smem + G::oQl);            // Ql                       [C][LDA]
    T *MI = (T *)(smem + G::oMI);            // A's off-diagonal blocks, block (J, I) stored at (I, J) [L][LDL]
    float *AdT = (float *)(smem + G::oAd);   // A, diagonal 16-blocks, transposed: [J][p][i] = A_J[i][p]
    T *MT = (T *)(smem + G::oMT);            // diagonal blocks of M = (I + A)^{-1}, transposed [NB][16][MTW]
    T *Zs = (T *)(smem + G::oPh);            // Z = P M (packed like P), over P's high part
    T *Ph = (T *)(smem + G::oPh);            // P, high bf16 part (packed)
    T *Pl = (T *)(smem + G::oPl);            // P, low bf16 part (packed)
    float *bp = (float *)(smem + G::oMisc);  // b' per sub-step          [L]
    float *sb = bp + L, *sg = sb + C;        // beta, gamma per token    [C]
    float *ers = sg + C;                     // e^r per channel (1 if wide) [D]
    float *wtot = (float *)(smem + G::oMI);  // per-wave decay totals of the scan [NW][D]

    const int tid = threadIdx.x, lane = tid & 63;
    int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int grp = H / Hk;                  // value heads per key head
    const float *alpha = (const float *)decay;
    const bf16 *agate = (const bf16 *)decay;
    const int items = BH * NC;

    auto chunk_of = [&](int it) __attribute__((always_inline)) { return NC - 1 - it / BH; };
    auto head_of = [&](int it) __attribute__((always_inline)) { return it % BH; };
    auto is_fast = [&](int cidx) __attribute__((always_inline)) { return VEC && cidx * C + C <= Tlen; };

    // Lane (r, o) of wave w owns key channels c0 .. c0 + 7 (c0 = 8 o) of tokens
    // w TPW + i TI + r, i < NI: each wave instruction moves TI whole token rows,
    // and the operand stores are 16-byte row pieces (consecutive lanes, no LDS
    // bank conflicts).  Its raw q, e, k (bf16) and alpha (fp32) stay in registers.
    const int o = lane % NO, r = lane / NO;
    const bool act = r < RA;                 // lanes holding tokens
    const int c0 = 8 * o;
    auto tok = [&](int i) __attribute__((always_inline)) { return wave * G::TPW + i * TI + r; };
    uint4 xq[NI], xe[NI], xk[NI];
    f32x4 xa[NI][2];         // alpha of the 8 channels
    uint4 xg[NI];            // LAYER: the gate input a (8 bf16)
    f32x4 xA[2], xB[2];      // LAYER: A_log, dt_bias of the 8 channels
    float pbeta = 0.f, pgamma = 0.f;

    // ---- full aligned chunk: fetched one item ahead.  Rows are clamped to the
    //      sequence so the same loads are issued for every item and the only
    //      wait on them is where they are first used. -----------------------------
    auto prefetch_at = [&](int it, auto part) __attribute__((always_inline)) {
        // part 1: the decay input (alpha, or the layer form's gate input and
        // parameters), consumed by the scan; part 2: q, e, k and the gates,
        // consumed by the formation; 3: both
        constexpr int PART = decltype(part)::value;
        const int bh = head_of(it), cidx = chunk_of(it);
        const int b = bh / H, h = bh % H;
        const int t0 = cidx * C, last = Tlen - 1 - t0, hk = h / grp;
        const long tok0 = ((long)b * Tlen + t0) * H + h;       // value-head rows
        const long tokk0 = ((long)b * Tlen + t0) * Hk + hk;    // key-head rows
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const long off = (tokk0 + (long)min(tok(i), last) * Hk) * dk + c0;
            if constexpr (PART & 2) {
                xq[i] = *(const uint4 *)(q + off);
                xe[i] = *(const uint4 *)(e + off);
                xk[i] = *(const uint4 *)(k + off);
            }
            if constexpr (PART & 1) {
                if constexpr (LAYER) {
                    xg[i] = *(const uint4 *)(agate + off);
                } else {
                    xa[i][0] = *(const f32x4 *)(alpha + off);
                    xa[i][1] = *(const f32x4 *)(alpha + off + 4);
                }
            }
        }
        if constexpr (LAYER && (PART & 1)) {
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                xA[hh] = *(const f32x4 *)(A_log + (long)hk * dk + c0 + 4 * hh);
                xB[hh] = *(const f32x4 *)(dt_bias + (long)hk * dk + c0 + 4 * hh);
            }
        }
        if constexpr (PART & 2) {
            const long tb = tok0 + (long)min(tid % C, last) * H;
            pbeta = DPLR ? 1.f : beta[tb];
            pgamma = DPLR ? 0.f : gamma[tb];
        }
    };
    auto prefetch = [&](int it) __attribute__((always_inline)) { prefetch_at(it, std::integral_constant<int, 3>{}); };
    // the next item of this workgroup (clamped: the last item refetches itself)
    auto next_item = [&](int it) __attribute__((always_inline)) {
        const int nx = it + gridDim.x;
        return nx < items ? nx : items - 1;
    };
    // ---- ragged or unaligned chunk: element-wise, zero keys and queries and
    //      alpha = 1 outside the sequence and beyond d_k -----------------------------
    auto fetch_slow = [&](int it) __attribute__((always_inline)) {
        const int bh = head_of(it), cidx = chunk_of(it);
        const int b = bh / H, h = bh % H;
        const int t0 = cidx * C, nval = min(C, Tlen - t0), hk = h / grp;
        const long tok0 = ((long)b * Tlen + t0) * H + h;
        const long tokk0 = ((long)b * Tlen + t0) * Hk + hk;
        auto pack8 = [](const float *x) __attribute__((always_inline)) {
            return make_uint4(pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]),
                              pack_bf16(x[6], x[7]));
        };
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            const int tau = tok(i);
            float qv[8], ev[8], kv[8], av[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool ok = act && tau < nval && c0 + j < dk;
                const long off = (tokk0 + (long)tau * Hk) * dk + c0 + j;
                qv[j] = ok ? to_f32(q[off]) : 0.f;
                ev[j] = ok ? to_f32(e[off]) : 0.f;
                kv[j] = ok ? to_f32(k[off]) : 0.f;
                // (LAYER: a = -inf gives softplus = 0, i.e. alpha = 1, for padding)
                if constexpr (LAYER) av[j] = ok ? to_f32(agate[off]) : -INFINITY;
                else av[j] = ok ? alpha[off] : 1.f;
            }
            // (exact: the values are bf16 already)
            xq[i] = pack8(qv);
            xe[i] = pack8(ev);
            xk[i] = pack8(kv);
            if constexpr (LAYER) {
                xg[i] = pack8(av);
            } else {
                xa[i][0] = f32x4{av[0], av[1], av[2], av[3]};
                xa[i][1] = f32x4{av[4], av[5], av[6], av[7]};
            }
        }
        if constexpr (LAYER) {
            float pa[8], pb[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const bool ok = act && c0 + j < dk;
                pa[j] = ok ? A_log[(long)hk * dk + c0 + j] : 0.f;
                pb[j] = ok ? dt_bias[(long)hk * dk + c0 + j] : 0.f;
            }
            xA[0] = f32x4{pa[0], pa[1], pa[2], pa[3]};
            xA[1] = f32x4{pa[4], pa[5], pa[6], pa[7]};
            xB[0] = f32x4{pb[0], pb[1], pb[2], pb[3]};
            xB[1] = f32x4{pb[4], pb[5], pb[6], pb[7]};
        }
        const bool okt = tid < nval;
        pbeta = okt ? (DPLR ? 1.f : beta[tok0 + (long)tid * H]) : 0.f;
        pgamma = okt && !DPLR ? gamma[tok0 + (long)tid * H] : 0.f;
        // Drain these loads here (vmcnt(0)): they fill the registers the fast
        // path prefetches, and the waits where both paths meet would otherwise
        // be counted for this path's short tail of loads, which on the fast path
        // also waits for the previous item's workspace stores.
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_sched_barrier(0);
    };

    // ---- diagonal 16x16 blocks of (I + A)^{-1}: fp32 forward substitution over
    //      the whole wave.  Lane 4 col + s holds rows 4 s .. 4 s + 3 of solution
    //      column col; at step p every row below p takes -A[i][p] x[p], with x[p]
    //      broadcast inside the lane quad (rows on or above p see A = 0).
    auto invert_diag = [&](int J) __attribute__((always_inline)) {
        const int ln = lane_ids(tid).lane;
        const int col = ln >> 2, s4 = 4 * (ln & 3);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (s4 + i == col) ? 1.f : 0.f;
        // the block's columns (A[s4 + i][p]) are read RD steps ahead of the
        // serial steps that use them
        constexpr int RD = 6;
        f32x4 ac[15];
        auto acol = [&](int p) __attribute__((always_inline)) { return *(const f32x4 *)(AdT + (J * 16 + p) * ADS + s4); };
#pragma unroll
        for (int p = 0; p < RD; ++p) ac[p] = acol(p);
#pragma unroll
        for (int p = 0; p < 15; ++p) {
            if (p + RD < 15) ac[p + RD] = acol(p + RD);
            __builtin_amdgcn_sched_barrier(0);
            const f32x4 a = ac[p];
            const float xs = x[p & 3];
            const float xp = (p >> 2) == 0 ? quad_bcast<0>(xs) : (p >> 2) == 1 ? quad_bcast<1>(xs)
                           : (p >> 2) == 2 ? quad_bcast<2>(xs) : quad_bcast<3>(xs);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] -= a[i] * xp;
        }
        // stored negated: the substitution then yields -X, which the bracket
        // updates take as they are (the consumers of -X absorb its sign)
        const uint32_t x01 = pack_bf16(-x[0], -x[1]), x23 = pack_bf16(-x[2], -x[3]);
        *(uint2 *)(MT + (16 * J + col) * MTW + s4) = make_uint2(x01, x23);
    };

    // P tile value -> P_hi, P_lo at row tau (packed), sub-steps i0 .. i0 + 3
    auto store_p = [&](int tau, int i0, float a0, float a1, float a2, float a3) __attribute__((always_inline)) {
        const int tb = tau >> 4;
        const int off = G::poff(tb) + (tau & 15) * G::pld(tb) + i0;
        const uint32_t h01 = pack_bf16(a0, a1), h23 = pack_bf16(a2, a3);
        *(uint2 *)(Ph + off) = make_uint2(h01, h23);
        *(uint2 *)(Pl + off) = make_uint2(pack_bf16(a0 - lo_bf16(h01), a1 - hi_bf16(h01)),
                                          pack_bf16(a2 - lo_bf16(h23), a3 - hi_bf16(h23)));
    };

    int it = blockIdx.x;
    if constexpr (VEC) {
        prefetch(it);
        // The first item's inputs are consumed (unused) right here, so the
        // compiler waits for them once, before the item loop.  The waits at the
        // top of the loop are then counted for the loop path alone, where the
        // previous item's workspace stores follow the prefetch, and leave those
        // stores in flight instead of waiting for them as well.
#pragma unroll
        for (int i = 0; i < NI; ++i) {
            asm volatile("" ::"v"(xq[i].x), "v"(xq[i].y), "v"(xq[i].z), "v"(xq[i].w), "v"(xe[i].x), "v"(xe[i].y),
                         "v"(xe[i].z), "v"(xe[i].w), "v"(xk[i].x), "v"(xk[i].y), "v"(xk[i].z), "v"(xk[i].w));
            if constexpr (LAYER)
                asm volatile("" ::"v"(xg[i].x), "v"(xg[i].y), "v"(xg[i].z), "v"(xg[i].w));
            else
                asm volatile("" ::"v"(xa[i][0][0]), "v"(xa[i][0][1]), "v"(xa[i][0][2]), "v"(xa[i][0][3]),
                             "v"(xa[i][1][0]), "v"(xa[i][1][1]), "v"(xa[i][1][2]), "v"(xa[i][1][3]));
        }
        asm volatile("" ::"v"(pbeta), "v"(pgamma));
        if constexpr (LAYER)
            asm volatile("" ::"v"(xA[0][0]), "v"(xA[0][1]), "v"(xA[0][2]), "v"(xA[0][3]), "v"(xA[1][0]),
                         "v"(xA[1][1]), "v"(xA[1][2]), "v"(xA[1][3]), "v"(xB[0][0]), "v"(xB[0][1]), "v"(xB[0][2]),
                         "v"(xB[0][3]), "v"(xB[1][0]), "v"(xB[1][1]), "v"(xB[1][2]), "v"(xB[1][3]));
    }
    for (; it < items; it += gridDim.x) {
        // Waves w and w + NW/2 share a SIMD and the arbiter favours the older one.
        // In the Phi/Qhat phase the second half carries the paired Qhat blocks, so
        // it runs at raised issue priority there; every other phase runs level
        // (raising either half in the scan or in the substitution did not pay).
        if constexpr (NW == 8) __builtin_amdgcn_s_setprio(0);
        // (layer form: the wave index made opaque again, so that nothing derived
        // from it is hoisted out of the item loop into spilled scalar registers;
        // in the other modes the hoisted values pay)
        if constexpr (LAYER) asm volatile("" : "+s"(wave));
        const int bh = head_of(it), cidx = chunk_of(it);
        if (!is_fast(cidx)) fetch_slow(it);
        // (nothing read after this item's last barrier uses bp, sb or sg)
        if (tid < C) {
            sb[tid] = pbeta;
            sg[tid] = pgamma;
            bp[2 * tid] = pgamma;
            bp[2 * tid + 1] = pbeta;
        }
        char *wsb = ws + ((long)bh * NC + cidx) * F::bytes;

        // ---- cumulative log2-decay per channel: an inclusive scan over the RA row
        //      groups of the wave (lanes NO apart) for each of the lane's token rows,
        //      carried across its rows; then the waves' totals through LDS --------------
        float g[NI][8];
        float glq[8];
        {
            f32x4 Ap[2];
            if constexpr (LAYER) {
#pragma unroll
                for (int hh = 0; hh < 2; ++hh)
#pragma unroll
                    for (int j = 0; j < 4; ++j) Ap[hh][j] = exp2f_(xA[hh][j] * L2E) * (L2E / -GATE_FLOOR);
            }
            float carry[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) carry[j] = -0.f;   // (x + -0 is x exactly: the first add folds away)
            const float rb1 = (r & 1) ? 1.f : 0.f, rb2 = (r & 2) ? 1.f : 0.f;
#pragma unroll
            for (int i = 0; i < NI; ++i)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float x;
                    if constexpr (LAYER) {
                        const uint32_t u = j < 2 ? xg[i].x : j < 4 ? xg[i].y : j < 6 ? xg[i].z : xg[i].w;
                        x = safe_gate_log2((j & 1) ? hi_bf16(u) : lo_bf16(u), Ap[j >> 2][j & 3], xB[j >> 2][j & 3]);
                    } else {
                        x = __builtin_amdgcn_logf(xa[i][j >> 2][j & 3]);
                    }
                    if constexpr (ROWS4) {
                        // rows 2 k + 1 add row 2 k; rows 2, 3 add the pair total of rows 0, 1
                        // (a = (row 2 k, row 2 k + 1) of the lane's pair, so a.x is x itself
                        // in an even row; the selections are products with the lane's 0/1
                        // row bits, exact, so no select and no copy of x is needed)
                        const float2 a = row_swap16(x);
                        const float pt = a.x + a.y;
                        const float sx = __builtin_fmaf(rb1, a.y, a.x);
                        const float2 b = row_swap32(pt);
                        g[i][j] = carry[j] + __builtin_fmaf(rb2, b.x, sx);
                        carry[j] += b.x + b.y;
                    } else {
#pragma unroll
                        for (int sh = 1; sh < RA; sh <<= 1) {
                            const float y = __shfl_up(x, sh * NO, 64);
                            if (r >= sh) x += y;
                        }
                        g[i][j] = carry[j] + x;
                        carry[j] += __shfl(x, (RA - 1) * NO + o, 64);
                    }
                }
            // the decay input is consumed: the next item's is fetched now
            if constexpr (VEC) prefetch_at(next_item(it), std::integral_constant<int, 1>{});
            if (r == 0) {
                *(f32x4 *)(wtot + wave * D + c0) = f32x4{carry[0], carry[1], carry[2], carry[3]};
                *(f32x4 *)(wtot + wave * D + c0 + 4) = f32x4{carry[4], carry[5], carry[6], carry[7]};
            }
        }
        __syncthreads();
        bool wide_here = false;
        {
            // running sums over the waves in order: the wave's prefix is the sum
            // before its own term, and the total (the same in every wave) the last
            float pre[8], tot[8];
            int wv = wave;   // (opaque: the eight comparisons below stay in the item)
            asm volatile("" : "+s"(wv));
#pragma unroll
            for (int j = 0; j < 8; ++j) pre[j] = tot[j] = -0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const f32x4 a = *(const f32x4 *)(wtot + w * D + c0), b = *(const f32x4 *)(wtot + w * D + c0 + 4);
                if (w == wv) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) pre[j] = tot[j];
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    tot[j] += a[j];
                    tot[4 + j] += b[j];
                }
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                glq[j] = tot[j];   // G_C of the channel
#pragma unroll
                for (int i = 0; i < NI; ++i) g[i][j] += pre[j];
                wide_here |= act && tot[j] < -WIDE_G2;
            }
        }
        // wide chunk: every wave sums the same totals in the same order, and its lanes
        // cover every channel, so a ballot gives each wave the same decision with no
        // barrier (the totals' region is next written after the formation barrier)
        const bool wide = __ballot(wide_here) != 0ull;

        // LAYER: (1/|q|, 1/|k|, 1/|e|) of token row i, reduced over the NO lanes of
        // the row (x / max(|x|, eps))
        auto inv_norms = [&](int i) __attribute__((always_inline)) {
            f32x4 res = zero4();
            if constexpr (LAYER) {
                const uint4 *src[3] = {&xq[i], &xk[i], &xe[i]};
#pragma unroll
                for (int v = 0; v < 3; ++v) {
                    const uint4 u = *src[v];
                    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
                    float sq = 0.f;
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const float a = lo_bf16(w4[m]), b = hi_bf16(w4[m]);
                        sq += a * a + b * b;
                    }
#pragma unroll
                    for (int m = 1; m < NO; m <<= 1) sq += __shfl_xor(sq, m, 64);
                    res[v] = sq > NORM_EPS * NORM_EPS ? __builtin_amdgcn_rsqf(sq) : 1.f / NORM_EPS;
                }
            }
            return res;
        };
        auto unpack8 = [](uint4 u, float *x, float sc) __attribute__((always_inline)) {
            const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                x[2 * m] = lo_bf16(w4[m]) * sc;
                x[2 * m + 1] = hi_bf16(w4[m]) * sc;
            }
        };
        auto store8 = [](T *p, const float *x, float sc, const float *f) __attribute__((always_inline)) {
            *(uint4 *)p = make_uint4(pack_bf16(sc * x[0] * f[0], sc * x[1] * f[1]), pack_bf16(sc * x[2] * f[2], sc * x[3] * f[3]),
                                     pack_bf16(sc * x[4] * f[4], sc * x[5] * f[5]), pack_bf16(sc * x[6] * f[6], sc * x[7] * f[7]));
        };

        // ---- scaled operands (LDS) and the per-channel scales ----------------------
        // Forms Diag(b') Kl, Kr and Ql from the lane's raw values; in a wide chunk the
        // exponents are unsplit (Kl = lam 2^G, Kr = kap 2^{G_C - G}).
        float er[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) er[j] = wide ? 1.f : exp2f_(0.5f * glq[j]);
        auto form_operands = [&]() __attribute__((always_inline)) {
            float rr[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) rr[j] = wide ? 0.f : 0.5f * glq[j];
#pragma unroll
            for (int i = 0; i < NI; ++i) {
                const int tau = tok(i);
                const f32x4 nv = LAYER ? inv_norms(i) : f32x4{1.f, 1.f, 1.f, 0.f};
                float ev[8], kv[8], qv[8];
                unpack8(xe[i], ev, nv[2]);
                unpack8(xk[i], kv, nv[1]);
                unpack8(xq[i], qv, nv[0]);
                const float gmt = sg[tau], btt = sb[tau];
                float f[8], fi[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const float d = g[i][j] - rr[j];   // (rr - g = -d exactly)
                    f[j] = exp2f_(d);
                    fi[j] = wide ? exp2f_(glq[j] - g[i][j]) : exp2f_(-d);
                }
                store8(Kl + (2 * tau) * LDA + c0, ev, gmt, f);
                // (DPLR: the delta sub-step reads along a, held in ev; its erase sub-step has no key)
                store8(Kl + (2 * tau + 1) * LDA + c0, DPLR ? ev : kv, btt, f);
                if constexpr (DPLR)
                    *(uint4 *)(Kr + (2 * tau) * LDA + c0) = make_uint4(0u, 0u, 0u, 0u);
                else
                    store8(Kr + (2 * tau) * LDA + c0, ev, 1.f, fi);
                store8(Kr + (2 * tau + 1) * LDA + c0, kv, 1.f, fi);
                store8(Ql + tau * LDA + c0, qv, 1.f, f);
            }
        };
        if (act) {
            if (wave == 0 && r == 0) {
                float dec[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) dec[j] = exp2f_(glq[j]);
                *(f32x4 *)(ers + c0) = f32x4{er[0], er[1], er[2], er[3]};
                *(f32x4 *)(ers + c0 + 4) = f32x4{er[4], er[5], er[6], er[7]};
                *(f32x4 *)(wsb + F::oDec + 4 * c0) = f32x4{dec[0], dec[1], dec[2], dec[3]};
                *(f32x4 *)(wsb + F::oDec + 4 * c0 + 16) = f32x4{dec[4], dec[5], dec[6], dec[7]};
            }
            if (!wide) {
                form_operands();
            } else {
                // raw keys and queries (normalised in the layer form), and G, for the
                // element-wise path
#pragma unroll
                for (int i = 0; i < NI; ++i) {
                    const int tau = tok(i);
                    const f32x4 nv = LAYER ? inv_norms(i) : f32x4{1.f, 1.f, 1.f, 0.f};
                    float ev[8], kv[8], qv[8];
                    const float one[8] = {1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f, 1.f};
                    unpack8(xe[i], ev, nv[2]);
                    unpack8(xk[i], kv, nv[1]);
                    unpack8(xq[i], qv, nv[0]);
                    store8(Kr + (2 * tau) * LDA + c0, ev, 1.f, one);
                    store8(Kr + (2 * tau + 1) * LDA + c0, kv, 1.f, one);
                    store8(Ql + tau * LDA + c0, qv, 1.f, one);
                    *(f32x4 *)(Gs + tau * D + c0) = f32x4{g[i][0], g[i][1], g[i][2], g[i][3]};
                    *(f32x4 *)(Gs + tau * D + c0 + 4) = f32x4{g[i][4], g[i][5], g[i][6], g[i][7]};
                }
            }
        }
        __syncthreads();

        // ---- A (strictly lower) and P (causal, as a bf16 pair); diagonal blocks
        //      of A inverted ------------------------------------------------------------
        constexpr int NOD = NB * (NB - 1) / 2;
        constexpr int NPV = NBC * (NBC + 1);   // P tiles (I, Tb) with rows i < 32 Tb + 32
        static_assert(NB == 2 * NBC, "two sub-step blocks per token block");
        if (!wide) {
            if (wave < NB) {
                const int J = wave;
                const auto [lane, g4, l16, gq] = lane_ids(tid);
                // both operands read as one group before the products
                constexpr int NKS = D / 32;
                bf16x8 xl[NKS], xr[NKS];
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) {
                    xl[ks] = *(const bf16x8 *)(Kl + (16 * J + l16) * LDA + 32 * ks + 8 * gq);
                    xr[ks] = *(const bf16x8 *)(Kr + (16 * J + l16) * LDA + 32 * ks + 8 * gq);
                }
                __builtin_amdgcn_sched_barrier(0);
                f32x4 a = zero4();
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks) a = mma32(xl[ks], xr[ks], a);
                // lane holds A[g4 + rr][l16]: one column run of the transposed block
                *(f32x4 *)(AdT + (J * 16 + l16) * ADS + g4) =
                    f32x4{g4 > l16 ? a[0] : 0.f, g4 + 1 > l16 ? a[1] : 0.f, g4 + 2 > l16 ? a[2] : 0.f,
                          g4 + 3 > l16 ? a[3] : 0.f};
                wave_lds_sync();
                invert_diag(J);
            }
            // off-diagonal A and P tiles, listed by the Kr row block I they share:
            // A tiles (J, I) for J > I, then P^T tiles (I, Tb) for the token blocks
            // Tb >= I / 2 whose stored rows reach block I.  Each wave takes a
            // contiguous run of the list and keeps Kr_I's fragments while I stays,
            // so a tile reads one operand from LDS instead of two.
            {
                const auto [lane, g4, l16, gq] = lane_ids(tid);
                constexpr int NKS = D / 32;
                constexpr int PER = (NOD + NPV + NW - 1) / NW;
                // with 8 waves, waves w and w + 4 share a SIMD; the first half, which
                // carries the paired substitution chains and Phi after this phase,
                // takes two tiles fewer and the second half two more (measured: even
                // shares, or one more tile on the first half, were 1-2 % slower)
                constexpr int SK = (NW == 8 && PER > 2) ? -2 : 0;
                auto count = [](int I) { return NB - 1 - I + NBC - I / 2; };
                const int tbeg = wave < NW / 2 ? wave * (PER + SK) : (NW / 2) * (PER + SK) + (wave - NW / 2) * (PER - SK);
                const int tend = imin(NOD + NPV, tbeg + (wave < NW / 2 ? PER + SK : PER - SK));
                int I = 0, r = tbeg;
                while (I < NB && r >= count(I)) { r -= count(I); ++I; }
                bf16x8 kr[NKS];
                int Ihave = -1;
                for (int t = tbeg; t < tend; ++t) {
                    if (I != Ihave) {
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) kr[ks] = *(const bf16x8 *)(Kr + (16 * I + l16) * LDA + 32 * ks + 8 * gq);
                        Ihave = I;
                    }
                    const int na = NB - 1 - I;
                    f32x4 a = zero4();
                    // the tile's other operand is read as one group before its
                    // products (left to the scheduler, each read sinks to its
                    // product and the tile pays one LDS round trip per k-step)
                    bf16x8 ot[NKS];
                    if (r < na) {
                        const int J = I + 1 + r;
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) ot[ks] = *(const bf16x8 *)(Kl + (16 * J + l16) * LDA + 32 * ks + 8 * gq);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) a = mma32(kr[ks], ot[ks], a);
                        // the tile transposed: lane holds A[16 J + l16][16 I + g4 + rr], which
                        // block (I, J) of M's storage keeps at row l16, columns g4 + rr (one
                        // 8-byte store)
                        *(uint2 *)(MI + (16 * I + l16) * LDL + 16 * J + g4) =
                            make_uint2(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]));
                    } else {
                        // P^T tile: rows = sub-steps i, cols = tokens; kept for i <= 2 tau + 1
                        const int Tb = I / 2 + (r - na);
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) ot[ks] = *(const bf16x8 *)(Ql + (16 * Tb + l16) * LDA + 32 * ks + 8 * gq);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int ks = 0; ks < NKS; ++ks) a = mma32(kr[ks], ot[ks], a);
                        const int tau = 16 * Tb + l16, i0 = 16 * I + g4;
                        float w4[4];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) w4[rr] = (i0 + rr <= 2 * tau + 1) ? a[rr] : 0.f;
                        store_p(tau, i0, w4[0], w4[1], w4[2], w4[3]);
                    }
                    if (++r == count(I)) {
                        r = 0;
                        ++I;
                    }
                }
            }
        } else {
            // exact element-wise path: e^{G_j - G_i} is never split (Kr, Ql hold raw keys)
            for (int idx = tid; idx < L * L; idx += NT) {
                const int j = idx / L, ii = idx % L;
                float s = 0.f;
                // (DPLR: only delta rows and columns; row j reads along a, held in row j - 1)
                if (ii < j && (!DPLR || ((j & 1) && (ii & 1)))) {
                    const int tj = j >> 1, ti = ii >> 1, jr = DPLR ? j - 1 : j;
#pragma unroll 2
                    for (int cc = 0; cc < D; ++cc)
                        s += to_f32(Kr[jr * LDA + cc]) * to_f32(Kr[ii * LDA + cc]) *
                             exp2f_(Gs[tj * D + cc] - Gs[ti * D + cc]);
                    s *= bp[j];
                }
                if ((j >> 4) == (ii >> 4)) AdT[((j >> 4) * 16 + (ii & 15)) * ADS + (j & 15)] = s;
                else if (ii < j) MI[(16 * (ii >> 4) + (j & 15)) * LDL + 16 * (j >> 4) + (ii & 15)] = from_f32<T>(s);
            }
            for (int idx = tid; idx < C * L; idx += NT) {
                const int tau = idx / L, ii = idx % L;
                if (ii >= 32 * (tau >> 4) + 32 || (ii & 3)) continue;   // four sub-steps per thread, stored rows only
                float s4[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = ii + u;
                    float s = 0.f;
                    if (i <= 2 * tau + 1 && (!DPLR || (i & 1))) {
                        const int ti = i >> 1;
#pragma unroll 2
                        for (int cc = 0; cc < D; ++cc)
                            s += to_f32(Ql[tau * LDA + cc]) * to_f32(Kr[i * LDA + cc]) *
                                 exp2f_(Gs[tau * D + cc] - Gs[ti * D + cc]);
                    }
                    s4[u] = s;
                }
                store_p(tau, ii, s4[0], s4[1], s4[2], s4[3]);
            }
            __syncthreads();
            if (wave < NB) invert_diag(wave);
            // every read of G and of the raw keys is done: form the operands in place
            if (act) form_operands();
        }
        // the raw keys and queries are consumed: the next item's are fetched now,
        // before the barrier, so waves with fewer tiles issue them while the others
        // finish (the decay input was fetched after the scan; spread out this way,
        // the fetches stall less on the memory system)
        if constexpr (VEC) prefetch_at(next_item(it), std::integral_constant<int, 2>{});
        __syncthreads();

        // ---- Y = M^T Khat and Z^T = M^T P^T, M = (I + A)^{-1}, by block backward
        //      substitution: (I + A)^T X = R for the right-hand sides R = [Khat | P^T],
        //      one 16-column block of R per wave, with no barrier:
        //          X_K = M_KK^T (R_K - sum_{J > K} A_JK^T X_J),   K = NB-1 .. 0.
        //      The solved blocks feed the later steps as bf16; the bracket enters the
        //      diagonal-inverse product as a bf16 pair.  The diagonal inverses are stored
        //      negated, so each step yields -X_K, which the bracket updates add as it is;
        //      -Y overwrites Kr and -Z overwrites P's high part, in place (each column
        //      block belongs to one wave, and each row block of it is read before it is
        //      written).  From the fp32 results:
        //      Psi = Yhat[delta rows]^T Diag(beta), Phat = Z[:, delta cols] Diag(beta).
        //      Every product here is the 16x16x16 instruction.  (Yhat = Y Diag(e^r) =
        //      M^T Khat is kept, bounded by |M|: Y^T Kl would otherwise reach e^{|G_C|},
        //      past the fp32 range, for channels decaying by more than about e^-88.)
        // Column blocks ("chains": Y blocks nb < NBD, then Z blocks tb) go round-robin
        // to the waves; a wave runs its chains two at a time, interleaved step by step,
        // so one chain's latency hides behind the other's work, and both share the
        // diagonal-inverse and off-diagonal block reads of each step.  The chain kinds
        // are template arguments, so the unrolled steps hold no branch: a Z chain runs
        // every step (its bracket is zero above its last row block, so X_K = 0 there
        // exactly, and its Phat entries there are the causal zeros), and sends its
        // dead Z stores to the diagonal blocks' fp32 region, unused by now.
        auto run_chains = [&](auto kinds, int c0, int c1) __attribute__((always_inline)) {
            // kinds: bit 0 set = first chain is a Z block, bit 1 = second is, bit 2 = a pair
            constexpr int KIND = decltype(kinds)::value;
            constexpr int NCH = (KIND & 4) ? 2 : 1;
            constexpr bool KY[2] = {(KIND & 1) == 0, (KIND & 2) == 0};
            const auto [lane, g4, l16, gq] = lane_ids(tid);
            const int cbs[2] = {c0, c1};
            int nb[NCH], tb[NCH], Jtop[NCH];
            char *ex[NCH];   // this lane's Psi or Phat entries of fragment column l16, step 0
            // per-lane LDS bases; every block's address is a fixed offset from one
            uint32_t kca[NCH], kya[NCH], pha[NCH], pla[NCH];
            const int ltr = 4 * gq + (l16 >> 2), ctr = 4 * (l16 & 3);   // transposed-read lane part
            const uint32_t mia = lds_addr(MI + ltr * LDL + ctr), mta = lds_addr(MT + l16 * MTW + g4);
            const uint32_t sba = lds_addr(sb + 2 * gq), dum = lds_addr(AdT + 4 * lane);
            const NegSel ns = neg_sel();
            // the identity as the row-by-k operand: lane (gq, l16) holds row l16, k = 4 gq .. + 3
            const s16x4 eye = __builtin_bit_cast(
                s16x4, make_uint2((4 * gq == l16 ? 0x3f80u : 0u) | (4 * gq + 1 == l16 ? 0x3f800000u : 0u),
                                  (4 * gq + 2 == l16 ? 0x3f80u : 0u) | (4 * gq + 3 == l16 ? 0x3f800000u : 0u)));
            f32x4 acc[NCH][NB];
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
                const int cb = cbs[c];
                nb[c] = cb;
                tb[c] = cb - NBD;
                // token t = 8 K + 2 gq (+1) sits in k-step t / 32 = K / 4, lane slot
                // 16 ((t & 31) / 8) + l16 = 16 (K & 3) + l16, bytes 2 (t & 7) = 4 gq
                ex[c] = wsb + (KY[c] ? F::oPsi + nb[c] * KSC * 1024 : F::oPh + tb[c] * KSC * 1024) + l16 * 16 + 4 * gq;
                Jtop[c] = KY[c] ? NB - 1 : imin(NB - 1, 2 * tb[c] + 1);   // Z: P is zero below 32 tb + 32
                if (KY[c]) {
                    kca[c] = lds_addr(Kr + l16 * LDA + 16 * nb[c] + 4 * gq);
                    kya[c] = lds_addr(Kr + g4 * LDA + 16 * nb[c] + l16);
                } else {
                    const int pr = G::poff(tb[c]) + l16 * G::pld(tb[c]);  // P row of token 16 tb + l16
                    pha[c] = lds_addr(Ph + pr + g4);                      // (Z overwrites P's high part)
                    pla[c] = lds_addr(Pl + pr + g4);
                }
                // right-looking: every row block's bracket starts as R_J; once X_K is solved
                // it updates all the brackets above it at once (independent products), so
                // the chain from one solved block to the next is one update, the pair split
                // and the two diagonal-inverse products
                // the brackets start on the matrix cores: Khat's block as Kr's block times
                // Diag(e^r) (e^r as a bf16 pair, the two products exact in fp32), P^T's
                // block as the identity times P^T (its high and low parts)
                if (KY[c]) {
                    const float scale = ers[16 * nb[c] + l16];   // Khat = Kr e^r, column n
                    const uint32_t shi = pack_bf16(scale, 0.f), slo = pack_bf16(minus_bf16(shi, ns.lo, scale), 0.f);
                    // Diag(s) as the k-by-column operand: lane (gq, l16) holds rows 4 gq + i of column l16
                    uint32_t d[2][2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const uint32_t sv = h ? slo : shi;   // the value in the low half
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const int k0 = 4 * gq + 2 * q;
                            d[h][q] = (k0 == l16 ? sv : 0u) | (k0 + 1 == l16 ? sv << 16 : 0u);
                        }
                    }
                    const s16x4 dhi = __builtin_bit_cast(s16x4, make_uint2(d[0][0], d[0][1]));
                    const s16x4 dlo = __builtin_bit_cast(s16x4, make_uint2(d[1][0], d[1][1]));
#pragma unroll
                    for (int J = 0; J < NB; ++J) {
                        // Kr rows 16 J + l16, channels 16 nb + 4 gq .. + 3 (row-by-k operand)
                        const s16x4 kb = __builtin_bit_cast(s16x4, lds_ld2(kca[c] + 2 * 16 * J * LDA));
                        acc[c][J] = mma16(kb, dlo, mma16(kb, dhi, zero4()));
                    }
                } else {
                    // (rows beyond the stored part enter as zero; all the reads are
                    // issued before the first product, or each waits for its own)
                    u32x2 h[NB], l[NB];
#pragma unroll
                    for (int J = 0; J < NB; ++J) {
                        const uint32_t off = J <= Jtop[c] ? 2 * 16 * J : 0;
                        h[J] = lds_ld2(pha[c] + off);
                        l[J] = lds_ld2(pla[c] + off);
                    }
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int J = 0; J < NB; ++J) {
                        const bool in = J <= Jtop[c];
                        const s16x4 hv = __builtin_bit_cast(s16x4, make_uint2(in ? h[J].x : 0u, in ? h[J].y : 0u));
                        const s16x4 lv = __builtin_bit_cast(s16x4, make_uint2(in ? l[J].x : 0u, in ? l[J].y : 0u));
                        acc[c][J] = mma16(eye, lv, mma16(eye, hv, zero4()));
                    }
                }
            }
            // each step's diagonal-inverse block and off-diagonal blocks are read one
            // step ahead (they are fixed by now), so the step's chain never waits on LDS;
            // A_KJ is stored at block (J, K)
            auto a_blk = [&](int J, int K) __attribute__((always_inline)) { return lds_ld_tr4(mia + 2 * (16 * J * LDL + 16 * K)); };
            s16x4 mt_n = __builtin_bit_cast(s16x4, lds_ld2(mta + 2 * 16 * (NB - 1) * MTW));
            s16x4 ak_n[NB];
#pragma unroll
            for (int J = NB - 2; J >= 0; --J) ak_n[J] = a_blk(J, NB - 1);
#pragma unroll
            for (int K = NB - 1; K >= 0; --K) {
                // x = -X_K = (-M_KK)^T acc[K], acc[K] as a bf16 pair
                const s16x4 mt = mt_n;
                s16x4 ak[NB];
#pragma unroll
                for (int J = K - 1; J >= 0; --J) ak[J] = ak_n[J];
                if (K > 0) {
                    mt_n = __builtin_bit_cast(s16x4, lds_ld2(mta + 2 * 16 * (K - 1) * MTW));
#pragma unroll
                    for (int J = K - 2; J >= 0; --J) ak_n[J] = a_blk(J, K - 1);
                }
                uint32_t x01[NCH], x23[NCH];
                f32x4 x[NCH];
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const f32x4 a = acc[c][K];
                    const uint32_t h01 = pack_bf16(a[0], a[1]), h23 = pack_bf16(a[2], a[3]);
                    const uint32_t l01 = pack_bf16(minus_bf16(h01, ns.lo, a[0]), minus_bf16(h01, ns.hi, a[1]));
                    const uint32_t l23 = pack_bf16(minus_bf16(h23, ns.lo, a[2]), minus_bf16(h23, ns.hi, a[3]));
                    x[c] = mma16(mt, __builtin_bit_cast(s16x4, make_uint2(h01, h23)), zero4());
                    x[c] = mma16(mt, __builtin_bit_cast(s16x4, make_uint2(l01, l23)), x[c]);
                }
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    x01[c] = pack_bf16(x[c][0], x[c][1]);
                    x23[c] = pack_bf16(x[c][2], x[c][3]);
                }
                // acc[J] -= A_KJ^T X_K (+= A_KJ^T x) for every J < K; the bracket solved
                // next (J = K - 1) is updated first
#pragma unroll
                for (int J = K - 1; J >= 0; --J)
#pragma unroll
                    for (int c = 0; c < NCH; ++c)
                        acc[c][J] = mma16(ak[J], __builtin_bit_cast(s16x4, make_uint2(x01[c], x23[c])), acc[c][J]);
                // lane: X[16 K + g4 + i][column l16 of the block]; delta rows j = 16 K + g4 + 1, + 3,
                // tokens 8 K + 2 gq and + 1
                // (taken as floats: this compiler's bit-cast of a vector element reads element 0)
                const f32x2 bt = lds_ldf2(sba + 4 * 8 * K);
#pragma unroll
                for (int c = 0; c < NCH; ++c) {
                    const uint32_t ev = pack_bf16(x[c][1] * -bt[0], x[c][3] * -bt[1]);
                    // Psi[n][t], n = 16 nb + l16, or Phat[t'][t], t' = 16 tb + l16
                    *(uint32_t *)(ex[c] + (K >> 2) * 1024 + (K & 3) * 256) = ev;
                    if (KY[c]) {
                        // -Yhat rows 16 K + g4 + i, column 16 nb + l16, over Kr
                        const uint32_t ya = kya[c] + 2 * 16 * K * LDA;
                        lds_st16(ya, (uint16_t)(x01[c] & 0xffffu));
                        lds_st16(ya + 2 * LDA, (uint16_t)(x01[c] >> 16));
                        lds_st16(ya + 4 * LDA, (uint16_t)(x23[c] & 0xffffu));
                        lds_st16(ya + 6 * LDA, (uint16_t)(x23[c] >> 16));
                    } else {
                        // -Z[t'][16 K + g4 ..]
                        lds_st2(K <= Jtop[c] ? pha[c] + 2 * 16 * K : dum, x01[c], x23[c]);
                    }
                }
            }
            if constexpr (C == 16) {
                // tokens 16 .. 31 of the k = 32 fragment are zero
#pragma unroll
                for (int c = 0; c < NCH; ++c)
                    if (KY[c] && lane >= 32)
                        *(uint4 *)(wsb + F::oPsi + (nb[c] * KSC * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
            }
        };
        for (int cb = wave; cb < NBD + NBC; cb += 2 * NW) {
            const int cb1 = cb + NW;
            if (cb1 < NBD + NBC) {
                if (cb1 < NBD) run_chains(std::integral_constant<int, 4>{}, cb, cb1);
                else if (cb < NBD) run_chains(std::integral_constant<int, 6>{}, cb, cb1);
                else run_chains(std::integral_constant<int, 7>{}, cb, cb1);
            } else {
                if (cb < NBD) run_chains(std::integral_constant<int, 0>{}, cb, 0);
                else run_chains(std::integral_constant<int, 1>{}, cb, 0);
            }
        }
        // Phat is causal: the Z tiles of token block tb write tokens t' < 16 (tb + 1);
        // the rest of its fragments (which the state pass reads whole) is zeroed
        // here, by lanes whose 8 tokens all lie beyond that range.
        for (int f = wave; f < NBC * KSC; f += NW) {
            const auto [lane, g4, l16, gq] = lane_ids(tid);
            const int tb = f / KSC, ks = f % KSC;
            if (32 * ks + 8 * gq >= 16 * (tb + 1))
                *(uint4 *)(wsb + F::oPh + (f * 64 + lane) * 16) = make_uint4(0u, 0u, 0u, 0u);
        }
        __syncthreads();

        if constexpr (NW == 8) {
            if (wave >= NW / 2) __builtin_amdgcn_s_setprio(1);
        }
        // ---- Phi = -(Yhat^T Kl) e^r (Kr holds -Yhat) as transposed tiles, BM x BN tiles per block
        //      (this and the Qhat loop are kept rolled: unrolled, their fragments
        //      are hoisted beside the next item's inputs and the kernel spills)
        for (int pb = wave; pb < G::NPB; pb += NW) {
            const auto [lane, g4, l16, gq] = lane_ids(tid);
            constexpr int BM = G::BM, BN = G::BN;
            const int mb0 = BM * (pb % (NBD / BM)), nb0 = BN * (pb / (NBD / BM));
            f32x4 acc[BM][BN];
#pragma unroll
            for (int a = 0; a < BM; ++a)
#pragma unroll
                for (int b = 0; b < BN; ++b) acc[a][b] = zero4();
#pragma unroll 1
            for (int s = 0; s < L / 32; ++s) {
                bf16x8 xa8[BM], yb8[BN];

#pragma unroll
                for (int a = 0; a < BM; ++a) xa8[a] = frag_col(Kl + 32 * s * LDA + 16 * (mb0 + a), LDA, lane);
#pragma unroll
                for (int b = 0; b < BN; ++b) yb8[b] = frag_col(Kr + 32 * s * LDA + 16 * (nb0 + b), LDA, lane);
#pragma unroll
                for (int a = 0; a < BM; ++a)
#pragma unroll
                    for (int b = 0; b < BN; ++b) acc[a][b] = mma32(xa8[a], yb8[b], acc[a][b]);
            }
            // lane: Phi[n = 16 nb + l16][m = 16 mb + g4 + i]
#pragma unroll
            for (int a = 0; a < BM; ++a) {
                const int mb = mb0 + a;
                const f32x4 erm = *(const f32x4 *)(ers + 16 * mb + g4);
#pragma unroll
                for (int b = 0; b < BN; ++b) {
                    const int nb = nb0 + b;
                    const f32x4 v = acc[a][b];
                    *(uint2 *)(wsb + F::oPhi + ((nb * KSD + mb / 2) * 64 + 16 * (2 * (mb & 1) + (gq >> 1)) + l16) * 16 +
                               8 * (gq & 1)) =
                        make_uint2(pack_bf16(v[0] * erm[0], v[1] * erm[1]), pack_bf16(v[2] * erm[2], v[3] * erm[3]));
                }
            }
        }
        // ---- Qhat = (Ql - Z Kl) e^r (P's high part holds -Z) as transposed tiles ----------
        if constexpr (G::PQSPLIT) {
            if (wave >= 4) {
                const auto [lane, g4, l16, gq] = lane_ids(tid);
                const int mb0 = 2 * (wave - 4);
                // all token blocks at once, k-step outer: each Kl fragment is read once per
                // k-step, each Z fragment once, and the 2 x NBC accumulations interleave
                f32x4 acc[2][NBC];
#pragma unroll
                for (int tb = 0; tb < NBC; ++tb)
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        const uint2 q0 = *(const uint2 *)(Ql + (16 * tb + l16) * LDA + 16 * (mb0 + a) + g4);
                        acc[a][tb] = f32x4{lo_bf16(q0.x), hi_bf16(q0.x), lo_bf16(q0.y), hi_bf16(q0.y)};
                    }
#pragma unroll
                for (int s = 0; s < NBC; ++s) {   // sub-steps 32 s .. 32 s + 31 reach token blocks tb >= s
                    bf16x8 kf[2];
#pragma unroll
                    for (int a = 0; a < 2; ++a) kf[a] = frag_col(Kl + 32 * s * LDA + 16 * (mb0 + a), LDA, lane);
#pragma unroll
                    for (int tb = s; tb < NBC; ++tb) {
                        const bf16x8 z = *(const bf16x8 *)(Zs + G::poff(tb) + l16 * G::pld(tb) + 32 * s + 8 * gq);
#pragma unroll
                        for (int a = 0; a < 2; ++a) acc[a][tb] = mma32(kf[a], z, acc[a][tb]);
                    }
                }
                f32x4 erm[2];
#pragma unroll
                for (int a = 0; a < 2; ++a) erm[a] = *(const f32x4 *)(ers + 16 * (mb0 + a) + g4);
#pragma unroll
                for (int tb = 0; tb < NBC; ++tb)
#pragma unroll
                    for (int a = 0; a < 2; ++a) {
                        const int mb = mb0 + a;
                        *(uint2 *)(wsb + F::oQh + ((tb * KSD + mb / 2) * 64 + 16 * (2 * (mb & 1) + (gq >> 1)) + l16) * 16 +
                                   8 * (gq & 1)) =
                            make_uint2(pack_bf16(acc[a][tb][0] * erm[a][0], acc[a][tb][1] * erm[a][1]),
                                       pack_bf16(acc[a][tb][2] * erm[a][2], acc[a][tb][3] * erm[a][3]));
                    }
            }
        } else
        for (int mb = wave; mb < NBD; mb += NW) {
            const auto [lane, g4, l16, gq] = lane_ids(tid);
            const f32x4 erm = *(const f32x4 *)(ers + 16 * mb + g4);
#pragma unroll 1
            for (int tb = 0; tb < NBC; ++tb) {
                const int pr = G::poff(tb) + l16 * G::pld(tb);

                const uint2 q0 = *(const uint2 *)(Ql + (16 * tb + l16) * LDA + 16 * mb + g4);
                f32x4 acc = {lo_bf16(q0.x), hi_bf16(q0.x), lo_bf16(q0.y), hi_bf16(q0.y)};
#pragma unroll
                for (int s = 0; s < tb + 1; ++s)
                    acc = mma32(frag_col(Kl + 32 * s * LDA + 16 * mb, LDA, lane),
                                *(const bf16x8 *)(Zs + pr + 32 * s + 8 * gq), acc);
                // lane: Qhat[t = 16 tb + l16][m = 16 mb + g4 + i] / e^r
                *(uint2 *)(wsb + F::oQh + ((tb * KSD + mb / 2) * 64 + 16 * (2 * (mb & 1) + (gq >> 1)) + l16) * 16 +
                           8 * (gq & 1)) =
                    make_uint2(pack_bf16(acc[0] * erm[0], acc[1] * erm[1]), pack_bf16(acc[2] * erm[2], acc[3] * erm[3]));
            }
        }
        // No barrier here: the next item writes LDS before its first barrier only
        // in b', beta, gamma (read above only by the Y and Z exports, before the
        // last barrier) and in the scan's per-wave decay totals (in M's region, not
        // read since that barrier).
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state pass.  The chunks of a head are walked in order; one
// workgroup owns a BV-column slice of one head's state over one range of
// chunks.  Per chunk c, one barrier, then
//   state waves (D/16): 16 rows of S <- e^{G_C} S + Phi S + Psi V, then S^T (bf16)
//                       for the next chunk;
//   output waves (C/16): 16 tokens of o = Qhat S + Phat V (transposed, so rows of
//                       o leave as 16-byte runs), and the value rows and outputs
//                       between HBM and LDS.
// Each wave fetches its own factor fragments two chunks ahead (chunk indices
// clamped, never skipped, so every wait covers only those fetches).  The
// slices of one (head, range) get workgroup ids congruent mod 8 (same XCD, one
// L2 for the shared factor blocks).
//
// Segments.  A workgroup's time per chunk is bound by fetching the chunk's
// factor blocks, whatever the slice width, so with few heads the chunks of a
// head are cut into P ranges ("segments") walked at the same time, with wide
// slices.  The chunk maps compose: over segment s, S_out = M_s S_in + N_s, with
// M_s the product of the chunk maps e^{G_C} + Phi and N_s the end state from a
// zero start.  KIND_SUMMARY walks segment s < P - 1 on the augmented state
// [M | N], started from [I | 0] (no outputs; the M columns take no value
// term); eda_bf16_combine takes the prefix S_in(s + 1) = M_s S_in(s) + N_s in
// fp32; KIND_PASS walks every segment from its start state, with outputs.
// ---------------------------------------------------------------------------
constexpr int KIND_PASS = 0, KIND_SUMMARY = 1;

template <int C, int D, int BV>
struct K2G {
    using F = Fac<C, D>;
    static constexpr int NBC = F::NBC, NBD = F::NBD, NCB = BV / 16;
    static constexpr int KSD = F::KSD, KSC = F::KSC;
    static constexpr int NSW = NBD, NW = NBD + NBC, NT = 64 * NW;
    static_assert(NT <= 1024, "workgroup size");
    static constexpr int LDT = D + 8, LDV = BV + 8, LDO = BV + 8;
    static constexpr int VR = imax(C, 32);                          // value rows (rows >= C stay zero)
    static constexpr int VPL = BV / 8;                              // 16-byte pieces per value row
    static constexpr int NPO = (16 * VPL + 63) / 64;                // pieces per output-wave lane
    static constexpr int szSt = align16(BV * LDT * 2), szVs = align16(VR * LDV * 2);
    static constexpr int oSt = 0;                                   // S^T [2][BV][LDT] bf16
    static constexpr int oVs = oSt + 2 * szSt;                      // V   [2][VR][LDV] bf16
    static constexpr int oOs = oVs + 2 * szVs;                      // o   [C][LDO] bf16 (per output wave: its rows)
    static constexpr int LDS = oOs + align16(C * LDO * 2);
};

template <int NF, int NPO>
struct FragSet {
    bf16x8 R[NF];   // the role's factor fragments of one chunk
    f32x4 dec;      // state role: e^{G_C} of its rows
    uint4 v[NPO];   // output role: 16-byte pieces of the value slice
    uint32_t pf[2]; // output role: L2 warm-up words
};

// L2 warm-up of the state pass (when the workspace exceeds the MALL): while
// fetching chunk c's operands, output wave w of slice j also reads one word
// of every (R NBC)-th 128-byte line of chunk c + warm's block, so the R slices
// of a head (same XCD, one L2) together bring that block into L2 before its
// fragments are fetched.  The words are consumed, unused, when the chunk's
// set is.  The distance `warm` (0: no warm-up) is two chunks without
// segments and one with them (eight segments' units per XCD keep more lines
// in flight); at four, the warmed lines were often evicted before their
// fetch and the pass read its blocks 1.7 times over.  The segment maps run
// without it (they read Phi and Psi alone, and their blocks met in L2 anyway).
constexpr int WARM_PLAIN = 2, WARM_SEGMENTS = 1;
constexpr size_t WARM_MIN_BYTES = (size_t)256 << 20;   // MI355X MALL capacity

// VV: every value slice is whole (d_v a multiple of BV) and v is 16-byte
// aligned, so values and outputs move as 16-byte row pieces.
//
// Work units: KIND_PASS, NSEG = P units per head (one per segment), R = the
// value slices; KIND_SUMMARY, NSEG = P - 1, R = RX + the value slices, slices
// below RX holding the M columns (key channels).  NCS chunks per segment.
// segbuf: KIND_PASS, the start states of segments 1 .. P-1, [BH][P-1][d_k][d_v]
// (NULL when P = 1); KIND_SUMMARY, the maps written, [BH][P-1][d_k][d_k + d_v]
// (M in the first d_k columns, N in the rest).
template <int C, int D, int BV, bool VV, int KIND>
__global__ void __launch_bounds__((K2G<C, D, BV>::NT))
eda_bf16_state(const bf16 *__restrict__ v, const float *S0, float *S_final, bf16 *__restrict__ o,
               const char *__restrict__ ws, float *segbuf, int Tlen, int H, int BH, int dk, int dv,
               int NC, int R, int RX, int NSEG, int NCS, int warm) {
    using G = K2G<C, D, BV>;
    using F = Fac<C, D>;
    using T = bf16;
    constexpr bool SUM = KIND == KIND_SUMMARY;
    constexpr int NCB = G::NCB, KSD = G::KSD, KSC = G::KSC, LDT = G::LDT, LDV = G::LDV, LDO = G::LDO;
    constexpr int NSW = G::NSW, VPL = G::VPL, NPO = G::NPO;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Os = (T *)(smem + G::oOs);

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int unit = (slot / R) * 8 + xcd, slice = slot % R;
    if (unit >= BH * NSEG) return;
    const int bh = unit / NSEG, seg = unit % NSEG;
    const int c_lo = seg * NCS, c_hi = min(NC, c_lo + NCS);
    // KIND_SUMMARY: slices below RX hold M's columns (identity start, no value term)
    const bool mcols = SUM && slice < RX;
    const int n0 = SUM && !mcols ? (slice - RX) * BV : slice * BV;   // first column within its part
    const int ncols = mcols ? dk : dv;                                // columns of that part
    const int b = bh / H, h = bh % H;
    const long hrow = (long)b * Tlen * H + h;
    const long HV = (long)H * dv;
    const T *vh = v + hrow * dv + (mcols ? 0 : n0);
    T *oh = o + hrow * dv + n0;
    const char *wsh = ws + (long)bh * NC * F::bytes;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;

    // the value rows beyond the chunk (read by the k = 32 products at C = 16) are zero
    if constexpr (C < G::VR) {
        for (int idx = tid; idx < 2 * (G::VR - C) * LDV; idx += G::NT) {
            const int bsel = idx / ((G::VR - C) * LDV), rem = idx % ((G::VR - C) * LDV);
            ((T *)(smem + G::oVs + bsel * G::szVs))[C * LDV + rem] = (T)0;
        }
    }
    auto St = [&](int c) __attribute__((always_inline)) { return (T *)(smem + G::oSt + (c & 1) * G::szSt); };
    auto Vs = [&](int c) __attribute__((always_inline)) { return (T *)(smem + G::oVs + (c & 1) * G::szVs); };

    auto run = [&](auto role) __attribute__((always_inline)) {
        constexpr bool RS = decltype(role)::value == 0;   // state role, else output role
        constexpr int NF = KSD + KSC;
        using Set = FragSet<NF, NPO>;
        const int rb = RS ? wave : wave - NSW;            // row block: state rows or tokens
        // output role: the lane's pieces p = lane + 64 j of the value slice (token
        // 16 rb + p / VPL, columns 8 (p % VPL) ..)
        auto vpiece = [&](int j) __attribute__((always_inline)) { return lane + 64 * j; };

        auto load = [&](Set &s, int c) __attribute__((always_inline)) {
            const char *blk = wsh + (long)c * F::bytes;
            if constexpr (RS) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) s.R[ks] = ld_frag(blk + F::oPhi + ((rb * KSD + ks) * 64 + lane) * 16);
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) s.R[KSD + ks] = ld_frag(blk + F::oPsi + ((rb * KSC + ks) * 64 + lane) * 16);
                s.dec = *(const f32x4 *)(blk + F::oDec + 4 * (16 * rb + g4));
            } else {
                if constexpr (!SUM) {
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) s.R[ks] = ld_frag(blk + F::oQh + ((rb * KSD + ks) * 64 + lane) * 16);
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) s.R[KSD + ks] = ld_frag(blk + F::oPh + ((rb * KSC + ks) * 64 + lane) * 16);
                }
#pragma unroll
                for (int j = 0; j < NPO; ++j) {
                    const int p = vpiece(j), vr = p / VPL, vc = p % VPL;
                    const int t = c * C + 16 * rb + vr, tc = t < Tlen ? t : Tlen - 1;
                    const bool ok = p < 16 * VPL && t < Tlen && !mcols;
                    const int vcc = p < 16 * VPL ? vc : 0;
                    uint4 x;
                    if constexpr (VV) {
                        x = *(const uint4 *)(vh + tc * HV + 8 * vcc);
                    } else {
                        uint32_t y[8];
#pragma unroll
                        for (int jj = 0; jj < 8; ++jj) {
                            const int col = 8 * vcc + jj, cc = n0 + col < dv ? col : dv - 1 - n0;
                            y[jj] = mcols ? 0u : (uint32_t)vh[tc * HV + (cc < 0 ? 0 : cc)];
                            if (n0 + col >= dv) y[jj] = 0u;
                        }
                        x = make_uint4(y[0] | (y[1] << 16), y[2] | (y[3] << 16), y[4] | (y[5] << 16), y[6] | (y[7] << 16));
                    }
                    s.v[j] = ok ? x : make_uint4(0u, 0u, 0u, 0u);
                }
                s.pf[0] = s.pf[1] = 0u;
                if (warm) {
                    const int cw = c + warm < NC ? c + warm : NC - 1;
                    const char *wb = wsh + (long)cw * F::bytes;
                    const int stride = R * G::NBC;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int off = (slice * G::NBC + rb + stride * (64 * i + lane)) * 128;
                        s.pf[i] = *(const uint32_t *)(wb + (off < F::bytes - 4 ? off : F::bytes - 4));
                    }
                }
            }
        };
        auto put_v = [&](const Set &s, int c) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < NPO; ++j) {
                const int p = vpiece(j);
                if (!RS && p < 16 * VPL) *(uint4 *)(Vs(c) + (16 * rb + p / VPL) * LDV + 8 * (p % VPL)) = s.v[j];
            }
        };

        // state rows 16 rb + g4 + i, columns n0 + 16 cb + l16 of its part (state role)
        f32x4 S[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            S[cb] = zero4();
            if (RS) {
                const int col = n0 + 16 * cb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rb + g4 + i;
                    if (row >= dk || col >= ncols) continue;
                    if constexpr (SUM) {
                        S[cb][i] = mcols && row == col ? 1.f : 0.f;
                    } else if (seg == 0) {
                        if (S0) S[cb][i] = S0[((long)bh * dk + row) * dv + col];
                    } else {
                        S[cb][i] = segbuf[(((long)bh * (NSEG - 1) + seg - 1) * dk + row) * dv + col];
                    }
                }
            }
        }
        auto write_St = [&](int c) __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store4<T>(St(c) + (16 * cb + l16) * LDT + 16 * rb + g4, S[cb][0], S[cb][1], S[cb][2], S[cb][3]);
        };

        // Phase c (one barrier): S_c^T is in St(c) and V_c in Vs(c).  The state
        // waves write S_{c+1}^T to St(c + 1), the output waves write V_{c+1} to
        // Vs(c + 1): both buffers were last read in phase c - 1.  Each 16-column
        // block's operands are read just before its products.
        auto body = [&](Set &cur, Set &nxt, Set &far, int c) __attribute__((always_inline)) {
            const int cf = c + 2 < c_hi ? c + 2 : c_hi - 1;   // chunk whose operands are fetched now
            __syncthreads();
            const T *Sc = St(c), *Vc = Vs(c);
            // k-step outer, column block inner: the NCB accumulation chains interleave,
            // and each k-step's operand fragments are read just before its products
            if constexpr (RS) {
                // S <- e^{G_C} S + Psi V + Phi S  (rows 16 rb.., all slice columns)
                f32x4 acc[NCB];
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc[cb][i] = cur.dec[i] * S[cb][i];
#pragma unroll
                for (int ks = 0; ks < KSC; ++ks) {
                    bf16x8 vf[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) vf[cb] = frag_col(Vc + 32 * ks * LDV + 16 * cb, LDV, lane);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(cur.R[KSD + ks], vf[cb], acc[cb]);
                }
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks) {
                    bf16x8 sf[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) sf[cb] = frag_row(Sc + 16 * cb * LDT + 32 * ks, LDT, lane);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(cur.R[ks], sf[cb], acc[cb]);
                }
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) S[cb] = acc[cb];
                if (c + 1 < c_hi) write_St(c + 1);
                load(far, cf);
            } else {
                if constexpr (!SUM) {
                    // o^T = V^T Phat^T + S^T Qhat^T for the wave's 16 tokens
                    f32x4 acc[NCB];
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[cb] = zero4();
#pragma unroll
                    for (int ks = 0; ks < KSC; ++ks) {
                        bf16x8 vf[NCB];
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) vf[cb] = frag_col(Vc + 32 * ks * LDV + 16 * cb, LDV, lane);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(vf[cb], cur.R[KSD + ks], acc[cb]);
                    }
#pragma unroll
                    for (int ks = 0; ks < KSD; ++ks) {
                        bf16x8 sf[NCB];
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) sf[cb] = frag_row(Sc + 16 * cb * LDT + 32 * ks, LDT, lane);
#pragma unroll
                        for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(sf[cb], cur.R[ks], acc[cb]);
                    }
                    if (c + 1 < c_hi) put_v(nxt, c + 1);
                    asm volatile("" ::"v"(cur.pf[0]), "v"(cur.pf[1]));   // the warm-up words, consumed
                    // the wave's own 16 token rows: staged in LDS, then written as
                    // 16-byte row pieces (the rows are this wave's alone: no barrier)
                    const int tr = 16 * rb + l16;
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb)
                        store4<T>(Os + tr * LDO + 16 * cb + g4, acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
                    wave_lds_sync();
                    load(far, cf);
#pragma unroll
                    for (int j = 0; j < NPO; ++j) {
                        const int p = vpiece(j), vr = p / VPL, vc = p % VPL;
                        const int t = c * C + 16 * rb + vr;
                        if (p < 16 * VPL && t < Tlen) {
                            const uint4 val = *(const uint4 *)(Os + (16 * rb + vr) * LDO + 8 * vc);
                            T *dst = oh + t * HV + 8 * vc;
                            if constexpr (VV) {
                                *(uint4 *)dst = val;
                            } else {
                                const uint32_t y[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                                for (int jj = 0; jj < 8; ++jj)
                                    if (n0 + 8 * vc + jj < dv) dst[jj] = (T)((y[jj >> 1] >> (16 * (jj & 1))) & 0xffffu);
                            }
                        }
                    }
                } else {
                    // (summary: the values only)
                    if (c + 1 < c_hi) put_v(nxt, c + 1);
                    asm volatile("" ::"v"(cur.pf[0]), "v"(cur.pf[1]));
                    load(far, cf);
                }
            }
        };

        // three operand sets in rotation: the chunk in use, the next, and the one
        // being fetched
        Set A, B, X;
        load(A, c_lo);
        load(B, c_lo + 1 < c_hi ? c_lo + 1 : c_lo);
        if constexpr (RS) write_St(c_lo);
        else put_v(A, c_lo);
        int c = c_lo;
        for (; c + 3 <= c_hi; c += 3) {
            body(A, B, X, c);
            body(B, X, A, c + 1);
            body(X, A, B, c + 2);
        }
        if (c < c_hi) body(A, B, X, c);
        if (c + 1 < c_hi) body(B, X, A, c + 1);

        if constexpr (RS) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                const int col = n0 + 16 * cb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rb + g4 + i;
                    if (row >= dk || col >= ncols) continue;
                    if constexpr (SUM) {
                        // M_s in columns 0 .. d_k - 1, N_s after them
                        segbuf[(((long)bh * NSEG + seg) * dk + row) * (dk + dv) + (mcols ? col : dk + col)] = S[cb][i];
                    } else if (seg == NSEG - 1 && S_final) {
                        // every read of S0 happened before the chunk loop, so S_final may be S0
                        S_final[((long)bh * dk + row) * dv + col] = S[cb][i];
                    }
                }
            }
        }
    };

    if (wave < NSW) run(std::integral_constant<int, 0>{});
    else run(std::integral_constant<int, 1>{});
}

// Prefix over segments, fp32: S_in(s + 1) = M_s S_in(s) + N_s for s = 0 .. P-2,
// with S_in(0) = S0 (zero when S0 is NULL), on the fp32 matrix cores (16x16x4:
// products exact in fp32, fp32 sums).  One workgroup per (head, 16-column slice
// of the value dimension); wave w owns rows 16 w .. 16 w + 15 of the slice.
// The A operands (rows of M_s) come straight from memory into registers, one
// step ahead; S_in(s) sits transposed in LDS as the B operand.  K-step (j, i)
// takes k = 16 j + 4 g + i in lane group g, so a lane's four consecutive k of a
// row of M_s arrive as one 16-byte piece (V4: d_k and d_k + d_v multiples of
// 4).  The slices of a head get workgroup ids congruent mod 8 (one XCD, one L2
// for the maps they all read).  maps: [BH][P-1][d_k][d_k + d_v]; starts
// (written): [BH][P-1][d_k][d_v] for segments 1 .. P-1.
constexpr int COMB_W = 8, COMB_T = 64 * COMB_W, COMB_LD = 128 + 4;
template <bool V4>
__global__ void __launch_bounds__(COMB_T)
eda_bf16_combine(const float *S0, const float *__restrict__ maps, float *__restrict__ starts, int BH, int dk,
                 int dv, int P) {
    __shared__ __attribute__((aligned(16))) float XT[16][COMB_LD];   // S_in^T: column, row (zero beyond d_k)
    const int nsl = (dv + 15) / 16, xcd = blockIdx.x & 7, slot = blockIdx.x >> 3;
    const int bh = (slot / nsl) * 8 + xcd, c0 = 16 * (slot % nsl);
    if (bh >= BH) return;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, gq = lane >> 4;
    const int col = c0 + l16;                 // the lane's column (B operand, output)
    const int arow = 16 * wave + l16;         // the lane's row of M_s (A operand)
    const int orow = 16 * wave + 4 * gq;      // the lane's first output row
    const long ld = (long)dk + dv;
    for (int idx = tid; idx < 16 * 128; idx += COMB_T) {
        const int c = idx >> 7, k = idx & 127;
        XT[c][k] = (S0 && k < dk && c0 + c < dv) ? S0[((long)bh * dk + k) * dv + c0 + c] : 0.f;
    }
    auto mbase = [&](int s) __attribute__((always_inline)) { return maps + ((long)bh * (P - 1) + s) * dk * ld; };
    auto fetch = [&](f32x4 (&a)[8], int s) __attribute__((always_inline)) {
        const float *m = mbase(s) + (arow < dk ? arow : 0) * ld;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int k = 16 * j + 4 * gq;
            if constexpr (V4) {
                a[j] = (arow < dk && k < dk) ? *(const f32x4 *)(m + k) : zero4();
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i) a[j][i] = (arow < dk && k + i < dk) ? m[k + i] : 0.f;
            }
        }
    };
    auto step = [&](const f32x4 (&a)[8], f32x4 (&an)[8], int s) __attribute__((always_inline)) {
        if (s + 2 < P) fetch(an, s + 1);   // the next map, in flight during this step
        f32x4 y;                           // N_s: rows orow + i, column col
        const float *nb = mbase(s) + dk + (col < dv ? col : 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) y[i] = (orow + i < dk && col < dv) ? nb[(orow + i) * ld] : 0.f;
        __syncthreads();   // XT holds S_in(s)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const f32x4 b = *(const f32x4 *)&XT[l16][16 * j + 4 * gq];
#pragma unroll
            for (int i = 0; i < 4; ++i) y = __builtin_amdgcn_mfma_f32_16x16x4f32(a[j][i], b[i], y, 0, 0, 0);
        }
        __syncthreads();   // every wave has read S_in(s)
        *(f32x4 *)&XT[l16][orow] = y;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (orow + i < dk && col < dv) starts[(((long)bh * (P - 1) + s) * dk + orow + i) * dv + col] = y[i];
    };
    f32x4 a0[8], a1[8];
    if (P > 1) fetch(a0, 0);
    for (int s = 0; s + 1 < P; s += 2) {
        step(a0, a1, s);
        if (s + 2 < P) step(a1, a0, s + 1);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static int pad_dim(int dk, int dv) {
    const int p = dk > dv ? dk : dv;
    return p <= 32 ? 32 : (p <= 64 ? 64 : 128);
}

// Plan of the state pass, a function of the sizes alone (the workspace size
// repeats it): the value-column slice width BV and the segment count P.
// Many heads: no segments, and the narrowest slice (>= 16 columns) that
// still leaves at most one workgroup per compute unit (256 on MI355X).
// Fewer heads than fill the chip even with 16-column slices, and a long
// sequence: 64-column slices and P segments, the largest power of two that
// keeps at least 64 chunks per segment and at most 256 workgroups both in the
// pass and in the segment maps, which walk whole-width slices (one for M's
// columns, one for the values; segment maps double the factor reads of the
// state side, so shorter segments cost more than they gain; measured on MI355X
// at d = 128).  NCS chunks per segment; P is recounted from NCS so that no
// segment is empty.
struct SegPlan {
    int BV, P, NCS;
};
static SegPlan seg_plan(int BH, int NC, int D, int dv) {
    SegPlan sp{16, 1, NC};
    while (sp.BV < 32 && sp.BV < D && (long)BH * (D / sp.BV) > 256) sp.BV *= 2;
    if (D >= 64 && (long)BH * (D / 16) < 256 && NC >= 256) {
        sp.BV = 64;
        const long units = (long)BH * ((dv + 63) / 64);        // pass workgroups per segment
        const long mapw = (long)BH * (1 + (dv + D - 1) / D);   // map workgroups per segment
        while (sp.P < 64 && NC >= 64 * 2 * sp.P && units * 2 * sp.P <= 256 && mapw * (2 * sp.P - 1) <= 256)
            sp.P *= 2;
    }
    sp.NCS = (NC + sp.P - 1) / sp.P;
    sp.P = (NC + sp.NCS - 1) / sp.NCS;
    return sp;
}

template <int C, int D>
size_t fac_bytes(int B, int Tlen, int H) {
    return (size_t)B * H * ((Tlen + C - 1) / C) * Fac<C, D>::bytes;
}

// segment maps [BH][P-1][d_k][d_k + d_v] and start states [BH][P-1][d_k][d_v]
// (fp32), after the chunk factors
static size_t seg_bytes(int BH, int dk, int dv, int P) {
    return P > 1 ? (size_t)BH * (P - 1) * dk * ((size_t)dk + 2 * (size_t)dv) * 4 : 0;
}

template <int C, int D>
size_t ws_bytes(int B, int Tlen, int H, int dk, int dv) {
    const int NC = (Tlen + C - 1) / C;
    const SegPlan sp = seg_plan(B * H, NC, D, dv);
    return fac_bytes<C, D>(B, Tlen, H) + seg_bytes(B * H, dk, dv, sp.P);
}

template <int C, int D, int BV>
hipError_t launch_t(const void *q, const void *k, const void *e, const void *v, const void *decay,
                    const float *A_log, const float *dt_bias, const float *beta, const float *gamma,
                    const float *S0, void *o, float *S_final, int B, int Tlen, int H, int Hk, int dk,
                    int dv, void *ws, hipStream_t stream, hipEvent_t const *ev) {
    using G1 = K1G<C, D>;
    using G2 = K2G<C, D, BV>;
    const int NC = (Tlen + C - 1) / C, BH = B * H;
    // 16-byte loads of whole rows need d_k == D and 16-byte aligned bases
    // (D is a multiple of 8, so every row start stays aligned)
    const bool layer = A_log != nullptr, dplr = beta == nullptr;
    const bool vec = (dk == D) && ((uintptr_t)q % 16 == 0) && ((uintptr_t)k % 16 == 0) &&
                     ((uintptr_t)e % 16 == 0) && ((uintptr_t)decay % 16 == 0) &&
                     (!layer || ((uintptr_t)A_log % 16 == 0 && (uintptr_t)dt_bias % 16 == 0));
    const bool vv = (dv % BV == 0) && ((uintptr_t)v % 16 == 0) && ((uintptr_t)o % 16 == 0);
    auto k1 = layer  ? (vec ? eda_bf16_factors<C, D, true, MODE_LAYER> : eda_bf16_factors<C, D, false, MODE_LAYER>)
              : dplr ? (vec ? eda_bf16_factors<C, D, true, MODE_DPLR> : eda_bf16_factors<C, D, false, MODE_DPLR>)
                     : (vec ? eda_bf16_factors<C, D, true, MODE_PLAIN> : eda_bf16_factors<C, D, false, MODE_PLAIN>);
    auto k2 = vv ? eda_bf16_state<C, D, BV, true, KIND_PASS> : eda_bf16_state<C, D, BV, false, KIND_PASS>;
    hipError_t err = hipFuncSetAttribute((const void *)k1, hipFuncAttributeMaxDynamicSharedMemorySize, G1::LDS);
    if (err != hipSuccess) return err;
    int dev = 0, ncu = 256;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const long items = (long)BH * NC;
    const long per_cu = G1::NW == 8 ? 1 : 2;   // workgroups per compute unit (LDS)
    const int grid1 = (int)(items < per_cu * ncu ? items : per_cu * ncu);
    if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(k1, dim3((unsigned)grid1), dim3(G1::NT), G1::LDS, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)e, decay, A_log, dt_bias, beta, gamma, (char *)ws,
                       Tlen, H, Hk, dk, NC, BH);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    const SegPlan sp = seg_plan(BH, NC, D, dv);
    const int R = (dv + BV - 1) / BV;
    const int warm = fac_bytes<C, D>(B, Tlen, H) <= WARM_MIN_BYTES ? 0 : sp.P > 1 ? WARM_SEGMENTS : WARM_PLAIN;
    float *maps = nullptr, *starts = nullptr;
    if (sp.P > 1) {
        // segment maps (whole-width slices: one for M's d_k columns, one for the
        // values), their prefix, then the segments' passes
        using G2S = K2G<C, D, D>;
        maps = (float *)((char *)ws + fac_bytes<C, D>(B, Tlen, H));
        starts = maps + (size_t)BH * (sp.P - 1) * dk * (dk + dv);
        const int RX = (dk + D - 1) / D, RS = (dv + D - 1) / D;
        const bool vvs = (dv % D == 0) && ((uintptr_t)v % 16 == 0);
        const int gridS = 8 * ((BH * (sp.P - 1) + 7) / 8) * (RX + RS);
        auto ks = vvs ? eda_bf16_state<C, D, D, true, KIND_SUMMARY> : eda_bf16_state<C, D, D, false, KIND_SUMMARY>;
        if ((err = hipFuncSetAttribute((const void *)ks, hipFuncAttributeMaxDynamicSharedMemorySize, G2S::LDS)) !=
            hipSuccess)
            return err;
        hipLaunchKernelGGL(ks, dim3((unsigned)gridS), dim3(G2S::NT), G2S::LDS, stream, (const bf16 *)v, S0,
                           S_final, (bf16 *)o, (const char *)ws, maps, Tlen, H, BH, dk, dv, NC, RX + RS, RX,
                           sp.P - 1, sp.NCS, 0);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        auto kc = (dk % 4 == 0 && (dk + dv) % 4 == 0) ? eda_bf16_combine<true> : eda_bf16_combine<false>;
        hipLaunchKernelGGL(kc, dim3((unsigned)(8 * ((BH + 7) / 8) * ((dv + 15) / 16))), dim3(COMB_T), 0, stream,
                           S0, (const float *)maps, starts, BH, dk, dv, sp.P);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const int grid2 = 8 * ((BH * sp.P + 7) / 8) * R;
    hipLaunchKernelGGL(k2, dim3((unsigned)grid2), dim3(G2::NT), G2::LDS, stream, (const bf16 *)v, S0,
                       S_final, (bf16 *)o, (const char *)ws, starts, Tlen, H, BH, dk, dv, NC, R, 0, sp.P,
                       sp.NCS, warm);
    err = hipGetLastError();
    if (err == hipSuccess && ev) err = hipEventRecord(ev[2], stream);
    return err;
}

}  // namespace b16

size_t bf16_ws_bytes(int B, int Tlen, int H, int dk, int dv, int chunk) {
    const int D = b16::pad_dim(dk, dv);
#define EDA_WS(CC, DD) if (chunk == CC && D == DD) return b16::ws_bytes<CC, DD>(B, Tlen, H, dk, dv);
    EDA_WS(16, 32) EDA_WS(16, 64) EDA_WS(16, 128)
    EDA_WS(32, 32) EDA_WS(32, 64) EDA_WS(32, 128)
    EDA_WS(64, 32) EDA_WS(64, 64) EDA_WS(64, 128)
#undef EDA_WS
    return 0;
}

// decay: alpha (fp32), or with A_log != NULL the safe gate's input a (bf16)
// of Hk key heads (the fused layer prologue); otherwise Hk == H.  beta ==
// NULL selects the rank-1 DPLR update, with its erase vector a in `e`.
hipError_t launch_bf16(const void *q, const void *k, const void *e, const void *v, const void *decay,
                       const float *A_log, const float *dt_bias, const float *beta, const float *gamma,
                       const float *S0, void *o, float *S_final, int B, int Tlen, int H, int Hk, int dk,
                       int dv, int chunk, void *ws, hipStream_t stream, hipEvent_t const *ev) {
    const int D = b16::pad_dim(dk, dv);
    const int BV = b16::seg_plan(B * H, (Tlen + chunk - 1) / chunk, D, dv).BV;
#define EDA_GO(CC, DD, BB)                                                                          \
    if (chunk == CC && D == DD && BV == BB)                                                         \
        return b16::launch_t<CC, DD, BB>(q, k, e, v, decay, A_log, dt_bias, beta, gamma, S0, o,     \
                                         S_final, B, Tlen, H, Hk, dk, dv, ws, stream, ev);
    EDA_GO(16, 32, 16) EDA_GO(16, 32, 32) EDA_GO(16, 64, 16) EDA_GO(16, 64, 32) EDA_GO(16, 64, 64)
    EDA_GO(16, 128, 16) EDA_GO(16, 128, 32) EDA_GO(16, 128, 64)
    EDA_GO(32, 32, 16) EDA_GO(32, 32, 32) EDA_GO(32, 64, 16) EDA_GO(32, 64, 32) EDA_GO(32, 64, 64)
    EDA_GO(32, 128, 16) EDA_GO(32, 128, 32) EDA_GO(32, 128, 64)
    EDA_GO(64, 32, 16) EDA_GO(64, 32, 32) EDA_GO(64, 64, 16) EDA_GO(64, 64, 32) EDA_GO(64, 64, 64)
    EDA_GO(64, 128, 16) EDA_GO(64, 128, 32) EDA_GO(64, 128, 64)
#undef EDA_GO
    return hipErrorInvalidValue;
}

}  // namespace eda
