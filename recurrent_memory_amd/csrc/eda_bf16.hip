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
// so A = Diag(b') strict_lower(Kl Kr^T) and P = causal(Ql Kr^T).  With the
// scaled state S' = Diag(e^r) S, M = (I + A)^{-1}, the WY factors
//   W = M Diag(b') Kl   [L x d_k],     T' = (M Diag(b'))[:, delta sub-steps]   [L x C]
// give, per chunk,
//   U = T' V - W S',   o = Ql S' + P U,   S_next = Diag(e^r) (Diag(e^r) S + Kr^T U)
// (e^{G_C} = e^{2r}).  Every factor stays within e^{+-|G_C|/2}; a chunk in
// which some channel decays by more than e^-120 (only possible below the safe
// gate's floor alpha = e^-5) computes A and P element-wise from e^{G_j - G_i}
// and uses the unsplit factors kap o e^G, q o e^G and Khat instead.
//
// Kernel 1 (eda_bf16_factors): persistent workgroups walk the (head, chunk)
//   items; each item's raw values are fetched into registers while the
//   previous item is processed.  Per item: the cumulative decay, the scaled
//   operands (and Diag(e^r) Kr^T straight to the workspace), A and P on the
//   matrix cores, (I + A)^{-1} (fp32 substitution on the 16x16 diagonal
//   blocks, then one column block of the rest per wave, held in registers),
//   W, Q^ and P^ on the matrix cores, and the export of -W Diag(e^r), T', Q^,
//   P^ and the per-channel decay to the workspace.
// Kernel 2 (eda_bf16_state): one workgroup per (head, slice of value
//   columns), serial over chunks, fp32 state in registers.  The factors are
//   stored in the exact per-lane order of the matrix-core operands, so each
//   wave fetches its own operands straight into registers three chunks
//   ahead; only S'^T, U^T, the value slice and the outputs pass through LDS,
//   and each role reads all its LDS operands before its first product.  Two
//   barriers per chunk.
//
// Workspace: one block of Fac<C, D>::bytes per chunk and head.  A "fragment"
// of a matrix M (rows x k, row-major view) is the 16 x 32 block at
// (16 rb, 32 ks): 64 lanes x 16 bytes, lane 16 g + r holding
// M[16 rb + r][32 ks + 8 g .. 32 ks + 8 g + 7] -- the operand layout of the
// 16x16x32 bf16 matrix instruction.
#include <type_traits>

#include "eda_common.h"

namespace eda {
namespace b16 {

// factor kernel: 4 waves per workgroup, so that two workgroups (two chunks in
// flight, each with its own barriers) share a compute unit
constexpr int K1WAVES = 4, K1THREADS = 64 * K1WAVES;

// wide-chunk threshold on a chunk's log2-decay (e^-120 = 2^-173)
constexpr float WIDE_G2 = 173.f;

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

__device__ __forceinline__ bf16x8 ld_frag(const char *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ void st_frag(char *p, bf16x8 x) { *reinterpret_cast<bf16x8 *>(p) = x; }

// Inclusive prefix sum over groups of N consecutive lanes (N a power of two);
// `seg` is the lane's index in its group.  Groups of 16 use DPP row shifts.
template <int N>
__device__ __forceinline__ float scan_group(float x, int seg) {
    // DPP row shifts (rows of 16 lanes; lanes shifted in from outside the row read 0)
#define EDA_ROW_SHR(n) \
    __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x110 + (n), 0xf, 0xf, true))
    if constexpr (N == 16) {
        x += EDA_ROW_SHR(1); x += EDA_ROW_SHR(2); x += EDA_ROW_SHR(4); x += EDA_ROW_SHR(8);
    } else if constexpr (N == 8) {
        // the upper 8 lanes of a row must not take values from the lower 8
        float y;
        y = EDA_ROW_SHR(1); x += seg >= 1 ? y : 0.f;
        y = EDA_ROW_SHR(2); x += seg >= 2 ? y : 0.f;
        y = EDA_ROW_SHR(4); x += seg >= 4 ? y : 0.f;
    } else {
#pragma unroll
        for (int off = 1; off < N; off <<= 1) {
            const float y = __shfl_up(x, off, N);
            if (seg >= off) x += y;
        }
    }
#undef EDA_ROW_SHR
    return x;
}

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

// Value of lane S of each group of four lanes (DPP quad permutation).
template <int S>
__device__ __forceinline__ float quad_bcast(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x55 * S, 0xf, 0xf, false));
}

// Value of the last lane of each group of N consecutive lanes.
template <int N>
__device__ __forceinline__ float group_last(float x) {
    if constexpr (N == 16) {
        // ds_swizzle bit mode: lane' = (lane & 0x10) | 0xF within each 32 lanes
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x1F0));
    } else if constexpr (N == 8) {
        // lane' = (lane & 0x18) | 0x7
        return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0xF8));
    } else {
        return __shfl(x, N - 1, N);
    }
}

// ---------------------------------------------------------------------------
// Workspace block of one chunk and head (byte offsets; fragments as above).
// ---------------------------------------------------------------------------
template <int C, int D>
struct Fac {
    static constexpr int L = 2 * C, NBL = L / 16, NBC = C / 16, NBD = D / 16;
    static constexpr int KSD = D / 32, KSL = L / 32;
    static constexpr int FR = 1024;                    // one fragment
    // (every factor with a key-channel index carries the scale e^r of that
    // channel, so the state pass works on the unscaled state)
    static constexpr int oWn = 0;                      // -W Diag(e^r)             [NBL][KSD] fragments
    static constexpr int oTv = oWn + NBL * KSD * FR;   // T'                       [NBL] (k = C, zero-padded)
    static constexpr int oKr = oTv + NBL * FR;         // Diag(e^r) Kr^T           [NBD][KSL]
    static constexpr int oQh = oKr + NBD * KSL * FR;   // (Ql - P W) Diag(e^r)     [NBC][KSD]
    static constexpr int oPh = oQh + NBC * KSD * FR;   // P T'                     [NBC] (k = C, zero-padded)
    static constexpr int oDec = oPh + NBC * FR;        // e^{G_C}                  [D] fp32
    static constexpr int bytes = align256(oDec + D * 4);
    static_assert(C == 16 || C == 32, "chunk");
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
    static constexpr int L = 2 * C, NB = L / 16, NT = K1THREADS, NW = K1WAVES;
    static constexpr int LDA = D + 8, LDL = L + 8, ADS = 20, MTW = 24;
    static constexpr int NQ = D / 4;
    static constexpr int TPC = imin(NT / NQ, C);       // threads per channel quad
    static constexpr int TPT = C / TPC;                // tokens per thread
    static constexpr int ACT = NQ * TPC;               // threads with an element-wise role
    static_assert((TPC & (TPC - 1)) == 0 && TPC <= 64 && C % TPC == 0 && ACT <= NT, "split");
    static_assert(TPT == 1 || TPT == 2 || TPT == 4, "token run");
    static_assert(NB <= NW, "one diagonal block per wave");
    // W^T tiles
    static constexpr int NWT = F::NBD * F::NBL;
    // LDS (bytes).  In a wide chunk Kl holds G (fp32 [C][D]) and Kr, Ql the raw
    // keys and queries until the operands are formed.  Once the W tiles are
    // formed, the Kr region stages -W Diag(e^r).
    static constexpr int szKl = align16(L * LDA * 2), szQl = align16(C * LDA * 2);
    static_assert(C * D * 4 <= szKl, "Kl region reuse");
    static constexpr int szLL = align16(L * LDL * 2), szAd = NB * 16 * ADS * 4;
    static constexpr int szMT = NB * 16 * MTW * 2, szPs = align16(C * LDL * 2);
    static constexpr int szMisc = (L + 2 * C + D) * 4 + NW * C * 16 + NW * 4;   // + norm partials, votes
    static constexpr int LDTV = C + 8;                 // T' and P T' staging rows (after the inverse)
    static_assert(L * LDTV * 2 <= szLL && C * LDTV * 2 <= szAd, "staging reuse");
    static constexpr int oKl = 0, oKr = oKl + szKl, oQl = oKr + szKl, oAbf = oQl + szQl;
    static constexpr int oAd = oAbf + szLL, oMI = oAd + szAd, oMT = oMI + szLL, oPs = oMT + szMT;
    static constexpr int oMisc = oPs + szPs;
    static constexpr int LDS = oMisc + szMisc;
    static_assert(LDS <= 80 * 1024, "two workgroups per compute unit");
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
__global__ void __launch_bounds__(K1THREADS) __attribute__((amdgpu_waves_per_eu(2)))
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
    constexpr int ADS = G::ADS, MTW = G::MTW, TPC = G::TPC, TPT = G::TPT;
    constexpr int NWT = G::NWT;
    constexpr int NBD = F::NBD, NBL = F::NBL, NBC = F::NBC, KSD = F::KSD, KSL = F::KSL;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *Kl = (T *)(smem + G::oKl);            // Diag(b') Kl              [L][LDA]
    float *Gs = (float *)(smem + G::oKl);    // wide chunk: G (log2) [C][D]
    T *Kr = (T *)(smem + G::oKr);            // Kr                       [L][LDA]
    T *Wst = Kr;                             // -W Diag(e^r), once A and P are done [L][LDA]
    T *Ql = (T *)(smem + G::oQl);            // Ql                       [C][LDA]
    T *Abf = (T *)(smem + G::oAbf);          // A, off-diagonal 16-blocks [L][LDL]
    float *AdT = (float *)(smem + G::oAd);   // A, diagonal 16-blocks, transposed: [J][p][i] = A_J[i][p]
    T *MI = (T *)(smem + G::oMI);            // (I + A)^{-1}             [L][LDL]
    T *MT = (T *)(smem + G::oMT);            // its diagonal blocks, transposed [NB][16][MTW]
    T *Ps = (T *)(smem + G::oPs);            // P (causal)               [C][LDL]
    float *bp = (float *)(smem + G::oMisc);  // b' per sub-step          [L]
    float *sb = bp + L, *sg = sb + C;        // beta, gamma per token    [C]
    float *ers = sg + C;                     // e^r per channel (1 if wide) [D]
    float *nrm = ers + D;                    // LAYER: per-wave |q|^2, |k|^2, |e|^2 partials [NW][C][4]
    uint32_t *vote = (uint32_t *)(nrm + NW * C * 4);   // LAYER: per-wave wide-chunk votes [NW]
    T *Tvs = (T *)(smem + G::oAbf);          // T', after the inverse    [L][LDTV]
    T *Phs = (T *)(smem + G::oAd);           // P T', after the inverse  [C][LDTV]
    constexpr int LDTV = G::LDTV;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;
    const int grp = H / Hk;                  // value heads per key head
    const float *alpha = (const float *)decay;
    const bf16 *agate = (const bf16 *)decay;
    const int items = BH * NC;

    // The blocks of (I + A)^{-1} above the diagonal are never written: zero
    // them (and the row padding) once.
    for (int idx = tid; idx < L * LDL; idx += NT) {
        const int r = idx / LDL, c = idx % LDL;
        if (c >= L || (c >> 4) > (r >> 4)) MI[idx] = (T)0;
    }

    auto chunk_of = [&](int it) __attribute__((always_inline)) { return NC - 1 - it / BH; };
    auto head_of = [&](int it) __attribute__((always_inline)) { return it % BH; };
    auto is_fast = [&](int cidx) __attribute__((always_inline)) { return VEC && cidx * C + C <= Tlen; };

    // Thread (seg, quad) owns tokens TPT seg .. TPT seg + TPT - 1 of the chunk and
    // key channels c0 .. c0 + 3 for the decay scan and the operand formation; its
    // raw q, e, k (bf16) and alpha (fp32) values stay in registers.
    const bool act = tid < G::ACT;
    const int seg = tid % TPC, c0 = act ? 4 * (tid / TPC) : 0;
    uint2 xq[TPT], xe[TPT], xk[TPT];
    f32x4 xa[TPT];           // alpha (or, LAYER, the gate input a in .x, .y as bf16 pairs)
    f32x4 xA, xB;            // LAYER: A_log, dt_bias of the thread's channels
    float pbeta = 0.f, pgamma = 0.f;

    // ---- full aligned chunk: fetched one item ahead.  Rows are clamped to the
    //      sequence so the same loads are issued for every item and the only
    //      wait on them is where they are first used. -----------------------------
    auto prefetch = [&](int it) __attribute__((always_inline)) {
        const int bh = head_of(it), cidx = chunk_of(it);
        const int b = bh / H, h = bh % H;
        const int t0 = cidx * C, last = Tlen - 1 - t0, hk = h / grp;
        const long tok0 = ((long)b * Tlen + t0) * H + h;       // value-head rows
        const long tokk0 = ((long)b * Tlen + t0) * Hk + hk;    // key-head rows
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const long off = (tokk0 + (long)min(TPT * seg + i, last) * Hk) * dk + c0;
            xq[i] = *(const uint2 *)(q + off);
            xe[i] = *(const uint2 *)(e + off);
            xk[i] = *(const uint2 *)(k + off);
            if constexpr (LAYER) {
                const uint2 u = *(const uint2 *)(agate + off);
                xa[i] = f32x4{__uint_as_float(u.x), __uint_as_float(u.y), 0.f, 0.f};
            } else {
                xa[i] = *(const f32x4 *)(alpha + off);
            }
        }
        if constexpr (LAYER) {
            xA = *(const f32x4 *)(A_log + (long)hk * dk + c0);
            xB = *(const f32x4 *)(dt_bias + (long)hk * dk + c0);
        }
        const long tb = tok0 + (long)min(tid % C, last) * H;
        pbeta = DPLR ? 1.f : beta[tb];
        pgamma = DPLR ? 0.f : gamma[tb];
    };
    // ---- ragged or unaligned chunk: element-wise, zero keys and queries and
    //      alpha = 1 outside the sequence and beyond d_k -----------------------------
    auto fetch_slow = [&](int it) __attribute__((always_inline)) {
        const int bh = head_of(it), cidx = chunk_of(it);
        const int b = bh / H, h = bh % H;
        const int t0 = cidx * C, nval = min(C, Tlen - t0), hk = h / grp;
        const long tok0 = ((long)b * Tlen + t0) * H + h;
        const long tokk0 = ((long)b * Tlen + t0) * Hk + hk;
#pragma unroll
        for (int i = 0; i < TPT; ++i) {
            const int tau = TPT * seg + i;
            float qv[4], ev[4], kv[4], av[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
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
            xq[i] = make_uint2(pack_bf16(qv[0], qv[1]), pack_bf16(qv[2], qv[3]));
            xe[i] = make_uint2(pack_bf16(ev[0], ev[1]), pack_bf16(ev[2], ev[3]));
            xk[i] = make_uint2(pack_bf16(kv[0], kv[1]), pack_bf16(kv[2], kv[3]));
            if constexpr (LAYER)
                xa[i] = f32x4{__uint_as_float(pack_bf16(av[0], av[1])), __uint_as_float(pack_bf16(av[2], av[3])), 0.f, 0.f};
            else
                xa[i] = f32x4{av[0], av[1], av[2], av[3]};
        }
        if constexpr (LAYER) {
            float pa[4], pb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = act && c0 + j < dk;
                pa[j] = ok ? A_log[(long)hk * dk + c0 + j] : 0.f;
                pb[j] = ok ? dt_bias[(long)hk * dk + c0 + j] : 0.f;
            }
            xA = f32x4{pa[0], pa[1], pa[2], pa[3]};
            xB = f32x4{pb[0], pb[1], pb[2], pb[3]};
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
        const int col = lane >> 2, s4 = 4 * (lane & 3);
        f32x4 x;
#pragma unroll
        for (int i = 0; i < 4; ++i) x[i] = (s4 + i == col) ? 1.f : 0.f;
#pragma unroll
        for (int p = 0; p < 15; ++p) {
            const f32x4 a = *(const f32x4 *)(AdT + (J * 16 + p) * ADS + s4);   // A[s4 + i][p]
            const float xs = x[p & 3];
            const float xp = (p >> 2) == 0 ? quad_bcast<0>(xs) : (p >> 2) == 1 ? quad_bcast<1>(xs)
                           : (p >> 2) == 2 ? quad_bcast<2>(xs) : quad_bcast<3>(xs);
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] -= a[i] * xp;
        }
        const uint32_t x01 = pack_bf16(x[0], x[1]), x23 = pack_bf16(x[2], x[3]);
        T *mi = MI + (16 * J + s4) * LDL + 16 * J + col;
        mi[0] = (T)(x01 & 0xffffu);
        mi[LDL] = (T)(x01 >> 16);
        mi[2 * LDL] = (T)(x23 & 0xffffu);
        mi[3 * LDL] = (T)(x23 >> 16);
        *(uint2 *)(MT + (16 * J + col) * MTW + s4) = make_uint2(x01, x23);
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
        for (int i = 0; i < TPT; ++i)
            asm volatile("" ::"v"(xq[i].x), "v"(xq[i].y), "v"(xe[i].x), "v"(xe[i].y), "v"(xk[i].x),
                         "v"(xk[i].y), "v"(xa[i][0]), "v"(xa[i][1]), "v"(xa[i][2]), "v"(xa[i][3]));
        asm volatile("" ::"v"(pbeta), "v"(pgamma));
        if constexpr (LAYER) asm volatile("" ::"v"(xA[0]), "v"(xA[1]), "v"(xA[2]), "v"(xA[3]), "v"(xB[0]),
                                          "v"(xB[1]), "v"(xB[2]), "v"(xB[3]));
    }
    for (; it < items; it += gridDim.x) {
        const int bh = head_of(it), cidx = chunk_of(it);
        if (!is_fast(cidx)) fetch_slow(it);
        if (tid < C) {
            sb[tid] = pbeta;
            sg[tid] = pgamma;
            bp[2 * tid] = pgamma;
            bp[2 * tid + 1] = pbeta;
        }
        char *wsb = ws + ((long)bh * NC + cidx) * F::bytes;

        // ---- cumulative log2-decay per channel: a sequential sum over the
        //      thread's own tokens, then one scan of the run totals over the
        //      TPC threads of the channel quad; wide-chunk vote -----------------------
        float g[TPT][4];
        f32x4 glq;
        bool wide_here = false;
        {
            float run[4] = {0.f, 0.f, 0.f, 0.f};
            f32x4 Ap;
            if constexpr (LAYER) {
#pragma unroll
                for (int j = 0; j < 4; ++j) Ap[j] = exp2f_(xA[j] * L2E) * (L2E / -GATE_FLOOR);
            }
#pragma unroll
            for (int i = 0; i < TPT; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if constexpr (LAYER) {
                        const uint32_t u = __float_as_uint(xa[i][j >> 1]);
                        run[j] += safe_gate_log2((j & 1) ? hi_bf16(u) : lo_bf16(u), Ap[j], xB[j]);
                    } else {
                        run[j] += __builtin_amdgcn_logf(xa[i][j]);
                    }
                    g[i][j] = run[j];
                }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float incl = scan_group<TPC>(run[j], seg);
                const float excl = incl - run[j];
#pragma unroll
                for (int i = 0; i < TPT; ++i) g[i][j] += excl;
                glq[j] = group_last<TPC>(incl);   // G_C of the channel
            }
            if (act && seg == TPC - 1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) wide_here |= glq[j] < -WIDE_G2;
            }
        }
        // LAYER: squared norms of q, k, e per token, summed over the channel
        // quads of a wave here and over the waves after the barrier
        if constexpr (LAYER) {
            constexpr int NWA = (G::ACT + 63) / 64;   // waves with channels
            if (wave < NWA) {
#pragma unroll
                for (int i = 0; i < TPT; ++i) {
                    f32x4 ps = zero4();
                    const uint2 *src[3] = {&xq[i], &xk[i], &xe[i]};
#pragma unroll
                    for (int v = 0; v < 3; ++v) {
                        const uint2 u = *src[v];
                        const float x0 = lo_bf16(u.x), x1 = hi_bf16(u.x), x2 = lo_bf16(u.y), x3 = hi_bf16(u.y);
                        float sq = x0 * x0 + x1 * x1 + x2 * x2 + x3 * x3;
#pragma unroll
                        for (int m = TPC; m < 64; m <<= 1) sq += __shfl_xor(sq, m, 64);
                        ps[v] = sq;
                    }
                    if (lane < TPC) *(f32x4 *)(nrm + (wave * C + TPT * seg + i) * 4) = ps;
                }
            }
        }
        // Wide-chunk vote.  Layer mode: one slot per wave and one barrier (a wave
        // rewrites its slot only at the next item's vote, after barriers of this
        // item that every wave passes once its reads below are done), which
        // spares the mode's registers.  The plain and DPLR modes keep the
        // block-wide OR, measured faster there.
        bool wide = false;
        if constexpr (LAYER) {
            const bool wv = __ballot(wide_here) != 0ull;
            if (lane == 0) vote[wave] = wv ? 1u : 0u;
            __syncthreads();
#pragma unroll
            for (int w = 0; w < NW; ++w) wide |= vote[w] != 0u;
        } else {
            wide = __syncthreads_or(wide_here) != 0;
        }
        // LAYER: 1 / max(|x|, eps) of the thread's token i, for q, k, e (formed
        // where each token is used, so the scales are not held across the loop)
        auto inv_norms = [&](int i) __attribute__((always_inline)) {
            f32x4 tot = zero4();
            if constexpr (LAYER) {
                constexpr int NWA = (G::ACT + 63) / 64;
#pragma unroll
                for (int w = 0; w < NWA; ++w) tot += *(const f32x4 *)(nrm + (w * C + TPT * seg + i) * 4);
                auto inv = [](float ss) { return ss > NORM_EPS * NORM_EPS ? __builtin_amdgcn_rsqf(ss) : 1.f / NORM_EPS; };
                tot = f32x4{inv(tot[0]), inv(tot[1]), inv(tot[2]), 0.f};
            }
            return tot;   // (1/|q|, 1/|k|, 1/|e|)
        };

        // ---- scaled operands (LDS), Diag(e^r) Kr^T (workspace) and the
        //      per-channel scales -------------------------------------------------------
        // Forms Diag(b') Kl, Kr and Ql from the thread's raw values; in a wide
        // chunk the exponents are unsplit (Kl = kap 2^G, Kr = kap 2^{G_C - G}).
        // Diag(e^r) Kr^T = Khat^T in both cases: each thread's run of 2 TPT
        // sub-steps of one channel is one piece of a fragment lane.
        f32x4 er;
#pragma unroll
        for (int j = 0; j < 4; ++j) er[j] = wide ? 1.f : exp2f_(0.5f * glq[j]);
        auto form_operands = [&]() __attribute__((always_inline)) {
            float r[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = wide ? 0.f : 0.5f * glq[j];
            uint32_t kh[4][TPT];   // Khat^T run per channel: (e, k) of each token, packed
#pragma unroll
            for (int i = 0; i < TPT; ++i) {
                const int tau = TPT * seg + i;
                float ev[4] = {lo_bf16(xe[i].x), hi_bf16(xe[i].x), lo_bf16(xe[i].y), hi_bf16(xe[i].y)};
                float kv[4] = {lo_bf16(xk[i].x), hi_bf16(xk[i].x), lo_bf16(xk[i].y), hi_bf16(xk[i].y)};
                float qv[4] = {lo_bf16(xq[i].x), hi_bf16(xq[i].x), lo_bf16(xq[i].y), hi_bf16(xq[i].y)};
                if constexpr (LAYER) {
                    const f32x4 nv = inv_norms(i);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        ev[j] *= nv[2];
                        kv[j] *= nv[1];
                        qv[j] *= nv[0];
                    }
                }
                const float gmt = sg[tau], btt = sb[tau];
                float f[4], fi[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f[j] = exp2f_(g[i][j] - r[j]);
                    fi[j] = wide ? exp2f_(glq[j] - g[i][j]) : exp2f_(r[j] - g[i][j]);
                    const float fh = fi[j] * er[j];
                    kh[j][i] = pack_bf16(DPLR ? 0.f : ev[j] * fh, kv[j] * fh);
                }
                store4<T>(Kl + (2 * tau) * LDA + c0, gmt * ev[0] * f[0], gmt * ev[1] * f[1],
                          gmt * ev[2] * f[2], gmt * ev[3] * f[3]);
                // (DPLR: the delta sub-step reads along a, held in ev; its erase sub-step has no key)
                if constexpr (DPLR)
                    store4<T>(Kl + (2 * tau + 1) * LDA + c0, btt * ev[0] * f[0], btt * ev[1] * f[1],
                              btt * ev[2] * f[2], btt * ev[3] * f[3]);
                else
                    store4<T>(Kl + (2 * tau + 1) * LDA + c0, btt * kv[0] * f[0], btt * kv[1] * f[1],
                              btt * kv[2] * f[2], btt * kv[3] * f[3]);
                if constexpr (DPLR)
                    store4<T>(Kr + (2 * tau) * LDA + c0, 0.f, 0.f, 0.f, 0.f);
                else
                    store4<T>(Kr + (2 * tau) * LDA + c0, ev[0] * fi[0], ev[1] * fi[1], ev[2] * fi[2],
                              ev[3] * fi[3]);
                store4<T>(Kr + (2 * tau + 1) * LDA + c0, kv[0] * fi[0], kv[1] * fi[1], kv[2] * fi[2],
                          kv[3] * fi[3]);
                store4<T>(Ql + tau * LDA + c0, qv[0] * f[0], qv[1] * f[1], qv[2] * f[2], qv[3] * f[3]);
            }
            // fragment (16 x 32 block (n / 16, j0 / 32)), lane 16 ((j0 % 32) / 8) + n % 16, element j0 % 8
            const int j0 = 2 * TPT * seg;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int n = c0 + j;
                char *dst = wsb + F::oKr + (((n >> 4) * KSL + (j0 >> 5)) * 64 + 16 * ((j0 & 31) >> 3) + (n & 15)) * 16 +
                            2 * (j0 & 7);
                if constexpr (TPT == 4) *(uint4 *)dst = make_uint4(kh[j][0], kh[j][1], kh[j][2], kh[j][3]);
                else if constexpr (TPT == 2) *(uint2 *)dst = make_uint2(kh[j][0], kh[j][1]);
                else *(uint32_t *)dst = kh[j][0];
            }
        };
        if (act) {
            if (seg == 0) {
                f32x4 dec;
#pragma unroll
                for (int j = 0; j < 4; ++j) dec[j] = exp2f_(glq[j]);
                *(f32x4 *)(ers + c0) = er;
                *(f32x4 *)(wsb + F::oDec + 4 * c0) = dec;
            }
            if (!wide) {
                form_operands();
            } else {
                // raw keys and queries, and G, for the element-wise path
#pragma unroll
                for (int i = 0; i < TPT; ++i) {
                    const int tau = TPT * seg + i;
                    auto nz = [&](uint2 u, float s) __attribute__((always_inline)) {
                        if constexpr (!LAYER) return u;
                        return make_uint2(pack_bf16(lo_bf16(u.x) * s, hi_bf16(u.x) * s),
                                          pack_bf16(lo_bf16(u.y) * s, hi_bf16(u.y) * s));
                    };
                    const f32x4 nv = inv_norms(i);
                    *(uint2 *)(Kr + (2 * tau) * LDA + c0) = nz(xe[i], nv[2]);
                    *(uint2 *)(Kr + (2 * tau + 1) * LDA + c0) = nz(xk[i], nv[1]);
                    *(uint2 *)(Ql + tau * LDA + c0) = nz(xq[i], nv[0]);
                    *(f32x4 *)(Gs + tau * D + c0) = f32x4{g[i][0], g[i][1], g[i][2], g[i][3]};
                }
            }
        }
        __syncthreads();

        // ---- A (strictly lower) and P (causal); diagonal blocks inverted ----------
        constexpr int NOD = NB * (NB - 1) / 2;
        constexpr int NPT = NB * (C / 16);
        if (!wide) {
            if (wave < NB) {
                const int J = wave;
                const f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * J * LDA, LDA, zero4(), lane);
                // lane holds A[g4 + rr][l16]: one column run of the transposed block
                *(f32x4 *)(AdT + (J * 16 + l16) * ADS + g4) =
                    f32x4{g4 > l16 ? a[0] : 0.f, g4 + 1 > l16 ? a[1] : 0.f, g4 + 2 > l16 ? a[2] : 0.f,
                          g4 + 3 > l16 ? a[3] : 0.f};
                wave_lds_sync();
                invert_diag(J);
            }
            // off-diagonal A and P tiles, spread over every wave
            for (int t = (wave + NW - NB) % NW; t < NOD + NPT; t += NW) {
                if (t < NOD) {
                    int J = 1, I = t;
                    while (I >= J) { I -= J; ++J; }
                    const f32x4 a = tile_nt<T, D>(Kl + 16 * J * LDA, LDA, Kr + 16 * I * LDA, LDA, zero4(), lane);
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        Abf[(16 * J + g4 + rr) * LDL + 16 * I + l16] = from_f32<T>(a[rr]);
                } else {
                    // P^T tile: rows = sub-steps i, cols = tokens; kept for i <= 2 tau + 1
                    const int I = (t - NOD) / (C / 16), Tb = (t - NOD) % (C / 16);
                    const int tau = 16 * Tb + l16, i0 = 16 * I + g4;
                    float w4[4] = {0.f, 0.f, 0.f, 0.f};
                    if (16 * I <= 32 * Tb + 31) {   // else beyond every token's causal range
                        const f32x4 a = tile_nt<T, D>(Kr + 16 * I * LDA, LDA, Ql + 16 * Tb * LDA, LDA, zero4(), lane);
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) w4[rr] = (i0 + rr <= 2 * tau + 1) ? a[rr] : 0.f;
                    }
                    store4<T>(Ps + tau * LDL + i0, w4[0], w4[1], w4[2], w4[3]);
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
                else if (ii < j) Abf[j * LDL + ii] = from_f32<T>(s);
            }
            for (int idx = tid; idx < C * L; idx += NT) {
                const int tau = idx / L, ii = idx % L;
                float s = 0.f;
                if (ii <= 2 * tau + 1 && (!DPLR || (ii & 1))) {
                    const int ti = ii >> 1;
#pragma unroll 2
                    for (int cc = 0; cc < D; ++cc)
                        s += to_f32(Ql[tau * LDA + cc]) * to_f32(Kr[ii * LDA + cc]) *
                             exp2f_(Gs[tau * D + cc] - Gs[ti * D + cc]);
                }
                Ps[tau * LDL + ii] = from_f32<T>(s);
            }
            __syncthreads();
            if (wave < NB) invert_diag(wave);
            // every read of G and of the raw keys is done: form the operands in place
            if (act) form_operands();
        }
        __syncthreads();

        // the next item's raw values: fetched now, first used by the next item's
        // scan (the current item's raw registers are dead once the operands exist)
        if constexpr (VEC) {
            const int nx = it + gridDim.x;
            prefetch(nx < items ? nx : items - 1);
        }

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
                    t = mma16(a, xb[K], t);
                }
                const s16x4 tb = __builtin_bit_cast(s16x4, make_uint2(pack_bf16(t[0], t[1]), pack_bf16(t[2], t[3])));
                const s16x4 m = *(const s16x4 *)(MI + (16 * J + l16) * LDL + 16 * J + g4);
                const f32x4 x = mma16(m, tb, zero4());
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

        // T'[j][tau] = M[j][2 tau + 1] beta_tau (tau >= C: zero): row block rb -> workspace and LDS
        auto export_tv = [&](int rb) __attribute__((always_inline)) {
            const int gg = lane >> 4;
            const T *mrow = MI + (16 * rb + l16) * LDL;
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (8 * gg < C) {
                const uint4 u0 = *(const uint4 *)(mrow + 16 * gg);
                const uint4 u1 = *(const uint4 *)(mrow + 16 * gg + 8);
                const f32x4 b0 = *(const f32x4 *)(sb + 8 * gg), b1 = *(const f32x4 *)(sb + 8 * gg + 4);
                x = make_uint4(pack_bf16(hi_bf16(u0.x) * b0[0], hi_bf16(u0.y) * b0[1]),
                               pack_bf16(hi_bf16(u0.z) * b0[2], hi_bf16(u0.w) * b0[3]),
                               pack_bf16(hi_bf16(u1.x) * b1[0], hi_bf16(u1.y) * b1[1]),
                               pack_bf16(hi_bf16(u1.z) * b1[2], hi_bf16(u1.w) * b1[3]));
                *(uint4 *)(Tvs + (16 * rb + l16) * LDTV + 8 * gg) = x;
            }
            *(uint4 *)(wsb + F::oTv + (rb * 64 + lane) * 16) = x;
        };
        // W^T tile (channel block nb, sub-step block jb) = Kl^T Diag(b') M^T, staged
        // as -W Diag(e^r) in the Kr region (Kr was last read by the A and P tiles)
        auto w_tile = [&](int jb, int nb) __attribute__((always_inline)) {
            // M's row block jb is zero beyond column 16 (jb + 1); round up to 32
            const int K = 32 * ((jb + 2) / 2);
            f32x4 acc = zero4();
            for (int k0 = 0; k0 < K; k0 += 32)
                acc = mma32(frag_col(Kl + k0 * LDA + 16 * nb, LDA, lane),
                            frag_row(MI + 16 * jb * LDL + k0, LDL, lane), acc);
            // lane holds W[16 jb + l16][16 nb + g4 + i]
            const f32x4 es = *(const f32x4 *)(ers + 16 * nb + g4);
            store4<T>(Wst + (16 * jb + l16) * LDA + 16 * nb + g4, -acc[0] * es[0], -acc[1] * es[1],
                      -acc[2] * es[2], -acc[3] * es[3]);
        };
        // Q^T tile (channels 16 nb.., tokens 16 tb..) = ((Ql - P W) Diag(e^r))^T, in
        // place over Ql; P is zero beyond sub-step 2t + 1
        auto qh_tile = [&](int nb, int tb) __attribute__((always_inline)) {
            const uint2 q0 = *(const uint2 *)(Ql + (16 * tb + l16) * LDA + 16 * nb + g4);
            const f32x4 es = *(const f32x4 *)(ers + 16 * nb + g4);
            f32x4 acc = {lo_bf16(q0.x) * es[0], hi_bf16(q0.x) * es[1], lo_bf16(q0.y) * es[2],
                         hi_bf16(q0.y) * es[3]};
            const int K = imin(L, 32 * (tb + 1));
            for (int k0 = 0; k0 < K; k0 += 32)
                acc = mma32(frag_col(Wst + k0 * LDA + 16 * nb, LDA, lane),
                            frag_row(Ps + 16 * tb * LDL + k0, LDL, lane), acc);
            store4<T>(Ql + (16 * tb + l16) * LDA + 16 * nb + g4, acc[0], acc[1], acc[2], acc[3]);
        };
        // P^ ^T tile (tokens tau 16 nb.., tokens t 16 tb..) = (P T')^T, staged
        auto ph_tile = [&](int nb, int tb) __attribute__((always_inline)) {
            f32x4 acc = zero4();
            const int K = imin(L, 32 * (tb + 1));
            for (int k0 = 0; k0 < K; k0 += 32)
                acc = mma32(frag_col(Tvs + k0 * LDTV + 16 * nb, LDTV, lane),
                            frag_row(Ps + 16 * tb * LDL + k0, LDL, lane), acc);
            store4<T>(Phs + (16 * tb + l16) * LDTV + 16 * nb + g4, acc[0], acc[1], acc[2], acc[3]);
        };
        auto export_ph = [&](int rb) __attribute__((always_inline)) {
            uint4 x = make_uint4(0u, 0u, 0u, 0u);
            if (8 * (lane >> 4) < C) x = __builtin_bit_cast(uint4, frag_row(Phs + 16 * rb * LDTV, LDTV, lane));
            *(uint4 *)(wsb + F::oPh + (rb * 64 + lane) * 16) = x;
        };

        if constexpr (NBD == 2 * NW) {
            // ---- wave-local exports: wave w owns channels 32 w .. 32 w + 31 (one
            //      fragment column): its W tiles, -W fragments, Q^ tiles and Q^
            //      fragments need no other wave's results, so no barrier; wave 0
            //      also forms T' and P^ = P T' ----------------------------------------------
            const int ks = wave;
            for (int jb = 0; jb < NBL; ++jb) {
                w_tile(jb, 2 * wave);
                w_tile(jb, 2 * wave + 1);
            }
            if (wave == 0)
                for (int rb = 0; rb < NBL; ++rb) export_tv(rb);
            wave_lds_sync();
            for (int rb = 0; rb < NBL; ++rb)
                st_frag(wsb + F::oWn + ((rb * KSD + ks) * 64 + lane) * 16,
                        frag_row(Wst + 16 * rb * LDA + 32 * ks, LDA, lane));
            for (int tb = 0; tb < NBC; ++tb) {
                qh_tile(2 * wave, tb);
                qh_tile(2 * wave + 1, tb);
            }
            if (wave == 0)
                for (int t = 0; t < NBC * NBC; ++t) ph_tile(t % NBC, t / NBC);
            wave_lds_sync();
            for (int tb = 0; tb < NBC; ++tb)
                st_frag(wsb + F::oQh + ((tb * KSD + ks) * 64 + lane) * 16,
                        frag_row(Ql + 16 * tb * LDA + 32 * ks, LDA, lane));
            if (wave == 0)
                for (int rb = 0; rb < NBC; ++rb) export_ph(rb);
        } else {
            // ---- W tiles and T' over all waves; barrier; -W fragments, Q^ and P^
            //      tiles; barrier; Q^ and P^ fragments ------------------------------------
            for (int t = wave; t < NWT; t += NW) w_tile(t / NBD, t % NBD);
            for (int rb = wave; rb < NBL; rb += NW) export_tv(rb);
            __syncthreads();
            constexpr int NWF = NBL * KSD, NQT = NBD * NBC, NPT2 = NBC * NBC;
            for (int f = wave; f < NWF + NQT + NPT2; f += NW) {
                if (f < NWF) {
                    const int rb = f / KSD, ks = f % KSD;
                    st_frag(wsb + F::oWn + (f * 64 + lane) * 16, frag_row(Wst + 16 * rb * LDA + 32 * ks, LDA, lane));
                } else if (f < NWF + NQT) {
                    const int t = f - NWF;
                    qh_tile(t % NBD, t / NBD);
                } else {
                    const int t = f - NWF - NQT;
                    ph_tile(t % NBC, t / NBC);
                }
            }
            __syncthreads();
            constexpr int NQF = NBC * KSD;
            for (int f = wave; f < NQF + NBC; f += NW) {
                if (f < NQF) {
                    const int rb = f / KSD, ks = f % KSD;
                    st_frag(wsb + F::oQh + (f * 64 + lane) * 16, frag_row(Ql + 16 * rb * LDA + 32 * ks, LDA, lane));
                } else {
                    export_ph(f - NQF);
                }
            }
        }
        // No barrier here: the exports above read only Wst, Ql, Tvs, Phs, Ps, MI,
        // ers and sb, and the next item first writes any of those after its
        // wide-chunk vote, which every wave reaches only after finishing its own
        // exports; before the vote it writes only b', beta and gamma (by wave 0,
        // after its own reads of sb) and the norm partials, which nothing above
        // reads.
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state pass.  One workgroup per (head, BV-column slice); the
// slices of one head get workgroup ids congruent mod 8 (same XCD, one L2 for
// the shared factor blocks).
//
// Every wave has one role, and each role fetches the operands it needs two
// chunks ahead during the half of the chunk in which it has nothing else to
// do, so the vector-memory traffic of the factors overlaps the products:
//   U waves   (L/16):  U = T' V - W S for 16 rows of U, all slice columns;
//                      fetch -W, T' while the state is updated
//   state     (D/16):  S <- e^{G_C} S + Kr^T U for 16 state rows, then S^T
//                      (bf16) for the next chunk; fetch Kr^T while U is formed
//   output    (C/16):  o = Q^ S + P^ V for 16 tokens (transposed, so rows of o
//                      leave as runs), Q^ = Ql - P W, P^ = P T'; fetch them
//                      while the state is updated
//   movers:            value slice and per-row decay in, outputs out.
// (W, Kr^T and Q^ carry the per-channel e^r of the split, so S is unscaled.)
// ---------------------------------------------------------------------------
template <int C, int D, int BV>
struct K2G {
    using F = Fac<C, D>;
    static constexpr int L = 2 * C;
    static constexpr int NBL = F::NBL, NBC = F::NBC, NBD = F::NBD, NCB = BV / 16;
    static constexpr int KSD = F::KSD, KSL = F::KSL;
    static constexpr int NR = KSD + KSL;               // role operands per chunk
    static constexpr int VU = C * BV / 8;              // 16-byte units of a value (or output) slice
    static constexpr int SCU = D / 2;                  // 8-byte units of a chunk's decay e^{G_C}
    static constexpr int NM = imax((VU + 63) / 64, (SCU + 63) / 64);
    // wave order: U, state, output, movers
    static constexpr int S0W = NBL, O0 = S0W + NBD, M0 = O0 + NBC, NW = M0 + NM, NT = 64 * NW;
    static_assert(NT <= 1024, "workgroup size");
    static constexpr int LDT = D + 8, LDU = L + 8, LDV = BV + 8, LDO = BV + 8;
    static constexpr int oSt = 0;                                   // S'^T [BV][LDT] bf16
    static constexpr int oUt = align16(oSt + BV * LDT * 2);         // U^T  [BV][LDU] bf16
    static constexpr int VR = 32;                                   // value rows (>= C; rows >= C stay zero)
    static constexpr int szVs = align16(VR * LDV * 2);
    static constexpr int oVs = align16(oUt + BV * LDU * 2);         // V    [2][VR][LDV] bf16
    static constexpr int oOs = oVs + 2 * szVs;                      // o    [C][LDO] bf16
    static constexpr int oSc = align16(oOs + C * LDO * 2);          // e^{G_C} [2][D] fp32
    static constexpr int LDS = oSc + 2 * 4 * D;
};

template <int NR, int KSL>
struct FragSet {
    bf16x8 R[NR];   // role operands: -W and T' (U), Q^ and P^ (output), Kr^T (state), v (movers)
    uint2 sc;       // movers: one 8-byte piece of the chunk's decay
    uint32_t pf[2]; // movers: one word of each of this slice's lines of a later chunk's block
};

// L2 warm-up of the state pass (when the workspace exceeds the MALL): while
// fetching chunk c's operands, the mover wave of slice j also reads one word
// of every R-th 128-byte line (j, j + R, ...) of chunk c + WARM_AHEAD's block,
// so the R slices of a head (same XCD, one L2) together bring that block into
// L2 before its fragments are fetched, at 1/R of a block of extra traffic per
// compute unit.  The words are consumed, unused, when the chunk's set is.
constexpr int WARM_AHEAD = 4;
constexpr size_t WARM_MIN_BYTES = (size_t)256 << 20;   // MI355X MALL capacity

// VV: every value slice is whole (d_v a multiple of BV) and v is 16-byte
// aligned, so values and outputs move as 16-byte row pieces.
template <int C, int D, int BV, bool VV>
__global__ void __launch_bounds__((K2G<C, D, BV>::NT))
eda_bf16_state(const bf16 *__restrict__ v, const float *S0, float *S_final, bf16 *__restrict__ o,
               const char *__restrict__ ws, int Tlen, int H, int BH, int dk, int dv, int NC, int R,
               int warm) {
    using G = K2G<C, D, BV>;
    using F = Fac<C, D>;
    using T = bf16;
    constexpr int NCB = G::NCB, KSD = G::KSD, KSL = G::KSL, LDT = G::LDT, LDU = G::LDU;
    constexpr int LDV = G::LDV, LDO = G::LDO, VU = G::VU, O0 = G::O0, S0W = G::S0W, M0 = G::M0;
    extern __shared__ __attribute__((aligned(16))) char smem[];
    T *St = (T *)(smem + G::oSt);
    T *Ut = (T *)(smem + G::oUt);
    T *Os = (T *)(smem + G::oOs);

    const int w = blockIdx.x, xcd = w & 7, slot = w >> 3;
    const int bh = (slot / R) * 8 + xcd, slice = slot % R;
    if (bh >= BH) return;
    const int b = bh / H, h = bh % H, n0 = slice * BV;
    const long sbase = (long)bh * dk * dv;
    const long hrow = (long)b * Tlen * H + h;
    const long HV = (long)H * dv;
    const T *vh = v + hrow * dv + n0;
    T *oh = o + hrow * dv + n0;
    const char *wsh = ws + (long)bh * NC * F::bytes;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g4 = 4 * (lane >> 4), l16 = lane & 15;

    if constexpr (C < G::VR) {
        // the value rows beyond the chunk are read by the k = 32 product: zero them
        for (int idx = tid; idx < 2 * (G::VR - C) * LDV; idx += G::NT) {
            const int bsel = idx / ((G::VR - C) * LDV), rem = idx % ((G::VR - C) * LDV);
            ((T *)(smem + G::oVs + bsel * G::szVs))[C * LDV + rem] = (T)0;
        }
    }

    // One chunk loop per role: straight-line code with a fixed number of
    // memory operations per chunk, so the waits before each use only cover
    // operands fetched three chunks earlier (chunk indices clamped, never
    // skipped).
    auto run = [&](auto role) __attribute__((always_inline)) {
        constexpr int RL = decltype(role)::value;   // 0 U, 1 state, 2 output, 3 mover
        constexpr bool RU = RL == 0, RS = RL == 1, RO = RL == 2, RM = RL == 3;
        using Set = FragSet<G::NR, KSL>;
        const int rb = RU ? wave : (RS ? wave - S0W : (RO ? wave - O0 : 0));   // row block of the role
        const int mu = (wave - M0) * 64 + lane;                                 // mover unit
        const bool mact = RM && mu < VU;
        const int muc = mact ? mu : 0;
        const int mtau = muc / (BV / 8), mn = 8 * (muc % (BV / 8));

        auto load = [&](Set &s, int c) __attribute__((always_inline)) {
            const char *blk = wsh + (long)c * F::bytes;
            if constexpr (RU) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    s.R[ks] = ld_frag(blk + F::oWn + ((rb * KSD + ks) * 64 + lane) * 16);
                s.R[KSD] = ld_frag(blk + F::oTv + (rb * 64 + lane) * 16);
            }
            if constexpr (RS) {
#pragma unroll
                for (int ks = 0; ks < KSL; ++ks)
                    s.R[ks] = ld_frag(blk + F::oKr + ((rb * KSL + ks) * 64 + lane) * 16);
            }
            if constexpr (RO) {
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
                    s.R[ks] = ld_frag(blk + F::oQh + ((rb * KSD + ks) * 64 + lane) * 16);
                s.R[KSD] = ld_frag(blk + F::oPh + (rb * 64 + lane) * 16);
            }
            if constexpr (RM) {
                const int t = c * C + mtau, tc = t < Tlen ? t : Tlen - 1;
                const bool ok = mact && t < Tlen;
                uint4 x;
                if constexpr (VV) {
                    x = *(const uint4 *)(vh + tc * HV + mn);
                } else {
                    uint32_t y[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int col = mn + j, cc = n0 + col < dv ? col : dv - 1 - n0;
                        y[j] = vh[tc * HV + cc];
                        if (n0 + col >= dv) y[j] = 0u;
                    }
                    x = make_uint4(y[0] | (y[1] << 16), y[2] | (y[3] << 16), y[4] | (y[5] << 16), y[6] | (y[7] << 16));
                }
                if (!ok) x = make_uint4(0u, 0u, 0u, 0u);
                s.R[0] = __builtin_bit_cast(bf16x8, x);
                s.sc = *(const uint2 *)(blk + F::oDec + 8 * (mu < G::SCU ? mu : G::SCU - 1));
                s.pf[0] = s.pf[1] = 0u;
                if (warm) {
                    const int cw = c + WARM_AHEAD < NC ? c + WARM_AHEAD : NC - 1;
                    const char *wb = wsh + (long)cw * F::bytes;
#pragma unroll
                    for (int i = 0; i < 2; ++i) {
                        const int off = (slice + R * (64 * i + lane)) * 128;   // beyond the block: its last word
                        s.pf[i] = *(const uint32_t *)(wb + (off < F::bytes - 4 ? off : F::bytes - 4));
                    }
                }
            }
        };
        // movers: value slice and scales of chunk c -> LDS
        auto put_v = [&](const Set &s, int c) __attribute__((always_inline)) {
            if (mact)
                *(uint4 *)((T *)(smem + G::oVs + (c & 1) * G::szVs) + mtau * LDV + mn) = __builtin_bit_cast(uint4, s.R[0]);
            if (mu < G::SCU) *(uint2 *)(smem + G::oSc + (c & 1) * 4 * D + 8 * mu) = s.sc;
        };
        auto flush = [&](int cp) __attribute__((always_inline)) {
            const int t = cp * C + mtau;
            if (mact && t < Tlen) {
                const uint4 val = *(const uint4 *)(Os + mtau * LDO + mn);
                T *dst = oh + t * HV + mn;
                if constexpr (VV) {
                    *(uint4 *)dst = val;
                } else {
                    const uint32_t y[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        if (n0 + mn + j < dv) dst[j] = (T)((y[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                }
            }
        };
        auto decay = [&](int c) __attribute__((always_inline)) {
            return *(const f32x4 *)(smem + G::oSc + (c & 1) * 4 * D + 4 * (16 * rb + g4));
        };

        // state rows 16 rb + g4 + i, columns n0 + 16 cb + l16 (state role)
        f32x4 S[NCB];
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) {
            S[cb] = zero4();
            if (RS && S0) {
                const int col = n0 + 16 * cb + l16;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int row = 16 * rb + g4 + i;
                    if (row < dk && col < dv) S[cb][i] = S0[sbase + (long)row * dv + col];
                }
            }
        }
        auto write_St = [&]() __attribute__((always_inline)) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb)
                store4<T>(St + (16 * cb + l16) * LDT + 16 * rb + g4, S[cb][0], S[cb][1], S[cb][2], S[cb][3]);
        };

        // T'V (U role) and P^V (output role) of the next chunk, formed during the
        // half of this chunk in which those roles wait, so that their chains on
        // the next chunk start from it
        f32x4 pre[NCB];
        auto body = [&](Set &cur, Set &nxt, Set &far, int c) __attribute__((always_inline)) {
            const int cf = c + 3 < NC ? c + 3 : NC - 1;   // chunk whose operands are fetched now
            __syncthreads();   // S^T, the value slice of chunk c and its decay are in LDS
            f32x4 acc[NCB];
            const T *Vs = (const T *)(smem + G::oVs + (c & 1) * G::szVs);
            if constexpr (RU) {
                // U = T' V - W S  (16 rows, all slice columns) -> U^T in LDS
                // (one instruction shape for the whole accumulation chain: at C = 16
                // the k = 32 product reads 16 zero rows of the value buffer).  All
                // LDS operands are read before the first product, so the chain pays
                // one LDS latency instead of one per step.
                bf16x8 sf[KSD][NCB];
                if (c == 0) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) pre[cb] = mma32(cur.R[KSD], frag_col(Vs + 16 * cb, LDV, lane), zero4());
                }
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) sf[ks][cb] = frag_row(St + 16 * cb * LDT + 32 * ks, LDT, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[cb] = pre[cb];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(cur.R[ks], sf[ks][cb], acc[cb]);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    store4<T>(Ut + (16 * cb + l16) * LDU + 16 * rb + g4, acc[cb][0], acc[cb][1], acc[cb][2],
                              acc[cb][3]);
            }
            if constexpr (RS) load(far, cf);
            if constexpr (RO) {
                // o^T = S^T Q^^T + V^T P^^T for the wave's 16 tokens -> rows of o in LDS
                bf16x8 sf[KSD][NCB];
                if (c == 0) {
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) pre[cb] = mma32(frag_col(Vs + 16 * cb, LDV, lane), cur.R[KSD], zero4());
                }
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) sf[ks][cb] = frag_row(St + 16 * cb * LDT + 32 * ks, LDT, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[cb] = pre[cb];
#pragma unroll
                for (int ks = 0; ks < KSD; ++ks)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[cb] = mma32(sf[ks][cb], cur.R[ks], acc[cb]);
                const int tr = 16 * rb + l16;
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb)
                    store4<T>(Os + tr * LDO + 16 * cb + g4, acc[cb][0], acc[cb][1], acc[cb][2], acc[cb][3]);
            }
            if constexpr (RM) {
                if (c + 1 < NC) put_v(nxt, c + 1);
                asm volatile("" ::"v"(cur.pf[0]), "v"(cur.pf[1]));   // the warm-up words, consumed
                load(far, cf);
            }
            __syncthreads();   // U^T and the outputs complete; S^T no longer read
            if constexpr (RU || RO) {
                load(far, cf);
                // the next chunk's value slice is in LDS (written by the movers before
                // the barrier above, into the other buffer)
                if (c + 1 < NC) {
                    const T *Vn = (const T *)(smem + G::oVs + ((c + 1) & 1) * G::szVs);
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) {
                        const bf16x8 vn = frag_col(Vn + 16 * cb, LDV, lane);
                        pre[cb] = RU ? mma32(nxt.R[KSD], vn, zero4()) : mma32(vn, nxt.R[KSD], zero4());
                    }
                }
            }
            if constexpr (RS) {
                // S <- e^{G_C} S + Kr^T U; S^T of the next chunk
                const f32x4 dc = decay(c);
                bf16x8 uf[KSL][NCB];
#pragma unroll
                for (int ks = 0; ks < KSL; ++ks)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) uf[ks][cb] = frag_row(Ut + 16 * cb * LDU + 32 * ks, LDU, lane);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    f32x4 a;
#pragma unroll
                    for (int i = 0; i < 4; ++i) a[i] = dc[i] * S[cb][i];
#pragma unroll
                    for (int ks = 0; ks < KSL; ++ks) a = mma32(cur.R[ks], uf[ks][cb], a);
                    S[cb] = a;
                }
                if (c + 1 < NC) write_St();
            }
            // stores last: nothing after them waits on the vector-memory counter
            if constexpr (RM) flush(c);
        };

        // four operand sets in rotation: the chunk in use, the next two, and
        // the one being fetched
        Set A, B, X, Y;
        load(A, 0);
        load(B, NC > 1 ? 1 : 0);
        load(X, NC > 2 ? 2 : NC - 1);
        if constexpr (RM) put_v(A, 0);
        if constexpr (RS) write_St();
        int c = 0;
        for (; c + 4 <= NC; c += 4) {
            body(A, B, Y, c);
            body(B, X, A, c + 1);
            body(X, Y, B, c + 2);
            body(Y, A, X, c + 3);
        }
        if (c < NC) body(A, B, Y, c);
        if (c + 1 < NC) body(B, X, A, c + 1);
        if (c + 2 < NC) body(X, Y, B, c + 2);

        if constexpr (RS) {
            if (S_final) {
                // every read of S0 happened before the chunk loop, so S_final may be S0
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) {
                    const int col = n0 + 16 * cb + l16;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int row = 16 * rb + g4 + i;
                        if (row < dk && col < dv) S_final[sbase + (long)row * dv + col] = S[cb][i];
                    }
                }
            }
        }
    };

    if (wave < S0W) run(std::integral_constant<int, 0>{});
    else if (wave < O0) run(std::integral_constant<int, 1>{});
    else if (wave < M0) run(std::integral_constant<int, 2>{});
    else run(std::integral_constant<int, 3>{});
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
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
    return (size_t)B * H * ((Tlen + C - 1) / C) * Fac<C, D>::bytes;
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
    auto k2 = vv ? eda_bf16_state<C, D, BV, true> : eda_bf16_state<C, D, BV, false>;
    hipError_t err = hipFuncSetAttribute((const void *)k1, hipFuncAttributeMaxDynamicSharedMemorySize, G1::LDS);
    if (err != hipSuccess) return err;
    int dev = 0, ncu = 256;
    err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    err = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const long items = (long)BH * NC;
    const int grid1 = (int)(items < 2L * ncu ? items : 2L * ncu);   // two per compute unit (LDS)
    if (ev && (err = hipEventRecord(ev[0], stream)) != hipSuccess) return err;
    hipLaunchKernelGGL(k1, dim3((unsigned)grid1), dim3(G1::NT), G1::LDS, stream, (const bf16 *)q,
                       (const bf16 *)k, (const bf16 *)e, decay, A_log, dt_bias, beta, gamma, (char *)ws,
                       Tlen, H, Hk, dk, NC, BH);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (ev && (err = hipEventRecord(ev[1], stream)) != hipSuccess) return err;
    const int R = (dv + BV - 1) / BV;
    const int grid2 = 8 * ((BH + 7) / 8) * R;
    const int warm = ws_bytes<C, D>(B, Tlen, H) > WARM_MIN_BYTES;
    hipLaunchKernelGGL(k2, dim3((unsigned)grid2), dim3(G2::NT), G2::LDS, stream, (const bf16 *)v, S0,
                       S_final, (bf16 *)o, (const char *)ws, Tlen, H, BH, dk, dv, NC, R, warm);
    err = hipGetLastError();
    if (err == hipSuccess && ev) err = hipEventRecord(ev[2], stream);
    return err;
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

// decay: alpha (fp32), or with A_log != NULL the safe gate's input a (bf16)
// of Hk key heads (the fused layer prologue); otherwise Hk == H.  beta ==
// NULL selects the rank-1 DPLR update, with its erase vector a in `e`.
hipError_t launch_bf16(const void *q, const void *k, const void *e, const void *v, const void *decay,
                       const float *A_log, const float *dt_bias, const float *beta, const float *gamma,
                       const float *S0, void *o, float *S_final, int B, int Tlen, int H, int Hk, int dk,
                       int dv, int chunk, void *ws, hipStream_t stream, hipEvent_t const *ev) {
    const int D = b16::pad_dim(dk, dv), BV = b16::slice_width(B * H, D);
#define EDA_GO(CC, DD, BB)                                                                          \
    if (chunk == CC && D == DD && BV == BB)                                                         \
        return b16::launch_t<CC, DD, BB>(q, k, e, v, decay, A_log, dt_bias, beta, gamma, S0, o,     \
                                         S_final, B, Tlen, H, Hk, dk, dv, ws, stream, ev);
    EDA_GO(16, 32, 16) EDA_GO(16, 32, 32) EDA_GO(16, 64, 16) EDA_GO(16, 64, 32)
    EDA_GO(16, 128, 16) EDA_GO(16, 128, 32)
    EDA_GO(32, 32, 16) EDA_GO(32, 32, 32) EDA_GO(32, 64, 16) EDA_GO(32, 64, 32)
    EDA_GO(32, 128, 16) EDA_GO(32, 128, 32)
#undef EDA_GO
    return hipErrorInvalidValue;
}

}  // namespace eda
