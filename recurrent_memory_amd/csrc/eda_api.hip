// eda_api.hip -- the C ABI declared in include/eda.h: argument checks, then
// kernel launches.  Every check runs before anything is enqueued.
#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/eda.h"
#include "eda_common.h"

// Workspace of eda_fwd_chunked_noalloc: one array per device, loaded with the
// library's code object and held until the process ends.  In host code its
// name is a stand-in, not a device address: the address is looked up once per
// device with hipGetSymbolAddress and only that address is used.
static __device__ __align__(256) char scratch[EDA_NOALLOC_SCRATCH_BYTES];

namespace eda {
template <typename Tin>
hipError_t launch_decode(const void *, const void *, const void *, const void *, const void *,
                         const float *, const float *, const float *, const float *, const float *,
                         float *, void *, int, int, int, int, int, hipStream_t);
template <typename Tin>
hipError_t launch_layer_prep(const void *, const void *, const void *, const void *, const float *,
                             const float *, float *, float *, float *, float *, int, int, int, int,
                             int, hipStream_t);
template <typename T>
size_t chunked_ws_t(int, int, int, int, int, int);
template <typename T>
hipError_t launch_chunked(int, const void *, const void *, const void *, const void *,
                          const float *, const float *, const float *, const float *, void *,
                          float *, int, int, int, int, int, int, void *, hipStream_t,
                          hipEvent_t const *);
size_t bf16_ws_bytes(int, int, int, int, int, int);
size_t bwd_ws_bytes(int, int, int, int, int);
template <typename Tin>
hipError_t launch_bwd(const void *, const void *, const void *, const void *, const float *, const float *,
                      const float *, const float *, const void *, const float *, float *, float *, float *,
                      float *, float *, float *, float *, float *, int, int, int, int, int, void *,
                      hipStream_t);
hipError_t launch_bf16(const void *, const void *, const void *, const void *, const void *,
                       const float *, const float *, const float *, const float *, const float *,
                       void *, float *, int, int, int, int, int, int, int, void *, hipStream_t,
                       hipEvent_t const *);
}  // namespace eda

namespace {

constexpr int kDefaultChunk = 64;

struct Range {
    uintptr_t lo, hi;  // [lo, hi)
    bool set;
};

Range range_of(const void *p, size_t bytes) {
    Range r;
    r.lo = (uintptr_t)p;
    r.hi = r.lo + bytes;
    r.set = p != nullptr && bytes > 0;
    return r;
}

bool overlap(const Range &a, const Range &b) { return a.set && b.set && a.lo < b.hi && b.lo < a.hi; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

size_t elem_size(eda_dtype_t dt) { return dt == EDA_BF16 ? 2 : 4; }

bool dtype_ok(eda_dtype_t dt) { return dt == EDA_F32 || dt == EDA_BF16; }

bool dims_ok(long a, long b, long c, int dk, int dv) {
    if (a <= 0 || b <= 0 || c <= 0 || dk <= 0 || dv <= 0) return false;
    const long dmax = dk > dv ? dk : dv;
    return a * b * c * dmax < (1L << 31);
}

bool head_dims_supported(int dk, int dv) { return dk >= 1 && dk <= 128 && dv >= 1 && dv <= 128; }

int resolve_chunk(int chunk) { return chunk == 0 ? kDefaultChunk : chunk; }

bool chunk_supported(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64; }

// Device address of `scratch` on the current device, looked up on the first
// call per device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void *> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_address(void **out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    void *p = g_scratch[dev].load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        p = g_scratch[dev].load(std::memory_order_relaxed);
        if (!p) {
            err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (err != hipSuccess) return err;
            if (!p) return hipErrorInvalidSymbol;
            g_scratch[dev].store(p, std::memory_order_release);
        }
    }
    *out = p;
    return hipSuccess;
}

// fp32 inputs: a 64-token chunk's fp32 operands (two 128 x 128 key-side
// tiles and their inverse) exceed one compute unit's LDS, so the fp32 path
// computes chunk 64 as 32-token chunks; the chunk size does not change the
// exact result.
int f32_chunk(int chunk) { return chunk == 64 ? 32 : chunk; }

}  // namespace

extern "C" {

const char *eda_status_string(eda_status_t s) {
    switch (s) {
        case EDA_OK: return "ok";
        case EDA_ERR_NULL: return "required pointer is NULL";
        case EDA_ERR_SHAPE: return "size out of range";
        case EDA_ERR_DTYPE: return "unknown dtype";
        case EDA_ERR_ALIGN: return "pointer misaligned (see eda.h)";
        case EDA_ERR_UNSUPPORTED: return "head dims or chunk size not supported";
        case EDA_ERR_WORKSPACE: return "workspace missing or too small";
        case EDA_ERR_ALIAS: return "output overlaps an input";
        case EDA_ERR_HIP: return "HIP launch failed";
        case EDA_ERR_SCRATCH: return "workspace needed exceeds the no-allocation scratch array (EDA_NOALLOC_SCRATCH_BYTES)";
    }
    return "unknown status";
}

size_t eda_fwd_chunked_workspace_size(int B, int T, int H, int d_k, int d_v, eda_dtype_t dtype,
                                      int chunk) {
    chunk = resolve_chunk(chunk);
    if (!dtype_ok(dtype) || !dims_ok(B, T, H, d_k, d_v) || !head_dims_supported(d_k, d_v) ||
        !chunk_supported(chunk))
        return 0;
    return dtype == EDA_BF16 ? eda::bf16_ws_bytes(B, T, H, d_k, d_v, chunk)
                             : eda::chunked_ws_t<float>(B, T, H, d_k, d_v, f32_chunk(chunk));
}

}  // extern "C"

namespace {

eda_status_t step_call(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                       const float *beta, const float *gamma, const float *S_in, float *S_out, void *o,
                       int N, int H, int d_k, int d_v, eda_dtype_t dtype, void *stream);

// Checks, then the launch.  Both dtypes run two kernels: the chunk factors
// (all chunks in parallel) go to the workspace, then the state pass walks the
// chunks of each head in order.
eda_status_t chunked_call(const void *q, const void *k, const void *e, const void *v,
                          const float *alpha, const float *beta, const float *gamma,
                          const float *S0, void *o, float *S_final, int B, int T, int H, int d_k,
                          int d_v, eda_dtype_t dtype, int chunk, void *workspace,
                          size_t workspace_bytes, void *stream, void *const *events,
                          bool dplr = false, bool use_scratch = false) {
    // (dplr: the rank-1 DPLR update; `e` is its erase vector, beta and gamma are NULL;
    //  use_scratch: the workspace is the device's scratch array, not an argument)
    if (!q || !k || !e || !v || !alpha || !o || (!dplr && (!beta || !gamma))) return EDA_ERR_NULL;
    if (!dtype_ok(dtype)) return EDA_ERR_DTYPE;
    if (!dims_ok(B, T, H, d_k, d_v)) return EDA_ERR_SHAPE;
    chunk = resolve_chunk(chunk);
    if (!head_dims_supported(d_k, d_v) || !chunk_supported(chunk)) return EDA_ERR_UNSUPPORTED;
    // Element alignment for arrays read element-wise; 16 bytes where the
    // kernels use vector accesses (o, states).
    const size_t es = elem_size(dtype);
    const void *elem_ptrs[] = {q, k, e, v};
    for (const void *p : elem_ptrs)
        if (!aligned(p, es)) return EDA_ERR_ALIGN;
    const void *f32_ptrs[] = {alpha, beta, gamma};
    for (const void *p : f32_ptrs)
        if (!aligned(p, 4)) return EDA_ERR_ALIGN;
    const void *vec_ptrs[] = {S0, o, S_final};
    for (const void *p : vec_ptrs)
        if (p && !aligned(p, 16)) return EDA_ERR_ALIGN;
    const size_t need = eda_fwd_chunked_workspace_size(B, T, H, d_k, d_v, dtype, chunk);
    if (use_scratch && need > 0) {
        // every argument check above runs first; this is the first HIP call
        if (need > EDA_NOALLOC_SCRATCH_BYTES) return EDA_ERR_SCRATCH;
        if (scratch_address(&workspace) != hipSuccess) return EDA_ERR_HIP;
        workspace_bytes = EDA_NOALLOC_SCRATCH_BYTES;
    }
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return EDA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return EDA_ERR_ALIGN;
    }

    const size_t btH = (size_t)B * T * H;
    const Range in[] = {range_of(q, btH * d_k * es), range_of(k, btH * d_k * es),
                        range_of(e, btH * d_k * es), range_of(v, btH * d_v * es),
                        range_of(alpha, btH * d_k * 4), range_of(beta, btH * 4),
                        range_of(gamma, btH * 4)};   // (NULL pointers give empty ranges)
    const Range rS0 = range_of(S0, (size_t)B * H * d_k * d_v * 4);
    const Range rSf = range_of(S_final, (size_t)B * H * d_k * d_v * 4);
    const Range rO = range_of(o, btH * d_v * es);
    const Range rW = range_of(need > 0 ? workspace : nullptr, need);
    for (const Range &r : in) {
        if (overlap(rO, r) || overlap(rSf, r) || overlap(rW, r)) return EDA_ERR_ALIAS;
    }
    if (overlap(rO, rS0) || overlap(rO, rSf) || overlap(rO, rW)) return EDA_ERR_ALIAS;
    if (overlap(rW, rS0) || overlap(rW, rSf)) return EDA_ERR_ALIAS;
    if (overlap(rSf, rS0) && S_final != S0) return EDA_ERR_ALIAS;

    hipError_t err =
        dtype == EDA_BF16
            ? eda::launch_bf16(q, k, e, v, alpha, nullptr, nullptr, beta, gamma, S0, o, S_final, B,
                               T, H, H, d_k, d_v, chunk, workspace, (hipStream_t)stream,
                               (hipEvent_t const *)events)
            : eda::launch_chunked<float>(3, q, k, e, v, alpha, beta, gamma, S0, o, S_final, B,
                                         T, H, d_k, d_v, f32_chunk(chunk), workspace, (hipStream_t)stream,
                                         (hipEvent_t const *)events);
    return err == hipSuccess ? EDA_OK : EDA_ERR_HIP;
}

}  // namespace

extern "C" {

eda_status_t eda_fwd_chunked(const void *q, const void *k, const void *e, const void *v,
                             const float *alpha, const float *beta, const float *gamma,
                             const float *S0, void *o, float *S_final, int B, int T, int H,
                             int d_k, int d_v, eda_dtype_t dtype, int chunk, void *workspace,
                             size_t workspace_bytes, void *stream) {
    return chunked_call(q, k, e, v, alpha, beta, gamma, S0, o, S_final, B, T, H, d_k, d_v, dtype,
                        chunk, workspace, workspace_bytes, stream, nullptr);
}

eda_status_t eda_fwd_chunked_noalloc(const void *q, const void *k, const void *e, const void *v,
                                     const float *alpha, const float *beta, const float *gamma,
                                     const float *S0, void *o, float *S_final, int B, int T, int H,
                                     int d_k, int d_v, eda_dtype_t dtype, int chunk, void *stream) {
    return chunked_call(q, k, e, v, alpha, beta, gamma, S0, o, S_final, B, T, H, d_k, d_v, dtype,
                        chunk, nullptr, 0, stream, nullptr, false, true);
}

eda_status_t eda_fwd_chunked_timed(const void *q, const void *k, const void *e, const void *v,
                                   const float *alpha, const float *beta, const float *gamma,
                                   const float *S0, void *o, float *S_final, int B, int T, int H,
                                   int d_k, int d_v, eda_dtype_t dtype, int chunk, void *workspace,
                                   size_t workspace_bytes, void *stream, void *const *events) {
    if (events && (!events[0] || !events[1] || !events[2])) return EDA_ERR_NULL;
    return chunked_call(q, k, e, v, alpha, beta, gamma, S0, o, S_final, B, T, H, d_k, d_v, dtype,
                        chunk, workspace, workspace_bytes, stream, events);
}

eda_status_t eda_fwd_recurrent_step(const void *q, const void *k, const void *e, const void *v,
                                    const float *alpha, const float *beta, const float *gamma,
                                    const float *S_in, float *S_out, void *o, int N, int H,
                                    int d_k, int d_v, eda_dtype_t dtype, void *stream) {
    if (!beta || !gamma) return EDA_ERR_NULL;
    return step_call(q, k, e, v, alpha, beta, gamma, S_in, S_out, o, N, H, d_k, d_v, dtype, stream);
}

eda_status_t eda_fwd_recurrent_step_dplr(const void *q, const void *k, const void *a, const void *v,
                                         const float *alpha, const float *S_in, float *S_out, void *o,
                                         int N, int H, int d_k, int d_v, eda_dtype_t dtype,
                                         void *stream) {
    if (!a) return EDA_ERR_NULL;
    return step_call(q, k, a, v, alpha, nullptr, nullptr, S_in, S_out, o, N, H, d_k, d_v, dtype, stream);
}

eda_status_t eda_fwd_chunked_dplr(const void *q, const void *k, const void *a, const void *v,
                                  const float *alpha, const float *S0, void *o, float *S_final, int B,
                                  int T, int H, int d_k, int d_v, eda_dtype_t dtype, int chunk,
                                  void *workspace, size_t workspace_bytes, void *stream) {
    if (!a) return EDA_ERR_NULL;
    return chunked_call(q, k, a, v, alpha, nullptr, nullptr, S0, o, S_final, B, T, H, d_k, d_v, dtype,
                        chunk, workspace, workspace_bytes, stream, nullptr, true);
}

}  // extern "C"

namespace {

// Checks, then the decode launch; beta == gamma == NULL is the DPLR update.
eda_status_t step_call(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                       const float *beta, const float *gamma, const float *S_in, float *S_out, void *o,
                       int N, int H, int d_k, int d_v, eda_dtype_t dtype, void *stream) {
    if (!q || !k || !e || !v || !alpha || !S_out || !o) return EDA_ERR_NULL;
    if (!dtype_ok(dtype)) return EDA_ERR_DTYPE;
    if (!dims_ok(N, 1, H, d_k, d_v)) return EDA_ERR_SHAPE;
    if (!head_dims_supported(d_k, d_v)) return EDA_ERR_UNSUPPORTED;
    const size_t es0 = elem_size(dtype);
    const void *elem_ptrs[] = {q, k, e, v, o};
    for (const void *p : elem_ptrs)
        if (!aligned(p, es0)) return EDA_ERR_ALIGN;
    const void *f32_ptrs[] = {alpha, beta, gamma};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4)) return EDA_ERR_ALIGN;
    const void *vec_ptrs[] = {S_in, S_out};
    for (const void *p : vec_ptrs)
        if (p && !aligned(p, 16)) return EDA_ERR_ALIGN;

    const size_t es = elem_size(dtype), nH = (size_t)N * H;
    const Range in[] = {range_of(q, nH * d_k * es), range_of(k, nH * d_k * es),
                        range_of(e, nH * d_k * es), range_of(v, nH * d_v * es),
                        range_of(alpha, nH * d_k * 4), range_of(beta, nH * 4),
                        range_of(gamma, nH * 4)};
    const Range rSi = range_of(S_in, nH * d_k * d_v * 4);
    const Range rSo = range_of(S_out, nH * d_k * d_v * 4);
    const Range rO = range_of(o, nH * d_v * es);
    for (const Range &r : in)
        if (overlap(rO, r) || overlap(rSo, r)) return EDA_ERR_ALIAS;
    if (overlap(rO, rSi) || overlap(rO, rSo)) return EDA_ERR_ALIAS;
    if (overlap(rSo, rSi) && S_out != S_in) return EDA_ERR_ALIAS;

    hipError_t err =
        dtype == EDA_BF16
            ? eda::launch_decode<eda::bf16>(q, k, e, v, alpha, nullptr, nullptr, beta, gamma, S_in,
                                            S_out, o, N, H, H, d_k, d_v, (hipStream_t)stream)
            : eda::launch_decode<float>(q, k, e, v, alpha, nullptr, nullptr, beta, gamma, S_in,
                                        S_out, o, N, H, H, d_k, d_v, (hipStream_t)stream);
    return err == hipSuccess ? EDA_OK : EDA_ERR_HIP;
}

// ---------------------------------------------------------------------------
// Layer-form entry points: safe gate, q/k/e normalisation and grouped value
// heads in front of the same recurrence.
// ---------------------------------------------------------------------------

}  // namespace

extern "C" {
}  // extern "C"

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

bool heads_ok(int H_k, int H_v) { return H_k >= 1 && H_v >= 1 && H_v % H_k == 0; }

// fp32: the prologue pass writes q, k, e and alpha per value head after the
// chunked path's own workspace
size_t layer_prep_bytes(int B, int T, int H_v, int d_k) { return align256((size_t)B * T * H_v * d_k * 4); }

}  // namespace

extern "C" {

size_t eda_fwd_chunked_layer_workspace_size(int B, int T, int H_k, int H_v, int d_k, int d_v,
                                            eda_dtype_t dtype, int chunk) {
    if (!heads_ok(H_k, H_v)) return 0;
    const size_t base = eda_fwd_chunked_workspace_size(B, T, H_v, d_k, d_v, dtype, chunk);
    if (base == 0 || dtype == EDA_BF16) return base;
    return align256(base) + 4 * layer_prep_bytes(B, T, H_v, d_k);
}

eda_status_t eda_fwd_chunked_layer(const void *q, const void *k, const void *e, const void *v,
                                   const void *a, const float *A_log, const float *dt_bias,
                                   const float *beta, const float *gamma, const float *S0, void *o,
                                   float *S_final, int B, int T, int H_k, int H_v, int d_k, int d_v,
                                   eda_dtype_t dtype, int chunk, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    if (!q || !k || !e || !v || !a || !A_log || !dt_bias || !beta || !gamma || !o) return EDA_ERR_NULL;
    if (!dtype_ok(dtype)) return EDA_ERR_DTYPE;
    if (!heads_ok(H_k, H_v) || !dims_ok(B, T, H_v, d_k, d_v)) return EDA_ERR_SHAPE;
    chunk = resolve_chunk(chunk);
    if (!head_dims_supported(d_k, d_v) || !chunk_supported(chunk)) return EDA_ERR_UNSUPPORTED;
    const size_t es = elem_size(dtype);
    const void *elem_ptrs[] = {q, k, e, v, a};
    for (const void *p : elem_ptrs)
        if (!aligned(p, es)) return EDA_ERR_ALIGN;
    const void *f32_ptrs[] = {A_log, dt_bias, beta, gamma};
    for (const void *p : f32_ptrs)
        if (!aligned(p, 4)) return EDA_ERR_ALIGN;
    const void *vec_ptrs[] = {S0, o, S_final};
    for (const void *p : vec_ptrs)
        if (p && !aligned(p, 16)) return EDA_ERR_ALIGN;
    const size_t need = eda_fwd_chunked_layer_workspace_size(B, T, H_k, H_v, d_k, d_v, dtype, chunk);
    if (need > 0) {
        if (!workspace || workspace_bytes < need) return EDA_ERR_WORKSPACE;
        if (((uintptr_t)workspace & 255u) != 0) return EDA_ERR_ALIGN;
    }

    const size_t btk = (size_t)B * T * H_k, btv = (size_t)B * T * H_v;
    const Range in[] = {range_of(q, btk * d_k * es), range_of(k, btk * d_k * es),
                        range_of(e, btk * d_k * es), range_of(a, btk * d_k * es),
                        range_of(v, btv * d_v * es), range_of(A_log, (size_t)H_k * d_k * 4),
                        range_of(dt_bias, (size_t)H_k * d_k * 4), range_of(beta, btv * 4),
                        range_of(gamma, btv * 4)};
    const Range rS0 = range_of(S0, (size_t)B * H_v * d_k * d_v * 4);
    const Range rSf = range_of(S_final, (size_t)B * H_v * d_k * d_v * 4);
    const Range rO = range_of(o, btv * d_v * es);
    const Range rW = range_of(need > 0 ? workspace : nullptr, need);
    for (const Range &r : in)
        if (overlap(rO, r) || overlap(rSf, r) || overlap(rW, r)) return EDA_ERR_ALIAS;
    if (overlap(rO, rS0) || overlap(rO, rSf) || overlap(rO, rW)) return EDA_ERR_ALIAS;
    if (overlap(rW, rS0) || overlap(rW, rSf)) return EDA_ERR_ALIAS;
    if (overlap(rSf, rS0) && S_final != S0) return EDA_ERR_ALIAS;

    hipError_t err;
    if (dtype == EDA_BF16) {
        err = eda::launch_bf16(q, k, e, v, a, A_log, dt_bias, beta, gamma, S0, o, S_final, B, T, H_v,
                               H_k, d_k, d_v, chunk, workspace, (hipStream_t)stream, nullptr);
    } else {
        char *w = (char *)workspace;
        const size_t base = align256(eda_fwd_chunked_workspace_size(B, T, H_v, d_k, d_v, dtype, chunk));
        const size_t pb = layer_prep_bytes(B, T, H_v, d_k);
        float *qn = (float *)(w + base), *kn = (float *)(w + base + pb);
        float *en = (float *)(w + base + 2 * pb), *al = (float *)(w + base + 3 * pb);
        err = eda::launch_layer_prep<float>(q, k, e, a, A_log, dt_bias, qn, kn, en, al, B, T, H_v, H_k,
                                            d_k, (hipStream_t)stream);
        if (err == hipSuccess)
            err = eda::launch_chunked<float>(3, qn, kn, en, v, al, beta, gamma, S0, o, S_final, B, T,
                                             H_v, d_k, d_v, f32_chunk(chunk), workspace, (hipStream_t)stream,
                                             nullptr);
    }
    return err == hipSuccess ? EDA_OK : EDA_ERR_HIP;
}

eda_status_t eda_fwd_recurrent_step_layer(const void *q, const void *k, const void *e, const void *v,
                                          const void *a, const float *A_log, const float *dt_bias,
                                          const float *beta, const float *gamma, const float *S_in,
                                          float *S_out, void *o, int N, int H_k, int H_v, int d_k,
                                          int d_v, eda_dtype_t dtype, void *stream) {
    if (!q || !k || !e || !v || !a || !A_log || !dt_bias || !beta || !gamma || !S_out || !o)
        return EDA_ERR_NULL;
    if (!dtype_ok(dtype)) return EDA_ERR_DTYPE;
    if (!heads_ok(H_k, H_v) || !dims_ok(N, 1, H_v, d_k, d_v)) return EDA_ERR_SHAPE;
    if (!head_dims_supported(d_k, d_v)) return EDA_ERR_UNSUPPORTED;
    const size_t es = elem_size(dtype);
    const void *elem_ptrs[] = {q, k, e, v, a, o};
    for (const void *p : elem_ptrs)
        if (!aligned(p, es)) return EDA_ERR_ALIGN;
    const void *f32_ptrs[] = {A_log, dt_bias, beta, gamma};
    for (const void *p : f32_ptrs)
        if (!aligned(p, 4)) return EDA_ERR_ALIGN;
    const void *vec_ptrs[] = {S_in, S_out};
    for (const void *p : vec_ptrs)
        if (p && !aligned(p, 16)) return EDA_ERR_ALIGN;

    const size_t nk = (size_t)N * H_k, nv = (size_t)N * H_v;
    const Range in[] = {range_of(q, nk * d_k * es), range_of(k, nk * d_k * es),
                        range_of(e, nk * d_k * es), range_of(a, nk * d_k * es),
                        range_of(v, nv * d_v * es), range_of(A_log, (size_t)H_k * d_k * 4),
                        range_of(dt_bias, (size_t)H_k * d_k * 4), range_of(beta, nv * 4),
                        range_of(gamma, nv * 4)};
    const Range rSi = range_of(S_in, nv * d_k * d_v * 4);
    const Range rSo = range_of(S_out, nv * d_k * d_v * 4);
    const Range rO = range_of(o, nv * d_v * es);
    for (const Range &r : in)
        if (overlap(rO, r) || overlap(rSo, r)) return EDA_ERR_ALIAS;
    if (overlap(rO, rSi) || overlap(rO, rSo)) return EDA_ERR_ALIAS;
    if (overlap(rSo, rSi) && S_out != S_in) return EDA_ERR_ALIAS;

    hipError_t err =
        dtype == EDA_BF16
            ? eda::launch_decode<eda::bf16>(q, k, e, v, a, A_log, dt_bias, beta, gamma, S_in, S_out, o,
                                            N, H_v, H_k, d_k, d_v, (hipStream_t)stream)
            : eda::launch_decode<float>(q, k, e, v, a, A_log, dt_bias, beta, gamma, S_in, S_out, o, N,
                                        H_v, H_k, d_k, d_v, (hipStream_t)stream);
    return err == hipSuccess ? EDA_OK : EDA_ERR_HIP;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward pass.
// ---------------------------------------------------------------------------
extern "C" {

size_t eda_bwd_workspace_size(int B, int T, int H, int d_k, int d_v) {
    if (!dims_ok(B, T, H, d_k, d_v) || !head_dims_supported(d_k, d_v)) return 0;
    return eda::bwd_ws_bytes(B, T, H, d_k, d_v);
}

eda_status_t eda_bwd(const void *q, const void *k, const void *e, const void *v, const float *alpha,
                     const float *beta, const float *gamma, const float *S0, const void *dO,
                     const float *dS_final, float *dq, float *dk, float *de, float *dv, float *dalpha,
                     float *dbeta, float *dgamma, float *dS0, int B, int T, int H, int d_k, int d_v,
                     eda_dtype_t dtype, void *workspace, size_t workspace_bytes, void *stream) {
    if (!q || !k || !e || !v || !alpha || !beta || !gamma || !dO || !dq || !dk || !de || !dv || !dalpha ||
        !dbeta || !dgamma)
        return EDA_ERR_NULL;
    if (!dtype_ok(dtype)) return EDA_ERR_DTYPE;
    if (!dims_ok(B, T, H, d_k, d_v)) return EDA_ERR_SHAPE;
    if (!head_dims_supported(d_k, d_v)) return EDA_ERR_UNSUPPORTED;
    const size_t es = elem_size(dtype);
    const void *elem_ptrs[] = {q, k, e, v, dO};
    for (const void *p : elem_ptrs)
        if (!aligned(p, es)) return EDA_ERR_ALIGN;
    const void *f32_ptrs[] = {alpha, beta, gamma, S0, dS_final, dq, dk, de, dv, dalpha, dbeta, dgamma, dS0};
    for (const void *p : f32_ptrs)
        if (p && !aligned(p, 4)) return EDA_ERR_ALIGN;
    const size_t need = eda_bwd_workspace_size(B, T, H, d_k, d_v);
    if (!workspace || workspace_bytes < need) return EDA_ERR_WORKSPACE;
    if (((uintptr_t)workspace & 255u) != 0) return EDA_ERR_ALIGN;

    const size_t btH = (size_t)B * T * H, st = (size_t)B * H * d_k * d_v * 4;
    const Range in[] = {range_of(q, btH * d_k * es), range_of(k, btH * d_k * es), range_of(e, btH * d_k * es),
                        range_of(v, btH * d_v * es), range_of(alpha, btH * d_k * 4), range_of(beta, btH * 4),
                        range_of(gamma, btH * 4), range_of(S0, st), range_of(dO, btH * d_v * es),
                        range_of(dS_final, st)};
    const Range out[] = {range_of(dq, btH * d_k * 4), range_of(dk, btH * d_k * 4), range_of(de, btH * d_k * 4),
                         range_of(dv, btH * d_v * 4), range_of(dalpha, btH * d_k * 4), range_of(dbeta, btH * 4),
                         range_of(dgamma, btH * 4), range_of(dS0, st), range_of(workspace, need)};
    // no output may overlap an input, the workspace or another output
    for (size_t a = 0; a < sizeof(out) / sizeof(out[0]); ++a) {
        for (const Range &r : in)
            if (overlap(out[a], r)) return EDA_ERR_ALIAS;
        for (size_t c = a + 1; c < sizeof(out) / sizeof(out[0]); ++c)
            if (overlap(out[a], out[c])) return EDA_ERR_ALIAS;
    }

    hipError_t err =
        dtype == EDA_BF16
            ? eda::launch_bwd<eda::bf16>(q, k, e, v, alpha, beta, gamma, S0, dO, dS_final, dq, dk, de, dv,
                                         dalpha, dbeta, dgamma, dS0, B, T, H, d_k, d_v, workspace,
                                         (hipStream_t)stream)
            : eda::launch_bwd<float>(q, k, e, v, alpha, beta, gamma, S0, dO, dS_final, dq, dk, de, dv, dalpha,
                                     dbeta, dgamma, dS0, B, T, H, d_k, d_v, workspace, (hipStream_t)stream);
    return err == hipSuccess ? EDA_OK : EDA_ERR_HIP;
}

}  // extern "C"
