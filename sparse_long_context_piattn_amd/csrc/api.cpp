// api.cpp -- the C ABI of libpiattn: argument validation, kernel selection
// and launches on the caller's stream.  Declarations and the contract of
// every entry point are in include/piattn.h.
#include <math.h>
#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime.h>

#include "piattn.h"
#include "kernels.hpp"
#include "api_internal.hpp"

namespace {

thread_local char g_err[512] = "";

// Kernel overrides set by piattn_debug_force_kernels (0 = automatic choice).
std::atomic<int32_t> g_force_fwd{0};
std::atomic<int32_t> g_force_bwd{0};

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return PIATTN_OK;
}

constexpr int32_t kMaxExtent = 1 << 30;  // n + k and friends stay far from int32 overflow

int check_pattern(const piattn_pattern* p, PiPattern* out) {
    if (!p) return fail(PIATTN_EINVAL, "pattern is NULL");
    if (p->window_k < 0 || p->window_k >= kMaxExtent)
        return fail(PIATTN_EINVAL, "window_k=%d out of range [0, 2^30)", p->window_k);
    if (p->period_pi < 1 || p->period_pi >= kMaxExtent)
        return fail(PIATTN_EINVAL, "period_pi=%d out of range [1, 2^30)", p->period_pi);
    if (p->num_skips_M < 0 || p->num_skips_M >= kMaxExtent)
        return fail(PIATTN_EINVAL, "num_skips_M=%d out of range [0, 2^30)", p->num_skips_M);
    if (p->bidirectional != 0 && p->bidirectional != 1)
        return fail(PIATTN_EINVAL, "bidirectional=%d must be 0 or 1", p->bidirectional);
    if (!isfinite(p->scale)) return fail(PIATTN_EINVAL, "scale is not finite");
    if (p->num_levels < 0 || p->num_levels > PIATTN_MAX_LEVELS)
        return fail(PIATTN_EINVAL, "num_levels=%d out of range [0, %d]", p->num_levels, PIATTN_MAX_LEVELS);
    for (int r = 0; r < p->num_levels; ++r) {
        if (p->level_pi[r] < 1 || p->level_pi[r] >= kMaxExtent)
            return fail(PIATTN_EINVAL, "level_pi[%d]=%d out of range [1, 2^30)", r, p->level_pi[r]);
        if (p->level_M[r] < 0 || p->level_M[r] >= kMaxExtent)
            return fail(PIATTN_EINVAL, "level_M[%d]=%d out of range [0, 2^30)", r, p->level_M[r]);
    }
    *out = PiPattern{};
    out->k = p->window_k;
    out->pi = p->period_pi;
    out->M = p->num_skips_M;
    out->bidir = p->bidirectional;
    out->mlo = p->window_k / p->period_pi + 1;
    if (p->num_levels == 0) return PIATTN_OK;
    // A schedule: the union of the levels' skip distances beyond the window,
    // as multiples of g = gcd of the periods (of the levels with M > 0).
    int32_t lp[PIATTN_MAX_LEVELS + 1], lm[PIATTN_MAX_LEVELS + 1];
    lp[0] = p->period_pi;
    lm[0] = p->num_skips_M;
    for (int r = 0; r < p->num_levels; ++r) {
        lp[r + 1] = p->level_pi[r];
        lm[r + 1] = p->level_M[r];
    }
    const int nl = p->num_levels + 1;
    int64_t g = 0;
    for (int r = 0; r < nl; ++r) {
        if (lm[r] == 0) continue;
        int64_t a = g, b = lp[r];
        while (b) {
            const int64_t t = a % b;
            a = b;
            b = t;
        }
        g = a;
    }
    if (g == 0) {                                       // no level has skips
        out->M = 0;
        return PIATTN_OK;
    }
    uint32_t mask[4] = {0, 0, 0, 0};
    for (int r = 0; r < nl; ++r) {
        const int64_t step = lp[r] / g;                 // multiples of g per multiple of lp[r]
        for (int64_t m = 1; m <= lm[r]; ++m) {
            const int64_t mm = m * step;                 // distance mm * g
            if (mm * g <= p->window_k) continue;        // inside the window
            if (mm >= kMaskBits)
                return fail(PIATTN_EUNSUPPORTED,
                            "skip schedule reaches distance %lld = %lld * gcd %lld (at most 127 multiples of the "
                            "periods' gcd)", (long long)(mm * g), (long long)mm, (long long)g);
            mask[mm >> 5] |= 1u << (mm & 31);
        }
    }
    int32_t lo = -1, hi = 0, cnt = 0;
    for (int32_t m = 0; m < kMaskBits; ++m)
        if ((mask[m >> 5] >> (m & 31)) & 1u) {
            if (lo < 0) lo = m;
            hi = m;
            ++cnt;
        }
    out->pi = (int32_t)g;
    out->M = hi;
    out->mlo = lo < 0 ? out->k / out->pi + 1 : lo;
    if (lo >= 0 && cnt != hi - lo + 1) {                // not one contiguous range of multiples
        out->masked = 1;
        for (int w = 0; w < 4; ++w) out->mask[w] = mask[w];
    }
    return PIATTN_OK;
}

// Skip keys per direction at most: multiples in the mask, else M.
int64_t skip_cap(const PiPattern& p) {
    if (!p.masked) return p.M;
    return __builtin_popcount(p.mask[0]) + __builtin_popcount(p.mask[1]) + __builtin_popcount(p.mask[2]) +
           __builtin_popcount(p.mask[3]);
}

float scale_nat(const piattn_pattern* p, int d) { return p->scale > 0.0f ? p->scale : 1.0f / sqrtf((float)d); }

float scale_log2(const piattn_pattern* p, int d) { return scale_nat(p, d) * 1.4426950408889634f; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_tensor(const char* name, const void* p, const int64_t s[3], int64_t mult,
                 bool use_seq) {
    if (!p) return fail(PIATTN_EINVAL, "%s is NULL", name);
    if (!aligned(p, 16)) return fail(PIATTN_EINVAL, "%s is not 16-byte aligned", name);
    for (int j = 0; j < 3; ++j) {
        if (j == 0 && !use_seq) continue;
        if (s[j] < 0) return fail(PIATTN_EINVAL, "%s stride[%d]=%lld is negative", name, j,
                                  (long long)s[j]);
        if (s[j] % mult)
            return fail(PIATTN_EINVAL, "%s stride[%d]=%lld is not a multiple of %lld elements",
                        name, j, (long long)s[j], (long long)mult);
    }
    return PIATTN_OK;
}

Str3 str3(const int64_t s[3]) { return Str3{s[0], s[1], s[2]}; }

int launch_status(hipError_t e) {
    if (e != hipSuccess) return fail(PIATTN_EHIP, "kernel launch failed: %s", hipGetErrorString(e));
    return ok();
}

int decode_splits_for(int32_t S, int32_t H, const PiPattern& p) {
    // Enough workgroups to cover the chip several times, but at least 64
    // union positions per split so that each split still streams rows.
    const int64_t rows = (int64_t)S * H;
    const int64_t umax = (int64_t)p.k + 1 + p.M;
    int64_t want = (2048 + rows - 1) / rows;
    int64_t cap = umax / 64 > 0 ? umax / 64 : 1;
    if (want > cap) want = cap;
    if (want < 1) want = 1;
    if (want > 64) want = 64;
    return (int)want;
}

}  // namespace

int api_fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

extern "C" {

const char* piattn_last_error(void) { return g_err; }

const char* piattn_version(void) { return "libpiattn 0.2 (gfx950)"; }

int piattn_debug_force_kernels(int32_t fwd_kernel, int32_t bwd_kernel) {
    if (fwd_kernel < PIATTN_KERNEL_AUTO || fwd_kernel > PIATTN_FWD_LAST)
        return fail(PIATTN_EINVAL, "fwd_kernel=%d is not a prefill kernel id", fwd_kernel);
    if (bwd_kernel < PIATTN_KERNEL_AUTO || bwd_kernel > PIATTN_BWD_GATHER)
        return fail(PIATTN_EINVAL, "bwd_kernel=%d is not a backward kernel id", bwd_kernel);
    g_force_fwd.store(fwd_kernel, std::memory_order_relaxed);
    g_force_bwd.store(bwd_kernel, std::memory_order_relaxed);
    return ok();
}

int32_t piattn_neighbors_cap(const piattn_pattern* pattern) {
    PiPattern p;
    if (check_pattern(pattern, &p) != PIATTN_OK) return -1;
    const int64_t sk = skip_cap(p);
    const int64_t cap = p.bidir ? 2LL * p.k + 1 + 2 * sk : (int64_t)p.k + 1 + sk;
    return cap > INT32_MAX ? -1 : (int32_t)cap;
}

int piattn_neighbors(int32_t n, const piattn_pattern* pattern, int32_t q_begin, int32_t q_count,
                     int32_t cap, int32_t* idx, int8_t* kind, int32_t* count, void* stream) {
    PiPattern p;
    int rc = check_pattern(pattern, &p);
    if (rc) return rc;
    if (n < 1 || n >= kMaxExtent) return fail(PIATTN_EINVAL, "n=%d out of range [1, 2^30)", n);
    if (q_begin < 0 || q_count < 0 || (int64_t)q_begin + q_count > n)
        return fail(PIATTN_EINVAL, "query range [%d, %d+%d) not inside [0, %d)", q_begin, q_begin,
                    q_count, n);
    const int64_t sk = skip_cap(p);
    const int64_t need = p.bidir ? 2LL * p.k + 1 + 2 * sk : (int64_t)p.k + 1 + sk;
    const int64_t need_n = need < n ? need : n;  // a list never exceeds n keys
    if (cap < need_n)
        return fail(PIATTN_EINVAL, "cap=%d is smaller than the longest list (%lld)", cap,
                    (long long)need_n);
    if (q_count == 0) return ok();
    if (!idx || !kind || !count) return fail(PIATTN_EINVAL, "idx, kind and count must be non-NULL");
    return launch_status(launch_neighbors(n, p, q_begin, q_count, cap, idx, kind, count,
                                          static_cast<hipStream_t>(stream)));
}

// Workspace of the split prefill path: one (log2-sum-exp, exponent) float
// pair per row, written by its skip pass and read by its window pass.  Only
// bf16 at d = 64 / 128 with a non-empty skip set can take that path.
static size_t fwd_split_workspace(int dtype, int32_t B, int32_t H, int32_t n, int32_t d, const PiPattern& p) {
    if (dtype != PIATTN_BF16 || (d != 64 && d != 128)) return 0;
    if (p.M < p.mlo) return 0;
    return (size_t)B * H * n * 2 * sizeof(float);
}

size_t piattn_fwd_workspace_bytes(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d,
                                  const piattn_pattern* pattern) {
    PiPattern p;
    if (check_pattern(pattern, &p) != PIATTN_OK || B < 1 || H < 1 || n < 1) return 0;
    return fwd_split_workspace(dtype, B, H, n, d, p);
}

}  // extern "C"

// Validates the arguments piattn_fwd and piattn_bwd share and fills a.
static int fwd_args(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q,
                    const void* k, const void* v, const float* gate_logits, void* out, float* lse_out,
                    const int64_t strides[5][3], const int32_t* cu_seqlens, const piattn_pattern* pattern,
                    FwdArgs& a, PiPattern& p) {
    int rc;
    if (dtype != PIATTN_F32 && dtype != PIATTN_BF16)
        return fail(PIATTN_EINVAL, "dtype=%d is not PIATTN_F32 or PIATTN_BF16", (int)dtype);
    rc = check_pattern(pattern, &p);
    if (rc) return rc;
    if (B < 1 || B > 65535) return fail(PIATTN_EINVAL, "B=%d out of range [1, 65535]", B);
    if (H < 1 || H > 65535) return fail(PIATTN_EINVAL, "H=%d out of range [1, 65535]", H);
    if (n < 1 || n >= kMaxExtent - p.k)
        return fail(PIATTN_EINVAL, "n=%d out of range (n >= 1, n + k < 2^30)", n);
    if (d < 1) return fail(PIATTN_EINVAL, "d=%d must be positive", d);
    if (d != 32 && d != 64 && d != 128)
        return fail(PIATTN_EUNSUPPORTED, "d=%d unsupported (32, 64 or 128)", d);
    if (!strides) return fail(PIATTN_EINVAL, "strides is NULL");
    const int64_t mult = dtype == PIATTN_BF16 ? 8 : 4;
    const bool dense = cu_seqlens == nullptr;
    if ((rc = check_tensor("q", q, strides[0], mult, dense))) return rc;
    if ((rc = check_tensor("k", k, strides[1], mult, dense))) return rc;
    if ((rc = check_tensor("v", v, strides[2], mult, dense))) return rc;
    if ((rc = check_tensor("out", out, strides[3], mult, dense))) return rc;
    if (!gate_logits) return fail(PIATTN_EINVAL, "gate_logits is NULL");
    if (!aligned(gate_logits, 4) || (lse_out && !aligned(lse_out, 4)))
        return fail(PIATTN_EINVAL, "gate_logits / lse_out must be 4-byte aligned");
    for (int j = 0; j < 3; ++j)
        if (strides[4][j] < 0) return fail(PIATTN_EINVAL, "gate stride[%d] is negative", j);
    if (out == q || out == k || out == v) return fail(PIATTN_EINVAL, "out aliases an input");
    if (!dense && !aligned(cu_seqlens, 4))
        return fail(PIATTN_EINVAL, "cu_seqlens must be 4-byte aligned");

    a.q = q;
    a.k = k;
    a.v = v;
    a.g = gate_logits;
    a.o = out;
    a.lse = lse_out;
    a.sq = str3(strides[0]);
    a.sk = str3(strides[1]);
    a.sv = str3(strides[2]);
    a.so = str3(strides[3]);
    a.sg = str3(strides[4]);
    a.cu = cu_seqlens;
    a.B = B;
    a.H = H;
    a.n = n;
    a.d = d;
    a.pat = p;
    a.scale_log2 = scale_log2(pattern, d);
    return PIATTN_OK;
}

int api_check_fwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q, const void* k,
                  const void* v, const float* gate_logits, void* out, float* lse_out, const int64_t strides[5][3],
                  const int32_t* cu_seqlens, const piattn_pattern* pattern) {
    FwdArgs a;
    PiPattern p;
    return fwd_args(dtype, B, H, n, d, q, k, v, gate_logits, out, lse_out, strides, cu_seqlens, pattern, a, p);
}

extern "C" {

int piattn_fwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q,
               const void* k, const void* v, const float* gate_logits, void* out, float* lse_out,
               const int64_t strides[5][3], const int32_t* cu_seqlens,
               const piattn_pattern* pattern, void* workspace, size_t workspace_bytes, void* stream) {
    FwdArgs a;
    PiPattern p;
    const int rc = fwd_args(dtype, B, H, n, d, q, k, v, gate_logits, out, lse_out, strides, cu_seqlens,
                            pattern, a, p);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int dt = dtype == PIATTN_BF16 ? 1 : 0;
    // Kernel choice: the first kernel that can take the call, unless
    // piattn_debug_force_kernels forced one (EUNSUPPORTED if it cannot).
    // The split path checks the workspace first (the other kernels take none).
    auto split = [&]() -> int {
        const size_t need = fwd_split_workspace(dtype, B, H, n, d, p);
        if (need) {
            if (!workspace) return fail(PIATTN_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
            if (workspace_bytes < need)
                return fail(PIATTN_EWORKSPACE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, need);
            if (!aligned(workspace, 256)) return fail(PIATTN_EINVAL, "workspace is not 256-byte aligned");
        }
        float* ws = need ? static_cast<float*>(workspace) : nullptr;
        return launch_status(launch_fwd_split(a, ws, st));
    };
    const int32_t force = g_force_fwd.load(std::memory_order_relaxed);
    if (force != PIATTN_KERNEL_AUTO) {
        if (force == PIATTN_FWD_RESID && fwd_resid_supported(dt, a)) return launch_status(launch_fwd_resid(a, st));
        if (force == PIATTN_FWD_SPLIT && fwd_split_supported(dt, a)) return split();
        if (force == PIATTN_FWD_GATHER) return launch_status(launch_fwd_gather(dt, a, st));
        if (force == PIATTN_FWD_F32MFMA && fwd_f32mfma_supported(dt, a))
            return launch_status(launch_fwd_f32mfma(a, st));
        return fail(PIATTN_EUNSUPPORTED, "the forced prefill kernel (%d) cannot take this call", force);
    }
    if (fwd_split_supported(dt, a)) return split();
    if (fwd_resid_supported(dt, a)) return launch_status(launch_fwd_resid(a, st));
    if (fwd_f32mfma_supported(dt, a) && fwd_f32mfma_preferred(a)) return launch_status(launch_fwd_f32mfma(a, st));
    return launch_status(launch_fwd_gather(dt, a, st));
}

size_t piattn_bwd_workspace_bytes(int32_t B, int32_t H, int32_t n) {
    if (B < 1 || H < 1 || n < 1) return 0;
    return (size_t)B * H * n * 4 * sizeof(float);
}

int piattn_bwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q, const void* k,
               const void* v, const float* gate_logits, const void* out, const float* lse, const void* dout,
               void* dq, void* dk,
               void* dv, float* dgate, const int64_t strides[5][3], const int32_t* cu_seqlens,
               const piattn_pattern* pattern, void* workspace, size_t workspace_bytes, void* stream) {
    BwdArgs ba;
    PiPattern p;
    int rc = fwd_args(dtype, B, H, n, d, q, k, v, gate_logits, const_cast<void*>(out), nullptr, strides,
                      cu_seqlens, pattern, ba.f, p);
    if (rc) return rc;
    const int64_t mult = dtype == PIATTN_BF16 ? 8 : 4;
    const bool dense = cu_seqlens == nullptr;
    if ((rc = check_tensor("dout", dout, strides[3], mult, dense))) return rc;
    if ((rc = check_tensor("dq", dq, strides[0], mult, dense))) return rc;
    if ((rc = check_tensor("dk", dk, strides[1], mult, dense))) return rc;
    if ((rc = check_tensor("dv", dv, strides[2], mult, dense))) return rc;
    if (!dgate || !aligned(dgate, 4)) return fail(PIATTN_EINVAL, "dgate is NULL or misaligned");
    const void* ins[5] = {q, k, v, out, dout};
    void* outs[3] = {dq, dk, dv};
    for (void* o : outs)
        for (const void* in : ins)
            if (o == in) return fail(PIATTN_EINVAL, "a gradient aliases an input");
    if (dq == dk || dq == dv || dk == dv) return fail(PIATTN_EINVAL, "gradients alias each other");
    if (static_cast<const void*>(dgate) == gate_logits) return fail(PIATTN_EINVAL, "dgate aliases gate_logits");
    if (lse && !aligned(lse, 4)) return fail(PIATTN_EINVAL, "lse must be 4-byte aligned");
    if (lse && static_cast<const void*>(lse) == static_cast<const void*>(dgate))
        return fail(PIATTN_EINVAL, "dgate aliases lse");
    const size_t need = piattn_bwd_workspace_bytes(B, H, n);
    if (!workspace) return fail(PIATTN_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
    if (workspace_bytes < need)
        return fail(PIATTN_EWORKSPACE, "workspace of %zu bytes is smaller than %zu", workspace_bytes, need);
    if (!aligned(workspace, 256)) return fail(PIATTN_EINVAL, "workspace is not 256-byte aligned");
    ba.dout = dout;
    ba.dq = dq;
    ba.dk = dk;
    ba.dv = dv;
    ba.dg = dgate;
    ba.rowstat = static_cast<float*>(workspace);
    ba.lse_in = lse;
    ba.scale = scale_nat(pattern, d);
    const int dt = dtype == PIATTN_BF16 ? 1 : 0;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // Kernel choice: the MFMA band kernels when they take the call (bf16,
    // d 64 / 128, lse given), else the gather kernels, unless
    // piattn_debug_force_kernels forced one (EUNSUPPORTED if it cannot).
    const int32_t force = g_force_bwd.load(std::memory_order_relaxed);
    const bool band_ok = bwd_band_supported(dt, ba);
    if (force == PIATTN_BWD_BAND) {
        if (!band_ok) return fail(PIATTN_EUNSUPPORTED, "the forced band backward cannot take this call");
        return launch_status(launch_bwd_band(ba, st));
    }
    if (force == PIATTN_BWD_GATHER) return launch_status(launch_bwd(dt, ba, st));
    return launch_status(band_ok ? launch_bwd_band(ba, st) : launch_bwd(dt, ba, st));
}

int piattn_gate_logits(piattn_dtype dtype, int32_t B, int32_t n, int32_t Dm, int32_t H, const void* x,
                       const int64_t x_strides[2], const void* w, const float* bias, float* g,
                       const int64_t g_strides[3], void* stream) {
    if (dtype != PIATTN_F32 && dtype != PIATTN_BF16)
        return fail(PIATTN_EINVAL, "dtype=%d is not PIATTN_F32 or PIATTN_BF16", (int)dtype);
    if (B < 1 || n < 1 || Dm < 1 || H < 1)
        return fail(PIATTN_EINVAL, "B=%d n=%d Dm=%d H=%d must all be >= 1", B, n, Dm, H);
    if (!x || !w || !g || !x_strides || !g_strides) return fail(PIATTN_EINVAL, "a pointer argument is NULL");
    const int64_t mult = dtype == PIATTN_BF16 ? 8 : 1;
    if (x_strides[0] < 0 || x_strides[1] < 0 || x_strides[0] % mult || x_strides[1] % mult)
        return fail(PIATTN_EINVAL, "x strides must be non-negative multiples of %lld elements", (long long)mult);
    for (int j = 0; j < 3; ++j)
        if (g_strides[j] < 0) return fail(PIATTN_EINVAL, "g stride[%d] is negative", j);
    if (dtype == PIATTN_BF16) {
        if (!aligned(x, 16) || !aligned(w, 16)) return fail(PIATTN_EINVAL, "x and w must be 16-byte aligned");
        if (Dm % 32) return fail(PIATTN_EUNSUPPORTED, "bf16 gate: Dm=%d must be a multiple of 32", Dm);
        if (H > 32) return fail(PIATTN_EUNSUPPORTED, "bf16 gate: H=%d above 32", H);
    } else if (!aligned(x, 4) || !aligned(w, 4)) {
        return fail(PIATTN_EINVAL, "x and w must be 4-byte aligned");
    }
    if (!aligned(g, 4) || (bias && !aligned(bias, 4))) return fail(PIATTN_EINVAL, "g and bias must be 4-byte aligned");
    if (static_cast<const void*>(g) == x || static_cast<const void*>(g) == w)
        return fail(PIATTN_EINVAL, "g aliases an input");
    GateArgs a;
    a.x = x;
    a.sx_b = x_strides[0];
    a.sx_t = x_strides[1];
    a.w = w;
    a.bias = bias;
    a.g = g;
    a.sg_b = g_strides[0];
    a.sg_h = g_strides[1];
    a.sg_t = g_strides[2];
    a.B = B;
    a.n = n;
    a.H = H;
    a.Dm = Dm;
    return launch_status(launch_gate(dtype == PIATTN_BF16 ? 1 : 0, a, static_cast<hipStream_t>(stream)));
}

int piattn_out_proj(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* o,
                    const int64_t o_strides[3], int32_t Dout, const void* w, int64_t ldw, const float* bias,
                    void* y, const int64_t y_strides[2], void* stream) {
    if (dtype != PIATTN_F32 && dtype != PIATTN_BF16)
        return fail(PIATTN_EINVAL, "dtype=%d is not PIATTN_F32 or PIATTN_BF16", (int)dtype);
    if (B < 1 || H < 1 || n < 1 || d < 1 || Dout < 1)
        return fail(PIATTN_EINVAL, "B=%d H=%d n=%d d=%d Dout=%d must all be >= 1", B, H, n, d, Dout);
    if (!o || !w || !y || !o_strides || !y_strides) return fail(PIATTN_EINVAL, "a pointer argument is NULL");
    const int64_t mult = dtype == PIATTN_BF16 ? 8 : 1;
    for (int j = 0; j < 3; ++j)
        if (o_strides[j] < 0 || o_strides[j] % mult)
            return fail(PIATTN_EINVAL, "o stride[%d] must be a non-negative multiple of %lld", j, (long long)mult);
    for (int j = 0; j < 2; ++j)
        if (y_strides[j] < 0 || y_strides[j] % mult)
            return fail(PIATTN_EINVAL, "y stride[%d] must be a non-negative multiple of %lld", j, (long long)mult);
    if (ldw < (int64_t)H * d || ldw % mult)
        return fail(PIATTN_EINVAL, "ldw=%lld must be >= H*d and a multiple of %lld", (long long)ldw, (long long)mult);
    const size_t al = dtype == PIATTN_BF16 ? 16 : 4;
    if (!aligned(o, al) || !aligned(w, al) || !aligned(y, al))
        return fail(PIATTN_EINVAL, "o, w and y must be %zu-byte aligned", al);
    if (bias && !aligned(bias, 4)) return fail(PIATTN_EINVAL, "bias must be 4-byte aligned");
    if (y == o || y == w) return fail(PIATTN_EINVAL, "y aliases an input");
    ProjArgs a;
    a.o = o;
    a.so_b = o_strides[0];
    a.so_h = o_strides[1];
    a.so_t = o_strides[2];
    a.w = w;
    a.ldw = ldw;
    a.bias = bias;
    a.y = y;
    a.sy_b = y_strides[0];
    a.sy_t = y_strides[1];
    a.B = B;
    a.n = n;
    a.H = H;
    a.d = d;
    a.Dout = Dout;
    return launch_status(launch_out_proj(dtype == PIATTN_BF16 ? 1 : 0, a, static_cast<hipStream_t>(stream)));
}

size_t piattn_decode_workspace_bytes(int32_t S, int32_t H, int32_t d, int32_t num_splits,
                                     const piattn_pattern* pattern) {
    if (S < 1 || H < 1 || d < 1 || num_splits < 0 || num_splits > 64) return 0;
    int splits = num_splits;
    if (splits == 0) {
        PiPattern p;
        if (check_pattern(pattern, &p) != PIATTN_OK) return 0;
        splits = decode_splits_for(S, H, p);
    }
    if (splits <= 1) return 0;
    return (size_t)S * H * splits * (d + 2) * sizeof(float);
}

int32_t piattn_decode_auto_splits(int32_t S, int32_t H, int32_t d, const piattn_pattern* pattern) {
    PiPattern p;
    (void)d;
    if (check_pattern(pattern, &p) != PIATTN_OK || S < 1 || H < 1) return -1;
    return decode_splits_for(S, H, p);
}

}  // extern "C"

// Rows a rolling cache needs so that every key of the newest position is
// still held: the window reaches back k positions, the skips M*pi (when the
// pattern has skip keys outside the window).  -1 when that exceeds int32.
static int64_t rolling_slots_for(const PiPattern& p) {
    const int64_t back = p.M >= p.mlo ? (int64_t)p.M * p.pi : 0;
    const int64_t w = (back > p.k ? back : p.k) + 1;
    return w < kMaxExtent ? w : -1;
}

static int decode_impl(piattn_dtype dtype, int32_t S, int32_t H, int32_t d, const void* q,
                       const void* k_cache, const void* v_cache, const int32_t* cache_lens,
                       int32_t cache_capacity, const float* gate_logits, void* out,
                       const int64_t strides[5][3], const piattn_pattern* pattern, int32_t num_splits,
                       void* workspace, size_t workspace_bytes, void* stream, bool rolling) {
    if (dtype != PIATTN_F32 && dtype != PIATTN_BF16)
        return fail(PIATTN_EINVAL, "dtype=%d is not PIATTN_F32 or PIATTN_BF16", (int)dtype);
    PiPattern p;
    int rc = check_pattern(pattern, &p);
    if (rc) return rc;
    if (p.bidir) return fail(PIATTN_EINVAL, "decode needs a causal pattern (bidirectional=0)");
    if (S < 1 || H < 1 || (int64_t)S * H > INT32_MAX)
        return fail(PIATTN_EINVAL, "S=%d H=%d out of range", S, H);
    if (cache_capacity < 1 || cache_capacity >= kMaxExtent - p.k)
        return fail(PIATTN_EINVAL, "cache_capacity=%d out of range", cache_capacity);
    if (rolling) {
        const int64_t need = rolling_slots_for(p);
        if (need < 0 || cache_capacity < need)
            return fail(PIATTN_EINVAL, "a rolling cache of %d rows is smaller than max(k, M*pi) + 1 = %lld",
                        cache_capacity, (long long)need);
    }
    if (d < 1) return fail(PIATTN_EINVAL, "d=%d must be positive", d);
    if (d != 32 && d != 64 && d != 128)
        return fail(PIATTN_EUNSUPPORTED, "d=%d unsupported (32, 64 or 128)", d);
    if (!strides) return fail(PIATTN_EINVAL, "strides is NULL");
    if (num_splits < 0 || num_splits > 64)
        return fail(PIATTN_EINVAL, "num_splits=%d out of range [0, 64]", num_splits);
    const int64_t mult = dtype == PIATTN_BF16 ? 8 : 4;
    int64_t sq[3] = {strides[0][0], strides[0][1], 0};
    int64_t so[3] = {strides[3][0], strides[3][1], 0};
    if ((rc = check_tensor("q", q, sq, mult, true))) return rc;
    if ((rc = check_tensor("k_cache", k_cache, strides[1], mult, true))) return rc;
    if ((rc = check_tensor("v_cache", v_cache, strides[2], mult, true))) return rc;
    if ((rc = check_tensor("out", out, so, mult, true))) return rc;
    if (!gate_logits || !aligned(gate_logits, 4))
        return fail(PIATTN_EINVAL, "gate_logits is NULL or misaligned");
    if (strides[4][0] < 0 || strides[4][1] < 0)
        return fail(PIATTN_EINVAL, "gate strides are negative");
    if (!cache_lens || !aligned(cache_lens, 4))
        return fail(PIATTN_EINVAL, "cache_lens is NULL or misaligned");
    if (out == q || out == k_cache || out == v_cache)
        return fail(PIATTN_EINVAL, "out aliases an input");

    const int splits = num_splits == 0 ? decode_splits_for(S, H, p) : num_splits;
    const size_t need = splits > 1 ? (size_t)S * H * splits * (d + 2) * sizeof(float) : 0;
    if (need) {
        if (!workspace) return fail(PIATTN_EWORKSPACE, "workspace is NULL (%zu bytes needed)", need);
        if (workspace_bytes < need)
            return fail(PIATTN_EWORKSPACE, "workspace of %zu bytes is smaller than %zu", workspace_bytes,
                        need);
        if (!aligned(workspace, 256)) return fail(PIATTN_EINVAL, "workspace is not 256-byte aligned");
    }
    const int64_t umax = (int64_t)p.k + 1 + p.M;

    DecodeArgs a;
    a.q = q;
    a.kc = k_cache;
    a.vc = v_cache;
    a.lens = cache_lens;
    a.g = gate_logits;
    a.o = out;
    a.ws = static_cast<float*>(workspace);
    a.sq = Str3{strides[0][0], strides[0][1], 0};
    a.sk = str3(strides[1]);
    a.sv = str3(strides[2]);
    a.so = Str3{strides[3][0], strides[3][1], 0};
    a.sg = Str3{strides[4][0], strides[4][1], 0};
    a.S = S;
    a.H = H;
    a.d = d;
    a.cap = cache_capacity;
    a.ring = rolling ? cache_capacity : 0;
    a.splits = splits;
    a.chunk = (int32_t)((umax + splits - 1) / splits);
    a.pat = p;
    a.scale_log2 = scale_log2(pattern, d);
    return launch_status(launch_decode(dtype == PIATTN_BF16 ? 1 : 0, a,
                                       static_cast<hipStream_t>(stream)));
}

extern "C" {

int piattn_decode(piattn_dtype dtype, int32_t S, int32_t H, int32_t d, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* cache_lens,
                  int32_t cache_capacity, const float* gate_logits, void* out,
                  const int64_t strides[5][3], const piattn_pattern* pattern, int32_t num_splits,
                  void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(dtype, S, H, d, q, k_cache, v_cache, cache_lens, cache_capacity, gate_logits, out,
                       strides, pattern, num_splits, workspace, workspace_bytes, stream, false);
}

int piattn_decode_rolling(piattn_dtype dtype, int32_t S, int32_t H, int32_t d, const void* q,
                          const void* k_cache, const void* v_cache, const int32_t* cache_lens,
                          int32_t cache_slots, const float* gate_logits, void* out,
                          const int64_t strides[5][3], const piattn_pattern* pattern, int32_t num_splits,
                          void* workspace, size_t workspace_bytes, void* stream) {
    return decode_impl(dtype, S, H, d, q, k_cache, v_cache, cache_lens, cache_slots, gate_logits, out,
                       strides, pattern, num_splits, workspace, workspace_bytes, stream, true);
}

int32_t piattn_rolling_slots(const piattn_pattern* pattern) {
    PiPattern p;
    if (check_pattern(pattern, &p) != PIATTN_OK) return -1;
    return (int32_t)rolling_slots_for(p);
}

int piattn_cache_append(piattn_dtype dtype, int32_t S, int32_t H, int32_t d, const void* k_new,
                        const void* v_new, void* k_cache, void* v_cache, const int32_t* positions,
                        int32_t cache_slots, const int64_t strides[4][3], void* stream) {
    if (dtype != PIATTN_F32 && dtype != PIATTN_BF16)
        return fail(PIATTN_EINVAL, "dtype=%d is not PIATTN_F32 or PIATTN_BF16", (int)dtype);
    if (S < 1 || H < 1 || (int64_t)S * H > INT32_MAX)
        return fail(PIATTN_EINVAL, "S=%d H=%d out of range", S, H);
    if (d < 1) return fail(PIATTN_EINVAL, "d=%d must be positive", d);
    if (d != 32 && d != 64 && d != 128)
        return fail(PIATTN_EUNSUPPORTED, "d=%d unsupported (32, 64 or 128)", d);
    if (cache_slots < 1) return fail(PIATTN_EINVAL, "cache_slots=%d must be positive", cache_slots);
    if (!strides) return fail(PIATTN_EINVAL, "strides is NULL");
    if (!positions || !aligned(positions, 4)) return fail(PIATTN_EINVAL, "positions is NULL or misaligned");
    const int64_t esz = dtype == PIATTN_BF16 ? 2 : 4;
    const void* ptrs[4] = {k_new, v_new, k_cache, v_cache};
    const char* names[4] = {"k_new", "v_new", "k_cache", "v_cache"};
    for (int t = 0; t < 4; ++t) {
        if (!ptrs[t] || !aligned(ptrs[t], esz)) return fail(PIATTN_EINVAL, "%s is NULL or misaligned", names[t]);
        for (int j = 0; j < 3; ++j)
            if (strides[t][j] < 0) return fail(PIATTN_EINVAL, "%s stride[%d] is negative", names[t], j);
    }
    if (k_cache == v_cache) return fail(PIATTN_EINVAL, "k_cache and v_cache are the same buffer");
    AppendArgs a;
    a.kn = k_new;
    a.vn = v_new;
    a.kc = k_cache;
    a.vc = v_cache;
    a.pos = positions;
    a.skn = Str3{strides[0][0], strides[0][1], 0};
    a.svn = Str3{strides[1][0], strides[1][1], 0};
    a.skc = str3(strides[2]);
    a.svc = str3(strides[3]);
    a.S = S;
    a.H = H;
    a.d = d;
    a.slots = cache_slots;
    return launch_status(launch_cache_append(dtype == PIATTN_BF16 ? 1 : 0, a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
