// pattern.hpp -- the one closed-form neighbour enumerator of libpiattn.
//
// Every kernel (neighbour dump, prefill, decode) derives its key lists from
// RowSpan, so the bit-exact check of the dump covers the compute kernels'
// index arithmetic too.
//
// pi-Attention pattern (gist.science "pi-Attention: Periodic Sparse
// Transformers ...", section 2 "Methodology", items "Ring-Local Attention"
// and "pi-Skip Attention"): query i of a length-n sequence sees the window
// [i-k, i] (causal) or [i-k, i+k] (bidirectional), clipped to [0, n), and
// the keys i -/+ m*pi for m = 1..M that lie in [0, n) and outside the
// window.  A multiple m*pi lies outside the window exactly when m*pi > k,
// i.e. m >= floor(k/pi) + 1, so the skips are a contiguous range of m.
#pragma once

#include <stdint.h>

struct PiPattern {
    int32_t k, pi, M, bidir;
};

struct RowSpan {
    int32_t lo, hi;  // local keys [lo, hi]
    int32_t mlo;     // smallest skip multiple outside the window
    int32_t mb;      // largest backward multiple (count max(0, mb - mlo + 1))
    int32_t mf;      // largest forward multiple (0 when causal)

    __host__ __device__ int32_t n_local() const { return hi - lo + 1; }
    __host__ __device__ int32_t n_back() const { return mb >= mlo ? mb - mlo + 1 : 0; }
    __host__ __device__ int32_t n_fwd() const { return mf >= mlo ? mf - mlo + 1 : 0; }
    __host__ __device__ int32_t total() const { return n_local() + n_back() + n_fwd(); }
    __host__ __device__ bool has_skip() const { return mb >= mlo || mf >= mlo; }
};

__host__ __device__ inline int32_t imin32(int32_t a, int32_t b) { return a < b ? a : b; }
__host__ __device__ inline int32_t imax32(int32_t a, int32_t b) { return a > b ? a : b; }

// Requires 0 <= i < n, k >= 0, pi >= 1, M >= 0 and n + k < 2^31.
__host__ __device__ inline RowSpan row_span(int32_t i, int32_t n, const PiPattern& p) {
    RowSpan r;
    r.lo = imax32(0, i - p.k);
    r.hi = p.bidir ? imin32(n - 1, i + p.k) : i;
    r.mlo = p.k / p.pi + 1;
    r.mb = imin32(p.M, i / p.pi);
    r.mf = p.bidir ? imin32(p.M, (n - 1 - i) / p.pi) : 0;
    return r;
}

// Union position u in [0, total) -> key index, ascending in u:
// backward skips (farthest first), the window, forward skips.
__host__ __device__ inline int32_t span_key(const RowSpan& r, int32_t i, int32_t pi, int32_t u,
                                            bool* is_local) {
    const int32_t nb = r.n_back(), nl = r.n_local();
    if (u < nb) {
        *is_local = false;
        return i - (r.mb - u) * pi;
    }
    u -= nb;
    if (u < nl) {
        *is_local = true;
        return r.lo + u;
    }
    u -= nl;
    *is_local = false;
    return i + (r.mlo + u) * pi;
}
