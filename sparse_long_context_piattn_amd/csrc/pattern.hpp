// pattern.hpp -- the closed-form neighbour enumerator of libpiattn.
//
// The neighbour dump, the gather prefill and backward kernels and decode
// walk their key lists through RowSpan.  The MFMA kernels (the split skip and
// window passes, the residue-tiled kernel, the band backward) do not: they
// test block membership with their own range arithmetic over 16-key blocks.
// Each kernel's membership is therefore checked on its own, bit-exactly,
// through its outputs (a probe key that dominates its row's scores, read back
// per row and kind), besides the dump's check of RowSpan.
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

// Skip schedules (the hierarchical skip schedules the Dutch gist.science
// summary names as future work, section 5 "Betekenis en Conclusie"): the skip
// sets of several levels (pi_r, M_r) are unioned.  The host reduces a
// schedule to its base period pi = gcd of the periods and the set of skip
// multiples m (distances m*pi beyond the window), held as a 128-bit mask; a
// single-period pattern keeps the contiguous range [floor(k/pi)+1, M].
constexpr int32_t kMaskBits = 128;

struct PiPattern {
    int32_t k, pi, M, bidir;
    int32_t mlo;        // smallest skip multiple (floor(k/pi)+1, or the mask's lowest bit)
    int32_t masked;     // 1: the skip multiples are the set bits of mask; M is the highest
    uint32_t mask[4];   // bit m: m*pi is a skip distance (masked patterns only)
};

__host__ __device__ inline int32_t imin32(int32_t a, int32_t b) { return a < b ? a : b; }
__host__ __device__ inline int32_t imax32(int32_t a, int32_t b) { return a > b ? a : b; }

// Word w of the mask with a constant index pattern (no dynamic indexing into
// the kernel argument, which would go through scratch memory).
__host__ __device__ inline uint32_t mask_word(const PiPattern& p, int32_t w) {
    const uint32_t a = (w & 1) ? p.mask[1] : p.mask[0];
    const uint32_t b = (w & 1) ? p.mask[3] : p.mask[2];
    return (w & 2) ? b : a;
}

// Whether multiple m (0 <= m) is in the mask.
__host__ __device__ inline bool mask_has(const PiPattern& p, int32_t m) {
    return (uint32_t)m < (uint32_t)kMaskBits && ((mask_word(p, m >> 5) >> (m & 31)) & 1u);
}

// Number of set multiples <= lim.
__host__ __device__ inline int32_t mask_rank(const PiPattern& p, int32_t lim) {
    if (lim < 0) return 0;
    if (lim >= kMaskBits) lim = kMaskBits - 1;
    int32_t c = 0;
    for (int32_t w = 0; w < 4; ++w) {
        const int32_t base = 32 * w;
        if (base > lim) break;
        uint32_t v = mask_word(p, w);
        if (lim - base < 31) v &= (2u << (lim - base)) - 1u;
        c += __builtin_popcount(v);
    }
    return c;
}

// The r-th smallest set multiple (0 <= r < popcount).
__host__ __device__ inline int32_t mask_select(const PiPattern& p, int32_t r) {
    int32_t w = 0;
    uint32_t v = mask_word(p, 0);
    for (; w < 3; ++w) {
        const int32_t c = __builtin_popcount(v);
        if (r < c) break;
        r -= c;
        v = mask_word(p, w + 1);
    }
    int32_t pos = 32 * w;
    for (int32_t sh = 16; sh > 0; sh >>= 1) {
        const int32_t c = __builtin_popcount(v & ((1u << sh) - 1u));
        if (c <= r) {
            r -= c;
            v >>= sh;
            pos += sh;
        }
    }
    return pos;
}

struct RowSpan {
    int32_t lo, hi;  // local keys [lo, hi]
    int32_t nb, nf;  // backward / forward skip keys

    __host__ __device__ int32_t n_local() const { return hi - lo + 1; }
    __host__ __device__ int32_t n_back() const { return nb; }
    __host__ __device__ int32_t n_fwd() const { return nf; }
    __host__ __device__ int32_t total() const { return n_local() + nb + nf; }
    __host__ __device__ bool has_skip() const { return nb + nf > 0; }
};

// The enumeration comes in two compile-time forms, MASKED (a schedule's
// mask) and not (the range [mlo, M]), so that the gather kernels of plain
// patterns carry none of the mask code; the runtime forms below dispatch.

// Number of skip multiples m <= lim (lim = the largest that fits in range).
template <bool MASKED>
__host__ __device__ inline int32_t skips_upto_t(const PiPattern& p, int32_t lim) {
    if (MASKED) return mask_rank(p, imin32(lim, p.M));
    return imax32(0, imin32(p.M, lim) - p.mlo + 1);
}

// The r-th smallest skip multiple (r < skips_upto(p, M)).
template <bool MASKED>
__host__ __device__ inline int32_t skip_multiple_t(const PiPattern& p, int32_t r) {
    return MASKED ? mask_select(p, r) : p.mlo + r;
}

// Requires 0 <= i < n, k >= 0, pi >= 1, M >= 0 and n + k < 2^31.
template <bool MASKED>
__host__ __device__ inline RowSpan row_span_t(int32_t i, int32_t n, const PiPattern& p) {
    RowSpan r;
    r.lo = imax32(0, i - p.k);
    r.hi = p.bidir ? imin32(n - 1, i + p.k) : i;
    r.nb = skips_upto_t<MASKED>(p, i / p.pi);
    r.nf = p.bidir ? skips_upto_t<MASKED>(p, (n - 1 - i) / p.pi) : 0;
    return r;
}

// Union position u in [0, total) -> key index, ascending in u:
// backward skips (farthest first), the window, forward skips.
template <bool MASKED>
__host__ __device__ inline int32_t span_key_t(const RowSpan& r, int32_t i, const PiPattern& p, int32_t u,
                                              bool* is_local) {
    const int32_t nb = r.nb, nl = r.n_local();
    if (u < nb) {
        *is_local = false;
        return i - skip_multiple_t<MASKED>(p, nb - 1 - u) * p.pi;
    }
    u -= nb;
    if (u < nl) {
        *is_local = true;
        return r.lo + u;
    }
    u -= nl;
    *is_local = false;
    return i + skip_multiple_t<MASKED>(p, u) * p.pi;
}

__host__ __device__ inline int32_t skips_upto(const PiPattern& p, int32_t lim) {
    return p.masked ? skips_upto_t<true>(p, lim) : skips_upto_t<false>(p, lim);
}
__host__ __device__ inline int32_t skip_multiple(const PiPattern& p, int32_t r) {
    return p.masked ? skip_multiple_t<true>(p, r) : skip_multiple_t<false>(p, r);
}
__host__ __device__ inline RowSpan row_span(int32_t i, int32_t n, const PiPattern& p) {
    return p.masked ? row_span_t<true>(i, n, p) : row_span_t<false>(i, n, p);
}
__host__ __device__ inline int32_t span_key(const RowSpan& r, int32_t i, const PiPattern& p, int32_t u,
                                            bool* is_local) {
    return p.masked ? span_key_t<true>(r, i, p, u, is_local) : span_key_t<false>(r, i, p, u, is_local);
}
