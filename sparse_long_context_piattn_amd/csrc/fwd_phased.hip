// fwd_phased.hip -- residue-tiled prefill for head dim 64, in two phases
// (gfx950, bf16 MFMA).
//
// Tile and ownership as in fwd_tiled.hip: a workgroup owns 64 consecutive
// residues [a0, a0+64) (residue a = i mod pi) over T = 8 consecutive periods
// (t = i div pi); each of its 8 waves owns one 16-residue a-group for 4 of the
// periods (TW = 4 row groups of 16 rows) and keeps their online-softmax state
// (running max m, partial sums l, fp32 O^T) in registers.
//
// Phase 1, ring-local windows (pi-Attention "Ring-Local Attention").  Step s
// stages the windows of periods t0 + 2s and t0 + 2s + 1 (rows
// [a0 + t pi - k, a0 + t pi + 64 (+k)) for each), so that every wave computes
// the window of its own row group j = s at every step: S^T = K Q^T on
// v_mfma_f32_16x16x32_bf16, mask, log(alpha) prior, online softmax,
// O^T += V^T P^T on 16x16x32.
//
// Phase 2, periodic skips ("pi-Skip Attention").  Each step stages the
// 64-row "own blocks" [a0 + t' pi, a0 + t' pi + 64) of G = 4 consecutive key
// periods t'.  For row group (period t) and staged period t' with t - t' = m in
// [floor(k/pi)+1, M] (or t' - t when bidirectional) the 16 rows' skip keys
// are the 16 rows of the a-group's part of the own block -- the diagonal of a
// 16 x 16 S^T tile.  The diagonal score (log(1-alpha) prior) joins the same
// online softmax ("Dynamic Adaptive Fusion"), lazily rescaled, and P being
// diagonal, O^T += V^T P^T is one 16x16x16 MFMA per 16 head-dim rows.
//
// Staging: global_load_lds_dwordx4 writes each lane's 16 bytes straight to
// LDS; two stage arrays alternate, the next step's rows are in flight while
// the current step computes.  Rows are XOR-swizzled by 16-byte chunk.  Rows a
// step does not need, or that fall outside the sequence, are filled from a
// clamped (valid) row and masked out.
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace {

constexpr int D = 64;
constexpr int NA = 4, AT = 64, PW = 2, TW = 4, T = PW * TW;
constexpr int CH = D / 8, DC = D / 32, DB = D / 16;
constexpr int RMAX = 128;                     // staged rows of one window
constexpr int G = 4;                          // own blocks per skip step
constexpr int SROWS = PW * RMAX;              // rows per stage (= G * AT)
constexpr int STAGE = 2 * SROWS * D;          // elements per stage: K rows then V rows
constexpr int DMA_PER_WAVE = 2 * SROWS * CH / (NW * 64);  // 16-byte loads per lane per stage
static_assert(SROWS == G * AT, "stage shapes");
static_assert(2 * SROWS * CH % (NW * 64) == 0, "stage split");

typedef __attribute__((address_space(3))) void lds_void_t;

struct Ctx {
    const uint16_t* Kb;
    const uint16_t* Vb;
    int32_t skt, svt;   // token strides (the host guarantees 32-bit element offsets)
    int32_t n;
};

// Issue the 16-byte LDS-direct loads of one stage.  Load i of wave w covers
// stage chunks [64 (w*DMA_PER_WAVE + i), +64); lane l takes chunk
// c0 + l, i.e. stage row c0/8 + l/8 and physical chunk l%8, which holds
// logical chunk (l%8) ^ (l/8) (rows are swizzled by row%8 and c0/8 is a
// multiple of 8).  Stage row r maps to sequence row row0(r) = base +
// off(r/64) + r%64, where off() is uniform per load; rows are clamped into
// [0, n) (out-of-range rows are masked by the consumer).
template <class Base>
__device__ __forceinline__ void dma_stage(uint16_t* stage, const Ctx& c, Base base) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int lhi = lane >> 3;
    const int lc8 = ((lane & 7) ^ lhi) << 3;       // element offset of the logical chunk
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int c0 = (wave * DMA_PER_WAVE + i) * 64;       // wave-uniform
        const bool isv = c0 >= SROWS * CH;
        const int r0 = (isv ? c0 - SROWS * CH : c0) >> 3;    // first stage row (multiple of 8)
        int32_t srow = base(r0) + lhi;                       // base(): uniform sequence row of stage row r0
        srow = imin32(imax32(srow, 0), c.n - 1);
        const uint16_t* src = isv ? c.Vb + (uint32_t)(srow * c.svt + lc8) : c.Kb + (uint32_t)(srow * c.skt + lc8);
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(stage + c0 * 8), 16, 0, 0);
    }
}

template <bool BIDIR>
__global__ __launch_bounds__(NT) void fwd_phased_kernel(FwdArgs a, int32_t a_tiles, int32_t t_tiles,
                                                        int32_t total_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t stA[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[STAGE];

    // XCD-aware order (see fwd_tiled.hip)
    const int32_t hw = blockIdx.x;
    const int32_t per = total_tiles / 8, rem = total_tiles % 8;
    const int32_t xcd = hw % 8, loc = hw / 8;
    const int32_t logical = (xcd < rem ? xcd * (per + 1) : rem * (per + 1) + (xcd - rem) * per) + loc;
    const int32_t at = logical % a_tiles;
    int32_t rest = logical / a_tiles;
    const int32_t tt = rest % t_tiles;
    rest /= t_tiles;
    const int32_t h = rest % a.H;
    const int32_t b = rest / a.H;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in SGPRs
    const int lane = tid & 63;
    const int x = lane & 15, g = lane >> 4;
    const int ga = wave % NA, wp = wave / NA;

    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) {
        tok0 = a.cu[b];
        n = a.cu[b + 1] - a.cu[b];
    }
    const int32_t pi = a.pat.pi, kw = a.pat.k, M = a.pat.M;
    const int32_t a0 = at * AT;
    if (a0 >= n) return;
    const int32_t P = (n - a0 + pi - 1) / pi;
    const int32_t t0 = tt * T;
    if (t0 >= P) return;
    const int32_t mlo = kw / pi + 1;
    const int32_t W = kw + 16 + (BIDIR ? kw : 0);
    const int32_t NB = (W + 15) >> 4;
    // key periods holding skip keys of the tile's rows
    const int32_t slo = imax32(0, t0 - M);
    const int32_t shi = imin32(P - 1, t0 + T - 1 + (BIDIR ? M : -mlo));
    const int32_t nss = (M >= mlo && shi >= slo) ? (shi - slo + G) / G : 0;

    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    Ctx cx;
    cx.Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    cx.Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    cx.skt = (int32_t)a.sk.t;
    cx.svt = (int32_t)a.sv.t;
    cx.n = n;
    uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    const int64_t gbase = bq * a.sg.s + h * a.sg.h + tok0 * a.sg.t;

    // window stage of phase-1 step s: window w = r/RMAX holds period t0 + 2s + w
    auto win_map = [=](int s) {
        return [=](int r) { return a0 + (t0 + PW * s + r / RMAX) * pi - kw + r % RMAX; };
    };
    // own-block stage of phase-2 step q: block r/AT holds period slo + G q + r/AT
    auto own_map = [=](int q) {
        return [=](int r) { return a0 + (slo + G * q + r / AT) * pi + r % AT; };
    };

    // ---- row groups of this wave: period t_j = t0 + wp + 2j
    bf16x8_t qf[TW][DC];
    f32x4_t acc[TW][DB];
    float mrun[TW], lrun[TW], pl[TW], ps[TW];
    int32_t ij[TW];
    bool qv[TW];
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const int32_t tj = t0 + wp + PW * j;
        ij[j] = a0 + 16 * ga + x + tj * pi;
        qv[j] = tj < P && ij[j] < n;
        const int32_t ic = qv[j] ? ij[j] : 0;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            uint4 u = make_uint4(0, 0, 0, 0);
            if (qv[j]) u = *reinterpret_cast<const uint4*>(Qb + (int64_t)ic * a.sq.t + 32 * c + 8 * g);
            qf[j][c] = as_bf16x8(u);
        }
        const RowSpan sp = row_span(ic, n, a.pat);
        const float gl = qv[j] ? a.g[gbase + (int64_t)ic * a.sg.t] : 0.0f;
        gate_priors(gl, sp.has_skip(), &pl[j], &ps[j]);
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) acc[j][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mrun[j] = -INFINITY;
        lrun[j] = 0.0f;
    }

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bool owner = g == (x >> 2);
    const int xr = x & 3;
    const uint2 dmask = make_uint2(owner ? (xr == 0 ? 0x0000ffffu : xr == 1 ? 0xffff0000u : 0u) : 0u,
                                   owner ? (xr == 2 ? 0x0000ffffu : xr == 3 ? 0xffff0000u : 0u) : 0u);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    // ---------------------------------------------------------- window step
    auto local = [&](int j, const uint16_t* st) {
        const int32_t tp = t0 + wp + PW * j;
        if (tp >= P) return;                          // wave-uniform
        const uint16_t* Ks = st;
        const uint16_t* Vs = st + SROWS * D;
        const int wrow0 = wp * RMAX + 16 * ga;         // stage row of this group's window start
        const int32_t i = ij[j];
        const int32_t key0 = tp * pi + a0 - kw + 16 * ga;
        const int32_t vlo = imax32(0, i - kw) - key0;
        const int32_t vhi = (qv[j] ? imin32(n - 1, BIDIR ? i + kw : i) : -1) - key0;
        const uint32_t vspan = (uint32_t)(vhi - vlo);
        const int32_t rel0 = 4 * g - vlo;
        constexpr int KBC = 4;
        for (int32_t kb0 = 0; kb0 < NB; kb0 += KBC) {
            float sc[KBC][4];
#pragma unroll
            for (int u = 0; u < KBC; ++u) {
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[u][r] = -INFINITY;
                if (kb0 + u < NB) {
                    const int rb = wrow0 + 16 * (kb0 + u);
                    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(Ks + swz<D>(rb + x, 4 * c + g));
                        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qf[j][c], s4, 0, 0, 0);
                    }
                    const int32_t relb = rel0 + 16 * (kb0 + u);
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        sc[u][r] = (uint32_t)(relb + r) <= vspan ? fmaf(s4[r], sl2, pl[j]) : -INFINITY;
                }
            }
            float mx = -INFINITY;
#pragma unroll
            for (int u = 0; u < KBC; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) mx = fmaxf(mx, sc[u][r]);
            mx = max4(mx);
            const float mnew = fmaxf(mrun[j], mx);
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            const float fac = exp2_fast(mrun[j] - mu);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) acc[j][bb] *= fac;
            lrun[j] *= fac;
            mrun[j] = mnew;
            s16x4_t pb[KBC];
#pragma unroll
            for (int u = 0; u < KBC; ++u) {
                if (kb0 + u < NB) {
                    const uint32_t w0 = cvt_pk_bf16(exp2_fast(sc[u][0] - mu), exp2_fast(sc[u][1] - mu));
                    const uint32_t w1 = cvt_pk_bf16(exp2_fast(sc[u][2] - mu), exp2_fast(sc[u][3] - mu));
                    pb[u] = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
                } else {
                    pb[u] = s16x4_t{0, 0, 0, 0};
                }
            }
            f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < KBC; u += 2) {
                if (kb0 + u >= NB) continue;
                const int rb = wrow0 + 16 * (kb0 + u);
                if (kb0 + u + 1 < NB) {
                    const bf16x8_t pp = __builtin_bit_cast(
                        bf16x8_t, __builtin_shufflevector(pb[u], pb[u + 1], 0, 1, 2, 3, 4, 5, 6, 7));
                    lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pp, lsum, 0, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb) {
                        const s16x4_t v0 = ld_tr16(Vs + swz<D>(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        const s16x4_t v1 =
                            ld_tr16(Vs + swz<D>(rb + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        const bf16x8_t va =
                            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp, acc[j][bb], 0, 0, 0);
                    }
                } else {
                    lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb[u], lsum, 0, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb) {
                        const s16x4_t v0 = ld_tr16(Vs + swz<D>(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pb[u], acc[j][bb], 0, 0, 0);
                    }
                }
            }
            lrun[j] += 0.25f * lsum[0];   // quarter per lane; sum4 at the end restores the row sum
        }
    };

    // ---------------------------------------------------------- skip step
    auto skips = [&](int q, const uint16_t* st) {
        const uint16_t* Ks = st;
        const uint16_t* Vs = st + SROWS * D;
#pragma unroll
        for (int bk = 0; bk < G; ++bk) {
            const int32_t tp = slo + G * q + bk;
            if (tp > shi) break;                      // wave-uniform
            bool sk[TW];
            bool any_sk = false;
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                const int32_t tj = t0 + wp + PW * j;
                const int32_t delta = tj - tp;
                const int32_t m = delta > 0 ? delta : -delta;
                sk[j] = m >= mlo && m <= M && (delta > 0 || (BIDIR && delta < 0)) && tj < P;
                any_sk |= sk[j];
            }
            if (!any_sk) continue;
            const int ro = AT * bk + 16 * ga;          // stage row of the a-group's own rows
            const bool own_key_ok = a0 + 16 * ga + x + tp * pi < n;
            bf16x8_t kf[DC];
#pragma unroll
            for (int c = 0; c < DC; ++c) kf[c] = *reinterpret_cast<const bf16x8_t*>(Ks + swz<D>(ro + x, 4 * c + g));
            float sd[TW];
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < DC; ++c) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[j][c], s4, 0, 0, 0);
                const float v = diag_pick(s4, xr);
                sd[j] = (owner && sk[j] && qv[j] && own_key_ok) ? fmaf(v, sl2, ps[j]) : -INFINITY;
            }
            bool need_any = false;
#pragma unroll
            for (int j = 0; j < TW; ++j) need_any |= sd[j] > mrun[j] + LAZY;
            if (__any(need_any)) {
                // rare: raise the running max of rows whose skip score exceeds
                // it by more than LAZY (broadcast from the diagonal-owner lane)
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const float sb = max4(sd[j]);
                    const bool need = sb > mrun[j] + LAZY;
                    const float mnew = need ? sb : mrun[j];
                    const float fac = need ? exp2_fast(mrun[j] - mnew) : 1.0f;
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb) acc[j][bb] *= fac;
                    lrun[j] *= fac;
                    mrun[j] = mnew;
                }
            }
            s16x4_t vf[DB];
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) vf[bb] = ld_tr16(Vs + swz<D>(ro + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                if (!sk[j]) continue;                 // wave-uniform
                const float p = (sd[j] == -INFINITY) ? 0.0f : exp2_fast(sd[j] - mrun[j]);
                const uint32_t pw = cvt_pk_bf16(p, p);
                lrun[j] += __uint_as_float(pw << 16);  // owner lane only (others add 0)
                const s16x4_t pbv = __builtin_bit_cast(s16x4_t, make_uint2(pw & dmask.x, pw & dmask.y));
#pragma unroll
                for (int bb = 0; bb < DB; ++bb)
                    acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[bb], pbv, acc[j][bb], 0, 0, 0);
            }
        }
    };

    // ---------------------------------------------------------- schedule
    // Steps alternate between stA and stB; the next step's rows are loaded
    // (asynchronously, straight to LDS) while the current step computes.
    // __syncthreads() both waits for this wave's loads and publishes them.
    dma_stage(stA, cx, win_map(0));
    __syncthreads();
    dma_stage(stB, cx, win_map(1));
    local(0, stA);
    __syncthreads();
    dma_stage(stA, cx, win_map(2));
    local(1, stB);
    __syncthreads();
    dma_stage(stB, cx, win_map(3));
    local(2, stA);
    __syncthreads();
    if (nss > 0) dma_stage(stA, cx, own_map(0));
    local(3, stB);
    for (int q = 0; q < nss; q += 2) {
        __syncthreads();
        if (q + 1 < nss) dma_stage(stB, cx, own_map(q + 1));
        skips(q, stA);
        if (q + 1 >= nss) break;
        __syncthreads();
        if (q + 2 < nss) dma_stage(stA, cx, own_map(q + 2));
        skips(q + 1, stB);
    }

    // ---- normalise and store (bf16, round to nearest even)
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const float ltot = sum4(lrun[j]);
        if (!qv[j]) continue;
        const float inv = 1.0f / ltot;
        uint16_t* orow = Ob + (int64_t)ij[j] * a.so.t;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) {
            uint2 w;
            w.x = cvt_pk_bf16(acc[j][bb][0] * inv, acc[j][bb][1] * inv);
            w.y = cvt_pk_bf16(acc[j][bb][2] * inv, acc[j][bb][3] * inv);
            *reinterpret_cast<uint2*>(orow + 16 * bb + 4 * g) = w;
        }
        if (a.lse && g == 0) a.lse[gbase + (int64_t)ij[j] * a.sg.t] = (mrun[j] + __log2f(ltot)) * PIATTN_LN2;
    }
}

template <bool BIDIR>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    const int32_t a_tiles = a.pat.pi / AT;
    const int32_t periods = (a.n + a.pat.pi - 1) / a.pat.pi;
    const int32_t t_tiles = (periods + T - 1) / T;
    const int64_t total = (int64_t)a_tiles * t_tiles * a.H * a.B;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_phased_kernel<BIDIR>), dim3((uint32_t)total), dim3(NT), 0, stream, a, a_tiles,
                       t_tiles, (int32_t)total);
    return hipGetLastError();
}

}  // namespace

bool fwd_phased_supported(int dtype, const FwdArgs& a) {
    if (dtype != 1 || a.d != 64 || a.pat.pi % AT != 0) return false;
    // staging addresses are 32-bit element offsets from the (sequence, head) base
    const int64_t ts = a.sk.t > a.sv.t ? a.sk.t : a.sv.t;
    if ((int64_t)a.n * ts + D >= ((int64_t)1 << 31)) return false;
    const int64_t w = (int64_t)a.pat.k + 16 + (a.pat.bidir ? a.pat.k : 0);
    return 16 * (NA - 1) + 16 * ((w + 15) / 16) <= RMAX;
}

hipError_t launch_fwd_phased(const FwdArgs& a, hipStream_t stream) {
    return a.pat.bidir ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}
