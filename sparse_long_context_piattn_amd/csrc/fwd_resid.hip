// fwd_resid.hip -- residue-tiled prefill for head dim 64 with the periodic
// skips computed as a dense band in residue layout (gfx950, bf16 MFMA).
//
// Write a query row as i = a + t*pi (residue a = i mod pi, period t).  A
// workgroup owns 64 residues [a0, a0+64) x T = 8 periods [t0, t0+8): 512
// rows, 16 row groups of 16 rows (one period, 16 consecutive residues).  Each
// of the 8 waves owns the 4 row groups of one 16-residue a-group and a period
// parity, and keeps their online-softmax state (max m, per-lane partial sums
// l, fp32 O^T) in registers.
//
// Phase 1, ring-local windows (pi-Attention "Ring-Local Attention"): step s
// stages the windows of periods t0+2s and t0+2s+1 ([a0 + t pi - k,
// a0 + t pi + 64 (+k)) each) and every wave runs its group's band on MFMA.
//
// Phase 2, periodic skips ("pi-Skip Attention").  The skip keys of row
// (a, t) are (a, t - m) -- same residue, earlier (and, bidirectional, later)
// periods -- so for one residue they form a band of width M over the
// pi-strided sequence.  For each a-group (16 residues), LDS stages hold 16
// key periods x 16 residues of K and V; an "item" is one residue with its T
// query periods as the MFMA query columns, and S^T = K Q^T, the band mask,
// the log(1-alpha) prior, an online softmax and O^T += V^T P^T run densely
// on MFMA.  When an a-group's key periods are done, its items' partial states
// (m, l, O^T) pass through a small LDS buffer into the row groups' registers,
// merged exactly (m = max, O and l rescaled by 2^(m_part - m)).  One softmax
// over window and skips results ("Dynamic Adaptive Fusion").
//
// Staging: global_load_lds_dwordx4 into two alternating LDS stages (the
// next stage's rows are in flight while the current one computes); rows are
// XOR-swizzled by 16-byte chunk with key (row ^ row/16) % 8 so that both
// consecutive rows and rows 16 apart spread over the banks.  Rows outside
// the sequence are filled from a clamped valid row and masked out.
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace {

constexpr int D = 64;
constexpr int NA = 4, AT = 64, PW = 2, TW = 4, T = PW * TW;
constexpr int CH = D / 8, DC = D / 32, DB = D / 16;
constexpr int RMAX = 128;                     // staged rows of one window
constexpr int SROWS = 256;                    // rows per stage (2 windows, or 16 periods x 16 residues)
constexpr int STAGE = 2 * SROWS * D;          // elements per stage: K rows then V rows
constexpr int DMA_PER_WAVE = 2 * SROWS * CH / (NW * 64);
constexpr int IW = 2;                         // skip items (residues) per wave
constexpr int REC = 4 + D / 2;                // merge record: m, l, 2 pad, half of O^T
constexpr int RSTR = T * REC + 4;             // records of one residue (padded against bank conflicts)
static_assert(2 * SROWS * CH % (NW * 64) == 0, "stage split");
static_assert(T <= 16, "query columns");

typedef __attribute__((address_space(3))) void lds_void_t;

// Element offset of 16-byte chunk c of stage row r.
__device__ __forceinline__ int sw(int r, int c) { return r * D + ((c ^ ((r ^ (r >> 4)) & 7)) << 3); }

struct Ctx {
    const uint16_t* Kb;
    const uint16_t* Vb;
    int32_t skt, svt, n;
};

// One stage of LDS-direct loads.  Load i of wave w covers stage chunks
// [64 (w*DMA_PER_WAVE + i), +64): rows r0 .. r0+7 (r0 a multiple of 8), lane l
// taking row r0 + l/8 and physical chunk l%8.  base(r0) is the sequence row
// of stage row r0; rows r0..r0+7 are consecutive sequence rows.
template <class Base>
__device__ __forceinline__ void dma_stage(uint16_t* stage, const Ctx& c, Base base) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const int lhi = lane >> 3;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int c0 = (wave * DMA_PER_WAVE + i) * 64;
        const bool isv = c0 >= SROWS * CH;
        const int r0 = (isv ? c0 - SROWS * CH : c0) >> 3;
        const int key = (lhi ^ (r0 >> 4)) & 7;          // swizzle key of row r0 + lhi
        const int lc8 = ((lane & 7) ^ key) << 3;
        int32_t srow = base(r0) + lhi;
        srow = imin32(imax32(srow, 0), c.n - 1);
        const uint16_t* src = isv ? c.Vb + (uint32_t)(srow * c.svt + lc8) : c.Kb + (uint32_t)(srow * c.skt + lc8);
        __builtin_amdgcn_global_load_lds(src, (lds_void_t*)(stage + c0 * 8), 16, 0, 0);
    }
}

template <bool BIDIR>
__global__ __launch_bounds__(NT) void fwd_resid_kernel(FwdArgs a, int32_t a_tiles, int32_t t_tiles,
                                                       int32_t total_tiles) {
    __shared__ __attribute__((aligned(16))) uint16_t stA[STAGE];
    __shared__ __attribute__((aligned(16))) uint16_t stB[STAGE];
    __shared__ __attribute__((aligned(16))) float mrec[16 * RSTR];

    // XCD-aware order: each XCD gets a contiguous run of logical tiles.
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
    // key periods of the tile's skips, in blocks of 16
    const int32_t klo = imax32(0, t0 - M);
    const int32_t khi = imin32(P - 1, t0 + T - 1 + (BIDIR ? M : -mlo));
    const int32_t nkb = (M >= mlo && khi >= klo) ? (khi - klo + 16) >> 4 : 0;
    const int32_t nss = NA * nkb;                  // skip steps: a-group major, key block minor

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

    auto win_map = [=](int s) {
        return [=](int r) { return a0 + (t0 + PW * s + r / RMAX) * pi - kw + r % RMAX; };
    };
    // skip step q: a-group q / nkb, key block q % nkb; stage row 16u + xx holds
    // residue a0 + 16*ag + xx of key period klo + 16*kb + u
    auto own_map = [=](int q) {
        const int ag = q / nkb, kb = q % nkb;
        return [=](int r) { return a0 + 16 * ag + (klo + 16 * kb + (r >> 4)) * pi + (r & 15); };
    };

    // ---- row groups of this wave: period t_j = t0 + wp + 2j
    bf16x8_t qf[TW][DC];
    f32x4_t acc[TW][DB];
    float mrun[TW], lrun[TW], pl[TW];
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
        float psk;
        gate_priors(gl, sp.has_skip(), &pl[j], &psk);
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) acc[j][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        mrun[j] = -INFINITY;
        lrun[j] = 0.0f;
    }

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    // ---------------------------------------------------------- window step
    auto local = [&](int j, const uint16_t* st) {
        const int32_t tp = t0 + wp + PW * j;
        if (tp >= P) return;                          // wave-uniform
        const uint16_t* Ks = st;
        const uint16_t* Vs = st + SROWS * D;
        const int wrow0 = wp * RMAX + 16 * ga;
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
                        const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(Ks + sw(rb + x, 4 * c + g));
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
                for (int r = 0; r < 4; ++r) mx = mx > sc[u][r] ? mx : sc[u][r];
            mx = max4(mx);
            const float mnew = mrun[j] > mx ? mrun[j] : mx;
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
                        const s16x4_t v0 = ld_tr16(Vs + sw(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        const s16x4_t v1 = ld_tr16(Vs + sw(rb + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        const bf16x8_t va =
                            __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp, acc[j][bb], 0, 0, 0);
                    }
                } else {
                    lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb[u], lsum, 0, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb) {
                        const s16x4_t v0 = ld_tr16(Vs + sw(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pb[u], acc[j][bb], 0, 0, 0);
                    }
                }
            }
            lrun[j] += 0.25f * lsum[0];   // quarter per lane; sum4 at the end restores the row sum
        }
    };

    // ---------------------------------------------------------- skip items
    // Item it of this wave: residue xr = a0 + 16*ag + 2*wave + it; query
    // column col = lane % 16 is period t0 + col (valid for col < T).
    bf16x8_t sq[IW][DC];
    f32x4_t sacc[IW][DB];
    float sm[IW], sl[IW], sps[IW];
    bool sqv[IW];
    const int col = x;
    auto item_begin = [&](int ag) {
#pragma unroll
        for (int it = 0; it < IW; ++it) {
            const int32_t tq = t0 + col;
            const int32_t iq = a0 + 16 * ag + 2 * wave + it + tq * pi;
            sqv[it] = col < T && tq < P && iq < n;
            const int32_t ic = sqv[it] ? iq : 0;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                uint4 u = make_uint4(0, 0, 0, 0);
                if (sqv[it]) u = *reinterpret_cast<const uint4*>(Qb + (int64_t)ic * a.sq.t + 32 * c + 8 * g);
                sq[it][c] = as_bf16x8(u);
            }
            const RowSpan sp = row_span(ic, n, a.pat);
            const float gl = sqv[it] ? a.g[gbase + (int64_t)ic * a.sg.t] : 0.0f;
            float plk;
            gate_priors(gl, sp.has_skip(), &plk, &sps[it]);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) sacc[it][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            sm[it] = -INFINITY;
            sl[it] = 0.0f;
        }
    };
    auto item_block = [&](int ag, int kb, const uint16_t* st) {
        const uint16_t* Ks = st;
        const uint16_t* Vs = st + SROWS * D;
        const int32_t tq = t0 + col;
        const int32_t kp0 = klo + 16 * kb + 4 * g;      // key period of this lane's value r = 0
#pragma unroll
        for (int it = 0; it < IW; ++it) {
            const int xx = 2 * wave + it;                // residue within the a-group
            f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(Ks + sw(16 * x + xx, 4 * c + g));
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, sq[it][c], s4, 0, 0, 0);
            }
            float sc[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int32_t kp = kp0 + r;
                const int32_t delta = tq - kp;
                const int32_t m = delta > 0 ? delta : -delta;
                const bool band = m >= mlo && m <= M && (delta > 0 || (BIDIR && delta < 0));
                const bool ok = band && sqv[it] && kp <= khi && a0 + 16 * ag + xx + kp * pi < n;
                sc[r] = ok ? fmaf(s4[r], sl2, sps[it]) : -INFINITY;
            }
            float mx = sc[0] > sc[1] ? sc[0] : sc[1];
            const float mx2 = sc[2] > sc[3] ? sc[2] : sc[3];
            mx = max4(mx > mx2 ? mx : mx2);
            const float mnew = sm[it] > mx ? sm[it] : mx;
            const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
            const float fac = exp2_fast(sm[it] - mu);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) sacc[it][bb] *= fac;
            sl[it] *= fac;
            sm[it] = mnew;
            const uint32_t w0 = cvt_pk_bf16(exp2_fast(sc[0] - mu), exp2_fast(sc[1] - mu));
            const uint32_t w1 = cvt_pk_bf16(exp2_fast(sc[2] - mu), exp2_fast(sc[3] - mu));
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
            const f32x4_t ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
            sl[it] += ls[0];                         // full column sum in every lane
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) {
                const s16x4_t vv = ld_tr16(Vs + sw(16 * tr_row + xx, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                sacc[it][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, pb, sacc[it][bb], 0, 0, 0);
            }
        }
    };
    // Fold the items' partial states for a-group ag into the row groups'
    // registers, half of the head dimension per pass.
    auto item_merge = [&](int ag) {
        float fl[TW], fs[TW];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
            __syncthreads();                          // buffer free (previous pass read)
#pragma unroll
            for (int it = 0; it < IW; ++it) {
                if (col < T) {
                    float* rp = mrec + (2 * wave + it) * RSTR + col * REC;
                    if (g == 0 && hh == 0) {
                        rp[0] = sm[it];
                        rp[1] = sl[it];
                    }
#pragma unroll
                    for (int q = 0; q < DB / 2; ++q) {
                        const int bb = hh * (DB / 2) + q;
                        *reinterpret_cast<f32x4_t*>(rp + 4 + 16 * q + 4 * g) = sacc[it][bb];
                    }
                }
            }
            __syncthreads();
            if (ga == ag) {
#pragma unroll
                for (int j = 0; j < TW; ++j) {
                    const int cj = wp + PW * j;             // column of row group j
                    const float* rp = mrec + x * RSTR + cj * REC;
                    if (hh == 0) {
                        const float msk = rp[0], lsk = rp[1];
                        const float mnew = mrun[j] > msk ? mrun[j] : msk;
                        const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
                        fl[j] = exp2_fast(mrun[j] - mu);
                        fs[j] = exp2_fast(msk - mu);
                        lrun[j] = lrun[j] * fl[j] + 0.25f * lsk * fs[j];
                        mrun[j] = mnew;
                    }
#pragma unroll
                    for (int q = 0; q < DB / 2; ++q) {
                        const int bb = hh * (DB / 2) + q;
                        const f32x4_t sv = *reinterpret_cast<const f32x4_t*>(rp + 4 + 16 * q + 4 * g);
                        acc[j][bb] = acc[j][bb] * fl[j] + sv * fs[j];
                    }
                }
            }
        }
    };
    auto sstep = [&](int q, const uint16_t* st) {
        const int ag = q / nkb, kb = q % nkb;
        if (kb == 0) item_begin(ag);
        item_block(ag, kb, st);
        if (kb == nkb - 1) item_merge(ag);         // workgroup-uniform
    };

    // ---------------------------------------------------------- schedule
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
        sstep(q, stA);
        if (q + 1 >= nss) break;
        __syncthreads();
        if (q + 2 < nss) dma_stage(stA, cx, own_map(q + 2));
        sstep(q + 1, stB);
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
    hipLaunchKernelGGL((fwd_resid_kernel<BIDIR>), dim3((uint32_t)total), dim3(NT), 0, stream, a, a_tiles,
                       t_tiles, (int32_t)total);
    return hipGetLastError();
}

}  // namespace

bool fwd_resid_supported(int dtype, const FwdArgs& a) {
    if (dtype != 1 || a.d != 64 || a.pat.pi % AT != 0) return false;
    const int64_t ts = a.sk.t > a.sv.t ? a.sk.t : a.sv.t;
    if ((int64_t)a.n * ts + D >= ((int64_t)1 << 31)) return false;
    const int64_t w = (int64_t)a.pat.k + 16 + (a.pat.bidir ? a.pat.k : 0);
    return 16 * (NA - 1) + 16 * ((w + 15) / 16) <= RMAX;
}

hipError_t launch_fwd_resid(const FwdArgs& a, hipStream_t stream) {
    return a.pat.bidir ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}
