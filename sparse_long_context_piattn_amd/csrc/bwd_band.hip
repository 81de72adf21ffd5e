// bwd_band.hip -- backward of the prefill on bf16 MFMA for head dim 64 or
// 128 (gfx950): a row-record kernel, then two passes of one banded kernel,
// the skip keys in residue layout and then the window in sequence layout.
//
// With the forward's log-sum-exp lse_i (natural log, from piattn_fwd's
// lse_out) the softmax of row i is P_ij = exp2(s_ij + c_i), where
// s_ij = scale log2(e) <q_i, k_j> and c_i = prior - lse_i log2(e).  The
// prior is log2(alpha_i) on window keys and log2(1 - alpha_i) on skip keys,
// and 0 on rows without skip keys (pi-Attention "Dynamic Adaptive Fusion").
// With D_i = <dout_i, out_i>:
//   dS_ij = P_ij (<dout_i, v_j> - D_i),
//   dq_i = scale sum_j dS_ij k_j,   dk_j = scale sum_i dS_ij q_i,
//   dv_j = sum_i P_ij dout_i.
// Every one of these sums splits exactly into a window part and a skip
// part that share only lse_i and D_i, so the two parts run separately.
//
// bwd_record_kernel: each row's record {D_i, c_i (window), c_i (skip)}.
// When every residue view is one tile long the skip pass forms these
// records itself (REC below) and this kernel does not run.
//
// bwd_band_kernel: a view is the rows of one sequence at positions
// base + p step, p = 0 .. L-1: the whole sequence (step 1) for the window,
// one residue class (base a < pi, step pi) for the skips, whose keys
// i -/+ m pi, m in [floor(k/pi)+1, M], are then the view rows p -/+ m.
// Both parts are a band: query p sees key p' when p - p' lies in
// [dlo, dhi] (and, for bidirectional skips, |p - p'| >= floor(k/pi)+1).
// A workgroup owns the 64 rows of view tile t, as queries and as keys:
//   phase A  the key tiles of t's band stream through two LDS slots; each
//            wave takes 16 query rows: S^T = K Q^T and dP^T = V dO^T on
//            v_mfma_f32_16x16x32_bf16, P and dS in fp32, dq^T += K^T dS^T;
//   phase B  the query tiles whose band holds t stream through the same
//            slots (Q, dO and the rows' records); each wave takes 16 key
//            rows: S = Q K^T, dP = dO V^T, dv^T += dO^T P, dk^T += Q^T dS.
// A block pair is computed in both phases (the MFMA work is small next to
// the memory traffic), so no partial sum crosses workgroups.  The skip pass
// stores its dq, dk, dv as bf16 partials in the gradient rows and each row's
// skip sum of dS in its record; the window pass adds the partials and forms
// the gate gradient (1 - alpha) sum_L dS - alpha sum_S dS.
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace {

constexpr int BT = 64;    // rows per tile of the skip pass (query side and key side)
// Rows per tile of the window pass.  128-row tiles on eight waves (fewer
// halo rows per own row) measured 5-14% slower: eight waves meet at every
// barrier.
constexpr int BTW = 64;

// Per-row record in the workspace.
struct alignas(16) RowRec {
    float D;    // <dout_i, out_i>
    float cw;   // window keys: prior - lse2
    float cs;   // skip keys: prior - lse2
    float ss;   // sum of dS over the skip keys (written by the skip pass)
};

struct SeqLoc {
    int64_t tok0;
    int64_t bq;
    int32_t n;
};

__device__ __forceinline__ SeqLoc seq_loc(const FwdArgs& a, int32_t b) {
    SeqLoc r;
    r.n = a.n;
    r.tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &r.tok0, &r.n);
    }
    r.bq = a.cu ? 0 : (int64_t)b;
    return r;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One record per row: D_i = <dout_i, out_i> over D/8 lanes (16 bytes each),
// and c_i = prior - lse_i log2(e) for both key kinds.  A wave takes RG
// groups of 64 / (D/8) rows and issues all their loads (out, dout, gate,
// lse) before the first product: one memory round trip per wave.
constexpr int RG = 4;
template <int D>
__global__ __launch_bounds__(256) void bwd_record_kernel(BwdArgs ba) {
    constexpr int LPK = D / 8, NS = 64 / LPK;
    const FwdArgs& a = ba.f;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = lane / LPK, c = (lane % LPK) * 8;
    const int32_t h = blockIdx.y, b = blockIdx.z;
    const SeqLoc sl = seq_loc(a, b);
    if (sl.n < 1) return;
    uint4 o[RG], g[RG];
    float gl[RG], ls[RG];
    int32_t row[RG];
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const int32_t i0 = ((blockIdx.x * 4 + wave) * RG + r) * NS + slot;
        row[r] = i0;
        const int32_t i = i0 < sl.n ? i0 : sl.n - 1;
        const int64_t tok = sl.tok0 + i;
        const int64_t orow = sl.bq * a.so.s + h * a.so.h + tok * a.so.t + c;
        const int64_t goff = sl.bq * a.sg.s + h * a.sg.h + tok * a.sg.t;
        o[r] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.o) + orow);
        g[r] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(ba.dout) + orow);
        gl[r] = a.g[goff];                                     // every lane of the row: one address
        ls[r] = ba.lse_in[goff];
    }
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        float dp = 0.0f;
        dp = fmaf(bf16_lo(o[r].x), bf16_lo(g[r].x), dp);
        dp = fmaf(bf16_hi(o[r].x), bf16_hi(g[r].x), dp);
        dp = fmaf(bf16_lo(o[r].y), bf16_lo(g[r].y), dp);
        dp = fmaf(bf16_hi(o[r].y), bf16_hi(g[r].y), dp);
        dp = fmaf(bf16_lo(o[r].z), bf16_lo(g[r].z), dp);
        dp = fmaf(bf16_hi(o[r].z), bf16_hi(g[r].z), dp);
        dp = fmaf(bf16_lo(o[r].w), bf16_lo(g[r].w), dp);
        dp = fmaf(bf16_hi(o[r].w), bf16_hi(g[r].w), dp);
#pragma unroll
        for (int off = 1; off < LPK; off <<= 1) dp += __shfl_xor(dp, off, 64);
        const int32_t i = row[r];
        if (i < sl.n && (lane % LPK) == 0) {
            float pl, ps;
            gate_priors(gl[r], row_span(i, sl.n, a.pat).has_skip(), &pl, &ps);
            const float lse2 = ls[r] * PIATTN_LOG2E;
            RowRec rec;
            rec.D = dp;
            rec.cw = pl - lse2;
            rec.cs = ps - lse2;
            rec.ss = 0.0f;
            reinterpret_cast<RowRec*>(ba.rowstat)[((int64_t)b * a.H + h) * a.n + i] = rec;
        }
    }
}

// MASKED: the skip multiples are a schedule's mask (skip pass only); a
// separate instantiation keeps the mask test out of the other kernels'
// register budget.
// REC (skip pass only, every view one tile long): the pass forms the row
// records itself, in place of bwd_record_kernel.  Its phase B then reads
// only its own tile's records; a prologue computes them into LDS from out,
// dout, the gate and lse, and finishA stores each own row's whole record
// (the window pass reads them there).
// TB: rows per tile, 16 per wave.
template <int D, bool SKIP, bool BIDIR, bool MASKED, bool REC, int TB>
__global__ __launch_bounds__(TB * 4, D == 64 ? 4 : 2) void bwd_band_kernel(BwdArgs ba, int32_t step, int32_t nres,
                                                                            int32_t tiles, int32_t total,
                                                                            int32_t merge) {
    constexpr int BT = TB, NW = TB / 16;                // tile rows, waves
    constexpr int DC = D / 32, DB = D / 16, CH = D / 8, RPI = 64 / CH;
    constexpr int LPH = 32 / RPI;                       // 1 KB loads per wave per stage: 32 rows of one tensor
    __shared__ __attribute__((aligned(16))) uint16_t x0s[BT * D];
    __shared__ __attribute__((aligned(16))) uint16_t x1s[BT * D];
    __shared__ __attribute__((aligned(16))) uint16_t y0s[BT * D];
    __shared__ __attribute__((aligned(16))) uint16_t y1s[BT * D];
    // the stages' records (c and D of the query rows: two slots each), or
    // with REC those of the tile's own rows (c, then D)
    __shared__ __attribute__((aligned(16))) float recs[(REC ? 2 : 4) * BT];
    // (REC: the stages load no records, and both stage slots name the own
    // tile's c and D)
    float* const c0s = recs;
    float* const c1s = recs + (REC ? 0 : 1) * BT;
    float* const d0s = recs + (REC ? 1 : 2) * BT;
    float* const d1s = recs + (REC ? 1 : 3) * BT;

    const FwdArgs& a = ba.f;
    // Each pass walks its tiles in the reverse of the order of the kernel
    // before it (record kernel, skip pass, window pass), so that it starts
    // on the heads whose rows the memory-side cache still holds.
    const bool reverse = SKIP || !merge;
    const int32_t logical = reverse ? total - 1 - xcd_logical(blockIdx.x, total) : xcd_logical(blockIdx.x, total);
    const int32_t t = logical % tiles;
    int32_t rest = logical / tiles;
    const int32_t res = rest % nres;
    rest /= nres;
    const int32_t h = rest % a.H, b = rest / a.H;
    const SeqLoc sq = seq_loc(a, b);
    if (res >= sq.n) return;                            // workgroup-uniform
    const int32_t L = (sq.n - 1 - res) / step + 1;
    const int32_t p0 = t * BT;
    if (p0 >= L) return;

    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    const int32_t kw = a.pat.k, M = a.pat.M, mlo = a.pat.mlo;
    const int32_t dlo = SKIP ? (BIDIR ? -M : mlo) : (BIDIR ? -kw : 0);
    const int32_t dhi = SKIP ? M : kw;

    // view row 0 of each tensor, and the view's row strides (elements)
    const int64_t r0tok = sq.tok0 + res;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + sq.bq * a.sq.s + h * a.sq.h + r0tok * a.sq.t;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + sq.bq * a.sk.s + h * a.sk.h + r0tok * a.sk.t;
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + sq.bq * a.sv.s + h * a.sv.h + r0tok * a.sv.t;
    const uint16_t* Ob = static_cast<const uint16_t*>(ba.dout) + sq.bq * a.so.s + h * a.so.h + r0tok * a.so.t;
    uint16_t* dQb = static_cast<uint16_t*>(ba.dq) + sq.bq * a.sq.s + h * a.sq.h + r0tok * a.sq.t;
    uint16_t* dKb = static_cast<uint16_t*>(ba.dk) + sq.bq * a.sk.s + h * a.sk.h + r0tok * a.sk.t;
    uint16_t* dVb = static_cast<uint16_t*>(ba.dv) + sq.bq * a.sv.s + h * a.sv.h + r0tok * a.sv.t;
    const int64_t qst = (int64_t)step * a.sq.t, kst = (int64_t)step * a.sk.t;
    const int64_t vst = (int64_t)step * a.sv.t, ost = (int64_t)step * a.so.t;
    RowRec* Rb = reinterpret_cast<RowRec*>(ba.rowstat) + ((int64_t)b * a.H + h) * a.n + res;

    // the key tiles of tile t's band (phase A) and the query tiles whose
    // band holds tile t (phase B)
    const int32_t alo = imax32(0, p0 - dhi), ahi = imin32(L - 1, p0 + BT - 1 - dlo);
    const int32_t jlo = alo / BT, NA = ahi >= alo ? ahi / BT - jlo + 1 : 0;
    const int32_t blo = imax32(0, p0 + dlo), bhi = imin32(L - 1, p0 + BT - 1 + dhi);
    const int32_t ilo = blo / BT, NB = bhi >= blo ? bhi / BT - ilo + 1 : 0;
    const int32_t N = NA + NB;

    // ---- staging: rows s0 .. s0+RPI-1 of the view into slot rows r0 ..;
    // lane row r0 + lane/CH, physical chunk lane%CH = logical chunk
    // (lane%CH) ^ (row%8); rows past the view load its last row
    // stream: rows only this workgroup reads (the skip partials the window
    // pass adds), loaded with the non-temporal hint; the staged tiles,
    // which neighbouring tiles read again, without it
    auto stage_rows = [&](const uint16_t* src, int64_t rst, int32_t s0, int r0, uint16_t* dst, int ln,
                          bool stream = false) __attribute__((always_inline)) {
        const int rl = r0 + ln / CH;
        const int lc = ((ln % CH) ^ (rl & 7)) << 3;
        const bool inside = s0 + RPI - 1 < L;
        const uint16_t* ub = inside ? src + (int64_t)s0 * rst : src;
        const int64_t row = inside ? (int64_t)(ln / CH) : (int64_t)imin32(s0 + ln / CH, L - 1);
        if (stream)
            dma16<true>(ub, (uint32_t)(row * rst + lc) * 2u, lds_addr(dst + r0 * D));
        else
            dma16(ub, (uint32_t)(row * rst + lc) * 2u, lds_addr(dst + r0 * D));
    };
    // stage s < NA: key tile jlo+s (K to x, V to y); then query tile
    // ilo+s-NA (Q to x, dO to y, the rows' c and D to cs, ds).  The first
    // half of the waves load the x tensor, the second half the y tensor, 32
    // rows each; each wave's two sources are fixed here, as values.
    const bool second = wave >= NW / 2;
    const uint16_t* const srcA = second ? Vb : Kb;
    const uint16_t* const srcB = second ? Ob : Qb;
    const int64_t rstA = second ? vst : kst;
    const int64_t rstB = second ? ost : qst;
    auto issue = [&](int32_t s, uint16_t* X, uint16_t* Y, float* C, float* Dd) __attribute__((always_inline)) {
        const bool pa = s < NA;
        const int32_t tb = (pa ? jlo + s : ilo + s - NA) * BT;
        const uint16_t* src = srcB;
        int64_t rst = rstB;
        if (pa) {
            src = srcA;
            rst = rstA;
        }
        uint16_t* dst = second ? Y : X;
#pragma unroll
        for (int j = 0; j < LPH; ++j) {
            const int r0 = (wave % (NW / 2)) * 32 + j * RPI;
            stage_rows(src, rst, tb + r0, r0, dst, lane);
        }
        if (!REC && !pa && wave % (NW / 2) == 0) {
            const uint32_t field = wave == 0 ? (SKIP ? 8u : 4u) : 0u;
#pragma unroll
            for (int q = 0; q < BT / 64; ++q) {
                const int32_t p = imin32(tb + 64 * q + lane, L - 1);
                dma4(Rb, (uint32_t)(p * step) * 16u + field, lds_addr((wave == 0 ? C : Dd) + 64 * q));
            }
        }
    };

    if (N > 0) issue(0, x0s, y0s, c0s, d0s);

    // ---- the lane's own row (query in phase A, key in phase B)
    const int32_t pw = p0 + 16 * wave;                  // the wave's first row
    const int32_t pme = pw + x;
    const bool mine = pme < L;
    const int32_t pc = mine ? pme : L - 1;
    bf16x8_t qf[DC], of[DC];
#pragma unroll
    for (int c = 0; c < DC; ++c) {
        qf[c] = *reinterpret_cast<const bf16x8_t*>(Qb + pc * qst + 32 * c + 8 * g);
        of[c] = *reinterpret_cast<const bf16x8_t*>(Ob + pc * ost + 32 * c + 8 * g);
    }
    RowRec own;
    if constexpr (REC) {
        // The own rows' records: D_i = <dout_i, out_i> (the lane's 8 DC
        // values of row pc, then the four lanes of the row) and
        // c_i = prior - lse_i log2(e).
        const uint16_t* Xb = static_cast<const uint16_t*>(a.o) + sq.bq * a.so.s + h * a.so.h + r0tok * a.so.t;
        float dp = 0.0f;
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            const uint4 ov = *reinterpret_cast<const uint4*>(Xb + pc * ost + 32 * c + 8 * g);
            const uint4 dv = __builtin_bit_cast(uint4, of[c]);
            dp = fmaf(bf16_lo(ov.x), bf16_lo(dv.x), dp);
            dp = fmaf(bf16_hi(ov.x), bf16_hi(dv.x), dp);
            dp = fmaf(bf16_lo(ov.y), bf16_lo(dv.y), dp);
            dp = fmaf(bf16_hi(ov.y), bf16_hi(dv.y), dp);
            dp = fmaf(bf16_lo(ov.z), bf16_lo(dv.z), dp);
            dp = fmaf(bf16_hi(ov.z), bf16_hi(dv.z), dp);
            dp = fmaf(bf16_lo(ov.w), bf16_lo(dv.w), dp);
            dp = fmaf(bf16_hi(ov.w), bf16_hi(dv.w), dp);
        }
        own.D = sum4(dp);
        const int32_t iseq = res + pc * step;
        const int64_t goff = sq.bq * a.sg.s + h * a.sg.h + (sq.tok0 + iseq) * a.sg.t;
        float pl, ps;
        gate_priors(a.g[goff], row_span(iseq, sq.n, a.pat).has_skip(), &pl, &ps);
        const float lse2 = ba.lse_in[goff] * PIATTN_LOG2E;
        own.cw = pl - lse2;
        own.cs = ps - lse2;
        own.ss = 0.0f;
        if (g == 0) {                                   // read by phase B after its first barrier
            recs[16 * wave + x] = own.cs;
            recs[BT + 16 * wave + x] = own.D;
        }
    } else {
        own = Rb[(int64_t)pc * step];
    }
    const float cq = SKIP ? own.cs : own.cw;

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bool wave_live = pw < L;                      // wave-uniform

    // whether view rows (query pq, key pk) form a pair of this part
    auto pair_ok = [&](int32_t pq, int32_t pk) __attribute__((always_inline)) {
        const int32_t dd = pq - pk;
        bool ok = dd >= dlo && dd <= dhi && pq < L && pk < L;
        if (SKIP && BIDIR) ok = ok && (dd >= mlo || dd <= -mlo);
        if (MASKED) ok = ok && mask_has(a.pat, BIDIR ? abs(dd) : dd);
        return ok;
    };
    auto pack4 = [](float a0, float a1, float a2, float a3) __attribute__((always_inline)) {
        return __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(a0, a1), cvt_pk_bf16(a2, a3)));
    };
    auto cat8 = [](s16x4_t lo, s16x4_t hi) __attribute__((always_inline)) {
        return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    // transposed operand of a 16-row block pair: A[m = column][k = rows]
    auto tr_pair = [&](const uint16_t* S, int u, int bb) __attribute__((always_inline)) {
        const s16x4_t lo = ld_tr16(S + swr<D>(16 * u + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        const s16x4_t hi = ld_tr16(S + swr<D>(16 * u + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        return cat8(lo, hi);
    };

    // ---- phase A: dq of the wave's 16 query rows
    f32x4_t dqa[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) dqa[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float ssum = 0.0f;                                  // sum of dS over this lane's keys of row pme
    const int32_t kmin = pw - dhi, kmax = imin32(pw + 15, L - 1) - dlo;   // the wave's key range
    auto computeA = [&](int32_t kb0, const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
        if (!wave_live) return;
#pragma unroll
        for (int u = 0; u < BT / 16; u += 2) {
            s16x4_t db[2];
            bool act[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int32_t k0 = kb0 + 16 * (u + e);
                act[e] = k0 <= imin32(kmax, L - 1) && k0 + 15 >= kmin;
                db[e] = s16x4_t{0, 0, 0, 0};
                if (act[e]) {
                    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f}, p4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const bf16x8_t kk =
                            *reinterpret_cast<const bf16x8_t*>(Ks + swr<D>(16 * (u + e) + x, 4 * c + g));
                        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qf[c], s4, 0, 0, 0);
                    }
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const bf16x8_t vv =
                            *reinterpret_cast<const bf16x8_t*>(Vs + swr<D>(16 * (u + e) + x, 4 * c + g));
                        p4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, of[c], p4, 0, 0, 0);
                    }
                    float dsv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool ok = pair_ok(pme, k0 + 4 * g + r);
                        const float p = exp2_fast(fmaf(s4[r], sl2, cq));
                        dsv[r] = ok ? p * (p4[r] - own.D) : 0.0f;
                        ssum += dsv[r];
                    }
                    db[e] = pack4(dsv[0], dsv[1], dsv[2], dsv[3]);
                }
            }
            if (!act[0] && !act[1]) continue;
            const bf16x8_t dd = cat8(db[0], db[1]);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                dqa[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_pair(Ks, u, bb), dd, dqa[bb], 0, 0, 0);
        }
    };
    // Result rows leave through LDS as whole rows.  The MFMA layout gives a
    // lane 4 consecutive values of one row, so a direct store would write 32
    // bytes of each of 16 rows per instruction; instead the wave writes its
    // 16 rows into its own 16-row region of a free slot (swizzled as the
    // stages are) and stores 16 bytes per lane, whole rows.  The window pass
    // first brings the skip pass's partial rows into the region with
    // LDS-direct loads and adds them in fp32.
    // the lane index afresh (volatile: not merged with the other uses), so
    // that no lane offset of the code after phase B stays live across it
    auto fresh_lane = []() __attribute__((always_inline)) {
        int32_t ln;
        asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
        return ln;
    };
    auto partial_in = [&](const uint16_t* gb, int64_t rst, uint16_t* reg) __attribute__((always_inline)) {
        const int ln = fresh_lane();
#pragma unroll
        for (int j = 0; j < 16 / RPI; ++j) stage_rows(gb, rst, pw + j * RPI, j * RPI, reg, ln, true);
    };
    // the wave's accumulators (MFMA layout, times mul, plus the partial in
    // the region when merging) into its region as bf16
    auto acc_to_lds = [&](const f32x4_t* acc, float mul, uint16_t* reg) __attribute__((always_inline)) {
        const int ln = fresh_lane();
        const int xl = ln & 15, gl = ln >> 4;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) {
            uint2* pl = reinterpret_cast<uint2*>(reg + swr<D>(xl, 2 * bb + (gl >> 1)) + 4 * (gl & 1));
            float v0 = acc[bb][0] * mul, v1 = acc[bb][1] * mul, v2 = acc[bb][2] * mul, v3 = acc[bb][3] * mul;
            if (!SKIP && merge) {
                const uint2 pr = *pl;
                v0 += bf16_lo(pr.x);
                v1 += bf16_hi(pr.x);
                v2 += bf16_lo(pr.y);
                v3 += bf16_hi(pr.y);
            }
            *pl = make_uint2(cvt_pk_bf16(v0, v1), cvt_pk_bf16(v2, v3));
        }
    };
    // the region's rows out, 16 bytes per lane (a 32-bit byte offset from
    // the view's first row: within the bound the launcher checks), with the
    // non-temporal hint: this kernel does not read them again
    auto lds_to_rows = [&](uint16_t* gb, int64_t rst, const uint16_t* reg) __attribute__((always_inline)) {
        const int ln = fresh_lane();
#pragma unroll
        for (int j = 0; j < 16 / RPI; ++j) {
            const int r = j * RPI + ln / CH, c = ln % CH;
            const uint4 val = *reinterpret_cast<const uint4*>(reg + swr<D>(r, c));
            const uint32_t off = (uint32_t)((pw + r) * (int32_t)rst + 8 * c) * 2u;
            if (pw + r < L) store_nt16(reinterpret_cast<char*>(gb) + off, val);
        }
    };
    // dq rows out (the skip pass stores partials, the window pass adds them)
    // and the row sums of dS: the skip pass records its sum, the window
    // pass forms the gate gradient.  reg: the wave's region of a slot no
    // stage occupies, after a barrier.
    auto finishA = [&](uint16_t* reg) __attribute__((always_inline)) {
        const float srow = sum4(ssum);
        if (wave_live) {
            if (!SKIP && merge) {
                partial_in(dQb, qst, reg);
                __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            }
            acc_to_lds(dqa, ba.scale, reg);
            lds_to_rows(dQb, qst, reg);
        }
        if (!mine) return;
        if (g == 0) {
            if (REC) {
                RowRec rr = own;
                rr.ss = srow;
                Rb[(int64_t)pme * step] = rr;
            } else if (SKIP) {
                Rb[(int64_t)pme * step].ss = srow;
            } else {
                const int64_t goff = sq.bq * a.sg.s + h * a.sg.h + (sq.tok0 + pme) * a.sg.t;
                const bool hs = merge && row_span(pme, sq.n, a.pat).has_skip();
                const float alpha = 1.0f / (1.0f + __expf(-a.g[goff]));
                ba.dg[goff] = hs ? (1.0f - alpha) * srow - alpha * own.ss : 0.0f;
            }
        }
    };

    // ---- phase B: dk, dv of the wave's 16 key rows
    f32x4_t dka[DB], dva[DB];
    bf16x8_t kf[DC], vf[DC];
    const int32_t qmin = pw + dlo, qmax = imin32(pw + 15, L - 1) + dhi;   // the wave's query range
    auto computeB = [&](int32_t qb0, const uint16_t* Qs, const uint16_t* Os, const float* C, const float* Dd)
        __attribute__((always_inline)) {
        if (!wave_live) return;
#pragma unroll
        for (int v = 0; v < BT / 16; v += 2) {
            s16x4_t pb[2], db[2];
            bool act[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int32_t q0 = qb0 + 16 * (v + e);
                act[e] = q0 <= imin32(qmax, L - 1) && q0 + 15 >= qmin;
                pb[e] = db[e] = s16x4_t{0, 0, 0, 0};
                if (act[e]) {
                    f32x4_t s4 = {0.f, 0.f, 0.f, 0.f}, p4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const bf16x8_t qq =
                            *reinterpret_cast<const bf16x8_t*>(Qs + swr<D>(16 * (v + e) + x, 4 * c + g));
                        s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qq, kf[c], s4, 0, 0, 0);
                    }
#pragma unroll
                    for (int c = 0; c < DC; ++c) {
                        const bf16x8_t oo =
                            *reinterpret_cast<const bf16x8_t*>(Os + swr<D>(16 * (v + e) + x, 4 * c + g));
                        p4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(oo, vf[c], p4, 0, 0, 0);
                    }
                    const f32x4_t c4 = *reinterpret_cast<const f32x4_t*>(C + 16 * (v + e) + 4 * g);
                    const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(Dd + 16 * (v + e) + 4 * g);
                    float pv[4], dsv[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bool ok = pair_ok(q0 + 4 * g + r, pme);
                        const float p = exp2_fast(fmaf(s4[r], sl2, c4[r]));
                        pv[r] = ok ? p : 0.0f;
                        dsv[r] = ok ? p * (p4[r] - d4[r]) : 0.0f;
                    }
                    pb[e] = pack4(pv[0], pv[1], pv[2], pv[3]);
                    db[e] = pack4(dsv[0], dsv[1], dsv[2], dsv[3]);
                }
            }
            if (!act[0] && !act[1]) continue;
            const bf16x8_t pp = cat8(pb[0], pb[1]);
            const bf16x8_t dd = cat8(db[0], db[1]);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) {
                dva[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_pair(Os, v, bb), pp, dva[bb], 0, 0, 0);
                dka[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(tr_pair(Qs, v, bb), dd, dka[bb], 0, 0, 0);
            }
        }
    };
    // loaded: the partial rows were issued into the regions already
    auto finishB = [&](uint16_t* regk, uint16_t* regv, bool loaded) __attribute__((always_inline)) {
        if (!wave_live) return;
        if (!SKIP && merge) {
            if (!loaded) {
                partial_in(dKb, kst, regk);
                partial_in(dVb, vst, regv);
            }
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        }
        acc_to_lds(dka, ba.scale, regk);
        acc_to_lds(dva, 1.0f, regv);
        lds_to_rows(dKb, kst, regk);
        lds_to_rows(dVb, vst, regv);
    };

    // step s: this wave's loads of stage s landed (wait), every wave's
    // landed and stage s-1 fully read (barrier); issue stage s+1 into the
    // other slot, compute stage s.  Phase A and phase B run as separate
    // loops so that q, dout and dq of phase A are dead in phase B.
    auto waitissue = [&](int32_t s, uint16_t* Xn, uint16_t* Yn, float* Cn, float* Dn) __attribute__((always_inline)) {
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
        lds_barrier();
        if (s + 1 < N) issue(s + 1, Xn, Yn, Cn, Dn);
    };
    // The tile's own key and value rows, phase B's operands: taken from LDS
    // when the tile is one of phase A's key tiles (always for the window),
    // else loaded after phase A.
    const int32_t sown = t - jlo;
    auto grab_kv = [&](const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            kf[c] = *reinterpret_cast<const bf16x8_t*>(Ks + swr<D>(16 * wave + x, 4 * c + g));
            vf[c] = *reinterpret_cast<const bf16x8_t*>(Vs + swr<D>(16 * wave + x, 4 * c + g));
        }
    };
    for (int32_t s = 0; s < NA; ++s) {
        if (s & 1) {
            waitissue(s, x0s, y0s, c0s, d0s);
            computeA((jlo + s) * BT, x1s, y1s);
            if (s == sown) grab_kv(x1s, y1s);
        } else {
            waitissue(s, x1s, y1s, c1s, d1s);
            computeA((jlo + s) * BT, x0s, y0s);
            if (s == sown) grab_kv(x0s, y0s);
        }
    }
    // the slot that does not hold stage NA, free once every wave is past
    // its last phase-A step
    lds_barrier();
    if (NA & 1)
        finishA(x0s + 16 * wave * D);
    else
        finishA(x1s + 16 * wave * D);

    if (sown < 0 || sown >= NA) {
#pragma unroll
        for (int c = 0; c < DC; ++c) {
            kf[c] = *reinterpret_cast<const bf16x8_t*>(Kb + pc * kst + 32 * c + 8 * g);
            vf[c] = *reinterpret_cast<const bf16x8_t*>(Vb + pc * vst + 32 * c + 8 * g);
        }
    }
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) dka[bb] = dva[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // The window pass adds the skip pass's dk and dv partials.  During the
    // last phase-B step the slot that does not hold its stage is free, so
    // each wave loads its partial rows into its region there one step early,
    // under that step's MFMAs, instead of after the last barrier.
    const bool pre = !SKIP && merge && N > NA;           // workgroup-uniform
    uint16_t* const fk = ((N - 1) & 1) ? x0s : x1s;      // the free slot at step N-1
    uint16_t* const fv = ((N - 1) & 1) ? y0s : y1s;
    for (int32_t s = NA; s < N; ++s) {
        const int32_t qt = ilo + s - NA;                // the stage's query tile
        if (s & 1)
            waitissue(s, x0s, y0s, c0s, d0s);
        else
            waitissue(s, x1s, y1s, c1s, d1s);
        if (pre && s == N - 1 && wave_live) {
            partial_in(dKb, kst, fk + 16 * wave * D);
            partial_in(dVb, vst, fv + 16 * wave * D);
        }
        if (s & 1)
            computeB(qt * BT, x1s, y1s, c1s, d1s);
        else
            computeB(qt * BT, x0s, y0s, c0s, d0s);
    }
    lds_barrier();
    if (pre)
        finishB(fk + 16 * wave * D, fv + 16 * wave * D, true);
    else
        finishB(x0s + 16 * wave * D, y0s + 16 * wave * D, false);
}

template <int D, bool BIDIR>
hipError_t launch_t(const BwdArgs& ba, hipStream_t stream) {
    const FwdArgs& a = ba.f;
    constexpr int NS = 64 / (D / 8);
    const bool skips = a.pat.M >= a.pat.mlo;
    // The skip pass forms the records itself when every residue view is one
    // tile long (phase B then needs only the tile's own rows).  With longer
    // views it would recompute its neighbour tiles' records: measured slower
    // on a causal prefill of 32 heads x 131072 tokens at d = 128, pi = 256
    // (8 tiles per view: 6.37 against 6.29 ms), so there, and without skips,
    // the record kernel runs.
    const bool rec = skips && (a.n - 1) / a.pat.pi + 1 <= BT;
    hipError_t e = hipSuccess;
    if (!rec) {
        const dim3 rgrid((a.n + 4 * RG * NS - 1) / (4 * RG * NS), a.H, a.B);
        hipLaunchKernelGGL((bwd_record_kernel<D>), rgrid, dim3(256), 0, stream, ba);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (skips) {
        const int32_t nres = imin32(a.pat.pi, a.n);
        const int32_t lmax = (a.n - 1) / a.pat.pi + 1;
        const int32_t tiles = (lmax + BT - 1) / BT;
        const int64_t total = (int64_t)tiles * nres * a.H * a.B;
        if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
        auto kern = a.pat.masked ? (rec ? bwd_band_kernel<D, true, BIDIR, true, true, BT>
                                        : bwd_band_kernel<D, true, BIDIR, true, false, BT>)
                                 : (rec ? bwd_band_kernel<D, true, BIDIR, false, true, BT>
                                        : bwd_band_kernel<D, true, BIDIR, false, false, BT>);
        hipLaunchKernelGGL(kern, dim3((uint32_t)total), dim3(BT * 4), 0, stream, ba, a.pat.pi, nres, tiles,
                           (int32_t)total, 0);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int32_t tiles = (a.n + BTW - 1) / BTW;
    const int64_t total = (int64_t)tiles * a.H * a.B;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_band_kernel<D, false, BIDIR, false, false, BTW>), dim3((uint32_t)total), dim3(BTW * 4), 0, stream,
                       ba, 1, 1, tiles, (int32_t)total, skips ? 1 : 0);
    return hipGetLastError();
}

}  // namespace

bool bwd_band_supported(int dtype, const BwdArgs& ba) {
    const FwdArgs& a = ba.f;
    if (dtype != 1 || (a.d != 64 && a.d != 128) || !ba.lse_in) return false;
    // 32-bit byte offsets from a view's first row: any row of the sequence
    // (elements of the token-strided tensors, records of 16 bytes)
    int64_t ts = a.sq.t;
    const int64_t s4[3] = {a.sk.t, a.sv.t, a.so.t};
    for (int64_t s : s4) ts = s > ts ? s : ts;
    const int64_t rows = (int64_t)a.n + BTW;
    return rows * ts * 2 + a.d * 2 < ((int64_t)1 << 31) && rows * 16 < ((int64_t)1 << 31) &&
           (int64_t)a.n + 2LL * a.pat.k + 2LL * a.pat.M + 2 * BTW < ((int64_t)1 << 30);
}

hipError_t launch_bwd_band(const BwdArgs& ba, hipStream_t stream) {
    if (ba.f.d == 64) return ba.f.pat.bidir ? launch_t<64, true>(ba, stream) : launch_t<64, false>(ba, stream);
    return ba.f.pat.bidir ? launch_t<128, true>(ba, stream) : launch_t<128, false>(ba, stream);
}
