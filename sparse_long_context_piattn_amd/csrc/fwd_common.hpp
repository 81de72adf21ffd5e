// fwd_common.hpp -- pieces of the split prefill (skip pass, then window
// pass): geometry, the skip-partial hand-off format, the band tests of the
// residue layout, and the window tile (a device function the window pass
// runs once per workgroup).
//
// Skip partial hand-off.  Row i's skip part (its keys i -/+ m*pi) is a
// normalised partial output O_s and its log2-sum-exp; it travels from the
// skip pass to the window pass in the row's output slots (fp16, scaled by a
// per-row power of two) and a two-float record per row in the workspace.
// The window pass merges it with the window part (one softmax over the
// union: the partials' log-sum-exp weights, the gate prior log(1 - alpha)
// added to the skip part's).
#pragma once

#include "kernels.hpp"
#include "mfma_util.hpp"

namespace fwdk {


constexpr int32_t EMPTY = 0x40000000;   // lower bound of an empty key range

template <int D>
struct Geo {
    static constexpr int DC = D / 32;    // QK^T depth chunks (16x16x32)
    static constexpr int DB = D / 16;    // O^T row blocks
    static constexpr int CH = D / 8;     // 16-byte chunks per row
    static constexpr int RPI = 64 / CH;  // rows covered by one 64-lane 16-byte load
};

// Same, swizzled by (r / 2) % 8: the 16 rows of a K-operand read then fall
// on distinct banks when a row is 128 bytes.
template <int D>
__device__ __forceinline__ int swu(int r, int c) { return r * D + ((c ^ ((r >> 1) & 7)) << 3); }

// Whether key period kp is a skip key of query period tq under a skip
// schedule's mask of multiples (masked patterns only).
template <bool BIDIR>
__device__ __forceinline__ bool in_schedule(const PiPattern& p, int32_t tq, int32_t kp) {
    return mask_has(p, BIDIR ? abs(tq - kp) : tq - kp);
}

// Whether row (residue a, period t) with pr periods in its residue has any
// skip key.
template <bool BIDIR>
__device__ __forceinline__ bool row_has_skip(int32_t t, int32_t pr, int32_t mlo, int32_t M) {
    return M >= mlo && (t >= mlo || (BIDIR && t + mlo < pr));
}

// Skip partial of one row, handed from the skip pass to the window pass.
// The normalised O_s goes into the row's output slots as fp16 scaled by
// 2^-e, e chosen from the row's largest magnitude m so that m 2^-e lies in
// [2^14, 2^15): no overflow, full fp16 precision (4x that of bf16, so the
// merge adds well under a quarter ulp of the final bf16 rounding).  Its
// log2-sum-exp and e go into the row's two-float record of the workspace.
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t cvt_pk_f16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
}
__device__ __forceinline__ float f16lo(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[0]; }
__device__ __forceinline__ float f16hi(uint32_t w) { return (float)__builtin_bit_cast(f16x2_t, w)[1]; }

// One wave's chunk of the skip partial -- query periods 16c .. 16c+15 of
// residue res -- goes through the free LDS tile tt (16 D elements) so that
// every store instruction writes whole rows: the lanes write their MFMA
// layout (lane (x, g) holds d = 16 bb + 4 g + 0..3 of row x), then read back
// 16 bytes each, a row's 2D bytes from 2D/16 neighbouring lanes.  Rows past
// the residue or without skip keys are not stored; hs says whether row x has
// skip keys (its record (lse2, e) is written then).  sl is the sum of the
// bf16 P the accumulators were built from (the partial is normalised by it,
// so it is an exact convex combination of the value rows); sl32 the sum of
// the same exponentials in fp32, the row's skip mass (its record).
template <int D, bool BIDIR>
__device__ __forceinline__ void store_skip_chunk(uint16_t* tt, const f32x4_t (&sacc)[D / 16], float sl, float sl32,
                                                 float sm,
                                                 bool hs, int32_t c, int32_t res, int32_t pr, int32_t pi,
                                                 int32_t mlo, int32_t M, uint16_t* Ob, int64_t sot, float* Ls,
                                                 int lane) {
    constexpr int DB = D / 16;
    const int x = lane & 15, g = lane >> 4;
    const float inv = 1.0f / sl;
    float mloc = 0.0f;
#pragma unroll
    for (int bb = 0; bb < DB; ++bb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mloc = fmax_ieee(mloc, fabsf(sacc[bb][r]));
    const float m = max4(mloc) * inv;
    const int32_t ex = (int32_t)((__float_as_uint(m) >> 23) & 0xff);   // m < 2^(ex - 126)
    const int32_t e = imax32(-64, ex - 141);                           // m * 2^-e in [2^14, 2^15)
    const float sc = __builtin_amdgcn_ldexpf(inv, -e);
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) {
        uint2 w;
        w.x = cvt_pk_f16(sacc[bb][0] * sc, sacc[bb][1] * sc);
        w.y = cvt_pk_f16(sacc[bb][2] * sc, sacc[bb][3] * sc);
        *reinterpret_cast<uint2*>(tt + swr<D>(x, 2 * bb + (g >> 1)) + 4 * (g & 1)) = w;
    }
    if (hs && g == 0)
        *reinterpret_cast<f32x2_t*>(Ls + 2 * (res + (16 * c + x) * pi)) = f32x2_t{sm + __log2f(sl32), (float)e};
#pragma unroll
    for (int j = 0; j < 32 * D / 1024; ++j) {
        const int o = 1024 * j + 16 * lane;               // byte offset in the [16][D] fp16 tile
        const int r = o / (2 * D), cc = (o % (2 * D)) / 16;
        const uint4 val = *reinterpret_cast<const uint4*>(tt + swr<D>(r, cc));
        const int32_t tr = 16 * c + r;
        if (tr < pr && row_has_skip<BIDIR>(tr, pr, mlo, M))   // read again only by the window pass
            store_nt16(Ob + (int64_t)(res + tr * pi) * sot + 8 * cc, val);
    }
}

// Waves per skip workgroup (one residue each).
constexpr int SW = 4;

// Window-pass shape: WW waves of 16 query rows (a 64-row tile), KT key rows
// per LDS slot.  Small workgroups with small slots keep several tiles in
// flight per CU, each at a different point of its load / compute cycle:
// 24 KB of LDS at d = 64 (the register budget set for four waves per
// SIMD), 33 KB at d = 128 (four per CU).  A 128-row
// tile with 64-key slots, which halves the halo re-reads, measured slower
// at both head dims: 97 KB of LDS at d = 128 allow one workgroup per CU,
// whose loads then stall at every tile start.
template <int D>
struct WinShape {
    static constexpr int WW = 4;
    static constexpr int KT = 32;
    static constexpr int QTW = 16 * WW;
    // K/V slot pairs in the ring: three (loads two tiles ahead) at d = 64;
    // two (one ahead) at d = 128, where 33 KB instead of 49 KB of LDS lets
    // four workgroups share a CU instead of three (32 heads x 131072 tokens,
    // k = 128: 1.883-1.888 -> 1.832-1.835 ms; at d = 64 two pairs measured
    // no faster)
    static constexpr int NSL = D == 64 ? 3 : 2;
    static constexpr int EU = 4;                             // waves per SIMD the register budget must allow
    static constexpr int LDS = 2 * NSL * KT * D * 2 + QTW * 4;   // bytes: NSL K and NSL V slots, the gates
};

// Window tile qt of (sequence b, head h): 64 query rows, their window keys,
// and (merge) the merge with the rows' skip partials.  lds: WinShape<D>::LDS
// bytes.
template <int D, bool BIDIR>
__device__ __forceinline__ void window_tile(const FwdArgs& a, const float* lse_s, int32_t merge, int32_t qt,
                                            int32_t h, int32_t b, uint16_t* lds) {
    using G = Geo<D>;
    constexpr int DC = G::DC, DB = G::DB, CH = G::CH, RPI = G::RPI;
    constexpr int WW = WinShape<D>::WW, KT = WinShape<D>::KT, QT = WinShape<D>::QTW, NB = KT / 16;
    constexpr int LPW = KT / RPI / (WW / 2);            // loads per wave per slot (first half K, second V)
    static_assert(KT % (RPI * (WW / 2)) == 0, "slot split");
    static_assert(2 * KT == QT, "query rows are staged through one slot pair");
    static_assert(NB % 2 == 0, "PV runs on pairs of 16-key blocks");
    constexpr int NSL = WinShape<D>::NSL;
    static_assert(NSL == 2 || NSL == 3, "two or three slot pairs");
    uint16_t* const k0s = lds;
    uint16_t* const k1s = lds + KT * D;
    uint16_t* const k2s = lds + 2 * KT * D;                  // NSL = 3 only
    uint16_t* const v0s = lds + NSL * KT * D;
    uint16_t* const v1s = lds + (NSL + 1) * KT * D;
    uint16_t* const v2s = lds + (NSL + 2) * KT * D;          // NSL = 3 only
    float* const gls = reinterpret_cast<float*>(lds + 2 * NSL * KT * D);
    // the query rows are staged through the last slot pair
    uint16_t* const kqs = NSL == 3 ? k2s : k1s;
    uint16_t* const vqs = NSL == 3 ? v2s : v1s;

    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &tok0, &n);
    }
    const int32_t q0 = qt * QT;
    if (q0 >= n) return;                                // workgroup-uniform
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    const int32_t pi = a.pat.pi, kw = a.pat.k, M = a.pat.M, mlo = a.pat.mlo;

    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    const float* Gb = a.g + bq * a.sg.s + h * a.sg.h + tok0 * a.sg.t;
    const float* Ls = lse_s ? lse_s + ((int64_t)b * a.H + h) * a.n * 2 : nullptr;

    const int32_t klo = imax32(0, q0 - kw);
    const int32_t khi = imin32(n - 1, q0 + QT - 1 + (BIDIR ? kw : 0));
    const int32_t ntiles = (khi - klo) / KT + 1;

    // ---- the lane's query row
    const int32_t i = q0 + 16 * wave + x;
    const bool qv = i < n;
    const int32_t ic = qv ? i : n - 1;
    const int32_t ti = ic / pi, ai = ic - ti * pi;
    const int32_t pr = (n - 1 - ai) / pi + 1;
    const bool hs = row_has_skip<BIDIR>(ti, pr, mlo, M);
    const int32_t lo = qv ? imax32(0, i - kw) : EMPTY;
    const uint32_t span = qv ? (uint32_t)(imin32(n - 1, BIDIR ? i + kw : i) - lo) : 0u;
    const int32_t w0 = q0 + 16 * wave;                  // the wave's key span
    const int32_t wlo = imax32(0, w0 - kw);
    const int32_t whi = w0 < n ? imin32(n - 1, imin32(w0 + 15, n - 1) + (BIDIR ? kw : 0)) : -1;
    // the record of the lane's row (written by the skip pass): (log2-sum-exp, e)
    const bool mg = merge && hs && qv;
    f32x2_t rec = {0.0f, 0.0f};

    // ---- staging: slot rows r0 .. r0+RPI-1 per load; lane row r0 + lane/CH,
    // physical chunk lane%CH = logical chunk (lane%CH) ^ (row%8)
    const bool isv = wave >= WW / 2;
    const uint16_t* src0 = isv ? Vb : Kb;
    const int32_t st = isv ? (int32_t)a.sv.t : (int32_t)a.sk.t;
    // stream: rows this tile alone reads (its query and skip-partial rows),
    // loaded with the non-temporal hint; the key rows, which the next tile
    // reads again from L2 as its halo, without it
    auto stage_rows = [&](const uint16_t* src, int32_t stt, int32_t s0, int r0, uint16_t* dst, bool stream)
        __attribute__((always_inline)) {
        const int rl = r0 + lane / CH;
        const int lc = ((lane % CH) ^ (rl & 7)) << 3;
        const bool inside = s0 >= 0 && s0 + RPI - 1 < n;
        const uint16_t* ub = inside ? src + (int64_t)s0 * stt : src;
        const uint32_t off = inside ? (uint32_t)((lane / CH) * stt + lc)
                                    : (uint32_t)(imin32(imax32(s0 + lane / CH, 0), n - 1) * stt + lc);
        if (stream)
            dma16<true>(ub, off * 2u, lds_addr(dst + r0 * D));
        else
            dma16(ub, off * 2u, lds_addr(dst + r0 * D));
    };
    // Stage t < ntiles: key tile t.  Stage ntiles, when skip partials are
    // merged: the tile's fp16 skip partial rows, each wave its own 16 rows
    // (the layout of the query rows: rows 0..KT-1 in the K array, the rest
    // in the V array).  Later stages: a harmless reload of the last key
    // tile, which keeps every wave's count of loads in flight uniform.
    auto issue = [&](uint16_t* Ks, uint16_t* Vs, int32_t t) __attribute__((always_inline)) {
        if (merge && t == ntiles) {
#pragma unroll
            for (int j = 0; j < LPW; ++j) {
                const int r0 = ((wave % (WW / 2)) * LPW + j) * RPI;
                stage_rows(Ob, (int32_t)a.so.t, q0 + (isv ? KT : 0) + r0, r0, isv ? Vs : Ks, true);
            }
            return;
        }
        t = imin32(t, ntiles - 1);
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r0 = ((wave % (WW / 2)) * LPW + j) * RPI;
            stage_rows(src0, st, klo + t * KT + r0, r0, isv ? Vs : Ks, false);
        }
    };

    // ---- prologue: key tile 0 (and tile 1 with three pairs), the 64 query
    // rows through the last pair (rows 0..KT-1 in its K slot, the rest in
    // its V slot) and the gate logits
    issue(k0s, v0s, 0);
    {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r0 = ((wave % (WW / 2)) * LPW + j) * RPI;
            stage_rows(Qb, (int32_t)a.sq.t, q0 + (isv ? KT : 0) + r0, r0, isv ? vqs : kqs, true);
        }
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < QT / 64; ++j) {
                const int32_t rr = imin32(q0 + 64 * j + lane, n - 1);
                dma4(Gb, (uint32_t)(rr * (int32_t)a.sg.t) * 4u, lds_addr(gls + 64 * j));
            }
        }
    }
    if (NSL == 3) issue(k1s, v1s, 1);

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));


    // wait for tile 0, the query rows and the gates (tile 1 may be in flight)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(NSL == 3 ? LPW : 0));
    lds_barrier();
    bf16x8_t qf[DC];
    float pl, ps;
    {
        const int qr = 16 * wave + x;                   // the query pair holds rows 0..KT-1 in K, the rest in V
        const uint16_t* qsrc = qr < KT ? kqs : vqs;
        const int rr = qr & (KT - 1);
#pragma unroll
        for (int c = 0; c < DC; ++c) qf[c] = *reinterpret_cast<const bf16x8_t*>(qsrc + swr<D>(rr, 4 * c + g));
        gate_priors(gls[qr], hs, &pl, &ps);
    }
    lds_barrier();                                       // the query pair is free for the next tile

    // the record of the lane's row, loaded now so that its latency hides
    // behind the window loop
    if (mg) rec = *reinterpret_cast<const f32x2_t*>(Ls + 2 * ic);

    f32x4_t acc[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) acc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // lrun: this lane's quarter of the row's sum of the bf16 P that acc is
    // built from (the normaliser); l32: this lane's 4 keys of every block in
    // fp32 (the row's window mass: its log-sum-exp)
    float mrun = -INFINITY, lrun = 0.0f, l32 = 0.0f, mL = -INFINITY, cst = pl;

    auto compute = [&](int32_t t, const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
        const int32_t kt0 = klo + t * KT;
        if (kt0 > whi || kt0 + KT - 1 < wlo) return;    // wave-uniform
        float sc[NB][4];
        bool act[NB];
        float mx = -INFINITY;
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int32_t kb0 = kt0 + 16 * u;
            act[u] = kb0 <= whi && kb0 + 15 >= wlo;     // wave-uniform
#pragma unroll
            for (int r = 0; r < 4; ++r) sc[u][r] = -INFINITY;
            if (act[u]) {
                f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < DC; ++c) {
                    const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(Ks + swr<D>(16 * u + x, 4 * c + g));
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qf[c], s4, 0, 0, 0);
                }
                const int32_t rel = kb0 + 4 * g - lo;
#pragma unroll
                for (int r = 0; r < 4; ++r) sc[u][r] = (uint32_t)(rel + r) <= span ? s4[r] : -INFINITY;
                mx = fmax_ieee(mx, fmax_ieee(fmax_ieee(sc[u][0], sc[u][1]), fmax_ieee(sc[u][2], sc[u][3])));
            }
        }
        mx = fmaf(max4(mx), sl2, pl);
        if (__builtin_amdgcn_ballot_w64(mx > mL)) {
            const float mnew = fmax_ieee(mrun, mx);
            const float mu = mnew == -INFINITY ? 0.0f : mnew;
            const float fac = exp2_fast(mrun - mu);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) acc[bb] *= fac;
            lrun *= fac;
            l32 *= fac;
            mrun = mnew;
            mL = mnew + LAZY;
            cst = pl - mu;
        }
        // P in bf16 for the PV products and the normaliser; the mass from the
        // fp32 values
        s16x4_t pb[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = exp2_fast(fmaf(sc[u][r], sl2, cst));
            pb[u] = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));
            l32 += (p[0] + p[1]) + (p[2] + p[3]);
        }
        f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < NB; u += 2) {
            if (!act[u] && !act[u + 1]) continue;
            const bf16x8_t pp =
                __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(pb[u], pb[u + 1], 0, 1, 2, 3, 4, 5, 6, 7));
            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pp, lsum, 0, 0, 0);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) {
                const s16x4_t v0 = ld_tr16(Vs + swr<D>(16 * u + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                const s16x4_t v1 = ld_tr16(Vs + swr<D>(16 * u + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                const bf16x8_t va = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp, acc[bb], 0, 0, 0);
            }
        }
        lrun += 0.25f * lsum[0];                        // quarter per lane; sum4 restores the row sum
    };
    // Epilogue, with the slot of stage ntiles (P):
    // the window partial, merged with the skip partial (read from P) when
    // the row has skip keys (its lse gets the log(1-alpha) prior here); the
    // bf16 rows then go back through the wave's own rows of P so that each
    // store instruction writes whole rows.
    auto epilogue = [&](uint16_t* Kp, uint16_t* Vp) __attribute__((always_inline)) {
        // stage ntiles landed (with three pairs stage ntiles+1 may be in
        // flight); the barrier also lets every wave's reload into P land
        // when P holds no partials
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(NSL == 3 ? LPW : 0));
        lds_barrier();
        uint16_t* prow = (16 * wave < KT ? Kp : Vp);
        const int qr = 16 * wave + x, rr = qr & (KT - 1), rr0 = (16 * wave) & (KT - 1);
        const float ltot = sum4(lrun);                  // normaliser of acc
        const float lw = mrun + __log2f(sum4(l32));     // log2-sum-exp of the window part
        float fw = 1.0f / ltot, fs = 0.0f, lfin = lw;
        uint2 os[DB];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) os[bb] = make_uint2(0, 0);
        if (mg) {
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                os[bb] = *reinterpret_cast<const uint2*>(prow + swr<D>(rr, 2 * bb + (g >> 1)) + 4 * (g & 1));
            const float lsk = rec[0] + ps;
            const float mx = fmaxf(lw, lsk);
            const float aw = exp2_fast(lw - mx), as = exp2_fast(lsk - mx);
            const float inv = 1.0f / (aw + as);
            fw = ltot > 0.0f ? aw * inv / ltot : 0.0f; // alpha = 0: the window part is empty
            fs = __builtin_amdgcn_ldexpf(as * inv, (int)rec[1]);   // undo the fp16 scaling
            lfin = mx + __log2f(aw + as);
        }
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) {
            uint2 w;
            w.x = cvt_pk_bf16(fmaf(acc[bb][0], fw, f16lo(os[bb].x) * fs), fmaf(acc[bb][1], fw, f16hi(os[bb].x) * fs));
            w.y = cvt_pk_bf16(fmaf(acc[bb][2], fw, f16lo(os[bb].y) * fs), fmaf(acc[bb][3], fw, f16hi(os[bb].y) * fs));
            *reinterpret_cast<uint2*>(prow + swr<D>(rr, 2 * bb + (g >> 1)) + 4 * (g & 1)) = w;
        }
        if (a.lse && qv && g == 0) a.lse[bq * a.sg.s + h * a.sg.h + (tok0 + i) * a.sg.t] = lfin * PIATTN_LN2;
#pragma unroll
        for (int j = 0; j < 32 * D / 1024; ++j) {
            const int o = 1024 * j + 16 * lane;           // byte offset in the wave's [16][D] bf16 rows
            const int r = o / (2 * D), cc = (o % (2 * D)) / 16;
            const uint4 val = *reinterpret_cast<const uint4*>(prow + swr<D>(rr0 + r, cc));
            const int32_t row = q0 + 16 * wave + r;
            if (row < n) store_nt16(Ob + (int64_t)row * a.so.t + 8 * cc, val);   // the result
        }
    };
    // step t: wait for this wave's loads of tile t (tile t+1 may be in
    // flight), barrier (everyone's tile t landed, tile t-1 fully read), issue
    // stage t+2 into the slot of tile t-1, compute tile t
    auto step = [&](int32_t t, const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn, uint16_t* Vn)
        __attribute__((always_inline)) {
        if (t > 0) {
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(LPW));
            lds_barrier();
        }
        issue(Kn, Vn, t + 2);
        compute(t, Kc, Vc);
    };
    // two pairs: step t waits for all of its loads (tile t, issued one step
    // before), barrier (tile t-1 fully read), issues stage t+1 into the pair
    // of tile t-1, computes tile t
    auto step2 = [&](int32_t t, const uint16_t* Kc, const uint16_t* Vc, uint16_t* Kn, uint16_t* Vn)
        __attribute__((always_inline)) {
        if (t > 0) {
            __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));
            lds_barrier();
        }
        issue(Kn, Vn, t + 1);
        compute(t, Kc, Vc);
    };
    if constexpr (NSL == 3) {
        for (int32_t t = 0; t < ntiles; t += 3) {
            step(t, k0s, v0s, k2s, v2s);
            if (t + 1 >= ntiles) break;
            step(t + 1, k1s, v1s, k0s, v0s);
            if (t + 2 >= ntiles) break;
            step(t + 2, k2s, v2s, k1s, v1s);
        }
        // stage ntiles went to slot ntiles % 3
        const int pslot = ntiles % 3;
        epilogue(pslot == 0 ? k0s : pslot == 1 ? k1s : k2s, pslot == 0 ? v0s : pslot == 1 ? v1s : v2s);
    } else {
        for (int32_t t = 0; t < ntiles; t += 2) {
            step2(t, k0s, v0s, k1s, v1s);
            if (t + 1 >= ntiles) break;
            step2(t + 1, k1s, v1s, k0s, v0s);
        }
        // stage ntiles went to pair ntiles % 2
        const int pslot = ntiles % 2;
        epilogue(pslot == 0 ? k0s : k1s, pslot == 0 ? v0s : v1s);
    }
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));         // loads past the end land before the LDS retires
}

}  // namespace fwdk
