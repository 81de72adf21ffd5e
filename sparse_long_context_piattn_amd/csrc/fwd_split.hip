// fwd_split.hip -- split prefill for head dim 64 or 128 (gfx950, bf16 MFMA):
// a skip pass in residue layout, then a window pass in sequence layout that
// merges the two partial softmaxes.
//
// Skip pass ("pi-Skip Attention").  Row i = a + t*pi has its skip keys at
// the same residue a in the periods t -/+ m, m in [floor(k/pi)+1, M].  One
// wave takes one residue and sweeps its periods in chunks of 16 query periods
// (the 16 MFMA columns); the keys of a chunk are the NK = ceil(M/16)+1
// (bidirectional: 2 ceil(M/16)+1) 16-period key blocks around it.  Per key
// block ("unit") the wave stages the 16 K and V rows into its private LDS
// slice with LDS-direct loads, several units ahead, and runs S^T = K Q^T, the
// band mask, an online softmax and O^T += V^T P^T.  At the end of a chunk it
// writes the normalised skip partial O_s (fp16, scaled) into the output rows
// and its log-sum-exp (log2 units, without the gate prior) into the caller's
// workspace.  For short bands (NK <= 5) each key block is staged once per
// residue and its operands reused from a register ring; otherwise it is
// staged NK times.
//
// Window pass ("Ring-Local Attention" + "Dynamic Adaptive Fusion").  A
// workgroup takes 64 consecutive query rows of one (sequence, head); the
// keys [i-k, i] (bidirectional [i-k, i+k]) of all its rows stream through a
// ring of three LDS slots of 32 rows, two slots ahead of the compute.  Each
// wave owns 16 rows: S^T = K Q^T on v_mfma_f32_16x16x32_bf16, window mask,
// log(alpha) prior, online softmax, O^T += V^T P^T.  The tile's skip partial
// rows arrive as one more stage of the ring; in the epilogue, rows that have
// skip keys combine their window partial with the skip partial (whose
// log-sum-exp gets the log(1-alpha) prior here): one softmax over the union
// of window and skip keys.
//
// Both passes keep the LDS-direct loads out of the compiler's view (dma16)
// and wait for them explicitly, so no compiler-inserted wait drains the
// pipelines.  Rows outside the sequence are loaded from a clamped valid row
// and masked.  Row data leaves (and the partial re-enters) through LDS as
// whole rows: 16 bytes per lane, a row from neighbouring lanes, rather than
// the MFMA layout's 8 bytes of each of 16 rows per instruction.
#include "kernels.hpp"
#include "mfma_util.hpp"

#include <type_traits>

namespace {

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
// skip keys (its record (lse2, e) is written then).
template <int D, bool BIDIR>
__device__ __forceinline__ void store_skip_chunk(uint16_t* tt, const f32x4_t (&sacc)[D / 16], float sl, float sm,
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
        *reinterpret_cast<f32x2_t*>(Ls + 2 * (res + (16 * c + x) * pi)) = f32x2_t{sm + __log2f(sl), (float)e};
#pragma unroll
    for (int j = 0; j < 32 * D / 1024; ++j) {
        const int o = 1024 * j + 16 * lane;               // byte offset in the [16][D] fp16 tile
        const int r = o / (2 * D), cc = (o % (2 * D)) / 16;
        const uint4 val = *reinterpret_cast<const uint4*>(tt + swr<D>(r, cc));
        const int32_t tr = 16 * c + r;
        if (tr < pr && row_has_skip<BIDIR>(tr, pr, mlo, M))
            *reinterpret_cast<uint4*>(Ob + (int64_t)(res + tr * pi) * sot + 8 * cc) = val;
    }
}

// ================================================================= skip pass
constexpr int SW = 4;                    // waves per skip workgroup (one residue each)

template <int D>
struct SkipGeo {
    static constexpr int NS = D == 64 ? 3 : 2;       // unit slots per wave
    static constexpr int PF = NS - 1;                // units in flight ahead
    static constexpr int UNIT = 32 * D;              // elements: 16 K rows, then 16 V rows
    static constexpr int LPU = UNIT * 2 / 1024;      // 1 KB loads per unit
    static constexpr int QROWS = 16 * D;             // elements: the chunk's 16 query rows
    static constexpr int LPQ = QROWS * 2 / 1024;     // 1 KB loads per query chunk
};

template <int D, bool BIDIR>
__global__ __launch_bounds__(SW * 64) void fwd_skip_kernel(FwdArgs a, float* lse_s, int32_t rgroups,
                                                           int32_t total) {
    using G = Geo<D>;
    using S = SkipGeo<D>;
    constexpr int DC = G::DC, DB = G::DB, CH = G::CH, RPI = G::RPI;
    constexpr int NS = S::NS, PF = S::PF, UNIT = S::UNIT, LPU = S::LPU, LPQ = S::LPQ;
    __shared__ __attribute__((aligned(16))) uint16_t us[NS * SW * UNIT];   // NS unit slots
    __shared__ __attribute__((aligned(16))) uint16_t qs[SW * S::QROWS];
    uint16_t* const u0s = us;
    uint16_t* const u1s = us + SW * UNIT;
    uint16_t* const u2s = us + (NS - 1) * SW * UNIT;

    const int32_t logical = xcd_logical(blockIdx.x, total);
    const int32_t rg = logical % rgroups;
    const int32_t rest = logical / rgroups;
    const int32_t h = rest % a.H, b = rest / a.H;
    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &tok0, &n);
    }
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    const int32_t pi = a.pat.pi, M = a.pat.M, mlo = a.pat.mlo;
    const int32_t res = rg * SW + wave;
    if (res >= pi || res >= n) return;                // no barriers in this kernel
    const int32_t pr = (n - 1 - res) / pi + 1;        // periods of this residue
    const int32_t nch = (pr + 15) >> 4;
    const int32_t NBL = (M + 15) >> 4;
    const int32_t NK = BIDIR ? 2 * NBL + 1 : NBL + 1;
    const int32_t NU = nch * NK;

    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    float* Ls = lse_s + ((int64_t)b * a.H + h) * a.n * 2;
    const int32_t sqt = (int32_t)a.sq.t, skt = (int32_t)a.sk.t, svt = (int32_t)a.sv.t;

    // Lane constants of the loads: within load j of a 16-row block the lane
    // takes row j*RPI + lane/CH (period offset u) and physical chunk lane%CH,
    // which holds logical chunk (lane%CH) ^ ((u/2)%8).
    int32_t lrow[16 / RPI], lch[16 / RPI];
#pragma unroll
    for (int j = 0; j < 16 / RPI; ++j) {
        lrow[j] = j * RPI + lane / CH;
        lch[j] = ((lane % CH) ^ ((lrow[j] >> 1) & 7)) << 3;
    }
    // 16 rows of residue res at periods p0 .. p0+15 (clamped into [0, pr-1])
    // from src (token stride st) to LDS dst: 16/RPI loads.
    auto load_rows = [&](const uint16_t* src, int32_t st, int32_t p0, uint16_t* dst) __attribute__((always_inline)) {
        const bool inside = p0 >= 0 && p0 + 15 < pr;
        const int32_t pb = imin32(imax32(p0, 0), pr - 1);   // base period (offsets below are >= 0)
        const uint16_t* ub = src + (int64_t)(res + pb * pi) * st;
#pragma unroll
        for (int j = 0; j < 16 / RPI; ++j) {
            const int32_t p = imin32(imax32(p0 + lrow[j], 0), pr - 1) - pb;
            const uint32_t off = inside ? (uint32_t)(lrow[j] * pi * st + lch[j]) : (uint32_t)(p * pi * st + lch[j]);
            dma16(ub, off * 2u, lds_addr(dst + j * RPI * D));
        }
    };
    auto issue = [&](uint16_t* slot, int32_t v) __attribute__((always_inline)) {
        v = imin32(v, NU - 1);                        // past the last unit: harmless reload
        const int32_t c = v / NK, kb = c - NBL + v % NK;
        uint16_t* ud = slot + wave * UNIT;
        load_rows(Kb, skt, 16 * kb, ud);
        load_rows(Vb, svt, 16 * kb, ud + 16 * D);
    };
    auto issue_q = [&](int32_t c) __attribute__((always_inline)) { load_rows(Qb, sqt, 16 * imin32(c, nch - 1), qs + wave * S::QROWS); };
    static_assert(LPU == 2 * (16 / RPI) && LPQ == 16 / RPI, "load counts");

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    // ---- state of the current chunk (query periods 16c + col, col = x)
    bf16x8_t sq[DC];
    f32x4_t sacc[DB];
    float sm = -INFINITY, sl = 0.0f, smL = -INFINITY, scst = 0.0f;
    int32_t slo = EMPTY, stq = 0;
    uint32_t sspan = 0;
    bool shs = false;

    auto chunk_init = [&](int32_t c) __attribute__((always_inline)) {
        const uint16_t* qd = qs + wave * S::QROWS;
#pragma unroll
        for (int cc = 0; cc < DC; ++cc)
            sq[cc] = *reinterpret_cast<const bf16x8_t*>(qd + swu<D>(x, 4 * cc + g));
        const int32_t tq = 16 * c + x;
        shs = tq < pr && row_has_skip<BIDIR>(tq, pr, mlo, M);
        const int32_t lo = imax32(tq - M, 0);
        const int32_t hi = BIDIR ? imin32(tq + M, pr - 1) : tq - mlo;
        slo = shs ? lo : EMPTY;
        sspan = shs ? (uint32_t)(hi - lo) : 0u;
        stq = tq;
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) sacc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        sm = -INFINITY;
        smL = -INFINITY;
        sl = 0.0f;
        scst = 0.0f;
    };
    // (through the slot of the chunk's last unit: the next unit issues into
    // it only after these stores, which wait for their LDS reads)
    auto chunk_store = [&](int32_t c, uint16_t* slot) __attribute__((always_inline)) {
        store_skip_chunk<D, BIDIR>(slot + wave * UNIT, sacc, sl, sm, shs, c, res, pr, pi, mlo, M, Ob, a.so.t, Ls,
                                   lane);
    };
    auto unit_compute = [&](int32_t kb, const uint16_t* slot) __attribute__((always_inline)) {
        const uint16_t* Ks = slot + wave * UNIT;
        const uint16_t* Vs = Ks + 16 * D;
        f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int cc = 0; cc < DC; ++cc) {
            const bf16x8_t kk = *reinterpret_cast<const bf16x8_t*>(Ks + swu<D>(x, 4 * cc + g));
            s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, sq[cc], s4, 0, 0, 0);
        }
        const int32_t kp0 = 16 * kb + 4 * g;          // key period of this lane's value r = 0
        const int32_t e0 = kp0 - slo;
        const int32_t h0 = kp0 - stq + mlo - 1;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bool ok = (uint32_t)(e0 + r) <= sspan;
            if (BIDIR) ok = ok && (uint32_t)(h0 + r) > (uint32_t)(2 * mlo - 2);
            if (a.pat.masked) ok = ok && in_schedule<BIDIR>(a.pat, stq, kp0 + r);
            sc[r] = ok ? s4[r] : -INFINITY;
        }
        const float mx = max4(fmax_ieee(fmax_ieee(sc[0], sc[1]), fmax_ieee(sc[2], sc[3]))) * sl2;
        if (__builtin_amdgcn_ballot_w64(mx > smL)) {
            const float mnew = fmax_ieee(sm, mx);
            const float mu = mnew == -INFINITY ? 0.0f : mnew;
            const float fac = exp2_fast(sm - mu);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) sacc[bb] *= fac;
            sl *= fac;
            sm = mnew;
            smL = mnew + LAZY;
            scst = -mu;
        }
        const uint32_t w0 = cvt_pk_bf16(exp2_fast(fmaf(sc[0], sl2, scst)), exp2_fast(fmaf(sc[1], sl2, scst)));
        const uint32_t w1 = cvt_pk_bf16(exp2_fast(fmaf(sc[2], sl2, scst)), exp2_fast(fmaf(sc[3], sl2, scst)));
        const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
        s16x4_t vv[DB];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) vv[bb] = ld_tr16(Vs + swu<D>(tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        const f32x4_t ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        sl += ls[0];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb)
            sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv[bb], pb, sacc[bb], 0, 0, 0);
    };
    // Unit u: issue unit u+PF into nxt (its slot was consumed at unit u-1),
    // wait until this wave's loads of unit u have landed, compute.  The query
    // rows of chunk c+1 are loaded right after chunk c has read its own.
    auto unit = [&](int32_t u, uint16_t* cur, uint16_t* nxt) __attribute__((always_inline)) {
        issue(nxt, u + PF);
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(PF * LPU));
        const int32_t c = u / NK, kbi = u - c * NK;
        if (kbi == 0) {
            chunk_init(c);
            __builtin_amdgcn_s_waitcnt(0xC07F);       // lgkmcnt(0): query rows read
            issue_q(c + 1);
        }
        unit_compute(c - NBL + kbi, cur);
        if (kbi == NK - 1) chunk_store(c, cur);
    };

    // The query rows of chunk c are issued while chunk c-1 starts, and NK >= 2
    // >= PF units' loads follow them before chunk c's first wait: that wait
    // also covers them.
    issue_q(0);
    issue(u0s, 0);
    if (PF > 1) issue(u1s, 1);
    if (NS == 3) {
        for (int32_t u = 0; u < NU; u += 3) {
            unit(u, u0s, u2s);
            if (u + 1 >= NU) break;
            unit(u + 1, u1s, u0s);
            if (u + 2 >= NU) break;
            unit(u + 2, u2s, u1s);
        }
    } else {
        for (int32_t u = 0; u < NU; u += 2) {
            unit(u, u0s, u1s);
            if (u + 1 >= NU) break;
            unit(u + 1, u1s, u0s);
        }
    }
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));       // reloads past the end land before the LDS retires
}

// Register-ring variant of the skip pass for short bands (NK = NBL+1, or
// 2 NBL+1 bidirectional, <= 5 blocks).  The key blocks of a
// residue form a stream: entry j is block j - NBL, chunk c uses entries
// c .. c+NK-1, and each chunk adds exactly one.  Every entry is staged into
// LDS once (two entries ahead), then its MFMA operands -- the K chunks and
// the transposed V^T chunks -- are read into a ring of NK register sets and
// reused by all NK chunks that need them, so K and V are fetched once per
// residue instead of NK times.  The loop starts NK-1 "virtual" chunks early,
// which only fill the ring.  At head dim 128 a ring of five entries takes
// 160 registers per lane and a wave's LDS slice 32 KB: one wave per SIMD,
// its loads two entries deep.
template <int D, int NBL, bool BIDIR>
__global__ __launch_bounds__(SW * 64) void fwd_skip_ring_kernel(FwdArgs a, float* lse_s, int32_t rgroups,
                                                                int32_t total) {
    using G = Geo<D>;
    constexpr int DC = G::DC, DB = G::DB, CH = G::CH, RPI = G::RPI;
    constexpr int NK = BIDIR ? 2 * NBL + 1 : NBL + 1;
    constexpr int LPB = 16 / RPI;                        // 1 KB loads per 16-row block
    constexpr int BLK = 32 * D;                          // elements of one staged entry: 16 K + 16 V rows
    constexpr int QR = 16 * D;                           // elements of one chunk's query rows
    constexpr int WSLICE = 3 * BLK + 2 * QR;             // per wave: 3 entry slots, 2 query slots
    __shared__ __attribute__((aligned(16))) uint16_t lds[SW * WSLICE];

    const int32_t logical = xcd_logical(blockIdx.x, total);
    const int32_t rg = logical % rgroups;
    const int32_t rest = logical / rgroups;
    const int32_t h = rest % a.H, b = rest / a.H;
    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &tok0, &n);
    }
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    const int32_t pi = a.pat.pi, M = a.pat.M, mlo = a.pat.mlo;
    const int32_t res = rg * SW + wave;
    if (res >= pi || res >= n) return;                  // no barriers in this kernel
    const int32_t pr = (n - 1 - res) / pi + 1;
    const int32_t nch = (pr + 15) >> 4;

    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    float* Ls = lse_s + ((int64_t)b * a.H + h) * a.n * 2;
    const int32_t sqt = (int32_t)a.sq.t, skt = (int32_t)a.sk.t, svt = (int32_t)a.sv.t;
    uint16_t* const ws = lds + wave * WSLICE;

    int32_t lrow[16 / RPI], lch[16 / RPI];
#pragma unroll
    for (int j = 0; j < 16 / RPI; ++j) {
        lrow[j] = j * RPI + lane / CH;
        lch[j] = ((lane % CH) ^ ((lrow[j] >> 1) & 7)) << 3;
    }
    auto load_rows = [&](const uint16_t* src, int32_t st, int32_t p0, uint16_t* dst) __attribute__((always_inline)) {
        const bool inside = p0 >= 0 && p0 + 15 < pr;
        const int32_t pb = imin32(imax32(p0, 0), pr - 1);
        const uint16_t* ub = src + (int64_t)(res + pb * pi) * st;
#pragma unroll
        for (int j = 0; j < 16 / RPI; ++j) {
            const int32_t p = imin32(imax32(p0 + lrow[j], 0), pr - 1) - pb;
            const uint32_t off = inside ? (uint32_t)(lrow[j] * pi * st + lch[j]) : (uint32_t)(p * pi * st + lch[j]);
            dma16(ub, off * 2u, lds_addr(dst + j * RPI * D));
        }
    };
    // stream entry j (block j - NBL) into entry slot j % 3: 2 blocks
    auto issue_entry = [&](int32_t j) __attribute__((always_inline)) {
        uint16_t* d = ws + (((j % 3) + 3) % 3) * BLK;
        load_rows(Kb, skt, 16 * (j - NBL), d);
        load_rows(Vb, svt, 16 * (j - NBL), d + 16 * D);
    };
    // query rows of chunk c (clamped into the residue) into query slot c % 2: 1 block
    auto issue_q = [&](int32_t c) __attribute__((always_inline)) {
        load_rows(Qb, sqt, 16 * imin32(imax32(c, 0), nch - 1), ws + 3 * BLK + (c & 1) * QR);
    };

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    bf16x8_t kr[NK][DC];                                  // ring of entry operands
    s16x4_t vr[NK][DB];
    bf16x8_t sq[DC];
#pragma unroll
    for (int e = 0; e < NK; ++e) {
#pragma unroll
        for (int c = 0; c < DC; ++c) kr[e][c] = bf16x8_t{};
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) vr[e][bb] = s16x4_t{0, 0, 0, 0};
    }

    // chunk c (>= -(NK-1)); RS = (entry c+NK-1) % NK, the ring slot it fills
    auto chunk = [&](int32_t c, auto rsc) __attribute__((always_inline)) {
        constexpr int RS = decltype(rsc)::value;
        const int32_t e = c + NK - 1;
        // entry e and the query rows of chunk c have landed: after them only
        // entry e+1 and the query rows of chunk c+1 were issued (2 + 1 blocks)
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(3 * LPB));
        {
            const uint16_t* es = ws + ((e % 3 + 3) % 3) * BLK;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc)
                kr[RS][cc] = *reinterpret_cast<const bf16x8_t*>(es + swu<D>(x, 4 * cc + g));
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                vr[RS][bb] = ld_tr16(es + 16 * D + swu<D>(tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        }
        if (c >= 0) {
            const uint16_t* qd = ws + 3 * BLK + (c & 1) * QR;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) sq[cc] = *reinterpret_cast<const bf16x8_t*>(qd + swu<D>(x, 4 * cc + g));
        }
        __builtin_amdgcn_s_waitcnt(0xC07F);               // lgkmcnt(0): both slots read
        issue_entry(e + 2);
        issue_q(c + 2);
        if (c < 0) return;                                // wave-uniform: filling the ring

        const int32_t tq = 16 * c + x;
        const bool hs = tq < pr && row_has_skip<BIDIR>(tq, pr, mlo, M);
        const int32_t lo = imax32(tq - M, 0);
        const int32_t hi = BIDIR ? imin32(tq + M, pr - 1) : tq - mlo;
        const int32_t slo = hs ? lo : EMPTY;
        const uint32_t sspan = hs ? (uint32_t)(hi - lo) : 0u;
        // All NK score blocks first, then one softmax over the chunk's keys
        // with the exact row max: no running max, no rescaling.
        float sc[NK][4];
        float mxl = -INFINITY;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int slot = (RS + 1 + i) % NK;           // entry c + i
            const int32_t kb = c + i - NBL;
            f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[slot][cc], sq[cc], s4, 0, 0, 0);
            const int32_t kp0 = 16 * kb + 4 * g;
            const int32_t e0 = kp0 - slo;
            const int32_t h0 = kp0 - tq + mlo - 1;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                bool ok = (uint32_t)(e0 + r) <= sspan;
                if (BIDIR) ok = ok && (uint32_t)(h0 + r) > (uint32_t)(2 * mlo - 2);
                if (a.pat.masked) ok = ok && in_schedule<BIDIR>(a.pat, tq, kp0 + r);
                sc[i][r] = ok ? s4[r] : -INFINITY;
            }
            mxl = fmax_ieee(mxl, fmax_ieee(fmax_ieee(sc[i][0], sc[i][1]), fmax_ieee(sc[i][2], sc[i][3])));
        }
        const float sm = max4(mxl) * sl2;                 // the column's max, log2 units
        const float scst = sm == -INFINITY ? 0.0f : -sm;
        f32x4_t sacc[DB];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) sacc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int slot = (RS + 1 + i) % NK;
            const uint32_t w0 = cvt_pk_bf16(exp2_fast(fmaf(sc[i][0], sl2, scst)), exp2_fast(fmaf(sc[i][1], sl2, scst)));
            const uint32_t w1 = cvt_pk_bf16(exp2_fast(fmaf(sc[i][2], sl2, scst)), exp2_fast(fmaf(sc[i][3], sl2, scst)));
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
            lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, lsum, 0, 0, 0);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[slot][bb], pb, sacc[bb], 0, 0, 0);
        }
        const float sl = lsum[0];
        // the chunk's skip partial, through the slot of entry e: free until
        // entry e+3 is issued after the next chunk's LDS reads
        store_skip_chunk<D, BIDIR>(ws + ((e % 3 + 3) % 3) * BLK, sacc, sl, sm, hs, c, res, pr, pi, mlo, M, Ob,
                                   a.so.t, Ls, lane);
    };

    // entries 0, 1 and the query rows of chunks c0, c0+1 in the order the
    // chunk loop keeps (entry, query, entry, query)
    const int32_t c0 = -(NK - 1);
    issue_entry(0);
    issue_q(c0);
    issue_entry(1);
    issue_q(c0 + 1);
    for (int32_t c = c0; c < nch; c += NK) {
        chunk(c, std::integral_constant<int, 0>{});
        if (NK > 1) { if (c + 1 >= nch) break; chunk(c + 1, std::integral_constant<int, 1 % NK>{}); }
        if (NK > 2) { if (c + 2 >= nch) break; chunk(c + 2, std::integral_constant<int, 2 % NK>{}); }
        if (NK > 3) { if (c + 3 >= nch) break; chunk(c + 3, std::integral_constant<int, 3 % NK>{}); }
        if (NK > 4) { if (c + 4 >= nch) break; chunk(c + 4, std::integral_constant<int, 4 % NK>{}); }
    }
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));         // loads issued past the end land before the LDS retires
}

// =============================================================== window pass

// Window-pass shape: WW waves of 16 query rows (a 64-row tile), KT key rows
// per LDS slot.  Small workgroups with small slots keep several tiles in
// flight per CU, each at a different point of its load / compute cycle:
// 24 KB of LDS at d = 64 (four workgroups per CU, the register budget set
// for four waves per SIMD), 48 KB at d = 128 (three per CU).  A 128-row
// tile with 64-key slots, which halves the halo re-reads, measured slower
// at both head dims: 97 KB of LDS at d = 128 allow one workgroup per CU,
// whose loads then stall at every tile start.
template <int D>
struct WinShape {
    static constexpr int WW = 4;
    static constexpr int KT = 32;
    static constexpr int QTW = 16 * WW;
    static constexpr int EU = D == 64 ? 4 : 3;           // waves per SIMD the register budget must allow
};

template <int D, bool BIDIR>
__global__ __launch_bounds__(WinShape<D>::WW * 64, WinShape<D>::EU) void fwd_window_kernel(FwdArgs a, const float* lse_s,
                                                                        int32_t q_tiles, int32_t total,
                                                                        int32_t merge) {
    using G = Geo<D>;
    constexpr int DC = G::DC, DB = G::DB, CH = G::CH, RPI = G::RPI;
    constexpr int WW = WinShape<D>::WW, KT = WinShape<D>::KT, QT = WinShape<D>::QTW, NB = KT / 16;
    constexpr int LPW = KT / RPI / (WW / 2);            // loads per wave per slot (first half K, second V)
    static_assert(KT % (RPI * (WW / 2)) == 0, "slot split");
    static_assert(2 * KT == QT, "query rows are staged through one slot pair");
    static_assert(NB % 2 == 0, "PV runs on pairs of 16-key blocks");
    __shared__ __attribute__((aligned(16))) uint16_t k0s[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t k1s[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t k2s[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v0s[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v1s[KT * D];
    __shared__ __attribute__((aligned(16))) uint16_t v2s[KT * D];
    __shared__ __attribute__((aligned(16))) float gls[QT];

    // Tiles in the reverse of the skip pass's order: the window pass starts
    // on the heads the skip pass touched last, whose q, k, v and partials
    // the memory-side cache still holds.
    const int32_t logical = total - 1 - xcd_logical(blockIdx.x, total);
    const int32_t qt = logical % q_tiles;
    const int32_t rest = logical / q_tiles;
    const int32_t h = rest % a.H, b = rest / a.H;
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

    // ---- staging: slot rows r0 .. r0+RPI-1 per load; lane row r0 + lane/CH,
    // physical chunk lane%CH = logical chunk (lane%CH) ^ (row%8)
    const bool isv = wave >= WW / 2;
    const uint16_t* src0 = isv ? Vb : Kb;
    const int32_t st = isv ? (int32_t)a.sv.t : (int32_t)a.sk.t;
    auto stage_rows = [&](const uint16_t* src, int32_t stt, int32_t s0, int r0, uint16_t* dst) __attribute__((always_inline)) {
        const int rl = r0 + lane / CH;
        const int lc = ((lane % CH) ^ (rl & 7)) << 3;
        const bool inside = s0 >= 0 && s0 + RPI - 1 < n;
        const uint16_t* ub = inside ? src + (int64_t)s0 * stt : src;
        const uint32_t off = inside ? (uint32_t)((lane / CH) * stt + lc)
                                    : (uint32_t)(imin32(imax32(s0 + lane / CH, 0), n - 1) * stt + lc);
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
                stage_rows(Ob, (int32_t)a.so.t, q0 + (isv ? KT : 0) + r0, r0, isv ? Vs : Ks);
            }
            return;
        }
        t = imin32(t, ntiles - 1);
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r0 = ((wave % (WW / 2)) * LPW + j) * RPI;
            stage_rows(src0, st, klo + t * KT + r0, r0, isv ? Vs : Ks);
        }
    };

    // ---- prologue: key tiles 0 and 1, the 128 query rows through slot 2
    // (rows 0-63 in k2s, 64-127 in v2s) and the gate logits
    issue(k0s, v0s, 0);
    {
#pragma unroll
        for (int j = 0; j < LPW; ++j) {
            const int r0 = ((wave % (WW / 2)) * LPW + j) * RPI;
            stage_rows(Qb, (int32_t)a.sq.t, q0 + (isv ? KT : 0) + r0, r0, isv ? v2s : k2s);
        }
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < QT / 64; ++j) {
                const int32_t rr = imin32(q0 + 64 * j + lane, n - 1);
                dma4(Gb, (uint32_t)(rr * (int32_t)a.sg.t) * 4u, lds_addr(gls + 64 * j));
            }
        }
    }
    issue(k1s, v1s, 1);

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

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

    // wait for tile 0, the query rows and the gates (tile 1 may be in flight)
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(LPW));
    lds_barrier();
    bf16x8_t qf[DC];
    float pl, ps;
    {
        const int qr = 16 * wave + x;                   // slot 2 holds rows 0..KT-1 in K, the rest in V
        const uint16_t* qsrc = qr < KT ? k2s : v2s;
        const int rr = qr & (KT - 1);
#pragma unroll
        for (int c = 0; c < DC; ++c) qf[c] = *reinterpret_cast<const bf16x8_t*>(qsrc + swr<D>(rr, 4 * c + g));
        gate_priors(gls[qr], hs, &pl, &ps);
    }
    lds_barrier();                                       // slot 2 is free for tile 2

    // the record of the lane's row (written by the skip pass), loaded now so
    // that its latency hides behind the window loop
    const bool mg = merge && hs && qv;
    f32x2_t rec = {0.0f, 0.0f};                          // (log2-sum-exp, e)
    if (mg) rec = *reinterpret_cast<const f32x2_t*>(Ls + 2 * ic);

    f32x4_t acc[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) acc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lrun = 0.0f, mL = -INFINITY, cst = pl;

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
            mrun = mnew;
            mL = mnew + LAZY;
            cst = pl - mu;
        }
        s16x4_t pb[NB];
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const uint32_t w0 = cvt_pk_bf16(exp2_fast(fmaf(sc[u][0], sl2, cst)), exp2_fast(fmaf(sc[u][1], sl2, cst)));
            const uint32_t w1 = cvt_pk_bf16(exp2_fast(fmaf(sc[u][2], sl2, cst)), exp2_fast(fmaf(sc[u][3], sl2, cst)));
            pb[u] = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
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
        // stage ntiles landed (stage ntiles+1 may be in flight); the
        // barrier also lets every wave's reload into P land when P holds no
        // partials
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(LPW));
        lds_barrier();
        uint16_t* prow = (16 * wave < KT ? Kp : Vp);
        const int qr = 16 * wave + x, rr = qr & (KT - 1), rr0 = (16 * wave) & (KT - 1);
        const float ltot = sum4(lrun);
        const float lw = mrun + __log2f(ltot);          // log2-sum-exp of the window part
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
            if (row < n) *reinterpret_cast<uint4*>(Ob + (int64_t)row * a.so.t + 8 * cc) = val;
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
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));         // loads past the end land before the LDS retires
}

// lse_s: the caller's workspace of B*H*n (log2-sum-exp, e) float pairs, or
// null when the pattern has no skip keys.
template <int D, bool BIDIR>
hipError_t launch_t(const FwdArgs& a, float* lse_s, hipStream_t stream) {
    const bool skips = a.pat.M >= a.pat.mlo;
    if (skips) {
        if (!lse_s) return hipErrorInvalidValue;
        const int32_t rgroups = (imin32(a.pat.pi, a.n) + SW - 1) / SW;
        const int64_t total = (int64_t)rgroups * a.H * a.B;
        if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
        const int32_t nbl = (a.pat.M + 15) / 16;
        if (nbl <= (BIDIR ? 2 : 4)) {
            // short bands: every key block staged once per residue (register ring)
            auto ring = nbl == 1 ? fwd_skip_ring_kernel<D, 1, BIDIR>
                      : nbl == 2 ? fwd_skip_ring_kernel<D, 2, BIDIR>
                      : nbl == 3 ? fwd_skip_ring_kernel<D, BIDIR ? 2 : 3, BIDIR>
                                 : fwd_skip_ring_kernel<D, BIDIR ? 2 : 4, BIDIR>;
            hipLaunchKernelGGL(ring, dim3((uint32_t)total), dim3(SW * 64), 0, stream, a, lse_s, rgroups,
                               (int32_t)total);
        } else {
            hipLaunchKernelGGL((fwd_skip_kernel<D, BIDIR>), dim3((uint32_t)total), dim3(SW * 64), 0, stream, a,
                               lse_s, rgroups, (int32_t)total);
        }
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    constexpr int QTW = WinShape<D>::QTW;
    const int32_t q_tiles = (a.n + QTW - 1) / QTW;
    const int64_t total = (int64_t)q_tiles * a.H * a.B;
    hipError_t e = hipSuccess;
    if (total > 0x7fffffff) {
        e = hipErrorInvalidConfiguration;
    } else {
        hipLaunchKernelGGL((fwd_window_kernel<D, BIDIR>), dim3((uint32_t)total), dim3(WinShape<D>::WW * 64), 0,
                           stream, a, skips ? lse_s : nullptr, q_tiles, (int32_t)total, skips ? 1 : 0);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

bool fwd_split_supported(int dtype, const FwdArgs& a) {
    if (dtype != 1 || (a.d != 64 && a.d != 128)) return false;
    // 32-bit byte offsets below 2^31 (the same value read as signed or
    // unsigned): rows of the sequence, and the lane offsets of 16 rows one
    // period apart
    int64_t ts = a.sk.t > a.sv.t ? a.sk.t : a.sv.t;
    ts = ts > a.sq.t ? ts : a.sq.t;
    ts = ts > a.so.t ? ts : a.so.t;                    // the window pass reads the skip partials from out
    ts = ts > 2 * a.sg.t ? ts : 2 * a.sg.t;            // the gate's byte offsets are twice as large
    const int64_t span = (int64_t)a.n + 16LL * a.pat.pi + a.d;
    return span * ts * 2 < ((int64_t)1 << 31) &&
           (int64_t)a.n + 2LL * a.pat.k + WinShape<64>::QTW < ((int64_t)1 << 30);
}

hipError_t launch_fwd_split(const FwdArgs& a, float* ws, hipStream_t stream) {
    if (a.d == 64) return a.pat.bidir ? launch_t<64, true>(a, ws, stream) : launch_t<64, false>(a, ws, stream);
    return a.pat.bidir ? launch_t<128, true>(a, ws, stream) : launch_t<128, false>(a, ws, stream);
}
