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
#include "fwd_common.hpp"

#include <type_traits>

namespace {

using namespace fwdk;

// ================================================================= skip pass

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

    // ---- state of the current chunk (query periods 16c + col, col = x);
    // sl: the column's sum of the bf16 P the accumulators are built from;
    // sl32: this lane's 4 keys of every block in fp32 (the column's mass)
    bf16x8_t sq[DC];
    f32x4_t sacc[DB];
    float sm = -INFINITY, sl = 0.0f, sl32 = 0.0f, smL = -INFINITY, scst = 0.0f;
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
        sl32 = 0.0f;
        scst = 0.0f;
    };
    // (through the slot of the chunk's last unit: the next unit issues into
    // it only after these stores, which wait for their LDS reads)
    auto chunk_store = [&](int32_t c, uint16_t* slot) __attribute__((always_inline)) {
        store_skip_chunk<D, BIDIR>(slot + wave * UNIT, sacc, sl, sum4(sl32), sm, shs, c, res, pr, pi, mlo, M, Ob,
                                   a.so.t, Ls, lane);
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
            sl32 *= fac;
            sm = mnew;
            smL = mnew + LAZY;
            scst = -mu;
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = exp2_fast(fmaf(sc[r], sl2, scst));
        const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));
        s16x4_t vv[DB];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) vv[bb] = ld_tr16(Vs + swu<D>(tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        sl32 += (p[0] + p[1]) + (p[2] + p[3]);
        const f32x4_t ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        sl += ls[0];                                  // full column sum in every lane
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
        // the accumulators and the normaliser from the bf16 P, the mass
        // from the fp32 values (this lane's keys)
        const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));
        f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
        float lpart = 0.0f;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int slot = (RS + 1 + i) % NK;
            float p[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) p[r] = exp2_fast(fmaf(sc[i][r], sl2, scst));
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));
            lpart += (p[0] + p[1]) + (p[2] + p[3]);
            lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, lsum, 0, 0, 0);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[slot][bb], pb, sacc[bb], 0, 0, 0);
        }
        const float sl = lsum[0], sl32 = sum4(lpart);
        // the chunk's skip partial, through the slot of entry e: free until
        // entry e+3 is issued after the next chunk's LDS reads
        store_skip_chunk<D, BIDIR>(ws + ((e % 3 + 3) % 3) * BLK, sacc, sl, sl32, sm, hs, c, res, pr, pi, mlo, M, Ob,
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

template <int D, bool BIDIR>
__global__ __launch_bounds__(WinShape<D>::WW * 64, WinShape<D>::EU) void fwd_window_kernel(FwdArgs a, const float* lse_s,
                                                                        int32_t q_tiles, int32_t total,
                                                                        int32_t merge) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[WinShape<D>::LDS / 2];
    // Tiles in the reverse of the skip pass's order: the window pass starts
    // on the heads the skip pass touched last, whose q, k, v and partials
    // the memory-side cache still holds.
    const int32_t logical = total - 1 - xcd_logical(blockIdx.x, total);
    const int32_t qt = logical % q_tiles;
    const int32_t rest = logical / q_tiles;
    window_tile<D, BIDIR>(a, lse_s, merge, qt, rest % a.H, rest / a.H, lds);
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
