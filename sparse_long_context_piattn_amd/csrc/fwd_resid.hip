// fwd_resid.hip -- residue-tiled prefill for head dim 64 with the periodic
// skips computed as a dense band in residue layout (gfx950, bf16 MFMA).
//
// Write a query row as i = a + t*pi (residue a = i mod pi, period t).  A
// workgroup owns 64 residues [a0, a0+64) x T = 8 periods [t0, t0+8): 512
// rows, 32 row groups of 16 rows (one period, 16 consecutive residues).  Each
// of the 8 waves owns the 4 row groups of one 16-residue a-group and one
// period parity and keeps their online-softmax state (max m, per-lane partial
// sums l, fp32 O^T) in registers.
//
// Phase 1, ring-local windows (pi-Attention "Ring-Local Attention"): step s
// stages the windows of periods t0+2s and t0+2s+1 ([a0 + t pi - k,
// a0 + t pi + 64 (+k)) each) and every wave runs its row group's band:
// S^T = K Q^T on v_mfma_f32_16x16x32_bf16, mask, log(alpha) prior, online
// softmax, O^T += V^T P^T.
//
// Phase 2, periodic skips ("pi-Skip Attention").  The skip keys of row
// (a, t) are (a, t -/+ m) -- the same residue in other periods -- so for one
// residue they form a band of width M over the pi-strided sequence.  For each
// a-group (16 residues), an LDS stage holds 16 key periods x 16 residues of K
// and V; an "item" is one residue with the tile's T query periods as MFMA
// columns, and S^T = K Q^T, the band mask, the log(1-alpha) prior, an online
// softmax and O^T += V^T P^T run densely on MFMA.  After an a-group's key
// periods, its items' partial states (m, l, O^T) pass through a small LDS
// buffer into the owners' registers and are merged exactly (m = max, l and O
// rescaled by 2^(m_part - m)): one softmax over window and skips ("Dynamic
// Adaptive Fusion").
//
// Softmax bookkeeping is lazy: the running max of a column moves only when a
// new score exceeds it by more than 2^8, so in steady state a block costs
// mask + fma + exp per score and no rescale of the accumulators.
//
// Staging: global_load_lds_dwordx4 into two alternating LDS stages (the next
// stage's rows are in flight while the current one computes); rows are
// XOR-swizzled by 16-byte chunk with key (row ^ row/16) % 8 so that both
// consecutive rows and rows 16 apart spread over the banks.  Rows outside the
// sequence are loaded from a clamped valid row and masked out.
#include "kernels.hpp"
#include "mfma_util.hpp"

#include <type_traits>

namespace {

constexpr int D = 64;
constexpr int NA = 4, AT = 64, PW = 2, TW = 4, T = PW * TW;
constexpr int CH = D / 8, DC = D / 32, DB = D / 16;
constexpr int RMAX = 128;                     // staged rows of one window
constexpr int SROWS = 256;                    // rows per stage (2 windows, or 16 periods x 16 residues)
constexpr int STG = SROWS * D;                // elements of one stage array (32 KB)
constexpr int DMA_PER_WAVE = 2 * SROWS * CH / (NW * 64);
constexpr int UNIT = 32 * D;                  // one wave's skip unit: 16 K rows + 16 V rows
static_assert(NW * UNIT == STG, "skip units of all waves fill one stage array");
constexpr int IW = 2;                         // skip items (residues) per wave
constexpr int QSLOT = T * D;                  // one item's query rows (T periods)
constexpr int32_t EMPTY = 0x40000000;         // lower bound of an empty key range
static_assert(2 * SROWS * CH % (NW * 64) == 0, "stage split");
static_assert(SROWS * CH % (DMA_PER_WAVE * 64) == 0, "a wave stages only K or only V");
static_assert(T <= 16, "query columns");

typedef __attribute__((address_space(3))) void lds_void_t;

// Element offset of 16-byte chunk c of stage row r.
__device__ __forceinline__ int sw(int r, int c) { return r * D + ((c ^ ((r ^ (r >> 4)) & 7)) << 3); }

struct Ctx {
    const uint16_t* Kb;
    const uint16_t* Vb;
    int32_t skt, svt, n;
};

// One window stage of LDS-direct loads (K rows into Ks, V rows into Vs).
// Load i of wave w covers chunks [64 ((w%4)*DMA_PER_WAVE + i), +64) of K
// (waves 0-3) or V (waves 4-7): rows r0 .. r0+7 (r0 a multiple of 8), lane l
// taking row r0 + l/8 and physical chunk l%8.  base(r0) is the sequence row
// of stage row r0; rows r0..r0+7 are consecutive sequence rows.  lc0 is
// ((l%8) ^ (l/8)) * 8, loff the lane's row offset (l/8) * token stride.
template <class Base>
__device__ __forceinline__ void dma_window(uint16_t* Ks, uint16_t* Vs, const Ctx& c, int32_t lc0, uint32_t loff,
                                           Base base) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const bool isv = wave >= NW / 2;
    const uint16_t* src0 = isv ? c.Vb : c.Kb;
    uint16_t* dst = isv ? Vs : Ks;
    const int32_t st = isv ? c.svt : c.skt;
#pragma unroll
    for (int i = 0; i < DMA_PER_WAVE; ++i) {
        const int c0 = ((wave % (NW / 2)) * DMA_PER_WAVE + i) * 64;
        const int r0 = c0 >> 3;
        const int32_t lc8 = lc0 ^ (((r0 >> 4) & 7) << 3);
        const int32_t s0 = __builtin_amdgcn_readfirstlane(base(r0));
        // uniform base + 32-bit lane offset (rows r0..r0+7 all inside the
        // sequence: no per-lane clamp)
        const bool inside = s0 >= 0 && s0 + 7 < c.n;
        const uint16_t* ub = inside ? src0 + (int64_t)s0 * st : src0;
        const uint32_t off = inside ? loff + (uint32_t)lc8
                                    : (uint32_t)(imin32(imax32(s0 + (lane >> 3), 0), c.n - 1) * st + lc8);
        const char* srcb = reinterpret_cast<const char*>(ub) + (uint32_t)(off * 2u);   // byte offset
        __builtin_amdgcn_global_load_lds(srcb, (lds_void_t*)(dst + c0 * 8), 16, 0, 0);
    }
}

// Element offset of 16-byte chunk c of row r (0..15) of a skip unit; the key
// (r/2) % 8 puts the 16 rows of a K-operand read on distinct banks.
__device__ __forceinline__ int swu(int r, int c) { return r * D + ((c ^ ((r >> 1) & 7)) << 3); }

// All LDS reads of one skip unit -- two 16-byte K-operand chunks and four
// transposed V-operand reads -- issued together and completed inside the
// block.  The unit's slice was filled by this wave's own LDS-direct loads,
// which the caller has already waited for with vmcnt; keeping these reads
// out of the compiler's view keeps it from adding its own (conservative,
// pipeline-draining) vmcnt waits in front of them.
__device__ __forceinline__ void unit_reads(uint32_t k0, uint32_t k1, uint32_t v0, uint32_t v1, uint32_t v2,
                                           uint32_t v3, bf16x8_t& ka, bf16x8_t& kb, s16x4_t (&vv)[4]) {
    asm volatile(
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %1, %7\n\t"
        "ds_read_b64_tr_b16 %2, %8\n\t"
        "ds_read_b64_tr_b16 %3, %9\n\t"
        "ds_read_b64_tr_b16 %4, %10\n\t"
        "ds_read_b64_tr_b16 %5, %11\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(ka), "=&v"(kb), "=&v"(vv[0]), "=&v"(vv[1]), "=&v"(vv[2]), "=&v"(vv[3])
        : "v"(k0), "v"(k1), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
        : "memory");
}

// LDS reads of one item's query operand (two 16-byte chunks) and gate
// logit, completed inside the block (same reasoning as unit_reads).
__device__ __forceinline__ void item_reads(uint32_t q0, uint32_t q1, uint32_t ga, bf16x8_t& qa, bf16x8_t& qb,
                                           float& gl) {
    asm volatile(
        "ds_read_b128 %0, %3\n\t"
        "ds_read_b128 %1, %4\n\t"
        "ds_read_b32 %2, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(qa), "=&v"(qb), "=&v"(gl)
        : "v"(q0), "v"(q1), "v"(ga)
        : "memory");
}

// Merge-record LDS traffic, also kept out of the compiler's view (the
// stage arrays it uses receive LDS-direct loads at other times).  Record
// layout: 4 f32x4 (one per 16-row block of O^T) 512 bytes apart.
__device__ __forceinline__ void lds_write_o(uint32_t a, f32x4_t v0, f32x4_t v1, f32x4_t v2, f32x4_t v3) {
    asm volatile(
        "ds_write_b128 %0, %1\n\t"
        "ds_write_b128 %0, %2 offset:512\n\t"
        "ds_write_b128 %0, %3 offset:1024\n\t"
        "ds_write_b128 %0, %4 offset:1536"
        :
        : "v"(a), "v"(v0), "v"(v1), "v"(v2), "v"(v3)
        : "memory");
}
__device__ __forceinline__ void lds_write_ml(uint32_t a, float m, float l) {
    asm volatile("ds_write2_b32 %0, %1, %2 offset1:1" : : "v"(a), "v"(m), "v"(l) : "memory");
}
__device__ __forceinline__ void lds_read_oml(uint32_t a, uint32_t aml, f32x4_t (&v)[4], float& m, float& l) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    f32x2_t ml;
    asm volatile(
        "ds_read_b128 %0, %5\n\t"
        "ds_read_b128 %1, %5 offset:512\n\t"
        "ds_read_b128 %2, %5 offset:1024\n\t"
        "ds_read_b128 %3, %5 offset:1536\n\t"
        "ds_read2_b32 %4, %6 offset1:1\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(ml)
        : "v"(a), "v"(aml)
        : "memory");
    m = ml.x;
    l = ml.y;
}


// Number of periods t >= 0 with res + t*pi < n, for a residue res in
// [a0, a0 + pi) of a sequence in which residue a0 has P periods.
__device__ __forceinline__ int32_t periods_of(int32_t res, int32_t P, int32_t pi, int32_t n) {
    return P - (res + (P - 1) * pi >= n ? 1 : 0);
}

// Whether row (residue res, period t) has any skip key: a backward skip
// needs t >= mlo, a forward one t + mlo < periods of res; none if M < mlo.
template <bool BIDIR>
__device__ __forceinline__ bool has_skip_rt(int32_t t, int32_t pr, int32_t mlo, int32_t M) {
    return M >= mlo && (t >= mlo || (BIDIR && t + mlo < pr));
}

template <bool BIDIR>
__global__ __launch_bounds__(NT) void fwd_resid_kernel(FwdArgs a, int32_t a_tiles, int32_t t_tiles,
                                                       int32_t total_tiles) {
    // window stages: A = (st0 K, st1 V), B = (st2 K, st3 V); skip units
    // rotate through st0..st3, each wave in its own UNIT-sized slice
    __shared__ __attribute__((aligned(16))) uint16_t st0[STG];
    __shared__ __attribute__((aligned(16))) uint16_t st1[STG];
    __shared__ __attribute__((aligned(16))) uint16_t st2[STG];
    __shared__ __attribute__((aligned(16))) uint16_t st3[STG];
    __shared__ __attribute__((aligned(16))) uint16_t qst[NW * IW * QSLOT];   // items' query rows
    __shared__ __attribute__((aligned(16))) float gst[NW * IW * 64];          // items' gate logits
    __shared__ __attribute__((aligned(16))) float mrec[16 * T * 2];             // items' (m, l)
    __shared__ __attribute__((aligned(16))) float mrec32[16 * T];               // items' fp32 mass

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
        varlen_seq(a.cu, b, a.n, &tok0, &n);
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
    const int32_t NU = NA * nkb * IW;              // skip units per wave: a-group, key block, item

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
    const int32_t lc0 = ((lane & 7) ^ (lane >> 3)) << 3;
    const uint32_t loff = (uint32_t)((lane >> 3) * (wave >= NW / 2 ? cx.svt : cx.skt));
    // skip-unit loads: lane l takes row 8*half + l/8 (key period offset) and
    // physical chunk l%8 of K (loads 0, 1) or V (loads 2, 3)
    uint32_t uoff[2][2];
    int32_t ulc[2];
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
        const int r = 8 * hf + (lane >> 3);
        ulc[hf] = ((lane & 7) ^ ((r >> 1) & 7)) << 3;
        uoff[0][hf] = (uint32_t)r * (uint32_t)pi * (uint32_t)cx.skt + (uint32_t)ulc[hf];
        uoff[1][hf] = (uint32_t)r * (uint32_t)pi * (uint32_t)cx.svt + (uint32_t)ulc[hf];
    }

    auto win_map = [=](int s) {
        return [=](int r) { return a0 + (t0 + PW * s + r / RMAX) * pi - kw + r % RMAX; };
    };
    // Skip unit (ag, kb, it) of this wave: residue a0 + 16*ag + 2*wave + it,
    // key periods klo + 16*kb + [0, 16); row u of the unit's K and V is key
    // period klo + 16*kb + u (rows past the sequence: clamped, masked).
    // Rows past the last key period any of the tile's queries uses (or past
    // the sequence) repeat the last needed row: the repeated lines are
    // fetched once per load, and the rows are masked out.
    auto dma_unit = [&](uint16_t* stj, int ag, int kb, int it) __attribute__((always_inline)) {
        const int32_t res = a0 + 16 * ag + 2 * wave + it;
        const int32_t row0 = res + (klo + 16 * kb) * pi;
        const int32_t umax = imin32(khi, periods_of(res, P, pi, n) - 1) - (klo + 16 * kb);
        const bool full = umax >= 15;
        uint16_t* Kd = stj + wave * UNIT;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int isv = i >> 1, hf = i & 1;
            const uint16_t* src0 = isv ? cx.Vb : cx.Kb;
            const int32_t stv = isv ? cx.svt : cx.skt;
            const uint16_t* ub = full ? src0 + (int64_t)row0 * stv : src0;
            const int32_t ue = imin32(8 * hf + (lane >> 3), imax32(umax, 0));
            const uint32_t off =
                full ? uoff[isv][hf] : (uint32_t)(imin32(row0 + ue * pi, n - 1) * stv + ulc[hf]);
            const char* srcb = reinterpret_cast<const char*>(ub) + (uint32_t)(off * 2u);
            __builtin_amdgcn_global_load_lds(srcb, (lds_void_t*)(Kd + isv * 16 * D + hf * 8 * D), 16, 0, 0);
        }
    };

    const float sl2 = a.scale_log2;
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    // ---- row groups of this wave: period t_j = t0 + wp + 2j
    bf16x8_t qf[TW][DC];
    f32x4_t acc[TW][DB];
    // lrun: this lane's quarter of the row's sum of the bf16 P that acc is
    // built from (the normaliser); l32: this lane's keys' exponentials in
    // fp32 (the row's mass: its log-sum-exp)
    float mrun[TW], lrun[TW], l32[TW], pl[TW];
    int32_t ij[TW];
    bool qv[TW];
    {
        const int32_t res = a0 + 16 * ga + x;
        const int32_t pr = periods_of(res, P, pi, n);
#pragma unroll
        for (int j = 0; j < TW; ++j) {
            const int32_t tj = t0 + wp + PW * j;
            ij[j] = res + tj * pi;
            qv[j] = tj < pr;
            const int32_t ic = qv[j] ? ij[j] : 0;
#pragma unroll
            for (int c = 0; c < DC; ++c) {
                uint4 u = make_uint4(0, 0, 0, 0);
                if (qv[j]) u = *reinterpret_cast<const uint4*>(Qb + (int64_t)ic * a.sq.t + 32 * c + 8 * g);
                qf[j][c] = as_bf16x8(u);
            }
            // gate logit; its prior is formed at the row group's first window
            // step, so these loads are all in flight together
            pl[j] = qv[j] ? a.g[gbase + (int64_t)ic * a.sg.t] : 0.0f;
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) acc[j][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            mrun[j] = -INFINITY;
            lrun[j] = 0.0f;
            l32[j] = 0.0f;
        }
    }

    // ---------------------------------------------------------- window step
    auto local = [&](int j, const uint16_t* Ks, const uint16_t* Vs) __attribute__((always_inline)) {
        const int32_t tp = t0 + wp + PW * j;
        if (tp >= P) return;                          // wave-uniform
        {
            float psk;
            gate_priors(pl[j], has_skip_rt<BIDIR>(tp, periods_of(a0 + 16 * ga + x, P, pi, n), mlo, M), &pl[j], &psk);
        }
        const int wrow0 = wp * RMAX + 16 * ga;
        const int32_t i = ij[j];
        const int32_t key0 = tp * pi + a0 - kw + 16 * ga;
        const int32_t vlo = qv[j] ? imax32(0, i - kw) - key0 : EMPTY;
        const uint32_t vspan = qv[j] ? (uint32_t)(imin32(n - 1, BIDIR ? i + kw : i) - key0 - vlo) : 0u;
        const int32_t rel0 = 4 * g - vlo;
        float mL = mrun[j] + LAZY, cst = pl[j] - (mrun[j] == -INFINITY ? 0.0f : mrun[j]);
        constexpr int KBC = 4;
        for (int32_t kb0 = 0; kb0 < NB; kb0 += KBC) {
            float sc[KBC][4];
            float mx = -INFINITY;
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
                    for (int r = 0; r < 4; ++r) sc[u][r] = (uint32_t)(relb + r) <= vspan ? s4[r] : -INFINITY;
                    mx = fmax_ieee(mx, fmax_ieee(fmax_ieee(sc[u][0], sc[u][1]), fmax_ieee(sc[u][2], sc[u][3])));
                }
            }
            mx = fmaf(max4(mx), sl2, pl[j]);
            if (__builtin_amdgcn_ballot_w64(mx > mL)) {
                const float mnew = fmax_ieee(mrun[j], mx);
                const float mu = mnew == -INFINITY ? 0.0f : mnew;
                const float fac = exp2_fast(mrun[j] - mu);
#pragma unroll
                for (int bb = 0; bb < DB; ++bb) acc[j][bb] *= fac;
                lrun[j] *= fac;
                l32[j] *= fac;
                mrun[j] = mnew;
                mL = mnew + LAZY;
                cst = pl[j] - mu;
            }
            s16x4_t pb[KBC];
#pragma unroll
            for (int u = 0; u < KBC; ++u) {
                if (kb0 + u < NB) {
                    // P in bf16 for the PV products and the normaliser,
                    // the mass from the fp32 values
                    float p[4];
#pragma unroll
                    for (int r = 0; r < 4; ++r) p[r] = exp2_fast(fmaf(sc[u][r], sl2, cst));
                    pb[u] = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));
                    l32[j] += (p[0] + p[1]) + (p[2] + p[3]);
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
                    bf16x8_t va[DB];
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb) {
                        const s16x4_t v0 = ld_tr16(Vs + sw(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        const s16x4_t v1 = ld_tr16(Vs + sw(rb + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                        va[bb] = __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                    }
                    lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pp, lsum, 0, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb)
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[bb], pp, acc[j][bb], 0, 0, 0);
                } else {
                    s16x4_t va[DB];
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb)
                        va[bb] = ld_tr16(Vs + sw(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                    lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb[u], lsum, 0, 0, 0);
#pragma unroll
                    for (int bb = 0; bb < DB; ++bb)
                        acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va[bb], pb[u], acc[j][bb], 0, 0, 0);
                }
            }
            lrun[j] += 0.25f * lsum[0];   // quarter per lane; sum4 at the end restores the row sum
        }
    };

    // ---------------------------------------------------------- skip items
    // Item it of this wave: residue a0 + 16*ag + 2*wave + it; query column
    // col = lane % 16 is period t0 + col (a query for col < T).
    bf16x8_t sq[IW][DC];
    f32x4_t sacc[IW][DB];
    float sm[IW], sl[IW], sl32[IW], sps[IW], smL[IW], scst[IW];
    int32_t slo[IW], stq[IW];
    uint32_t sspan[IW];
    const int col = x;
    // LDS-direct loads of the items' query rows (lane l: period l/8, chunk
    // l%8; one 16-byte load per lane covers the T = 8 rows of an item) and
    // gate logits (lane l: period l%8) for a-group ag, into this wave's
    // private slots: 4 loads.
    // lane constants: query row p = l/8 of the item, its swizzled chunk, and
    // gate period l%8 (32-bit offsets from a uniform row base)
    const int32_t lcq = ((lane & 7) ^ (((lane >> 3) >> 1) & 7)) << 3;
    const uint32_t qoff = (uint32_t)(lane >> 3) * (uint32_t)pi * (uint32_t)a.sq.t + (uint32_t)lcq;
    const uint32_t goff = (uint32_t)(lane & 7) * (uint32_t)pi * (uint32_t)a.sg.t;
    auto item_dma = [&](int ag) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < IW; ++it) {
            const int32_t rb = a0 + 16 * ag + 2 * wave + it + t0 * pi;   // row of period t0
            const int slot = wave * IW + it;
            const bool inside = rb + (T - 1) * pi < n;
            const uint16_t* qsrc;
            const float* gsrc;
            if (inside) {
                qsrc = Qb + (int64_t)rb * a.sq.t + qoff;
                gsrc = a.g + gbase + (int64_t)rb * a.sg.t + goff;
            } else {
                const int32_t row = imin32(rb + (lane >> 3) * pi, n - 1);
                const int32_t grow = imin32(rb + (lane & 7) * pi, n - 1);
                qsrc = Qb + (int64_t)row * a.sq.t + lcq;
                gsrc = a.g + gbase + (int64_t)grow * a.sg.t;
            }
            __builtin_amdgcn_global_load_lds(qsrc, (lds_void_t*)(qst + slot * QSLOT), 16, 0, 0);
            __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)(gst + slot * 64), 4, 0, 0);
        }
    };
    auto item_init = [&](int ag) __attribute__((always_inline)) {
#pragma unroll
        for (int it = 0; it < IW; ++it) {
            const int32_t res = a0 + 16 * ag + 2 * wave + it;
            const int32_t tq = t0 + col;
            const int32_t pr = periods_of(res, P, pi, n);
            const bool v = col < T && tq < pr;
            const int slot = wave * IW + it;
            const int xr = x & 7;                        // columns >= T read a valid row and are masked
            const uint32_t qa = lds_addr(qst + slot * QSLOT) + 2u * (uint32_t)(xr * D);
            float gl;
            item_reads(qa + 16u * (uint32_t)((g ^ ((xr >> 1) & 7))), qa + 16u * (uint32_t)(((4 + g) ^ ((xr >> 1) & 7))),
                       lds_addr(gst + slot * 64) + 4u * (uint32_t)xr, sq[it][0], sq[it][1], gl);
            float plk;
            gate_priors(gl, has_skip_rt<BIDIR>(tq, pr, mlo, M), &plk, &sps[it]);
            // key periods [lo, hi] (bidirectional: minus the hole |kp - tq| < mlo)
            const int32_t lo = imax32(tq - M, 0);
            const int32_t hi = BIDIR ? imin32(tq + M, pr - 1) : tq - mlo;
            const bool ne = v && M >= mlo && hi >= lo;
            slo[it] = ne ? lo : EMPTY;
            sspan[it] = ne ? (uint32_t)(hi - lo) : 0u;
            stq[it] = tq;
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) sacc[it][bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            sm[it] = -INFINITY;
            smL[it] = -INFINITY;
            sl[it] = 0.0f;
            sl32[it] = 0.0f;
            scst[it] = sps[it];
        }
    };
    auto item_unit = [&](int kb, const uint16_t* stj, auto itc) __attribute__((always_inline)) {
        constexpr int it = decltype(itc)::value;
        const uint32_t base = lds_addr(stj) + (uint32_t)(wave * UNIT * 2);
        bf16x8_t kk[DC];
        s16x4_t vv[DB];
        static_assert(DC == 2 && DB == 4, "unit_reads shape");
        unit_reads(base + 2 * swu(x, g), base + 2 * swu(x, 4 + g),
                   base + 2 * (16 * D + swu(tr_row, 0 + (tr_col >> 3)) + (tr_col & 7)),
                   base + 2 * (16 * D + swu(tr_row, 2 + (tr_col >> 3)) + (tr_col & 7)),
                   base + 2 * (16 * D + swu(tr_row, 4 + (tr_col >> 3)) + (tr_col & 7)),
                   base + 2 * (16 * D + swu(tr_row, 6 + (tr_col >> 3)) + (tr_col & 7)), kk[0], kk[1], vv);
        const int32_t kp0 = klo + 16 * kb + 4 * g;      // key period of this lane's value r = 0
        f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DC; ++c) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk[c], sq[it][c], s4, 0, 0, 0);
        const int32_t e0 = kp0 - slo[it];
        const int32_t h0 = kp0 - stq[it] + mlo - 1;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            bool ok = (uint32_t)(e0 + r) <= sspan[it];
            if (BIDIR) ok = ok && (uint32_t)(h0 + r) > (uint32_t)(2 * mlo - 2);
            sc[r] = ok ? s4[r] : -INFINITY;
        }
        const float mx = fmaf(max4(fmax_ieee(fmax_ieee(sc[0], sc[1]), fmax_ieee(sc[2], sc[3]))), sl2, sps[it]);
        if (__builtin_amdgcn_ballot_w64(mx > smL[it])) {
            const float mnew = fmax_ieee(sm[it], mx);
            const float mu = mnew == -INFINITY ? 0.0f : mnew;
            const float fac = exp2_fast(sm[it] - mu);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb) sacc[it][bb] *= fac;
            sl[it] *= fac;
            sl32[it] *= fac;
            sm[it] = mnew;
            smL[it] = mnew + LAZY;
            scst[it] = sps[it] - mu;
        }
        float p[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = exp2_fast(fmaf(sc[r], sl2, scst[it]));
        const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])));
        sl32[it] += (p[0] + p[1]) + (p[2] + p[3]);  // this lane's keys, fp32; sum4 when merged
        const f32x4_t ls = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        sl[it] += ls[0];                         // full column sum in every lane
#pragma unroll
        for (int bb = 0; bb < DB; ++bb)
            sacc[it][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv[bb], pb, sacc[it][bb], 0, 0, 0);
    };
    // Fold the items' partial states for a-group ag into the row groups'
    // registers, in one exchange.  Each wave writes its two items' O^T
    // (2 x 8 columns x 64 floats = its 4 KB slice) into its own slice of the
    // stage array stj whose unit it has just consumed -- private, so no
    // barrier before -- and m, l into mrec; after a barrier the owners of the
    // a-group read all slices; a second barrier frees stj for the next loads.
    // Slice layout [it][bb][g][col ^ (xx % 8)][4]: writes of a wave are
    // contiguous and the owners' 16 residues spread over the banks.
    auto item_merge = [&](int ag, uint16_t* stj) __attribute__((always_inline)) {
        const uint32_t sbase = lds_addr(stj);
#pragma unroll
        for (int it = 0; it < IW; ++it) {
            const int xx = 2 * wave + it;
            const float slf = sum4(sl32[it]);               // the column's fp32 mass (every lane)
            if (col < T) {
                const uint32_t rec = sbase + (uint32_t)(wave * UNIT * 2) +
                                     4u * (uint32_t)(((it * DB) * 4 + g) * 32 + ((col ^ (xx & 7)) << 2));
                lds_write_o(rec, sacc[it][0], sacc[it][1], sacc[it][2], sacc[it][3]);
                if (g == 0) {
                    lds_write_ml(lds_addr(mrec) + 8u * (uint32_t)(xx * T + col), sm[it], sl[it]);
                    mrec32[xx * T + col] = slf;
                }
            }
        }
        lds_barrier();
        if (ga == ag) {
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                const int cj = wp + PW * j;                 // column of row group j
                const uint32_t rec = sbase + (uint32_t)((x >> 1) * UNIT * 2) +
                                     4u * (uint32_t)((((x & 1) * DB) * 4 + g) * 32 + ((cj ^ (x & 7)) << 2));
                f32x4_t sv[DB];
                float msk, lsk;
                lds_read_oml(rec, lds_addr(mrec) + 8u * (uint32_t)(x * T + cj), sv, msk, lsk);
                const float mnew = fmax_ieee(mrun[j], msk);
                const float mu = mnew == -INFINITY ? 0.0f : mnew;
                const float fl = exp2_fast(mrun[j] - mu);
                const float fs = exp2_fast(msk - mu);
                lrun[j] = lrun[j] * fl + 0.25f * lsk * fs;
                l32[j] = l32[j] * fl + 0.25f * mrec32[x * T + cj] * fs;
                mrun[j] = mnew;
#pragma unroll
                for (int bb = 0; bb < DB; ++bb) acc[j][bb] = acc[j][bb] * fl + sv[bb] * fs;
            }
        }
        lds_barrier();
    };
    // Process unit u (a-group ag, key block kb, item IT) from stage array
    // stj after issuing unit u+3 into nxt; each wave waits only for its own
    // loads (its slice is private), so units need no workgroup barrier.
    // Every unit issues exactly 4 loads (past the last unit: a harmless
    // reload of the last one), so the loads of unit u are always followed by
    // those of units u+1..u+3 and vmcnt(12) waits for exactly unit u.
    auto issue = [&](uint16_t* stj, int v) __attribute__((always_inline)) {
        const int q = imin32(v, NU - 1) >> 1;          // IW == 2 units per (a-group, key block)
        dma_unit(stj, q / nkb, q % nkb, imin32(v, NU - 1) & 1);
    };
    auto unit = [&](int u, const uint16_t* stj, uint16_t* nxt, auto itc) __attribute__((always_inline)) {
        constexpr int it = decltype(itc)::value;
        issue(nxt, u + 3);
        __builtin_amdgcn_s_waitcnt(0xF7C);             // vmcnt(12): unit u has landed
        const int q = u >> 1, ag = q / nkb, kb = q % nkb;
        if (it == 0 && kb == 0) {
            // The query/gate loads of a-group ag were issued while processing
            // the first unit of a-group ag-1 (after that step's unit issue),
            // so 8*nkb unit loads follow them by now: vmcnt(12) covers them
            // once nkb >= 2.
            if (nkb == 1) __builtin_amdgcn_s_waitcnt(0xF78);   // vmcnt(8)
            item_init(ag);
            if (ag + 1 < NA) item_dma(ag + 1);         // the slots were just read
        }
        item_unit(kb, stj, itc);
        if (it == IW - 1 && kb == nkb - 1) item_merge(ag, const_cast<uint16_t*>(stj));   // workgroup-uniform
    };

    // ---------------------------------------------------------- schedule
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    static_assert(IW == 2, "unit loop unrolled for two items");
    dma_window(st0, st1, cx, lc0, loff, win_map(0));
    __syncthreads();
    dma_window(st2, st3, cx, lc0, loff, win_map(1));
    local(0, st0, st1);
    __syncthreads();
    dma_window(st0, st1, cx, lc0, loff, win_map(2));
    local(1, st2, st3);
    __syncthreads();
    dma_window(st2, st3, cx, lc0, loff, win_map(3));
    local(2, st0, st1);
    __syncthreads();
    if (NU > 0) {
        item_dma(0);
        issue(st0, 0);
        issue(st1, 1);
    }
    local(3, st2, st3);
    if (NU > 0) {
        lds_barrier();                                  // every wave is done with st2, st3
        issue(st2, 2);
        for (int u = 0; u < NU; u += 4) {
            unit(u, st0, st3, I0{});
            unit(u + 1, st1, st0, I1{});
            if (u + 2 >= NU) break;
            unit(u + 2, st2, st1, I0{});
            unit(u + 3, st3, st2, I1{});
        }
        // the reloads issued past the last unit must land before the
        // workgroup (and its LDS) can retire
        __builtin_amdgcn_s_waitcnt(0xF70);             // vmcnt(0)
    }

    // ---- normalise and store (bf16, round to nearest even)
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const float ltot = sum4(lrun[j]);
        const float lmass = sum4(l32[j]);                // cross-lane: before the lane exits
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
        if (a.lse && g == 0) a.lse[gbase + (int64_t)ij[j] * a.sg.t] = (mrun[j] + __log2f(lmass)) * PIATTN_LN2;
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
    // the contiguous skip range [floor(k/pi)+1, M] only (no skip schedules)
    if (a.pat.masked || a.pat.mlo != a.pat.k / a.pat.pi + 1) return false;
    int64_t ts = a.sk.t > a.sv.t ? a.sk.t : a.sv.t;
    ts = ts > a.sq.t ? ts : a.sq.t;
    // row offsets in bytes below 2^31 (the same value read as signed or unsigned)
    if (((int64_t)a.n * ts + D) * 2 >= ((int64_t)1 << 31)) return false;
    if ((int64_t)a.n * a.sg.t * 4 >= ((int64_t)1 << 31)) return false;
    // row indices such as a0 + (t0 + T + 15) * pi stay in int32
    if ((int64_t)a.n + (int64_t)(2 * T + 16) * a.pat.pi >= ((int64_t)1 << 31)) return false;
    const int64_t w = (int64_t)a.pat.k + 16 + (a.pat.bidir ? a.pat.k : 0);
    return 16 * (NA - 1) + 16 * ((w + 15) / 16) <= RMAX;
}

hipError_t launch_fwd_resid(const FwdArgs& a, hipStream_t stream) {
    return a.pat.bidir ? launch_t<true>(a, stream) : launch_t<false>(a, stream);
}
