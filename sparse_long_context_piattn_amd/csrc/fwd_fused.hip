// fwd_fused.hip -- fused prefill for head dim 64 or 128 (gfx950, bf16 MFMA):
// the skip work and the window work of the split path in one kernel, ordered
// so that the window work reads what the skip work just wrote, and the q, k,
// v rows both read, from the L2 of the same XCD rather than from HBM.
//
// Work items.  A (sequence, head) is cut into segments of 16 periods (rows
// [16 c pi, 16 (c+1) pi)).  Segment c has R = ceil(min(pi, n) / 4) skip items
// -- four residues, one per wave, each taking the segment's 16 query periods
// of its residue in the residue layout (the pi-Skip Attention part: keys
// i -/+ m pi) and leaving the rows' skip partials in their output slots and
// records -- and W = pi / 4 window tiles of 64 rows (the Ring-Local Attention
// part and the merge with the skip partials).  A window tile needs the
// partials of its own rows only, which all lie in its segment (pi % 4 == 0
// keeps tiles inside segments).
//
// Queues.  Each (sequence, head) belongs to one of NQ queues, one per XCD.
// A queue lists its segments g = 0, 1, ... (its heads one after the other)
// as blocks: the skip items of segment g, then the window tiles of segment
// g - LA, so that the skip work runs LA segments ahead of the window work
// that waits for it.  A workgroup takes the next ticket of the queue of the
// XCD it runs on (the XCC_ID hardware register) and never another's, so the
// producer and the consumer of every hand-off share that XCD's L2: a skip
// wave counts itself in its segment's counter once its stores are complete in
// L2, and a window tile polls the counter in L2 and reads the partials with
// loads that L2 serves (no cache write-back or invalidate).  The grid is
// persistent (a fixed number of workgroups per CU, dealt to the XCDs in
// turn); each workgroup claims tickets until its queue is empty.  An item
// waits only on items with smaller tickets of its own queue, which are held
// by workgroups that are already running and wait on nothing larger, so the
// smallest unfinished ticket always progresses: no deadlock, however many
// workgroups are resident.  The waits are bounded anyway (kWaitTicks).
//
// Measured against the split path on gfx950 (prefill of 4 x 16 heads x 8192
// rows, d = 64, k = 64, pi = 128, M = 16): 0.132 ms per call against 0.111,
// and 612 MB of HBM traffic against 617 -- the partials and the second reads
// of q, k, v still reach HBM, because the XCD's 4 MB L2 does not hold the
// segments in flight between a skip item and the window tiles that wait for
// it.  The library therefore runs this kernel only when asked to by name.
//
// The counters live in the caller's workspace after the per-row records; a
// small kernel zeroes them before each call.
#include "fwd_common.hpp"

#include <type_traits>

namespace {

using namespace fwdk;

// Segments of skip work a queue runs ahead of its window work.
#ifndef PIATTN_FUSED_LOOKAHEAD
#define PIATTN_FUSED_LOOKAHEAD 3
#endif
constexpr int32_t kLookahead = PIATTN_FUSED_LOOKAHEAD;
// Workgroups per CU in the grid (persistent; 0: one workgroup per batch).
#ifndef PIATTN_FUSED_WG_PER_CU
#define PIATTN_FUSED_WG_PER_CU 6
#endif
// Consecutive tickets a workgroup claims with one atomic (fewer atomics on
// the queue's counter, whose line every workgroup of the XCD hits).
#ifndef PIATTN_FUSED_BATCH
#define PIATTN_FUSED_BATCH 1
#endif
constexpr int32_t kBatch = PIATTN_FUSED_BATCH;

// Schedule of one call (host-computed).
struct FusedSched {
    int32_t* tick;      // next ticket of each queue (kCounterStride apart)
    int32_t* segcnt;    // [BH][S] skip waves done per segment (kCounterStride apart)
    int32_t* err;       // set when a wait gave up
    int32_t BH;         // (sequence, head) pairs
    int32_t S;          // segments per (sequence, head)
    int32_t R;          // skip items per segment
    int32_t W;          // window tiles per segment (the last one padded with empty tiles)
    int32_t T;          // window tiles per (sequence, head)
    int32_t NQ;         // queues: XCDs of the device
    int32_t QI;         // workgroups per queue (the longest queue's items)
};

template <int D>
struct FusedGeo {
    static constexpr int VW = 16 * D;                          // elements: one block of 16 V rows
    static constexpr int LDS = WinShape<D>::LDS;               // the skip item needs less (checked below)
};

// Skip item: residues rg*SW .. rg*SW+SW-1 (one per wave) of (sequence b,
// head h), query periods [16 c, 16 c + 16).  The keys of those periods are the
// NK 16-period blocks c - NBL .. c (.. c + NBL bidirectional) of the residue.
// One batch of loads brings everything: the query rows and the key rows
// straight into their MFMA operand registers (a lane's 16 bytes of one row),
// the value rows into LDS (the PV operand is read transposed from there).
// Then all NK score blocks are formed and one softmax with the exact column
// max runs over them, as in the split path's register-ring skip pass.  The
// partial leaves through the wave's value slots.  Every wave then signals
// `done` once, whether or not it had rows.
template <int D, int NBL, bool BIDIR>
__device__ __forceinline__ void skip_item(const FwdArgs& a, float* lse_s, int32_t b, int32_t h, int32_t rg,
                                          int32_t c, uint16_t* lds, int32_t* done) {
    using G = Geo<D>;
    constexpr int DC = G::DC, DB = G::DB, CH = G::CH, RPI = G::RPI;
    constexpr int NK = BIDIR ? 2 * NBL + 1 : NBL + 1;
    constexpr int VW = FusedGeo<D>::VW;
    static_assert(SW * NK * VW * 2 <= FusedGeo<D>::LDS, "the skip item's value slots fit the tile's LDS");
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) varlen_seq(a.cu, b, a.n, &tok0, &n);
    const int32_t pi = a.pat.pi, M = a.pat.M, mlo = a.pat.mlo;
    const int32_t res = rg * SW + wave;
    const int32_t pr = res < n ? (n - 1 - res) / pi + 1 : 0;  // periods of this residue
    if (res < pi && 16 * c < pr) {                              // wave-uniform
        const int64_t bq = a.cu ? 0 : (int64_t)b;
        const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
        const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
        const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
        uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
        float* Ls = lse_s + ((int64_t)b * a.H + h) * a.n * 2;
        const int32_t sqt = (int32_t)a.sq.t, skt = (int32_t)a.sk.t, svt = (int32_t)a.sv.t;
        uint16_t* const vs = lds + wave * NK * VW;              // this wave's NK value slots

        // a lane's 16 bytes of the MFMA operand row x (period p0 + x of the
        // residue, clamped into it; rows outside are masked later)
        auto operand_rows = [&](const uint16_t* src, int32_t st, int32_t p0, bf16x8_t (&dst)[DC])
            __attribute__((always_inline)) {
            const int32_t p = imin32(imax32(p0 + x, 0), pr - 1);
            const uint16_t* row = src + (int64_t)(res + p * pi) * st;
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) dst[cc] = *reinterpret_cast<const bf16x8_t*>(row + 8 * (4 * cc + g));
        };
        // 16 value rows of periods p0 .. p0+15 into slot dst: row j*RPI +
        // lane/CH, physical chunk lane%CH holding logical chunk
        // (lane%CH) ^ ((row/2)%8)
        auto value_rows = [&](int32_t p0, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
            for (int j = 0; j < 16 / RPI; ++j) {
                const int32_t lr = j * RPI + lane / CH;
                const int32_t lc = ((lane % CH) ^ ((lr >> 1) & 7)) << 3;
                const int32_t p = imin32(imax32(p0 + lr, 0), pr - 1);
                dma16(Vb, (uint32_t)(((res + p * pi) * svt + lc) * 2), lds_addr(dst + j * RPI * D));
            }
        };

        bf16x8_t sq[DC];
        bf16x8_t kr[NK][DC];
        s16x4_t vr[NK][DB];
#pragma unroll
        for (int e = 0; e < NK; ++e) value_rows(16 * (c - NBL + e), vs + e * VW);
        operand_rows(Qb, sqt, 16 * c, sq);
#pragma unroll
        for (int e = 0; e < NK; ++e) operand_rows(Kb, skt, 16 * (c - NBL + e), kr[e]);
        __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));             // the value rows (the rest waits by itself)

        const int tr_row = 4 * g + (x >> 2);
        const int tr_col = 4 * (x & 3);
#pragma unroll
        for (int e = 0; e < NK; ++e)
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                vr[e][bb] = ld_tr16(vs + e * VW + swu<D>(tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
        __builtin_amdgcn_s_waitcnt(0xC07F);                     // lgkmcnt(0): the slots are free again

        const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));
        const float sl2 = a.scale_log2;
        const int32_t tq = 16 * c + x;
        const bool hs = tq < pr && row_has_skip<BIDIR>(tq, pr, mlo, M);
        const int32_t lo = imax32(tq - M, 0);
        const int32_t hi = BIDIR ? imin32(tq + M, pr - 1) : tq - mlo;
        const int32_t slo = hs ? lo : EMPTY;
        const uint32_t sspan = hs ? (uint32_t)(hi - lo) : 0u;
        // all NK score blocks, then one softmax with the exact column max
        float sc[NK][4];
        float mxl = -INFINITY;
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const int32_t kb = c - NBL + i;
            f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cc = 0; cc < DC; ++cc) s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[i][cc], sq[cc], s4, 0, 0, 0);
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
        const float sm = max4(mxl) * sl2;
        const float scst = sm == -INFINITY ? 0.0f : -sm;
        f32x4_t sacc[DB];
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) sacc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < NK; ++i) {
            const uint32_t w0 = cvt_pk_bf16(exp2_fast(fmaf(sc[i][0], sl2, scst)), exp2_fast(fmaf(sc[i][1], sl2, scst)));
            const uint32_t w1 = cvt_pk_bf16(exp2_fast(fmaf(sc[i][2], sl2, scst)), exp2_fast(fmaf(sc[i][3], sl2, scst)));
            const s16x4_t pb = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
            lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb, lsum, 0, 0, 0);
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                sacc[bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vr[i][bb], pb, sacc[bb], 0, 0, 0);
        }
        store_skip_chunk<D, BIDIR>(vs, sacc, lsum[0], sm, hs, c, res, pr, pi, mlo, M, Ob, a.so.t, Ls, lane);
    }
    // this wave's partial rows and records are written: hand them to the
    // segment's window tiles (one increment per wave)
    signal_segment(done);
}

template <int D>
struct FusedShape {
    static constexpr int EU = D == 64 ? 4 : 3;                   // waves per SIMD the register budget must allow
};

// Ticket t of queue q -> item (((hs * S + c) * (R + W) + slot), or -1 past
// the queue's end.  Blocks: LA skip-only blocks (R items), G - LA mixed
// blocks (R skip items of segment g, then W tiles of segment g - LA), LA
// window-only blocks (W tiles); slot < R is skip item `slot` of the segment,
// else its window tile slot - R.
__device__ __forceinline__ int32_t item_of_ticket(const FusedSched& sc, int32_t q, int32_t G, int32_t t) {
    const int32_t LA = imin32(kLookahead, G);
    int32_t g = -1, r = 0;
    if (t < LA * sc.R) {
        g = t / sc.R;
        r = t - g * sc.R;
    } else if (t < LA * sc.R + (G - LA) * (sc.R + sc.W)) {
        const int32_t t2 = t - LA * sc.R;
        g = LA + t2 / (sc.R + sc.W);
        r = t2 % (sc.R + sc.W);
    } else if (t < G * (sc.R + sc.W)) {
        const int32_t t3 = t - LA * sc.R - (G - LA) * (sc.R + sc.W);
        g = G + t3 / sc.W;
        r = sc.R + t3 % sc.W;
    }
    if (g < 0) return -1;
    const int32_t seg = r < sc.R ? g : g - LA;
    const int32_t hs = seg / sc.S * sc.NQ + q;
    return (hs * sc.S + seg % sc.S) * (sc.R + sc.W) + r;
}

// Persistent workgroups: each claims batches of kBatch consecutive tickets
// of the queue of the XCD it runs on and works through them in order.  A
// workgroup's current item is the smallest ticket it holds, so the smallest
// unfinished ticket is always being worked on.
template <int D, int NBL, bool BIDIR>
__global__ __launch_bounds__(SW * 64, FusedShape<D>::EU) void fwd_fused_kernel(FwdArgs a, float* lse_s,
                                                                               FusedSched sc) {
    static_assert(WinShape<D>::WW == SW, "skip items and window tiles share the workgroup shape");
    __shared__ int32_t base_sh[1];
    __shared__ __attribute__((aligned(16))) uint16_t lds[FusedGeo<D>::LDS / 2];
    uint32_t xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int32_t q = (int32_t)(xcc % (uint32_t)sc.NQ);
    const int32_t heads = (sc.BH - q + sc.NQ - 1) / sc.NQ;       // (sequence, head) pairs q, q+NQ, ...
    const int32_t G = heads > 0 ? heads * sc.S : 0;             // segments of the queue
    const int32_t tickets = G * (sc.R + sc.W);
    int32_t* const tick = sc.tick + q * kCounterStride;
    for (;;) {
        if (threadIdx.x == 0)
            base_sh[0] = tickets > 0 ? kBatch * __hip_atomic_fetch_add(tick, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                     : 0;
        __syncthreads();                                         // the batch is visible; the last item's LDS is free
        const int32_t base = base_sh[0];
        if (base >= tickets) break;                              // workgroup-uniform
        for (int32_t j = 0; j < kBatch && base + j < tickets; ++j) {
            if (j > 0) __syncthreads();                          // the last item's LDS is free
            const int32_t item = item_of_ticket(sc, q, G, base + j);
            const int32_t RW = sc.R + sc.W;
            const int32_t hc = item / RW, r = item - hc * RW;    // (sequence, head) and segment; slot
            const int32_t hs = hc / sc.S, c = hc - hs * sc.S;
            const int32_t b = hs / a.H, h = hs - b * a.H;
            if (r < sc.R) {
                skip_item<D, NBL, BIDIR>(a, lse_s, b, h, r, c, lds, sc.segcnt + (int64_t)hc * kCounterStride);
            } else {
                const int32_t qt = c * sc.W + (r - sc.R);
                if (qt < sc.T) {                                 // else padding of the last segment
                    const SegWait w{sc.segcnt + (int64_t)hs * sc.S * kCounterStride, c, c, SW * sc.R, sc.err};
                    window_tile<D, BIDIR, true>(a, lse_s, 1, qt, h, b, lds, w);
                }
            }
        }
        __syncthreads();                                         // every wave is past base_sh before it changes
    }
}

// Zeroes the queue tickets, the error word and the segment counters.
__global__ __launch_bounds__(256) void fused_clear_kernel(int32_t* p, int32_t count) {
    for (int32_t i = blockIdx.x * 256 + threadIdx.x; i < count; i += gridDim.x * 256) p[i] = 0;
}

template <int D, int NBL, bool BIDIR>
hipError_t launch_t(const FwdArgs& a, float* ws, const FusedLayout& L, hipStream_t stream) {
    int32_t* ctr = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + L.counters_offset);
    const int64_t blocks = (L.counters + 255) / 256;
    hipLaunchKernelGGL(fused_clear_kernel, dim3((uint32_t)(blocks < 64 ? blocks : 64)), dim3(256), 0, stream, ctr,
                       (int32_t)L.counters);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    FusedSched sc;
    sc.tick = ctr;                                               // queue q's ticket at q * kCounterStride
    sc.err = ctr + 8 * kCounterStride;
    sc.segcnt = ctr + 9 * kCounterStride;
    sc.BH = (int32_t)L.BH;
    sc.S = (int32_t)L.S;
    sc.R = (int32_t)L.R;
    sc.W = (int32_t)L.W;
    sc.T = (int32_t)L.T;
    sc.NQ = (int32_t)L.NQ;
    sc.QI = (int32_t)L.QI;
    const int64_t grid = PIATTN_FUSED_WG_PER_CU > 0 ? (int64_t)L.CUs * PIATTN_FUSED_WG_PER_CU
                                                    : L.NQ * ((L.QI + kBatch - 1) / kBatch);
    hipLaunchKernelGGL((fwd_fused_kernel<D, NBL, BIDIR>), dim3((uint32_t)grid), dim3(SW * 64), 0, stream, a, ws, sc);
    return hipGetLastError();
}

}  // namespace

// CUs and XCDs of the current device: MI355X has 32 CUs per XCD (8 in one
// partition of 256 CUs); a device that shows fewer CUs is a partition of
// fewer XCDs.  Looked up once per device.
static void device_shape(int32_t* cus_out, int32_t* xcds_out) {
    static int32_t cache[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    int32_t cus = dev < 64 ? cache[dev] : 0;
    if (cus == 0) {
        int v = 0;
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v < 1) v = 32;
        cus = v;
        if (dev < 64) cache[dev] = cus;
    }
    int32_t nq = cus / 32;
    *cus_out = cus;
    *xcds_out = nq < 1 ? 1 : (nq > 8 ? 8 : nq);
}

// The call's schedule and workspace layout (host).
bool fused_layout(const FwdArgs& a, FusedLayout* L) {
    const int64_t pi = a.pat.pi, n = a.n;
    if (pi % 4 != 0) return false;
    int32_t cus = 0, xcds = 0;
    device_shape(&cus, &xcds);
    L->NQ = xcds;
    L->CUs = cus;
    const int64_t P = (n + pi - 1) / pi;                         // periods of the longest sequence
    L->BH = (int64_t)a.B * a.H;
    L->S = (P + 15) / 16;
    L->R = ((pi < n ? pi : n) + SW - 1) / SW;
    L->W = pi / 4;                                               // 64-row tiles in 16 periods
    L->T = (n + 63) / 64;
    L->E = L->S * (L->R + L->W);                                 // items per pair, the last segment padded
    L->items = L->BH * L->E;
    L->QI = (L->BH + L->NQ - 1) / L->NQ * L->E;
    L->counters = (9 + L->BH * L->S) * kCounterStride;
    L->counters_offset = ((int64_t)a.B * a.H * a.n * 2 * 4 + 255) / 256 * 256;
    return L->T <= L->S * L->W && L->NQ * L->QI < ((int64_t)1 << 31) && L->items < ((int64_t)1 << 31) &&
           L->counters < ((int64_t)1 << 31);
}

bool fwd_fused_supported(int dtype, const FwdArgs& a) {
    if (!fwd_split_supported(dtype, a)) return false;            // bf16, d 64 / 128, 32-bit offsets
    if (a.pat.M < a.pat.mlo) return false;                      // no skip keys: nothing to fuse
    const int32_t nbl = (a.pat.M + 15) / 16;
    if (a.pat.bidir ? nbl > 1 : nbl > 2) return false;         // key blocks held in registers
    FusedLayout L;
    return fused_layout(a, &L);
}

hipError_t launch_fwd_fused(const FwdArgs& a, float* ws, hipStream_t stream) {
    FusedLayout L;
    if (!fused_layout(a, &L)) return hipErrorInvalidValue;
    const int32_t nbl = (a.pat.M + 15) / 16;
    if (a.d == 64) {
        if (a.pat.bidir) return launch_t<64, 1, true>(a, ws, L, stream);
        return nbl == 1 ? launch_t<64, 1, false>(a, ws, L, stream) : launch_t<64, 2, false>(a, ws, L, stream);
    }
    if (a.pat.bidir) return launch_t<128, 1, true>(a, ws, L, stream);
    return nbl == 1 ? launch_t<128, 1, false>(a, ws, L, stream) : launch_t<128, 2, false>(a, ws, L, stream);
}
