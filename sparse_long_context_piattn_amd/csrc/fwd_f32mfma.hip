// fwd_f32mfma.hip -- fp32 prefill on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, gfx950), head dim 32, 64 or 128.
//
// One wave per 16 consecutive query rows of a (sequence, head).  Its keys are
// the union of the rows' windows and skip keys (gist.science "pi-Attention
// ...", section 2, items "Ring-Local Attention" and "pi-Skip Attention"),
// visited as 16-key blocks in increasing key order: the backward skip ranges
// [i0 - m pi, i0 + 15 - m pi] from the farthest m, the window, then (both
// directions) the forward skip ranges.  Those ranges are non-decreasing, so a
// block shared by two of them is visited once, and a per-element membership
// test picks each key's kind.  Per block:
//   S^T = K Q^T     d/4 MFMAs; the contraction runs over d in the order
//                   (lane group g, step c) -> d = g d/4 + c, so each lane
//                   reads d/4 consecutive floats of one K row and one Q row;
//   P = exp2(S scale log2(e) + prior - running max), the union's single
//                   online softmax in fp32 (the "Dynamic Adaptive Fusion"
//                   prior: log alpha on window keys, log(1 - alpha) on skip
//                   keys, none on rows without skip keys);
//   O^T += V^T P^T  4 MFMAs per 16 output dims; the contraction runs over
//                   the block's keys in the order (g, step s) -> key 4 g + s,
//                   which is where the S^T result already holds P, so P
//                   feeds the MFMA from its own registers.
// Everything stays fp32: no rounding of P, sums of the exponentials in fp32.
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace {

template <int D, bool MASKED>
__global__ __launch_bounds__(256) void fwd_f32mfma_kernel(FwdArgs a, int32_t qblocks, int64_t total) {
    constexpr int DQ = D / 4;                        // d values per lane group in S^T = K Q^T
    constexpr int DB = D / 16;                       // 16-dim output blocks
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
    const int64_t item = (int64_t)blockIdx.x * 4 + wave;   // (sequence, head, 16-row block)
    if (item >= total) return;                             // wave-uniform; no barriers below
    const int32_t qb = (int32_t)(item % qblocks);
    const int64_t rest = item / qblocks;
    const int32_t h = (int32_t)(rest % a.H), b = (int32_t)(rest / a.H);
    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) varlen_seq(a.cu, b, a.n, &tok0, &n);
    const int32_t i0 = 16 * qb;
    if (i0 >= n) return;
    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const float* Qb = static_cast<const float*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    const float* Kb = static_cast<const float*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const float* Vb = static_cast<const float*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    float* Ob = static_cast<float*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    const PiPattern& p = a.pat;

    // the lane's query row (column x of S^T) and its priors
    const int32_t i = i0 + x;
    const bool qv = i < n;
    const int32_t ic = qv ? i : n - 1;
    float qr[DQ];
#pragma unroll
    for (int c = 0; c < DQ; c += 4) {
        const float4 v4 = *reinterpret_cast<const float4*>(Qb + ic * a.sq.t + g * DQ + c);
        qr[c] = v4.x, qr[c + 1] = v4.y, qr[c + 2] = v4.z, qr[c + 3] = v4.w;
    }
    const RowSpan sp = row_span_t<MASKED>(ic, n, p);
    float pl, ps;
    gate_priors(a.g[bq * a.sg.s + h * a.sg.h + (tok0 + ic) * a.sg.t], sp.has_skip(), &pl, &ps);
    const float sl2 = a.scale_log2;

    // membership of key j in row i's union: 0 none, 1 window, 2 skip
    auto kind_of = [&](int32_t j) __attribute__((always_inline)) {
        if ((uint32_t)j >= (uint32_t)n) return 0;
        const int32_t dd = i - j;
        const int32_t ad = dd < 0 ? -dd : dd;
        if (dd >= (p.bidir ? -p.k : 0) && dd <= p.k) return 1;
        if (dd < 0 && !p.bidir) return 0;
        if (ad % p.pi != 0) return 0;
        const int32_t m = ad / p.pi;
        if (m < p.mlo || m > p.M) return 0;
        if (MASKED && !mask_has(p, m)) return 0;
        return 2;
    };

    f32x4_t acc[DB];
#pragma unroll
    for (int bb = 0; bb < DB; ++bb) acc[bb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float mrun = -INFINITY, lpart = 0.0f;            // running max (log2 units); this lane's part of the sum

    auto block = [&](int32_t k0) __attribute__((always_inline)) {
        // S^T[key k0 + 4 g + r][query x]
        const int32_t kr = imin32(k0 + x, n - 1);    // A operand row: key k0 + x (clamped; masked below)
        const float* krow = Kb + kr * a.sk.t + g * DQ;
        f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < DQ; c += 4) {
            const float4 kv = *reinterpret_cast<const float4*>(krow + c);
            s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.x, qr[c], s4, 0, 0, 0);
            s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.y, qr[c + 1], s4, 0, 0, 0);
            s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.z, qr[c + 2], s4, 0, 0, 0);
            s4 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv.w, qr[c + 3], s4, 0, 0, 0);
        }
        float lg[4];
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int kd = qv ? kind_of(k0 + 4 * g + r) : 0;
            lg[r] = kd == 0 ? -INFINITY : fmaf(s4[r], sl2, kd == 1 ? pl : ps);
            mx = fmax_ieee(mx, lg[r]);
        }
        mx = max4(mx);
        const float mnew = fmax_ieee(mrun, mx);
        const float mu = mnew == -INFINITY ? 0.0f : mnew;
        const float fac = exp2_fast(mrun - mu);
#pragma unroll
        for (int bb = 0; bb < DB; ++bb) acc[bb] *= fac;
        lpart *= fac;
        mrun = mnew;
        float pv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            pv[r] = exp2_fast(lg[r] - mu);
            lpart += pv[r];
        }
        // O^T[d = 16 bb + 4 g + r][x] += sum over steps s of V[k0 + 4 g' + s][16 bb + x] P[x][4 g' + s]
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int32_t vr = imin32(k0 + 4 * g + s, n - 1);
            const float* vrow = Vb + vr * a.sv.t + x;
#pragma unroll
            for (int bb = 0; bb < DB; ++bb)
                acc[bb] = __builtin_amdgcn_mfma_f32_16x16x4f32(vrow[16 * bb], pv[s], acc[bb], 0, 0, 0);
        }
    };

    // the union's 16-key blocks in increasing key order, each once
    int32_t last = -1;                               // last block visited
    auto range = [&](int32_t lo, int32_t hi) __attribute__((always_inline)) {
        lo = imax32(lo, 0);
        hi = imin32(hi, n - 1);
        if (lo > hi) return;
        for (int32_t bk = imax32(lo >> 4, last + 1); bk <= (hi >> 4); ++bk) block(16 * bk);
        last = imax32(last, hi >> 4);
    };
    const int32_t i1 = imin32(i0 + 15, n - 1);
    for (int32_t m = imin32(p.M, i1 / p.pi); m >= p.mlo; --m) {   // multiples with a key at or after 0
        if (MASKED && !mask_has(p, m)) continue;
        const int32_t dist = m * p.pi;
        range(i0 - dist, i1 - dist);
    }
    range(i0 - p.k, p.bidir ? i1 + p.k : i1);
    if (p.bidir) {
        for (int32_t m = p.mlo; m <= imin32(p.M, (n - 1 - i0) / p.pi); ++m) {   // keys before n
            if (MASKED && !mask_has(p, m)) continue;
            const int32_t dist = m * p.pi;
            range(i0 + dist, i1 + dist);
        }
    }

    const float l = sum4(lpart);
    if (!qv) return;
    const float inv = 1.0f / l;
    float* orow = Ob + (int64_t)i * a.so.t;
#pragma unroll
    for (int bb = 0; bb < DB; ++bb)
        *reinterpret_cast<float4*>(orow + 16 * bb + 4 * g) =
            make_float4(acc[bb][0] * inv, acc[bb][1] * inv, acc[bb][2] * inv, acc[bb][3] * inv);
    if (a.lse && g == 0) a.lse[bq * a.sg.s + h * a.sg.h + (tok0 + i) * a.sg.t] = (mrun + __log2f(l)) * PIATTN_LN2;
}

template <int D>
hipError_t launch_d(const FwdArgs& a, hipStream_t stream) {
    const int32_t qblocks = (a.n + 15) / 16;
    const int64_t total = (int64_t)a.B * a.H * qblocks;
    const int64_t grid = (total + 3) / 4;
    if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (a.pat.masked)
        hipLaunchKernelGGL((fwd_f32mfma_kernel<D, true>), dim3((uint32_t)grid), dim3(256), 0, stream, a, qblocks, total);
    else
        hipLaunchKernelGGL((fwd_f32mfma_kernel<D, false>), dim3((uint32_t)grid), dim3(256), 0, stream, a, qblocks, total);
    return hipGetLastError();
}

}  // namespace

// fp32 inputs at head dim 32, 64 or 128 (16-byte aligned rows, strides of
// whole float4s: the API's fp32 requirements).  Addressing is 64-bit, so no
// size bound applies beyond the API's.
bool fwd_f32mfma_supported(int dtype, const FwdArgs& a) {
    return dtype == 0 && (a.d == 32 || a.d == 64 || a.d == 128);
}

// Whether this kernel beats the per-row gather kernel on a call.  The MFMA
// kernel scans whole 16-key blocks: the window's, and per skip multiple one
// block (two when pi is not a multiple of 16) of which each row uses one key,
// against a row's (k + 1 [+ k]) + skips keys for the gather kernel.  Measured
// on gfx950 at d = 64: 4.1 scanned key slots per useful pair ran 1.36x
// faster than the gather kernel (B4 H16 n8192, k64 pi128 M16), 8.6 ran
// 1.67x slower (bidirectional n32768, k32 pi64 M32); break-even near 5.5.
// Calls of at most 65536 rows sit at the launch floor either way (B1 H2
// n256 d32: 12.7 against 12.9 us) and take this kernel.
bool fwd_f32mfma_preferred(const FwdArgs& a) {
    const PiPattern& p = a.pat;
    if ((int64_t)a.B * a.H * a.n <= 65536) return true;
    const int64_t dirs = p.bidir ? 2 : 1;
    const int64_t nsk = p.M < p.mlo ? 0 : p.masked ? mask_rank(p, p.M) : p.M - p.mlo + 1;
    const int64_t win_blocks = ((int64_t)p.k * dirs + 15) / 16 + 1 + (p.k % 16 != 0);
    const int64_t skip_blocks = dirs * nsk * (p.pi % 16 == 0 ? 1 : 2);
    const int64_t pairs = (int64_t)p.k * dirs + 1 + dirs * nsk;
    return 16 * (win_blocks + skip_blocks) * 2 <= 11 * pairs;
}

hipError_t launch_fwd_f32mfma(const FwdArgs& a, hipStream_t stream) {
    switch (a.d) {
        case 32: return launch_d<32>(a, stream);
        case 64: return launch_d<64>(a, stream);
        case 128: return launch_d<128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}
