// fwd_tiled.hip -- residue-tiled prefill on bf16 MFMA (gfx950).
//
// Geometry.  Write a query row as i = a + t*pi: residue a in [0, pi), period
// t.  A workgroup owns A = 16*NA consecutive residues [a0, a0+A) over T
// consecutive periods [t0, t0+T): A*T query rows.  Each of its 8 waves owns
// one 16-residue "a-group" (16 consecutive rows of one period: the MFMA
// query dimension) for TW of the tile's periods and keeps the online-softmax
// state of those rows (running max m, sum l, fp32 accumulator O^T) in
// registers for the whole kernel.
//
// Stream.  The workgroup walks key periods t' from t0 - M (causal) to
// t0 + T - 1 (+M when bidirectional), one LDS stage per t' (double buffered:
// the rows of step t'+1 are fetched into registers while step t' computes).
// A stage holds rows [a0 + t'pi - k, a0 + t'pi + A (+k)) of K and V,
// row-major, 16-byte chunks XOR-swizzled by row; when t' is not one of the
// tile's periods only the A-row "own block" [a0 + t'pi, a0 + t'pi + A) is
// fetched.  Then every wave, for each row group it owns at period t:
//   * t - t' = m in [floor(k/pi)+1, M] (or t' - t when bidirectional) -- the
//     pages' "pi-Skip Attention": the skip key of row a + t*pi is a + t'*pi,
//     i.e. row x of the own block for the group's row x.  The 16 scores are
//     VALU bf16 dot products (v_dot2) reduced over the 4 lanes of a query with
//     v_permlane16/32_swap; they get the log(1-alpha) prior and join the
//     online softmax (lazy rescale: the running max moves only when a score
//     exceeds it by 8 in log2 units); P is diagonal, so O^T += V^T P^T is one
//     v_mfma_f32_16x16x16_bf16 per 16 head-dim rows.  All of a wave's groups
//     are updated together for instruction-level parallelism.
//   * t == t' -- "Ring-Local Attention": the window of the 16 rows is a band
//     of 16 x (k+16) (or 16 x (2k+16)) keys: S^T = K Q^T on
//     v_mfma_f32_16x16x32_bf16, mask, log(alpha) prior, online softmax,
//     O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 over 32-key pairs.
// One softmax covers window and skips ("Dynamic Adaptive Fusion").  Each own
// block is fetched once per tile and serves up to T row groups, so skip K/V
// is re-read (T+M)/T times per query instead of M times.
//
// Layouts.  S^T = K Q^T keeps the query in the lane index (lane = 16*g + x:
// query x, key rows 4g..4g+3 of a 16-key block), which is the B layout P^T
// needs for O^T = V^T P^T and the layout of the O^T accumulator (lane: query
// x, head-dim rows 16b + 4g + r).  m and l are per-lane values for query x,
// replicated over the 4 lanes g.  The V^T operand is read from row-major V
// with ds_read_b64_tr_b16: lane L of lane group g supplies the address of
// V[row0 + 4g + L/4][col0 + 4(L%4)] and receives V[row0 + 4g + s][col0 + L]
// for s = 0..3.
#include "common.hpp"
#include "kernels.hpp"

#include "mfma_util.hpp"

namespace {

template <int D, int NA, int TW, int RMAX, bool BIDIR>
__global__ __launch_bounds__(NT) void fwd_tiled_kernel(FwdArgs a, int32_t a_tiles, int32_t t_tiles,
                                                       int32_t total_tiles) {
    constexpr int AT = 16 * NA;         // residues per tile
    constexpr int PW = NW / NA;         // waves per a-group
    constexpr int T = PW * TW;          // periods per tile
    constexpr int CH = D / 8;           // 16-byte chunks per row
    constexpr int KIT = RMAX * CH / NT; // staging chunks per thread (K, and again V)
    constexpr int DC = D / 32;          // QK^T MFMA depth chunks
    constexpr int DB = D / 16;          // O^T row blocks
    constexpr int STAGE = 2 * RMAX * D; // elements per stage (K then V)
    constexpr int KBC = D == 64 ? 4 : 2; // 16-key blocks per softmax chunk of the window
    static_assert(RMAX * CH % NT == 0, "staging split");

    __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

    // XCD-aware order: consecutive hardware ids go round-robin over the 8
    // XCDs; give each XCD a contiguous run of logical tiles so that tiles
    // sharing K/V rows share an L2.
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
    const int32_t P = (n - a0 + pi - 1) / pi;  // periods holding a row of this residue tile
    const int32_t t0 = tt * T;
    if (t0 >= P) return;
    const int32_t mlo = kw / pi + 1;
    const bool any_skip = M >= mlo;
    const int32_t ts = any_skip ? imax32(0, t0 - M) : t0;
    const int32_t te = imin32(P - 1, t0 + T - 1 + ((BIDIR && any_skip) ? M : 0));
    // Window of a row group: W = k + 16 (+k) keys in NB 16-key blocks; group
    // ga's window starts at region row 16*ga, so a local step stages
    // RR = 16*(NA-1) + 16*NB rows (<= RMAX, checked on the host); rows past
    // the window are real rows (or copies of row 0) and are masked out.
    const int32_t W = kw + 16 + (BIDIR ? kw : 0);
    const int32_t NB = (W + 15) >> 4;
    const int32_t RR = 16 * (NA - 1) + 16 * NB;

    const int64_t bq = a.cu ? 0 : (int64_t)b;
    const uint16_t* Qb = static_cast<const uint16_t*>(a.q) + bq * a.sq.s + h * a.sq.h + tok0 * a.sq.t;
    const uint16_t* Kb = static_cast<const uint16_t*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const uint16_t* Vb = static_cast<const uint16_t*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    uint16_t* Ob = static_cast<uint16_t*>(a.o) + bq * a.so.s + h * a.so.h + tok0 * a.so.t;
    const int64_t gbase = bq * a.sg.s + h * a.sg.h + tok0 * a.sg.t;

    // ---- per-wave row groups: period t_j, rows a0 + 16*ga + x + t_j*pi
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

    // ---- staging: global -> registers (one step ahead) -> swizzled LDS
    uint4 kreg[KIT], vreg[KIT];
    auto fetch = [&](int32_t tp) {
        const bool local = tp >= t0 && tp < t0 + T;
        const int32_t lo = local ? 0 : kw;           // first staged region row
        const int32_t hi = local ? RR : kw + AT;      // one past the last
        const int32_t rstart = a0 + tp * pi - kw;     // sequence row of region row 0
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int id = tid + it * NT;
            const int row = lo + id / CH, cc = id % CH;
            const int32_t r = rstart + row;
            uint4 ku = make_uint4(0, 0, 0, 0), vu = make_uint4(0, 0, 0, 0);
            if (row < hi && r >= 0 && r < n) {
                ku = *reinterpret_cast<const uint4*>(Kb + (int64_t)r * a.sk.t + 8 * cc);
                vu = *reinterpret_cast<const uint4*>(Vb + (int64_t)r * a.sv.t + 8 * cc);
            }
            kreg[it] = ku;
            vreg[it] = vu;
        }
    };
    auto commit = [&](int32_t tp, int stage) {
        const bool local = tp >= t0 && tp < t0 + T;
        const int32_t lo = local ? 0 : kw;
        const int32_t hi = local ? RR : kw + AT;
        uint16_t* Ks = smem + stage * STAGE;
        uint16_t* Vs = Ks + RMAX * D;
#pragma unroll
        for (int it = 0; it < KIT; ++it) {
            const int id = tid + it * NT;
            const int row = lo + id / CH, cc = id % CH;
            if (row < hi) {
                *reinterpret_cast<uint4*>(Ks + swz<D>(row, cc)) = kreg[it];
                *reinterpret_cast<uint4*>(Vs + swz<D>(row, cc)) = vreg[it];
            }
        }
    };

    const float sl2 = a.scale_log2;
    const int ro = kw + 16 * ga;                  // region row of the own block
    // transposing-read lane roles: row offset and column within a 16-col block
    const int tr_row = 4 * g + (x >> 2);
    const int tr_col = 4 * (x & 3);
    // diagonal-owner lane of query x: g == x/4, element r == x%4
    const bool owner = g == (x >> 2);
    const int xr = x & 3;
    const uint2 dmask = make_uint2(owner ? (xr == 0 ? 0x0000ffffu : xr == 1 ? 0xffff0000u : 0u) : 0u,
                                   owner ? (xr == 2 ? 0x0000ffffu : xr == 3 ? 0xffff0000u : 0u) : 0u);
    const bf16x8_t ones8 = __builtin_bit_cast(bf16x8_t, make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u));
    const s16x4_t ones4 = __builtin_bit_cast(s16x4_t, make_uint2(0x3f803f80u, 0x3f803f80u));

    fetch(ts);
    commit(ts, 0);
    __syncthreads();
    int stage = 0;
    for (int32_t tp = ts; tp <= te; ++tp) {
        if (tp < te) fetch(tp + 1);
        const uint16_t* Ks = smem + stage * STAGE;
        const uint16_t* Vs = Ks + RMAX * D;

        // ---------------- periodic skips: diagonal of the own block
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
        if (any_sk) {
            // S^T = K_own Q^T per group on MFMA; only the diagonal is used.
            // Lane (x, g) holds key rows 4g..4g+3, so the diagonal element of
            // query x sits in the "owner" lane g = x/4 at r = x%4.
            const bool own_key_ok = a0 + 16 * ga + x + tp * pi < n;
            bf16x8_t kf[DC];
#pragma unroll
            for (int c = 0; c < DC; ++c)
                kf[c] = *reinterpret_cast<const bf16x8_t*>(Ks + swz<D>(ro + x, 4 * c + g));
            float sd[TW];
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int c = 0; c < DC; ++c)
                    s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[j][c], s4, 0, 0, 0);
                const float v = diag_pick(s4, xr);
                sd[j] = (owner && sk[j] && qv[j] && own_key_ok) ? fmaf(v, sl2, ps[j]) : -INFINITY;
            }
            bool need_any = false;
#pragma unroll
            for (int j = 0; j < TW; ++j) need_any |= sd[j] > mrun[j] + LAZY;
            if (__any(need_any)) {
                // rare: move the running max of the rows whose skip score
                // exceeds it by more than LAZY (broadcast from the owner lane)
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
            for (int bb = 0; bb < DB; ++bb)
                vf[bb] = ld_tr16(Vs + swz<D>(ro + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                if (!sk[j]) continue;                 // wave-uniform
                const float p = (sd[j] == -INFINITY) ? 0.0f : exp2_fast(sd[j] - mrun[j]);
                const uint32_t pw = cvt_pk_bf16(p, p);      // p rounded, in both halves
                lrun[j] += __uint_as_float(pw << 16);       // owner lane only (others add 0)
                const uint2 pbw = make_uint2(pw & dmask.x, pw & dmask.y);
                const s16x4_t pb = __builtin_bit_cast(s16x4_t, pbw);
#pragma unroll
                for (int bb = 0; bb < DB; ++bb)
                    acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vf[bb], pb, acc[j][bb], 0, 0, 0);
            }
        }

        // ---------------- ring-local window of the group whose period is t'
        const int32_t jl_raw = tp - t0 - wp;          // owner: PW*j == tp - t0 - wp
        if (jl_raw >= 0 && jl_raw % PW == 0 && jl_raw / PW < TW && tp < P) {
#pragma unroll
            for (int j = 0; j < TW; ++j) {
                if (j != jl_raw / PW) continue;       // wave-uniform
                const int32_t i = ij[j];
                const int32_t key0 = tp * pi + a0 - kw + 16 * ga;  // sequence row of window row 0
                // valid keys of query x relative to key0: [vlo, vhi] (empty if row invalid)
                const int32_t vlo = imax32(0, i - kw) - key0;
                const int32_t vhi = (qv[j] ? imin32(n - 1, BIDIR ? i + kw : i) : -1) - key0;
                const uint32_t vspan = (uint32_t)(vhi - vlo);
                const int32_t rel0 = 4 * g - vlo;      // lane's relative key offset in block 0
                for (int32_t kb0 = 0; kb0 < NB; kb0 += KBC) {
                    float sc[KBC][4];
#pragma unroll
                    for (int u = 0; u < KBC; ++u) {
                        if (kb0 + u < NB) {
                            const int rb = 16 * ga + 16 * (kb0 + u);
                            f32x4_t s4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                            for (int c = 0; c < DC; ++c) {
                                const bf16x8_t kk =
                                    *reinterpret_cast<const bf16x8_t*>(Ks + swz<D>(rb + x, 4 * c + g));
                                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kk, qf[j][c], s4, 0, 0, 0);
                            }
                            const int32_t relb = rel0 + 16 * (kb0 + u);
#pragma unroll
                            for (int r = 0; r < 4; ++r) {
                                const bool ok = (uint32_t)(relb + r) <= vspan;
                                sc[u][r] = ok ? fmaf(s4[r], sl2, pl[j]) : -INFINITY;
                            }
                        } else {
#pragma unroll
                            for (int r = 0; r < 4; ++r) sc[u][r] = -INFINITY;
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
                        const uint32_t w0 = cvt_pk_bf16(exp2_fast(sc[u][0] - mu), exp2_fast(sc[u][1] - mu));
                        const uint32_t w1 = cvt_pk_bf16(exp2_fast(sc[u][2] - mu), exp2_fast(sc[u][3] - mu));
                        pb[u] = __builtin_bit_cast(s16x4_t, make_uint2(w0, w1));
                    }
                    // O^T += V^T P^T: pairs of 16-key blocks on 16x16x32 (keys
                    // {4g..4g+3} of block u then of block u+1 per lane), an odd
                    // last block on 16x16x16.  The row sum of the same bf16 P
                    // comes from one more MFMA with an all-ones V^T operand.
                    f32x4_t lsum = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int u = 0; u < KBC; u += 2) {
                        if (kb0 + u >= NB) continue;
                        const int rb = 16 * ga + 16 * (kb0 + u);
                        if (kb0 + u + 1 < NB) {
                            const bf16x8_t pp = __builtin_bit_cast(
                                bf16x8_t, __builtin_shufflevector(pb[u], pb[u + 1], 0, 1, 2, 3, 4, 5, 6, 7));
                            lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones8, pp, lsum, 0, 0, 0);
#pragma unroll
                            for (int bb = 0; bb < DB; ++bb) {
                                const s16x4_t v0 =
                                    ld_tr16(Vs + swz<D>(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                                const s16x4_t v1 =
                                    ld_tr16(Vs + swz<D>(rb + 16 + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                                const bf16x8_t va = __builtin_bit_cast(
                                    bf16x8_t, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
                                acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pp, acc[j][bb], 0, 0, 0);
                            }
                        } else {
                            lsum = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ones4, pb[u], lsum, 0, 0, 0);
#pragma unroll
                            for (int bb = 0; bb < DB; ++bb) {
                                const s16x4_t v0 =
                                    ld_tr16(Vs + swz<D>(rb + tr_row, 2 * bb + (tr_col >> 3)) + (tr_col & 7));
                                acc[j][bb] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(v0, pb[u], acc[j][bb], 0, 0, 0);
                            }
                        }
                    }
                    // every row of the ones block holds the full sum; keep a
                    // quarter per lane so that sum4 at the end restores it
                    lrun[j] += 0.25f * lsum[0];
                }
            }
        }

        if (tp < te) {
            commit(tp + 1, stage ^ 1);
            __syncthreads();
            stage ^= 1;
        }
    }

    // ---- normalise and store (bf16, round to nearest even)
#pragma unroll
    for (int j = 0; j < TW; ++j) {
        const float ltot = sum4(lrun[j]);             // per-lane partial sums -> row sum
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
        if (a.lse && g == 0)
            a.lse[gbase + (int64_t)ij[j] * a.sg.t] = (mrun[j] + __log2f(ltot)) * PIATTN_LN2;
    }
}

template <int D, int NA, int TW, int RMAX, bool BIDIR>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    constexpr int T = (NW / NA) * TW;
    const int32_t a_tiles = a.pat.pi / (16 * NA);
    const int32_t periods = (a.n + a.pat.pi - 1) / a.pat.pi;
    const int32_t t_tiles = (periods + T - 1) / T;
    const int64_t total = (int64_t)a_tiles * t_tiles * a.H * a.B;
    if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((fwd_tiled_kernel<D, NA, TW, RMAX, BIDIR>), dim3((uint32_t)total), dim3(NT), 0,
                       stream, a, a_tiles, t_tiles, (int32_t)total);
    return hipGetLastError();
}

// Staged rows a local step needs with NA a-groups per tile.
int64_t region_rows(const FwdArgs& a, int na) {
    const int64_t w = (int64_t)a.pat.k + 16 + (a.pat.bidir ? a.pat.k : 0);
    return 16 * (na - 1) + 16 * ((w + 15) / 16);
}

}  // namespace

bool fwd_tiled_supported(int dtype, const FwdArgs& a) {
    if (dtype != 1) return false;
    if (a.d == 64) return a.pat.pi % 64 == 0 && region_rows(a, 4) <= 256;
    if (a.d == 128) return a.pat.pi % 32 == 0 && region_rows(a, 2) <= 160;
    return false;
}

hipError_t launch_fwd_tiled(const FwdArgs& a, hipStream_t stream) {
    if (a.d == 64) {
        if (region_rows(a, 4) <= 128)
            return a.pat.bidir ? launch_t<64, 4, 4, 128, true>(a, stream)
                               : launch_t<64, 4, 4, 128, false>(a, stream);
        return a.pat.bidir ? launch_t<64, 4, 4, 256, true>(a, stream)
                           : launch_t<64, 4, 4, 256, false>(a, stream);
    }
    return a.pat.bidir ? launch_t<128, 2, 2, 160, true>(a, stream)
                       : launch_t<128, 2, 2, 160, false>(a, stream);
}
