// bwd.hip -- backward of the prefill: gradients of q, k, v and the gate
// logits, on the per-row gather path (gfx950, wave64).
//
// For row i with keys j in L(i) u S(i) (the forward's one softmax):
//   P_ij  = exp2(s_ij - lse2_i),  s_ij in log2 units with the gate prior
//   dP_ij = <dout_i, v_j>,   D_i = <dout_i, out_i> = sum_j P_ij dP_ij
//   dS_ij = P_ij (dP_ij - D_i)                 (gradient of the natural logit)
//   dq_i  = scale sum_j dS_ij k_j,  dk_j = scale sum_i dS_ij q_i,
//   dv_j  = sum_i P_ij dout_i,
//   dg_i  = (1 - alpha_i) sum_{j in L} dS_ij - alpha_i sum_{j in S} dS_ij
//           (the derivatives of log(alpha) and log(1 - alpha); 0 on rows
//           without skip keys, which carry no prior).
// Two kernels, one wavefront per row each, in the lane layout of gather.hpp
// (NS key slots of LPK lanes, 8 head-dim elements per lane):
//   bwd_dq_kernel   query row i: its log-sum-exp recomputed in fp32 (first
//                   sweep over its keys), D_i from the forward output, then
//                   dq_i and dg_i (second sweep); (lse2_i, D_i) go to the
//                   workspace;
//   bwd_dkv_kernel  key row j: the queries whose union holds j -- the window
//                   rows around j and the rows j +- m pi, m in [floor(k/pi)+1,
//                   M] (the transpose of the pattern) -- give dk_j and dv_j.
#include "gather.hpp"
#include "kernels.hpp"

namespace {

struct RowLoc {
    int64_t tok0;   // first token of the sequence
    int64_t bq;     // sequence index for the sequence stride (0 in varlen mode)
    int32_t n;      // sequence length
};

__device__ __forceinline__ RowLoc row_loc(const FwdArgs& a, int32_t b) {
    RowLoc r;
    r.n = a.n;
    r.tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &r.tok0, &r.n);
    }
    r.bq = a.cu ? 0 : (int64_t)b;
    return r;
}

// Sum over the LPK lanes of a key slot (every lane gets the slot's sum).
template <int D>
__device__ __forceinline__ float slot_sum(float x) {
#pragma unroll
    for (int off = 1; off < GatherShape<D>::LPK; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

// Sum over the NS key slots (lanes LPK apart).
template <int D>
__device__ __forceinline__ float across_slots(float x) {
#pragma unroll
    for (int off = GatherShape<D>::LPK; off < 64; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs ba) {
    using G = GatherShape<D>;
    const FwdArgs& a = ba.f;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = lane / G::LPK, c = (lane % G::LPK) * 8;
    const int32_t i = blockIdx.x * 4 + wave;
    const int32_t h = blockIdx.y, b = blockIdx.z;
    const RowLoc rl = row_loc(a, b);
    if (i >= rl.n) return;
    const int64_t tok = rl.tok0 + i;
    const T* qrow = static_cast<const T*>(a.q) + rl.bq * a.sq.s + h * a.sq.h + tok * a.sq.t;
    const T* kb = static_cast<const T*>(a.k) + rl.bq * a.sk.s + h * a.sk.h + rl.tok0 * a.sk.t;
    const T* vb = static_cast<const T*>(a.v) + rl.bq * a.sv.s + h * a.sv.h + rl.tok0 * a.sv.t;
    const int64_t orow = rl.bq * a.so.s + h * a.so.h + tok * a.so.t;
    const int64_t goff = rl.bq * a.sg.s + h * a.sg.h + tok * a.sg.t;

    const RowSpan sp = row_span(i, rl.n, a.pat);
    const int32_t U = sp.total();
    const float gl = a.g[goff];
    float pl, ps;
    gate_priors(gl, sp.has_skip(), &pl, &ps);

    float q8[8], do8[8], o8[8];
    Elem<T>::load8(qrow + c, q8);
    Elem<T>::load8(static_cast<const T*>(ba.dout) + orow + c, do8);
    Elem<T>::load8(static_cast<const T*>(a.o) + orow + c, o8);
    float dpart = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        dpart = fmaf(do8[e], o8[e], dpart);
        q8[e] *= a.scale_log2;
    }
    const float Drow = slot_sum<D>(dpart);

    // sweep 1: the row's log2-sum-exp (running max shared by the wave)
    float m = -INFINITY, l = 0.0f;
    for (int32_t base = 0; base < U; base += G::NS) {
        const int32_t u = base + slot;
        float s = -INFINITY;
        if (u < U) {
            bool loc;
            const int32_t key = span_key(sp, i, a.pat, u, &loc);
            float k8[8];
            Elem<T>::load8(kb + (int64_t)key * a.sk.t + c, k8);
            float dot = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) dot = fmaf(q8[e], k8[e], dot);
            s = slot_sum<D>(dot) + (loc ? pl : ps);
        }
        float cm = s;
#pragma unroll
        for (int off = G::LPK; off < 64; off <<= 1) cm = fmaxf(cm, __shfl_xor(cm, off, 64));
        const float mn = fmaxf(m, cm);
        const float mu = mn == -INFINITY ? 0.0f : mn;
        l = l * exp2_fast(m - mu) + exp2_fast(s - mu);
        m = mn;
    }
    const float lse2 = m + __log2f(across_slots<D>(l));

    // sweep 2: dS, dq, the gate sums
    float dq8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dq8[e] = 0.0f;
    float sum_l = 0.0f, sum_s = 0.0f;
    for (int32_t base = 0; base < U; base += G::NS) {
        const int32_t u = base + slot;
        if (u < U) {
            bool loc;
            const int32_t key = span_key(sp, i, a.pat, u, &loc);
            float k8[8], v8[8];
            Elem<T>::load8(kb + (int64_t)key * a.sk.t + c, k8);
            Elem<T>::load8(vb + (int64_t)key * a.sv.t + c, v8);
            float dot = 0.0f, dpv = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dot = fmaf(q8[e], k8[e], dot);
                dpv = fmaf(do8[e], v8[e], dpv);
            }
            const float p = exp2_fast(slot_sum<D>(dot) + (loc ? pl : ps) - lse2);
            const float ds = p * (slot_sum<D>(dpv) - Drow);
#pragma unroll
            for (int e = 0; e < 8; ++e) dq8[e] = fmaf(ds, k8[e], dq8[e]);
            if (loc)
                sum_l += ds;
            else
                sum_s += ds;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) dq8[e] = across_slots<D>(dq8[e]) * ba.scale;
    sum_l = across_slots<D>(sum_l);
    sum_s = across_slots<D>(sum_s);
    if (lane < G::LPK)
        Elem<T>::store8(static_cast<T*>(ba.dq) + rl.bq * a.sq.s + h * a.sq.h + tok * a.sq.t + c, dq8);
    if (lane == 0) {
        const float alpha = 1.0f / (1.0f + __expf(-gl));
        ba.dg[goff] = sp.has_skip() ? (1.0f - alpha) * sum_l - alpha * sum_s : 0.0f;
        float* st = ba.rowstat + (((int64_t)b * a.H + h) * a.n + i) * 2;
        st[0] = lse2;
        st[1] = Drow;
    }
}

// The queries whose union holds key j, as union positions u in [0, total):
// the window rows [wlo, whi], then (bidirectional) the rows j - m pi, then
// the rows j + m pi, m running over the pattern's skip multiples.
struct KeySpan {
    int32_t wlo, whi;   // window rows
    int32_t nb;         // rows j - m pi (bidirectional only)
    int32_t nf;         // rows j + m pi
    __device__ int32_t n_win() const { return whi - wlo + 1; }
    __device__ int32_t total() const { return n_win() + nb + nf; }
    __device__ int32_t row(int32_t j, const PiPattern& p, int32_t u, bool* loc) const {
        if (u < n_win()) {
            *loc = true;
            return wlo + u;
        }
        u -= n_win();
        *loc = false;
        if (u < nb) return j - skip_multiple(p, u) * p.pi;
        return j + skip_multiple(p, u - nb) * p.pi;
    }
};

// Key j is in L(i) iff |i - j| <= k (and i >= j when causal); it is in S(i)
// iff i - j = +-m pi for a skip multiple m of the pattern (all beyond k).
__device__ __forceinline__ KeySpan key_span(int32_t j, int32_t n, const PiPattern& p) {
    KeySpan r;
    r.wlo = p.bidir ? imax32(0, j - p.k) : j;
    r.whi = imin32(n - 1, j + p.k);
    r.nb = p.bidir ? skips_upto(p, j / p.pi) : 0;
    r.nf = skips_upto(p, (n - 1 - j) / p.pi);
    return r;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_dkv_kernel(BwdArgs ba) {
    using G = GatherShape<D>;
    const FwdArgs& a = ba.f;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = lane / G::LPK, c = (lane % G::LPK) * 8;
    const int32_t j = blockIdx.x * 4 + wave;
    const int32_t h = blockIdx.y, b = blockIdx.z;
    const RowLoc rl = row_loc(a, b);
    if (j >= rl.n) return;
    const int64_t tokj = rl.tok0 + j;
    const T* qb = static_cast<const T*>(a.q) + rl.bq * a.sq.s + h * a.sq.h + rl.tok0 * a.sq.t;
    const T* dob = static_cast<const T*>(ba.dout) + rl.bq * a.so.s + h * a.so.h + rl.tok0 * a.so.t;
    const float* gb = a.g + rl.bq * a.sg.s + h * a.sg.h + rl.tok0 * a.sg.t;
    const float* stb = ba.rowstat + ((int64_t)b * a.H + h) * a.n * 2;

    float k8[8], v8[8];
    Elem<T>::load8(static_cast<const T*>(a.k) + rl.bq * a.sk.s + h * a.sk.h + tokj * a.sk.t + c, k8);
    Elem<T>::load8(static_cast<const T*>(a.v) + rl.bq * a.sv.s + h * a.sv.h + tokj * a.sv.t + c, v8);
#pragma unroll
    for (int e = 0; e < 8; ++e) k8[e] *= a.scale_log2;

    const KeySpan ks = key_span(j, rl.n, a.pat);
    const int32_t U = ks.total();
    float dk8[8], dv8[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dk8[e] = dv8[e] = 0.0f;
    for (int32_t base = 0; base < U; base += G::NS) {
        const int32_t u = base + slot;
        if (u < U) {
            bool loc;
            const int32_t i = ks.row(j, a.pat, u, &loc);
            float q8[8], do8[8];
            Elem<T>::load8(qb + (int64_t)i * a.sq.t + c, q8);
            Elem<T>::load8(dob + (int64_t)i * a.so.t + c, do8);
            float dot = 0.0f, dpv = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dot = fmaf(q8[e], k8[e], dot);
                dpv = fmaf(do8[e], v8[e], dpv);
            }
            float pl, ps;
            gate_priors(gb[(int64_t)i * a.sg.t], row_span(i, rl.n, a.pat).has_skip(), &pl, &ps);
            const float2 st = *reinterpret_cast<const float2*>(stb + (int64_t)i * 2);
            const float p = exp2_fast(slot_sum<D>(dot) + (loc ? pl : ps) - st.x);
            const float ds = p * (slot_sum<D>(dpv) - st.y);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                dk8[e] = fmaf(ds, q8[e], dk8[e]);
                dv8[e] = fmaf(p, do8[e], dv8[e]);
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        dk8[e] = across_slots<D>(dk8[e]) * ba.scale;
        dv8[e] = across_slots<D>(dv8[e]);
    }
    if (lane < G::LPK) {
        Elem<T>::store8(static_cast<T*>(ba.dk) + rl.bq * a.sk.s + h * a.sk.h + tokj * a.sk.t + c, dk8);
        Elem<T>::store8(static_cast<T*>(ba.dv) + rl.bq * a.sv.s + h * a.sv.h + tokj * a.sv.t + c, dv8);
    }
}

template <typename T, int D>
hipError_t launch_t(const BwdArgs& ba, hipStream_t stream) {
    const dim3 grid((ba.f.n + 3) / 4, ba.f.H, ba.f.B);
    hipLaunchKernelGGL((bwd_dq_kernel<T, D>), grid, dim3(256), 0, stream, ba);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dkv_kernel<T, D>), grid, dim3(256), 0, stream, ba);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd(int dtype, const BwdArgs& ba, hipStream_t stream) {
    if (dtype == 0) {
        switch (ba.f.d) {
            case 32: return launch_t<float, 32>(ba, stream);
            case 64: return launch_t<float, 64>(ba, stream);
            case 128: return launch_t<float, 128>(ba, stream);
        }
    } else {
        switch (ba.f.d) {
            case 32: return launch_t<uint16_t, 32>(ba, stream);
            case 64: return launch_t<uint16_t, 64>(ba, stream);
            case 128: return launch_t<uint16_t, 128>(ba, stream);
        }
    }
    return hipErrorInvalidValue;
}
