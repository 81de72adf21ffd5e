// fwd_gather.hip -- prefill on the per-row gather path: one wavefront per
// query row, four rows per 256-thread workgroup.  Grid (ceil(n/4), H, B).
#include "gather.hpp"
#include "kernels.hpp"

namespace {

template <typename T, int D, bool MASKED>
__global__ __launch_bounds__(256) void fwd_gather_kernel(FwdArgs a) {
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int32_t i = blockIdx.x * 4 + wave;
    const int32_t h = blockIdx.y, b = blockIdx.z;
    int32_t n = a.n;
    int64_t tok0 = 0;
    if (a.cu) {
        varlen_seq(a.cu, b, a.n, &tok0, &n);
    }
    if (i >= n) return;
    const int64_t tok = tok0 + i;
    const int64_t bq = a.cu ? 0 : (int64_t)b;  // sequence stride ignored in varlen mode

    const T* qrow = static_cast<const T*>(a.q) + bq * a.sq.s + h * a.sq.h + tok * a.sq.t;
    const T* kb = static_cast<const T*>(a.k) + bq * a.sk.s + h * a.sk.h + tok0 * a.sk.t;
    const T* vb = static_cast<const T*>(a.v) + bq * a.sv.s + h * a.sv.h + tok0 * a.sv.t;
    const int64_t goff = bq * a.sg.s + h * a.sg.h + tok * a.sg.t;

    const RowSpan sp = row_span_t<MASKED>(i, n, a.pat);
    float pl, ps;
    gate_priors(a.g[goff], sp.has_skip(), &pl, &ps);

    RowPartial st;
    gather_row<T, D, MASKED>(qrow, kb, vb, a.sk.t, a.sv.t, sp, i, a.pat, 0, sp.total(), pl, ps,
                     a.scale_log2, st);
    reduce_slots<D>(st);

    using G = GatherShape<D>;
    if (lane < G::LPK) {
        const float inv = 1.0f / st.l;
        float o[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) o[j] = st.acc[j] * inv;
        T* orow = static_cast<T*>(a.o) + bq * a.so.s + h * a.so.h + tok * a.so.t;
        Elem<T>::store8(orow + lane * 8, o);
    }
    if (a.lse && lane == 0) a.lse[goff] = (st.m + __log2f(st.l)) * PIATTN_LN2;
}

template <typename T, int D>
hipError_t launch_t(const FwdArgs& a, hipStream_t stream) {
    dim3 grid((a.n + 3) / 4, a.H, a.B);
    auto kern = a.pat.masked ? fwd_gather_kernel<T, D, true> : fwd_gather_kernel<T, D, false>;
    hipLaunchKernelGGL(kern, grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_gather(int dtype, const FwdArgs& a, hipStream_t stream) {
    if (dtype == 0) {
        switch (a.d) {
            case 32: return launch_t<float, 32>(a, stream);
            case 64: return launch_t<float, 64>(a, stream);
            case 128: return launch_t<float, 128>(a, stream);
        }
    } else {
        switch (a.d) {
            case 32: return launch_t<uint16_t, 32>(a, stream);
            case 64: return launch_t<uint16_t, 64>(a, stream);
            case 128: return launch_t<uint16_t, 128>(a, stream);
        }
    }
    return hipErrorInvalidValue;
}
