// decode.hip -- one new query per (sequence, head) against a KV cache,
// split-K over the union of its window and skips.
//
// Grid (S*H, splits), 256 threads.  Workgroup (sh, sp) owns union positions
// [sp*chunk, (sp+1)*chunk) of row len-1; its four waves take consecutive
// quarters of that range with the per-row gather loop, merge their online-
// softmax states in LDS, and either write the normalised output (one split)
// or the partial (m, l, acc[d]) to the workspace, which a second kernel
// merges:  m = max_p m_p,  l = sum_p l_p 2^(m_p - m),  o = sum_p acc_p 2^(m_p - m) / l.
// The query position is len-1: the pages' inference mode, in which the new
// token's own key and value are appended before it attends.
#include "gather.hpp"
#include "kernels.hpp"

namespace {

template <typename T, int D, bool MASKED>
__global__ __launch_bounds__(256) void decode_split_kernel(DecodeArgs a) {
    using G = GatherShape<D>;
    __shared__ float sm_acc[4][D];
    __shared__ float sm_m[4], sm_l[4];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int32_t sh = blockIdx.x;
    const int32_t split = blockIdx.y;
    const int32_t s = sh / a.H, h = sh % a.H;
    const int32_t len = a.lens[s];
    const bool bad = len < 1 || (a.ring == 0 && len > a.cap);

    RowPartial st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] = 0.0f;

    if (!bad) {
        const int32_t i = len - 1;
        const RowSpan sp = row_span_t<MASKED>(i, len, a.pat);
        const int32_t U = sp.total();
        const int32_t u0 = imin32(U, split * a.chunk);
        const int32_t u1 = imin32(U, u0 + a.chunk);
        const int32_t quarter = (u1 - u0 + 3) / 4;
        const int32_t w0 = imin32(u1, u0 + wave * quarter);
        const int32_t w1 = imin32(u1, w0 + quarter);
        const T* qrow = static_cast<const T*>(a.q) + (int64_t)s * a.sq.s + (int64_t)h * a.sq.h;
        const T* kb = static_cast<const T*>(a.kc) + (int64_t)s * a.sk.s + (int64_t)h * a.sk.h;
        const T* vb = static_cast<const T*>(a.vc) + (int64_t)s * a.sv.s + (int64_t)h * a.sv.h;
        float pl, ps;
        gate_priors(a.g[(int64_t)s * a.sg.s + (int64_t)h * a.sg.h], sp.has_skip(), &pl, &ps);
        gather_row<T, D, MASKED, true>(qrow, kb, vb, a.sk.t, a.sv.t, sp, i, a.pat, w0, w1, pl, ps,
                         a.scale_log2, st, a.ring);
        reduce_slots<D>(st);
    }

    if (lane < G::LPK) {
#pragma unroll
        for (int j = 0; j < 8; ++j) sm_acc[wave][lane * 8 + j] = st.acc[j];
    }
    if (lane == 0) {
        sm_m[wave] = st.m;
        sm_l[wave] = st.l;
    }
    __syncthreads();

    // Merge the four waves; thread c < D owns head-dim element c.
    const int c = threadIdx.x;
    if (c < D) {
        float m = fmaxf(fmaxf(sm_m[0], sm_m[1]), fmaxf(sm_m[2], sm_m[3]));
        const float mu = (m == -INFINITY) ? 0.0f : m;
        float l = 0.0f, acc = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float f = exp2_fast(sm_m[w] - mu);
            l = fmaf(sm_l[w], f, l);
            acc = fmaf(sm_acc[w][c], f, acc);
        }
        if (a.splits == 1) {
            const float o = bad ? __int_as_float(0x7fc00000) : acc / l;
            T* orow = static_cast<T*>(a.o) + (int64_t)s * a.so.s + (int64_t)h * a.so.h;
            if constexpr (sizeof(T) == 4) {
                orow[c] = o;
            } else {
                orow[c] = (T)f32_to_bf16_bits(o);
            }
        } else {
            float* p = a.ws + ((int64_t)sh * a.splits + split) * (D + 2);
            p[2 + c] = acc;
            if (c == 0) {
                p[0] = m;
                p[1] = l;
            }
        }
    }
}

template <typename T, int D>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeArgs a) {
    const int32_t sh = blockIdx.x;
    const int32_t s = sh / a.H, h = sh % a.H;
    const int c = threadIdx.x;
    const int32_t len = a.lens[s];
    const bool bad = len < 1 || (a.ring == 0 && len > a.cap);
    const float* p = a.ws + (int64_t)sh * a.splits * (D + 2);
    float m = -INFINITY;
    for (int32_t sp = 0; sp < a.splits; ++sp) m = fmaxf(m, p[sp * (D + 2)]);
    const float mu = (m == -INFINITY) ? 0.0f : m;
    float l = 0.0f, acc = 0.0f;
    for (int32_t sp = 0; sp < a.splits; ++sp) {
        const float* q = p + sp * (D + 2);
        const float f = exp2_fast(q[0] - mu);
        l = fmaf(q[1], f, l);
        acc = fmaf(q[2 + c], f, acc);
    }
    const float o = bad ? __int_as_float(0x7fc00000) : acc / l;
    T* orow = static_cast<T*>(a.o) + (int64_t)s * a.so.s + (int64_t)h * a.so.h;
    if constexpr (sizeof(T) == 4) {
        orow[c] = o;
    } else {
        orow[c] = (T)f32_to_bf16_bits(o);
    }
}

template <typename T, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
    dim3 grid(a.S * a.H, a.splits);
    auto split = a.pat.masked ? decode_split_kernel<T, D, true> : decode_split_kernel<T, D, false>;
    hipLaunchKernelGGL(split, grid, dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.splits == 1) return e;
    hipLaunchKernelGGL((decode_combine_kernel<T, D>), dim3(a.S * a.H), dim3(D), 0, stream, a);
    return hipGetLastError();
}

// One (sequence, head) row per workgroup of 64 threads: the new key and
// value (d elements each) go to row pos mod slots of the rolling cache.
template <typename T, int D>
__global__ __launch_bounds__(64) void cache_append_kernel(AppendArgs a) {
    const int32_t sh = blockIdx.x;
    const int32_t s = sh / a.H, h = sh % a.H;
    const int32_t pos = a.pos[s];
    if (pos < 0) return;
    const int64_t row = pos % a.slots;
    const T* kn = static_cast<const T*>(a.kn) + (int64_t)s * a.skn.s + (int64_t)h * a.skn.h;
    const T* vn = static_cast<const T*>(a.vn) + (int64_t)s * a.svn.s + (int64_t)h * a.svn.h;
    T* kc = static_cast<T*>(a.kc) + (int64_t)s * a.skc.s + (int64_t)h * a.skc.h + row * a.skc.t;
    T* vc = static_cast<T*>(a.vc) + (int64_t)s * a.svc.s + (int64_t)h * a.svc.h + row * a.svc.t;
    for (int c = threadIdx.x; c < D; c += 64) {
        kc[c] = kn[c];
        vc[c] = vn[c];
    }
}

template <typename T>
hipError_t append_t(const AppendArgs& a, hipStream_t stream) {
    switch (a.d) {
        case 32: hipLaunchKernelGGL((cache_append_kernel<T, 32>), dim3(a.S * a.H), dim3(64), 0, stream, a); break;
        case 64: hipLaunchKernelGGL((cache_append_kernel<T, 64>), dim3(a.S * a.H), dim3(64), 0, stream, a); break;
        case 128: hipLaunchKernelGGL((cache_append_kernel<T, 128>), dim3(a.S * a.H), dim3(64), 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_cache_append(int dtype, const AppendArgs& a, hipStream_t stream) {
    return dtype == 0 ? append_t<float>(a, stream) : append_t<uint16_t>(a, stream);
}

hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream) {
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
