// gather.hpp -- per-row gather attention on one wavefront (gfx950, wave64).
//
// A wave owns one query row.  Its 64 lanes form NS = 512/D key slots of
// LPK = D/8 lanes each; a lane holds 8 consecutive head-dimension elements
// of the query, of the slot's key and value, and of the running output.
// Keys are taken NS at a time from the row's union (RowSpan order); each
// slot reduces its dot product over its LPK lanes, the chunk maximum is
// reduced over the slots, and one online softmax (running max m in log2
// units, shared by the wave; per-lane partial sum l and accumulator) absorbs
// local and skip keys alike, the gate prior being added to each logit
// according to the key's kind (pi-Attention "Dynamic Adaptive Fusion":
// log(alpha) on local logits, log(1 - alpha) on skip logits, one softmax).
//
// This path serves fp32 and d = 32 prefill (the MFMA kernels take bf16 with
// d = 64 or 128), and is the building block of split-K decode.
#pragma once

#include "common.hpp"

template <typename T>
struct Elem;

typedef unsigned int gather_u32x4 __attribute__((ext_vector_type(4)));

// 16 bytes at p, with the non-temporal hint when NT (rows read once).
template <bool NT>
__device__ __forceinline__ uint4 load16(const void* p) {
    if constexpr (NT)
        return __builtin_bit_cast(uint4, __builtin_nontemporal_load(static_cast<const gather_u32x4*>(p)));
    else
        return *static_cast<const uint4*>(p);
}

template <>
struct Elem<float> {
    template <bool NT = false>
    static __device__ __forceinline__ void load8(const float* p, float x[8]) {
        const uint4 a = load16<NT>(p);
        const uint4 b = load16<NT>(p + 4);
        x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y); x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
        x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y); x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    }
    static __device__ __forceinline__ void store8(float* p, const float x[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
    }
};

// bf16 is carried as its raw 16-bit pattern.
template <>
struct Elem<uint16_t> {
    template <bool NT = false>
    static __device__ __forceinline__ void load8(const uint16_t* p, float x[8]) {
        const uint4 w = load16<NT>(p);
        x[0] = bf16lo(w.x); x[1] = bf16hi(w.x); x[2] = bf16lo(w.y); x[3] = bf16hi(w.y);
        x[4] = bf16lo(w.z); x[5] = bf16hi(w.z); x[6] = bf16lo(w.w); x[7] = bf16hi(w.w);
    }
    static __device__ __forceinline__ void store8(uint16_t* p, const float x[8]) {
        uint4 w;
        w.x = pack_bf16x2(x[0], x[1]);
        w.y = pack_bf16x2(x[2], x[3]);
        w.z = pack_bf16x2(x[4], x[5]);
        w.w = pack_bf16x2(x[6], x[7]);
        *reinterpret_cast<uint4*>(p) = w;
    }
};

template <int D>
struct GatherShape {
    static_assert(D == 32 || D == 64 || D == 128, "head dim");
    static constexpr int LPK = D / 8;   // lanes per key
    static constexpr int NS = 64 / LPK; // key slots per wave
};

// Online-softmax partial state of one wave over a range of union positions.
struct RowPartial {
    float m;       // running max (log2 units), wave-uniform
    float l;       // sum of exp2(s - m) over this lane's slot
    float acc[8];  // sum of exp2(s - m) * v over this lane's slot
};

// Process union positions [u0, u1) of row i.  kbase/vbase point at token 0
// of the row's (sequence, head); k_tok_stride / v_tok_stride are the token
// strides of the key and value tensors.  ring > 0: key position j lives in
// row j mod ring (a rolling cache); 0: in row j.  NT: the key and value
// rows are loaded with the non-temporal hint (decode reads each once).
template <typename T, int D, bool MASKED, bool NT = false>
__device__ __forceinline__ void gather_row(const T* __restrict__ qrow, const T* __restrict__ kbase,
                                           const T* __restrict__ vbase, int64_t k_tok_stride,
                                           int64_t v_tok_stride,
                                           const RowSpan& sp, int32_t i, const PiPattern& pat, int32_t u0,
                                           int32_t u1, float pl, float ps, float scale_log2,
                                           RowPartial& st, int32_t ring = 0) {
    using G = GatherShape<D>;
    const int lane = threadIdx.x & 63;
    const int slot = lane / G::LPK;
    const int c = (lane % G::LPK) * 8;
    float qv[8];
    Elem<T>::load8(qrow + c, qv);
#pragma unroll
    for (int j = 0; j < 8; ++j) qv[j] *= scale_log2;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) st.acc[j] = 0.0f;

    const int32_t ri = ring > 0 ? i % ring : 0;          // row of position i in a rolling cache
    for (int32_t base = u0; base < u1; base += G::NS) {
        const int32_t u = base + slot;
        const bool valid = u < u1;
        float kv[8], vv[8];
        float prior = 0.0f;
        if (valid) {
            bool loc;
            int32_t key = span_key_t<MASKED>(sp, i, pat, u, &loc);
            if (ring > 0) {                               // key >= i - ring + 1: row (i - delta) mod ring
                const int32_t r = ri - (i - key);
                key = r < 0 ? r + ring : r;
            }
            Elem<T>::template load8<NT>(kbase + (int64_t)key * k_tok_stride + c, kv);
            Elem<T>::template load8<NT>(vbase + (int64_t)key * v_tok_stride + c, vv);
            prior = loc ? pl : ps;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) kv[j] = vv[j] = 0.0f;
        }
        float dot = 0.0f;
#pragma unroll
        for (int j = 0; j < 8; ++j) dot = fmaf(qv[j], kv[j], dot);
#pragma unroll
        for (int off = 1; off < G::LPK; off <<= 1) dot += __shfl_xor(dot, off, 64);
        const float s = valid ? dot + prior : -INFINITY;
        float cmax = s;
#pragma unroll
        for (int off = G::LPK; off < 64; off <<= 1) cmax = fmaxf(cmax, __shfl_xor(cmax, off, 64));
        const float mnew = fmaxf(st.m, cmax);
        const float mu = (mnew == -INFINITY) ? 0.0f : mnew;
        const float fac = exp2_fast(st.m - mu);
        const float p = exp2_fast(s - mu);
        st.l = fmaf(st.l, fac, p);
#pragma unroll
        for (int j = 0; j < 8; ++j) st.acc[j] = fmaf(st.acc[j], fac, p * vv[j]);
        st.m = mnew;
    }
}

// Sum l and acc over the key slots; afterwards every lane holds the wave's
// totals for its 8 head-dimension elements.
template <int D>
__device__ __forceinline__ void reduce_slots(RowPartial& st) {
    using G = GatherShape<D>;
#pragma unroll
    for (int off = G::LPK; off < 64; off <<= 1) {
        st.l += __shfl_xor(st.l, off, 64);
#pragma unroll
        for (int j = 0; j < 8; ++j) st.acc[j] += __shfl_xor(st.acc[j], off, 64);
    }
}
