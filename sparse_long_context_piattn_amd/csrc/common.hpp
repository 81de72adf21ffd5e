// common.hpp -- argument blocks and small device helpers shared by the
// libpiattn kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pattern.hpp"

#define PIATTN_LOG2E 1.4426950408889634f
#define PIATTN_LN2 0.6931471805599453f

// Strides of one tensor, in elements: sequence, head, token.
struct Str3 {
    int64_t s, h, t;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    void* o;
    float* lse;
    Str3 sq, sk, sv, so, sg;
    const int32_t* cu;   // varlen offsets or nullptr
    int32_t B, H, n, d;
    PiPattern pat;
    float scale_log2;    // logit scale * log2(e)
};

// Backward of the prefill: the forward's arguments (o = its output), plus the
// incoming gradient and the gradients written.  dq, dk, dv use the strides of
// q, k, v; dout those of o; dg those of g.
struct BwdArgs {
    FwdArgs f;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* dg;
    float* rowstat;      // workspace: 16 bytes per row, [B][H][n]
    const float* lse_in; // the forward's log-sum-exp (natural log, layout of g), or null
    float scale;         // logit scale (natural units)
};

// Gate logits g[b, h, i] = <x[b, i, :], w[h, :]> + bias[h] (strides in elements;
// the last dim of x contiguous, w row-major [H][Dm]).
struct GateArgs {
    const void* x;
    int64_t sx_b, sx_t;
    const void* w;
    const float* bias;   // [H] or null
    float* g;
    int64_t sg_b, sg_h, sg_t;
    int32_t B, n, H, Dm;
};

// Output projection y[b, i, :] = sum_{h,c} o[b, h, i, c] w[:, h d + c] + bias.
struct ProjArgs {
    const void* o;
    int64_t so_b, so_h, so_t;
    const void* w;       // [Dout] rows of ldw elements, columns h d + c
    int64_t ldw;
    const float* bias;   // [Dout] or null
    void* y;
    int64_t sy_b, sy_t;
    int32_t B, n, H, d, Dout;
};

// Appends one token's key and value per (sequence, head) to a rolling cache.
struct AppendArgs {
    const void* kn;
    const void* vn;
    void* kc;
    void* vc;
    const int32_t* pos;  // position of the new token per sequence; < 0: skipped
    Str3 skn, svn, skc, svc;
    int32_t S, H, d, slots;
};

struct DecodeArgs {
    const void* q;
    const void* kc;
    const void* vc;
    const int32_t* lens;
    const float* g;
    void* o;
    float* ws;           // partials [S*H][splits][d + 2] when splits > 1
    Str3 sq, sk, sv, so, sg;
    int32_t S, H, d, cap;
    int32_t ring;        // 0: position j in cache row j; else rolling cache, row j mod ring (= cap)
    int32_t splits;
    int32_t chunk;       // union positions per split
    PiPattern pat;
    float scale_log2;
};

// Sequence b of a varlen batch: its first packed token and its length,
// clamped into [0, nmax].  Grids and per-row workspaces are sized for nmax
// rows per sequence, so a sequence longer than nmax is cut at nmax rows (its
// later rows are left unwritten) rather than indexed past those buffers.
__device__ __forceinline__ void varlen_seq(const int32_t* cu, int32_t b, int32_t nmax, int64_t* tok0,
                                           int32_t* n) {
    const int32_t c0 = cu[b], c1 = cu[b + 1];
    *tok0 = c0;
    const int32_t len = c1 - c0;
    *n = len < 0 ? 0 : (len > nmax ? nmax : len);
}

// ---------------------------------------------------------------- bf16

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 with round-to-nearest-even; NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- gate

// log2(sigmoid(x)) computed without overflow: -softplus(-x) / ln 2, with
// softplus(y) = max(y, 0) + log(1 + exp(-|y|)).  In log2 units:
// -max(-x, 0) * log2(e) - log2(1 + 2^(-|x| log2 e)); the second term is
// evaluated in fp32 (absolute error ~1e-7, below the logits' rounding).
__device__ __forceinline__ float log2_sigmoid(float x) {
    const float t = exp2_fast(-fabsf(x) * PIATTN_LOG2E);
    return -fmaxf(-x, 0.0f) * PIATTN_LOG2E - __log2f(1.0f + t);
}

// Priors in log2 units for a row: local gets log2(alpha), skip log2(1-alpha);
// both zero when the row has no skip keys.
__device__ __forceinline__ void gate_priors(float g, bool has_skip, float* pl, float* ps) {
    if (has_skip) {
        *pl = log2_sigmoid(g);
        *ps = log2_sigmoid(-g);
    } else {
        *pl = 0.0f;
        *ps = 0.0f;
    }
}

// ---------------------------------------------------------------- wave helpers

template <int MASK>
__device__ __forceinline__ float shfl_xor_f(float x) {
    return __shfl_xor(x, MASK, 64);
}


