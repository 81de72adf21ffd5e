// mfma_util.hpp -- small gfx950 helpers shared by the MFMA prefill kernels:
// bf16 vector types, hardware bf16 packing, 4-lane reductions with
// v_permlane16/32_swap, the transposing LDS read and the XOR swizzle of the
// [rows][D] LDS tiles.
#pragma once

#include "common.hpp"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;


constexpr int NW = 8;          // waves per workgroup
constexpr int NT = NW * 64;    // threads per workgroup
constexpr float LAZY = 8.0f;   // lazy-rescale threshold (log2 units)

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ short bf16_short(float f) { return (short)f32_to_bf16_bits(f); }

__device__ __forceinline__ float bf16_round(float f) {
    return __uint_as_float(f32_to_bf16_bits(f) << 16);
}

// Sum / max over the four lanes {x, x+16, x+32, x+48} of a query.
__device__ __forceinline__ float sum4(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// Maximum that propagates NaN (v_maximum3_f32 on gfx950: no input
// canonicalisation, unlike fmaxf).
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ float max4(float v) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmax_ieee(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmax_ieee(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// bf16 dot product of 8 element pairs, accumulated in fp32.
__device__ __forceinline__ float dot8(bf16x8_t a, bf16x8_t b, float c) {
    const uint4 ua = __builtin_bit_cast(uint4, a), ub = __builtin_bit_cast(uint4, b);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ua.x), __builtin_bit_cast(bf16x2_t, ub.x), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ua.y), __builtin_bit_cast(bf16x2_t, ub.y), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ua.z), __builtin_bit_cast(bf16x2_t, ub.z), c, false);
    c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, ua.w), __builtin_bit_cast(bf16x2_t, ub.w), c, false);
    return c;
}

// Element xr of a 4-vector without branches (two selects).
__device__ __forceinline__ float diag_pick(f32x4_t s4, int xr) {
    const float a = (xr & 1) ? s4[1] : s4[0];
    const float b = (xr & 1) ? s4[3] : s4[2];
    return (xr & 2) ? b : a;
}

// Two fp32 values to packed bf16 (hardware round to nearest even).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Transposing LDS read (ds_read_b64_tr_b16) of the 8 bytes at p.
__device__ __forceinline__ s16x4_t ld_tr16(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
}

// Element offset of 16-byte chunk c of row r in a swizzled [rows][D] tile.
template <int D>
__device__ __forceinline__ int swz(int r, int c) {
    return r * D + ((c ^ (r & 7)) << 3);
}

// LDS byte address of a pointer into a __shared__ array: the low 32 bits of
// its flat address (the shared aperture sits in the high half).  A cast to
// the LDS address space would add a null check (a compare and a select per
// address; -O1 builds even lower it to a compare the gfx950 backend rejects).
__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }

// Workgroup barrier for LDS traffic only: waits for this wave's LDS
// operations, not for its loads in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// the wave are outstanding (loads complete in order), other counters free.
constexpr int vm_wait_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// LDS-direct 16-byte loads issued through inline assembly: lane l's 16 bytes
// at sbase + voff land at LDS byte address lds + 16*l.  The compiler does not
// see these loads, so it adds no (pipeline-draining) waits for them: the
// caller waits with vm_wait_imm before reading the data, and no compiler-
// visible load may be consumed while they are in flight unless an explicit
// wait covers them.  sbase must be wave-uniform.
//
// The compiler's hazard recognizer does not look inside the asm, so the
// block supplies the wait states the ISA requires before the load: a VMEM
// instruction that reads an SGPR written by a VALU instruction
// (v_readfirstlane, or v_readlane restoring a spilled SGPR) needs 5, and an
// LDS-DMA load after an SALU write of M0 needs 1.  s_nop 4 gives 5; without
// it the load can use the SGPR's previous value as its base address.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
    const uint64_t v = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo);
}
// NT: with the non-temporal hint, for rows nothing in the kernel reads again.
template <bool NT = false>
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t lds) {
    if constexpr (NT)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" : : "v"(voff), "s"(uniform_ptr(sbase)),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
    else
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(uniform_ptr(sbase)),
                     "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// 16-byte store with the non-temporal hint (global_store_dwordx4 ... nt),
// for rows nothing in the kernel reads again.
__device__ __forceinline__ void store_nt16(void* p, uint4 v) {
    __builtin_nontemporal_store(__builtin_bit_cast(u32x4_t, v), static_cast<u32x4_t*>(p));
}

// 4-byte LDS-direct load of each active lane (lane l writes lds + 4 l);
// wait states as for dma16.
__device__ __forceinline__ void dma4(const void* sbase, uint32_t voff, uint32_t lds) {
    asm volatile("s_nop 4\n\tglobal_load_lds_dword %0, %1" : : "v"(voff), "s"(uniform_ptr(sbase)),
                 "{m0}"(__builtin_amdgcn_readfirstlane(lds)) : "memory");
}

// Element offset of 16-byte chunk c of row r of a row-major [rows][D] tile
// whose chunks are XOR-swizzled by r % 8.
template <int D>
__device__ __forceinline__ int swr(int r, int c) { return r * D + ((c ^ (r & 7)) << 3); }

// Tile order.  Workgroup hw runs on XCD hw % 8 as that XCD's (hw / 8)-th.
// Logical tiles are dealt to the XCDs in runs of XG consecutive tiles, run
// r to XCD r % 8: neighbouring tiles (which share halo rows) share an L2,
// and the runs of long and short sequences spread over all XCDs.  With
// runs of 32 the window pass's halo rows come from L2 (its HBM reads fall
// to q, k, v, the partial and the records once each); with runs of 16 about
// 70% of them were fetched again.
constexpr int32_t XG = 32;
__device__ __forceinline__ int32_t xcd_logical(int32_t hw, int32_t total) {
    const int32_t xcd = hw % 8, loc = hw / 8;
    const int32_t logical = ((loc / XG) * 8 + xcd) * XG + loc % XG;
    // the last, partial round of runs: fall back to the plain order so that
    // every logical tile below total is produced exactly once
    const int32_t full = total / (8 * XG) * (8 * XG);
    return hw < full ? logical : hw;
}
