// proj.hip -- the linear maps around pi-Attention (gfx950): the gate logits
// in front of the kernel and the output projection behind it.
//
// The pages give the gate as a learnable shallow MLP that sets alpha from
// the input (gist.science section 2 "Methodology", item "Dynamic Adaptive
// Fusion") and end the pipeline with a fusion-and-projection stage (section
// 2 "Execution & Scheduling", "Streaming Stages").  The plainest form is
// taken: one linear layer per head for the gate logit, and the usual output
// projection of the concatenated heads.
//
//   gate:      g[b, h, i] = <x[b, i, :], Wg[h, :]> + bg[h]        (fp32 out)
//   out-proj:  y[b, i, :] = sum_{h, c} o[b, h, i, c] Wo[:, h d + c] + bo
//
// bf16 runs on v_mfma_f32_16x16x32_bf16.  The gate is a skinny contraction
// (N = H heads, K = Dm) bound by reading x once: each wave takes 16 tokens,
// its A operand straight from the x rows, its B operand (the gate weights)
// from L2.  The output projection is a GEMM over M = tokens, N = Dout,
// K = H d with the head concatenation folded into the A operand's addresses
// (o stays in the attention's [B, H, n, d] layout, any strides): 256 x 256
// or 320 x 256 tiles, K in chunks of 32 (always inside one head), a ring of
// five or four LDS slots filled ahead by LDS-direct loads, XOR-swizzled rows so
// that the MFMA operand reads are free of bank conflicts, two groups of four
// waves that alternate between reading a chunk's operands and running its
// MFMAs, and an epilogue that turns the accumulators into whole bf16 rows
// through LDS.  fp32 inputs take plain per-element kernels.
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace {

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }
__device__ __forceinline__ void store_as(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_as(uint16_t* p, float v) { *p = (uint16_t)(cvt_pk_bf16(v, 0.0f) & 0xffffu); }

// ------------------------------------------------------------------ gate (bf16)
// One wave per MB blocks of 16 tokens, NB = ceil(H / 16) column blocks of
// heads.  The gate weights (B operand) are read once per k-chunk for all MB
// token blocks, so larger MB cuts their re-reads per token.
template <int NB, int MB>
__global__ __launch_bounds__(256) void gate_mfma_kernel(GateArgs a) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, x = lane & 15, g = lane >> 4;
    const int64_t t0 = ((int64_t)blockIdx.x * 4 + wave) * 16 * MB;   // first token of the wave (flat b * n + i)
    const int64_t T = (int64_t)a.B * a.n;
    if (t0 >= T) return;
    const uint16_t* xr[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
        const int64_t tl = t0 + 16 * mb + x < T ? t0 + 16 * mb + x : T - 1;   // the lane's A row (clamped)
        const int64_t bl = tl / a.n, il = tl % a.n;
        xr[mb] = static_cast<const uint16_t*>(a.x) + bl * a.sx_b + il * a.sx_t;
    }
    const uint16_t* wr[NB];
#pragma unroll
    for (int cb = 0; cb < NB; ++cb)
        wr[cb] = static_cast<const uint16_t*>(a.w) + (int64_t)imin32(16 * cb + x, a.H - 1) * a.Dm;
    f32x4_t acc[MB][NB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) acc[mb][cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    // four k-chunks of 32 per step: 4 MB independent A loads and 4 NB B loads in flight
    int32_t k0 = 0;
    for (; k0 + 128 <= a.Dm; k0 += 128) {
        bf16x8_t av[4][MB], bv[4][NB];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) av[u][mb] = *reinterpret_cast<const bf16x8_t*>(xr[mb] + k0 + 32 * u + 8 * g);
#pragma unroll
            for (int cb = 0; cb < NB; ++cb)
                bv[u][cb] = *reinterpret_cast<const bf16x8_t*>(wr[cb] + k0 + 32 * u + 8 * g);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int mb = 0; mb < MB; ++mb)
#pragma unroll
                for (int cb = 0; cb < NB; ++cb)
                    acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][mb], bv[u][cb], acc[mb][cb], 0, 0, 0);
    }
    for (; k0 < a.Dm; k0 += 32) {                                  // Dm % 128 chunks of 32
#pragma unroll
        for (int cb = 0; cb < NB; ++cb) {
            const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(wr[cb] + k0 + 8 * g);
#pragma unroll
            for (int mb = 0; mb < MB; ++mb) {
                const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(xr[mb] + k0 + 8 * g);
                acc[mb][cb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[mb][cb], 0, 0, 0);
            }
        }
    }
    // lane (x, g) holds tokens t0 + 16 mb + 4g + r of head 16 cb + x
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
        const int32_t h = 16 * cb + x;
        if (h >= a.H) continue;
        const float bias = a.bias ? a.bias[h] : 0.0f;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t t = t0 + 16 * mb + 4 * g + r;
                if (t >= T) continue;
                const int64_t b = t / a.n, i = t % a.n;
                a.g[b * a.sg_b + h * a.sg_h + i * a.sg_t] = acc[mb][cb][r] + bias;
            }
    }
}

// ------------------------------------------------------------------ gate (fp32)
__global__ __launch_bounds__(256) void gate_f32_kernel(GateArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;     // (token, head)
    const int64_t T = (int64_t)a.B * a.n;
    if (e >= T * a.H) return;
    const int64_t t = e / a.H;
    const int32_t h = (int32_t)(e % a.H);
    const int64_t b = t / a.n, i = t % a.n;
    const float* xr = static_cast<const float*>(a.x) + b * a.sx_b + i * a.sx_t;
    const float* wr = static_cast<const float*>(a.w) + (int64_t)h * a.Dm;
    float s = 0.0f;
    for (int32_t k = 0; k < a.Dm; ++k) s = fmaf(xr[k], wr[k], s);
    a.g[b * a.sg_b + h * a.sg_h + i * a.sg_t] = s + (a.bias ? a.bias[h] : 0.0f);
}

// ------------------------------------------------------------ output projection
constexpr int PN = 256, PK = 32;             // tile columns (outputs), k-chunk
constexpr int PW = 8;                        // waves per workgroup (two per SIMD)
// WB 16-row blocks per wave: TM = 64 WB tile rows (tokens); the ring slot
// holds TM A rows and PN W rows; as many slots as fit 160 KB
template <int WB>
struct ProjTile {
    static constexpr int TM = 64 * WB;
    static constexpr int SLOT = (TM + PN) * PK;
    static constexpr int SLOTS = (160 * 1024) / (SLOT * 2);
};

// Element offset of 16-byte chunk c (of 4) of row r in a [rows][32] bf16
// tile, XOR-swizzled by (r / 2) % 4: the 16 rows x 4 chunks of an MFMA
// operand read then fall on distinct banks.
__device__ __forceinline__ int psw(int r, int c) { return r * PK + ((c ^ ((r >> 1) & 3)) << 3); }

// TM x 256 tile (TM = 256 or 320), eight waves of 16 WB x 128 (WB x 8 MFMA
// blocks, WB = 4 or 5), two per SIMD: per k-chunk a wave reads WB + 8
// operand rows of 16 bytes for 8 WB MFMAs.  A wave's LDS reads arrive at
// about 20 bytes a clock, so its 12 KB (WB = 4) take a little longer than
// its 32 MFMAs; WB = 5 brings the two closer.  The two waves of a SIMD work
// in opposite phases: waves 0-3 run the MFMAs of chunk s while waves 4-7
// read the operands of chunk s into registers, then they swap at a barrier,
// so each SIMD's matrix unit is fed by one wave while the LDS serves the
// other (a wave's own reads in flight slow its MFMA issue, the other
// wave's do not).
// Tile order: groups of GM row tiles, rows fastest inside a group, so that
// each XCD's run of 32 consecutive tiles is about 8 row tiles x 4 column
// tiles sharing their A and W slabs in that XCD's L2.
constexpr int32_t GM = 8;

template <int WB>
__global__ __launch_bounds__(PW * 64, 1) void out_proj_mfma_kernel(ProjArgs a, int32_t mtiles, int32_t ntiles,
                                                                 int32_t total) {
    constexpr int TM = ProjTile<WB>::TM, PS = ProjTile<WB>::SLOTS, SLOT = ProjTile<WB>::SLOT;
    __shared__ __attribute__((aligned(16))) uint16_t ring[PS * SLOT];
    const int32_t logical = xcd_logical(blockIdx.x, total);
    const int32_t gsize = GM * ntiles, grp = logical / gsize, first = grp * GM;
    const int32_t gm = imin32(mtiles - first, GM), w_in = logical - grp * gsize;
    const int32_t mt = first + w_in % gm, nt = w_in / gm;
    const int64_t M = (int64_t)a.B * a.n;
    const int64_t m0 = (int64_t)mt * TM;
    const int32_t n0 = nt * PN;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, x = lane & 15, g = lane >> 4;
    const int32_t K = a.H * a.d;
    const int32_t nk = K / PK;

    // ---- staging.  One 1 KB load covers 16 rows x 64 bytes; lane l fills
    // row l / 4, physical chunk l % 4 = logical chunk (l % 4) ^ ((row / 2) % 4).
    // Waves 0-3 load the A rows (tokens), TM / 4 each, waves 4-7 the W rows
    // (outputs), 64 each.
    const bool isw = wave >= PW / 2;
    const int rbase = (wave & 3) * (isw ? 64 : TM / 4);
    uint32_t voff[WB];
#pragma unroll
    for (int j = 0; j < WB; ++j) {
        const int rr = rbase + 16 * j + lane / 4;                 // tile row of this lane's 16 bytes
        const int lc = (lane % 4) ^ ((rr >> 1) & 3);
        if (!isw) {
            int64_t t = m0 + rr;
            t = t < M ? t : M - 1;
            const int64_t b = t / a.n, i = t % a.n;
            voff[j] = (uint32_t)((b * a.so_b + i * a.so_t + 8 * lc) * 2);
        } else {
            const int32_t nn = imin32(n0 + rr, a.Dout - 1);
            voff[j] = (uint32_t)(((int64_t)nn * a.ldw + 8 * lc) * 2);
        }
    }
    // stages are issued in order: the source of the next one advances by a
    // k-chunk, for A to the next head's column 0 after a head's last chunk;
    // past the last stage the last one is reloaded (harmless, keeps the
    // per-stage load count and so the waits uniform)
    const uint16_t* src = isw ? static_cast<const uint16_t*>(a.w) : static_cast<const uint16_t*>(a.o);
    int32_t next = 0, kcol = 0;
    auto issue = [&](uint16_t* slot) __attribute__((always_inline)) {
        uint16_t* dst = slot + (isw ? TM * PK : 0) + rbase * PK;
#pragma unroll
        for (int j = 0; j < WB; ++j)
            if (!isw || j < 4) dma16(src, voff[j], lds_addr(dst + 16 * j * PK));
        if (next < nk - 1) {
            ++next;
            kcol += PK;
            if (!isw && kcol == a.d) {
                kcol = 0;
                src += a.so_h - (a.d - PK);
            } else {
                src += PK;
            }
        }
    };

    f32x4_t acc[WB][8];
#pragma unroll
    for (int i = 0; i < WB; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const int wm = (wave >> 1) * 16 * WB, wn = (wave & 1) * 128;  // the wave's 16 WB x 128 sub-tile

    // Phases, one barrier after each: waves 0-3 (group 0) take the read
    // phase of chunk s in phase 2s and its MFMAs in phase 2s+1; waves 4-7
    // (group 1) one phase later.  The read phase of chunk s also issues the
    // wave's loads of stage s+PS-1 into the slot of chunk s-1, which both
    // groups finished reading by phase 2s-1.  Stage c must have landed for
    // every wave before phase 2c: each wave waits for its own share at the
    // end of phase 2c-1 (group 0 after the MFMAs of c-1, group 1 after
    // reading c-1), when the stages after c that it has issued are
    // c+1..c+PS-2.
    const int group = wave >> 2;
    auto bar = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        lds_barrier();
        __builtin_amdgcn_sched_barrier(0);
    };
    bf16x8_t av[WB], bv[8];
    // a wave's loads per stage: WB (A rows) or 4 (W rows); the waits below
    // leave the wave's PS - 2 newest stages in flight
    auto wait_own = [&]() __attribute__((always_inline)) {
        if (isw) __builtin_amdgcn_s_waitcnt(vm_wait_imm(4 * (PS - 2)));
        else __builtin_amdgcn_s_waitcnt(vm_wait_imm(WB * (PS - 2)));
    };
#pragma unroll
    for (int j = 0; j < PS - 1; ++j) issue(ring + j * SLOT);
    wait_own();                                                    // own stage 0
    bar();
    if (group == 1) bar();
    for (int32_t s = 0; s < nk; ++s) {
        const uint16_t* slot = ring + (s % PS) * SLOT;
#pragma unroll
        for (int j = 0; j < 8; ++j) bv[j] = *reinterpret_cast<const bf16x8_t*>(slot + TM * PK + psw(wn + 16 * j + x, g));
#pragma unroll
        for (int i = 0; i < WB; ++i) av[i] = *reinterpret_cast<const bf16x8_t*>(slot + psw(wm + 16 * i + x, g));
        issue(ring + ((s + PS - 1) % PS) * SLOT);
        if (group == 1) wait_own();
        bar();
#pragma unroll
        for (int i = 0; i < WB; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[i], bv[j], acc[i][j], 0, 0, 0);
        if (group == 0) wait_own();
        bar();
    }
    if (group == 0) bar();                                         // as many barriers as group 1
    __builtin_amdgcn_s_waitcnt(vm_wait_imm(0));                   // the trailing reloads land
    lds_barrier();                                                 // every wave done with the ring

    // ---- epilogue: bias, bf16, and whole rows through LDS, in two halves of
    // 32 rows per wave ([32 rows][128 columns] = 8 KB, 16-byte chunks
    // swizzled by row % 16)
    uint16_t* tile = ring + wave * 32 * 128;
    uint16_t* yb = static_cast<uint16_t*>(a.y);
    float bias[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int32_t col = n0 + wn + 16 * j + x;
        bias[j] = (a.bias && col < a.Dout) ? a.bias[col] : 0.0f;
    }
#pragma unroll
    for (int half = 0; half < (WB + 1) / 2; ++half) {
        const int nb = 2 * half + 1 < WB ? 2 : 1;                 // 16-row blocks in this pass
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (2 * half + i >= WB) break;
#pragma unroll
            for (int j = 0; j < 8; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int rr = 16 * i + 4 * g + r, cc = 16 * j + x;
                    tile[rr * 128 + ((((cc >> 3) ^ (rr & 15)) << 3) | (cc & 7))] =
                        (uint16_t)(cvt_pk_bf16(acc[2 * half + i][j][r] + bias[j], 0.0f) & 0xffffu);
                }
        }
        lds_barrier();
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            if (q >= 4 * nb) break;
            const int rr = 4 * q + lane / 16, ch = lane % 16;      // 4 rows x 16 chunks per instruction
            const int64_t t = m0 + wm + 32 * half + rr;
            const int32_t col = n0 + wn + 8 * ch;
            if (t >= M || col >= a.Dout) continue;
            const uint4 v = *reinterpret_cast<const uint4*>(tile + rr * 128 + ((ch ^ (rr & 15)) << 3));
            const int64_t b = t / a.n, i = t % a.n;
            uint16_t* dst = yb + b * a.sy_b + i * a.sy_t + col;
            if (col + 8 <= a.Dout) {
                *reinterpret_cast<uint4*>(dst) = v;
            } else {
                const uint16_t* e = reinterpret_cast<const uint16_t*>(&v);
                for (int c = 0; c < a.Dout - col; ++c) dst[c] = e[c];
            }
        }
        lds_barrier();                                             // the tile is rewritten next half
    }
}

// fp32 (and a fallback for any shape): one thread per output element.
template <typename T>
__global__ __launch_bounds__(256) void out_proj_plain_kernel(ProjArgs a) {
    const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t M = (int64_t)a.B * a.n;
    if (e >= M * a.Dout) return;
    const int64_t t = e / a.Dout;
    const int32_t col = (int32_t)(e % a.Dout);
    const int64_t b = t / a.n, i = t % a.n;
    const T* ob = static_cast<const T*>(a.o) + b * a.so_b + i * a.so_t;
    const T* wr = static_cast<const T*>(a.w) + (int64_t)col * a.ldw;
    float s = 0.0f;
    for (int32_t h = 0; h < a.H; ++h)
        for (int32_t c = 0; c < a.d; ++c) s = fmaf(to_f32(ob[h * a.so_h + c]), to_f32(wr[h * a.d + c]), s);
    s += a.bias ? a.bias[col] : 0.0f;
    store_as(static_cast<T*>(a.y) + b * a.sy_b + i * a.sy_t + col, s);
}

}  // namespace

hipError_t launch_gate(int dtype, const GateArgs& a, hipStream_t stream) {
    const int64_t T = (int64_t)a.B * a.n;
    if (dtype == 1) {
        // token blocks per wave: the most that still leave 1024 waves (four
        // per CU); measured at the 8K and 128K layer shapes, 2 and 4 blocks
        // read x at 4.2 and 3.6 TB/s against 3.8 and 2.9 with one
        const int mbs = T >= 4 * 16 * 1024 ? 4 : T >= 2 * 16 * 1024 ? 2 : 1;
        const int64_t blocks = (T + 64 * mbs - 1) / (64 * mbs);
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        auto k = a.H <= 16 ? (mbs == 4 ? gate_mfma_kernel<1, 4> : mbs == 2 ? gate_mfma_kernel<1, 2> : gate_mfma_kernel<1, 1>)
                           : (mbs == 4 ? gate_mfma_kernel<2, 4> : mbs == 2 ? gate_mfma_kernel<2, 2> : gate_mfma_kernel<2, 1>);
        hipLaunchKernelGGL(k, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    } else {
        const int64_t blocks = (T * a.H + 255) / 256;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(gate_f32_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    }
    return hipGetLastError();
}

bool out_proj_mfma_ok(int dtype, const ProjArgs& a) {
    if (dtype != 1 || a.d % PK != 0) return false;
    // 32-bit byte offsets of the LDS-direct loads: any row of o from its base
    // plus a head's columns, any row of W
    const int64_t M = (int64_t)a.B * a.n;
    const int64_t orow = (int64_t)(a.B - 1) * a.so_b + (int64_t)(a.n - 1) * a.so_t + a.d;
    const int64_t wrow = (int64_t)(a.Dout - 1) * a.ldw + (int64_t)a.H * a.d;
    return M >= 1 && orow * 2 < ((int64_t)1 << 31) && wrow * 2 < ((int64_t)1 << 31);
}

hipError_t launch_out_proj(int dtype, const ProjArgs& a, hipStream_t stream) {
    const int64_t M = (int64_t)a.B * a.n;
    if (out_proj_mfma_ok(dtype, a)) {
        // 80-row waves (320-row tiles) when there are enough tiles for the
        // grid's last round not to matter: at M = 131072, N = K = 4096 3.54
        // against 3.68 ms; at M = 32768, N = K = 1024 (412 tiles against
        // 512) 0.096 against 0.087 ms
        const int64_t ntiles = ((int64_t)a.Dout + PN - 1) / PN;
        const int64_t mt5 = (M + ProjTile<5>::TM - 1) / ProjTile<5>::TM;
        if (mt5 * ntiles >= 2048) {
            const int64_t total = mt5 * ntiles;
            if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
            hipLaunchKernelGGL(out_proj_mfma_kernel<5>, dim3((uint32_t)total), dim3(PW * 64), 0, stream, a,
                               (int32_t)mt5, (int32_t)ntiles, (int32_t)total);
            return hipGetLastError();
        }
        const int64_t mtiles = (M + ProjTile<4>::TM - 1) / ProjTile<4>::TM;
        const int64_t total = mtiles * ntiles;
        if (total > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(out_proj_mfma_kernel<4>, dim3((uint32_t)total), dim3(PW * 64), 0, stream, a,
                           (int32_t)mtiles, (int32_t)ntiles, (int32_t)total);
        return hipGetLastError();
    }
    const int64_t blocks = (M * a.Dout + 255) / 256;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (dtype == 1)
        hipLaunchKernelGGL(out_proj_plain_kernel<uint16_t>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    else
        hipLaunchKernelGGL(out_proj_plain_kernel<float>, dim3((uint32_t)blocks), dim3(256), 0, stream, a);
    return hipGetLastError();
}
