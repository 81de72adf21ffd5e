// kernels.hpp -- launchers exported by the kernel translation units to the
// host dispatch in api.cpp.  Each returns hipGetLastError() after launching.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

// dtype: 0 = fp32, 1 = bf16 (same values as piattn_dtype).
hipError_t launch_fwd_gather(int dtype, const FwdArgs& a, hipStream_t stream);
// Residue-layout single-kernel prefill for head dim 64 (window phase + dense
// skip band merged in LDS); selectable with PIATTN_FWD_KERNEL=resid.
bool fwd_resid_supported(int dtype, const FwdArgs& a);
hipError_t launch_fwd_resid(const FwdArgs& a, hipStream_t stream);
// Split prefill (bf16, d 64/128, any pi): skip pass in residue layout, then a
// window pass that merges the two partial softmaxes.
bool fwd_split_supported(int dtype, const FwdArgs& a);
// fp32 prefill on fp32 MFMA (d 32/64/128): 16 query rows per wave, the
// union's 16-key blocks in key order.
bool fwd_f32mfma_supported(int dtype, const FwdArgs& a);
bool fwd_f32mfma_preferred(const FwdArgs& a);   // cost model against the gather kernel
hipError_t launch_fwd_f32mfma(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_split(const FwdArgs& a, float* ws, hipStream_t stream);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_cache_append(int dtype, const AppendArgs& a, hipStream_t stream);
// Backward of the prefill (gather path, any supported dtype and d; the
// rows' log-sum-exp recomputed).
hipError_t launch_bwd(int dtype, const BwdArgs& a, hipStream_t stream);
// Backward on MFMA (bf16, d 64/128, the forward's log-sum-exp given): skip
// pass in residue layout, then the window pass.
bool bwd_band_supported(int dtype, const BwdArgs& a);
hipError_t launch_bwd_band(const BwdArgs& a, hipStream_t stream);
// Gate logits and output projection around the attention (bf16 on MFMA).
hipError_t launch_gate(int dtype, const GateArgs& a, hipStream_t stream);
bool out_proj_mfma_ok(int dtype, const ProjArgs& a);
hipError_t launch_out_proj(int dtype, const ProjArgs& a, hipStream_t stream);
hipError_t launch_neighbors(int32_t n, const PiPattern& p, int32_t q_begin, int32_t q_count,
                            int32_t cap, int32_t* idx, int8_t* kind, int32_t* count,
                            hipStream_t stream);
