// kernels.hpp -- launchers exported by the kernel translation units to the
// host dispatch in api.cpp.  Each returns hipGetLastError() after launching.
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

// dtype: 0 = fp32, 1 = bf16 (same values as piattn_dtype).
hipError_t launch_fwd_gather(int dtype, const FwdArgs& a, hipStream_t stream);
hipError_t launch_decode(int dtype, const DecodeArgs& a, hipStream_t stream);
hipError_t launch_neighbors(int32_t n, const PiPattern& p, int32_t q_begin, int32_t q_count,
                            int32_t cap, int32_t* idx, int8_t* kind, int32_t* count,
                            hipStream_t stream);
