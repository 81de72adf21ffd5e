// api_internal.hpp -- host-side helpers of the C ABI shared between api.cpp
// and the entry points defined in other sources (noalloc.hip).
#pragma once

#include "piattn.h"

// Sets the thread's error string (piattn_last_error) and returns code.
int api_fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));

// piattn_fwd's argument checks alone (no launch): PIATTN_OK or the error.
int api_check_fwd(piattn_dtype dtype, int32_t B, int32_t H, int32_t n, int32_t d, const void* q, const void* k,
                  const void* v, const float* gate_logits, void* out, float* lse_out, const int64_t strides[5][3],
                  const int32_t* cu_seqlens, const piattn_pattern* pattern);
