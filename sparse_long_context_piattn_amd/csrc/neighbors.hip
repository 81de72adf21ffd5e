// neighbors.hip -- debug dump of the neighbour lists, one thread per query,
// written from the same RowSpan enumerator the compute kernels use.
#include "kernels.hpp"

namespace {

__global__ __launch_bounds__(256) void neighbors_kernel(int32_t n, PiPattern p, int32_t q_begin,
                                                        int32_t q_count, int32_t cap,
                                                        int32_t* __restrict__ idx,
                                                        int8_t* __restrict__ kind,
                                                        int32_t* __restrict__ count) {
    const int32_t r = blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= q_count) return;
    const int32_t i = q_begin + r;
    const RowSpan sp = row_span(i, n, p);
    const int32_t tot = sp.total();
    int32_t* ir = idx + (int64_t)r * cap;
    int8_t* kr = kind + (int64_t)r * cap;
    for (int32_t u = 0; u < cap; ++u) {
        if (u < tot) {
            bool loc;
            ir[u] = span_key(sp, i, p, u, &loc);
            kr[u] = loc ? 1 : 2;
        } else {
            ir[u] = -1;
            kr[u] = 0;
        }
    }
    count[r] = tot;
}

}  // namespace

hipError_t launch_neighbors(int32_t n, const PiPattern& p, int32_t q_begin, int32_t q_count,
                            int32_t cap, int32_t* idx, int8_t* kind, int32_t* count,
                            hipStream_t stream) {
    dim3 grid((q_count + 255) / 256);
    hipLaunchKernelGGL(neighbors_kernel, grid, dim3(256), 0, stream, n, p, q_begin, q_count, cap,
                       idx, kind, count);
    return hipGetLastError();
}
