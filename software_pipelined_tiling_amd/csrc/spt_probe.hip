// spt_probe.hip -- a measurement probe: the sustained MFMA rate of the chip
// with operands drawn from a caller's buffer and no memory traffic in the
// loop.  Under MI355X's board power limit the dense MFMA rate depends on the
// operand bits (their switching), so the attainable peak for a workload is
// measured with its own data; the GEMM's roofline fraction is read against
// the published peak and, as context, against this.
//
// One workgroup of 4 waves per CU (one wave per SIMD, the GEMM's layout):
// every wave loads 4 A-like and 4 B-like 16-byte fragments per lane from the
// buffer, then issues `iters` rounds of 64 independent 16x16 MFMAs into 64
// accumulators (the GEMM's 128 x 128 wave tile).  A checksum of the
// accumulators goes to `sink` so nothing is optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "spt_kernel.hpp"

namespace spt {

template <int DT>
__global__ __launch_bounds__(256) void mfma_probe_kernel(const i32x4_t* ops, int64_t n_vec, int64_t iters,
                                                         float* sink)
{
    typedef typename AccT<DT>::type acc_t;
    const int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x;
    i32x4_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = ops[(g * 8 + i) % n_vec];
        b[i] = ops[(g * 8 + 4 + i) % n_vec];
    }
    acc_t acc[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) acc[i] = (acc_t){0, 0, 0, 0};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 64; ++i) mma<DT>(acc[i], b[(i >> 2) & 3], a[i & 3]);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
        if constexpr (DT == DT_I8) {  // int32 sums held bit for bit in the float vector
            const i32x4_t v = __builtin_bit_cast(i32x4_t, acc[i]);
            s += (float)v[0] + (float)v[3];
        } else {
            s += acc[i][0] + acc[i][3];
        }
    }
    sink[g] = s;
}

hipError_t launch_mfma_probe(int dtype, const void* ops, int64_t n_vec, int64_t iters, float* sink,
                             hipStream_t stream)
{
    const i32x4_t* o = (const i32x4_t*)ops;
    void* args[] = {&o, &n_vec, &iters, &sink};
    const void* k = dtype == DT_F16    ? (const void*)&mfma_probe_kernel<DT_F16>
                    : dtype == DT_BF16 ? (const void*)&mfma_probe_kernel<DT_BF16>
                                       : (const void*)&mfma_probe_kernel<DT_I8>;
    return hipLaunchKernel(k, dim3(256), dim3(256), args, 0, stream);
}

}  // namespace spt
