// bench_probe.hip -- a measurement probe for bench.py, built as its own
// library (libspt_probe.so) and not part of libspt.so or its C ABI: the
// sustained MFMA rate of the chip with operands drawn from a caller's buffer
// and no memory traffic in the loop.  Under MI355X's board power limit the
// dense MFMA rate depends on the operand bits (their switching), so the
// attainable peak for a workload is measured with its own data; the GEMM's
// roofline fraction is read against the published peak and, as context,
// against this ("Kernel-Engpass analysieren", Schritt 1: the roofline's
// compute roof is the attainable peak).
//
// One workgroup of 4 waves per CU (one wave per SIMD, the GEMM's layout):
// every wave loads 4 A-like and 4 B-like 16-byte fragments per lane from the
// buffer, then issues `iters` rounds of 64 independent 16x16 MFMAs into 64
// accumulators (the GEMM's 128 x 128 wave tile), with the GEMM's own MFMA
// wrapper.  A checksum of the accumulators goes to `sink` so nothing is
// optimised away.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "software_pipelined_tiling_amd/csrc/spt_kernel.hpp"

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

}  // namespace spt

extern "C" {

// Launches one grid of 256 workgroups x 256 threads (one wave per SIMD on
// every CU); each lane takes 8 sixteen-byte fragments from `operands`
// (wrapping inside `operand_bytes`) and each wave issues `iters` rounds of 64
// independent 16x16 MFMAs (v_mfma_f32_16x16x32_f16 / _bf16 for dtype 0 / 1,
// v_mfma_i32_16x16x64_i8 for dtype 2): 256 * 4 * 64 * iters MFMAs of 16384
// (fp16/bf16) or 32768 (int8) operations.  `sink` receives 65536 floats of
// checksum.  Device pointers owned by the caller, `operands` 16-byte aligned;
// asynchronous on `stream`.  Returns 0, -1 (dtype other than 0..2, null
// pointer, fewer than 16 bytes, negative iters), -3 (misaligned operands) or
// -4 (launch failure); arguments are checked before any HIP call.
int spt_probe_mfma(int dtype, const void* operands, int64_t operand_bytes, int64_t iters, void* sink,
                   void* stream)
{
    using namespace spt;
    if (dtype != DT_F16 && dtype != DT_BF16 && dtype != DT_I8) return -1;
    if (!operands || !sink || operand_bytes < 16 || iters < 0) return -1;
    if ((uintptr_t)operands % 16) return -3;
    const i32x4_t* o = (const i32x4_t*)operands;
    int64_t n_vec = operand_bytes / 16;
    float* s = (float*)sink;
    void* args[] = {&o, &n_vec, &iters, &s};
    const void* k = dtype == DT_F16    ? (const void*)&mfma_probe_kernel<DT_F16>
                    : dtype == DT_BF16 ? (const void*)&mfma_probe_kernel<DT_BF16>
                                       : (const void*)&mfma_probe_kernel<DT_I8>;
    return hipLaunchKernel(k, dim3(256), dim3(256), args, 0, (hipStream_t)stream) == hipSuccess ? 0 : -4;
}

}  // extern "C"
