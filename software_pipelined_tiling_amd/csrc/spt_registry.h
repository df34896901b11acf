// spt_registry.h -- the built (dtype, B layout, tile, variant, stages)
// instantiations of the K-loop kernel and their launchers.
#pragma once

#include <hip/hip_runtime.h>

#include "spt_config.h"

namespace spt {

typedef hipError_t (*LaunchFn)(const GemmArgs&, unsigned grid, hipStream_t);

struct KernelEntry {
    int dtype, bcol, tile, variant, stages, exact;
    int window;  // V_PERSIST: K tiles over which a wave writes the previous output tile (else 0)
    int threads, lds_bytes, loads_per_tile;
    LaunchFn launch;
    const void* kernel;
};

struct KernelTable {
    const KernelEntry* entries;
    int count;
};

// One table per (element type, B layout), each in its own translation unit.
KernelTable kernels_f16_row();
KernelTable kernels_f16_col();
KernelTable kernels_bf16_row();
KernelTable kernels_bf16_col();
KernelTable kernels_i8_row();
KernelTable kernels_i8_col();
KernelTable kernels_f32_row();
KernelTable kernels_f32_col();

// The streaming pipeline y = 2 x (spt_stream.hip); arguments already validated.
hipError_t launch_scale_by_two(const void* x, void* y, int64_t n, int stages, unsigned blocks, hipStream_t stream);

// The attention-style consumer (spt_attention.hip); arguments already validated.
// c = scale * log2(e).
hipError_t launch_attention(int dtype, int D, int variant, int stages, const void* Q, const void* K, const void* V,
                            void* O, int BH, int Sq, int Sk, float c, hipStream_t stream);

// nullptr when that combination is not built.  exact = 1 asks for the
// instantiation that assumes M, N, K are multiples of the tile.
const KernelEntry* find_kernel(int dtype, int bcol, int tile, int variant, int stages, int exact, int window = 0);

}  // namespace spt
