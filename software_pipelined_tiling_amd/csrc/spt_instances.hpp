// spt_instances.hpp -- explicit instantiations of the K-loop kernel for one
// element type.  Included once per element type so the translation units
// compile in parallel.
#pragma once

#include "spt_kernel.hpp"
#include "spt_persist.hpp"
#include "spt_registry.h"

namespace spt {

// hipLaunchKernel returns the status of this launch itself (hipGetLastError
// would also report an error left over from an earlier, unrelated call).
template <class C>
hipError_t launch_gemm(const GemmArgs& a, unsigned grid, hipStream_t stream)
{
    GemmArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&gemm_kernel<C>, dim3(grid), dim3(C::THREADS), args, 0, stream);
}

template <int DT, int BC, int TI, int V, int S, int EX = 0>
constexpr KernelEntry entry()
{
    typedef Cfg<DT, BC != 0, TI, V, S, EX != 0> C;
    return KernelEntry{DT, BC, TI, V, S, EX, 0, C::THREADS, C::LDS_BYTES, C::LOADS, &launch_gemm<C>,
                       (const void*)&gemm_kernel<C>};
}

// Persistent workgroups (spt_persist.hpp): the 128 x 128 tile, exact fit, a
// ring of S stages, the previous tile's C written over P K tiles.
template <class C, int P>
hipError_t launch_persist(const GemmArgs& a, unsigned grid, hipStream_t stream)
{
    GemmArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&gemm_persist_kernel<C, P>, dim3(grid), dim3(C::THREADS), args, 0, stream);
}

template <int DT, int BC, int TI, int S, int P>
constexpr KernelEntry pentry()
{
    typedef Cfg<DT, BC != 0, TI, V_PERSIST, S, true> C;
    return KernelEntry{DT, BC, TI, V_PERSIST, S, 1, P, C::THREADS, C::LDS_BYTES, C::LOADS, &launch_persist<C, P>,
                       (const void*)&gemm_persist_kernel<C, P>};
}
// Windows of 2, 4 and 8 K tiles (8, 4 or 2 stores per K tile of the 16
// blocks of a 64 x 64 wave tile); a window covers at least S-1 K tiles.
#define SPT_PERSIST(DT, BC)                                                                          \
    pentry<DT, BC, 3, 2, 2>(), pentry<DT, BC, 3, 2, 4>(), pentry<DT, BC, 3, 2, 8>(),                 \
        pentry<DT, BC, 3, 3, 2>(), pentry<DT, BC, 3, 3, 4>(), pentry<DT, BC, 3, 3, 8>(),             \
        pentry<DT, BC, 3, 4, 4>(), pentry<DT, BC, 3, 4, 8>()

// Every (variant, stages) pair of the boundary for one (dtype, layout, tile).
#define SPT_PAIRS(DT, BC, TI)                                                              \
    entry<DT, BC, TI, V_SYNC, 1>(), entry<DT, BC, TI, V_REG, 1>(), entry<DT, BC, TI, V_REG, 2>(), \
        entry<DT, BC, TI, V_DIRECT, 2>()
// The 3- and 4-stage rings where they fit in LDS (not the 256 x 256 x 64-byte
// tiles: 3 x 64 KiB).
#define SPT_RING3(DT, BC, TI) entry<DT, BC, TI, V_DIRECT, 3>()
#define SPT_RING34(DT, BC, TI) entry<DT, BC, TI, V_DIRECT, 3>(), entry<DT, BC, TI, V_DIRECT, 4>()

// Exact-fit instantiations (no K tail, no edge checks) of every (variant, stages) pair: the
// unpipelined and register-staged loops are compared with the ring in the same form.  (The
// general 256 x 256 kernels spill: their edge and tail code needs registers the 256
// accumulators of a 128 x 128 wave tile leave no room for.)
#define SPT_EXACT(DT, BC, TI)                                                                    \
    entry<DT, BC, TI, V_SYNC, 1, 1>(), entry<DT, BC, TI, V_REG, 1, 1>(), entry<DT, BC, TI, V_REG, 2, 1>(), \
        entry<DT, BC, TI, V_DIRECT, 2, 1>()
#define SPT_EXACT34(DT, BC, TI) entry<DT, BC, TI, V_DIRECT, 3, 1>(), entry<DT, BC, TI, V_DIRECT, 4, 1>()

#define SPT_TILE_ALL(DT, BC, TI) SPT_PAIRS(DT, BC, TI), SPT_RING34(DT, BC, TI), SPT_EXACT(DT, BC, TI), SPT_EXACT34(DT, BC, TI)
#define SPT_TILE_BIG(DT, BC, TI) SPT_PAIRS(DT, BC, TI), SPT_EXACT(DT, BC, TI)
// The 3-stage rings of the 256 x 256 x 128-byte tiles, as 5 half-stage slots.
#define SPT_HALF(DT, BC) entry<DT, BC, 4, V_DIRECT, 3>(), entry<DT, BC, 4, V_DIRECT, 3, 1>(), \
        entry<DT, BC, 2, V_DIRECT, 3>(), entry<DT, BC, 2, V_DIRECT, 3, 1>()

// The table of one (element type, B layout): NAME is e.g. f16_row.  Race-detection
// builds (SPT_POISON) hold the ring kernels only: DIRECT on every tile and PERSIST.
#ifdef SPT_POISON
#define SPT_RING_ONLY(DT, BC, TI) entry<DT, BC, TI, V_DIRECT, 2>(), entry<DT, BC, TI, V_DIRECT, 2, 1>()
#define SPT_TABLE_ENTRIES(DT, BC)                                                                      \
    SPT_RING_ONLY(DT, BC, 1), SPT_RING34(DT, BC, 1), SPT_EXACT34(DT, BC, 1), SPT_RING_ONLY(DT, BC, 2),   \
        entry<DT, BC, 3, V_DIRECT, 2>(), SPT_RING34(DT, BC, 3), SPT_RING_ONLY(DT, BC, 4),               \
        SPT_RING_ONLY(DT, BC, 5), SPT_RING34(DT, BC, 5), SPT_EXACT34(DT, BC, 5), SPT_RING_ONLY(DT, BC, 6),  \
        SPT_HALF(DT, BC), SPT_PERSIST(DT, BC)
#else
#define SPT_TABLE_ENTRIES(DT, BC)                                                                      \
    SPT_TILE_ALL(DT, BC, 1), SPT_TILE_BIG(DT, BC, 2), SPT_PAIRS(DT, BC, 3), SPT_RING34(DT, BC, 3),      \
        SPT_TILE_BIG(DT, BC, 4), SPT_TILE_ALL(DT, BC, 5), SPT_TILE_BIG(DT, BC, 6), SPT_HALF(DT, BC),      \
        SPT_PERSIST(DT, BC)
#endif
#define SPT_DEFINE_TABLE(NAME, DT, BC)                                                          \
    static const KernelEntry k_##NAME[] = {                                                    \
        SPT_TABLE_ENTRIES(DT, BC),                                                             \
    };                                                                                         \
    KernelTable kernels_##NAME() { return KernelTable{k_##NAME, (int)(sizeof(k_##NAME) / sizeof(k_##NAME[0]))}; }

}  // namespace spt
