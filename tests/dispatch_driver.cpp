// Checks the launches the C ABI's dispatcher makes (built and run on the host
// by tests/test_dispatch.py).  spt_api.cpp is linked with kernel tables that
// hold an entry for every (tile, variant, stages, exact, window) and whose
// launchers only record the grid and kernel arguments, so nothing reaches a
// GPU.  For each shape on stdin ("dtype layout variant stages tile M N K") it
// prints the plan (spt_plan) and every launch spt_gemm_ex made:
//   plan <rc> <grid> <tiles_m> <tiles_n> <band_grid> <band_m> <variant> <tile>
//   launch <grid> <M> <tiles_m> <tiles_n> <k_full> <k_tail>
//   end <rc>
// Pointers are fake, aligned, disjoint device-range addresses that are never
// dereferenced.
#include <stdint.h>
#include <stdio.h>

#include <vector>

#include <hip/hip_runtime.h>

#include "../include/spt.h"
#include "../software_pipelined_tiling_amd/csrc/spt_registry.h"

namespace spt {

struct Launch {
    unsigned grid;
    GemmArgs a;
};
static std::vector<Launch> g_launches;

static hipError_t record(const GemmArgs& a, unsigned grid, hipStream_t)
{
    g_launches.push_back(Launch{grid, a});
    return hipSuccess;
}

static std::vector<KernelEntry> make_table(int dtype, int bcol)
{
    std::vector<KernelEntry> t;
    for (int tile = 1; tile < kNumTiles; ++tile)
        for (int v = V_SYNC; v <= V_PERSIST; ++v)
            for (int s = 1; s <= 4; ++s)
                for (int ex = 0; ex <= 1; ++ex)
                    for (int w : {0, 2, 4, 8}) {
                        if ((v == V_PERSIST) != (w != 0)) continue;
                        t.push_back(KernelEntry{dtype, bcol, tile, v, s, ex, w, 256, 0, 0, &record, nullptr});
                    }
    return t;
}

#define SPT_RECORDING_TABLE(NAME, DT, BC)                               \
    KernelTable kernels_##NAME()                                        \
    {                                                                   \
        static const std::vector<KernelEntry> t = make_table(DT, BC);   \
        return KernelTable{t.data(), (int)t.size()};                    \
    }
SPT_RECORDING_TABLE(f16_row, DT_F16, 0)
SPT_RECORDING_TABLE(f16_col, DT_F16, 1)
SPT_RECORDING_TABLE(bf16_row, DT_BF16, 0)
SPT_RECORDING_TABLE(bf16_col, DT_BF16, 1)
SPT_RECORDING_TABLE(i8_row, DT_I8, 0)
SPT_RECORDING_TABLE(i8_col, DT_I8, 1)
SPT_RECORDING_TABLE(f32_row, DT_F32, 0)
SPT_RECORDING_TABLE(f32_col, DT_F32, 1)
hipError_t launch_scale_by_two(const void*, void*, int64_t, int, unsigned, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_attention(int, int, int, int, const void*, const void*, const void*, void*, int, int, int, float,
                            hipStream_t)
{
    return hipErrorInvalidValue;
}
}  // namespace spt

int main()
{
    int dtype, layout, variant, stages, tile;
    long long M, N, K;
    while (scanf("%d %d %d %d %d %lld %lld %lld", &dtype, &layout, &variant, &stages, &tile, &M, &N, &K) == 8) {
        spt_plan_info p;
        int rc = spt_plan(dtype, M, N, K, layout, variant, stages, tile, &p);
        printf("plan %d %lld %lld %lld %lld %lld %d %d\n", rc, (long long)p.grid, (long long)p.tiles_m,
               (long long)p.tiles_n, (long long)p.band_grid, (long long)p.band_m, p.variant, p.tile_id);
        const int elt = dtype == 2 ? 1 : dtype == 3 ? 4 : 2;
        const int64_t lda = ((K > 0 ? K : 1) * elt + 15) / 16 * 16 / elt;
        const int64_t ldb = layout == SPT_COL ? lda : (N * elt + 15) / 16 * 16 / elt;
        const int64_t ldc = (N + 3) / 4 * 4;
        spt::g_launches.clear();
        rc = spt_gemm_ex(M, N, K, (const void*)(uintptr_t)(1ull << 40), lda, (const void*)(uintptr_t)(1ull << 41),
                         ldb, (void*)(uintptr_t)(1ull << 42), ldc, dtype, nullptr, layout, variant, stages, tile);
        for (const auto& l : spt::g_launches)
            printf("launch %u %d %d %d %d %d\n", l.grid, l.a.M, l.a.tiles_m, l.a.tiles_n, l.a.k_full, l.a.k_tail);
        printf("end %d\n", rc);
    }
    return 0;
}
