// spt_config.h -- tile menu and kernel argument block shared by the host
// planner/dispatcher and the gfx950 kernels of libspt.
#pragma once

#include <stdint.h>

namespace spt {

enum DType { DT_F16 = 0, DT_BF16 = 1, DT_I8 = 2, DT_F32 = 3 };
enum Variant { V_AUTO = 0, V_SYNC = 1, V_REG = 2, V_DIRECT = 3, V_PERSIST = 4 };

// One workgroup tile: BM x BN outputs, K depth of BKB bytes per row (BK =
// BKB / elt elements), WAVES_M x WAVES_N waves of 64 lanes.
struct TileShape {
    int BM, BN, BKB, WAVES_M, WAVES_N;
};

// Index = spt_tile enum value.  Entry 1 is the 128 x 256 x 32 (fp16) tile
// with 256 threads of "Hiding Memory Latency in CUDA: Asynchronous Loads and
// Software Pipelines", section 6.
constexpr TileShape kTiles[] = {
    {0, 0, 0, 0, 0},          // AUTO (resolved by the planner)
    {128, 256, 64, 2, 2},     // SPT_TILE_128x256, 256 threads
    {256, 256, 128, 2, 4},    // SPT_TILE_256x256, 512 threads
    {128, 128, 64, 2, 2},     // SPT_TILE_128x128, 256 threads
    {256, 256, 128, 2, 2},    // SPT_TILE_256x256_4W, 256 threads, 128 x 128 per wave
    {256, 256, 64, 2, 2},     // SPT_TILE_256x256_4W_K64B: the same with a 64-byte K depth
    {256, 192, 128, 2, 4},    // SPT_TILE_256x192, 512 threads, 128 x 48 per wave
};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

constexpr int elt_bytes(int dt) { return dt == DT_I8 ? 1 : dt == DT_F32 ? 4 : 2; }

// Tiles whose general DIRECT kernels copy a chunk-aligned partial K tile through the
// ring (GemmArgs::tail_ring).  The 256 x 256 tiles with 128 x 64 and 128 x 128 wave
// tiles keep the VGPR tail: the in-ring tail costs them registers they do not have
// (the 8-wave form would spill).
constexpr bool ring_tail_tile(int tile) { return tile != 2 && tile != 4; }

// gfx950 (CDNA4) per-CU resources (AMD public specification).
constexpr int kLdsPerCu = 163840;   // 160 KiB
constexpr int kSimdsPerCu = 4;
constexpr int kWaveSize = 64;
constexpr int kMaxWavesPerSimd = 8;
constexpr int kVgprsPerSimdLane = 512;  // unified arch + acc VGPR file per lane

// Kernel arguments.  Sizes fit in int32 (checked on the host); byte offsets
// inside one workgroup's operand panel fit in 31 bits (also checked).
struct GemmArgs {
    const char* A;
    const char* B;
    char* C;
    int M, N, K;
    int lda, ldb, ldc;   // in elements
    int tiles_m, tiles_n;
    int k_full;          // number of full BK-deep tiles
    int k_tail;          // K - k_full * BK (0 = none)
    int tail_ring;       // 1: the partial tile goes through the DIRECT ring as tile k_full
                         // (k_tail * elt a multiple of 16: whole chunks are in or past K)
};

}  // namespace spt
