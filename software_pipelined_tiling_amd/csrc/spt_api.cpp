// spt_api.cpp -- the C ABI of libspt: argument validation, planning and
// dispatch of the K-loop kernels (declared in include/spt.h).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/spt.h"
#include "spt_config.h"
#include "spt_registry.h"

namespace spt {

static thread_local char g_last_error[256] = "";

static int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
static int fail(int status, const char* fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return status;
}

static const KernelTable& table_for(int dtype, int bcol)
{
    static const KernelTable t[4][2] = {{kernels_f16_row(), kernels_f16_col()},
                                        {kernels_bf16_row(), kernels_bf16_col()},
                                        {kernels_i8_row(), kernels_i8_col()},
                                        {kernels_f32_row(), kernels_f32_col()}};
    return t[dtype][bcol ? 1 : 0];
}

const KernelEntry* find_kernel(int dtype, int bcol, int tile, int variant, int stages, int exact, int window)
{
    if (dtype < 0 || dtype > 3) return nullptr;
    const KernelTable& t = table_for(dtype, bcol);
    for (int i = 0; i < t.count; ++i) {
        const KernelEntry& e = t.entries[i];
        if (e.bcol == bcol && e.tile == tile && e.variant == variant && e.stages == stages && e.exact == exact &&
            e.window == window)
            return &e;
    }
    return nullptr;
}

// The library's default when the caller passes AUTO (chosen from measured
// sweeps on MI355X).  Tile:
//  - 256 x 256 with one wave per SIMD (the least LDS and global traffic per
//    MFMA) when the shape is an exact multiple of it, its grid gives each of
//    the 256 CUs a workgroup and K spans at least 2 KiB of each row (shorter K
//    is bound by the C store, where two 128 x 256 workgroups per CU do better);
//  - else 128 x 128 when the 128 x 256 grid leaves CUs without a workgroup;
//  - else the 128 x 256 tile (two workgroups per CU) or the 256 x 256 tile of 8
//    waves (one per CU), whichever leaves the lower load on the busiest CU,
//    counted in 256 x 256 tiles with the larger tile's ~10% better throughput
//    per FLOP.  The larger tile is taken only with K of at least 1 KiB per row,
//    and, below 2 KiB, only when its grid fits in one round (a single resident
//    workgroup per CU waits out each round's C store).  Measured fp16/bf16/int8:
//    4000 x 3000 x 1000..4000, 3000^3, 5000^2 x 1024 and 8000 x 2000 x 8000
//    run 4-25% faster on the 256 x 256 tile; 2000 x 4000 x 1000, 4100^3 and
//    6000^2 x 2000, whose large tiles leave CUs idle or a long partial round,
//    run faster on 128 x 256.  Where the 8-wave 256 x 256 grid would leave CUs
//    idle in its single round and a 256 x 192 grid still fits one round, the
//    256 x 192 tile: 2-11% faster on 4000 x 3000 x 1000, 3000^3, 4000 x 3008 x
//    4000, 2048 x 6144 x 2048 and 4096 x 3072 x 1024 (bit-identical results).
//    Exact-fit fp16/bf16 shapes whose 256 x 256 grid ends in a partly filled
//    round also take the 256 x 192 tile when 0.9 x its rounds are fewer:
//    4608^3, 6144^3, 6144^2 x 2048 and 4096 x 6144 x 4096 run 9-13% faster;
//    4096^3, 5120^2 x 4096, 5376^2 x 4096, 7168^2 x 4096 and 8192^3 keep
//    256 x 256 (the 256 x 192 tile measured 2-35% slower there).  int8
//    follows the same rule: with column-major B 13-18% faster on 4608^3, 6144^3
//    and 4096 x 6144 x 4096, slower on 5120^2 x 4096 and 8192^3; with row-major
//    B 20% faster than the 256 x 256 tile on 4608^3.
// Variant: the DIRECT ring, 2 stages for 128-byte K tiles (two fill the LDS),
// else 3.
static constexpr int64_t kCus = 256;
static constexpr int64_t kPersistResident = kCus * 2;  // two 128 x 128 workgroups per CU
static void resolve(int dtype, int64_t M, int64_t N, int64_t K, int& variant, int& stages, int& tile)
{
    if (variant == V_PERSIST && tile == 0) tile = 3;
    if (tile == 0) {
        const int elt = elt_bytes(dtype);
        const int64_t bk4 = kTiles[4].BKB / elt;
        const bool fits4 = M % 256 == 0 && N % 256 == 0 && K % bk4 == 0 && K * elt >= 2048;
        const int64_t n4 = (M / 256) * (N / 256);
        const int64_t n1 = ((M + 127) / 128) * ((N + 255) / 256);
        const int64_t n2 = ((M + 255) / 256) * ((N + 255) / 256);
        if (fits4 && n4 >= kCus) {
            tile = 4;
            // A partly filled last round of 256 x 256 tiles: the 256 x 192 grid when its
            // rounds, at 3/4 of the work and ~1.2x the cost per FLOP, take less
            // (fp16/bf16 and int8, N a multiple of 192: as measured).
            const int64_t n6e = (M / 256) * (N / 192);
            if (elt <= 2 && N % 192 == 0 && 9 * ((n6e + kCus - 1) / kCus) < 10 * ((n4 + kCus - 1) / kCus)) tile = 6;
        } else if (n1 < kCus) {
            tile = 3;
        } else {
            const int64_t load2 = (n2 + kCus - 1) / kCus;  // 256 x 256 tiles on the busiest CU
            const int64_t c1 = (n1 + kCus - 1) / kCus;     // 128 x 256 tiles on the busiest CU
            const bool deep = K * elt >= 2048, mid = K * elt >= 1024;
            // load2 <= (c1 / 2) / 0.9
            const bool big = mid && (deep || load2 == 1) && 9 * load2 <= 5 * c1;
            tile = big ? 2 : 1;
            // A 256 x 256 grid that leaves CUs idle in its one round, where the
            // 256 x 192 grid still fits one round: each CU then computes 3/4 as much,
            // at ~1.25x the cost per FLOP (more copies and LDS reads per FLOP).
            const int64_t n6 = ((M + 255) / 256) * ((N + 191) / 192);
            if (big && n2 < kCus && n6 <= kCus) tile = 6;
        }
    }
    if (variant == V_AUTO) {
        variant = V_DIRECT;
        // One or two K tiles leave the ring nothing to overlap ("Pipeline GPU Kernel",
        // Schritt 6: K / BK >= 4 amortises the prologue and epilogue).  Where the C store
        // dominates as well (fp16/bf16/int8 grids of four or more rounds of two workgroups
        // per CU) the unpipelined loop is faster; elsewhere the ring still is.  MI355X,
        // medians, us, DIRECT ring -> SYNC: bf16 8192^2 x 32 45.1 -> 44.3, x 64 50.1 ->
        // 48.9, fp16 8192^2 x 64 50.5 -> 49.1, int8 8192^2 x 128 (B col) 48.5 -> 47.8;
        // kept: bf16 4096^2 x 64 14.6 (SYNC 15.4), 6144^2 x 64 31.8 (32.5), fp16 8192 x
        // 4096 x 64 25.3 (26.9), fp32 8192^2 x 32 67.3 (71.4), bf16 8192^2 x 96 52.6 (55.1).
        const int elt = elt_bytes(dtype);
        const TileShape& T = kTiles[tile];
        const int64_t bk = T.BKB / elt, k_tiles = (K + bk - 1) / bk;
        const int64_t tiles = ((M + T.BM - 1) / T.BM) * ((N + T.BN - 1) / T.BN);
        if (stages == 0 && elt <= 2 && k_tiles >= 1 && k_tiles <= 2 && tiles >= 8 * kCus) variant = V_SYNC;
    }
    if (stages == 0)
        stages = variant == V_SYNC ? 1 : variant == V_REG ? 2 : variant == V_PERSIST ? 3 : (kTiles[tile].BKB >= 128 ? 2 : 3);
}

// PERSIST: the store window (K tiles over which the previous output tile is
// written; 16 / window stores per K tile) for k_full K tiles: the longest of
// 2, 4, 8 that fits (the built instantiations).  Two or more stores per K tile
// keep the two 64-byte halves of every 128-byte line of C in one K tile (one
// store per K tile split the lines and raised the HBM write traffic by a
// fifth, measured).
static int store_window(int64_t k_full) { return k_full >= 8 ? 8 : k_full >= 4 ? 4 : 2; }

static bool valid_pair(int variant, int stages)
{
    return (variant == V_SYNC && stages == 1) || (variant == V_REG && (stages == 1 || stages == 2)) ||
           ((variant == V_DIRECT || variant == V_PERSIST) && stages >= 2 && stages <= 4);
}

// Row band of a nearly empty last round.  A grid whose last round fills at
// most half of the resident workgroup slots (two per CU where the LDS holds
// two, else one) runs the whole rows of tiles that fit the earlier rounds,
// then the rows below them (the band) as a second launch of 128 x 128 tiles
// (DIRECT ring): twice the workgroups of 128 x 256 tiles, each with
// half the work, so the band takes less of a round.  K of at least 2 KiB per
// row: measured through AUTO (medians, us, one grid -> main + band) fp16
// 4100 x 4104 x 4104 170.3 -> 169.1, int8 4100 x 4112 x 4112 (B col) 125.1 ->
// 117.3, bf16 6000^2 x 2000 152.2 -> 149.4, fp32 4100^2 x 1024 348.7 -> 300.5,
// int8 4224 x 4096 x 8192 170.8 -> 162.5, bf16 8448 x 8192 x 2048 257.8 -> 244.6,
// fp16 4352 x 4096 x 8192 329.5 -> 257.7, fp16 4608 x 5120 x 4096 (a band of
// 480 workgroups) 190.4 -> 180.5, fp16 1152 x 32760 x 4096 366.2 -> 330.7;
// below 2 KiB fp16 4224 x 4000 x 520 lost (41.2 -> 44.3).
// (Splitting the band over K instead, added into C with device-scope atomics,
// measured 1.3-2.2x slower than no split at all.)
static constexpr int kBandTile = 3;
static void plan_band(int64_t M, int64_t N, int64_t K, spt_plan_info& p)
{
    if (K * p.elt_bytes < 2048) return;
    const int64_t per_cu = std::min<int64_t>(2, kLdsPerCu / p.lds_bytes);
    const int64_t cap = kCus * per_cu, total = p.tiles_m * p.tiles_n;
    if (total <= cap) return;
    const int64_t rounds = (total + cap - 1) / cap, last = total - (rounds - 1) * cap;
    if (2 * last > cap) return;
    const int64_t rows_main = (rounds - 1) * cap / p.tiles_n;  // whole rows of tiles before the band
    if (rows_main <= 0 || rows_main >= p.tiles_m) return;
    // whole rows must nearly fill the earlier rounds (wide rows of tiles may
    // not), and the band must fit one round of two 128 x 128 workgroups per CU
    if ((rounds - 1) * cap - rows_main * p.tiles_n > cap / 8) return;
    const TileShape& T = kTiles[kBandTile];
    const int64_t band_m = rows_main * p.BM;
    const int64_t band_grid = ((M - band_m + T.BM - 1) / T.BM) * ((N + T.BN - 1) / T.BN);
    if (band_grid > 2 * kCus) return;
    p.band_tile = kBandTile;
    // a band of at most one workgroup per CU with K of at least 8 KiB per row
    // hides more latency with 4 stages (fp16 band rows alone, us, 3 -> 4
    // stages: 256 x 4096 x 8192 68.8 -> 60.1, 128 x 32760 x 4096 66.1 -> 63.4,
    // 260 x 4104 x 4104 42.9 -> 42.8); a band of two per CU keeps 3 (1536 x 5120
    // x 4096: 76.5 against 77.0), and so does bf16 6000^2 x 2000 (AUTO 149.4 us
    // with 3 stages, 157.5 with 4)
    // The same holds for int8, bf16 and fp32 bands (band rows alone, 128 x 128 tile,
    // us, 3 -> 4 stages: int8 128 x 4096 x 8192 with column-major B 35.6 -> 30.8, with
    // row-major B 37.6 -> 37.5; bf16 128 x 4096 x 8192 68.7 -> 60.8, with column-major
    // B 256 x 4096 x 8192 61.6 -> 53.1; fp32 128 x 4096 x 4096 230.5 -> 230.6).
    p.band_stages = band_grid <= kCus && K * p.elt_bytes >= 8192 ? 4 : 3;
    p.band_m = band_m;
    p.band_grid = band_grid;
    p.grid = rows_main * p.tiles_n;
}

// The DIRECT ring copies a partial last K tile itself when its k_tail elements
// are whole 16-byte chunks (each chunk then lies wholly below K or wholly past
// it, and the copies past K are pointed outside the buffer so they read zeros);
// else the general kernels load that tile through VGPRs with per-byte masks.
static int tail_in_ring(int variant, int tile, int k_tail, int elt)
{
    return variant == V_DIRECT && ring_tail_tile(tile) && k_tail > 0 && (k_tail * elt) % 16 == 0 ? 1 : 0;
}

// Checks every argument except the pointers; fills `pi` on success.
static int make_plan(int dtype, int64_t M, int64_t N, int64_t K, int b_layout, int variant,
                     int stages, int tile, spt_plan_info* pi)
{
    if (dtype < 0 || dtype > 3) return fail(SPT_ERR_INVALID, "dtype %d is not an spt_dtype", dtype);
    if (b_layout != SPT_ROW && b_layout != SPT_COL)
        return fail(SPT_ERR_INVALID, "b_layout %d is not an spt_layout", b_layout);
    if (variant < 0 || variant > 4) return fail(SPT_ERR_INVALID, "variant %d is not an spt_variant", variant);
    if (stages < 0 || stages > 4) return fail(SPT_ERR_INVALID, "stages %d not in 0..4", stages);
    if (tile < 0 || tile >= kNumTiles) return fail(SPT_ERR_INVALID, "tile_id %d is not an spt_tile", tile);
    if (M < 0 || N < 0 || K < 0) return fail(SPT_ERR_INVALID, "negative size");
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX) return fail(SPT_ERR_UNSUPPORTED, "size above 2^31-1");
    if (dtype == DT_I8 && K > 131071)
        return fail(SPT_ERR_UNSUPPORTED, "int8 K=%lld exceeds 131071 (exact int32 sum)", (long long)K);
    const bool auto_choice = variant == V_AUTO && stages == 0 && tile == 0;
    resolve(dtype, M, N, K, variant, stages, tile);
    if (!valid_pair(variant, stages))
        return fail(SPT_ERR_UNSUPPORTED, "variant %d has no %d-stage form", variant, stages);
    if (variant == V_PERSIST && tile != 3)
        return fail(SPT_ERR_UNSUPPORTED, "the persistent variant runs the 128 x 128 tile only");

    const TileShape& T = kTiles[tile];
    const int elt = elt_bytes(dtype);
    spt_plan_info p;
    memset(&p, 0, sizeof p);
    p.dtype = dtype;
    p.b_layout = b_layout;
    p.variant = variant;
    p.stages = stages;
    p.tile_id = tile;
    p.BM = T.BM;
    p.BN = T.BN;
    p.BK = T.BKB / elt;
    p.waves = T.WAVES_M * T.WAVES_N;
    p.threads = kWaveSize * p.waves;
    p.wave_m = T.BM / T.WAVES_M;
    p.wave_n = T.BN / T.WAVES_N;
    p.elt_bytes = elt;
    p.tiles_m = (M + T.BM - 1) / T.BM;
    p.tiles_n = (N + T.BN - 1) / T.BN;
    p.grid = p.tiles_m * p.tiles_n;
    p.k_tiles = (K + p.BK - 1) / p.BK;
    p.k_full_tiles = K / p.BK;
    if (variant == V_PERSIST) {
        // as many workgroups as the CUs hold at once: two per CU (64 x 64 per
        // wave, two accumulator sets in 128 registers, two waves per SIMD).
        // The grid stays a multiple of the 8 XCDs, so that a workgroup's tile
        // stream stays on one XCD.  The previous tile's C is written over the
        // store window.
        if (p.grid > kPersistResident) p.grid = kPersistResident;
        p.store_window = store_window(p.k_full_tiles);
    }
    p.band_m = M;
    p.k_tail = (int32_t)(K - p.k_full_tiles * p.BK);
    p.tail_ring = tail_in_ring(variant, tile, p.k_tail, elt);
    // "Pipeline GPU Kernel", Schritt 1: smem_a = BM*BK*sizeof(T), smem_b = BK*BN*sizeof(T).
    p.a_stage_bytes = p.BM * p.BK * elt;
    p.b_stage_bytes = p.BK * p.BN * elt;
    p.stage_bytes = p.a_stage_bytes + p.b_stage_bytes;
    p.lds_bytes = stages * p.stage_bytes;
    // A DIRECT ring of S stages that does not fit, of a tile whose A and B parts are the
    // same size, runs as 2S - 1 half-stage slots (the kernel's half-stage ring).
    if (variant == V_DIRECT && p.lds_bytes > kLdsPerCu && p.a_stage_bytes == p.b_stage_bytes &&
        (2 * stages - 1) * p.a_stage_bytes <= kLdsPerCu) {
        p.half_stage_slots = 2 * stages - 1;
        p.lds_bytes = p.half_stage_slots * p.a_stage_bytes;
    }
    if (p.lds_bytes > kLdsPerCu)
        return fail(SPT_ERR_UNSUPPORTED, "a %d-stage ring of %d-byte stages exceeds the 160 KiB of LDS", stages,
                    p.stage_bytes);
    // "Hiding Memory Latency ...", section 6: 16-byte accesses per thread per stage.
    p.a_copies_per_thread = p.a_stage_bytes / 16 / p.threads;
    p.b_copies_per_thread = p.b_stage_bytes / 16 / p.threads;
    // "Kernel-Engpass analysieren", Schritt 3 / 6: the LDS limit on resident workgroups.
    p.wg_per_cu_lds = kLdsPerCu / p.lds_bytes;
    p.waves_per_simd_lds = p.wg_per_cu_lds * p.waves / kSimdsPerCu;
    p.steady_vmcnt = variant == V_DIRECT ? (stages - 2) * (p.a_copies_per_thread + p.b_copies_per_thread) : 0;
    if (p.half_stage_slots)  // B of the next tile landed, A of the tile after it in flight
        p.steady_vmcnt = (p.half_stage_slots - 4) * p.a_copies_per_thread;
    if (variant == V_PERSIST)  // the younger copies, and the stores issued after the awaited copies
        p.steady_vmcnt = (stages - 2) * (p.a_copies_per_thread + p.b_copies_per_thread) +
                         (stages - 1) * ((p.wave_m / 16) * (p.wave_n / 16) / p.store_window);
    // one 16x16 MFMA step covers 64 bytes of k per lane group; fp32 issues 4 MFMAs per step
    if (auto_choice && variant == V_DIRECT) plan_band(M, N, K, p);
    p.tiles_per_wg = p.grid > 0 ? (int32_t)((p.tiles_m * p.tiles_n + p.grid - 1) / p.grid) : 0;
    if (p.band_tile) p.tiles_per_wg = 1;
    const int kstep = 4 * (16 / elt);
    p.mfma_per_ktile_per_wave = (p.wave_m / 16) * (p.wave_n / 16) * (p.BK / kstep) * (dtype == DT_F32 ? 4 : 1);
    // "Pipeline GPU Kernel", Schritt 2: 2*BM*BN*BK / ((BM*BK + BK*BN) * sizeof(T)).
    p.ratio_flop_per_byte = (2.0 * p.BM * p.BN * p.BK) / ((double)(p.BM * p.BK + p.BK * p.BN) * elt);
    // "Kernel-Engpass analysieren", Schritt 4: compute instructions per load instruction.
    p.ratio_mfma_per_load =
        (double)p.mfma_per_ktile_per_wave / (double)(p.a_copies_per_thread + p.b_copies_per_thread);
    *pi = p;
    return SPT_OK;
}

// Workgroups of the main launch: one per output tile, except for the
// persistent variant (at most the resident workgroups, each walking a stream
// of tiles) and a row band (the whole rows of tiles before the band; the band
// is a second launch).  spt_plan reports the same number.
static int64_t main_grid(const spt_plan_info& pi, bool band)
{
    if (pi.variant == V_PERSIST || band) return pi.grid;
    return pi.tiles_m * pi.tiles_n;
}

static int gemm_impl(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B,
                     int64_t ldb, void* C, int64_t ldc, int dtype, void* stream, int b_layout,
                     int variant, int stages, int tile)
{
    spt_plan_info pi;
    int rc = make_plan(dtype, M, N, K, b_layout, variant, stages, tile, &pi);
    if (rc != SPT_OK) return rc;
    if (M == 0 || N == 0) return SPT_OK;

    const int elt = pi.elt_bytes;
    const bool bcol = b_layout == SPT_COL;
    if (!C) return fail(SPT_ERR_INVALID, "C is null");
    if (K > 0 && (!A || !B)) return fail(SPT_ERR_INVALID, "A or B is null");
    const int64_t kmin = K > 0 ? K : 1;
    if (lda < kmin) return fail(SPT_ERR_INVALID, "lda=%lld < K", (long long)lda);
    if (bcol ? ldb < kmin : ldb < N) return fail(SPT_ERR_INVALID, "ldb=%lld too small", (long long)ldb);
    if (ldc < N) return fail(SPT_ERR_INVALID, "ldc=%lld < N", (long long)ldc);
    if (lda > INT32_MAX || ldb > INT32_MAX || ldc > INT32_MAX)
        return fail(SPT_ERR_UNSUPPORTED, "row pitch above 2^31-1");
    if (((uintptr_t)C % 16) || (ldc * 4) % 16) return fail(SPT_ERR_MISALIGNED, "C or ldc not 16-byte aligned");
    if (K > 0 && (((uintptr_t)A % 16) || ((uintptr_t)B % 16) || (lda * elt) % 16 || (ldb * elt) % 16))
        return fail(SPT_ERR_MISALIGNED, "A, B, lda or ldb not 16-byte aligned");
    // Buffer descriptors hold 48-bit base addresses (the copy path lowers a
    // base by a few KiB before adding offsets back).
    if (K > 0 && ((uintptr_t)A >> 47 || (uintptr_t)B >> 47 || (uintptr_t)A < 65536 || (uintptr_t)B < 65536))
        return fail(SPT_ERR_UNSUPPORTED, "A or B outside the device address range of buffer descriptors");
    // Byte offsets inside one workgroup's operand panel are 32-bit buffer offsets.
    const int64_t lim = INT64_C(0x7ffffff0);
    if ((int64_t)pi.BM * lda * elt >= lim || (bcol ? (int64_t)pi.BN * ldb * elt : (int64_t)pi.BK * ldb * elt) >= lim)
        return fail(SPT_ERR_UNSUPPORTED, "operand panel exceeds 2 GiB of buffer offsets");
    // (tile indices, and a persistent stream's next index, are 32-bit in the kernels)
    if (pi.grid > INT32_MAX || pi.tiles_m * pi.tiles_n > INT32_MAX - 4096)
        return fail(SPT_ERR_UNSUPPORTED, "too many output tiles");
    // C is written while A and B are read: it must not share a byte with either
    // (the byte ranges from each base to the end of its last row's used part)
    if (K > 0) {
        const uintptr_t c0 = (uintptr_t)C, c1 = c0 + (uintptr_t)((M - 1) * ldc + N) * 4;
        const uintptr_t a0 = (uintptr_t)A, a1 = a0 + (uintptr_t)((M - 1) * lda + K) * elt;
        const uintptr_t b0 = (uintptr_t)B,
                        b1 = b0 + (uintptr_t)(bcol ? (N - 1) * ldb + K : (K - 1) * ldb + N) * elt;
        if ((c0 < a1 && a0 < c1) || (c0 < b1 && b0 < c1))
            return fail(SPT_ERR_INVALID, "C overlaps A or B");
    }

    // The exact-fit instantiation when M, N and K are multiples of the tile
    // (same arithmetic, no tail or edge code), else the general one.
    // A tile of one 64-byte MFMA k-step runs its ring in pairs of tiles (the
    // register slot of step 0 alternates); the exact-fit form has no odd last tile.
    // Row band (AUTO): the band kernel's B panel must also fit 32-bit offsets,
    // else the grid runs as one launch.
    const TileShape& TB = kTiles[kBandTile];
    bool band = pi.band_tile > 0;
    if (band && (bcol ? (int64_t)TB.BN * ldb * elt : (int64_t)(TB.BKB / elt) * ldb * elt) >= lim) band = false;
    const int64_t M_main = band ? pi.band_m : M;
    const int64_t grid = main_grid(pi, band);
    if (pi.variant == V_PERSIST && grid > kPersistResident)
        return fail(SPT_ERR_LAUNCH, "internal: persistent grid of %lld workgroups", (long long)grid);
    const bool one_step = kTiles[pi.tile_id].BKB == 64;
    const bool fits = M_main % pi.BM == 0 && N % pi.BN == 0 && pi.k_tail == 0 && (!one_step || pi.k_full_tiles % 2 == 0);
    const KernelEntry* e = nullptr;
    if (pi.variant == V_PERSIST) {
        if (!fits || pi.k_full_tiles < 2 || pi.store_window < pi.stages - 1)
            return fail(SPT_ERR_UNSUPPORTED,
                        "the persistent variant needs M %% %d == 0, N %% %d == 0 and an even number (>= %d) of "
                        "whole K tiles of %d",
                        pi.BM, pi.BN, pi.stages == 4 ? 4 : 2, pi.BK);
        // the C store of one output tile is a 32-bit buffer range of BM row pitches
        if ((int64_t)pi.BM * ldc * 4 >= lim) return fail(SPT_ERR_UNSUPPORTED, "C row panel exceeds 2 GiB");
        e = find_kernel(dtype, bcol, pi.tile_id, pi.variant, pi.stages, 1, pi.store_window);
    } else {
        e = fits ? find_kernel(dtype, bcol, pi.tile_id, pi.variant, pi.stages, 1) : nullptr;
        if (!e) e = find_kernel(dtype, bcol, pi.tile_id, pi.variant, pi.stages, 0);
    }
    if (!e) return fail(SPT_ERR_UNSUPPORTED, "no kernel built for dtype %d layout %d tile %d variant %d stages %d",
                        dtype, b_layout, pi.tile_id, pi.variant, pi.stages);
    const KernelEntry* eb = band ? find_kernel(dtype, bcol, kBandTile, V_DIRECT, pi.band_stages, 0) : nullptr;
    if (band && !eb) return fail(SPT_ERR_UNSUPPORTED, "no band kernel built for dtype %d layout %d", dtype, b_layout);

    GemmArgs a;
    a.A = (const char*)A;
    a.B = (const char*)B;
    a.C = (char*)C;
    a.M = (int)M_main;
    a.N = (int)N;
    a.K = (int)K;
    a.lda = (int)lda;
    a.ldb = (int)ldb;
    a.ldc = (int)ldc;
    a.tiles_m = (int)(band ? M_main / pi.BM : pi.tiles_m);
    a.tiles_n = (int)pi.tiles_n;
    a.k_full = (int)pi.k_full_tiles;
    a.k_tail = pi.k_tail;
    a.tail_ring = pi.tail_ring;
    hipError_t err = e->launch(a, (unsigned)grid, (hipStream_t)stream);
    if (err != hipSuccess) return fail(SPT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(err));
    if (band) {  // rows [M_main, M) on the band tile, after the main grid in stream order
        GemmArgs b = a;
        b.A = (const char*)A + M_main * lda * elt;
        b.C = (char*)C + M_main * ldc * 4;
        b.M = (int)(M - M_main);
        b.tiles_m = (b.M + TB.BM - 1) / TB.BM;
        b.tiles_n = (int)((N + TB.BN - 1) / TB.BN);
        b.k_full = (int)(K / (TB.BKB / elt));
        b.k_tail = (int)(K - (int64_t)b.k_full * (TB.BKB / elt));
        b.tail_ring = tail_in_ring(V_DIRECT, kBandTile, b.k_tail, elt);
        if ((int64_t)b.tiles_m * b.tiles_n != pi.band_grid)
            return fail(SPT_ERR_LAUNCH, "internal: band grid mismatch");
        err = eb->launch(b, (unsigned)pi.band_grid, (hipStream_t)stream);
        if (err != hipSuccess) return fail(SPT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(err));
    }
    return SPT_OK;
}

// The streaming pipeline: validation, then one launch.
static int scale_by_two_impl(int64_t n, const void* x, void* y, int stages, int blocks, void* stream)
{
    if (n < 0) return fail(SPT_ERR_INVALID, "negative n");
    if (stages < 0 || stages > 4) return fail(SPT_ERR_INVALID, "stages %d not in 0..4", stages);
    if (blocks < 0) return fail(SPT_ERR_INVALID, "negative blocks");
    if (n > (int64_t)1 << 40) return fail(SPT_ERR_UNSUPPORTED, "n above 2^40");
    if (n == 0) return SPT_OK;
    if (!x || !y) return fail(SPT_ERR_INVALID, "x or y is null");
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    const uintptr_t bytes = (uintptr_t)n * 4;
    if (xa != ya && xa < ya + bytes && ya < xa + bytes)
        return fail(SPT_ERR_INVALID, "x and y overlap without being the same array");
    if (xa % 16 || ya % 16) return fail(SPT_ERR_MISALIGNED, "x or y not 16-byte aligned");
    if (xa >> 47 || ya >> 47 || xa < 65536 || ya < 65536)
        return fail(SPT_ERR_UNSUPPORTED, "x or y outside the device address range of buffer descriptors");
    const int64_t tiles = (n + 1023) / 1024;
    // default: the pages' three stages.  Blocks: about 3-4 MiB of copies in
    // flight over the chip, blocks x (S - 1) x 4 KiB (measured on MI355X at 2^28
    // floats, TB/s: S = 2 with 512 / 768 / 1024 blocks 4.97 / 5.74 / 5.61; S = 3
    // with 256 / 512 / 768 5.08 / 5.79 / 5.59; S = 4 with 256 / 512 5.94 / 5.34;
    // more in flight runs slower still, 4.3-4.6 at 2048-4096 blocks).
    const int s = stages == 0 ? 3 : stages;
    const int64_t want = blocks != 0 ? blocks : (s == 1 ? 1024 : s == 2 ? 768 : s == 3 ? 512 : 256);
    const int64_t g = want < tiles ? want : tiles;
    const hipError_t err = launch_scale_by_two(x, y, n, s, (unsigned)g, (hipStream_t)stream);
    if (err != hipSuccess) return fail(SPT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(err));
    return SPT_OK;
}

// The attention-style consumer: validation, then one launch.
static int attention_impl(int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const void* Q, const void* K,
                          const void* V, void* O, float scale, int dtype, void* stream, int variant, int stages)
{
    if (dtype != DT_F16 && dtype != DT_BF16) return fail(SPT_ERR_UNSUPPORTED, "attention: dtype %d (f16, bf16)", dtype);
    if (variant < 0 || variant > 3) return fail(SPT_ERR_INVALID, "variant %d is not a producer", variant);
    if (stages < 0 || stages > 4) return fail(SPT_ERR_INVALID, "stages %d not in 0..4", stages);
    if (BH < 0 || Sq < 0 || Sk < 0 || D < 0) return fail(SPT_ERR_INVALID, "negative size");
    if (!(scale >= 0.0f) || scale > 3.0e38f) return fail(SPT_ERR_INVALID, "scale must be finite and >= 0");
    // AUTO: the DIRECT ring of two stages (measured the fastest producer at 4096 keys;
    // three stages ran 0-3% slower and take more registers)
    if (variant == V_AUTO) variant = V_DIRECT;
    if (stages == 0) stages = variant == V_SYNC ? 1 : 2;
    if (!((variant == V_SYNC && stages == 1) || (variant == V_REG && (stages == 1 || stages == 2)) ||
          (variant == V_DIRECT && (stages == 2 || stages == 3))))
        return fail(SPT_ERR_UNSUPPORTED, "attention: variant %d has no %d-stage form", variant, stages);
    if (D != 64 && D != 128) return fail(SPT_ERR_UNSUPPORTED, "attention: head dimension %lld (64, 128)", (long long)D);
    if (BH == 0 || Sq == 0) return SPT_OK;
    if (Sk == 0) return fail(SPT_ERR_INVALID, "attention over no keys (a softmax over an empty row)");
    if (Sq > INT32_MAX || Sk > INT32_MAX || BH > INT32_MAX) return fail(SPT_ERR_UNSUPPORTED, "size above 2^31-1");
    if ((uint64_t)BH * (uint64_t)Sq > (UINT64_C(1) << 40) || (uint64_t)BH * (uint64_t)Sk > (UINT64_C(1) << 40))
        return fail(SPT_ERR_UNSUPPORTED, "Q, K or V above 2^40 rows");
    // (the kernel reads a slice's K and V through one buffer descriptor each, with
    // 32-bit offsets that run up to two key blocks past the slice's end)
    if ((uint64_t)Sk * (uint64_t)D * 2 > (UINT64_C(1) << 31))
        return fail(SPT_ERR_UNSUPPORTED, "attention: one slice's K or V above 2^31 bytes");
    if (BH * ((Sq + 255) / 256) > INT32_MAX) return fail(SPT_ERR_UNSUPPORTED, "too many workgroups");
    if (!Q || !K || !V || !O) return fail(SPT_ERR_INVALID, "Q, K, V or O is null");
    if ((uintptr_t)Q % 16 || (uintptr_t)K % 16 || (uintptr_t)V % 16 || (uintptr_t)O % 16)
        return fail(SPT_ERR_MISALIGNED, "Q, K, V or O not 16-byte aligned");
    const uintptr_t hi = (uintptr_t)1 << 47;
    const uintptr_t q0 = (uintptr_t)Q, k0 = (uintptr_t)K, v0 = (uintptr_t)V, o0 = (uintptr_t)O;
    const uintptr_t q1 = q0 + (uintptr_t)(BH * Sq * D * 2), k1 = k0 + (uintptr_t)(BH * Sk * D * 2),
                    v1 = v0 + (uintptr_t)(BH * Sk * D * 2), o1 = o0 + (uintptr_t)(BH * Sq * D * 4);
    if (q0 < 65536 || k0 < 65536 || v0 < 65536 || q1 > hi || k1 > hi || v1 > hi)
        return fail(SPT_ERR_UNSUPPORTED, "Q, K or V outside the device address range of buffer descriptors");
    if ((o0 < q1 && q0 < o1) || (o0 < k1 && k0 < o1) || (o0 < v1 && v0 < o1))
        return fail(SPT_ERR_INVALID, "O overlaps Q, K or V");
    const double c = (double)scale * 1.4426950408889634;  // log2(e)
    const hipError_t err = launch_attention(dtype, (int)D, variant, stages, Q, K, V, O, (int)BH, (int)Sq, (int)Sk,
                                            (float)c, (hipStream_t)stream);
    if (err != hipSuccess) return fail(SPT_ERR_LAUNCH, "launch failed: %s", hipGetErrorString(err));
    return SPT_OK;
}

// Every entry point returns through here: the thread's message describes its
// most recent call, and is empty when that call succeeded.
static int done(int status)
{
    if (status == SPT_OK) g_last_error[0] = 0;
    return status;
}

}  // namespace spt

extern "C" {

int spt_attention(int64_t BH, int64_t Sq, int64_t Sk, int64_t D, const void* Q, const void* K, const void* V,
                  void* O, float scale, int dtype, void* stream, int variant, int stages)
{
    return spt::done(spt::attention_impl(BH, Sq, Sk, D, Q, K, V, O, scale, dtype, stream, variant, stages));
}


int spt_scale_by_two(int64_t n, const void* x, void* y, int stages, int blocks, void* stream)
{
    return spt::done(spt::scale_by_two_impl(n, x, y, stages, blocks, stream));
}


int spt_gemm(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
             void* C, int64_t ldc, int dtype, void* stream)
{
    return spt::done(spt::gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream, SPT_ROW, SPT_VARIANT_AUTO, 0,
                                    SPT_TILE_AUTO));
}

int spt_gemm_ex(int64_t M, int64_t N, int64_t K, const void* A, int64_t lda, const void* B, int64_t ldb,
                void* C, int64_t ldc, int dtype, void* stream, int b_layout, int variant, int stages,
                int tile_id)
{
    return spt::done(spt::gemm_impl(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream, b_layout, variant, stages,
                                    tile_id));
}

int spt_plan(int dtype, int64_t M, int64_t N, int64_t K, int b_layout, int variant, int stages,
             int tile_id, spt_plan_info* out)
{
    if (!out) return spt::fail(SPT_ERR_INVALID, "out is null");
    return spt::done(spt::make_plan(dtype, M, N, K, b_layout, variant, stages, tile_id, out));
}

const char* spt_status_string(int status)
{
    switch (status) {
    case SPT_OK: return "SPT_OK";
    case SPT_ERR_INVALID: return "SPT_ERR_INVALID";
    case SPT_ERR_UNSUPPORTED: return "SPT_ERR_UNSUPPORTED";
    case SPT_ERR_MISALIGNED: return "SPT_ERR_MISALIGNED";
    case SPT_ERR_LAUNCH: return "SPT_ERR_LAUNCH";
    default: return "SPT_ERR_UNKNOWN";
    }
}

const char* spt_last_error(void) { return spt::g_last_error; }

int spt_version(void) { return SPT_VERSION; }

}  // extern "C"
