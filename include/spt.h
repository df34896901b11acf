/*
 * spt.h -- software-pipelined tiled GEMM for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libspt.so.  Plain pointers and sizes only.
 *
 * The operation.  "Hiding Memory Latency in CUDA: Asynchronous Loads and
 * Software Pipelines" (introduction) states the problem: a tiled GEMM in
 * which each workgroup repeatedly loads a tile of A and B from global
 * memory, stages it in shared memory (here: LDS), loads fragments into
 * registers, runs matrix-core multiply-accumulates and advances to the next
 * K tile.  Every entry point below computes
 *
 *        C[i][j] = sum_{k<K} A[i][k] * B[k][j]     (0 <= i < M, 0 <= j < N)
 *
 * overwriting C (no alpha/beta scaling).  K = 0 writes zeros.  M = 0 or
 * N = 0 returns SPT_OK without launching anything.
 *
 * Element types.  SPT_F16 (IEEE binary16) and SPT_BF16 (bfloat16) inputs
 * accumulate in fp32 and write fp32 C; SPT_I8 inputs accumulate in int32
 * and write int32 C (exact; K <= 131071 so no partial sum can overflow);
 * SPT_F32 inputs accumulate in fp32 and write fp32 C.
 *
 * Layouts.  A is row-major M x K: element (i,k) at A[i*lda + k], lda >= K.
 * B is row-major K x N (SPT_ROW): element (k,j) at B[k*ldb + j], ldb >= N,
 * or column-major (SPT_COL): element (k,j) at B[j*ldb + k], ldb >= K.
 * C is row-major M x N: element (i,j) at C[i*ldc + j], ldc >= N.  Only the
 * M x N elements of C are written; the rest of each row of C is untouched.
 *
 * Alignment.  A, B and C must be 16-byte aligned and every row pitch must be
 * a whole number of 16-byte units (lda*elt, ldb*elt, ldc*4 divisible by 16),
 * else SPT_ERR_MISALIGNED.  Operands are read in 16-byte units that never
 * cross a row's pitch: the library may read A up to M*lda elements, B up to
 * K*ldb (row-major) or N*ldb (column-major) elements; padding beyond K or N
 * never enters the result.
 *
 * Aliasing.  C must not share a byte with the used part of A (from A to the
 * end of row M-1's first K elements) or of B (to the end of the last used
 * row or column); such calls return SPT_ERR_INVALID.  A and B may overlap.
 *
 * Ownership.  All matrix pointers are DEVICE pointers owned by the caller.
 * The library never allocates or frees device memory and keeps no pointer
 * after a call returns.  `stream` is a hipStream_t (NULL = the null
 * stream) of the calling thread's current HIP device, which must also hold
 * the matrices.  A GEMM is one kernel launch, or two in stream order where
 * spt_plan reports a row band (band_tile > 0); launches are asynchronous and
 * the call never synchronizes.  SPT_ERR_LAUNCH carries the status of this
 * call's own launches, not an error left over from earlier HIP calls (if the
 * band's launch fails, C holds only rows [0, band_m)).
 * The library keeps no mutable global state apart from a thread-local
 * message for spt_last_error(); concurrent calls from several threads are
 * safe.
 *
 * Errors.  Every entry point returns an int status and never aborts.
 * Arguments are validated before any HIP call, so invalid calls return
 * without touching a device.
 */
#ifndef SPT_H
#define SPT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPT_VERSION 10100 /* 1.1.0 = major*10000 + minor*100 + patch */

/* Element type of A and B (C is fp32, or int32 for SPT_I8). */
enum spt_dtype { SPT_F16 = 0, SPT_BF16 = 1, SPT_I8 = 2, SPT_F32 = 3 };

/* Storage order of B. */
enum spt_layout { SPT_ROW = 0, SPT_COL = 1 };

/*
 * Global->LDS producer of the K-loop.
 *  SYNC    the sequential load-sync-compute-sync loop ("Hiding Memory
 *          Latency ...", section 1; "Pipeline GPU Kernel", Schritt 1): the
 *          unpipelined baseline, one LDS stage only.
 *  REG     register-staged prefetch ("Pipeline GPU Kernel", Schritt 2 and 3,
 *          the LDG-register variant): tile k+1 is loaded global->VGPR while
 *          tile k is computed, then written VGPR->LDS between barriers;
 *          1 LDS stage (register-only prefetch) or 2 (double buffer).
 *  DIRECT  asynchronous global->LDS copies (the pages' cp.async variant,
 *          on CDNA4 the buffer_load ... lds instruction, which bypasses the
 *          VGPRs), in an S-stage LDS ring with S = 2, 3 or 4 ("Hiding Memory
 *          Latency ...", sections 5 and 6).
 *  PERSIST the DIRECT ring run by persistent workgroups, two per CU (at
 *          most 512), each walking a stream of output tiles ("Hiding Memory
 *          Latency ...", section 8, closing remark on independent tile
 *          streams).  The ring runs on across tile boundaries, and each wave
 *          keeps two accumulator sets, so that the C store of one tile is
 *          issued during the K-loop of the next instead of after it (the
 *          epilogue of section 5 taken off the critical path).  Only the
 *          SPT_TILE_128x128 tile; only shapes with M % 128 == 0, N % 128 ==
 *          0, K % BK == 0 and an even number K / BK >= 2 of K tiles (>= 4
 *          for a 4-stage ring); SPT_ERR_UNSUPPORTED otherwise.  Never
 *          chosen by AUTO: on MI355X it measures slower than DIRECT (a
 *          wave's stores and copies share one in-order completion counter,
 *          so the ring's waits also wait for the overlapped stores).
 *  AUTO    the library's choice for the shape.
 * Valid (variant, stages) pairs: SYNC x 1, REG x {1,2}, DIRECT x {2,3,4},
 * PERSIST x {2,3,4};
 * a ring of S stages must fit in the 160 KiB of LDS (SPT_ERR_UNSUPPORTED
 * otherwise), except that DIRECT x 3 on the 256 x 256 x 128-byte tiles
 * (SPT_TILE_256x256, SPT_TILE_256x256_4W) runs as 5 half-stage slots of
 * 32 KiB (spt_plan_info.half_stage_slots).  stages = 0 picks the variant's
 * default (SYNC 1, REG 2, DIRECT 2 for tiles with a 128-byte K depth, else 3;
 * PERSIST 3).
 */
enum spt_variant {
    SPT_VARIANT_AUTO = 0,
    SPT_VARIANT_SYNC = 1,
    SPT_VARIANT_REG = 2,
    SPT_VARIANT_DIRECT = 3,
    SPT_VARIANT_PERSIST = 4
};

/*
 * Workgroup tile menu.  The K depth of a tile is 64 bytes of each row (BK =
 * 32 for fp16/bf16, 64 for int8, 16 for fp32) or 128 bytes (twice that).
 *  SPT_TILE_128x256  128 x 256, 64-byte K depth, 256 threads (2 x 2 waves
 *                    of 64 x 128): the tile of "Hiding Memory Latency ...",
 *                    section 6.
 *  SPT_TILE_256x256  256 x 256, 128-byte K depth, 512 threads (2 x 4 waves
 *                    of 128 x 64).
 *  SPT_TILE_128x128  128 x 128, 64-byte K depth, 256 threads (2 x 2 waves
 *                    of 64 x 64).
 *  SPT_TILE_256x256_4W  256 x 256, 128-byte K depth, 256 threads (2 x 2
 *                    waves of 128 x 128, one wave per SIMD).  AUTO picks it
 *                    for exact-fit shapes only; requested for other shapes,
 *                    or with the SYNC / REG producers, it runs forms that
 *                    spill registers (correct, but slower).
 *  SPT_TILE_256x256_4W_K64B  the same with a 64-byte K depth (room for a
 *                    3- or 4-stage ring; its int8 3- and 4-stage rings spill
 *                    too, and AUTO never picks them).
 *  SPT_TILE_256x192  256 x 192, 128-byte K depth, 512 threads (2 x 4 waves
 *                    of 128 x 48): fills a round of CUs that the 256 x 256
 *                    grid of a shape would leave partly idle.
 */
enum spt_tile {
    SPT_TILE_AUTO = 0,
    SPT_TILE_128x256 = 1,
    SPT_TILE_256x256 = 2,
    SPT_TILE_128x128 = 3,
    SPT_TILE_256x256_4W = 4,
    SPT_TILE_256x256_4W_K64B = 5,
    SPT_TILE_256x192 = 6
};

enum spt_status {
    SPT_OK = 0,
    SPT_ERR_INVALID = -1,     /* negative size, null pointer, pitch too small, bad enum, C overlapping
                                 A or B */
    SPT_ERR_UNSUPPORTED = -2, /* (variant, stages, tile, dtype, layout) not built; int8 K > 131071;
                                 more than 2^31 - 4097 output tiles;
                                 an operand panel too large for 32-bit buffer offsets; A or B
                                 below 64 KiB or at or above 2^47 (the 48-bit base of a buffer
                                 descriptor) */
    SPT_ERR_MISALIGNED = -3,  /* pointer or row pitch not a multiple of 16 bytes */
    SPT_ERR_LAUNCH = -4       /* the HIP launch reported an error */
};

/* What a call would launch, and the LDS / occupancy / ratio figures of that
 * plan ("Pipeline GPU Kernel", Schritt 1 and 2; "Kernel-Engpass
 * analysieren", Schritt 3 and 6), evaluated for gfx950. */
typedef struct spt_plan_info {
    int32_t dtype, b_layout, variant, stages, tile_id;
    int32_t BM, BN, BK;             /* workgroup tile, K depth in elements */
    int32_t threads, waves;         /* per workgroup (64-wide waves) */
    int32_t wave_m, wave_n;         /* per-wave output tile */
    int32_t elt_bytes;              /* bytes per A/B element */
    int64_t tiles_m, tiles_n;       /* workgroup tiles along M and N */
    int64_t grid;                   /* workgroups launched: tiles_m * tiles_n (PERSIST: at most 512) */
    int64_t k_tiles;                /* ceil(K / BK) */
    int64_t k_full_tiles;           /* floor(K / BK) */
    int32_t k_tail;                 /* K mod BK: width of the zero-filled last tile (0 = none) */
    int32_t a_stage_bytes;          /* BM*BK*elt */
    int32_t b_stage_bytes;          /* BK*BN*elt */
    int32_t stage_bytes;            /* a + b */
    int32_t lds_bytes;              /* stages * stage_bytes (LDS per workgroup; half_stage_slots *
                                       a_stage_bytes for a half-stage ring) */
    int32_t a_copies_per_thread;    /* 16-byte accesses per thread per stage */
    int32_t b_copies_per_thread;
    int32_t wg_per_cu_lds;          /* floor(163840 / lds_bytes): the LDS limit per CU */
    int32_t waves_per_simd_lds;     /* wg_per_cu_lds * waves / 4 */
    int32_t steady_vmcnt;           /* loads that may stay in flight at the steady-state wait */
    int32_t mfma_per_ktile_per_wave;
    double ratio_flop_per_byte;     /* 2*BM*BN*BK / ((BM*BK + BK*BN)*elt) */
    double ratio_mfma_per_load;     /* MFMA instructions per global load instruction, per wave */
    int32_t store_window;           /* PERSIST: K tiles (2, 4 or 8) over which a wave writes the
                                       previous output tile (16 / store_window stores per K tile);
                                       else 0 */
    int32_t tiles_per_wg;           /* output tiles per workgroup: ceil(tiles_m * tiles_n / grid) */
    /* Row band of a last, nearly empty round (AUTO choice only: tile, variant
       and stages all 0; K of at least 2 KiB per row).  When band_tile > 0,
       `grid` workgroups compute rows [0, band_m) of C as above, then, in stream
       order, band_grid workgroups of the 128 x 128 tile (DIRECT ring of
       band_stages stages: 4 for at most 256 workgroups and K of at least
       8 KiB per row, else 3) compute rows
       [band_m, M): two launches.  Each output is the same sum in
       the same order either way.  band_tile = 0: one launch, band_m = M. */
    int32_t band_tile;
    int32_t band_stages;
    int64_t band_m;
    int64_t band_grid;
    /* 1: the DIRECT ring copies the partial last K tile itself, zero-filled past K
       per 16-byte chunk ("Hiding Memory Latency ...", section 8: a partial tile's
       copy fills what lies outside the source with zeros); this needs k_tail * elt
       to be a multiple of 16 and a tile other than the 256 x 256 ones.  0: a
       partial tile (if any) is loaded through VGPRs with every element past K
       zeroed, after the ring. */
    int32_t tail_ring;
    /* DIRECT rings whose S full stages exceed the 160 KiB of LDS, on a tile whose A and
       B parts are the same size (S = 3 on the 256 x 256 x 128-byte tiles): 2S - 1, the
       ring runs as that many half-stage slots, each holding the A or the B part of one
       K tile, and lds_bytes = (2S - 1) * a_stage_bytes.  Copies of the half stage after
       the next K tile stay in flight at each wait (steady_vmcnt), where a 2-stage ring
       drains them ("Hiding Memory Latency ...", section 6: deeper pipelines keep more
       copies in flight).  0 otherwise. */
    int32_t half_stage_slots;
} spt_plan_info;

/* C = A*B with B row-major, the library's choice of tile and variant. */
int spt_gemm(int64_t M, int64_t N, int64_t K,
             const void* A, int64_t lda,
             const void* B, int64_t ldb,
             void* C, int64_t ldc,
             int dtype, void* stream);

/* C = A*B with an explicit B layout (spt_layout), producer variant
 * (spt_variant), LDS stage count (0 = variant default) and tile (spt_tile). */
int spt_gemm_ex(int64_t M, int64_t N, int64_t K,
                const void* A, int64_t lda,
                const void* B, int64_t ldb,
                void* C, int64_t ldc,
                int dtype, void* stream,
                int b_layout, int variant, int stages, int tile_id);

/* Fill *out with the plan spt_gemm_ex would launch for these arguments.
 * Pure host computation; needs no device.  Same status codes as
 * spt_gemm_ex for the shape arguments. */
int spt_plan(int dtype, int64_t M, int64_t N, int64_t K,
             int b_layout, int variant, int stages, int tile_id,
             spt_plan_info* out);

/*
 * y[i] = 2 * x[i] for 0 <= i < n: the streaming pipeline of "Hiding Memory
 * Latency ...", section 8 (the minimal working example) and section 9, on
 * gfx950.  x and y are DEVICE pointers to float32 arrays owned by the caller,
 * 16-byte aligned (SPT_ERR_MISALIGNED otherwise); y may be x itself (in
 * place) but must not overlap it otherwise (SPT_ERR_INVALID).  Tiles of 1024
 * elements are staged global -> LDS through a ring of `stages` stages (1 =
 * the synchronous loop, 2..4 = asynchronous copies; 0 = 3, the page's
 * choice); each of `blocks` workgroups of 256 threads walks its own stream of
 * tiles (0 = the library's choice: 1024 / 768 / 512 / 256 for 1 / 2 / 3 / 4
 * stages, never more than there are tiles; 1 = the page's single-block
 * demonstration).
 * Every result is exact (doubling is exact in float).  n = 0 returns SPT_OK
 * without launching; n < 0, stages outside 0..4 or blocks < 0 give
 * SPT_ERR_INVALID; n > 2^40 gives SPT_ERR_UNSUPPORTED.  Asynchronous on
 * `stream`, like spt_gemm.
 */
int spt_scale_by_two(int64_t n, const void* x, void* y, int stages, int blocks, void* stream);

/*
 * Attention forward pass, the high-ratio consumer of the same ring: for each
 * of BH independent (batch, head) slices,
 *
 *        O[i][d] = sum_j softmax_j(scale * sum_e Q[i][e] * K[j][e]) * V[j][d]
 *
 * (no mask).  "Kernel-Engpass analysieren" uses flash attention as its
 * example of a kernel with many matrix instructions per tile load (Schritt 4,
 * and the pitfalls section, where asynchronous copies measured a few percent
 * slower) and counts its work as 4 * BH * Sq * Sk * D FLOP (Schritt 1).
 * Key/value blocks stream through the producer `variant` (SPT_VARIANT_SYNC
 * with 1 stage, SPT_VARIANT_REG with 1-2, SPT_VARIANT_DIRECT with 2-3;
 * SPT_VARIANT_AUTO picks DIRECT; stages 0 picks two for REG and DIRECT),
 * the online softmax runs in fp32, and the probabilities are rounded to the
 * input type for the second product; each row is divided by the sum of
 * those rounded probabilities.
 *
 * dtype SPT_F16 or SPT_BF16 for Q, K, V; O is fp32.  D (head dimension) is 64
 * or 128.  Layouts (contiguous, DEVICE pointers owned by the caller, 16-byte
 * aligned): Q [BH][Sq][D], K and V [BH][Sk][D], O [BH][Sq][D].  O must not
 * overlap Q, K or V.  scale must be finite and >= 0 (the usual 1/sqrt(D) is
 * the caller's to pass).  Errors: SPT_ERR_INVALID (negative size, Sk = 0 with
 * work to do -- a softmax over no keys --, null pointer, bad scale, enum
 * out of range, overlap), SPT_ERR_UNSUPPORTED (dtype, D, a variant/stage
 * pairing, sizes above 2^31-1, one slice's K or V above 2^31 bytes
 * (Sk * D * 2), addresses outside the 48-bit range of buffer descriptors),
 * SPT_ERR_MISALIGNED, SPT_ERR_LAUNCH.  BH = 0 or Sq = 0 returns
 * SPT_OK without launching.  Asynchronous on `stream`, like spt_gemm.
 */
int spt_attention(int64_t BH, int64_t Sq, int64_t Sk, int64_t D,
                  const void* Q, const void* K, const void* V, void* O,
                  float scale, int dtype, void* stream, int variant, int stages);

/* Static string naming a status code. */
const char* spt_status_string(int status);

/* Thread-local detail of this thread's most recent call to the entry points
 * above: a message if it failed, "" if it returned SPT_OK or none was made. */
const char* spt_last_error(void);

/* SPT_VERSION of the loaded library. */
int spt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPT_H */
