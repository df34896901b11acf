// spt_kernel.hpp -- the software-pipelined tiled GEMM K-loop for gfx950.
//
// One workgroup owns one BM x BN tile of C and walks K in BK-deep tiles.
// Each K tile of A (BM x BK) and B (BK x BN) is staged global -> LDS and
// consumed by matrix-core MFMAs, following "Hiding Memory Latency in CUDA:
// Asynchronous Loads and Software Pipelines" (introduction, sections 5-7)
// and "Pipeline GPU Kernel" (Schritt 1-4).  Three producer variants:
//
//  V_SYNC    load -> barrier -> compute -> barrier, one LDS stage (the
//            sequential loop of section 1 / Schritt 1): the unpipelined
//            baseline.
//  V_REG     register-staged prefetch (the LDG-register variant of
//            Schritt 2/3): tile t+1 is fetched global -> VGPR with
//            buffer_load_dwordx4 while tile t is computed, then written
//            VGPR -> LDS with ds_write_b128.  S = 1 (one LDS buffer, the
//            register-only prefetch of Schritt 1) or S = 2 (double buffer).
//  V_DIRECT  asynchronous global -> LDS copies (the pages' cp.async, on CDNA4
//            buffer_load_dwordx4 ... lds, which writes LDS without a VGPR
//            round trip) into an S-stage ring, S = 2, 3 or 4 (sections 5, 6),
//            with a second, register-level pipeline of LDS -> VGPR fragment
//            reads (section 7).
//
// V_DIRECT schedule.  Fragments of one MFMA k-step of the wave tile sit in
// one of two register slots.  For K tile t with KS k-steps:
//     steps s < KS-1:  read the fragments of step s+1 into the free slot,
//                      interleaved with the MFMAs of step s;
//     last step:       s_waitcnt lgkmcnt(0)   -- this wave's reads of tile t
//                                                are complete,
//                      s_waitcnt vmcnt(n)     -- this wave's copies of tile
//                                                t+1 have landed (n: the
//                                                copies of younger tiles that
//                                                may stay in flight),
//                      s_barrier              -- every wave is past both
//                                                waits: tile t+1 is visible
//                                                and tile t's stage is free,
//                      then, interleaved with the MFMAs of the last step of
//                      tile t (whose operands are already in registers):
//                      the copies of tile t+S into tile t's stage, and the
//                      reads of step 0 of tile t+1 into the free slot.
// The prologue fills all S stages (tiles past the end of K are empty copies
// that move no memory).  The register slots act as one more
// stage, so one barrier per K tile serves both obligations of section 4
// (never expose a stage early, never release one early), the MFMA pipe
// always has independent work while loads are in flight, and S tiles of
// copies overlap the compute ("keep every level fed", section 7).
//
// vmcnt is the CDNA4 counterpart of cp.async.wait_group (section 3): the
// copies of one wave complete in issue order, so "at most N outstanding"
// means "every copy older than the N newest has landed".
//
// LDS layout.  K-contiguous tiles (A, column-major B) keep whole rows, with
// the 16-byte chunk index XOR-swizzled by row bits so that the fragment reads
// (ds_read_b128, 16 rows x one chunk per lane group) are bank-conflict free
// while every 1 KiB copy still covers whole row segments (full 128-byte
// lines when a K tile row is 128 bytes: copies of half lines run at two
// thirds of the rate).  Row-major B is either kept as swizzled k-rows (read
// by ds_read_b64_tr_b16 / tr_b8, full-line copies) or in "lane order": one
// block per transposing read, holding the data in the order of the lanes that
// read it (conflict free, half-line copies).  The producer computes which
// global 16-byte chunk belongs at each position.
//
// K tails: full tiles use 16-byte copies; the last partial tile (K mod BK
// elements) is loaded through VGPRs, and every element at k >= K is set to
// zero before it is written to LDS (the zero fill of section 8 and of
// Schritt "Boundary-Handhabung").  M / N edges clamp the source row into
// range; those rows only feed outputs that are never stored.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "spt_config.h"

namespace spt {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
#define SPT_LDS __attribute__((address_space(3)))

// ---------------------------------------------------------------------------
// Synchronisation.  Inline asm with a memory clobber: the compiler neither
// moves LDS / global accesses across these points nor adds waits of its own.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt is a 6-bit counter");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void barrier() { asm volatile("s_barrier" ::: "memory"); }
// Keep the instruction order written in the source around this point.
__device__ __forceinline__ void order_fence() { __builtin_amdgcn_sched_barrier(0); }

// f(integral_constant<int, I>) for I = B .. E-1, expanded at compile time (a
// `#pragma unroll` loop may be left rolled when its body is large, and a
// rolled loop would index the accumulator array at run time).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------
// EXACT_: M, N and K are multiples of the tile (no K tail, no edge checks in
// the epilogue); the dispatcher selects it only for such shapes.
// BLANE_: row-major B kept in the lane layout (fp32 B always is).
template <int DT_, bool BCOL_, int TILE_, int V_, int S_, bool EXACT_ = false, bool BLANE_ = false>
struct Cfg {
    static constexpr int DT = DT_;
    static constexpr bool BCOL = BCOL_;
    static constexpr bool EXACT = EXACT_;
    static constexpr bool BLANE = BLANE_ || elt_bytes(DT_) == 4;
    static constexpr int TILE = TILE_, V = V_, S = S_;
    static constexpr bool RING_TAIL = V_ == V_DIRECT && !EXACT_ && ring_tail_tile(TILE_);  // see GemmArgs::tail_ring
    static constexpr int BM = kTiles[TILE_].BM, BN = kTiles[TILE_].BN;
    static constexpr int ELT = elt_bytes(DT_);
    static constexpr int CE = 16 / ELT;           // elements per 16-byte chunk
    static constexpr int BK = kTiles[TILE_].BKB / ELT;
    static constexpr int WAVES_M = kTiles[TILE_].WAVES_M, WAVES_N = kTiles[TILE_].WAVES_N;
    static constexpr int WAVES = WAVES_M * WAVES_N, THREADS = 64 * WAVES;
    static constexpr int WTM = BM / WAVES_M, WTN = BN / WAVES_N;  // wave tile
    static constexpr int FM = WTM / 16, FN = WTN / 16;             // 16x16 MFMA tiles per wave
    static constexpr int KSTEP = 4 * CE;  // k per MFMA step: 4 lane groups x one 16-byte chunk
    static constexpr int KS = BK / KSTEP;  // MFMA k-steps per K tile
    static constexpr int MB = BM / 16, NB = BN / 16;  // 16-row / 16-column blocks
    static constexpr int A_BYTES = BM * BK * ELT;
    static constexpr int B_BYTES = BK * BN * ELT;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Half-stage ring: S full stages of a tile whose A and B parts are the same size
    // that do not fit in LDS (3 x 64 KiB for the 256 x 256 x 128-byte tiles) run as
    // 2S - 1 half-stage slots instead, each holding the A or the B part of one K tile.
    // Ring position 2t holds A of tile t, 2t + 1 its B, in slot (position mod 2S - 1).
    static constexpr bool SPLIT = V_ == V_DIRECT && A_BYTES == B_BYTES && S_ * STAGE_BYTES > kLdsPerCu &&
                                  (2 * S_ - 1) * A_BYTES <= kLdsPerCu;
    static constexpr int SLOTS = SPLIT ? 2 * S_ - 1 : 2 * S_;  // half-stage slots of the ring
    static constexpr int LDS_BYTES = SPLIT ? SLOTS * A_BYTES : S * STAGE_BYTES;
    static constexpr int A_CPT = A_BYTES / 16 / THREADS;  // 16-byte copies per thread per stage
    static constexpr int B_CPT = B_BYTES / 16 / THREADS;
    static constexpr int LOADS = A_CPT + B_CPT;            // vmcnt units per tile per thread
    // Copies of younger tiles that may stay in flight per thread: at the wait that
    // closes a K tile (the next tile must have landed) and after the prologue (tile
    // 0 must have landed).  A half-stage ring issues B of a tile before A of the
    // next one, so one half stage (A of the tile after next) stays in flight.
    static constexpr int VM_STEADY = SPLIT ? (SLOTS - 4) * A_CPT : (S_ - 2) * LOADS;
    static constexpr int VM_FIRST = SPLIT ? (SLOTS - 2) * A_CPT : (S_ - 1) * LOADS;
    // 16x16 wave tiles of 128 x 128 need the whole register file: one wave per
    // SIMD; so does a ring that leaves LDS for one workgroup of four waves per CU
    static constexpr int WG_PER_CU_LDS = kLdsPerCu / LDS_BYTES;
    // (V_PERSIST keeps two accumulator sets per wave: twice the accumulators)
    static constexpr int WAVES_PER_SIMD =
        ((V_ == V_PERSIST ? 2 : 1) * FM * FN > 32 || WG_PER_CU_LDS * WAVES < 8) ? 1 : 2;

    static_assert(BK % KSTEP == 0, "BK must hold whole MFMA steps");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0,
                  "a stage must split into whole 1 KiB copies per wave");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must hold whole 16x16 MFMA tiles");
    static_assert(LDS_BYTES <= kLdsPerCu, "LDS ring exceeds 160 KiB");
    static_assert(V_ != V_SYNC || S_ == 1, "SYNC has one stage");
    static_assert(V_ != V_REG || (S_ == 1 || S_ == 2), "REG has 1 or 2 stages");
    static_assert(V_ != V_DIRECT || (S_ >= 2 && S_ <= 4), "DIRECT has 2 to 4 stages");
    static_assert(!SPLIT || (!RING_TAIL && A_CPT == B_CPT), "half-stage rings: equal halves, no in-ring tail");
    static_assert(V_ != V_PERSIST || (S_ >= 2 && S_ <= 4 && EXACT_), "PERSIST: exact-fit 2- to 4-stage rings");
    static_assert((S_ - 1) * LOADS < 64, "vmcnt range");
};

// Accumulators are float vectors for every element type; int8 keeps its
// int32 sums in them bit for bit (bit casts around its MFMA).  With the same
// <4 x i32> type for operands and accumulators, the register allocator
// rotated int8 accumulators across the back edge of the 256 x 256 loop (72
// accumulator copies per iteration; 36 with float vectors, and the loop 2%
// faster, measured on MI355X).
template <int DT>
struct AccT {
    typedef f32x4_t type;
};

// acc += X * Y with X the B fragment and Y the A fragment (operands swapped so
// that each lane ends up holding 4 consecutive columns of one row of C).
template <int DT>
__device__ __forceinline__ void mma(typename AccT<DT>::type& acc, i32x4_t x, i32x4_t y)
{
    if constexpr (DT == DT_F16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, x),
                                                     __builtin_bit_cast(f16x8_t, y), acc, 0, 0, 0);
    } else if constexpr (DT == DT_BF16) {
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, x),
                                                      __builtin_bit_cast(bf16x8_t, y), acc, 0, 0, 0);
    } else if constexpr (DT == DT_I8) {
        acc = __builtin_bit_cast(
            f32x4_t, __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, __builtin_bit_cast(i32x4_t, acc), 0, 0, 0));
    } else {
        // fp32: a chunk holds 4 consecutive k per lane group; MFMA j takes element j,
        // so lane group g supplies k = 4g + j to both operands.  (Whole-vector bit
        // casts: a bit cast of one vector element does not honour the index.)
        const f32x4_t xf = __builtin_bit_cast(f32x4_t, x), yf = __builtin_bit_cast(f32x4_t, y);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(xf[j], yf[j], acc, 0, 0, 0);
    }
}

__device__ __forceinline__ long long min64(long long a, long long b) { return a < b ? a : b; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// One asynchronous 16-byte-per-lane copy global -> LDS (buffer_load_dwordx4
// ... lds): lane l's 16 bytes at rsrc + voffset + OFF land at LDS byte
// lds + OFF + 16*l (the immediate offset applies to both addresses, checked
// on gfx950).  `lds` must be wave-uniform.  Written as inline asm so that the
// compiler does not guard later LDS reads with waits of its own (it cannot
// tell the ring stages apart and would drain every copy in flight); the
// ring's s_waitcnt vmcnt + s_barrier placement is the only synchronisation.
// M0 carries the LDS address.  NOP: the s_nop covering the M0-write ->
// LDS-DMA hazard, needed by the first copy after M0 takes a new value; the
// copies that follow in a group see the same M0 value.
template <int OFF, bool NOP>
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds, int voffset)
{
    static_assert(OFF >= 0 && OFF < 4096, "12-bit immediate offset");
    if constexpr (NOP)
        asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds"
                     :
                     : "v"(voffset), "s"(rsrc), "{m0}"(lds), "n"(OFF)
                     : "memory");
    else
        asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:%3 lds"
                     :
                     : "v"(voffset), "s"(rsrc), "{m0}"(lds), "n"(OFF)
                     : "memory");
}

// Zero the bytes of a 16-byte chunk from byte `valid` on (little-endian: the
// low bytes hold the lower k).
__device__ __forceinline__ i32x4_t keep_bytes(i32x4_t v, int valid)
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const int vb = valid - 4 * d;
        const uint32_t keep = vb >= 4 ? 0xffffffffu : vb <= 0 ? 0u : ((1u << (8 * vb)) - 1u);
        v[d] = (int)((uint32_t)v[d] & keep);
    }
    return v;
}

// ---------------------------------------------------------------------------
template <class C>
struct Gemm {
    typedef typename AccT<C::DT>::type acc_t;
    typedef i32x4_t Slot[C::FM + C::FN];  // one k-step of A (FM) and B (FN) fragments

    // ---- LDS layout --------------------------------------------------------
    // K-contiguous tiles (A; column-major B): rows of RK = BK * ELT bytes
    // (NCK 16-byte chunks), chunk c of row r at chunk position c ^ swz_k(r).
    // Rows stay whole in LDS, so one 1 KiB copy covers 1024 / RK full row
    // segments; the XOR keeps the fragment reads (16 rows x one chunk) free of
    // bank conflicts on gfx950 (measured with the LDS bank-conflict counter).
    static constexpr int RK = C::BK * C::ELT, NCK = RK / 16;
    static_assert(NCK == 4 || NCK == 8, "K-contiguous rows of 64 or 128 bytes");
    static __device__ __forceinline__ constexpr int swz_k(int r) { return (r >> 1) & (NCK - 1); }
    // Row-major B, row layout: k-rows of RN = BN * ELT bytes (NCN chunks), chunk
    // c of k-row r at c ^ swz_n(r); read by ds_read_b64_tr_b16 / tr_b8.
    static constexpr int RN = C::BN * C::ELT, NCN = RN / 16;
    // The XOR permutes chunks within groups of SWG: 8, or 4 for int8 k-rows of 12
    // chunks (the 192-column tile), which hold no whole group of 8.  16-bit k-rows
    // of a whole number of 256-byte bank lines (16 chunks) XOR the chunk pair with
    // k-row bits 0, 1 and 3: the 8 k-rows one half-wave of a transposing read
    // touches (8g + 0..3 for g = 0, 1; 16 + 8g' + 0..3) then sit in 8 different
    // 32-byte bank groups.  With bits 0 and 1 alone, k-rows r and r + 8 shared
    // their banks: two conflict cycles per read (SQ_LDS_BANK_CONFLICT on MI355X).
    static constexpr bool WIDE16 = C::ELT == 2 && NCN % 16 == 0;
    static constexpr int SWG = WIDE16 ? 16 : (C::ELT == 1 && NCN % 8 != 0) ? 4 : 8;
    static __device__ __forceinline__ constexpr int swz_n(int r)
    {
        return WIDE16 ? (((r & 3) | ((r >> 1) & 4)) << 1) : C::ELT == 2 ? ((r & 3) << 1) : (r & (SWG - 1));
    }
    static_assert(C::BCOL || C::BLANE || NCN % SWG == 0, "the k-row swizzle permutes chunks within groups");
    // Row-major B, lane layout: block (nb, s, h) of 64 lanes x (8 | 8 | 4) bytes
    // in the order of the lanes of one ds_read_b64_tr_b16 / tr_b8 / ds_read_b32.
    static constexpr int BR_BLOCK = C::ELT == 4 ? 256 : 512;
    static constexpr int BR_SUB = C::ELT == 4 ? 4 : 2;  // blocks per (nb, s)
    static constexpr int br_block(int nb, int s, int h)
    {
        return C::A_BYTES + ((s * BR_SUB + h) * C::NB + nb) * BR_BLOCK;
    }

    // Stage chunk q of the A region -> (row, k) of the tile it holds.
    static __device__ __forceinline__ void a_src(int q, int& row, int& k)
    {
        row = q / NCK;
        k = ((q % NCK) ^ swz_k(row)) * C::CE;
    }
    // Stage chunk q of the B region -> (k, n) of the tile it holds.
    static __device__ __forceinline__ void b_src(int q, int& k, int& n)
    {
        if constexpr (C::BCOL) {
            n = q / NCK;
            k = ((q % NCK) ^ swz_k(n)) * C::CE;
        } else if constexpr (!C::BLANE) {
            k = q / NCN;
            n = ((q % NCN) ^ swz_n(k)) * C::CE;
        } else if constexpr (C::ELT == 2) {
            // lane l = 16 g + i of a tr_b16 read gets k-rows 8g + 4h + (i >> 2) ... at columns
            // 4 (i & 3) .. + 3; a 16-byte chunk c holds lanes 2c, 2c + 1.
            const int blk = q >> 5, c = q & 31;
            const int nb = blk % C::NB, sh = blk / C::NB;
            const int s = sh >> 1, h = sh & 1;
            k = s * C::KSTEP + 8 * (c >> 3) + 4 * h + ((c & 7) >> 1);
            n = 16 * nb + 8 * (c & 1);
        } else if constexpr (C::ELT == 1) {
            // tr_b8: lane 16 g + i gets k-rows 16 g + 8 h + (i >> 1) at columns 8 (i & 1) .. + 7.
            const int blk = q >> 5, c = q & 31;
            const int nb = blk % C::NB, sh = blk / C::NB;
            const int s = sh >> 1, h = sh & 1;
            k = s * C::KSTEP + 16 * (c >> 3) + 8 * h + (c & 7);
            n = 16 * nb;
        } else {
            // fp32, ds_read_b32 t: lane 16 g + j gets k-row 4 g + t at column j.
            const int blk = q >> 4, c = q & 15;
            const int nb = blk % C::NB, st = blk / C::NB;
            const int s = st >> 2, t = st & 3;
            k = s * C::KSTEP + 4 * (c >> 2) + t;
            n = 16 * nb + 4 * (c & 3);
        }
    }

    // Stage chunk (16 bytes) moved by copy i (0 .. cpt-1) of thread tid: each
    // wave's copies cover cpt consecutive 1 KiB blocks of the operand region,
    // one block per copy, lane l at byte 16 l of it.
    static __device__ __forceinline__ constexpr int chunk_of(int i, int tid, int cpt)
    {
        return ((tid >> 6) * cpt + i) * 64 + (tid & 63);
    }

    // ---- fragment reads ---------------------------------------------------------
    // Per-lane LDS byte offsets of this wave's fragments within a stage, for
    // MFMA row 0 / column 0 of the wave tile; other rows / columns add an
    // immediate.  A fragment (m, s): 16 rows x the 16-byte chunk 4s + g.
    // Row layout: the swizzle only permutes column blocks within groups of BQ
    // (4 for tr_b16, 8 for tr_b16 on 16-chunk groups and for tr_b8; the wave's
    // first block is a multiple of BQ), so blocks n and n + BQ sit BQ blocks
    // apart in every k-row and one lane offset per n mod BQ serves all FN blocks.
    static constexpr int BQ_ = C::ELT == 2 && !WIDE16 ? 4 : 8;
    static constexpr int BQ = C::FN % BQ_ == 0 ? BQ_ : C::FN;
    static constexpr int B_OFFS = C::BCOL ? C::KS : (C::BLANE ? 1 : BQ);
    // B's lane offsets count from the start of B's region: A_BYTES into a full stage,
    // 0 into a half-stage slot
    static constexpr int B_OFF = C::SPLIT ? 0 : C::A_BYTES;
    struct Lanes {
        int a[C::KS];
        int b[B_OFFS];
    };
    static __device__ void setup_lanes(int lane, int mb0, int nb0, Lanes& L)
    {
        const int g = lane >> 4, l16 = lane & 15;
        // swz_k(16 mb + l16) == swz_k(l16): the row-block index never reaches the XOR bits
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            L.a[s] = (16 * mb0 + l16) * RK + 16 * ((4 * s + g) ^ swz_k(l16));
            if constexpr (C::BCOL) L.b[s] = B_OFF + (16 * nb0 + l16) * RK + 16 * ((4 * s + g) ^ swz_k(l16));
        }
        if constexpr (!C::BCOL && C::BLANE) {
            L.b[0] = br_block(nb0, 0, 0) - C::A_BYTES + B_OFF + lane * (C::ELT == 4 ? 4 : 8);
        } else if constexpr (!C::BCOL && C::ELT == 2) {
            // tr_b16: lane (g, i) fetches k-row 8g + (i >> 2) (+ 4h + KSTEP s) at columns
            // 4 (i & 3) .. + 3 of column block nb; swz_n only sees k-row bits 0, 1 and 3,
            // which 4h + KSTEP s never change.
#pragma unroll
            for (int n = 0; n < BQ; ++n) {
                const int kr = 8 * g + (l16 >> 2);
                const int c = 2 * (nb0 + n) + ((l16 & 3) >> 1);
                L.b[n] = B_OFF + kr * RN + 16 * (c ^ swz_n(kr)) + 8 * (l16 & 1);
            }
        } else if constexpr (!C::BCOL && C::ELT == 1) {
            // tr_b8: lane (g, i) fetches k-row 16g + (i >> 1) (+ 8h + KSTEP s) at columns
            // 8 (i & 1) .. + 7 of column block nb; swz_n only sees k-row bits 0..2.
#pragma unroll
            for (int n = 0; n < BQ; ++n) {
                const int kr = 16 * g + (l16 >> 1);
                L.b[n] = B_OFF + kr * RN + 16 * ((nb0 + n) ^ swz_n(kr)) + 8 * (l16 & 1);
            }
        }
    }

    static __device__ __forceinline__ i32x4_t read_a(const SPT_LDS char* st, const Lanes& L, int m, int s)
    {
        return *(const SPT_LDS i32x4_t*)(st + L.a[s] + 16 * m * RK);
    }
    static __device__ __forceinline__ i32x4_t read_b(const SPT_LDS char* st, const Lanes& L, int n, int s)
    {
        if constexpr (C::BCOL) {
            return *(const SPT_LDS i32x4_t*)(st + L.b[s] + 16 * n * RK);
        } else if constexpr (C::ELT == 4) {  // lane layout only
            i32x4_t v;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                v[t] = *(const SPT_LDS int*)(st + L.b[0] + (br_block(n, s, t) - C::A_BYTES));
            return v;
        } else {
            int o0, o1;  // the two transposing reads (k-rows +0.. and +4 / +8 ..)
            if constexpr (C::BLANE) {
                o0 = L.b[0] + (br_block(n, s, 0) - C::A_BYTES);
                o1 = L.b[0] + (br_block(n, s, 1) - C::A_BYTES);
            } else {
                o0 = L.b[n % BQ] + (n / BQ) * (BQ * 16 * C::ELT) + s * C::KSTEP * RN;
                o1 = o0 + (C::ELT == 2 ? 4 : 8) * RN;
            }
            if constexpr (C::ELT == 2) {
                typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
                const fp16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS fp16x4_raw*)(st + o0));
                const fp16x4_raw hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS fp16x4_raw*)(st + o1));
                const i32x2_t l2 = __builtin_bit_cast(i32x2_t, lo), h2 = __builtin_bit_cast(i32x2_t, hi);
                return (i32x4_t){l2.x, l2.y, h2.x, h2.y};
            } else {
                const i32x2_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SPT_LDS i32x2_t*)(st + o0));
                const i32x2_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SPT_LDS i32x2_t*)(st + o1));
                return (i32x4_t){lo.x, lo.y, hi.x, hi.y};
            }
        }
    }

    // Per-thread copy geometry (loop invariant): byte offsets of this thread's
    // A and B chunks from the K tile's base.  V_DIRECT copies go in groups of
    // four that share one M0 value: copy i adds the immediate (i mod 4) KiB to
    // both its LDS and its global address, so its register offset is lowered
    // by the same amount, and every offset is raised by DMA_BIAS (the
    // descriptor base is lowered by as much) to keep it non-negative.
    static constexpr int DMA_BIAS = 3072;
    static __device__ __forceinline__ constexpr int dma_bias(int i)
    {
        return (C::V == V_DIRECT || C::V == V_PERSIST) ? DMA_BIAS - (i % 4) * 1024 : 0;
    }
    struct Copy {
        int a_voff[C::A_CPT];
        int b_voff[C::B_CPT];
    };

    static __device__ void setup_copy(const GemmArgs& p, int m0, int n0, int tid, Copy& cp)
    {
        const int rows_a = min(C::BM, p.M - m0);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) {
            int r, k;
            a_src(chunk_of(i, tid, C::A_CPT), r, k);
            r = min(r, rows_a - 1);  // M edge: any in-range row (its outputs are not stored)
            cp.a_voff[i] = r * p.lda * C::ELT + k * C::ELT + dma_bias(i);
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int k, n;
            b_src(chunk_of(i, tid, C::B_CPT), k, n);
            if constexpr (C::BCOL) {
                n = min(n, min(C::BN, p.N - n0) - 1);  // N edge
                cp.b_voff[i] = n * p.ldb * C::ELT + k * C::ELT + dma_bias(i);
            } else {
                if (n0 + n >= p.N) n = 0;  // N edge: any in-range chunk
                cp.b_voff[i] = k * p.ldb * C::ELT + n * C::ELT + dma_bias(i);
            }
        }
    }

    // The partial K tile through the ring (p.tail_ring): before its copies are issued,
    // every copy whose 16-byte chunk lies at k >= k_tail gets an offset past any
    // buffer extent, so it reads zeros ("Hiding Memory Latency ...", section 8: the
    // copy of a partial tile zero-fills what lies outside the source).  Row-major B
    // needs nothing here: its copies of that tile end after k_tail rows (tail_b).
    // The ring copies nothing after that tile, so the offsets stay changed.
    static constexpr int OFF_PAST = (int)0xfffff000u;  // + at most 3 KiB of immediate: past every extent
    static __device__ void mask_tail(const GemmArgs& p, int tid, Copy& cp)
    {
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) {
            int r, k;
            a_src(chunk_of(i, tid, C::A_CPT), r, k);
            if (k >= p.k_tail) cp.a_voff[i] = OFF_PAST;
        }
        if constexpr (C::BCOL) {
#pragma unroll
            for (int i = 0; i < C::B_CPT; ++i) {
                int k, n;
                b_src(chunk_of(i, tid, C::B_CPT), k, n);
                if (k >= p.k_tail) cp.b_voff[i] = OFF_PAST;
            }
        }
    }

    // Tile bases and readable byte counts for K tile t (wave-uniform values).
    // The count covers exactly what the caller guarantees readable from the
    // base: whole row pitches of the rows this tile touches.
    static __device__ __forceinline__ void span_a(const GemmArgs& p, int m0, int t, const char*& base,
                                                  uint32_t& bytes)
    {
        const int rows = min(C::BM, p.M - m0);
        const long long k0 = (long long)t * C::BK;
        base = p.A + ((long long)m0 * p.lda + k0) * C::ELT;
        bytes = (uint32_t)min64(((long long)rows * p.lda - k0) * C::ELT, 0x7ffffff0ll);
    }
    static __device__ __forceinline__ void span_b(const GemmArgs& p, int n0, int t, const char*& base,
                                                  uint32_t& bytes)
    {
        const long long k0 = (long long)t * C::BK;
        if constexpr (C::BCOL) {
            const int cols = min(C::BN, p.N - n0);
            base = p.B + ((long long)n0 * p.ldb + k0) * C::ELT;
            bytes = (uint32_t)min64(((long long)cols * p.ldb - k0) * C::ELT, 0x7ffffff0ll);
        } else {
            const long long rows = min64(C::BK, (long long)p.K - k0);
            base = p.B + (k0 * p.ldb + n0) * C::ELT;
            bytes = (uint32_t)min64((rows * p.ldb - n0) * C::ELT, 0x7ffffff0ll);
        }
    }

    // ---- V_DIRECT producer ---------------------------------------------------
    // Wave-uniform producer state, advanced by a constant per K tile so that
    // the steady loop spends a handful of scalar instructions per tile on it.
    // Every full K tile reads the same extent from its base: the rows (A,
    // column-major B) or k-rows (row-major B) it touches, which the caller
    // guarantees readable and which fits the 31-bit buffer range (the host
    // checks the panel).  Tiles past the last full one get extent 0: empty
    // copies that move nothing and still count in vmcnt.
    struct Ring {
        i32x4_t qa, qb;    // descriptors of the next K tile to copy: base - DMA_BIAS, extent
        uint64_t sa, sb;   // bytes between consecutive K tiles
        uint32_t na, nb;   // extent (with DMA_BIAS) of a full K tile
        int left;          // K tiles not yet copied (the in-ring partial tile included); of B
                           // in a half-stage ring, whose A runs one tile ahead
        int left_a;        // half-stage ring: K tiles of A not yet copied
        uint32_t m0a, m0b; // LDS byte address of this wave's first A / B block in stage 0
                           // (half-stage ring: in slot 0)
        uint32_t tail_b;   // extent of the partial tile's row-major B copies (else nb)
    };
    static __device__ __forceinline__ i32x4_t desc(uint64_t base, uint32_t bytes)
    {
        // base < 2^47 (checked on the host): word 1 holds its high bits with stride 0.
        // The words are wave-uniform; readfirstlane keeps them in scalar registers even
        // where they come from vector-ALU arithmetic (the copies take them only there).
        return (i32x4_t){__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                         __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)),
                         __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
    }
    static __device__ __forceinline__ void ring_init(const GemmArgs& p, int m0, int n0, int wave,
                                                     const SPT_LDS char* smem, Ring& r)
    {
        const int rows_a = min(C::BM, p.M - m0);
        const uint64_t a = (uint64_t)(uintptr_t)(p.A + (long long)m0 * p.lda * C::ELT) - DMA_BIAS;
        r.sa = (uint64_t)C::BK * C::ELT;
        r.na = (uint32_t)(((long long)(rows_a - 1) * p.lda + C::BK) * C::ELT) + DMA_BIAS;
        uint64_t b;
        if constexpr (C::BCOL) {
            const int cols = min(C::BN, p.N - n0);
            b = (uint64_t)(uintptr_t)(p.B + (long long)n0 * p.ldb * C::ELT) - DMA_BIAS;
            r.sb = (uint64_t)C::BK * C::ELT;
            r.nb = (uint32_t)(((long long)(cols - 1) * p.ldb + C::BK) * C::ELT) + DMA_BIAS;
        } else {
            b = (uint64_t)(uintptr_t)(p.B + (long long)n0 * C::ELT) - DMA_BIAS;
            r.sb = (uint64_t)C::BK * p.ldb * C::ELT;
            r.nb = (uint32_t)(((long long)C::BK * p.ldb - n0) * C::ELT) + DMA_BIAS;
        }
        const int tail = C::RING_TAIL ? p.tail_ring : 0;
        r.left = p.k_full + tail;
        r.tail_b = r.nb;
        if constexpr (!C::BCOL && C::RING_TAIL)
            // the partial tile's copies of row-major B end after its k_tail rows: the
            // rows past K read as zeros
            if (tail) r.tail_b = (uint32_t)(((long long)p.k_tail * p.ldb - n0) * C::ELT) + DMA_BIAS;
        r.left_a = r.left;
        r.qa = desc(a, r.left > 0 ? r.na : 0u);
        r.qb = desc(b, r.left > 0 ? (r.left == 1 ? r.tail_b : r.nb) : 0u);
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
        r.m0a = lds0 + (uint32_t)(wave * C::A_CPT) * 1024u;
        r.m0b = lds0 + (uint32_t)(C::SPLIT ? 0 : C::A_BYTES) + (uint32_t)(wave * C::B_CPT) * 1024u;
    }
    // Ring bookkeeping after a tile's copies were taken, in three parts that
    // the scheduler spreads over free MFMA slots: advance the A base, the B
    // base (64-bit adds on the descriptor words), then the extents.
    static __device__ __forceinline__ void add64(i32x4_t& q, uint64_t step)
    {
        uint64_t a = ((uint64_t)(uint32_t)q[1] << 32) | (uint32_t)q[0];
        a += step;
        q[0] = (int)(uint32_t)a;
        q[1] = (int)(uint32_t)(a >> 32);
    }
    static __device__ __forceinline__ void ring_advance(Ring& r, int part)
    {
        if (part == 0) add64(r.qa, r.sa);
        if (part == 1) add64(r.qb, r.sb);
        if (part == 2) {
            r.left -= 1;
            if constexpr (C::SPLIT) r.left_a -= 1;
            r.qa[2] = (int)((C::SPLIT ? r.left_a : r.left) > 0 ? r.na : 0u);
            r.qb[2] = (int)(r.left > 1 ? r.nb : r.left == 1 ? r.tail_b : 0u);
        }
    }
    // Half-stage ring prologue: one operand's copy taken, advance that operand alone.
    static __device__ __forceinline__ void ring_advance_a(Ring& r)
    {
        add64(r.qa, r.sa);
        r.left_a -= 1;
        r.qa[2] = (int)(r.left_a > 0 ? r.na : 0u);
    }
    static __device__ __forceinline__ void ring_advance_b(Ring& r)
    {
        add64(r.qb, r.sb);
        r.left -= 1;
        r.qb[2] = (int)(r.left > 0 ? r.nb : 0u);
    }

#ifdef SPT_POISON
    // Race-detection builds only (never in the shipped library): after the barrier
    // that frees a stage, fill the 1 KiB blocks this wave's copies are about to
    // refill with a poison pattern (NaN for the float types, 127 for int8) and wait
    // for those writes before the copies are issued.  A read of the stage before its
    // copies land then shows up in C as NaN, or as a wrong int8 sum.
    static __device__ __forceinline__ void poison(const Ring& r, uint32_t stage_off)
    {
        poison(r, stage_off, stage_off);
    }
    static __device__ __forceinline__ void poison(const Ring& r, uint32_t a_off, uint32_t b_off)
    {
        constexpr int pv = C::DT == DT_F16 ? 0x7E007E00 : C::DT == DT_BF16 ? 0x7FC07FC0
                           : C::DT == DT_F32 ? 0x7FC00000 : 0x7F7F7F7F;
        const i32x4_t v = {pv, pv, pv, pv};
        const uint32_t lane = (threadIdx.x & 63) * 16;
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i)
            *(SPT_LDS i32x4_t*)(size_t)(r.m0a + a_off + i * 1024 + lane) = v;
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i)
            *(SPT_LDS i32x4_t*)(size_t)(r.m0b + b_off + i * 1024 + lane) = v;
        wait_lgkmcnt0();
    }
#endif

    // The copies of one K tile into one stage: copy j < A_CPT of the wave moves
    // A block j of its run of A_CPT blocks, copy A_CPT + i B block i.
    struct Dma {
        i32x4_t ra, rb;
        uint32_t m0a, m0b;
    };
    static __device__ __forceinline__ Dma dma_of(const Ring& r, uint32_t stage_off)
    {
        return Dma{r.qa, r.qb, r.m0a + stage_off, r.m0b + stage_off};
    }
    static __device__ __forceinline__ Dma dma_of(const Ring& r, uint32_t a_off, uint32_t b_off)
    {
        return Dma{r.qa, r.qb, r.m0a + a_off, r.m0b + b_off};
    }
    // (a half-stage ring issues the B copies first: see VM_STEADY)
    template <int J>
    static __device__ __forceinline__ void dma_issue(const Dma& d, const Copy& cp)
    {
        constexpr bool IS_A = C::SPLIT ? J >= C::B_CPT : J < C::A_CPT;
        constexpr int i = C::SPLIT ? (IS_A ? J - C::B_CPT : J) : (IS_A ? J : J - C::A_CPT);  // copy index within the operand
        constexpr int g = i / 4, e = i % 4;          // group of four sharing one M0 value
        const uint32_t m0 = (IS_A ? d.m0a : d.m0b) + g * 4096;
        if constexpr (IS_A)
            dma16<e * 1024, e == 0>(d.ra, m0, cp.a_voff[i]);
        else
            dma16<e * 1024, e == 0>(d.rb, m0, cp.b_voff[i]);
    }

    // ---- V_REG / V_SYNC producer: global -> VGPR -> LDS ------------------------
    // Tile t (empty loads, which read as zero, for t >= k_full: the loop
    // prefetches one tile past its end without a branch).
    static __device__ __forceinline__ void load_regs(const GemmArgs& p, int m0, int n0, int t,
                                                     const Copy& cp, i32x4_t (&ra_)[C::A_CPT],
                                                     i32x4_t (&rb_)[C::B_CPT])
    {
        const char *pa, *pb;
        uint32_t na, nb;
        const bool live = t < p.k_full;
        span_a(p, m0, live ? t : 0, pa, na);
        span_b(p, n0, live ? t : 0, pb, nb);
        if (!live) na = nb = 0;
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(pa, na), rb = make_rsrc(pb, nb);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) ra_[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, cp.a_voff[i], 0, 0);
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) rb_[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, cp.b_voff[i], 0, 0);
    }

    // Thread tid's copies sit at the same stage chunks as in the V_DIRECT copies
    // (chunk i THREADS + tid), written with ds_write_b128.
    static __device__ __forceinline__ void store_regs(SPT_LDS char* st, int tid,
                                                      const i32x4_t (&ra_)[C::A_CPT],
                                                      const i32x4_t (&rb_)[C::B_CPT])
    {
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) *(SPT_LDS i32x4_t*)(st + chunk_of(i, tid, C::A_CPT) * 16) = ra_[i];
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i)
            *(SPT_LDS i32x4_t*)(st + C::A_BYTES + chunk_of(i, tid, C::B_CPT) * 16) = rb_[i];
    }

    // The partial last K tile (t = k_full, K - t*BK = k_tail elements), through
    // VGPRs with every element at k >= K set to zero.
    static __device__ void load_tail(const GemmArgs& p, int m0, int n0, int tid,
                                     i32x4_t (&ra_)[C::A_CPT], i32x4_t (&rb_)[C::B_CPT])
    {
        const int t = p.k_full;
        const int kt = p.k_tail;  // valid k inside the tile: [0, kt)
        const char *pa, *pb;
        uint32_t na, nb;
        span_a(p, m0, t, pa, na);
        span_b(p, n0, t, pb, nb);
        const __amdgpu_buffer_rsrc_t ra = make_rsrc(pa, na), rb = make_rsrc(pb, nb);
        const int rows_a = min(C::BM, p.M - m0);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) {
            int r, k;
            a_src(chunk_of(i, tid, C::A_CPT), r, k);
            r = min(r, rows_a - 1);
            const int valid = kt - k;  // elements of this chunk below K
            const int voff = r * p.lda * C::ELT + (valid > 0 ? k * C::ELT : 0);
            ra_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(ra, voff, 0, 0), valid * C::ELT);
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int k, n;
            b_src(chunk_of(i, tid, C::B_CPT), k, n);
            if constexpr (C::BCOL) {
                n = min(n, min(C::BN, p.N - n0) - 1);
                const int valid = kt - k;
                const int voff = n * p.ldb * C::ELT + (valid > 0 ? k * C::ELT : 0);
                rb_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0), valid * C::ELT);
            } else {
                if (n0 + n >= p.N) n = 0;
                const bool ok = k < kt;  // k-row of this chunk below K
                const int voff = (ok ? k : 0) * p.ldb * C::ELT + n * C::ELT;
                rb_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0), ok ? 16 : 0);
            }
        }
    }

    // ---- consumer ----------------------------------------------------------------
    // Fragment read j (0 .. FM+FN-1) of k-step s into `slot`.
    // B of a full stage at st: st + A_BYTES
    static __device__ __forceinline__ const SPT_LDS char* b_of(const SPT_LDS char* st)
    {
        return st + (C::A_BYTES - B_OFF);
    }
    static __device__ __forceinline__ void read_frag(const SPT_LDS char* st, const Lanes& L, int s, int j,
                                                     Slot& slot)
    {
        read_frag(st, b_of(st), L, s, j, slot);
    }
    // A from the stage or slot at sa; B at the base its lane offsets count from, sb
    // (b_of(st) for a full stage at st, the slot itself in a half-stage ring)
    static __device__ __forceinline__ void read_frag(const SPT_LDS char* sa, const SPT_LDS char* sb, const Lanes& L,
                                                     int s, int j, Slot& slot)
    {
        if (j < C::FM)
            slot[j] = read_a(sa, L, j, s);
        else
            slot[j] = read_b(sb, L, j - C::FM, s);
    }
    static __device__ __forceinline__ void read_slot(const SPT_LDS char* st, const Lanes& L, int s, Slot& slot)
    {
#pragma unroll
        for (int j = 0; j < C::FM + C::FN; ++j) read_frag(st, b_of(st), L, s, j, slot);
    }
    static __device__ __forceinline__ void read_slot(const SPT_LDS char* sa, const SPT_LDS char* sb, const Lanes& L,
                                                     int s, Slot& slot)
    {
#pragma unroll
        for (int j = 0; j < C::FM + C::FN; ++j) read_frag(sa, sb, L, s, j, slot);
    }
    static __device__ __forceinline__ void mma_one(const Slot& slot, int j, acc_t (&acc)[C::FM][C::FN])
    {
        const int m = j / C::FN, n = j % C::FN;
        mma<C::DT>(acc[m][n], slot[C::FM + n], slot[m]);
    }

    // ---- issue plan of one k-step ------------------------------------------------
    // With one wave per SIMD a wave issues at most one instruction every four
    // cycles, so a 16-cycle MFMA leaves room for about three more before the
    // next MFMA is delayed.  Side work is therefore placed slot by slot (slot j
    // = right after MFMA j): the FN B fragments of the next step in slots
    // 0 .. FN-1 (each MFMA row needs all of them), A fragment ma of the next
    // step once row ma has consumed the current one (its registers are then
    // free), and copies and ring bookkeeping spread over the remaining slots.
    static constexpr int NJ = C::FM * C::FN;
    static constexpr int a_read_at(int ma)
    {
        return (ma * C::FN + C::FN - 1) > (C::FN + ma) ? (ma * C::FN + C::FN - 1) : (C::FN + ma);
    }
    static constexpr int a_owner(int j)  // A fragment read after slot j, or -1
    {
        for (int ma = 0; ma < C::FM; ++ma)
            if (a_read_at(ma) == j) return ma;
        return -1;
    }
    static constexpr bool free_slot(int j) { return j >= C::FN && a_owner(j) < 0; }
    static constexpr int NFREE = [] {
        int n = 0;
        for (int j = 0; j < NJ; ++j) n += free_slot(j);
        return n;
    }();
    static constexpr int nth_free(int k)
    {
        for (int j = 0; j < NJ; ++j)
            if (free_slot(j) && k-- == 0) return j;
        return NJ;  // none left: after the last MFMA
    }
    // Copy d of NDMA: evenly over the free slots.
    static constexpr int dma_at(int d, int ndma)
    {
        return ndma <= NFREE ? nth_free((d * NFREE) / ndma) : (d < NJ ? d : NJ);
    }
    static constexpr int dma_owner(int j, int ndma)
    {
        for (int d = 0; d < ndma; ++d)
            if (dma_at(d, ndma) == j) return d;
        return -1;
    }
    // Ring bookkeeping part q (0 .. 2): the last free slots that hold no copy.
    static constexpr int adv_at(int q, int ndma)
    {
        int k = 2 - q;
        for (int j = NJ - 1; j >= 0; --j)
            if (free_slot(j) && dma_owner(j, ndma) < 0 && k-- == 0) return j;
        return NJ;
    }
    static constexpr int adv_owner(int j, int ndma)
    {
        for (int q = 0; q < 3; ++q)
            if (adv_at(q, ndma) == j) return q;
        return -1;
    }

    // The FM x FN MFMAs of one k-step from `use`, row by row, with side work
    // per the issue plan: the fragments of step `snext` of the stage that
    // `src` + L address into `nxt` (READ), NDMA copies of `d`,
    // and the ring bookkeeping (ADV).  A fence after every slot keeps the
    // written order.
    template <int NDMA, bool READ, bool ADV>
    static __device__ __forceinline__ void step(const Slot& use, Slot& nxt, const SPT_LDS char* src, const Lanes& L,
                                                int snext, const Dma& d, const Copy& cp, Ring& r,
                                                acc_t (&acc)[C::FM][C::FN])
    {
        step<NDMA, READ, ADV>(use, nxt, src, b_of(src), L, snext, d, cp, r, acc);
    }
    template <int NDMA, bool READ, bool ADV>
    static __device__ __forceinline__ void step(const Slot& use, Slot& nxt, const SPT_LDS char* src,
                                                const SPT_LDS char* srcb, const Lanes& L, int snext, const Dma& d,
                                                const Copy& cp, Ring& r, acc_t (&acc)[C::FM][C::FN])
    {
        static_assert(!ADV || NDMA > 0, "bookkeeping belongs to the step that copies");
        static_for<0, NJ>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            constexpr int dj = dma_owner(j, NDMA), aj = a_owner(j), qj = adv_owner(j, NDMA);
            mma_one(use, j, acc);
            if constexpr (dj >= 0) dma_issue<dj>(d, cp);
            if constexpr (READ && j < C::FN) read_frag(src, srcb, L, snext, C::FM + j, nxt);
            if constexpr (READ && aj >= 0) read_frag(src, srcb, L, snext, aj, nxt);
            if constexpr (ADV && qj >= 0) ring_advance(r, qj);
            order_fence();
        });
        static_for<0, NDMA>([&](auto dc) {
            constexpr int dd = decltype(dc)::value;
            if constexpr (dma_at(dd, NDMA) >= NJ) dma_issue<dd>(d, cp);
        });
        if constexpr (ADV) {
            static_for<0, 3>([&](auto qc) {
                constexpr int q = decltype(qc)::value;
                if constexpr (adv_at(q, NDMA) >= NJ) ring_advance(r, q);
            });
        }
    }

    // One stage, all k-steps (REG / SYNC / the K tail): the fragments of step
    // s+1 are read beside the MFMAs of step s.
    static __device__ __forceinline__ void compute(const SPT_LDS char* st, const Lanes& L, const Copy& cp,
                                                   acc_t (&acc)[C::FM][C::FN])
    {
        Slot sl[2];
        read_slot(st, L, 0, sl[0]);
        const Dma none{};
        Ring unused{};
        static_for<0, C::KS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            step<0, (s + 1 < C::KS), false>(sl[s & 1], sl[(s + 1) & 1], st, L, s + 1, none, cp, unused, acc);
        });
    }

    // XCD-aware placement.  Workgroups are dispatched round-robin over the 8
    // XCDs (each with its own L2); renumber so each XCD gets a contiguous run
    // of tiles, then walk tiles in bands of 8 tile-rows so that neighbouring
    // workgroups of one XCD share A rows and B columns in that XCD's L2.
    static __device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn)
    {
        const int total = tiles_m * tiles_n;
        const int q = total / 8, rem = total % 8;
        const int xcd = bid % 8, j = bid / 8;
        const int id = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + j;
        const int G = 8;
        const int band = id / (G * tiles_n);
        const int first = band * G;
        const int gs = min(G, tiles_m - first);
        const int in = id - band * G * tiles_n;
        tm = first + in % gs;
        tn = in / gs;
    }

    static __device__ void store_c(const GemmArgs& p, int m0, int n0, int wm0, int wn0, int lane,
                                   const acc_t (&acc)[C::FM][C::FN])
    {
        const int l16 = lane & 15, g = lane >> 4;
        if (C::EXACT || (m0 + C::BM <= p.M && n0 + C::BN <= p.N)) {  // whole tile inside C
            char* base = p.C + ((long long)(m0 + wm0 + l16) * p.ldc + n0 + wn0 + 4 * g) * 4;
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int n = 0; n < C::FN; ++n)
                    *(acc_t*)(base + ((long long)16 * m * p.ldc + 16 * n) * 4) = acc[m][n];
            return;
        }
#pragma unroll
        for (int m = 0; m < C::FM; ++m) {
            const int row = m0 + wm0 + 16 * m + l16;
            if (row >= p.M) continue;
            char* crow = p.C + (long long)row * p.ldc * 4;
#pragma unroll
            for (int n = 0; n < C::FN; ++n) {
                const int col = n0 + wn0 + 16 * n + 4 * g;
                if (col + 3 < p.N) {
                    *(acc_t*)(crow + (long long)col * 4) = acc[m][n];
                } else {
                    const f32x4_t v = __builtin_bit_cast(f32x4_t, acc[m][n]);  // raw 32-bit words
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < p.N) ((float*)crow)[col + e] = v[e];
                }
            }
        }
    }

    // V_DIRECT main loop (see the schedule at the top of this file).  Every
    // iteration is the same: past the last K tile the ring issues empty copies
    // (a zero-length buffer range moves no memory, lanes read as out of range),
    // as "Hiding Memory Latency ...", section 8, turns out-of-range tiles into
    // zero-filled stages, so the vmcnt count per tile never changes.  The
    // stage index is a run-time value (a loop body per stage would hold more
    // than the 256 accumulator registers of a 128 x 128 wave tile leave room
    // for); an odd number of k-steps flips the register slot of step 0 every
    // tile, so such tiles go in pairs to keep the slot a compile-time
    // constant.  The last tile's reads of "tile nf" are discarded; the ring is
    // drained before the kernel leaves.
    static __device__ __forceinline__ void loop_direct(const GemmArgs& p, int m0, int n0, int wave,
                                                       const Lanes& L, SPT_LDS char* smem, Copy& cp,
                                                       acc_t (&acc)[C::FM][C::FN])
    {
        const int nf = p.k_full + (C::RING_TAIL ? p.tail_ring : 0);
        if (nf == 0) return;
        Ring r;
        ring_init(p, m0, n0, wave, smem, r);
        // prologue: tiles 0 .. S-1 into stages 0 .. S-1
#pragma unroll
        for (int i = 0; i < C::S; ++i) {
            if constexpr (C::RING_TAIL)
                if (p.tail_ring && i == p.k_full) mask_tail(p, threadIdx.x, cp);
            const Dma d = dma_of(r, i * C::STAGE_BYTES);
            static_for<0, C::LOADS>([&](auto jc) { dma_issue<decltype(jc)::value>(d, cp); });
            ring_advance(r, 0);
            ring_advance(r, 1);
            ring_advance(r, 2);
        }
        wait_vmcnt<C::VM_FIRST>();  // tile 0 landed
        barrier();
        Slot sl[2];
        read_slot(smem, L, 0, sl[0]);

        int t = 0;
        uint32_t rs = 0;  // byte offset of the stage tile t sits in
        if constexpr (C::KS % 2 == 0) {
            for (; t < nf; ++t) tile_direct<0>(p, r, rs, L, smem, cp, sl, acc);
        } else {
            for (; t + 1 < nf; t += 2) {
                tile_direct<0>(p, r, rs, L, smem, cp, sl, acc);
                tile_direct<1>(p, r, rs, L, smem, cp, sl, acc);
            }
            // (exact-fit kernels with one k-step per tile are dispatched for an even nf only)
            if constexpr (!C::EXACT)
                if (t < nf) tile_direct<0>(p, r, rs, L, smem, cp, sl, acc);
        }
        wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
    }

    // One K tile in the stage at byte offset rs (advanced to the next stage on
    // return); its k-step s uses register slot (P + s) & 1.
    template <int P>
    static __device__ __forceinline__ void tile_direct(const GemmArgs& p, Ring& r, uint32_t& rs, const Lanes& L,
                                                       const SPT_LDS char* smem, Copy& cp, Slot (&sl)[2],
                                                       acc_t (&acc)[C::FM][C::FN])
    {
        const uint32_t nx = rs + C::STAGE_BYTES == (uint32_t)C::LDS_BYTES ? 0u : rs + C::STAGE_BYTES;
        const Dma none{};
        static_for<0, C::KS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            Slot& use = sl[(P + s) & 1];
            Slot& nxt = sl[(P + s + 1) & 1];
            if constexpr (s + 1 < C::KS) {
                step<0, true, false>(use, nxt, smem + rs, L, s + 1, none, cp, r, acc);
            } else {
                wait_lgkmcnt0();                       // this wave's reads of this tile are complete
                wait_vmcnt<C::VM_STEADY>();            // its copies of the next tile have landed
                barrier();                             // next tile visible to all; this stage free
                if constexpr (C::RING_TAIL)
                    if (r.left == 1 && p.tail_ring) mask_tail(p, threadIdx.x, cp);  // tile + S is the partial one
                const Dma d = dma_of(r, rs);           // tile + S into this stage
#ifdef SPT_POISON
                poison(r, rs);
#endif
                step<C::LOADS, true, true>(use, nxt, smem + nx, L, 0, d, cp, r, acc);
            }
        });
        rs = nx;
    }

    // Half-stage ring (C::SPLIT): SLOTS = 2S - 1 slots of A_BYTES; ring position 2t
    // holds A of K tile t, 2t + 1 its B, in slot (position mod SLOTS).  The prologue
    // copies positions 0 .. SLOTS-1.  At the barrier of tile t (the schedule of
    // loop_direct) tile t's two slots are free, and the next two positions go into
    // them: B of tile t + S - 1 into A's slot, then A of tile t + S into B's.  The
    // wait before that barrier needs tile t + 1 (positions up to 2t + 3); the copies
    // issued after it, A of tile t + 2, may stay in flight: the copy path never
    // drains, which a 2-stage ring of the same tile does at every K tile.
    static __device__ __forceinline__ void loop_split(const GemmArgs& p, int m0, int n0, int wave,
                                                      const Lanes& L, SPT_LDS char* smem, Copy& cp,
                                                      acc_t (&acc)[C::FM][C::FN])
    {
        static_assert(C::KS % 2 == 0, "half-stage rings: an even number of k-steps per K tile");
        constexpr uint32_t HB = C::A_BYTES;
        const int nf = p.k_full;
        if (nf == 0) return;
        Ring r;
        ring_init(p, m0, n0, wave, smem, r);
        static_for<0, C::SLOTS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            const Dma d = dma_of(r, i * HB, i * HB);
            if constexpr (i % 2 == 0) {
                static_for<C::B_CPT, C::LOADS>([&](auto jc) { dma_issue<decltype(jc)::value>(d, cp); });
                ring_advance_a(r);
            } else {
                static_for<0, C::B_CPT>([&](auto jc) { dma_issue<decltype(jc)::value>(d, cp); });
                ring_advance_b(r);
            }
        });
        wait_vmcnt<C::VM_FIRST>();  // tile 0 landed
        barrier();
        Slot sl[2];
        read_slot(smem, smem + HB, L, 0, sl[0]);
        uint32_t ao = 0, bo = HB;  // slots of tile t's A and B
        for (int t = 0; t < nf; ++t) tile_split(r, ao, bo, L, smem, cp, sl, acc);
        wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
    }
    static __device__ __forceinline__ void tile_split(Ring& r, uint32_t& ao, uint32_t& bo, const Lanes& L,
                                                      const SPT_LDS char* smem, Copy& cp, Slot (&sl)[2],
                                                      acc_t (&acc)[C::FM][C::FN])
    {
        constexpr uint32_t HB = C::A_BYTES, WRAP = C::SLOTS * HB;
        const uint32_t an = ao + 2 * HB >= WRAP ? ao + 2 * HB - WRAP : ao + 2 * HB;
        const uint32_t bn = bo + 2 * HB >= WRAP ? bo + 2 * HB - WRAP : bo + 2 * HB;
        const Dma none{};
        static_for<0, C::KS>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            Slot& use = sl[s & 1];
            Slot& nxt = sl[(s + 1) & 1];
            if constexpr (s + 1 < C::KS) {
                step<0, true, false>(use, nxt, smem + ao, smem + bo, L, s + 1, none, cp, r, acc);
            } else {
                wait_lgkmcnt0();                 // this wave's reads of this tile are complete
                wait_vmcnt<C::VM_STEADY>();      // its copies of the next tile have landed
                barrier();                       // next tile visible to all; this tile's slots free
                const Dma d = dma_of(r, bo, ao); // A of tile + S into B's slot, B of tile + S - 1 into A's
#ifdef SPT_POISON
                poison(r, bo, ao);
#endif
                step<C::LOADS, true, true>(use, nxt, smem + an, smem + bn, L, 0, d, cp, r, acc);
            }
        });
        ao = an;
        bo = bn;
    }

    static __device__ __forceinline__ void run(const GemmArgs& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
        SPT_LDS char* smem = (SPT_LDS char*)smem_raw;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        int tm, tn;
        tile_of(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
        // (the divisions of the tile order may run on the vector ALU: keep the results scalar)
        const int m0 = __builtin_amdgcn_readfirstlane(tm) * C::BM, n0 = __builtin_amdgcn_readfirstlane(tn) * C::BN;
        const int wm0 = (wave / C::WAVES_N) * C::WTM, wn0 = (wave % C::WAVES_N) * C::WTN;
        const int mb0 = wm0 / 16, nb0 = wn0 / 16;

        Copy cp;
        setup_copy(p, m0, n0, tid, cp);
        Lanes L;
        setup_lanes(lane, mb0, nb0, L);

        acc_t acc[C::FM][C::FN];
#pragma unroll
        for (int m = 0; m < C::FM; ++m)
#pragma unroll
            for (int n = 0; n < C::FN; ++n) acc[m][n] = (acc_t){0, 0, 0, 0};

        const int nf = p.k_full;
        i32x4_t ra[C::A_CPT], rb[C::B_CPT];

        if constexpr (C::V == V_SYNC) {
            // load -> barrier -> compute -> barrier
            for (int t = 0; t < nf; ++t) {
                load_regs(p, m0, n0, t, cp, ra, rb);
                wait_vmcnt<0>();
                store_regs(smem, tid, ra, rb);
                wait_lgkmcnt0();
                barrier();
                compute(smem, L, cp, acc);
                barrier();
            }
        } else if constexpr (C::V == V_REG) {
            if (nf > 0) {  // prologue: tile 0 into stage 0
                load_regs(p, m0, n0, 0, cp, ra, rb);
                wait_vmcnt<0>();
                store_regs(smem, tid, ra, rb);
                wait_lgkmcnt0();
                barrier();
            }
            // tile t+1 is fetched while tile t is computed (past the end: an empty
            // fetch whose zeros land in a stage nobody reads again)
            for (int t = 0; t < nf; ++t) {
                SPT_LDS char* cur = smem + (C::S == 2 ? (t & 1) : 0) * C::STAGE_BYTES;
                SPT_LDS char* nxt = smem + (C::S == 2 ? ((t + 1) & 1) : 0) * C::STAGE_BYTES;
                load_regs(p, m0, n0, t + 1, cp, ra, rb);  // in flight during compute
                compute(cur, L, cp, acc);
                if constexpr (C::S == 1) barrier();  // one buffer: all reads of it done first
                wait_vmcnt<0>();
                store_regs(nxt, tid, ra, rb);
                wait_lgkmcnt0();
                barrier();
            }
        } else if constexpr (C::SPLIT) {
            loop_split(p, m0, n0, wave, L, smem, cp, acc);
        } else {
            loop_direct(p, m0, n0, wave, L, smem, cp, acc);
        }

        if (!C::EXACT && p.k_tail && !(C::RING_TAIL && p.tail_ring)) {
            // partial last tile, zero-filled beyond K, through VGPRs
            load_tail(p, m0, n0, tid, ra, rb);
            wait_vmcnt<0>();
            wait_lgkmcnt0();
            barrier();  // every wave is done reading the stages
            store_regs(smem, tid, ra, rb);
            wait_lgkmcnt0();
            barrier();
            compute(smem, L, cp, acc);
        }

        store_c(p, m0, n0, wm0, wn0, lane, acc);
    }
};

// Two waves per SIMD (two 256-thread workgroups, or one 512-thread workgroup,
// per CU) keep VGPR + AGPR use within 256 per lane; a 128 x 128 wave tile
// runs one wave per SIMD with up to 512.
template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD))) void
gemm_kernel(GemmArgs p)
{
    Gemm<C>::run(p);
}

}  // namespace spt
