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
//            round trip) into an S-stage ring, S = 2 or 3 (sections 5, 6),
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

// ---------------------------------------------------------------------------
// EXACT_: M, N and K are multiples of the tile (no K tail, no edge checks in
// the epilogue); the dispatcher selects it only for such shapes.
// BLANE_: row-major B kept in the lane layout (fp32 B always is).
#ifndef SPT_B_LANE_DEFAULT
#define SPT_B_LANE_DEFAULT false
#endif
template <int DT_, bool BCOL_, int TILE_, int V_, int S_, bool EXACT_ = false, bool BLANE_ = SPT_B_LANE_DEFAULT>
struct Cfg {
    static constexpr int DT = DT_;
    static constexpr bool BCOL = BCOL_;
    static constexpr bool EXACT = EXACT_;
    static constexpr bool BLANE = BLANE_ || elt_bytes(DT_) == 4;
    static constexpr int TILE = TILE_, V = V_, S = S_;
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
    static constexpr int LDS_BYTES = S * STAGE_BYTES;
    static constexpr int A_CPT = A_BYTES / 16 / THREADS;  // 16-byte copies per thread per stage
    static constexpr int B_CPT = B_BYTES / 16 / THREADS;
    static constexpr int LOADS = A_CPT + B_CPT;            // vmcnt units per tile per thread
    // 16x16 wave tiles of 128 x 128 need the whole register file: one wave per SIMD
    static constexpr int WAVES_PER_SIMD = FM * FN > 32 ? 1 : 2;

    static_assert(BK % KSTEP == 0, "BK must hold whole MFMA steps");
    static_assert(A_BYTES % (1024 * WAVES) == 0 && B_BYTES % (1024 * WAVES) == 0,
                  "a stage must split into whole 1 KiB copies per wave");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must hold whole 16x16 MFMA tiles");
    static_assert(LDS_BYTES <= kLdsPerCu, "LDS ring exceeds 160 KiB");
    static_assert(V_ != V_SYNC || S_ == 1, "SYNC has one stage");
    static_assert(V_ != V_REG || (S_ == 1 || S_ == 2), "REG has 1 or 2 stages");
    static_assert(V_ != V_DIRECT || (S_ == 2 || S_ == 3), "DIRECT has 2 or 3 stages");
    static_assert((S_ - 1) * LOADS < 64, "vmcnt range");
};

template <int DT>
struct AccT {
    typedef f32x4_t type;
};
template <>
struct AccT<DT_I8> {
    typedef i32x4_t type;
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
        acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(x, y, acc, 0, 0, 0);
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

// The same buffer descriptor as four SGPR words, for inline asm: base
// address (48 bits, stride 0), num_records, and the gfx9 raw-buffer word 3.
__device__ __forceinline__ i32x4_t rsrc_words(const char* base, uint32_t bytes)
{
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return (i32x4_t){(int)(uint32_t)a, (int)((uint32_t)(a >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// One asynchronous 16-byte-per-lane copy global -> LDS (buffer_load_dwordx4
// ... lds): lane l's 16 bytes at rsrc + voffset land at LDS byte lds + 16*l.
// `lds` must be wave-uniform.  Written as inline asm so that the compiler
// does not guard later LDS reads with waits of its own (it cannot tell the
// ring stages apart and would drain every copy in flight); the ring's
// s_waitcnt vmcnt + s_barrier placement is the only synchronisation.  M0
// carries the LDS address; the s_nop covers the M0-write -> LDS-DMA hazard.
__device__ __forceinline__ void dma16(i32x4_t rsrc, uint32_t lds, int voffset)
{
    asm volatile(
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, 0 offen lds"
        :
        : "v"(voffset), "s"(rsrc), "{m0}"(lds)
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
    static __device__ __forceinline__ constexpr int swz_n(int r) { return C::ELT == 2 ? ((r & 3) << 1) : (r & 7); }
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

    // ---- fragment reads ---------------------------------------------------------
    // Per-lane LDS byte offsets of this wave's fragments within a stage, for
    // MFMA row 0 / column 0 of the wave tile; other rows / columns add an
    // immediate.  A fragment (m, s): 16 rows x the 16-byte chunk 4s + g.
    static constexpr int B_OFFS = C::BCOL ? C::KS : (C::BLANE ? 1 : C::FN);
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
            if constexpr (C::BCOL) L.b[s] = C::A_BYTES + (16 * nb0 + l16) * RK + 16 * ((4 * s + g) ^ swz_k(l16));
        }
        if constexpr (!C::BCOL && C::BLANE) {
            L.b[0] = br_block(nb0, 0, 0) + lane * (C::ELT == 4 ? 4 : 8);
        } else if constexpr (!C::BCOL && C::ELT == 2) {
            // tr_b16: lane (g, i) fetches k-row 8g + (i >> 2) (+ 4h + KSTEP s) at columns
            // 4 (i & 3) .. + 3 of column block nb; swz_n only sees k-row bits 0, 1.
#pragma unroll
            for (int n = 0; n < C::FN; ++n) {
                const int kr = 8 * g + (l16 >> 2);
                const int c = 2 * (nb0 + n) + ((l16 & 3) >> 1);
                L.b[n] = C::A_BYTES + kr * RN + 16 * (c ^ swz_n(kr)) + 8 * (l16 & 1);
            }
        } else if constexpr (!C::BCOL && C::ELT == 1) {
            // tr_b8: lane (g, i) fetches k-row 16g + (i >> 1) (+ 8h + KSTEP s) at columns
            // 8 (i & 1) .. + 7 of column block nb; swz_n only sees k-row bits 0..2.
#pragma unroll
            for (int n = 0; n < C::FN; ++n) {
                const int kr = 16 * g + (l16 >> 1);
                L.b[n] = C::A_BYTES + kr * RN + 16 * ((nb0 + n) ^ swz_n(kr)) + 8 * (l16 & 1);
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
                o0 = L.b[n] + s * C::KSTEP * RN;
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
    // A and B chunks from the K tile's base.
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
            a_src(i * C::THREADS + tid, r, k);
            r = min(r, rows_a - 1);  // M edge: any in-range row (its outputs are not stored)
            cp.a_voff[i] = r * p.lda * C::ELT + k * C::ELT;
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int k, n;
            b_src(i * C::THREADS + tid, k, n);
            if constexpr (C::BCOL) {
                n = min(n, min(C::BN, p.N - n0) - 1);  // N edge
                cp.b_voff[i] = n * p.ldb * C::ELT + k * C::ELT;
            } else {
                if (n0 + n >= p.N) n = 0;  // N edge: any in-range chunk
                cp.b_voff[i] = k * p.ldb * C::ELT + n * C::ELT;
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
    // Copy j (0 .. LOADS-1) of K tile t into the stage at LDS byte `st`: the
    // copies of wave w, number i of an operand cover that operand's stage
    // chunks [(i WAVES + w) 64, + 64).
    struct Dma {
        i32x4_t ra, rb;
        uint32_t st;
    };
    static __device__ __forceinline__ Dma dma_begin(const GemmArgs& p, int m0, int n0, int t, uint32_t st)
    {
        const char *pa, *pb;
        uint32_t na, nb;
        const int tt = t < p.k_full ? t : 0;  // beyond the last full tile: an empty copy
        span_a(p, m0, tt, pa, na);
        span_b(p, n0, tt, pb, nb);
        if (t >= p.k_full) na = nb = 0;
        return Dma{rsrc_words(pa, na), rsrc_words(pb, nb), st};
    }
    static __device__ __forceinline__ void dma_issue(const Dma& d, int j, int wave, const Copy& cp)
    {
        if (j < C::A_CPT)
            dma16(d.ra, d.st + (j * C::WAVES + wave) * 1024, cp.a_voff[j]);
        else
            dma16(d.rb, d.st + C::A_BYTES + ((j - C::A_CPT) * C::WAVES + wave) * 1024,
                  cp.b_voff[j - C::A_CPT]);
    }

    // ---- V_REG / V_SYNC producer: global -> VGPR -> LDS ------------------------
    static __device__ __forceinline__ void load_regs(const GemmArgs& p, int m0, int n0, int t,
                                                     const Copy& cp, i32x4_t (&ra_)[C::A_CPT],
                                                     i32x4_t (&rb_)[C::B_CPT])
    {
        const char *pa, *pb;
        uint32_t na, nb;
        span_a(p, m0, t, pa, na);
        span_b(p, n0, t, pb, nb);
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
        for (int i = 0; i < C::A_CPT; ++i) *(SPT_LDS i32x4_t*)(st + (i * C::THREADS + tid) * 16) = ra_[i];
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i)
            *(SPT_LDS i32x4_t*)(st + C::A_BYTES + (i * C::THREADS + tid) * 16) = rb_[i];
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
            a_src(i * C::THREADS + tid, r, k);
            r = min(r, rows_a - 1);
            const int valid = kt - k;  // elements of this chunk below K
            const int voff = r * p.lda * C::ELT + (valid > 0 ? k * C::ELT : 0);
            ra_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(ra, voff, 0, 0), valid * C::ELT);
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int k, n;
            b_src(i * C::THREADS + tid, k, n);
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
    static __device__ __forceinline__ void read_frag(const SPT_LDS char* st, const Lanes& L, int s, int j,
                                                     Slot& slot)
    {
        if (j < C::FM)
            slot[j] = read_a(st, L, j, s);
        else
            slot[j] = read_b(st, L, j - C::FM, s);
    }
    static __device__ __forceinline__ void read_slot(const SPT_LDS char* st, const Lanes& L, int s, Slot& slot)
    {
#pragma unroll
        for (int j = 0; j < C::FM + C::FN; ++j) read_frag(st, L, s, j, slot);
    }
    static __device__ __forceinline__ void mma_one(const Slot& slot, int j, acc_t (&acc)[C::FM][C::FN])
    {
        const int m = j / C::FN, n = j % C::FN;
        mma<C::DT>(acc[m][n], slot[C::FM + n], slot[m]);
    }

    // Slot in the MFMA sequence of one k-step after which the A fragment of row
    // ma of the next step is read: once row ma has used the old one (so its
    // registers are reused) and after the `lead` copies and FN B reads.
    static constexpr int a_read_at(int ma, int lead)
    {
        return (ma * C::FN + C::FN - 1) > (lead + C::FN + ma) ? (ma * C::FN + C::FN - 1) : (lead + C::FN + ma);
    }

    // The FM x FN MFMAs of one k-step from `use`, row by row, with side work
    // beside them in this order: NDMA copies (j < NDMA), then the FN B fragments
    // of step `snext` of stage `src` into `nxt`, then its A fragments as rows
    // free up (READ).  Every side instruction sits after one MFMA; a fence keeps
    // the written order.
    template <int NDMA, bool READ>
    static __device__ __forceinline__ void step(const Slot& use, Slot& nxt, const SPT_LDS char* src, int snext,
                                                const Lanes& L, const Dma& d, int wave, const Copy& cp,
                                                acc_t (&acc)[C::FM][C::FN])
    {
        constexpr int NJ = C::FM * C::FN;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            mma_one(use, j, acc);
            if (j < NDMA) dma_issue(d, j, wave, cp);
            if (READ) {
                const int nb = j - NDMA;
                if (nb >= 0 && nb < C::FN) read_frag(src, L, snext, C::FM + nb, nxt);
#pragma unroll
                for (int ma = 0; ma < C::FM; ++ma)
                    if (a_read_at(ma, NDMA) == j) read_frag(src, L, snext, ma, nxt);
            }
            order_fence();
        }
        // side work whose slot fell beyond the last MFMA
#pragma unroll
        for (int j = NJ; j < NDMA; ++j) dma_issue(d, j, wave, cp);
        if (READ) {
#pragma unroll
            for (int nb = 0; nb < C::FN; ++nb)
                if (nb + NDMA >= NJ) read_frag(src, L, snext, C::FM + nb, nxt);
#pragma unroll
            for (int ma = 0; ma < C::FM; ++ma)
                if (a_read_at(ma, NDMA) >= NJ) read_frag(src, L, snext, ma, nxt);
        }
    }

    // One stage, all k-steps (REG / SYNC / the K tail): the fragments of step
    // s+1 are read beside the MFMAs of step s.
    static __device__ __forceinline__ void compute(const SPT_LDS char* st, const Lanes& L, int wave,
                                                   const Copy& cp, acc_t (&acc)[C::FM][C::FN])
    {
        Slot sl[2];
        read_slot(st, L, 0, sl[0]);
        const Dma none{};
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            if (s + 1 < C::KS)
                step<0, true>(sl[s & 1], sl[(s + 1) & 1], st, s + 1, L, none, wave, cp, acc);
            else
                step<0, false>(sl[s & 1], sl[(s + 1) & 1], st, 0, L, none, wave, cp, acc);
        }
    }

    // Wait until at most n (0 .. S-1) younger tiles' copies are in flight.
    static __device__ __forceinline__ void wait_tiles(int n)
    {
        if constexpr (C::S >= 3) {
            if (n >= 2) {
                wait_vmcnt<2 * C::LOADS>();
                return;
            }
        }
        if (n >= 1) {
            wait_vmcnt<C::LOADS>();
            return;
        }
        wait_vmcnt<0>();
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
    // zero-filled stages, so the vmcnt count per tile never changes and the
    // loop body has no branches.  The last tile's reads of "tile nf" are
    // discarded; the ring is drained before the kernel leaves it.
    static __device__ __forceinline__ void loop_direct(const GemmArgs& p, int m0, int n0, int wave,
                                                       const Lanes& L, SPT_LDS char* smem, const Copy& cp,
                                                       acc_t (&acc)[C::FM][C::FN])
    {
        const int nf = p.k_full;
        if (nf == 0) return;
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
        // prologue: tiles 0 .. S-1 into stages 0 .. S-1
#pragma unroll
        for (int i = 0; i < C::S; ++i) {
            const Dma d = dma_begin(p, m0, n0, i, lds0 + i * C::STAGE_BYTES);
#pragma unroll
            for (int j = 0; j < C::LOADS; ++j) dma_issue(d, j, wave, cp);
        }
        wait_vmcnt<(C::S - 1) * C::LOADS>();  // tile 0 landed
        barrier();
        Slot sl[2];
        read_slot(smem, L, 0, sl[0]);

        int t = 0, rs = 0;  // tile, and the stage it sits in
        if constexpr (C::KS % 2 == 0) {
            for (; t < nf; ++t) {
                tile_direct<0>(p, m0, n0, t, rs, wave, L, smem, cp, sl, acc);
                rs = rs + 1 == C::S ? 0 : rs + 1;
            }
        } else {
            // an odd number of k-steps flips the register slot of step 0 every tile:
            // tiles go in pairs so the slot stays a compile-time constant
            for (; t + 1 < nf; t += 2) {
                tile_direct<0>(p, m0, n0, t, rs, wave, L, smem, cp, sl, acc);
                rs = rs + 1 == C::S ? 0 : rs + 1;
                tile_direct<1>(p, m0, n0, t + 1, rs, wave, L, smem, cp, sl, acc);
                rs = rs + 1 == C::S ? 0 : rs + 1;
            }
            if (t < nf) tile_direct<0>(p, m0, n0, t, rs, wave, L, smem, cp, sl, acc);
        }
        wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
    }

    // K tile t of the V_DIRECT loop; its step s uses register slot (P + s) & 1.
    template <int P>
    static __device__ __forceinline__ void tile_direct(const GemmArgs& p, int m0, int n0, int t, int rs,
                                                       int wave, const Lanes& L, SPT_LDS char* smem,
                                                       const Copy& cp, Slot (&sl)[2], acc_t (&acc)[C::FM][C::FN])
    {
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
        const SPT_LDS char* cur = smem + rs * C::STAGE_BYTES;
        const int rs_next = rs + 1 == C::S ? 0 : rs + 1;
        const Dma none{};
#pragma unroll
        for (int s = 0; s < C::KS; ++s) {
            Slot& use = sl[(P + s) & 1];
            Slot& nxt = sl[(P + s + 1) & 1];
            if (s + 1 < C::KS) {
                step<0, true>(use, nxt, cur, s + 1, L, none, wave, cp, acc);
                continue;
            }
            wait_lgkmcnt0();                       // this wave's reads of tile t are complete
            wait_vmcnt<(C::S - 2) * C::LOADS>();   // its copies of tile t+1 have landed
            barrier();                             // tile t+1 visible to all; tile t's stage free
            const Dma d = dma_begin(p, m0, n0, t + C::S, lds0 + rs * C::STAGE_BYTES);
            step<C::LOADS, true>(use, nxt, smem + rs_next * C::STAGE_BYTES, 0, L, d, wave, cp, acc);
        }
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
        const int m0 = tm * C::BM, n0 = tn * C::BN;
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
                compute(smem, L, wave, cp, acc);
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
            for (int t = 0; t < nf; ++t) {
                SPT_LDS char* cur = smem + (C::S == 2 ? (t & 1) : 0) * C::STAGE_BYTES;
                SPT_LDS char* nxt = smem + (C::S == 2 ? ((t + 1) & 1) : 0) * C::STAGE_BYTES;
                const bool more = t + 1 < nf;
                if (more) load_regs(p, m0, n0, t + 1, cp, ra, rb);  // in flight during compute
                compute(cur, L, wave, cp, acc);
                if constexpr (C::S == 1) barrier();  // one buffer: all reads of it done first
                if (more) {
                    wait_vmcnt<0>();
                    store_regs(nxt, tid, ra, rb);
                }
                wait_lgkmcnt0();
                barrier();
            }
        } else {
            loop_direct(p, m0, n0, wave, L, smem, cp, acc);
        }

        if (!C::EXACT && p.k_tail) {  // partial last tile, zero-filled beyond K, through VGPRs
            load_tail(p, m0, n0, tid, ra, rb);
            wait_vmcnt<0>();
            wait_lgkmcnt0();
            barrier();  // every wave is done reading the stages
            store_regs(smem, tid, ra, rb);
            wait_lgkmcnt0();
            barrier();
            compute(smem, L, wave, cp, acc);
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
