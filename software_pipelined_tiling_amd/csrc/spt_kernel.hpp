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
//            round trip) into an S-stage ring, S = 2 or 3 (sections 5, 6).
//
// Ring discipline for V_DIRECT (sections 3-5 and 9, with one ordering
// change, see below): the prologue issues tiles 0..S-2 into stages 0..S-2.
// Iteration t then
//     waits until tile t's copies of this wave have landed
//         (s_waitcnt vmcnt: at most (S-2) newer tiles' copies in flight),
//     s_barrier                 -- every wave's copies of tile t are in LDS
//                                  and every wave has finished reading tile
//                                  t-1, whose stage (t+S-1) mod S is free,
//     issues tile t+S-1 into stage (t+S-1) mod S,
//     computes tile t from stage t mod S.
// The pages' minimal example issues before it waits; waiting first lets a
// single barrier serve both obligations of section 4 (never expose a stage
// early, never release one early) and keeps S-1 tiles in flight during the
// compute of tile t.
//
// vmcnt is this CDNA4 counterpart of cp.async.wait_group: a wave's vector
// memory loads complete in issue order, so "at most N outstanding" is
// "every load older than the N newest has landed" (section 3).
//
// A second pipeline runs inside compute(): LDS -> VGPR fragment reads of the
// next k-step are issued before the MFMAs of the current one (section 7).
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
typedef short i16x4_t __attribute__((ext_vector_type(4)));
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

// ---------------------------------------------------------------------------
// LDS swizzles.  XOR of the 16-byte chunk index with bits of the row keeps
// the fragment reads of one wave on distinct banks (checked with the LDS
// bank-conflict counter), for both the 8-lane and the 16-lane phase of a
// 128-bit read.
//
// K-contiguous tiles (A; B stored column-major): rows of NC chunks.
template <int NC>
__device__ __host__ constexpr int swz_k(int r)
{
    return NC == 4 ? (((r >> 1) ^ (r >> 3)) & 3) : NC == 8 ? ((r ^ (r >> 3)) & 7) : 0;
}
// N-contiguous tiles (B stored row-major): k-rows of NC chunks, read by
// ds_read_b64_tr_b16 (ELT 2), ds_read_b64_tr_b8 (ELT 1) or ds_read_b32 (ELT 4).
template <int ELT, int NC>
__device__ __host__ constexpr int swz_n(int r)
{
    const int v = ELT == 2   ? (((r & 3) | (((r >> 3) & 1) << 2)) << 1)
                  : ELT == 1 ? ((r & 7) | (((r >> 4) & 1) << 3))
                             : (((r >> 2) & 3) << 2);
    return v & (NC - 1);
}

// ---------------------------------------------------------------------------
template <int DT_, bool BCOL_, int TILE_, int V_, int S_>
struct Cfg {
    static constexpr int DT = DT_;
    static constexpr bool BCOL = BCOL_;
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
    static constexpr int KSTEPS = BK / KSTEP;
    static constexpr int NCA = kTiles[TILE_].BKB / 16;  // chunks per row of A (and of B col-major)
    static constexpr int NCBR = BN * ELT / 16;          // chunks per k-row of B row-major
    static constexpr int A_BYTES = BM * BK * ELT;
    static constexpr int B_BYTES = BK * BN * ELT;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    static constexpr int LDS_BYTES = S * STAGE_BYTES;
    static constexpr int A_CPT = A_BYTES / 16 / THREADS;  // 16-byte copies per thread per stage
    static constexpr int B_CPT = B_BYTES / 16 / THREADS;
    static constexpr int LOADS = A_CPT + B_CPT;            // vmcnt units per tile per thread

    static_assert(BK % KSTEP == 0, "BK must hold whole MFMA steps");
    static_assert(A_BYTES % (16 * THREADS) == 0 && B_BYTES % (16 * THREADS) == 0,
                  "a stage must split into whole 16-byte copies per thread");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must hold whole 16x16 MFMA tiles");
    static_assert(LDS_BYTES <= kLdsPerCu, "LDS ring exceeds 160 KiB");
    static_assert(V_ != V_SYNC || S_ == 1, "SYNC has one stage");
    static_assert(V_ != V_REG || (S_ == 1 || S_ == 2), "REG has 1 or 2 stages");
    static_assert(V_ != V_DIRECT || (S_ == 2 || S_ == 3), "DIRECT has 2 or 3 stages");
    static_assert((S_ >= 2 ? (S_ - 2) * LOADS : 0) < 64, "vmcnt range");
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
        // so lane group g supplies k = 4g + j to both operands.
        // (whole-vector bit casts: a bit cast of one vector element is not used, it
        // does not honour the element index)
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
// s_waitcnt vmcnt + s_barrier placement is the only synchronisation.  The
// s_nop covers the M0-write -> LDS-DMA hazard.
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

    // Per-thread copy geometry (loop invariant).
    struct Copy {
        int a_voff[C::A_CPT];  // byte offset of this thread's A chunks from the tile base
        int b_voff[C::B_CPT];
    };
    // Per-lane LDS fragment offsets within one stage (loop invariant).
    struct Frag {
        int a[C::FM][C::KSTEPS];
        int b[C::FN][C::BCOL ? C::KSTEPS : 1];
    };

    // A chunk q of a stage sits at LDS byte 16q; it holds logical chunk c of row r.
    static __device__ __forceinline__ void a_chunk(int q, int& r, int& c)
    {
        r = q / C::NCA;
        c = (q % C::NCA) ^ swz_k<C::NCA>(r);
    }
    static __device__ __forceinline__ void b_chunk(int q, int& r, int& c)
    {
        if constexpr (C::BCOL) {
            r = q / C::NCA;
            c = (q % C::NCA) ^ swz_k<C::NCA>(r);
        } else {
            r = q / C::NCBR;
            c = (q % C::NCBR) ^ swz_n<C::ELT, C::NCBR>(r);
        }
    }

    static __device__ void setup_copy(const GemmArgs& p, int m0, int n0, int tid, Copy& cp)
    {
        const int rows_a = min(C::BM, p.M - m0);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) {
            int r, c;
            a_chunk(i * C::THREADS + tid, r, c);
            r = min(r, rows_a - 1);  // M edge: any in-range row (its outputs are not stored)
            cp.a_voff[i] = r * p.lda * C::ELT + c * 16;
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int r, c;
            b_chunk(i * C::THREADS + tid, r, c);
            if constexpr (C::BCOL) {
                r = min(r, min(C::BN, p.N - n0) - 1);  // N edge
                cp.b_voff[i] = r * p.ldb * C::ELT + c * 16;
            } else {
                if (n0 + c * C::CE >= p.N) c = 0;  // N edge: any in-range chunk
                cp.b_voff[i] = r * p.ldb * C::ELT + c * 16;
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
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_a(const GemmArgs& p, int m0, int t)
    {
        const char* b;
        uint32_t n;
        span_a(p, m0, t, b, n);
        return make_rsrc(b, n);
    }
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc_b(const GemmArgs& p, int n0, int t)
    {
        const char* b;
        uint32_t n;
        span_b(p, n0, t, b, n);
        return make_rsrc(b, n);
    }

    // V_DIRECT producer: issue all copies of tile t into the stage at `st`.
    // Each buffer_load ... lds writes 64 x 16 contiguous bytes at M0, so the
    // copies of wave w, instruction i cover stage chunks [i*THREADS + 64w, +64).
    static __device__ __forceinline__ void issue_direct(const GemmArgs& p, int m0, int n0, int t,
                                                        SPT_LDS char* st, int wave, const Copy& cp)
    {
        const char *pa, *pb;
        uint32_t na, nb;
        span_a(p, m0, t, pa, na);
        span_b(p, n0, t, pb, nb);
        const i32x4_t ra = rsrc_words(pa, na);
        const i32x4_t rb = rsrc_words(pb, nb);
        const uint32_t base = (uint32_t)(uintptr_t)st;
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i)
            dma16(ra, base + (i * C::THREADS + wave * 64) * 16, cp.a_voff[i]);
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i)
            dma16(rb, base + C::A_BYTES + (i * C::THREADS + wave * 64) * 16, cp.b_voff[i]);
    }

    // V_REG / V_SYNC producer, part 1: global -> VGPR.
    static __device__ __forceinline__ void load_regs(const GemmArgs& p, int m0, int n0, int t,
                                                     const Copy& cp, i32x4_t (&ra_)[C::A_CPT],
                                                     i32x4_t (&rb_)[C::B_CPT])
    {
        const __amdgpu_buffer_rsrc_t ra = rsrc_a(p, m0, t);
        const __amdgpu_buffer_rsrc_t rb = rsrc_b(p, n0, t);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) ra_[i] = __builtin_amdgcn_raw_buffer_load_b128(ra, cp.a_voff[i], 0, 0);
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) rb_[i] = __builtin_amdgcn_raw_buffer_load_b128(rb, cp.b_voff[i], 0, 0);
    }

    // Producer, part 2: VGPR -> LDS (ds_write_b128 at the chunk's stage position).
    static __device__ __forceinline__ void store_regs(SPT_LDS char* st, int tid,
                                                      const i32x4_t (&ra_)[C::A_CPT],
                                                      const i32x4_t (&rb_)[C::B_CPT])
    {
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i)
            *(SPT_LDS i32x4_t*)(st + (i * C::THREADS + tid) * 16) = ra_[i];
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
        const __amdgpu_buffer_rsrc_t ra = rsrc_a(p, m0, t);
        const __amdgpu_buffer_rsrc_t rb = rsrc_b(p, n0, t);
        const int rows_a = min(C::BM, p.M - m0);
#pragma unroll
        for (int i = 0; i < C::A_CPT; ++i) {
            int r, c;
            a_chunk(i * C::THREADS + tid, r, c);
            r = min(r, rows_a - 1);
            const int valid = kt - c * C::CE;  // elements of this chunk below K
            const int voff = r * p.lda * C::ELT + (valid > 0 ? c * 16 : 0);
            ra_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(ra, voff, 0, 0), valid * C::ELT);
        }
#pragma unroll
        for (int i = 0; i < C::B_CPT; ++i) {
            int r, c;
            b_chunk(i * C::THREADS + tid, r, c);
            if constexpr (C::BCOL) {
                r = min(r, min(C::BN, p.N - n0) - 1);
                const int valid = kt - c * C::CE;
                const int voff = r * p.ldb * C::ELT + (valid > 0 ? c * 16 : 0);
                rb_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0), valid * C::ELT);
            } else {
                if (n0 + c * C::CE >= p.N) c = 0;
                const bool ok = r < kt;  // k-row of this chunk below K
                const int voff = (ok ? r : 0) * p.ldb * C::ELT + c * 16;
                rb_[i] = keep_bytes(__builtin_amdgcn_raw_buffer_load_b128(rb, voff, 0, 0), ok ? 16 : 0);
            }
        }
    }

    static __device__ void setup_frag(int wm0, int wn0, int lane, Frag& f)
    {
        const int l16 = lane & 15, g = lane >> 4;
#pragma unroll
        for (int m = 0; m < C::FM; ++m)
#pragma unroll
            for (int s = 0; s < C::KSTEPS; ++s) {
                const int r = wm0 + 16 * m + l16;
                const int c = 4 * s + g;
                f.a[m][s] = r * C::NCA * 16 + ((c ^ swz_k<C::NCA>(r)) * 16);
            }
#pragma unroll
        for (int n = 0; n < C::FN; ++n) {
            if constexpr (C::BCOL) {
#pragma unroll
                for (int s = 0; s < C::KSTEPS; ++s) {
                    const int r = wn0 + 16 * n + l16;
                    const int c = 4 * s + g;
                    f.b[n][s] = C::A_BYTES + r * C::NCA * 16 + ((c ^ swz_k<C::NCA>(r)) * 16);
                }
            } else if constexpr (C::ELT == 2) {
                // ds_read_b64_tr_b16: in each 16-lane group, lane i fetches 4 elements of
                // k-row (i / 4) at columns 4*(i % 4) .. +3; afterwards lane j holds the 4
                // k-rows of column j.  Offsets for (s, h) = (0, 0); the swizzle does not
                // depend on the k-row bits that s and h add.
                const int kr = 8 * g + (l16 >> 2);
                const int col = wn0 + 16 * n + 4 * (l16 & 3);
                const int c = col / 8;
                f.b[n][0] = C::A_BYTES + kr * C::NCBR * 16 + ((c ^ swz_n<2, C::NCBR>(kr)) * 16) +
                            (col % 8) * 2;
            } else if constexpr (C::ELT == 1) {
                // ds_read_b64_tr_b8: lane i fetches 8 bytes of k-row (i / 2) at columns
                // 8*(i % 2) .. +7; afterwards lane j holds 8 k-rows of column j.
                const int kr = 16 * g + (l16 >> 1);
                const int col = wn0 + 16 * n + 8 * (l16 & 1);
                const int c = col / 16;
                f.b[n][0] = C::A_BYTES + kr * C::NCBR * 16 + ((c ^ swz_n<1, C::NCBR>(kr)) * 16) +
                            (col % 16);
            } else {
                // fp32, ds_read_b32: lane (g, j) reads k-row 4g + j' for MFMA j'.
                const int kr = 4 * g;
                const int col = wn0 + 16 * n + l16;
                const int c = col / 4;
                f.b[n][0] = C::A_BYTES + kr * C::NCBR * 16 + ((c ^ swz_n<4, C::NCBR>(kr)) * 16) +
                            (col % 4) * 4;
            }
        }
    }

    static __device__ __forceinline__ i32x4_t read_a(const SPT_LDS char* st, const Frag& f, int m, int s)
    {
        return *(const SPT_LDS i32x4_t*)(st + f.a[m][s]);
    }
    static __device__ __forceinline__ i32x4_t read_b(const SPT_LDS char* st, const Frag& f, int n, int s)
    {
        if constexpr (C::BCOL) {
            return *(const SPT_LDS i32x4_t*)(st + f.b[n][s]);
        } else if constexpr (C::ELT == 2) {
            typedef __fp16 fp16x4_raw __attribute__((__vector_size__(4 * sizeof(__fp16))));
            const SPT_LDS char* b = st + f.b[n][0] + s * C::KSTEP * C::NCBR * 16;
            const fp16x4_raw lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS fp16x4_raw*)b);
            const fp16x4_raw hi =
                __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS fp16x4_raw*)(b + 4 * C::NCBR * 16));
            const i32x2_t l2 = __builtin_bit_cast(i32x2_t, lo), h2 = __builtin_bit_cast(i32x2_t, hi);
            return (i32x4_t){l2.x, l2.y, h2.x, h2.y};
        } else if constexpr (C::ELT == 1) {
            const SPT_LDS char* b = st + f.b[n][0] + s * C::KSTEP * C::NCBR * 16;
            const i32x2_t lo = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SPT_LDS i32x2_t*)b);
            const i32x2_t hi = __builtin_amdgcn_ds_read_tr8_b64_v2i32((SPT_LDS i32x2_t*)(b + 8 * C::NCBR * 16));
            return (i32x4_t){lo.x, lo.y, hi.x, hi.y};
        } else {
            const SPT_LDS char* b = st + f.b[n][0] + s * C::KSTEP * C::NCBR * 16;
            i32x4_t v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = *(const SPT_LDS int*)(b + j * C::NCBR * 16);
            return v;
        }
    }

    // Consume one stage: KSTEPS MFMA steps over the FM x FN tiles of this wave.
    // Register double buffer: the fragments of step s+1 are read before the
    // MFMAs of step s are issued.
    static __device__ __forceinline__ void compute(const SPT_LDS char* st, const Frag& f,
                                                   acc_t (&acc)[C::FM][C::FN])
    {
        i32x4_t af[2][C::FM], bf[2][C::FN];
#pragma unroll
        for (int m = 0; m < C::FM; ++m) af[0][m] = read_a(st, f, m, 0);
#pragma unroll
        for (int n = 0; n < C::FN; ++n) bf[0][n] = read_b(st, f, n, 0);
#pragma unroll
        for (int s = 0; s < C::KSTEPS; ++s) {
            const int cur = s & 1, nxt = cur ^ 1;
            if (s + 1 < C::KSTEPS) {
#pragma unroll
                for (int m = 0; m < C::FM; ++m) af[nxt][m] = read_a(st, f, m, s + 1);
#pragma unroll
                for (int n = 0; n < C::FN; ++n) bf[nxt][n] = read_b(st, f, n, s + 1);
            }
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int n = 0; n < C::FN; ++n) mma<C::DT>(acc[m][n], bf[cur][n], af[cur][m]);
        }
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

        Copy cp;
        setup_copy(p, m0, n0, tid, cp);
        Frag fr;
        setup_frag(wm0, wn0, lane, fr);

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
                compute(smem, fr, acc);
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
                compute(cur, fr, acc);
                if constexpr (C::S == 1) barrier();  // one buffer: all reads of it done first
                if (more) {
                    wait_vmcnt<0>();
                    store_regs(nxt, tid, ra, rb);
                }
                wait_lgkmcnt0();
                barrier();
            }
        } else {
            // V_DIRECT: S-stage ring.  Prologue: tiles 0..S-2 into stages 0..S-2.
#pragma unroll
            for (int i = 0; i < C::S - 1; ++i)
                if (i < nf) issue_direct(p, m0, n0, i, smem + i * C::STAGE_BYTES, wave, cp);
            int rs = 0;           // read stage (consumer)
            int ws = C::S - 1;    // write stage (producer)
            for (int t = 0; t < nf; ++t) {
                if (t + C::S - 2 < nf)
                    wait_vmcnt<(C::S - 2) * C::LOADS>();  // tiles t+1..t+S-2 may stay in flight
                else
                    wait_vmcnt<0>();
                barrier();
                if (t + C::S - 1 < nf) {
                    issue_direct(p, m0, n0, t + C::S - 1, smem + ws * C::STAGE_BYTES, wave, cp);
                    ws = ws + 1 == C::S ? 0 : ws + 1;
                }
                compute(smem + rs * C::STAGE_BYTES, fr, acc);
                rs = rs + 1 == C::S ? 0 : rs + 1;
            }
        }

        if (p.k_tail) {  // partial last tile, zero-filled beyond K, through VGPRs
            load_tail(p, m0, n0, tid, ra, rb);
            wait_vmcnt<0>();
            barrier();  // every wave is done reading the stages
            store_regs(smem, tid, ra, rb);
            wait_lgkmcnt0();
            barrier();
            compute(smem, fr, acc);
        }

        store_c(p, m0, n0, wm0, wn0, lane, acc);
    }
};

// Two waves per SIMD: two 256-thread workgroups, or one 512-thread workgroup,
// per CU; the compiler keeps VGPR + AGPR use within 256 per lane.
template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(2, 2))) void gemm_kernel(GemmArgs p)
{
    Gemm<C>::run(p);
}

}  // namespace spt
