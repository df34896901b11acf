// spt_persist.hpp -- the DIRECT ring run by persistent workgroups whose C
// stores overlap the K-loop of the next output tile.
//
// A grid of as many workgroups as the CUs hold at once (G) walks the output
// tiles in streams: workgroup b takes tiles b, b + G, b + 2G, ... of the
// XCD-aware order ("Hiding Memory Latency in CUDA ...", section 8, closing
// remark: a real workload spreads independent tile streams over the
// blocks).  With the 128 x 128 tile (64 x 64 per wave) both accumulator sets
// take 128 registers, so two workgroups share a CU and each SIMD runs two
// waves, one issuing while the other waits.  The ring of section 5 does not
// stop at a tile boundary: the prologue fills its S stages once, and the
// steady-state copies run on into the next tile's K tiles, so a tile's first
// K tiles are already in LDS when its K-loop starts.
//
// The epilogue of a tile is its C store.  In the one-tile-per-workgroup
// kernel it follows the K-loop with nothing left to overlap, and every CU
// reaches it at about the same time, so HBM idles while the MFMAs run and
// the reverse.  Here each wave keeps two accumulator sets: while the K-loop
// of tile c accumulates into one (its first k-step starts from zero), the
// other, tile c-1, is written to C with ST 16-byte stores per K tile over the
// first P K tiles (P x ST = the FM x FN 16x16 blocks of the wave tile).  The
// last tile of the stream is stored after the loop.
//
// vmcnt.  Copies and stores share the in-order counter.  Every K tile issues
// its LOADS copies and then exactly ST stores (stores to a zero-length range
// where there is nothing to write: past the store window, in the first
// tile's window and in the prologue), so one wait fits every K tile: at the
// end of K tile t, the copies of tile t + 1 have landed once at most
// (S - 2) x LOADS younger copies and (S - 1) x ST younger stores are pending.
//
// Scope: shapes that are whole multiples of the tile and of BK, with an
// even number of K tiles (the register slot of each tile's first k-step then
// has the same parity in every tile) and at least P of them.  The store
// window P is the longest of 2, 4, 8 that fits, so that the stores of a tile
// spread over its K-loop where K is short (where the C store, not the MFMAs,
// bounds the run), in pairs that complete 128-byte lines of C.
//
// Measured on MI355X this kernel is slower than the one-tile kernel of the
// same tile (bf16 8192 x 8192 x 128: 88 us against 62; x 2048: 380 against
// 300).  The copies and the stores of a wave share its in-order vmcnt, so the
// ring's wait for a K tile also waits for every store issued before that K
// tile's copies: each store has S - 1 K tiles to be acknowledged, and a C
// store under load takes longer.  The stores a wave keeps in flight are
// therefore capped at (S - 1) x ST, where the one-tile kernel issues its
// whole C tile and leaves without waiting.  Decoupling them needs other
// waves to issue the stores (C staged through LDS), for which the ring leaves
// no room at these tiles.
#pragma once

#include "spt_kernel.hpp"

namespace spt {

// Lambdas passed to static_for are inlined like the functions they stand for
// (an outlined copy would receive the buffer descriptors in VGPRs).
#define SPT_INLINE __attribute__((always_inline))

template <class C, int P>
struct Persist {
    typedef Gemm<C> G;
    typedef typename G::acc_t acc_t;
    typedef typename G::Slot Slot;
    typedef acc_t Acc[C::FM][C::FN];

    static constexpr int NJ = G::NJ;             // MFMA slots per K tile (one k-step)
    static constexpr int NBLK = C::FM * C::FN;   // 16x16 blocks of the wave tile
    static constexpr int ST = NBLK / P;          // stores per K tile
    static constexpr int VM_STEADY = (C::S - 2) * C::LOADS + (C::S - 1) * ST;
    static constexpr int VM_FIRST = (C::S - 1) * C::LOADS + C::S * ST;
    static_assert(VM_STEADY < 64, "vmcnt is a 6-bit counter");
    static_assert(C::V == V_PERSIST && C::EXACT && C::KS == 1, "one MFMA k-step per K tile, exact fit");
    static_assert(NBLK % P == 0 && P % 2 == 0 && P >= C::S - 1, "store window");
    static_assert(VM_FIRST < 64, "vmcnt is a 6-bit counter");
    static_assert(G::NFREE >= C::LOADS + 3, "free MFMA slots for copies and bookkeeping");

    // ---- issue plan of one K tile ------------------------------------------------
    // Fragment reads as in the one-tile kernel; the copies in the first LOADS
    // free slots, then the ring bookkeeping, and the stores spread over the
    // free slots after the copies (so that they follow them in vmcnt order).
    static constexpr int dma_at(int d) { return G::nth_free(d); }
    static constexpr int adv_at(int q) { return G::nth_free(C::LOADS + q); }
    static constexpr int st_at(int s) { return G::nth_free(C::LOADS + (s * (G::NFREE - C::LOADS)) / ST); }
    static constexpr int dma_owner(int j)
    {
        for (int d = 0; d < C::LOADS; ++d)
            if (dma_at(d) == j) return d;
        return -1;
    }
    static constexpr int adv_owner(int j)
    {
        for (int q = 0; q < 3; ++q)
            if (adv_at(q) == j) return q;
        return -1;
    }

    // ---- producer: the ring across output tiles --------------------------------------
    struct PRing {
        typename G::Ring r;
        int v;      // output tile whose K tiles the copies are walking
        int step;   // workgroups in the grid
        int total;  // output tiles
    };
    // Descriptors of K tile 0 of output tile q.v.
    static __device__ __forceinline__ void ring_tile(const GemmArgs& p, PRing& q)
    {
        int tm, tn;
        G::tile_of(q.v, p.tiles_m, p.tiles_n, tm, tn);
        // (the divisions of the tile order run on the vector ALU: pin the
        // results to scalar registers, or the loop-carried descriptors would
        // follow them into VGPRs, where a copy cannot take them)
        const int m0 = __builtin_amdgcn_readfirstlane(tm) * C::BM, n0 = __builtin_amdgcn_readfirstlane(tn) * C::BN;
        const uint64_t a = (uint64_t)(uintptr_t)(p.A + (long long)m0 * p.lda * C::ELT) - G::DMA_BIAS;
        uint64_t b;
        uint32_t nb = q.r.nb;
        if constexpr (C::BCOL) {
            b = (uint64_t)(uintptr_t)(p.B + (long long)n0 * p.ldb * C::ELT) - G::DMA_BIAS;
        } else {
            b = (uint64_t)(uintptr_t)(p.B + (long long)n0 * C::ELT) - G::DMA_BIAS;
            nb = (uint32_t)(((long long)C::BK * p.ldb - n0) * C::ELT) + G::DMA_BIAS;
        }
        q.r.qa = G::desc(a, q.r.na);
        q.r.qb = G::desc(b, nb);
        q.r.left = p.k_full;
    }
    static __device__ __forceinline__ void ring_init(const GemmArgs& p, int wave, const SPT_LDS char* smem,
                                                     PRing& q)
    {
        q.v = blockIdx.x;
        q.step = gridDim.x;
        q.total = p.tiles_m * p.tiles_n;
        q.r.sa = (uint64_t)C::BK * C::ELT;
        q.r.na = (uint32_t)(((long long)(C::BM - 1) * p.lda + C::BK) * C::ELT) + G::DMA_BIAS;
        if constexpr (C::BCOL) {
            q.r.sb = (uint64_t)C::BK * C::ELT;
            q.r.nb = (uint32_t)(((long long)(C::BN - 1) * p.ldb + C::BK) * C::ELT) + G::DMA_BIAS;
        } else {
            q.r.sb = (uint64_t)C::BK * p.ldb * C::ELT;
            q.r.nb = 0;  // per tile (depends on the tile's first column)
        }
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
        q.r.m0a = lds0 + (uint32_t)(wave * C::A_CPT) * 1024u;
        q.r.m0b = lds0 + (uint32_t)C::A_BYTES + (uint32_t)(wave * C::B_CPT) * 1024u;
        ring_tile(p, q);
    }
    // After a K tile's copies: the A base, the B base, then the count of K
    // tiles left in this output tile; at zero the ring moves to the stream's
    // next tile, or past its end to empty copies.
    static __device__ __forceinline__ void advance(const GemmArgs& p, PRing& q, int part)
    {
        if (part == 0) G::add64(q.r.qa, q.r.sa);
        if (part == 1) G::add64(q.r.qb, q.r.sb);
        if (part == 2) {
            if (--q.r.left == 0) {
                q.v += q.step;
                if (q.v < q.total) {
                    ring_tile(p, q);
                } else {
                    q.r.qa[2] = 0;
                    q.r.qb[2] = 0;
                }
            }
        }
    }

    // ---- C stores ----------------------------------------------------------------------
    // Output tile v as a buffer range: its first element, and every row it
    // touches (BM row pitches; the host checks the range fits in 31 bits).
    static __device__ __forceinline__ void c_range(const GemmArgs& p, int v, const char*& base, uint32_t& bytes)
    {
        int tm, tn;
        G::tile_of(v, p.tiles_m, p.tiles_n, tm, tn);
        tm = __builtin_amdgcn_readfirstlane(tm);
        tn = __builtin_amdgcn_readfirstlane(tn);
        base = p.C + ((long long)tm * C::BM * p.ldc + (long long)tn * C::BN) * 4;
        bytes = (uint32_t)(C::BM * p.ldc * 4);
    }
    // Block BLK (row-major over FM x FN) of a wave tile: lane (g, i) holds 4
    // consecutive columns 4g .. 4g+3 of row i of the block.  vc[m] is the
    // lane's byte offset of block row m, column block 0, from the tile origin.
    template <int BLK>
    static __device__ __forceinline__ void store_blk(const Acc& a, __amdgpu_buffer_rsrc_t rs, const int (&vc)[C::FM])
    {
        constexpr int m = BLK / C::FN, n = BLK % C::FN;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, a[m][n]), rs, vc[m] + 64 * n, 0, 0);
    }

    // ---- one K tile --------------------------------------------------------------------------
    // The MFMAs of the K tile whose fragments are in `use` (into `acc`, from
    // zero when FIRST), with: the copies of the K tile S ahead (d), the
    // fragments of the next K tile from `src` into `nxt`, the ring
    // bookkeeping, and stores of blocks SB .. SB+ST-1 of `out` to `rs`.
    template <bool FIRST, int SB>
    static __device__ __forceinline__ void kstep(const Slot& use, Slot& nxt, const SPT_LDS char* src,
                                                 const typename G::Lanes& L, const typename G::Dma& d,
                                                 const typename G::Copy& cp, const GemmArgs& p, PRing& q, Acc& acc,
                                                 const Acc& out, __amdgpu_buffer_rsrc_t rs, const int (&vc)[C::FM])
    {
        static_for<0, NJ>([&](auto jc) SPT_INLINE {
            constexpr int j = decltype(jc)::value;
            constexpr int m = j / C::FN, n = j % C::FN;
            constexpr int dj = dma_owner(j), aj = G::a_owner(j), qj = adv_owner(j);
            if constexpr (FIRST) acc[m][n] = (acc_t){0, 0, 0, 0};
            mma<C::DT>(acc[m][n], use[C::FM + n], use[m]);
            if constexpr (dj >= 0) G::template dma_issue<dj>(d, cp);
            if constexpr (j < C::FN) G::read_frag(src, L, 0, C::FM + j, nxt);
            if constexpr (aj >= 0) G::read_frag(src, L, 0, aj, nxt);
            if constexpr (qj >= 0) advance(p, q, qj);
            static_for<0, ST>([&](auto sc) SPT_INLINE {
                constexpr int s = decltype(sc)::value;
                if constexpr (st_at(s) == j) store_blk<SB + s>(out, rs, vc);
            });
            order_fence();
        });
    }

    // K tile of the ring stage at byte offset rs (advanced on return), its
    // fragments in register slot PAR.
    template <int PAR, bool FIRST, int SB>
    static __device__ __forceinline__ void ktile(uint32_t& rs, const typename G::Lanes& L, const SPT_LDS char* smem,
                                                 const typename G::Copy& cp, const GemmArgs& p, PRing& q,
                                                 Slot (&sl)[2], Acc& acc, const Acc& out,
                                                 __amdgpu_buffer_rsrc_t crs, const int (&vc)[C::FM])
    {
        const uint32_t nx = rs + C::STAGE_BYTES == (uint32_t)C::LDS_BYTES ? 0u : rs + C::STAGE_BYTES;
        wait_lgkmcnt0();             // this wave's reads of this K tile are complete
        wait_vmcnt<VM_STEADY>();     // its copies of the next K tile have landed
        barrier();                   // next K tile visible to all; this stage free
        const typename G::Dma d = G::dma_of(q.r, rs);
#ifdef SPT_POISON
        G::poison(q.r, rs);
#endif
        kstep<FIRST, SB>(sl[PAR], sl[PAR ^ 1], smem + nx, L, d, cp, p, q, acc, out, crs, vc);
        rs = nx;
    }

    // Output tile into set X while set X^1 (the previous tile) goes to `prev`.
    template <int X>
    static __device__ __forceinline__ void otile(uint32_t& rs, const typename G::Lanes& L, const SPT_LDS char* smem,
                                                 const typename G::Copy& cp, const GemmArgs& p, PRing& q,
                                                 Slot (&sl)[2], Acc (&acc)[2], __amdgpu_buffer_rsrc_t prev,
                                                 const int (&vc)[C::FM])
    {
        static_for<0, P>([&](auto ic) SPT_INLINE {
            constexpr int i = decltype(ic)::value;
            ktile<i & 1, i == 0, i * ST>(rs, L, smem, cp, p, q, sl, acc[X], acc[X ^ 1], prev, vc);
        });
        const __amdgpu_buffer_rsrc_t none = make_rsrc(p.C, 0);
        for (int i = P; i < p.k_full; i += 2) {
            ktile<0, false, 0>(rs, L, smem, cp, p, q, sl, acc[X], acc[X ^ 1], none, vc);
            ktile<1, false, 0>(rs, L, smem, cp, p, q, sl, acc[X], acc[X ^ 1], none, vc);
        }
    }

    template <int X>
    static __device__ __forceinline__ void store_all(const Acc& a, __amdgpu_buffer_rsrc_t rs, const int (&vc)[C::FM])
    {
        static_for<0, NBLK>([&](auto bc) SPT_INLINE { store_blk<decltype(bc)::value>(a, rs, vc); });
    }

    static __device__ __forceinline__ void run(const GemmArgs& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
        SPT_LDS char* smem = (SPT_LDS char*)smem_raw;

        const int tid = threadIdx.x;
        const int lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int wm0 = (wave / C::WAVES_N) * C::WTM, wn0 = (wave % C::WAVES_N) * C::WTN;

        typename G::Copy cp;  // exact fit: the same offsets for every tile
        G::setup_copy(p, 0, 0, tid, cp);
        typename G::Lanes L;
        G::setup_lanes(lane, wm0 / 16, wn0 / 16, L);
        int vc[C::FM];
#pragma unroll
        for (int m = 0; m < C::FM; ++m) vc[m] = ((wm0 + 16 * m + (lane & 15)) * p.ldc + wn0 + 4 * (lane >> 4)) * 4;

        Acc acc[2];
#pragma unroll
        for (int m = 0; m < C::FM; ++m)
#pragma unroll
            for (int n = 0; n < C::FN; ++n) acc[1][m][n] = (acc_t){0, 0, 0, 0};

        PRing q;
        ring_init(p, wave, smem, q);
        const __amdgpu_buffer_rsrc_t none = make_rsrc(p.C, 0);
        // prologue: K tiles 0 .. S-1 of the stream into stages 0 .. S-1, each
        // followed by ST empty stores (the per-tile vmcnt pattern of the loop)
#pragma unroll
        for (int i = 0; i < C::S; ++i) {
            const typename G::Dma d = G::dma_of(q.r, i * C::STAGE_BYTES);
            static_for<0, C::LOADS>([&](auto jc) SPT_INLINE { G::template dma_issue<decltype(jc)::value>(d, cp); });
            advance(p, q, 0);
            advance(p, q, 1);
            advance(p, q, 2);
            static_for<0, ST>([&](auto sc) SPT_INLINE { store_blk<decltype(sc)::value>(acc[1], none, vc); });
        }
        wait_vmcnt<VM_FIRST>();  // K tile 0 landed
        barrier();
        Slot sl[2];
        G::read_slot(smem, L, 0, sl[0]);

        uint32_t rs = 0;
        int v = blockIdx.x;
        const int step = gridDim.x, total = p.tiles_m * p.tiles_n;
        const char* cb;
        uint32_t cn;
        __amdgpu_buffer_rsrc_t prev = none;  // the first tile has no predecessor
        int last;
        for (;;) {
            otile<0>(rs, L, smem, cp, p, q, sl, acc, prev, vc);
            c_range(p, v, cb, cn);
            prev = make_rsrc(cb, cn);
            v += step;
            if (v >= total) {
                last = 0;
                break;
            }
            otile<1>(rs, L, smem, cp, p, q, sl, acc, prev, vc);
            c_range(p, v, cb, cn);
            prev = make_rsrc(cb, cn);
            v += step;
            if (v >= total) {
                last = 1;
                break;
            }
        }
        wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
        if (last == 0)
            store_all<0>(acc[0], prev, vc);
        else
            store_all<1>(acc[1], prev, vc);
    }
};

template <class C, int P>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD))) void
gemm_persist_kernel(GemmArgs p)
{
    Persist<C, P>::run(p);
}

}  // namespace spt
