// spt_attention.hip -- the attention-style consumer of the K/V ring: a
// flash-attention forward pass, O = softmax(scale * Q K^T) V, for gfx950.
//
// "Kernel-Engpass analysieren" uses flash attention as its high-ratio kernel:
// many matrix instructions per tile load (Schritt 4), so that long compute
// phases already hide the load latency and asynchronous copies stop paying
// (the pitfalls section reports them a few percent slower there).  This file
// streams blocks of keys and values through the same three producers as the
// GEMM K-loop (spt_kernel.hpp), so the claim can be measured here:
//
//  V_SYNC    load -> barrier -> compute -> barrier, one LDS stage;
//  V_REG     block t+1 fetched global -> VGPR while block t is computed, then
//            written to LDS (S = 1 or 2 stages); the fetch is issued once block
//            t's S = Q K^T is done, when the registers it needs are free;
//  V_DIRECT  buffer_load_dwordx4 ... lds copies into an S-stage ring (S = 2
//            or 3): wait -> barrier -> copies of block t+S-1 into the stage
//            just freed -> compute block t ("Hiding Memory Latency in CUDA:
//            Asynchronous Loads and Software Pipelines", sections 3-5).
//
// One workgroup of 8 waves (two per SIMD, so that one wave's scalar, LDS and
// wait instructions issue beside the other's vector work) owns 256 query rows
// of one (batch, head) slice; each wave owns 32 rows, whose Q fragments stay in
// registers for the whole kernel.  For every block of BKV keys (64; 32 with 128
// columns, whose accumulators leave fewer registers) a wave computes
//     S = Q K^T           (v_mfma_f32_16x16x32, one per 16 x 16 score block and
//                          32-wide d-step),
//     the online softmax  (a reference row maximum m and a rescale of the output
//                          accumulators and row sums by 2^(m_old - m_new) when m
//                          moves; P = 2^(c S - m), rounded to the input type),
//     O += P V            (16-bit MFMAs),
//     l += P 1            (the row sums of the rounded P: one more MFMA per row
//                          block, against a fragment of ones),
// and finally writes O / l in fp32: the weights P / l of a row sum to one over
// the very values the second product used.  Exponentials are base 2 with
// log2(e) folded into the scale c.
//
// MFMA layouts (operands swapped as in the GEMM: the K or V fragment is the
// first operand).  S block (m, n): lane (g = lane/16, i = lane%16) holds query
// row 16m + i, keys 16n + 4g + 0..3.  The P fragment of key-step u takes, in
// this order, the keys 32u + 4g + 0..3 and 32u + 16 + 4g + 0..3 of its row --
// an MFMA may contract its 32 k values in any order, as long as the V
// fragment supplies the same keys in the same positions: two transposing
// ds_read_b64_tr_b16 reads at key rows 32u + 4g + (i/4) and 32u + 16 + 4g +
// (i/4).  O block (m, n): lane holds query row 16m + i, columns 16n + 4g + 0..3
// (one 16-byte store).
//
// LDS stage: the K block (BKV rows of 2D bytes) then the V block.  K rows are
// read 16 at a time at one 16-byte chunk (ds_read_b128), so chunk c of row r
// sits at c ^ (r' mod chunks) with r' = r / (rows per 256-byte bank line); V is
// read by 16 rows x 32 bytes (the transposing reads), so its chunk pairs are
// XOR-ed by (r' mod pairs).  The producer computes which global chunk belongs
// at each position; a copy of one wave moves 1 KiB of whole rows.
//
// Edges.  Keys past Sk: K and V are read through one descriptor per slice,
// which ends at the slice, so the last block's copies read zeros there, and
// those keys get no maximum and weight 0.  Query rows past Sq read zeros and
// are never stored.
//
// Loops.  The DIRECT loop is unrolled by one turn of the ring (the two-stage
// REG loop by two blocks), so that each block's LDS stage is a constant folded
// into the immediate offsets of its fragment reads.
//
// Registers.  This unit is built with every MFMA in its VGPR form (the build
// passes -amdgpu-mfma-vgpr-form to the compiler): the softmax reads the scores
// and the rare rescale multiplies the output accumulators where the vector ALU
// can reach them, with no accumulator-register copies, and the whole kernel
// still fits the 256 registers per lane that two waves per SIMD leave.
#include <hip/hip_runtime.h>

#include <math.h>

#include "spt_kernel.hpp"
#include "spt_registry.h"

namespace spt {

struct AttnArgs {
    const char* Q;
    const char* K;
    const char* V;
    char* O;
    int BH, Sq, Sk;
    int q_blocks;  // ceil(Sq / 256)
    int kv_blocks; // ceil(Sk / BKV)
    float c;       // scale * log2(e)
};

template <int DT_, int D_, int V_, int S_>
struct AttnCfg {
    static constexpr int DT = DT_, D = D_, V = V_, S = S_;
    static constexpr int WAVES = 8, THREADS = 64 * WAVES;  // two waves per SIMD
    static constexpr int WQ = 32, BQ = WAVES * WQ;  // query rows per wave / per workgroup
    static constexpr int BKV = D_ == 128 ? 32 : 64;  // keys per block (128 columns: 32, for registers)
    static constexpr int FM = WQ / 16;              // 16-row query blocks per wave
    static constexpr int NB = BKV / 16;             // 16-key blocks per key block
    static constexpr int KS = D / 32;               // d-steps of Q K^T
    static constexpr int US = BKV / 32;             // key-steps of P V
    static constexpr int DN = D / 16;               // 16-column blocks of O
    static constexpr int RB = D * 2;                // bytes per row of Q, K, V
    static constexpr int NCH = RB / 16;             // 16-byte chunks per row
    static constexpr int RPL = 256 / RB;            // rows per 256-byte bank line
    static constexpr int KV_BYTES = BKV * RB;       // one K (or V) block
    static constexpr int STAGE_BYTES = 2 * KV_BYTES;
    static constexpr int LDS_BYTES = S * STAGE_BYTES;
    static constexpr int CPW = KV_BYTES / 1024 / WAVES;  // 1 KiB copies per wave per operand
    static constexpr int LOADS = 2 * CPW;                // copies per thread per block
    static_assert(D == 64 || D == 128, "head dimension 64 or 128");
    static_assert(CPW >= 1 && CPW <= 4, "a wave's copies of one operand share one M0 value");
    static_assert(V_ != V_SYNC || S_ == 1, "SYNC has one stage");
    static_assert(V_ != V_REG || S_ == 1 || S_ == 2, "REG has 1 or 2 stages");
    static_assert(V_ != V_DIRECT || S_ == 2 || S_ == 3, "DIRECT has 2 or 3 stages");
    static_assert(LDS_BYTES <= kLdsPerCu, "LDS ring exceeds 160 KiB");
    static_assert((S_ - 1) * LOADS < 64, "vmcnt range");
};

template <class C>
struct Attn {
    typedef f32x4_t acc_t;
    // How far (in the base-2 logit domain) a row's maximum may exceed the reference
    // before the reference moves: probabilities stay below 2^8, well inside fp16.
    static constexpr float kSlack = 8.0f;
    // A row's reference m and the bound m + kSlack its scaled maximum is tested against.
    struct RowRef {
        float m, thr;
    };

    static __device__ __forceinline__ constexpr int swz_k(int r) { return (r / C::RPL) & (C::NCH - 1); }
    static __device__ __forceinline__ constexpr int swz_v(int r) { return ((r / C::RPL) & (C::NCH / 2 - 1)) << 1; }

    // Global byte offset (from the block's first row) of the chunk that sits at LDS
    // byte p of the K (or V) region.
    template <bool IS_V>
    static __device__ __forceinline__ int src_of(int p)
    {
        const int r = p / C::RB, pc = (p % C::RB) / 16;
        const int lc = pc ^ (IS_V ? swz_v(r) : swz_k(r));
        return r * C::RB + lc * 16;
    }

    // Copies go in groups that share one M0 value: copy j adds the immediate j KiB
    // to its LDS and global address, so its register offset is lowered by as much
    // and raised by BIAS (the descriptor base is lowered by BIAS).
    static constexpr int BIAS = 3072;

    struct Copy {
        int goff[C::LOADS];  // global offset of copy j (K copies first, then V) within its block
    };

    static __device__ __forceinline__ i32x4_t desc(uint64_t base, uint32_t bytes)
    {
        return (i32x4_t){__builtin_amdgcn_readfirstlane((int)(uint32_t)base),
                         __builtin_amdgcn_readfirstlane((int)(uint32_t)(base >> 32)),
                         __builtin_amdgcn_readfirstlane((int)bytes), 0x00020000};
    }

    // One descriptor per operand for the whole slice: its base lowered by BIAS, its
    // extent the slice's bytes raised by as much.  Block t adds t x BKV rows to the
    // register offsets, so the copies of the last block read zeros past Sk and those of
    // blocks past the last read only zeros (the host keeps a slice within 2^31 bytes,
    // so no offset wraps).  Nothing is recomputed per block but that offset.
    static constexpr uint32_t BLK = (uint32_t)C::BKV * C::RB;  // bytes of one key block
    static __device__ __forceinline__ void slice_desc(const AttnArgs& p, int slice, i32x4_t& dk, i32x4_t& dv)
    {
        const long long row0 = (long long)slice * p.Sk;
        const uint32_t e = (uint32_t)p.Sk * C::RB + BIAS;
        dk = desc((uint64_t)(uintptr_t)(p.K + row0 * C::RB) - BIAS, e);
        dv = desc((uint64_t)(uintptr_t)(p.V + row0 * C::RB) - BIAS, e);
    }

    // DIRECT: the copies of one block into the stage at LDS byte address `st`.
    // DIRECT: the copies of block t (descriptors of its slice) into the stage at LDS
    // byte address `st`.
    static __device__ __forceinline__ void dma_block(const Copy& cp, i32x4_t dk, i32x4_t dv, uint32_t st, int wave,
                                                     int t)
    {
        const uint32_t mk = st + (uint32_t)(wave * C::CPW) * 1024u;
        const uint32_t mv = mk + (uint32_t)C::KV_BYTES;
        const uint32_t bo = (uint32_t)t * BLK + BIAS;
        static_for<0, C::CPW>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            dma16<j * 1024, j == 0>(dk, mk, (int)((uint32_t)cp.goff[j] - j * 1024u + bo));
        });
        static_for<0, C::CPW>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            dma16<j * 1024, j == 0>(dv, mv, (int)((uint32_t)cp.goff[C::CPW + j] - j * 1024u + bo));
        });
    }

#ifdef SPT_POISON
    // Race-detection builds only (never in the shipped library): before the copies of
    // a block are issued into a stage, this wave fills the 1 KiB blocks they will
    // refill with NaN and waits for those writes.  A read of the stage before its
    // copies land then turns the output into NaN.
    static __device__ __forceinline__ void poison(uint32_t st, int wave, int lane)
    {
        constexpr int pv = C::DT == DT_F16 ? 0x7E007E00 : 0x7FC07FC0;
        const i32x4_t v = {pv, pv, pv, pv};
#pragma unroll
        for (int j = 0; j < C::CPW; ++j) {
            const uint32_t o = st + (uint32_t)((wave * C::CPW + j) * 1024 + 16 * lane);
            *(SPT_LDS i32x4_t*)(size_t)o = v;
            *(SPT_LDS i32x4_t*)(size_t)(o + C::KV_BYTES) = v;
        }
        wait_lgkmcnt0();
    }
#endif

    // REG / SYNC: the same chunks through VGPRs, from one descriptor per operand for
    // the slice (reads past Sk return zeros).
    static __device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const char* base, const AttnArgs& p,
                                                                        int slice)
    {
        return make_rsrc(base + (long long)slice * p.Sk * C::RB, (uint32_t)p.Sk * C::RB);
    }
    static __device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int t,
                                                      const Copy& cp, i32x4_t (&r)[C::LOADS])
    {
        const uint32_t bo = (uint32_t)t * BLK;
#pragma unroll
        for (int j = 0; j < C::CPW; ++j)
            r[j] = __builtin_amdgcn_raw_buffer_load_b128(rk, (int)((uint32_t)cp.goff[j] + bo), 0, 0);
#pragma unroll
        for (int j = 0; j < C::CPW; ++j)
            r[C::CPW + j] = __builtin_amdgcn_raw_buffer_load_b128(rv, (int)((uint32_t)cp.goff[C::CPW + j] + bo), 0, 0);
    }
    static __device__ __forceinline__ void store_block(SPT_LDS char* st, int wave, int lane,
                                                       const i32x4_t (&r)[C::LOADS])
    {
#pragma unroll
        for (int j = 0; j < C::CPW; ++j)
            *(SPT_LDS i32x4_t*)(st + (wave * C::CPW + j) * 1024 + 16 * lane) = r[j];
#pragma unroll
        for (int j = 0; j < C::CPW; ++j)
            *(SPT_LDS i32x4_t*)(st + C::KV_BYTES + (wave * C::CPW + j) * 1024 + 16 * lane) = r[C::CPW + j];
    }

    // Per-lane LDS offsets of the fragment reads (row 0 of each fragment; other
    // rows add an immediate).
    struct Lanes {
        int k[C::KS];   // K fragment of d-step s (16 key rows x one chunk)
        int v[C::DN];   // V fragment of column block n (first transposing read)
    };
    static __device__ void setup_lanes(int lane, Lanes& L)
    {
        const int g = lane >> 4, i = lane & 15;
        // swz_k(16 n + i) == swz_k(i) and swz_v(32 u + 16 h + r) == swz_v(r): the block
        // offsets never reach the XOR bits
#pragma unroll
        for (int s = 0; s < C::KS; ++s) L.k[s] = i * C::RB + 16 * ((4 * s + g) ^ swz_k(i));
        const int r = 4 * g + (i >> 2);
#pragma unroll
        for (int n = 0; n < C::DN; ++n)
            L.v[n] = C::KV_BYTES + r * C::RB + 16 * ((2 * n + ((i & 3) >> 1)) ^ swz_v(r)) + 8 * (i & 1);
    }

    static __device__ __forceinline__ i32x4_t read_k(const SPT_LDS char* st, const Lanes& L, int n, int s)
    {
        return *(const SPT_LDS i32x4_t*)(st + L.k[s] + 16 * n * C::RB);
    }
    static __device__ __forceinline__ i32x4_t read_v(const SPT_LDS char* st, const Lanes& L, int n, int u)
    {
        const int o0 = L.v[n] + 32 * u * C::RB;
        const int o1 = o0 + 16 * C::RB;
        {  // (bf16 moves the same 16-bit patterns)
            typedef __fp16 raw4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
            const raw4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS raw4*)(st + o0));
            const raw4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4f16((SPT_LDS raw4*)(st + o1));
            const i32x2_t l2 = __builtin_bit_cast(i32x2_t, lo), h2 = __builtin_bit_cast(i32x2_t, hi);
            return (i32x4_t){l2.x, l2.y, h2.x, h2.y};
        }
    }

    // A fragment of ones in the input type: P against it gives P's row sums.
    static constexpr int kOneWord = C::DT == DT_F16 ? 0x3C003C00 : 0x3F803F80;
    static constexpr i32x4_t kOnes = {kOneWord, kOneWord, kOneWord, kOneWord};

    // Two probabilities -> one 32-bit word of the input type (round to nearest even).
    static __device__ __forceinline__ int pack2(float a, float b)
    {
        if constexpr (C::DT == DT_F16) {
            typedef _Float16 h2 __attribute__((ext_vector_type(2)));
            return __builtin_bit_cast(int, (h2){(_Float16)a, (_Float16)b});
        } else {
            typedef __bf16 b2 __attribute__((ext_vector_type(2)));
            return __builtin_bit_cast(int, (b2){(__bf16)a, (__bf16)b});
        }
    }

    static __device__ __forceinline__ float xmax(float v)
    {
        v = fmaxf(v, __shfl_xor(v, 16));
        return fmaxf(v, __shfl_xor(v, 32));
    }


    // One key block from the stage at `st`: S = Q K^T, online softmax, O += P V, by
    // 16-row query blocks m (FM of them), so that the vector-ALU work of one row
    // block's softmax is issued between the MFMAs of the next (a wave issues the next
    // few instructions while an MFMA runs; a softmax issued alone leaves the matrix
    // pipe idle):
    //     S(0);  S(m) | sm(m-1) for m = 1 .. FM-1;  PV(0) | sm(FM-1);  PV(1 .. FM-1)
    // S(m): the 8 MFMAs of row block m's scores (the block's K fragments are all read
    // first); sm(m): its softmax in 8 pieces, one after each MFMA of the group; PV(m):
    // the 8 MFMAs of O(m) += P(m) V (the V fragments are all read during the last S
    // group).  `mid` runs once every K fragment is dead.
    //
    // The scores stay unscaled until the exponent: the test compares c max S (c >= 0)
    // with the row's reference, and each probability is 2^(c S - m) with one fma (at
    // the row maximum, 2 to the rounding residue of c S, which rounds to 1 in the
    // input type for logits below 2^10 in magnitude).  Each lane tests its own
    // logits: a row needs a new reference when one of them exceeds it by more than
    // kSlack, which the wave learns from one ballot per row block; only then are the
    // row maxima reduced across the row's four lanes, the row's output and sum rescaled
    // by 2^(old - new), and its probabilities taken again.  Any reference gives the
    // same softmax; this one keeps the probabilities below 2^kSlack and spares the
    // accumulators a rescale on every block.  MASK (the last block): keys past Sk get
    // no maximum and weight 0.
    template <bool MASK, class F>
    static __device__ __forceinline__ void block(const AttnArgs& p, const SPT_LDS char* st, const Lanes& L,
                                                 const i32x4_t (&qf)[C::FM][C::KS], acc_t (&o)[C::FM][C::DN],
                                                 RowRef (&ref)[C::FM], acc_t (&lacc)[C::FM], int t, int lane, F&& mid)
    {
        constexpr int NK = C::KS * C::NB;  // K fragment f: d-step f / NB, key block f % NB
        constexpr int NF = C::US * C::DN;  // V fragment f: key-step f / DN, column block f % DN
        constexpr int E = 4 * C::NB;       // scores of one row block per lane: key 16 (e / 4) + e % 4
        static_assert(NK == 8 && NF == 8, "8 MFMAs per row block in both products");
        const int lim = p.Sk - t * C::BKV - 4 * (lane >> 4);  // keys 16 n + e < lim are inside Sk

        i32x4_t kf[NK], vf[NF];
        static_for<0, NK>([&](auto fc) {
            constexpr int f = decltype(fc)::value;
            kf[f] = read_k(st, L, f % C::NB, f / C::NB);
        });
        acc_t s[C::FM][C::NB];
#pragma unroll
        for (int m = 0; m < C::FM; ++m)
#pragma unroll
            for (int n = 0; n < C::NB; ++n) s[m][n] = (acc_t){0, 0, 0, 0};
        i32x4_t pf[C::FM][C::US];
        float lmax[C::FM], pe[C::FM][E];
        bool up[C::FM];

        // piece j (0 .. 7) of the softmax of row block m: the lane's maximum (0, 1) and
        // the test (1), the probabilities and their sum (2 .. 5), packing (6, 7)
        auto sm = [&](auto mc, auto jc) {
            constexpr int m = decltype(mc)::value, j = decltype(jc)::value;
            const auto sc = [&](int e) { return s[m][e / 4][e % 4]; };
            const auto valid = [&](int e) { return !MASK || 16 * (e / 4) + e % 4 < lim; };
            if constexpr (j == 0) {
                float mx = -INFINITY;
#pragma unroll
                for (int e = 0; e < E / 2; ++e) mx = fmaxf(mx, valid(e) ? sc(e) : -INFINITY);
                lmax[m] = mx;
            } else if constexpr (j == 1) {
                float mx = lmax[m];
#pragma unroll
                for (int e = E / 2; e < E; ++e) mx = fmaxf(mx, valid(e) ? sc(e) : -INFINITY);
                lmax[m] = mx;
                // (a row with no valid key has mx = -inf, and c mx is -inf or NaN: never above)
                up[m] = p.c * mx > ref[m].thr;
            } else if constexpr (j <= 5) {
#pragma unroll
                for (int e = (j - 2) * E / 4; e < (j - 1) * E / 4; ++e) {
                    const float v = __builtin_amdgcn_exp2f(__builtin_fmaf(sc(e), p.c, -ref[m].m));
                    pe[m][e] = valid(e) ? v : 0.f;
                    // (an empty use, so that the compiler does not sink this work past the
                    // ballot's branch, out of the MFMA group it is meant to overlap)
                    asm volatile("" ::"v"(pe[m][e]));
                }
            } else if constexpr (j - 6 < C::US) {
                constexpr int u = j - 6;
                const float* x = pe[m] + 8 * u;
                pf[m][u] = (i32x4_t){pack2(x[0], x[1]), pack2(x[2], x[3]), pack2(x[4], x[5]), pack2(x[6], x[7])};
                asm volatile("" ::"v"(pf[m][u]));
            }
        };
        // after sm(m): a new reference where the ballot asks for one
        auto settle = [&](auto mc) {
            constexpr int m = decltype(mc)::value;
            if (__builtin_expect(__builtin_amdgcn_ballot_w64(up[m]) != 0, 0)) {
                const float mx = xmax(lmax[m]);
                const float bmax = mx == -INFINITY ? -INFINITY : p.c * mx;  // (c = 0: every logit is 0)
                const float mnew = bmax > ref[m].thr ? bmax : ref[m].m;
                const float alpha = __builtin_amdgcn_exp2f(ref[m].m - mnew);  // 0 in the first block
                ref[m] = RowRef{mnew, mnew + kSlack};
                lacc[m] *= alpha;
#pragma unroll
                for (int n = 0; n < C::DN; ++n) o[m][n] *= alpha;
                static_for<2, 8>([&](auto jc) { sm(mc, jc); });  // the probabilities again
            }
        };
        // group: the 8 MFMAs of S(m) (PV = false) or PV(m), piece j of sm(k) after MFMA j
        // (k < 0: none), the V fragments read beside the MFMAs of the last S group
        auto group = [&](auto mc, auto pvc, auto kc) {
            constexpr int m = decltype(mc)::value, k = decltype(kc)::value;
            constexpr bool PV = decltype(pvc)::value;
            static_for<0, 8>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                if constexpr (PV)
                    mma<C::DT>(o[m][j % C::DN], vf[j], pf[m][j / C::DN]);
                else
                    mma<C::DT>(s[m][j % C::NB], kf[j], qf[m][j / C::NB]);
                if constexpr (k >= 0) sm(std::integral_constant<int, k>{}, jc);
                if constexpr (!PV && m == C::FM - 1) vf[j] = read_v(st, L, j % C::DN, j / C::DN);
                order_fence();
            });
            // PV(m) also takes the row sums of P(m): an MFMA against a fragment of ones
            if constexpr (PV)
                static_for<0, C::US>([&](auto uc) { mma<C::DT>(lacc[m], kOnes, pf[m][decltype(uc)::value]); });
        };
        // S(0); S(m) | sm(m-1) for m = 1 .. FM-1; PV(0) | sm(FM-1); PV(m) for m = 1 .. FM-1
        static_for<0, C::FM>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            group(mc, std::false_type{}, std::integral_constant<int, m - 1>{});
            if constexpr (m >= 1) settle(std::integral_constant<int, m - 1>{});
        });
        mid();
        group(std::integral_constant<int, 0>{}, std::true_type{}, std::integral_constant<int, C::FM - 1>{});
        settle(std::integral_constant<int, C::FM - 1>{});
        static_for<1, C::FM>([&](auto mc) { group(mc, std::true_type{}, std::integral_constant<int, -1>{}); });
    }

    // XCD-aware placement: workgroups are dispatched round-robin over the 8 XCDs;
    // renumber so that each XCD gets a contiguous run, in which consecutive
    // workgroups are query blocks of one slice (they share its K and V in that
    // XCD's L2).
    static __device__ __forceinline__ void place(int bid, int total, int q_blocks, int& slice, int& qb)
    {
        const int q = total / 8, rem = total % 8;
        const int xcd = bid % 8, j = bid / 8;
        const int id = (xcd < rem ? xcd * (q + 1) : rem * (q + 1) + (xcd - rem) * q) + j;
        slice = id / q_blocks;
        qb = id - slice * q_blocks;
    }

    static __device__ __forceinline__ void run(const AttnArgs& p)
    {
        __shared__ __attribute__((aligned(1024))) char smem_raw[C::LDS_BYTES];
        SPT_LDS char* smem = (SPT_LDS char*)smem_raw;
        const uint32_t lds0 = (uint32_t)(uintptr_t)smem;

        const int tid = threadIdx.x, lane = tid & 63;
        const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
        const int g = lane >> 4, i = lane & 15;
        int slice_, qb_;
        place(blockIdx.x, p.BH * p.q_blocks, p.q_blocks, slice_, qb_);
        const int slice = __builtin_amdgcn_readfirstlane(slice_), qb = __builtin_amdgcn_readfirstlane(qb_);
        const int qw = qb * C::BQ + wave * C::WQ;  // this wave's first query row

        // Q fragments (m, s): row 16 m + i, chunk 4 s + g; rows past Sq read zeros
        i32x4_t qf[C::FM][C::KS];
        {
            const long long row0 = (long long)slice * p.Sq + qw;
            const int rows = max(0, min(C::WQ, p.Sq - qw));
            const __amdgpu_buffer_rsrc_t rq = make_rsrc(p.Q + row0 * C::RB, (uint32_t)(rows * C::RB));
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int s = 0; s < C::KS; ++s)
                    qf[m][s] = __builtin_amdgcn_raw_buffer_load_b128(rq, (16 * m + i) * C::RB + (4 * s + g) * 16, 0, 0);
            // Take the fragments here (an empty use), so that the waits for these loads
            // stay out of the key loop, where they would also wait for the ring's copies.
#pragma unroll
            for (int m = 0; m < C::FM; ++m)
#pragma unroll
                for (int s = 0; s < C::KS; ++s) asm volatile("" : "+v"(qf[m][s]));
        }

        Copy cp;
#pragma unroll
        for (int j = 0; j < C::CPW; ++j) {
            cp.goff[j] = src_of<false>((wave * C::CPW + j) * 1024 + 16 * lane);
            cp.goff[C::CPW + j] = src_of<true>((wave * C::CPW + j) * 1024 + 16 * lane);
        }
        Lanes L;
        setup_lanes(lane, L);

        acc_t o[C::FM][C::DN];
        RowRef ref[C::FM];
        acc_t lacc[C::FM];  // row sums of the probabilities: every element of lane (g, i) holds row i's
#pragma unroll
        for (int m = 0; m < C::FM; ++m) {
            ref[m] = RowRef{-INFINITY, -INFINITY};
            lacc[m] = (acc_t){0, 0, 0, 0};
#pragma unroll
            for (int n = 0; n < C::DN; ++n) o[m][n] = (acc_t){0, 0, 0, 0};
        }

        const int nb = p.kv_blocks;
        if constexpr (C::V == V_DIRECT) {
            i32x4_t dk, dv;
            slice_desc(p, slice, dk, dv);
            // prologue: blocks 0 .. S-2 into stages 0 .. S-2
#pragma unroll
            for (int b = 0; b < C::S - 1; ++b) {
#ifdef SPT_POISON
                poison(lds0 + b * C::STAGE_BYTES, wave, lane);
#endif
                dma_block(cp, dk, dv, lds0 + b * C::STAGE_BYTES, wave, b);
            }
            // rs: the stage of block t; ws: the stage of block t + S - 1 (that of t - 1)
            auto step = [&](int t, auto last, auto rs, auto ws) {
                wait_lgkmcnt0();                              // this wave's reads of block t-1 are done
                wait_vmcnt<(C::S - 2) * C::LOADS>();          // its copies of block t have landed
                barrier();                                    // block t visible; the stage of t-1 free
#ifdef SPT_POISON
                poison(lds0 + ws, wave, lane);
#endif
                dma_block(cp, dk, dv, lds0 + ws, wave, t + C::S - 1);  // block t+S-1 into that stage
                block<decltype(last)::value>(p, smem + rs, L, qf, o, ref, lacc, t, lane, [] {});
            };
            // Whole turns of the ring, unrolled, so that each block's stage is a constant
            // (folded into the offsets of its LDS reads); none of them holds the last block.
            int t = 0;
            for (; t + C::S < nb; t += C::S)
                static_for<0, C::S>([&](auto jc) {
                    constexpr int j = decltype(jc)::value;
                    step(t + j, std::false_type{}, std::integral_constant<uint32_t, j * C::STAGE_BYTES>{},
                         std::integral_constant<uint32_t, (j + C::S - 1) % C::S * C::STAGE_BYTES>{});
                });
            // the rest (block t in stage 0), the last block with the mask
            uint32_t rs = 0, ws = (C::S - 1) * C::STAGE_BYTES;
            for (; t + 1 < nb; ++t) {
                step(t, std::false_type{}, rs, ws);
                rs = rs + C::STAGE_BYTES == (uint32_t)C::LDS_BYTES ? 0u : rs + C::STAGE_BYTES;
                ws = ws + C::STAGE_BYTES == (uint32_t)C::LDS_BYTES ? 0u : ws + C::STAGE_BYTES;
            }
            if (nb > 0) step(nb - 1, std::true_type{}, rs, ws);
            wait_vmcnt<0>();  // no copy may still be writing this workgroup's LDS
        } else if constexpr (C::V == V_REG) {
            const __amdgpu_buffer_rsrc_t rk = slice_rsrc(p.K, p, slice), rv = slice_rsrc(p.V, p, slice);
            i32x4_t r[C::LOADS];
            if (nb > 0) {  // prologue: block 0 into stage 0
                load_block(rk, rv, 0, cp, r);
                wait_vmcnt<0>();
                store_block(smem, wave, lane, r);
                wait_lgkmcnt0();
                barrier();
            }
            // cs: the stage of block t; ns: that of block t + 1
            auto step = [&](int t, auto last, auto cs, auto ns) {
                // block t+1 is fetched while block t is computed: issued once S = Q K^T is
                // done (before it, the K fragments hold the registers the fetch needs),
                // in flight over the softmax and O += P V (past the end: zero-length, zeros)
                block<decltype(last)::value>(p, smem + cs, L, qf, o, ref, lacc, t, lane,
                                             [&] { load_block(rk, rv, t + 1, cp, r); });
                if constexpr (C::S == 1) barrier();       // one buffer: every read of it done first
                wait_vmcnt<0>();
                store_block(smem + ns, wave, lane, r);
                wait_lgkmcnt0();
                barrier();
            };
            // pairs of blocks, unrolled for S = 2 so that the stages are constants; none of
            // them holds the last block
            using Z = std::integral_constant<uint32_t, 0>;
            using Z1 = std::integral_constant<uint32_t, (C::S - 1) * C::STAGE_BYTES>;
            int t = 0;
            if constexpr (C::S == 2)
                for (; t + 2 < nb; t += 2) {
                    step(t, std::false_type{}, Z{}, Z1{});
                    step(t + 1, std::false_type{}, Z1{}, Z{});
                }
            // the rest (block t in stage 0), the last block with the mask
            for (; t + 1 < nb; ++t) step(t, std::false_type{}, (t & 1) * Z1::value, ((t + 1) & 1) * Z1::value);
            if (nb > 0) step(nb - 1, std::true_type{}, ((nb - 1) & 1) * Z1::value, (nb & 1) * Z1::value);
        } else {
            const __amdgpu_buffer_rsrc_t rk = slice_rsrc(p.K, p, slice), rv = slice_rsrc(p.V, p, slice);
            i32x4_t r[C::LOADS];
            auto step = [&](int t, auto last) {  // load -> barrier -> compute -> barrier
                load_block(rk, rv, t, cp, r);
                wait_vmcnt<0>();
                store_block(smem, wave, lane, r);
                wait_lgkmcnt0();
                barrier();
                block<decltype(last)::value>(p, smem, L, qf, o, ref, lacc, t, lane, [] {});
                barrier();
            };
            for (int t = 0; t + 1 < nb; ++t) step(t, std::false_type{});
            if (nb > 0) step(nb - 1, std::true_type{});
        }

        // O = acc / l for the rows this wave owns inside Sq
#pragma unroll
        for (int m = 0; m < C::FM; ++m) {
            const float l = lacc[m][0];
            const int q = qw + 16 * m + i;
            if (q < p.Sq) {
                // (a correctly rounded division, not a product with 1 / l: where every value
                // row is the same power of two, O is that value exactly)
                char* row = p.O + ((long long)slice * p.Sq + q) * (C::D * 4);
#pragma unroll
                for (int n = 0; n < C::DN; ++n) *(acc_t*)(row + (16 * n + 4 * g) * 4) = o[m][n] / l;
            }
        }
    }
};

template <class C>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WAVES / 4, C::WAVES / 4))) void
attention_kernel(AttnArgs p)
{
    Attn<C>::run(p);
}

template <class C>
static hipError_t launch_attn(const AttnArgs& a, unsigned grid, hipStream_t stream)
{
    AttnArgs arg = a;
    arg.kv_blocks = (a.Sk + C::BKV - 1) / C::BKV;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&attention_kernel<C>, dim3(grid), dim3(C::THREADS), args, 0, stream);
}

typedef hipError_t (*AttnLaunch)(const AttnArgs&, unsigned, hipStream_t);

template <int DT, int D>
static AttnLaunch pick(int variant, int stages)
{
    if (variant == V_SYNC) return &launch_attn<AttnCfg<DT, D, V_SYNC, 1>>;
    if (variant == V_REG) return stages == 1 ? &launch_attn<AttnCfg<DT, D, V_REG, 1>> : &launch_attn<AttnCfg<DT, D, V_REG, 2>>;
    return stages == 2 ? &launch_attn<AttnCfg<DT, D, V_DIRECT, 2>> : &launch_attn<AttnCfg<DT, D, V_DIRECT, 3>>;
}

hipError_t launch_attention(int dtype, int D, int variant, int stages, const void* Q, const void* K, const void* V,
                            void* O, int BH, int Sq, int Sk, float c, hipStream_t stream)
{
    AttnArgs a;
    a.Q = (const char*)Q;
    a.K = (const char*)K;
    a.V = (const char*)V;
    a.O = (char*)O;
    a.BH = BH;
    a.Sq = Sq;
    a.Sk = Sk;
    a.q_blocks = (Sq + 255) / 256;
    a.c = c;
    AttnLaunch f = dtype == DT_F16 ? (D == 64 ? pick<DT_F16, 64>(variant, stages) : pick<DT_F16, 128>(variant, stages))
                                   : (D == 64 ? pick<DT_BF16, 64>(variant, stages) : pick<DT_BF16, 128>(variant, stages));
    return f(a, (unsigned)(BH * a.q_blocks), stream);
}

}  // namespace spt
