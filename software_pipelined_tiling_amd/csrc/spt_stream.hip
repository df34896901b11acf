// spt_stream.hip -- the streaming pipeline of "Hiding Memory Latency in CUDA:
// Asynchronous Loads and Software Pipelines" (section 8, the minimal working
// example; section 9 walks through its schedule): every element of a float
// vector is scaled by two, y[i] = 2 x[i], with the input staged global -> LDS
// through an S-stage ring of asynchronous copies.
//
// gfx950 form.  A tile is 256 threads x 16 bytes = 1024 floats; each wave
// copies its 1 KiB with one buffer_load_dwordx4 ... lds.  Each block walks an
// independent stream of tiles b, b + G, b + 2G, ... (the page's closing
// remark: a real workload spreads independent tile streams over many
// blocks; one block reproduces its demonstration).
//
// Schedule for S >= 2, per tile j of the block's stream:
//     s_waitcnt vmcnt(2S - 3)   this thread's copy of tile j has landed
//     s_barrier                 every copy of tile j is visible, and every
//                               thread has consumed tile j-1 (its LDS read
//                               fed its store, which was issued before)
//     copy tile j + S - 1 into the stage of tile j - 1
//     ds_read_b128 of tile j, multiply by 2, buffer_store_dwordx4 to y
// so one barrier per tile serves both of section 4's obligations.  Copies
// and stores share the in-order vmcnt counter; every tile issues exactly one
// copy and one store per thread (the prologue pairs each copy with a store to
// an empty range), which makes the wait count the same constant on every
// tile.  Copies past the end of the stream have extent 0 (zero-filled
// stages, as the page turns out-of-range tiles into zero-filled stages) and
// stores are bounded to whole 16-byte chunks of y, so nothing is read or
// written out of range.  The one chunk that straddles n (n not a multiple of
// 4) is finished by scalar code after the ring.  S = 1 is the synchronous
// loop: copy, wait for everything, barrier, compute, barrier.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "spt_kernel.hpp"
#include "spt_registry.h"

namespace spt {

constexpr int kStreamThreads = 256;
constexpr int kStreamTileBytes = kStreamThreads * 16;  // 1024 floats

struct StreamArgs {
    const char* x;
    char* y;
    int64_t n;           // elements
    int64_t full_bytes;  // bytes of whole 16-byte chunks: 16 * floor(n / 4)
    int64_t tiles;       // ceil(n / 1024)
};

// Tile t of x or y as a buffer range: base at the tile, extent the bytes of
// whole chunks left from there (0 past the end, at most one tile).
__device__ __forceinline__ void stream_span(const char* base, int64_t t, int64_t full_bytes, const char*& p,
                                            uint32_t& bytes)
{
    const int64_t off = t * kStreamTileBytes;
    const int64_t rem = full_bytes - off;
    bytes = rem <= 0 ? 0u : rem >= kStreamTileBytes ? (uint32_t)kStreamTileBytes : (uint32_t)rem;
    p = base + (rem <= 0 ? 0 : off);
}
// The same range as the four descriptor words of an inline-asm copy.
__device__ __forceinline__ i32x4_t stream_desc(const char* base, int64_t t, int64_t full_bytes)
{
    const char* p;
    uint32_t bytes;
    stream_span(base, t, full_bytes, p, bytes);
    const uint64_t a = (uint64_t)(uintptr_t)p;
    return (i32x4_t){(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)bytes, 0x00020000};
}
// 16 bytes of this thread to tile t of y (dropped where the range is empty).
__device__ __forceinline__ void stream_store(char* y, int64_t t, int64_t full_bytes, int voff, f32x4_t v)
{
    const char* p;
    uint32_t bytes;
    stream_span(y, t, full_bytes, p, bytes);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4_t, v), make_rsrc(p, bytes), voff, 0, 0);
}

template <int S>
__global__ __launch_bounds__(kStreamThreads) void scale_by_two_kernel(StreamArgs a)
{
    __shared__ __attribute__((aligned(1024))) char ring[S * kStreamTileBytes];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int voff = tid * 16;  // this thread's 16 bytes of a tile (wave w: bytes [1024 w, +1024))
    const int64_t G = gridDim.x, b = blockIdx.x;
    const int64_t J = b < a.tiles ? (a.tiles - 1 - b) / G + 1 : 0;  // tiles of this block's stream
    const uint32_t m0 = (uint32_t)(uintptr_t)ring + (uint32_t)wave * 1024u;

    if constexpr (S == 1) {
        for (int64_t j = 0; j < J; ++j) {
            const int64_t t = b + j * G;
            dma16<0, true>(stream_desc(a.x, t, a.full_bytes), m0, voff);
            wait_vmcnt<0>();
            barrier();
            const f32x4_t v = *(const SPT_LDS f32x4_t*)((const SPT_LDS char*)ring + voff);
            stream_store(a.y, t, a.full_bytes, voff, v * 2.0f);
            wait_lgkmcnt0();
            barrier();  // every thread has read the stage before it is refilled
        }
    } else {
        const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
        // prologue: tiles 0 .. S-2 into stages 0 .. S-2, each copy paired with an empty store
#pragma unroll
        for (int i = 0; i < S - 1; ++i) {
            const int64_t t = b + i * G;
            dma16<0, true>(stream_desc(a.x, i < J ? t : a.tiles, a.full_bytes), m0 + i * kStreamTileBytes, voff);
            stream_store(a.y, a.tiles, a.full_bytes, voff, zero);  // extent 0: dropped
        }
        uint32_t rd = 0;                                      // stage of tile j
        uint32_t wr = (S - 1) * (uint32_t)kStreamTileBytes;   // stage of tile j + S - 1 (= tile j - 1)
        for (int64_t j = 0; j < J; ++j) {
            wait_vmcnt<2 * S - 3>();  // the copy of tile j has landed
            barrier();
            const int64_t tn = j + S - 1 < J ? b + (j + S - 1) * G : a.tiles;  // past the end: empty
            dma16<0, true>(stream_desc(a.x, tn, a.full_bytes), m0 + wr, voff);
            const f32x4_t v = *(const SPT_LDS f32x4_t*)((const SPT_LDS char*)ring + rd + voff);
            stream_store(a.y, b + j * G, a.full_bytes, voff, v * 2.0f);
            rd = rd + kStreamTileBytes == (uint32_t)(S * kStreamTileBytes) ? 0u : rd + kStreamTileBytes;
            wr = wr + kStreamTileBytes == (uint32_t)(S * kStreamTileBytes) ? 0u : wr + kStreamTileBytes;
        }
    }
    wait_vmcnt<0>();  // no copy may still be writing this block's LDS

    // the chunk that straddles n, by the thread whose tile position holds it
    if (a.n & 3) {
        const int64_t q = a.n >> 2;  // its chunk index
        const int64_t t = q / kStreamThreads;
        if (t % G == b && tid == (int)(q % kStreamThreads)) {
            const float* x = (const float*)a.x;
            float* y = (float*)a.y;
            for (int64_t i = 4 * q; i < a.n; ++i) y[i] = 2.0f * x[i];
        }
    }
}

template <int S>
static hipError_t launch_stream(const StreamArgs& a, unsigned blocks, hipStream_t stream)
{
    StreamArgs arg = a;
    void* args[] = {&arg};
    return hipLaunchKernel((const void*)&scale_by_two_kernel<S>, dim3(blocks), dim3(kStreamThreads), args, 0, stream);
}

hipError_t launch_scale_by_two(const void* x, void* y, int64_t n, int stages, unsigned blocks, hipStream_t stream)
{
    StreamArgs a;
    a.x = (const char*)x;
    a.y = (char*)y;
    a.n = n;
    a.full_bytes = (n >> 2) * 16;
    a.tiles = (n + 1023) / 1024;
    switch (stages) {
    case 1: return launch_stream<1>(a, blocks, stream);
    case 2: return launch_stream<2>(a, blocks, stream);
    case 3: return launch_stream<3>(a, blocks, stream);
    default: return launch_stream<4>(a, blocks, stream);
    }
}

}  // namespace spt
