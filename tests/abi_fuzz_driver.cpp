// Fuzzes the argument checks of the C ABI (include/spt.h) under AddressSanitizer and
// UndefinedBehaviorSanitizer, on the host (built by tests/test_abi_fuzz.py).
//
// spt_api.cpp is linked with empty kernel tables and launchers that report an
// error, so no call can reach a GPU: a call that passes every check either has
// nothing to compute (M = 0 or N = 0, OK with no launch) or finds no kernel
// (SPT_ERR_UNSUPPORTED), or, for the streaming entry point, reports the stub
// launcher's error (SPT_ERR_LAUNCH).  Arguments come from a fixed generator over edge
// values: negative, zero, one, tile and pitch boundaries, 2^31 - 1, 2^31, 2^40,
// INT64_MAX; null, small, misaligned, high and non-canonical pointers; every
// enum value and one past each end.  Pointers are never dereferenced by the
// checks, so fake addresses are safe.  Checked per call: the status is one of
// the five codes, OK only where nothing is launched, spt_last_error() is a
// terminated string, empty exactly after a call that returned OK, and no sanitizer fires (signed overflow in the size
// arithmetic, out-of-bounds table reads, ...).
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <map>
#include <string>

#include <hip/hip_runtime.h>

#include "../include/spt.h"
#include "../software_pipelined_tiling_amd/csrc/spt_registry.h"

namespace spt {
#define SPT_EMPTY_TABLE(NAME) \
    KernelTable kernels_##NAME() { return KernelTable{nullptr, 0}; }
SPT_EMPTY_TABLE(f16_row)
SPT_EMPTY_TABLE(f16_col)
SPT_EMPTY_TABLE(bf16_row)
SPT_EMPTY_TABLE(bf16_col)
SPT_EMPTY_TABLE(i8_row)
SPT_EMPTY_TABLE(i8_col)
SPT_EMPTY_TABLE(f32_row)
SPT_EMPTY_TABLE(f32_col)
hipError_t launch_scale_by_two(const void*, void*, int64_t, int, unsigned, hipStream_t) { return hipErrorInvalidValue; }
hipError_t launch_attention(int, int, int, int, const void*, const void*, const void*, void*, int, int, int, float,
                            hipStream_t)
{
    return hipErrorInvalidValue;
}
}  // namespace spt

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next()  // splitmix64
{
    uint64_t z = (state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
template <class T, size_t N>
static T pick(const T (&v)[N])
{
    return v[next() % N];
}

static const int64_t kSizes[] = {-1, 0, 1, 2, 3, 15, 16, 17, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, 257, 1000,
                                 4095, 4096, 4100, 131071, 131072, 1 << 20, INT32_MAX, (int64_t)INT32_MAX + 1,
                                 (int64_t)1 << 40, INT64_MAX, INT64_MIN};
static const uintptr_t kPtrs[] = {0, 0x10, 0x1000, 0x10000, 0x10008, 0x7f0000000000ull, 0x7ffffffff000ull,
                                  0x800000000000ull, 0xfffffffffffff000ull, 0x7f0000100000ull, 0x7f0000100010ull};
static const int kEnums[] = {-1, 0, 1, 2, 3, 4, 5, 6, 1 << 30, -(1 << 30)};

static int failures;
static void expect(bool ok, const char* what, int rc)
{
    if (!ok) {
        fprintf(stderr, "%s (rc %d): %s\n", what, rc, spt_last_error());
        ++failures;
    }
}

static bool known(int rc)
{
    return rc == SPT_OK || rc == SPT_ERR_INVALID || rc == SPT_ERR_UNSUPPORTED || rc == SPT_ERR_MISALIGNED ||
           rc == SPT_ERR_LAUNCH;
}

// Distinct messages (digits dropped) with counts: which checks the generator reaches.
static std::map<std::string, long> reached;
static void message_ok(int rc)
{
    const char* m = spt_last_error();
    expect(m != nullptr && strnlen(m, 512) < 256, "last-error message not a short terminated string", rc);
    expect((rc == SPT_OK) == (m != nullptr && m[0] == 0), "message empty exactly after a call that succeeded", rc);
    std::string key;
    for (const char* c = m; *c && key.size() < 48; ++c)
        if (*c < '0' || *c > '9') key += *c;
    ++reached[key];
}

int main()
{
    const int rounds = 200000;
    for (int it = 0; it < rounds; ++it) {
        const int64_t M = pick(kSizes), N = pick(kSizes), K = pick(kSizes);
        const int64_t lda = pick(kSizes), ldb = pick(kSizes), ldc = pick(kSizes);
        const int dtype = pick(kEnums), layout = pick(kEnums), variant = pick(kEnums), stages = pick(kEnums),
                  tile = pick(kEnums);
        const void* A = (const void*)pick(kPtrs);
        const void* B = (const void*)pick(kPtrs);
        void* C = (void*)pick(kPtrs);

        spt_plan_info pi;
        int rc = spt_plan(dtype, M, N, K, layout, variant, stages, tile, &pi);
        expect(rc == SPT_OK || rc == SPT_ERR_INVALID || rc == SPT_ERR_UNSUPPORTED, "spt_plan status", rc);
        if (rc == SPT_OK)
            expect(pi.lds_bytes > 0 && pi.lds_bytes <= 163840 && pi.grid >= 0 && pi.k_tail >= 0 && pi.BK > 0,
                   "plan fields out of range", rc);
        message_ok(rc);

        rc = spt_gemm_ex(M, N, K, A, lda, B, ldb, C, ldc, dtype, nullptr, layout, variant, stages, tile);
        expect(known(rc) && rc != SPT_ERR_LAUNCH, "spt_gemm_ex status", rc);
        expect(rc != SPT_OK || M == 0 || N == 0, "OK with work to launch and no kernel", rc);
        message_ok(rc);

        rc = spt_gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, nullptr);
        expect(known(rc) && rc != SPT_ERR_LAUNCH, "spt_gemm status", rc);
        expect(rc != SPT_OK || M == 0 || N == 0, "OK with work to launch and no kernel", rc);
        message_ok(rc);

        rc = spt_scale_by_two(M, A, C, stages, variant, nullptr);
        expect(known(rc), "spt_scale_by_two status", rc);
        expect(rc != SPT_OK || M == 0, "OK with work to launch", rc);
        message_ok(rc);

        rc = spt_attention(M, N, K, (int64_t)((unsigned)stages % 5) * 32, A, B, (const void*)((uintptr_t)B + 4096), C,
                           (float)(int)(next() % 3) - 0.5f, dtype, nullptr, variant, stages);
        expect(known(rc), "spt_attention status", rc);
        expect(rc != SPT_OK || M == 0 || N == 0, "OK with work to launch", rc);
        message_ok(rc);

        expect(spt_status_string(rc) != nullptr && spt_status_string(layout) != nullptr, "status string", rc);
    }
    // Structured rounds: valid enums, pitches that satisfy or just miss the limits,
    // aligned pointers with occasional misalignment, nulls and overlaps, so the later
    // checks (alignment, address range, panel size, tile count, overlap) are reached.
    static const int64_t kDims[] = {1, 2, 15, 16, 17, 127, 128, 129, 255, 256, 257, 4096, 4100, 65536, 131071,
                                    1 << 20, INT32_MAX};
    static const int64_t kPads[] = {0, 0, 0, 1, 8, 16, 64, -1};
    for (int it = 0; it < rounds; ++it) {
        const int dtype = (int)(next() % 4), layout = (int)(next() % 2), variant = (int)(next() % 5);
        const int stages = (int)(next() % 5), tile = (int)(next() % 7);
        const int64_t M = pick(kDims), N = pick(kDims), K = next() % 8 == 0 ? 0 : pick(kDims);
        const int64_t lda = K + pick(kPads), ldb = (layout ? K : N) + pick(kPads), ldc = N + pick(kPads);
        uintptr_t a = 0x7f0000000000ull, b = 0x7f4000000000ull, c = 0x7f8000000000ull;
        switch (next() % 8) {
        case 0: c = a + (next() % 4) * 0x1000; break;  // C inside or at the start of A
        case 1: c = b - 0x1000; break;                 // C just below B
        case 2: a += 4; break;                         // misaligned A
        case 3: c = 0; break;                          // null C
        case 4: b = 0; break;                          // null B
        case 5: a = 0x800000000000ull; break;          // beyond 47 bits
        default: break;
        }
        const int rc = spt_gemm_ex(M, N, K, (const void*)a, lda, (const void*)b, ldb, (void*)c, ldc, dtype, nullptr,
                                   layout, variant, stages, tile);
        expect(known(rc) && rc != SPT_ERR_LAUNCH, "structured spt_gemm_ex status", rc);
        expect(rc != SPT_OK || M == 0 || N == 0, "OK with work to launch and no kernel", rc);
        message_ok(rc);
    }
    if (failures) {
        fprintf(stderr, "%d failures\n", failures);
        return 1;
    }
    for (const auto& kv : reached) printf("%9ld  %s\n", kv.second, kv.first.c_str());
    printf("abi checks ok under the sanitizers: %d rounds\n", 2 * rounds);
    return 0;
}
