// Calls every compute entry point of the C ABI (include/gdn.h) with valid and invalid arguments,
// with api.cpp's validation built under AddressSanitizer and UndefinedBehaviorSanitizer and the
// kernel launchers replaced by host-only stand-ins (tests/sanitize/launch_stubs.cpp).  Pointers
// are fake, aligned, non-overlapping device addresses: validation only compares their ranges and
// never dereferences them.  A valid call ends as GDN_ERR_NO_DEVICE on a host without a GPU (or
// GDN_OK with one); every invalid one must return its documented status.  Built and run by
// tests/test_sanitizers.py; exit status 0 means every expectation held.
#include <climits>
#include <cstdint>
#include <cstdio>
#include <initializer_list>

#include "gdn.h"

static int fails = 0;
static void expect(const char* what, int line, gdn_status_t got, gdn_status_t want)
{
    if (got != want) {
        std::fprintf(stderr, "line %d %s: status %d (%s), expected %d\n", line, what, (int)got,
                     gdn_status_string(got), (int)want);
        ++fails;
    }
}
static void expect_valid(const char* what, int line, gdn_status_t got)
{
    if (got != GDN_OK && got != GDN_ERR_NO_DEVICE) {
        std::fprintf(stderr, "line %d %s: status %d (%s) for a valid call\n", line, what, (int)got,
                     gdn_status_string(got));
        ++fails;
    }
}
#define EXPECT(call, want) expect(#call, __LINE__, (call), (want))
#define VALID(call) expect_valid(#call, __LINE__, (call))

// fake device addresses 2^36 apart, 256-byte aligned
static void* P(int n) { return reinterpret_cast<void*>((uintptr_t)0x7f0000000000ull + ((uintptr_t)n << 36)); }
static float* F(int n) { return static_cast<float*>(P(n)); }
static void* MIS(int n) { return static_cast<char*>(P(n)) + 8; }

int main()
{
    for (int s = 0; s <= 9; ++s) (void)gdn_status_string((gdn_status_t)s);
    (void)gdn_status_string((gdn_status_t)1234);

    // sizes and queries over a grid, including extreme values (no arithmetic may overflow)
    const int vals[] = {-1, 0, 1, 2, 3, 16, 33, 64, 128, 4096, 65536, 1 << 20, INT_MAX};
    for (int B : vals)
        for (int T : vals)
            for (int d : {32, 64, 128, 48})
                for (int ch : {16, 32, 64, 7})
                    for (gdn_dtype_t dt : {GDN_F32, GDN_BF16}) {
                        (void)gdn_chunk_fwd_workspace_bytes(B, T, 16, 48, d, d, ch, dt);
                        (void)gdn_chunk_fwd_gated_workspace_bytes(B, T, 16, 32, d, d, ch, dt);
                        (void)gdn_chunk_fwd_kernel_name(B, T, 2, 6, d, 128, ch, dt);
                        (void)gdn_chunk_bwd_workspace_bytes(B, T, 4, 8, d, d, dt);
                        (void)gdn_kda_chunk_fwd_workspace_bytes(B, T, 4, 8, d, d, ch, dt);
                        (void)gdn_chunk_fwd_varlen_workspace_bytes(B, T, 4, 8, d, d, ch, dt);
                        (void)gdn_chunk_fwd_scan_workspace_bytes(B, T, 4, 8, d, d, ch, dt, 3);
                        (void)gdn_chunk_fwd_scan_segments(B, T, 4, 8, d, d, ch, dt, 5);
                        (void)gdn_chunk_transport_workspace_bytes(B, T, 4, 8, d, d, ch, dt);
                    }

    const gdn_dtype_t bf = GDN_BF16;
    const int B = 2, T = 300, Hqk = 2, Hv = 4, d = 128;
    const size_t ws = gdn_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, d, d, 64, bf);
    // prefill
    VALID(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr));
    VALID(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), F(6), F(6), P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr));
    EXPECT(gdn_chunk_fwd(nullptr, P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_chunk_fwd(MIS(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_ALIGN);
    EXPECT(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(2), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), B, T, 3, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), B, T, Hqk, Hv, 48, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_UNSUPPORTED);
    if (ws) EXPECT(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws - 1, nullptr), GDN_ERR_WORKSPACE);
    EXPECT(gdn_chunk_fwd(P(1), P(2), P(3), F(4), F(5), nullptr, nullptr, P(8), -1, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), ws, nullptr), GDN_ERR_SHAPE);
    VALID(gdn_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, F(6), F(7), nullptr, B, 0, Hqk, Hv, d, d, 64, bf, 1.f, nullptr, 0, nullptr));
    EXPECT(gdn_chunk_fwd(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, T, Hqk, Hv, d, d, 64, bf, 1.f, nullptr, 0, nullptr), GDN_OK);
    // gated prefill
    const size_t gws = gdn_chunk_fwd_gated_workspace_bytes(B, T, Hqk, Hv, d, d, 64, bf);
    VALID(gdn_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), nullptr, F(7), P(10), F(11), 1, 1e-6f, P(10), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), gws, nullptr));
    EXPECT(gdn_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), nullptr, F(7), P(10), F(11), 2, 1e-6f, P(12), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), gws, nullptr), GDN_ERR_SHAPE);
    EXPECT(gdn_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), nullptr, F(7), P(10), F(11), 0, -1.f, P(12), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), gws, nullptr), GDN_ERR_UNSUPPORTED);
    EXPECT(gdn_chunk_fwd_gated(P(1), P(2), P(3), F(4), F(5), nullptr, F(7), P(10), F(11), 0, 1e-6f, P(3), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), gws, nullptr), GDN_ERR_ALIAS);
    // decode
    VALID(gdn_recurrent_step(P(1), P(2), P(3), F(4), F(5), F(6), P(8), 256, 16, 32, d, d, bf, 1.f, nullptr));
    EXPECT(gdn_recurrent_step(P(1), P(2), P(3), F(4), F(5), nullptr, P(8), 256, 16, 32, d, d, bf, 1.f, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_recurrent_step(P(1), P(2), P(3), F(4), F(5), F(6), P(6), 256, 16, 32, d, d, bf, 1.f, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_recurrent_step(P(1), P(2), P(3), F(4), F(5), F(6), MIS(8), 256, 16, 32, d, d, bf, 1.f, nullptr), GDN_ERR_ALIGN);
    EXPECT(gdn_recurrent_step(P(1), P(2), P(3), F(4), F(5), F(6), P(8), 256, 16, 33, d, d, bf, 1.f, nullptr), GDN_ERR_SHAPE);
    // backward
    const size_t bws = gdn_chunk_bwd_workspace_bytes(B, T, Hqk, Hv, d, d, bf);
    VALID(gdn_chunk_bwd(P(1), P(2), P(3), F(4), F(5), F(6), P(7), F(8), P(10), P(11), P(12), F(13), F(14), F(15), B, T, Hqk, Hv, d, d, bf, 1.f, P(9), bws, nullptr));
    EXPECT(gdn_chunk_bwd(P(1), P(2), P(3), F(4), F(5), F(6), P(7), F(8), P(1), P(11), P(12), F(13), F(14), F(15), B, T, Hqk, Hv, d, d, bf, 1.f, P(9), bws, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_chunk_bwd(P(1), P(2), P(3), F(4), F(5), F(6), P(7), F(8), P(10), P(11), P(12), F(13), F(14), F(15), B, T, Hqk, Hv, d, d, bf, 1.f, P(9), bws - 1, nullptr), GDN_ERR_WORKSPACE);
    // KDA
    const size_t kws = gdn_kda_chunk_fwd_workspace_bytes(B, T, Hqk, Hv, d, d, 64, bf);
    VALID(gdn_kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), kws, nullptr));
    EXPECT(gdn_kda_chunk_fwd(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(4), B, T, Hqk, Hv, d, d, 64, bf, 1.f, P(9), kws, nullptr), GDN_ERR_ALIAS);
    // packed sequences
    const size_t vws = gdn_chunk_fwd_varlen_workspace_bytes(3, 200, Hqk, Hv, d, d, 64, bf);
    VALID(gdn_chunk_fwd_varlen(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(8), (const int*)P(12), 3, 200, 450, Hqk, Hv, d, d, 64, bf, 1.f, P(9), vws, nullptr));
    EXPECT(gdn_chunk_fwd_varlen(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(8), nullptr, 3, 200, 450, Hqk, Hv, d, d, 64, bf, 1.f, P(9), vws, nullptr), GDN_ERR_NULL);
    EXPECT(gdn_chunk_fwd_varlen(P(1), P(2), P(3), F(4), F(5), F(6), F(7), P(8), (const int*)((char*)P(12) + 2), 3, 200, 450, Hqk, Hv, d, d, 64, bf, 1.f, P(9), vws, nullptr), GDN_ERR_ALIGN);
    // affine chunk scan and transport
    const size_t sws = gdn_chunk_fwd_scan_workspace_bytes(B, T, Hqk, Hv, d, d, 64, bf, 3);
    VALID(gdn_chunk_fwd_scan(P(1), P(2), P(3), F(4), F(5), F(6), F(6), P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, 3, P(9), sws, nullptr));
    EXPECT(gdn_chunk_fwd_scan(P(1), P(2), P(3), F(4), F(5), F(6), F(6), P(8), B, T, Hqk, Hv, d, d, 64, bf, 1.f, 0, P(9), sws, nullptr), GDN_ERR_SHAPE);
    const size_t tws = gdn_chunk_transport_workspace_bytes(B, T, Hqk, Hv, d, d, 64, bf);
    VALID(gdn_chunk_transport(nullptr, P(2), P(3), F(4), F(5), F(6), F(7), B, T, Hqk, Hv, d, d, 64, bf, P(9), tws, nullptr));
    EXPECT(gdn_chunk_transport(nullptr, P(2), P(3), F(4), F(5), F(6), F(6), B, T, Hqk, Hv, d, d, 64, bf, P(9), tws, nullptr), GDN_ERR_ALIAS);
    // layer steps
    VALID(gdn_qkv_prologue(P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), P(10), P(11), P(12), B, T, Hqk, Hv, d, d, 4, bf, 1e-6f, nullptr));
    EXPECT(gdn_qkv_prologue(P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(7), P(10), P(11), P(12), B, T, Hqk, Hv, d, d, 4, bf, 1e-6f, nullptr), GDN_ERR_ALIAS);
    EXPECT(gdn_qkv_prologue(P(1), P(2), P(3), F(4), F(5), F(6), F(7), F(8), P(10), P(11), P(12), B, T, Hqk, Hv, d, d, 5, bf, 1e-6f, nullptr), GDN_ERR_UNSUPPORTED);
    VALID(gdn_gated_rmsnorm(P(1), P(2), F(3), 0, P(1), B, T, Hv, d, bf, 1e-6f, nullptr));
    EXPECT(gdn_gated_rmsnorm(P(1), P(2), F(3), 0, P(3), B, T, Hv, d, bf, 1e-6f, nullptr), GDN_ERR_ALIAS);
    if (fails) {
        std::fprintf(stderr, "%d expectation(s) failed\n", fails);
        return 1;
    }
    std::printf("abi driver: ok\n");
    return 0;
}
