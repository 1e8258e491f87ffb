// Runs the library's host-side validation (csrc/gdn_validate.cpp: size
// checks, workspace layout, device-content precondition checks) under
// AddressSanitizer and UBSan, with no GPU and no HIP: every array handed to
// a check is a heap block of exactly its size, so a read past it is
// reported, and extreme sizes exercise the overflow paths of the size
// arithmetic.  Prints "OK" and exits 0 when every expectation holds.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <vector>

#include "gdn.h"

#define EXPECT(cond, ...)                                                         \
    do {                                                                          \
        if (!(cond)) {                                                            \
            fprintf(stderr, "line %d: ", __LINE__);                               \
            fprintf(stderr, __VA_ARGS__);                                         \
            fprintf(stderr, " [%s]\n", gdn_get_last_error());                     \
            return 1;                                                             \
        }                                                                         \
    } while (0)

static gdn_dims dims(int n, long long T, int hqk, int hv, int dk = 128, int dv = 128) {
    gdn_dims d;
    d.n_seqs = n; d.total_tokens = T; d.n_heads_qk = hqk; d.n_heads_v = hv; d.d_k = dk; d.d_v = dv;
    return d;
}

int main() {
    size_t bytes = 0, seg = 0;
    int64_t slots = 0;
    // sizes: valid, and every rejection path
    gdn_dims d = dims(1, 4000, 16, 32);
    EXPECT(gdn_chunk_fwd_workspace_size(&d, &bytes) == GDN_SUCCESS && bytes > 0, "workspace size");
    EXPECT(gdn_chunk_state_slots(&d, &slots) == GDN_SUCCESS && slots == 1 + 4000 / 64 + 1, "slots");
    EXPECT(gdn_chunk_fwd_segmented_workspace_size(&d, 8, &seg) == GDN_SUCCESS && seg > bytes, "segmented size");
    const gdn_dims bad[] = {dims(-1, 0, 1, 1), dims(1, -5, 1, 1), dims(1, 1LL << 40, 1, 1), dims(0, 7, 1, 1),
                            dims(1, 8, 0, 1), dims(1, 8, 3, 4), dims(1, 8, 1, 70000), dims(1 << 20, 8, 1, 64),
                            dims(1, 8, 1, 1, 0, 128), dims(2000000, 2147483647LL, 1, 1)};
    for (const gdn_dims& b : bad) {
        bytes = 0;
        EXPECT(gdn_chunk_fwd_workspace_size(&b, &bytes) == GDN_ERR_INVALID_VALUE && bytes == 0,
               "bad dims accepted (N=%d T=%lld)", b.n_seqs, (long long)b.total_tokens);
    }
    gdn_dims d64 = dims(1, 8, 1, 1, 64, 64);
    EXPECT(gdn_chunk_fwd_workspace_size(&d64, &bytes) == GDN_ERR_NOT_SUPPORTED, "d = 64");
    EXPECT(gdn_chunk_fwd_workspace_size(nullptr, &bytes) == GDN_ERR_INVALID_VALUE, "NULL dims");
    EXPECT(gdn_chunk_fwd_workspace_size(&d, nullptr) == GDN_ERR_INVALID_VALUE, "NULL out");
    EXPECT(gdn_chunk_fwd_segmented_workspace_size(&d, 0, &seg) == GDN_ERR_INVALID_VALUE, "segment 0");
    // the largest accepted batch: sizes stay exact in 64-bit arithmetic
    gdn_dims big = dims(1, ((1LL << 24) - 2) * 64, 1, 1);   // exactly 2^24 chunk slots
    EXPECT(gdn_chunk_fwd_workspace_size(&big, &bytes) == GDN_SUCCESS && bytes > (size_t)1 << 36, "big");
    for (int s = 0; s <= 5; ++s) EXPECT(strlen(gdn_status_string((gdn_status)s)) > 0, "status text");
    EXPECT(strcmp(gdn_status_string((gdn_status)42), "unknown status") == 0, "unknown status");

    // device-content checks on exact-size host copies
    const int N = 3, HQK = 2, HV = 4, D = 128;
    const int32_t cu_ok[N + 1] = {0, 70, 70, 75};
    const long long T = 75;
    std::vector<uint16_t> q(T * HQK * D, 0x3c00), k(T * HQK * D, 0xbc00), v(T * HV * D, 0x3f80);
    std::vector<float> g(T * HV, -0.5f), b(T * HV, 0.5f), s0((size_t)N * HV * D * D, 0.01f);
    std::vector<int32_t> cu(cu_ok, cu_ok + N + 1);
    d = dims(N, T, HQK, HV);
    EXPECT(gdn_check_chunk_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), cu.data(), s0.data(), &d)
               == GDN_SUCCESS, "valid chunk inputs");
    EXPECT(gdn_check_step_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), s0.data(), N, &d)
               == GDN_SUCCESS, "valid step inputs");
    cu[2] = 80;
    EXPECT(gdn_check_chunk_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), cu.data(), nullptr, &d)
               == GDN_ERR_INVALID_VALUE, "decreasing cu_seqlens");
    cu[2] = 70;
    g.back() = 0.25f;
    EXPECT(gdn_check_chunk_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), cu.data(), nullptr, &d)
               == GDN_ERR_INVALID_VALUE, "positive g (last element)");
    g.back() = -0.5f;
    b.back() = NAN;
    EXPECT(gdn_check_step_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), nullptr, 0, &d)
               == GDN_ERR_INVALID_VALUE, "NaN beta (last element)");
    b.back() = 0.5f;
    v.back() = 0x4780;   // 65536 in bf16
    EXPECT(gdn_check_chunk_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), cu.data(), nullptr, &d)
               == GDN_ERR_INVALID_VALUE, "v past fp16 range (last element)");
    v.back() = 0x3f80;
    s0.back() = INFINITY;
    EXPECT(gdn_check_chunk_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), cu.data(), s0.data(), &d)
               == GDN_ERR_INVALID_VALUE, "infinite state (last element)");
    EXPECT(gdn_check_step_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), s0.data(), N, &d)
               == GDN_ERR_INVALID_VALUE, "infinite state, step");
    EXPECT(gdn_check_step_inputs_host(q.data(), k.data(), v.data(), g.data(), b.data(), s0.data(), -1, &d)
               == GDN_ERR_INVALID_VALUE, "negative state count");
    gdn_dims empty = dims(0, 0, 1, 1);
    EXPECT(gdn_check_chunk_inputs_host(nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, &empty)
               == GDN_SUCCESS, "no sequences");
    puts("OK");
    return 0;
}
