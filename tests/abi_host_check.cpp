// Host-only check of the C ABI's argument validation, built with the host
// address and undefined-behaviour sanitizers (tests/test_abi_sanitize.py).
//
// Every call here either fails validation, has an empty batch, or (only when
// no GPU is visible) reaches a kernel launch that the HIP runtime refuses:
// the pointers are fake device addresses 1 GiB apart that are never
// dereferenced.  Prints one line per failed expectation and exits non-zero
// if there was any.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "linattn.h"

namespace {

int failures = 0;
int checks = 0;

void expect(int got, int want, const char* what, int line) {
    ++checks;
    if (got != want) {
        ++failures;
        printf("line %d: %s returned %d (%s), expected %d\n", line, what, got, la_status_str(got), want);
    }
}
#define CHECK(call, want) expect((call), (want), #call, __LINE__)

const uintptr_t kBase = 0x7F0000000000ull;
const uintptr_t kGiB = 1ull << 30;
void* P(int i) { return reinterpret_cast<void*>(kBase + i * kGiB); }
void* Pofs(int i, uintptr_t off) { return reinterpret_cast<void*>(kBase + i * kGiB + off); }
float* F(int i) { return static_cast<float*>(P(i)); }
const size_t kBad = static_cast<size_t>(-1);

int gdn(int dtype, int B, int H, int T, int dk, int dv, int form, int chunk, void* ws, size_t wsb,
        const float* S0 = nullptr, float* S_out = nullptr, void* o = P(4)) {
    return gdn_prefill(dtype, B, H, T, dk, dv, P(1), P(2), P(3), F(5), F(6), S0, o, S_out, form, chunk, ws, wsb,
                       nullptr);
}

}  // namespace

int main() {
    int devices = 0;
    const bool no_device = hipGetDeviceCount(&devices) != hipSuccess || devices == 0;

    // ---- status strings and version
    CHECK(la_abi_version(), LA_ABI_VERSION);
    for (int s = -3; s < 12; ++s) CHECK(la_status_str(s) != nullptr && strlen(la_status_str(s)) > 0, 1);

    // ---- workspace queries, including sizes at and past the limits
    CHECK(la_workspace_bytes(9, LA_F32, 1, 1, 8, 16, 16, 0, 16) == kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, 1, 1, 1 << 30, 128, 128, 0, 64) != kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, 1, 1, (1 << 30) + 1, 128, 128, 0, 64) == kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, 0x7fffffff, 1, 1, 128, 128, 0, 64) != kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, 0x7fffffff, 0x7fffffff, 1, 128, 128, 0, 64) == kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_LIN_ATTN_PREFILL, LA_BF16, 1, 1 << 10, 1 << 30, 128, 128, 0, 64) != kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_VARLEN, LA_BF16, 1 << 10, 64, 1 << 24, 128, 128, 0, 64) != kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_KDA_PREFILL, LA_BF16, 1 << 10, 1 << 10, 1 << 20, 128, 128, 0, 64) != kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, -1, 1, 1, 128, 128, 0, 64) == kBad, 1);
    // past the size bound (B*H*T <= 2^40): rejected, not overflowed
    CHECK(la_workspace_bytes(LA_FN_GDN_VARLEN, LA_BF16, 1 << 20, 64, 1 << 30, 128, 128, 0, 64) == kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_KDA_PREFILL, LA_BF16, 1 << 12, 1 << 10, 1 << 20, 128, 128, 0, 64) == kBad, 1);
    CHECK(la_workspace_bytes(LA_FN_GDN_PREFILL, LA_BF16, 1, 1, 1, 128, 128, 0, 48) == kBad, 1);
    for (int fn = 0; fn <= 5; ++fn)
        for (int dt = 0; dt <= 1; ++dt)
            for (int d = 16; d <= 128; d *= 2)
                for (int c = 16; c <= 128; c *= 2)
                    for (int form = 0; form <= 2; ++form) (void)la_workspace_bytes(fn, dt, 3, 5, 1000, d, d, form, c);

    // ---- lin_attn_prefill
    CHECK(lin_attn_prefill(7, 1, 2, 8, 16, 16, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr, nullptr, 0, 16,
                           nullptr, 0, nullptr), LA_ERR_DTYPE);
    CHECK(lin_attn_prefill(LA_F32, 1, 2, 8, 16, 16, nullptr, P(2), P(3), nullptr, nullptr, P(4), nullptr, nullptr, 0,
                           16, nullptr, 0, nullptr), LA_ERR_NULL);
    CHECK(lin_attn_prefill(LA_F32, 1, 2, 8, 16, 16, P(1), P(2), P(3), nullptr, nullptr, P(1), nullptr, nullptr, 0, 16,
                           nullptr, 0, nullptr), LA_ERR_ARG);
    CHECK(lin_attn_prefill(LA_F32, 1 << 20, 1 << 12, 8, 16, 16, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr,
                           nullptr, 0, 16, nullptr, 0, nullptr), LA_ERR_SHAPE);
    CHECK(lin_attn_prefill(LA_F32, 1, 2, 9000, 16, 16, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr, nullptr,
                           LA_FORM_PARALLEL, 0, nullptr, 0, nullptr), LA_ERR_SHAPE);
    CHECK(lin_attn_prefill(LA_BF16, 1, 2, 1000, 128, 128, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr, nullptr,
                           0, 64, nullptr, 0, nullptr), LA_ERR_WORKSPACE);
    CHECK(lin_attn_prefill(LA_F32, 0, 2, 8, 16, 16, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                           nullptr, 0, 16, nullptr, 0, nullptr), LA_OK);

    // ---- gdn_prefill and its allocation-free variant
    CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, LA_FORM_PARALLEL, 64, nullptr, 0), LA_ERR_ARG);
    CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, 0, 64, nullptr, 0), LA_ERR_WORKSPACE);
    CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, 0, 64, P(1), 1 << 30), LA_ERR_ARG);      // workspace on q
    CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, 0, 64, Pofs(9, 8), 1 << 30), LA_ERR_ALIGN);
    CHECK(gdn(LA_F32, 1, 1, 256, 128, 128, 0, 128, nullptr, 0), LA_ERR_UNSUPPORTED);
    CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, 0, 64, P(9), 1 << 30, F(7), static_cast<float*>(Pofs(7, 64))),
          LA_ERR_ARG);
    CHECK(gdn_prefill_noalloc(LA_BF16, 1, 2, 100, 128, 128, nullptr, P(2), P(3), F(5), F(6), nullptr, P(4), nullptr,
                              0, 64, nullptr), LA_ERR_NULL);
    CHECK(gdn_prefill_noalloc(LA_BF16, 1, 2, 100, 128, 128, P(1), P(2), P(3), F(5), F(6), nullptr, P(5), nullptr, 0,
                              64, nullptr), LA_ERR_ARG);
    CHECK(gdn_prefill_noalloc(LA_BF16, 0, 2, 100, 128, 128, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                              nullptr, nullptr, 0, 64, nullptr), LA_OK);

    // ---- split halves
    CHECK(gdn_prefill_prep(LA_BF16, 1, 2, 100, 128, 128, P(1), P(2), P(3), F(5), F(6), 33, P(9), 1 << 30, nullptr),
          LA_ERR_SHAPE);
    CHECK(gdn_prefill_scan(LA_BF16, 1, 2, 100, 128, 128, P(1), P(2), P(3), F(5), F(6), nullptr, P(9), nullptr, 64,
                           P(9), 1 << 30, nullptr), LA_ERR_ARG);

    // ---- gla, kda, varlen, pre-operations, decode
    CHECK(gla_prefill(LA_BF16, 1, 2, 1000, 128, 128, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr, 0, 64, P(9),
                      1 << 30, nullptr), LA_ERR_NULL);
    CHECK(kda_prefill(LA_BF16, 1, 2, 100, 128, 128, P(1), P(2), P(3), F(5), F(6), nullptr, P(4), nullptr, 0, 64,
                      nullptr, 0, nullptr), LA_ERR_WORKSPACE);
    CHECK(gdn_prefill_varlen(LA_BF16, 3, 2, 500, 128, 128, static_cast<const int*>(Pofs(10, 2)), P(1), P(2), P(3),
                             F(5), F(6), nullptr, P(4), nullptr, 0, 0, nullptr, 0, 64, P(9), 1 << 30, nullptr),
          LA_ERR_ALIGN);
    CHECK(gdn_prefill_varlen(LA_BF16, 3, 2, 500, 128, 128, static_cast<const int*>(P(10)), P(1), P(2), P(3), F(5),
                             F(6), nullptr, P(4), nullptr, 100, 4, F(11), 0, 64, P(9), 1 << 30, nullptr),
          LA_ERR_SHAPE);
    // packed batches of the other kinds: z arguments only for the normalised kind, z snapshots required with S ones
    CHECK(lin_attn_prefill_varlen(LA_KIND_KDA, LA_BF16, 3, 2, 500, 128, 128, static_cast<const int*>(P(10)), P(1),
                                  P(2), P(3), F(5), F(6), nullptr, F(12), P(4), nullptr, nullptr, 0, 0, nullptr,
                                  nullptr, LA_FORM_RECURRENT, 0, P(9), 1 << 30, nullptr), LA_ERR_ARG);
    CHECK(lin_attn_prefill_varlen(LA_KIND_NORMALIZED, LA_BF16, 3, 2, 500, 128, 128, static_cast<const int*>(P(10)),
                                  P(1), P(2), P(3), nullptr, nullptr, nullptr, nullptr, P(4), nullptr, nullptr, 128, 4,
                                  F(11), nullptr, LA_FORM_RECURRENT, 0, P(9), 1 << 30, nullptr), LA_ERR_NULL);
    CHECK(lin_attn_prefill_varlen(LA_KIND_GATED, LA_F32, 3, 2, 500, 128, 128, static_cast<const int*>(P(10)), P(1),
                                  P(2), P(3), F(5), nullptr, nullptr, nullptr, P(4), nullptr, nullptr, 0, 0, nullptr,
                                  nullptr, LA_FORM_CHUNKED, 64, P(9), 1 << 30, nullptr), LA_ERR_UNSUPPORTED);
    CHECK(lin_attn_prefill_varlen(LA_KIND_GATED, LA_BF16, 3, 2, 500, 128, 128, static_cast<const int*>(P(10)), P(1),
                                  P(2), P(3), F(5), nullptr, nullptr, nullptr, P(4), nullptr, nullptr, 0, 0, nullptr,
                                  nullptr, LA_FORM_RECURRENT, 0, P(9), 15, nullptr), LA_ERR_WORKSPACE);
    CHECK(gdn_preprocess(LA_BF16, 2, 100, 4, 128, 128, P(1), F(2), F(3), F(4), nullptr, nullptr, P(1), P(6), P(7),
                         F(8), F(9), nullptr), LA_ERR_ARG);
    CHECK(gdn_preprocess_varlen(LA_BF16, 3, 100, 4, 128, 128, nullptr, P(1), F(2), F(3), F(4), nullptr, nullptr, P(5),
                                P(6), P(7), F(8), F(9), nullptr), LA_ERR_NULL);
    CHECK(lin_attn_decode_step(LA_KIND_GATED_DELTA, LA_BF16, 4, 2, 128, 128, P(1), P(2), P(3), F(5), F(6), F(7),
                               nullptr, P(7), nullptr), LA_ERR_ARG);
    CHECK(lin_attn_decode_step(9, LA_BF16, 4, 2, 128, 128, P(1), P(2), P(3), F(5), F(6), F(7), nullptr, P(4),
                               nullptr), LA_ERR_ARG);

    // ---- a grid of 2^32 or more work-items (sizes within every other bound):
    //      refused before anything is launched, with or without a device
    CHECK(lin_attn_decode_step(LA_KIND_GATED_DELTA, LA_BF16, 1 << 19, 32, 16, 16, P(1), P(2), P(3), F(5), F(6),
                               F(7), nullptr, P(4), nullptr), LA_ERR_SHAPE);
    CHECK(gdn(LA_F32, 1 << 19, 32, 1, 16, 16, LA_FORM_CHUNKED, 16, nullptr, 0), LA_ERR_SHAPE);

    // ---- valid calls with no device: the launch fails and is reported
    if (no_device) {
        CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, 0, 64, P(9), 1 << 30), LA_ERR_HIP);
        CHECK(gdn(LA_BF16, 1, 2, 100, 128, 128, LA_FORM_RECURRENT, 0, nullptr, 0), LA_ERR_HIP);
        CHECK(gdn(LA_F32, 1, 2, 100, 64, 64, 0, 32, nullptr, 0), LA_ERR_HIP);
        CHECK(gdn_prefill_noalloc(LA_BF16, 2, 16, 8192, 128, 128, P(1), P(2), P(3), F(5), F(6), nullptr, P(4),
                                  nullptr, 0, 64, nullptr), LA_ERR_HIP);
        CHECK(lin_attn_decode_step(LA_KIND_GATED_DELTA, LA_BF16, 4, 2, 128, 128, P(1), P(2), P(3), F(5), F(6), F(7),
                                   nullptr, P(4), nullptr), LA_ERR_HIP);
        CHECK(lin_attn_prefill(LA_BF16, 1, 2, 1000, 128, 128, P(1), P(2), P(3), nullptr, nullptr, P(4), nullptr,
                               nullptr, 0, 64, P(9), 1 << 30, nullptr), LA_ERR_HIP);
        CHECK(lin_attn_prefill_varlen(LA_KIND_NORMALIZED, LA_BF16, 3, 2, 500, 128, 128,
                                      static_cast<const int*>(P(10)), P(1), P(2), P(3), nullptr, nullptr, nullptr,
                                      nullptr, P(4), nullptr, nullptr, 128, 4, F(11), F(12), LA_FORM_RECURRENT, 0,
                                      P(9), 1 << 30, nullptr), LA_ERR_HIP);
    }
    printf("%d checks, %d failed%s\n", checks, failures, no_device ? " (no device: launches checked)" : "");
    return failures == 0 ? 0 : 1;
}
