// Host side of libspecverify without a GPU: the argument checks and the
// launch plan of sv_api.cpp, linked against launchers that only record what
// they were asked to run.  Built with AddressSanitizer and UBSan by
// tests/test_host_sanitizers.py; device pointers here are never dereferenced
// (the host code only checks and offsets them), so fake aligned addresses
// stand in for device memory.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <initializer_list>

#include "specverify.h"
#include "sv_internal.h"

namespace {
struct Launch {
    int calls = 0;
    sv::Params p{};
    int dtype = -1;
    bool vec = false, seq = false;
} last;
int fail_with = 0;  // nonzero: the launchers report this HIP error
}  // namespace

namespace sv {
int launch_stochastic(const Params& p, int dtype, bool vec, bool seq, void*) {
    ++last.calls;
    last.p = p;
    last.dtype = dtype;
    last.vec = vec;
    last.seq = seq;
    return fail_with;
}
int launch_greedy(const Params& p, int dtype, bool vec, bool seq, void* s) {
    return launch_stochastic(p, dtype, vec, seq, s);
}
int launch_tree(const Params& p, int dtype, bool vec, void* s) {
    return launch_stochastic(p, dtype, vec, false, s);
}
int launch_commit(const int32_t*, const int32_t*, int, int, int32_t*, int32_t*, long long, int,
                  int32_t*, long long, void*) {
    ++last.calls;
    return fail_with;
}
}  // namespace sv

static int fails = 0;
#define CHECK(c)                                                   \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++fails;                                               \
        }                                                          \
    } while (0)

// Fake device addresses: 256-byte aligned, far apart, never dereferenced.
static void* fake(uintptr_t i) { return reinterpret_cast<void*>((uintptr_t)0x100000000ull * (i + 1)); }

static int stoch(int B, int k, int V, void* ws, size_t wsb, bool dbg, const int32_t* cu = nullptr,
                 int total = 0) {
    last = Launch{};
    if (cu)
        return sv_verify_stochastic_ragged(fake(0), fake(1), (const int32_t*)fake(2), cu, total,
                                           (const float*)fake(3), (const float*)fake(4), B, k, V,
                                           V, SV_DTYPE_BF16, 1.0f, (int32_t*)fake(5),
                                           (int32_t*)fake(6), dbg ? (float*)fake(7) : nullptr, ws,
                                           wsb, nullptr);
    return sv_verify_stochastic(fake(0), fake(1), (const int32_t*)fake(2), (const float*)fake(3),
                                (const float*)fake(4), B, k, V, V, SV_DTYPE_BF16, 1.0f,
                                (int32_t*)fake(5), (int32_t*)fake(6),
                                dbg ? (float*)fake(7) : nullptr, ws, wsb, nullptr);
}

// The capped plan's workspace regions lie inside [ws, ws + bytes) in order.
static void check_capped_layout(void* ws, size_t bytes, int B, int k) {
    const sv::Params& p = last.p;
    const char* w = static_cast<const char*>(ws);
    const int rows = 2 * k + 1;
    CHECK((const char*)p.active == w);
    CHECK((const char*)p.part == w + sv::exit_flag_bytes(B));
    CHECK((const char*)p.tilesum == (const char*)p.part + sv::part_bytes(B, rows, p.S));
    CHECK((const char*)p.cnt == (const char*)p.tilesum + sv::tilesum_bytes(B));
    CHECK((const char*)p.xl == (const char*)p.cnt + sv::cnt_bytes(B));
    CHECK((const char*)p.xl + sv::xl_bytes(B, rows) <= w + bytes);
    CHECK(p.rows_per_seq == rows);
    CHECK(p.S >= 1 && p.S <= sv::kExitMaxSlices);
    CHECK(p.SD >= 1 && p.SD <= sv::kMaxTiles + 1);
}

int main() {
    const int V = 128256;
    // capped early exit: B >= 192, k >= 6, no diagnostics, enough workspace
    for (int B : {192, 256, 512, 1024}) {
        for (int k : {6, 7, 8, 64}) {
            const size_t wsb = sv_workspace_bytes(B, 1, k, V);
            CHECK(stoch(B, k, V, fake(8), wsb, false) == SV_OK);
            CHECK(last.calls == 1 && last.seq && last.p.active != nullptr);
            CHECK(last.p.exit_pairs == sv::plan_exit_pairs(k) && last.p.exit_pairs < k);
            check_capped_layout(fake(8), wsb, B, k);
            CHECK(last.p.S == sv::kExitMaxSlices);  // the bound leaves room for every slice
            // diagnostics: the full read, no capping
            CHECK(stoch(B, k, V, fake(8), wsb, true) == SV_OK);
            CHECK(last.seq && last.p.active == nullptr);
            // no workspace, or a misaligned one: the plain early exit
            CHECK(stoch(B, k, V, nullptr, 0, false) == SV_OK);
            CHECK(last.seq && last.p.active == nullptr);
            CHECK(stoch(B, k, V, (char*)fake(8) + 64, wsb, false) == SV_OK);
            CHECK(last.seq && last.p.active == nullptr);
        }
    }
    // a workspace smaller than the bound: fewer slices, still inside it
    {
        const int B = 256, k = 8;
        const size_t full = sv_workspace_bytes(B, 1, k, V);
        for (size_t wsb : {full / 2, full / 3, full / 4}) {
            CHECK(stoch(B, k, V, fake(8), wsb, false) == SV_OK);
            if (last.p.active) {
                check_capped_layout(fake(8), wsb, B, k);
                CHECK(last.p.S < sv::kExitMaxSlices);
            }
        }
        CHECK(stoch(B, k, V, fake(8), 4096, false) == SV_OK);  // far too small: plain
        CHECK(last.p.active == nullptr);
    }
    // no capping: k < 6, more than 1024 sequences, row-split batches
    CHECK(stoch(256, 5, V, fake(8), sv_workspace_bytes(256, 1, 5, V), false) == SV_OK);
    CHECK(last.seq && last.p.active == nullptr);
    CHECK(stoch(1025, 8, V, fake(8), sv_workspace_bytes(1025, 1, 8, V), false) == SV_OK);
    CHECK(last.seq && last.p.active == nullptr);
    // 128..191 sequences without diagnostics (k >= 6, a workspace): the
    // capped early exit too; with diagnostics, or below 128, row-split
    for (int B : {128, 160, 191}) {
        const size_t wsb = sv_workspace_bytes(B, 1, 8, V);
        CHECK(stoch(B, 8, V, fake(8), wsb, false) == SV_OK);
        CHECK(last.seq && last.p.active != nullptr);
        check_capped_layout(fake(8), wsb, B, 8);
        CHECK(stoch(B, 8, V, fake(8), wsb, true) == SV_OK);
        CHECK(!last.seq && last.p.active == nullptr);
        CHECK(stoch(B, 5, V, fake(8), sv_workspace_bytes(B, 1, 5, V), false) == SV_OK);
        CHECK(!last.seq && last.p.active == nullptr);  // no capping below k = 6
    }
    CHECK(stoch(127, 8, V, fake(8), sv_workspace_bytes(127, 1, 8, V), false) == SV_OK);
    CHECK(!last.seq && last.p.active == nullptr);
    // ragged batches take the capped exit too (k_max >= 6, no diagnostics)
    {
        const int B = 256, kmax = 8;
        const size_t wsb = sv_workspace_bytes(B, 1, kmax, V);
        CHECK(stoch(B, kmax, V, fake(8), wsb, false, (const int32_t*)fake(9), 1000) == SV_OK);
        CHECK(last.seq && last.p.active != nullptr && last.p.cu != nullptr);
        check_capped_layout(fake(8), wsb, B, kmax);
    }
    // the other layouts of the plan
    {
        const size_t big = (size_t)1 << 30;  // a workspace larger than any bound here
        int32_t* o = (int32_t*)fake(5);
        // greedy: one workgroup per sequence from 192 single candidates on
        last = Launch{};
        CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 192, 1, 8, V, V, SV_DTYPE_BF16,
                               o, o, nullptr, fake(8), big, nullptr) == SV_OK);
        CHECK(last.seq);
        CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 191, 1, 8, V, V, SV_DTYPE_BF16,
                               o, o, nullptr, fake(8), big, nullptr) == SV_OK);
        CHECK(!last.seq);
        // several candidates: always row-split (rows of all candidates spread)
        CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 512, 16, 4, 32000, 32000,
                               SV_DTYPE_F32, o, o, nullptr, fake(8), big, nullptr) == SV_OK);
        CHECK(!last.seq && last.p.G == 16 && last.p.rows_per_seq == 16 * 5);
        // trees: row-split, one row per node
        CHECK(sv_verify_greedy_tree(fake(0), (const int32_t*)fake(2), (const int32_t*)fake(3), 300,
                                    64, V, V, SV_DTYPE_BF16, o, o, o, fake(8), big,
                                    nullptr) == SV_OK);
        CHECK(!last.seq && last.p.rows_per_seq == 64);
        // ragged with diagnostics and unequal lengths: every row read, rows
        // balanced over the GPU (row-split); with equal lengths, one group
        // per sequence
        CHECK(stoch(256, 8, V, fake(8), big, true, (const int32_t*)fake(9), 1000) == SV_OK);
        CHECK(!last.seq && last.p.active == nullptr);
        CHECK(stoch(256, 8, V, fake(8), big, true, (const int32_t*)fake(9), 256 * 8) == SV_OK);
        CHECK(last.seq && last.p.active == nullptr);
        // plain sampling: one pass per row where that layout is faster,
        // else rows cut into slices drawn from their slice statistics
        last = Launch{};
        CHECK(sv_sample(fake(0), (const float*)fake(4), 256, V, V, SV_DTYPE_BF16, 1.0f, 0, o,
                        fake(8), big, nullptr) == SV_OK);
        CHECK(last.seq && last.p.k == 0);  // V <= 40960 + 352 * 256
        CHECK(sv_sample(fake(0), (const float*)fake(4), 64, V, V, SV_DTYPE_BF16, 1.0f, 0, o,
                        fake(8), big, nullptr) == SV_OK);
        CHECK(!last.seq && last.p.slice_draw == 1 && last.p.S >= 8);
        CHECK(sv_sample(fake(0), (const float*)fake(4), 512, 32000, 32000, SV_DTYPE_BF16, 1.0f, 0,
                        o, nullptr, 0, nullptr) == SV_OK);  // one pass needs no workspace
        CHECK(last.seq);
        // argmax sampling is greedy verification of rows with no drafts
        CHECK(sv_sample(fake(0), nullptr, 256, V, V, SV_DTYPE_BF16, 1.0f, 1, o, fake(8), big,
                        nullptr) == SV_OK);
        CHECK(last.seq && last.p.k == 0 && last.p.rows_per_seq == 1);
    }
    // argument checks answer before any launch
    CHECK(stoch(-1, 8, V, nullptr, 0, false) == SV_ERR_SHAPE && last.calls == 0);
    CHECK(stoch(4, SV_MAX_K + 1, V, nullptr, 0, false) == SV_ERR_SHAPE && last.calls == 0);
    CHECK(stoch(4, 8, V, nullptr, 0, false) == SV_ERR_NULL && last.calls == 0);  // row-split needs one
    CHECK(stoch(4, 8, V, fake(8), 16, false) == SV_ERR_WORKSPACE && last.calls == 0);
    CHECK(stoch(0, 8, V, nullptr, 0, false) == SV_OK && last.calls == 0);
    last = Launch{};
    CHECK(sv_verify_stochastic(fake(0), fake(1), (const int32_t*)fake(2), (const float*)fake(3),
                               (const float*)fake(4), 256, 8, V, V, SV_DTYPE_BF16, -1.0f,
                               (int32_t*)fake(5), (int32_t*)fake(6), nullptr, nullptr, 0,
                               nullptr) == SV_ERR_TEMPERATURE && last.calls == 0);
    CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 256, 1, 8, V, V - 1, SV_DTYPE_BF16,
                           (int32_t*)fake(5), (int32_t*)fake(6), nullptr, nullptr, 0,
                           nullptr) == SV_ERR_SHAPE && last.calls == 0);
    CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 256, 1, 8, V, V, 7,
                           (int32_t*)fake(5), (int32_t*)fake(6), nullptr, nullptr, 0,
                           nullptr) == SV_ERR_DTYPE && last.calls == 0);
    CHECK(strlen(sv_status_string(SV_ERR_HIP)) > 0);
    // a launch the HIP runtime refuses is reported as SV_ERR_HIP
    fail_with = 98;  // hipErrorInvalidDeviceFunction, say
    CHECK(stoch(256, 8, V, fake(8), sv_workspace_bytes(256, 1, 8, V), false) == SV_ERR_HIP);
    CHECK(stoch(4, 8, V, fake(8), sv_workspace_bytes(4, 1, 8, V), true) == SV_ERR_HIP);
    last = Launch{};
    CHECK(sv_verify_greedy(fake(0), (const int32_t*)fake(2), 256, 1, 8, V, V, SV_DTYPE_BF16,
                           (int32_t*)fake(5), (int32_t*)fake(6), nullptr, nullptr, 0,
                           nullptr) == SV_ERR_HIP);
    CHECK(sv_commit((const int32_t*)fake(2), (const int32_t*)fake(3), 4, 9, (int32_t*)fake(4),
                    (int32_t*)fake(5), 64, 64, (int32_t*)fake(6), 1, nullptr) == SV_ERR_HIP);
    fail_with = 0;
    if (fails) {
        fprintf(stderr, "%d checks failed\n", fails);
        return 1;
    }
    printf("host plan checks ok\n");
    return 0;
}
