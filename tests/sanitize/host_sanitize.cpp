// host_sanitize.cpp -- runs the library's host-only code (segment_isolated_packed_amd/csrc/
// kev_host.cpp: KEV_CHECK validation of device arrays copied to the host, the host-side work
// list, the decode split count) on random and edge-case inputs under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The work list is checked against a brute-force enumeration of
// the unmasked (query, key) pairs: every pair of every question is covered by exactly one
// item, and no item reaches past its question (the block-diagonal AND causal mask of the Kev
// article, icman.com.cn, sections 2.1 and 2.3).  Exit status 0 = every check passed.
#include <cstdint>
#include <cstdio>
#include <random>
#include <set>
#include <utility>
#include <vector>

#include "../../include/kev.h"
#include "../../segment_isolated_packed_amd/csrc/kev_host.h"
#include "../../segment_isolated_packed_amd/csrc/kev_tiles.h"

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

using namespace kev;

static void schedule_cases(std::mt19937 &rng) {
    for (int trial = 0; trial < 200; ++trial) {
        const int n_seg = 1 + (int)(rng() % 70);
        std::vector<int32_t> cu(n_seg + 1, 0);
        for (int s = 0; s < n_seg; ++s) {
            const int kind = (int)(rng() % 4);
            const int len = kind == 0 ? 0 : kind == 1 ? 1 : (int)(rng() % 300);
            cu[s + 1] = cu[s] + len;
        }
        const int br = (trial % 3 == 0) ? 32 : (trial % 3 == 1) ? 64 : 128;
        const int order = trial % 2;
        const int32_t cap = (int32_t)max_items(cu[n_seg], n_seg, br);
        std::vector<int32_t> items(2 * (size_t)cap + 1);
        int32_t n = -1;
        CHECK(host::schedule(cu.data(), n_seg, br, order, items.data(), cap, &n) == KEV_OK);
        // brute force: each (question, query row, key) with key <= row inside the question
        std::set<std::pair<int, int>> seen;   // (question, query block)
        int64_t covered = 0, expect = 0;
        for (int s = 0; s < n_seg; ++s) {
            const int64_t L = cu[s + 1] - cu[s];
            expect += L * (L + 1) / 2;
        }
        for (int i = 0; i < n; ++i) {
            const int s = items[2 * i], t = items[2 * i + 1];
            CHECK(s >= 0 && s < n_seg);
            if (s < 0 || s >= n_seg) continue;
            const int L = cu[s + 1] - cu[s];
            CHECK(t >= 0 && t < qblocks(L, br));
            CHECK(seen.insert({s, t}).second);
            for (int row = t * br; row < std::min((t + 1) * br, L); ++row) covered += row + 1;
        }
        CHECK(covered == expect);
        // too small an item buffer is refused, not overrun
        if (n > 0) CHECK(host::schedule(cu.data(), n_seg, br, order, items.data(), n - 1, &n) == KEV_ERR_INVALID_ARG);
    }
    const int32_t bad[] = {0, 5, 3};
    int32_t n = 0, items[16];
    CHECK(host::schedule(bad, 2, 32, 0, items, 8, &n) == KEV_ERR_BAD_SEQLENS);
    CHECK(host::schedule(bad, 2, 32, 7, items, 8, &n) == KEV_ERR_INVALID_ARG);
    const int32_t empty[] = {0};
    CHECK(host::schedule(empty, 0, 32, 0, nullptr, 0, &n) == KEV_OK && n == 0);
}

static void check_cases() {
    const int32_t cu_ok[] = {0, 0, 4, 9}, cu_bad[] = {1, 4, 9}, cu_dec[] = {0, 5, 4};
    CHECK(host::check_seqlens(cu_ok, 3, 9) == KEV_OK);
    CHECK(host::check_seqlens(cu_ok, 3, 8) == KEV_ERR_BAD_SEQLENS);
    CHECK(host::check_seqlens(cu_bad, 2, 9) == KEV_ERR_BAD_SEQLENS);
    CHECK(host::check_seqlens(cu_dec, 2, 4) == KEV_ERR_BAD_SEQLENS);

    const int32_t ids[] = {2, 0, 1}, dup[] = {2, 2, 1}, out_of_range[] = {2, 3, 1};
    const int32_t pre[] = {0, 6, 1};
    CHECK(host::check_slot_list(ids, nullptr, cu_ok, 3, 3, 5) == KEV_OK);
    CHECK(host::check_slot_list(dup, nullptr, cu_ok, 3, 3, 5) == KEV_ERR_BAD_SLOT);
    CHECK(host::check_slot_list(out_of_range, nullptr, cu_ok, 3, 3, 5) == KEV_ERR_BAD_SLOT);
    CHECK(host::check_slot_list(ids, nullptr, cu_ok, 3, 3, 4) == KEV_ERR_SLOT_OVERFLOW);
    CHECK(host::check_slot_list(ids, pre, cu_ok, 3, 3, 10) == KEV_OK);
    CHECK(host::check_slot_list(ids, pre, cu_ok, 3, 3, 9) == KEV_ERR_SLOT_OVERFLOW);

    const int32_t lens[] = {1, 5, 3}, lens0[] = {0, 5, 3}, lens_big[] = {1, 6, 3};
    CHECK(host::check_decode(ids, lens, 3, 3, 5) == KEV_OK);
    CHECK(host::check_decode(dup, lens, 3, 3, 5) == KEV_ERR_BAD_SLOT);
    CHECK(host::check_decode(ids, lens0, 3, 3, 5) == KEV_ERR_SLOT_OVERFLOW);
    CHECK(host::check_decode(ids, lens_big, 3, 3, 5) == KEV_ERR_SLOT_OVERFLOW);

    // paged: 3 requests, tables of 3 blocks of 4 rows; request 2 is longer than its table
    // (validated before any other request's append target is looked up)
    const int32_t tables[] = {0, 1, -1, 2, 3, -1, 4, 5, 6};
    const int32_t plens[] = {5, 4, 12}, plong[] = {5, 4, 13}, pshared[] = {5, 4, 12};
    CHECK(host::check_paged(tables, plens, 3, 3, 7, 4) == KEV_OK);
    CHECK(host::check_paged(tables, plong, 3, 3, 7, 4) == KEV_ERR_SLOT_OVERFLOW);
    const int32_t t_bad[] = {0, 1, -1, 2, 9, -1, 4, 5, 6}, lens_b[] = {5, 5, 12};
    CHECK(host::check_paged(t_bad, plens, 3, 3, 7, 4) == KEV_OK);   // block 9 lies past request 1's rows
    CHECK(host::check_paged(t_bad, lens_b, 3, 3, 7, 4) == KEV_ERR_BAD_SLOT);
    const int32_t t_clash[] = {0, 1, -1, 1, 3, -1, 4, 5, 6};   // request 1 reads block 1, where request 0 appends
    CHECK(host::check_paged(t_clash, pshared, 3, 3, 7, 4) == KEV_ERR_BAD_SLOT);

    CHECK(host::decode_splits(512, 256, 0) == 1);
    CHECK(host::decode_splits(8, 256, 0) == 8);
    CHECK(host::decode_splits(128, 256, 0) == 4);
    CHECK(host::decode_splits(8, 256, 100) == kMaxDecodeSplits);
    CHECK(host::decode_splits(0, 256, 0) == 1);
}

int main() {
    std::mt19937 rng(20261202u);
    schedule_cases(rng);
    check_cases();
    if (failures) {
        std::fprintf(stderr, "%d host checks failed\n", failures);
        return 1;
    }
    std::printf("host sanitizer run: all checks passed\n");
    return 0;
}
