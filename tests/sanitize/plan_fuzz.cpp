// Randomised driver for the library's host-side plan code (qm_plan_encode,
// qm_plan_info, qm_update_workspace_bytes), built with AddressSanitizer and
// UndefinedBehaviorSanitizer by tests/test_sanitizers_cpu.py.  Device
// addresses are fake (only their alignment and overlap are ever looked at on
// the host).  Any out-of-bounds access or undefined behaviour aborts; the
// driver itself checks the encoder's invariants on the plans it accepts.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "qmuon.h"

static int fails = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            fails++;                                                     \
        }                                                                \
    } while (0)

int main(int argc, char **argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 3000;
    std::mt19937_64 rng(12345);
    auto uni = [&](int64_t lo, int64_t hi) { return std::uniform_int_distribution<int64_t>(lo, hi)(rng); };
    int accepted = 0;
    for (int it = 0; it < iters; it++) {
        const int nt = (int)uni(1, 6);
        std::vector<qm_q8_tensor> t(nt);
        uintptr_t addr = (uintptr_t)1 << 40;
        for (int i = 0; i < nt; i++) {
            const int64_t n = uni(0, 9) == 0 ? uni(1, 300) : uni(1, 5000);
            const int dt = (int)uni(0, 3) == 3 ? (int)uni(-1, 5) : (int)uni(0, 2);
            t[i].numel = n;
            t[i].grad_dtype = dt;
            t[i].reserved = 0;
            t[i].codes = reinterpret_cast<int8_t *>(addr + (uni(0, 15) == 0 ? 8 : 0));
            addr += (uintptr_t)(n + 4096) / 4096 * 4096 + 4096;
            t[i].absmax = reinterpret_cast<float *>(addr);
            addr += (uintptr_t)((n + 255) / 256 * 4 + 4096) / 4096 * 4096 + 4096;
            t[i].grad = reinterpret_cast<void *>(addr);
            t[i].grad_cols = 0;
            t[i].grad_ld = 0;
            if (uni(0, 4) == 0) {   // a strided view, valid or not
                int64_t cols = 8 * uni(1, 16);
                while (cols > 8 && n % cols) cols -= 8;   // rows must divide numel (else refused)
                t[i].grad_cols = uni(0, 5) == 0 ? uni(-8, 40) : cols;
                t[i].grad_ld = cols + 8 * uni(0, 4) - (uni(0, 9) == 0 ? 4 : 0);
            }
            addr += (uintptr_t)(n * 4 * 4 + 4096) / 4096 * 4096 + 4096;
            if (uni(0, 30) == 0 && i > 0) t[i].grad = t[i - 1].grad;   // aliasing
        }
        // segments: mostly a valid cover, sometimes perturbed
        std::vector<qm_norm_segment> s;
        for (int i = 0; i < nt; i++) {
            int64_t pos = 0;
            const int64_t n = t[i].numel;
            while (pos < n) {
                int64_t len = 256 * uni(1, 4);
                if (pos + len > n) len = n - pos;
                s.push_back(qm_norm_segment{i, 0, pos, len});
                pos += len;
            }
        }
        // every group gets at least one segment (an empty group is refused)
        const int ng = (int)uni(1, std::min<int64_t>(5, (int64_t)s.size()));
        for (size_t k = 0; k < s.size(); k++) s[k].group_id = k < (size_t)ng ? (int32_t)k : (int32_t)uni(0, ng - 1);
        const int mode = (int)uni(0, 9);   // 0, 6..9: keep the cover valid
        if (mode == 1 && !s.empty()) s[uni(0, s.size() - 1)].start += uni(-300, 300);
        if (mode == 2 && !s.empty()) s[uni(0, s.size() - 1)].length += uni(-300, 300);
        if (mode == 3 && !s.empty()) s.erase(s.begin() + uni(0, s.size() - 1));
        if (mode == 4 && !s.empty()) s.push_back(s[uni(0, s.size() - 1)]);
        if (mode == 5 && !s.empty()) s[uni(0, s.size() - 1)].tensor_index = (int32_t)uni(-2, nt + 1);
        size_t bytes = 0;
        const qm_status st = qm_plan_encode(t.data(), nt, s.data(), (int32_t)s.size(), ng, nullptr, &bytes);
        CHECK(st == QM_OK || qm_last_error()[0] != 0);
        if (st != QM_OK) continue;
        std::vector<uint64_t> blob((bytes + 7) / 8 + 1);
        size_t b2 = bytes;
        CHECK(qm_plan_encode(t.data(), nt, s.data(), (int32_t)s.size(), ng, blob.data(), &b2) == QM_OK);
        CHECK(b2 <= bytes);
        size_t small = bytes - 8;   // a too-small buffer is refused
        if (bytes > 8) CHECK(qm_plan_encode(t.data(), nt, s.data(), (int32_t)s.size(), ng, blob.data(), &small) != QM_OK);
        CHECK(qm_plan_encode(t.data(), nt, s.data(), (int32_t)s.size(), ng, blob.data(), &b2) == QM_OK);
        int32_t ont = 0, ong = 0;
        int64_t onb = 0, onumel = 0;
        CHECK(qm_plan_info(blob.data(), &ont, &ong, &onb, &onumel) == QM_OK);
        int64_t blocks = 0, numel = 0;
        for (const auto &x : t) {
            blocks += (x.numel + 255) / 256;
            numel += x.numel;
        }
        CHECK(ont == nt && ong == ng && onb == blocks && onumel == numel);
        CHECK(qm_update_workspace_bytes(blob.data()) >= (size_t)blocks * 8);
        // a corrupted blob is refused, not read past its tables
        std::vector<uint64_t> bad(blob);
        bad[0] ^= 1;
        CHECK(qm_plan_info(bad.data(), nullptr, nullptr, nullptr, nullptr) != QM_OK);
        CHECK(qm_update_workspace_bytes(bad.data()) == 0);
        accepted++;
    }
    CHECK(qm_plan_info(nullptr, nullptr, nullptr, nullptr, nullptr) != QM_OK);
    printf("plan_fuzz: %d iterations, %d plans accepted, %d failed checks\n", iters, accepted, fails);
    return fails ? 1 : 0;
}
