// Host check of the decode work split and launch mapping in kvc_device.h.
// decode_split: for every key count L the items and wave shares cover keys
// [0, L) once, each share a multiple of 32 keys and at most DECODE_PART,
// every item has a wave with keys, the item count is ceil(L / 4096), and the
// active waves of an item are the ones the kernel counts.  decode_unit /
// decode_grid: over a launch of decode_grid(pairs, HC) ids, the ids with a
// unit hit every (pair, head chunk) exactly once, and the chunks of one pair
// share the id's residue mod 8 (one XCD).  Prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "kvc_device.h"

static int check_split(int L) {
    using namespace kvc;
    const DecodeSplit sp = decode_split(L);
    const int G = DECODE_GROUP, pw = sp.per_wave;
    if (sp.items != (L + G * DECODE_PART - 1) / (G * DECODE_PART)) return 1;
    if (pw <= 0 || pw % 32 != 0 || pw > DECODE_PART) return 2;
    int covered = 0;
    for (int i = 0; i < sp.items; ++i) {
        const int i0 = i * G * pw;
        int active = 0;
        for (int w = 0; w < G; ++w) {
            const int t0 = i0 + w * pw;
            if (t0 >= L) continue;
            if (t0 != covered) return 3;  // shares follow each other without gap or overlap
            const int t1 = t0 + pw < L ? t0 + pw : L;
            covered = t1;
            ++active;
        }
        if (active == 0) return 4;
        const int nact = (L - i0 + pw - 1) / pw < G ? (L - i0 + pw - 1) / pw : G;  // as the kernel counts
        if (nact != active) return 5;
    }
    return covered == L ? 0 : 6;
}

int main() {
    using namespace kvc;
    std::vector<int> lens;
    for (int L = 1; L <= 40000; ++L) lens.push_back(L);
    for (int L = 40001; L <= 1 << 20; L += 997) lens.push_back(L);
    for (int m = 1; m <= 256; ++m)
        for (int d = -2; d <= 2; ++d) lens.push_back(m * 4096 + d);
    for (int L : lens) {
        if (L < 1) continue;
        const int e = check_split(L);
        if (e) {
            std::printf("decode_split L=%d: check %d\n", L, e);
            return 1;
        }
    }
    for (int HC : {1, 2, 3, 4, 8, 16}) {
        for (int64_t pairs = 1; pairs <= 300; ++pairs) {
            const int64_t grid = decode_grid(pairs, HC);
            std::vector<int> seen(pairs * HC, 0);
            std::vector<int64_t> residue(pairs, -1);
            for (int64_t lid = 0; lid < grid; ++lid) {
                const DecodeUnit u = decode_unit(lid, HC);
                if (u.pair < 0 || u.hc < 0 || u.hc >= HC) {
                    std::printf("decode_unit out of range lid=%lld HC=%d\n", (long long)lid, HC);
                    return 1;
                }
                if (u.pair >= pairs) continue;
                ++seen[u.pair * HC + u.hc];
                if (HC > 1) {
                    if (residue[u.pair] < 0) residue[u.pair] = lid % 8;
                    if (residue[u.pair] != lid % 8) {
                        std::printf("chunks of pair %lld on different XCDs HC=%d\n", (long long)u.pair, HC);
                        return 1;
                    }
                }
            }
            for (int64_t i = 0; i < pairs * HC; ++i)
                if (seen[i] != 1) {
                    std::printf("unit %lld launched %d times pairs=%lld HC=%d\n", (long long)i, seen[i],
                                (long long)pairs, HC);
                    return 1;
                }
        }
    }
    std::printf("ok\n");
    return 0;
}
