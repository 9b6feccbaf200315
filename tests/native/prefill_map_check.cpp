// Host check of the prefill work mapping in kvc_device.h: for every row count
// q and position blocks per item npb, the snake order deals each 32-position
// block to exactly one (item, slot), every item holds at least one block, and
// prefill_item_end is the end of the item's last block.  Prints "ok" or the
// first failure.
#include <cstdio>
#include <vector>

#include "kvc_device.h"

int main() {
    using namespace kvc;
    for (int q = 1; q <= 6000; ++q) {
        for (int npb : {1, 2, 4, 8}) {
            const int nb = (q + PREFILL_QW - 1) / PREFILL_QW;
            const int span = PREFILL_QW * npb;
            const int T = (q + span - 1) / span;  // items per sequence, as the planner counts them
            if (T != (nb + npb - 1) / npb) {
                std::printf("item count q=%d npb=%d\n", q, npb);
                return 1;
            }
            std::vector<int> seen(nb, 0);
            for (int t = 0; t < T; ++t) {
                int end = 0, blocks = 0;
                for (int k = 0; k < npb; ++k) {
                    const int b = prefill_block(t, k, T);
                    if (b < 0 || b >= npb * T) {
                        std::printf("block out of range q=%d npb=%d t=%d k=%d\n", q, npb, t, k);
                        return 1;
                    }
                    if (b < nb) {
                        ++seen[b];
                        ++blocks;
                        const int e = (b + 1) * PREFILL_QW < q ? (b + 1) * PREFILL_QW : q;
                        end = e > end ? e : end;
                    }
                }
                if (blocks == 0 || prefill_item_end(t, q, npb) != end) {
                    std::printf("item end q=%d npb=%d t=%d\n", q, npb, t);
                    return 1;
                }
            }
            for (int b = 0; b < nb; ++b)
                if (seen[b] != 1) {
                    std::printf("block %d dealt %d times q=%d npb=%d\n", b, seen[b], q, npb);
                    return 1;
                }
        }
    }
    std::printf("ok\n");
    return 0;
}
