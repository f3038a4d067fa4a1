// Host check of balance_one_round (the forward's dispatch order when the whole grid is
// resident at once): for the tile weights of the tiled forward, the table must be a
// permutation of the positions, and the busiest CU (local indices i, C + i, 2C + i, ...
// share CU i) must carry no more than under the heaviest-first order.
#include "../../causal_gqa_flash_amd/csrc/cgqa_launch.hpp"

#include <algorithm>
#include <cstdio>
#include <vector>

int main() {
    int failures = 0, checked = 0;
    for (int T : {64, 300, 512, 700, 1000, 1024, 2048})
        for (int per_qt : {1, 3, 6, 12, 24})
            for (int C : {32, 31})
                for (int S : {2, 3}) {
                    const int nqt = (T + 127) / 128, L = per_qt * nqt;
                    auto weight = [&](int p) {
                        const int qt = nqt - 1 - p / per_qt;
                        long w = 0;
                        for (int wv = 0; wv < 4; ++wv) {
                            const int qw = qt * 128 + 32 * wv;
                            if (qw < T) w += qw / 32 + 3;
                        }
                        return w;
                    };
                    unsigned char perm[256];
                    const int n = cgqa::balance_one_round(perm, L, C, S, weight);
                    if (L > C * S || L > 256) {
                        if (n != 0) { std::printf("T=%d per_qt=%d C=%d S=%d: table for a grid of %d\n", T, per_qt, C, S, L); ++failures; }
                        continue;
                    }
                    ++checked;
                    std::vector<int> seen(L, 0);
                    std::vector<long> load(C, 0), load0(C, 0);
                    for (int l = 0; l < L; ++l) {
                        ++seen[perm[l]];
                        load[l % C] += weight(perm[l]);
                        load0[l % C] += weight(l);
                    }
                    bool ok = n == L;
                    for (int p = 0; p < L; ++p) ok = ok && seen[p] == 1;
                    long mx = 0, mx0 = 0;
                    for (int c = 0; c < C; ++c) { mx = std::max(mx, load[c]); mx0 = std::max(mx0, load0[c]); }
                    if (!ok || mx > mx0) {
                        std::printf("T=%d per_qt=%d C=%d S=%d: permutation %d, busiest CU %ld vs %ld\n", T, per_qt, C, S,
                                    ok, mx, mx0);
                        ++failures;
                    }
                }
    std::printf("checked %d tables, %d failures\n", checked, failures);
    return failures != 0;
}
