// Host build of the kernels' visibility ranges (ja_tiles.h), driven by
// tests/test_tiles_host.py. Reads lines "row Lq Lk causal window bsh x0 n" from
// stdin and prints, per line, the keys query `row` sees and the queries that see
// key `row` as "lo width lo width", then whether the key range misses / covers
// the block [x0, x0 + n).
#include <cstdio>

#include "ja_tiles.h"

int main() {
    int row, Lq, Lk, causal, window, bsh, x0, n;
    while (std::scanf("%d %d %d %d %d %d %d %d", &row, &Lq, &Lk, &causal, &window, &bsh, &x0, &n) == 8) {
        const ja::VisRange k = ja::keys_seen_by(row, Lk, causal, window, bsh);
        const ja::VisRange q = ja::queries_seeing(row, Lq, Lk, causal, window, bsh);
        std::printf("%d %d %d %d %d %d\n", k.lo, k.width, q.lo, q.width, (int)k.misses(x0, n),
                    (int)k.covers(x0, n));
    }
    return 0;
}
