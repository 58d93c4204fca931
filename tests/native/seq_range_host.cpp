// Host-side check of seq_range, the helper every attention kernel uses to turn
// a packed-sequence table into a token range: for any table contents (random
// or adversarial), the range it returns must lie inside [0, total] and be no
// longer than the caller's maximum, so no kernel access can leave the tensors.
// Reads cases from stdin: "total N Hq n e0 e1 ... en" per line, or
// "-1 N Hq B" for B fixed-length sequences (no table); prints
// "tok0 len lse0 st0 hs" for every sequence b of every case.
#include <cstdio>
#include <vector>

#include "../../ulysses_sequence_parallelism_attn_amd/csrc/ul_internal.h"

int main() {
    long long total, N;
    int Hq, n;
    while (std::scanf("%lld %lld %d %d", &total, &N, &Hq, &n) == 4) {
        if (total < 0) {  // fixed-length batches: no table
            for (int b = 0; b < n; ++b) {
                const ul::SeqRange r = ul::seq_range(nullptr, b, N, Hq, 0);
                std::printf("%lld %d %lld %lld %lld\n", (long long)r.tok0, r.len,
                            (long long)r.lse0, (long long)r.st0, (long long)r.hs);
            }
            continue;
        }
        std::vector<int32_t> cu(n + 1);
        for (int i = 0; i <= n; ++i) std::scanf("%d", &cu[i]);
        for (int b = 0; b < n; ++b) {
            const ul::SeqRange r = ul::seq_range(cu.data(), b, N, Hq, total);
            std::printf("%lld %d %lld %lld %lld\n", (long long)r.tok0, r.len, (long long)r.lse0,
                        (long long)r.st0, (long long)r.hs);
        }
    }
    return 0;
}
