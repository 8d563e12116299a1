// Checks of the work-item maps in attn_sched.h (compiled with g++ by tests/test_sched_cpu.py):
//   * work_item_of is a bijection from dispatch indices onto (head, tile) pairs, and with a head count
//     that is a multiple of the XCD count it keeps every head on one XCD and issues position-major;
//   * persistent_item maps each round of a persistent grid onto exactly that round's items, keeping
//     every item on the XCD of the workgroup that takes it;
//   * persistent_grid is 0 or a multiple of the XCD count no larger than the compute units, and is
//     0 exactly when the items fit in one round or the heads do not spread evenly over the XCDs.
#include "attn_sched.h"

#include <cstdio>
#include <vector>

static int failures = 0;
#define EXPECT(c, ...)                      \
    do {                                    \
        if (!(c)) {                         \
            if (failures < 20) {            \
                printf("FAIL: " __VA_ARGS__); \
                printf("\n");               \
            }                               \
            ++failures;                     \
        }                                   \
    } while (0)

int main()
{
    long long checks = 0;
    for (int nx : {1, 2, 4, 8}) {
        for (int n_heads : {1, 3, 7, 8, 16, 24, 32, 64}) {
            for (int n_tiles : {1, 2, 5, 8, 16, 33}) {
                const int G = n_heads * n_tiles;
                std::vector<int> seen(G, 0);
                for (int g = 0; g < G; ++g) {
                    int head, t;
                    attn::work_item_of(g, G, n_tiles, nx, head, t);
                    EXPECT(head >= 0 && head < n_heads && t >= 0 && t < n_tiles, "range nx=%d heads=%d tiles=%d g=%d", nx,
                           n_heads, n_tiles, g);
                    if (head >= 0 && head < n_heads && t >= 0 && t < n_tiles) ++seen[head * n_tiles + t];
                    if (n_heads % nx == 0) {
                        EXPECT(head % nx == g % nx, "xcd nx=%d heads=%d tiles=%d g=%d head=%d", nx, n_heads, n_tiles, g, head);
                        EXPECT(t == g / n_heads, "position-major nx=%d heads=%d g=%d", nx, n_heads, g);
                    }
                    ++checks;
                }
                for (int i = 0; i < G; ++i) EXPECT(seen[i] == 1, "bijection nx=%d heads=%d tiles=%d item=%d count=%d", nx, n_heads, n_tiles, i, seen[i]);
            }
        }
        for (int cus : {8, 32, 80, 96, 255, 256, 304}) {
            for (long long n_heads : {8LL, 16LL, 12LL, 64LL}) {
                for (long long n_items : {n_heads, n_heads * 32, n_heads * 100}) {
                    const long long P = attn::persistent_grid(n_items, n_heads, cus, nx);
                    const bool want = n_items > (long long)(cus / nx) * nx && n_heads % nx == 0;
                    EXPECT((P != 0) == want, "grid choice nx=%d cus=%d heads=%lld items=%lld P=%lld", nx, cus, n_heads, n_items, P);
                    if (P == 0) continue;
                    EXPECT(P % nx == 0 && P <= cus && P > cus - nx, "grid size nx=%d cus=%d P=%lld", nx, cus, P);
                    const long long rounds = (n_items + P - 1) / P;
                    for (long long r = 0; r < rounds; ++r) {
                        std::vector<int> hit(P, 0);
                        for (int g = 0; g < P; ++g) {
                            const long long item = attn::persistent_item((int)r, g, (int)P, nx);
                            EXPECT(item >= r * P && item < (r + 1) * P, "round nx=%d P=%lld r=%lld g=%d item=%lld", nx, P, r, g, item);
                            EXPECT(item % nx == g % nx, "persistent xcd nx=%d P=%lld r=%lld g=%d", nx, P, r, g);
                            if (item >= r * P && item < (r + 1) * P) ++hit[item - r * P];
                            ++checks;
                        }
                        for (int i = 0; i < P; ++i) EXPECT(hit[i] == 1, "round permutation nx=%d P=%lld r=%lld slot=%d", nx, P, r, i);
                    }
                }
            }
        }
    }
    // causal pairing: only while the paired grid fills every resident slot
    EXPECT(attn::causal_pairs(32, 16, 256), "c5 shape pairs (256 workgroups)");
    EXPECT(attn::causal_pairs(64, 16, 256), "c3 shape pairs");
    EXPECT(!attn::causal_pairs(32, 8, 256), "2048 query rows on 32 heads: 128 paired workgroups do not fill 256");
    EXPECT(!attn::causal_pairs(1, 1, 256), "one block");
    EXPECT(attn::causal_pairs(1, 3, 2) && !attn::causal_pairs(1, 3, 3), "odd count: the middle block is a pair of its own");
    checks += 5;
    printf("%lld checks, %d failures\n", checks, failures);
    return failures == 0 ? 0 : 1;
}
