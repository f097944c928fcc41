// Exhaustive scan of the oracle's fp32 exponential weight E(s) over every
// fp32 s in [-104, -0] (about 1.1e9 values), split across threads: reports
// the largest amount, in units in the last place (bit-pattern distance), by
// which E(s) falls below max{E(s') : s' <= s}, the largest value of E, and
// whether E(s) <= 1 everywhere.  Test infrastructure: loads the oracle
// library given on the command line.
#include <dlfcn.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

typedef float (*ExpFn)(float);

static uint32_t bits(float f) {
    uint32_t b;
    std::memcpy(&b, &f, 4);
    return b;
}

int main(int argc, char** argv) {
    if (argc < 3) return 2;
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) return 3;
    ExpFn E = (ExpFn)dlsym(h, "oracle_exp_weight");
    if (!E) return 4;
    const int nt = std::max(1, std::atoi(argv[2]));
    // s ascending: bit patterns from 0xC2D00000 (-104) down to 0x80000000 (-0).
    const uint32_t hi = 0xC2D00000u, lo = 0x80000000u;
    const uint64_t n = (uint64_t)hi - lo + 1;
    struct Part { float min, max; int drop; bool above_one; };
    std::vector<Part> parts(nt);
    std::vector<std::thread> pool;
    for (int t = 0; t < nt; ++t) {
        pool.emplace_back([&, t] {
            const uint64_t a = n * t / nt, b = n * (t + 1) / nt;  // offsets from hi downwards
            float run = 0.0f;
            int drop = 0;
            bool above = false;
            float mn = 2.0f;
            for (uint64_t i = a; i < b; ++i) {
                const uint32_t bb = hi - (uint32_t)i;
                float s;
                std::memcpy(&s, &bb, 4);
                const float e = E(s);
                mn = std::min(mn, e);
                above = above || e > 1.0f;
                if (e < run) drop = std::max(drop, (int)(bits(run) - bits(e)));
                else run = e;
            }
            parts[t] = {mn, run, drop, above};
        });
    }
    for (auto& th : pool) th.join();
    // Join the parts: a part's values also fall below the maxima of the
    // parts before it (its smallest value the furthest).
    float run = 0.0f;
    int drop = 0;
    bool above = false;
    for (int t = 0; t < nt; ++t) {
        drop = std::max(drop, parts[t].drop);
        above = above || parts[t].above_one;
        if (parts[t].min < run) drop = std::max(drop, (int)(bits(run) - bits(parts[t].min)));
        run = std::max(run, parts[t].max);
    }
    std::printf("drop_ulp %d max %a above_one %d\n", drop, run, above ? 1 : 0);
    return 0;
}
