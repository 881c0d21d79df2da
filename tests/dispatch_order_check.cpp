// Checks the dispatch maps of specv_dispatch.hpp over a grid of batch shapes:
// each is a bijection onto the tasks; every bonus workgroup comes after all
// rows of its sequence and the H bonus workgroups of a sequence come in
// order; in the fused order the T > 0 sequences' rows come first, the greedy
// sequences' draft rows all come before their target rows, and the greedy
// bonus workgroups come last. Prints "ok" or the first failure.
#include <cstdio>
#include <vector>

#include "specv_dispatch.hpp"

using specv::decode_chain;
using specv::decode_fused;

static int fail(const char* what, long B, long nS, long RS, long H, long g) {
    std::printf("FAIL %s B=%ld nS=%ld RS=%ld H=%ld g=%ld\n", what, B, nS, RS, H, g);
    return 1;
}

// pos[s * (RS + H) + w] = dispatch index of task (s, w), from either map.
static int check(long B, long nS, long RS, long H, bool fused) {
    const long n = B * (RS + H);
    std::vector<long> pos(n, -1);
    const long D = specv::bonus_delay(fused ? nS : B, RS);
    for (long g = 0; g < n; ++g) {
        int s;
        int64_t w;
        if (fused) decode_fused(g, B, nS, RS / 2, H, specv::bonus_delay(B, RS), s, w);
        else decode_chain(g, B, RS, H, D, s, w);
        if (s < 0 || s >= B || w < 0 || w >= RS + H) return fail("out of range", B, nS, RS, H, g);
        long& p = pos[s * (RS + H) + w];
        if (p != -1) return fail("task hit twice", B, nS, RS, H, g);
        p = g;
    }
    for (long s = 0; s < B; ++s) {
        const long* t = &pos[s * (RS + H)];
        long last_row = -1;
        for (long w = 0; w < RS; ++w) last_row = t[w] > last_row ? t[w] : last_row;
        for (long h = 0; h < H; ++h) {
            if (t[RS + h] <= last_row) return fail("bonus before a row", B, nS, RS, H, t[RS + h]);
            if (h > 0 && t[RS + h] <= t[RS + h - 1]) return fail("bonus out of order", B, nS, RS, H, t[RS + h]);
        }
    }
    if (fused) {
        // T > 0 rows before every greedy row; greedy draft rows, then greedy
        // target rows; the greedy bonus workgroups are the last nG * H.
        const long half = RS / 2, nG = B - nS;
        long last_sampled_row = -1, first_greedy_row = n, last_draft = -1, first_target = n, last_target = -1;
        for (long s = 0; s < B; ++s) {
            const long* t = &pos[s * (RS + H)];
            for (long w = 0; w < RS; ++w) {
                if (s < nS) {
                    last_sampled_row = t[w] > last_sampled_row ? t[w] : last_sampled_row;
                    continue;
                }
                first_greedy_row = t[w] < first_greedy_row ? t[w] : first_greedy_row;
                if (w >= half) last_draft = t[w] > last_draft ? t[w] : last_draft;
                else {
                    first_target = t[w] < first_target ? t[w] : first_target;
                    last_target = t[w] > last_target ? t[w] : last_target;
                }
            }
            if (s >= nS)
                for (long h = 0; h < H; ++h)
                    if (t[RS + h] < n - nG * H) return fail("greedy bonus not last", B, nS, RS, H, t[RS + h]);
        }
        if (last_sampled_row > first_greedy_row) return fail("greedy row before a T > 0 row", B, nS, RS, H, first_greedy_row);
        if (nG > 0 && last_draft > first_target) return fail("greedy target before draft", B, nS, RS, H, first_target);
    }
    return 0;
}

int main() {
    const long Bs[] = {1, 2, 3, 7, 64, 91, 92, 256, 300};
    const long RSs[] = {2, 3, 17, 18, 34, 130};
    const long Hs[] = {1, 2, 8, 16};
    int bad = 0;
    for (long B : Bs)
        for (long RS : RSs)
            for (long H : Hs) {
                bad += check(B, B, RS, H, false);
                if (RS % 2) continue;
                for (long nS : {0L, 1L, B / 3, B / 2, B - 1, B}) {
                    if (nS < 0 || nS > B) continue;
                    bad += check(B, nS, RS, H, true);
                }
                if (bad) return 1;
            }
    std::printf("ok\n");
    return 0;
}
