// Checks the dispatch maps of specv_dispatch.hpp over a grid of batch shapes:
// each is a bijection onto the tasks; every bonus workgroup comes after all
// rows of its sequence and the H bonus workgroups of a sequence come in
// order for a T > 0 sequence (a greedy one's last first in the fused order); in the fused order the T > 0 sequences' rows come first, the greedy
// sequences' draft rows all come before their target rows, and the greedy
// bonus workgroups come last. Also the row splits (choose_split,
// small_split): chunks cover the row exactly once, are multiples of 8
// elements, respect their minimum length and the count limits. Prints "ok"
// or the first failure.
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
    const long D = specv::bonus_delay(B, RS);
    for (long g = 0; g < n; ++g) {
        int s;
        int64_t w;
        if (fused) decode_fused(g, B, nS, RS / 2, H, specv::bonus_delay(B, RS), s, w);
        else decode_chain(g, B, nS, RS, H, D, s, w);
        if (s < 0 || s >= B || w < 0 || w >= RS + H) return fail("out of range", B, nS, RS, H, g);
        long& p = pos[s * (RS + H) + w];
        if (p != -1) return fail("task hit twice", B, nS, RS, H, g);
        p = g;
    }
    for (long s = 0; s < B; ++s) {
        const long* t = &pos[s * (RS + H)];
        long last_row = -1;
        for (long w = 0; w < RS; ++w) last_row = t[w] > last_row ? t[w] : last_row;
        // A T > 0 sequence's H bonus workgroups come in order h = 0 .. H-1
        // (the last collects what the others publish). A greedy sequence's
        // need no order (only the last has work); in the fused order its
        // last one comes first.
        for (long h = 0; h < H; ++h) {
            if (t[RS + h] <= last_row) return fail("bonus before a row", B, nS, RS, H, t[RS + h]);
            if (s < nS && h > 0 && t[RS + h] <= t[RS + h - 1])
                return fail("bonus out of order", B, nS, RS, H, t[RS + h]);
            if (fused && s >= nS && h < H - 1 && t[RS + h] <= t[RS + H - 1])
                return fail("greedy bonus: the last not first", B, nS, RS, H, t[RS + h]);
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

// One split of a row of V elements for `rows` row tasks: S chunks of `chunk`
// elements (the last one shorter) that cover [0, V) exactly.
static int check_split(const char* name, long rows, long V, int32_t S, int64_t chunk, long max_s, long min_chunk,
                       long target) {
    const bool ok = S >= 1 && S <= max_s && chunk % 8 == 0 && int64_t(S) * chunk >= V &&
                    int64_t(S - 1) * chunk < V && (S == 1 || chunk >= min_chunk) && rows * S <= target + rows;
    if (!ok) std::printf("FAIL %s rows=%ld V=%ld S=%d chunk=%lld\n", name, rows, V, S, (long long)chunk);
    return ok ? 0 : 1;
}

int main() {
    const long rowss[] = {1, 2, 3, 5, 9, 17, 18, 100, 513, 1023, 1024, 1025, 2047, 2048, 2049, 5000, 100000};
    const long Vs[] = {1, 2, 7, 8, 9, 4095, 4096, 4097, 8191, 16383, 16384, 16385, 32000, 128256, 152064, 600000,
                       1048576};
    for (long rows : rowss)
        for (long V : Vs) {
            int32_t S;
            int64_t chunk;
            specv::choose_split(rows, V, &S, &chunk);
            if (check_split("choose_split", rows, V, S, chunk, 64, 4096, 2048)) return 1;
            specv::small_split(rows, V, &S, &chunk);
            if (check_split("small_split", rows, V, S, chunk, specv::kMaxTopfChunks, 16384, 1024)) return 1;
        }
    const long Bs[] = {1, 2, 3, 7, 64, 91, 92, 256, 300};
    const long RSs[] = {2, 3, 17, 18, 34, 130};
    const long Hs[] = {1, 2, 8, 16};
    int bad = 0;
    for (long B : Bs)
        for (long RS : RSs)
            for (long H : Hs) {
                for (long nS : {0L, 1L, B / 3, B / 2, B - 1, B}) {
                    if (nS < 0 || nS > B) continue;
                    bad += check(B, nS, RS, H, false);
                    if (RS % 2 == 0) bad += check(B, nS, RS, H, true);
                }
                if (bad) return 1;
            }
    std::printf("ok\n");
    return 0;
}
