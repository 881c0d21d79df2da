// Launch shapes: how rows split into chunks (choose_split, small_split) and
// the dispatch order of the chain launches (which sequence and which task
// each workgroup index stands for). Plain integer arithmetic with no GPU
// types, so that the host (and a CPU test) can check it.
//
// The chain launches rely on two properties of these maps:
//   * each map is a bijection from [0, B * (RS + H)) onto the tasks;
//   * every bonus workgroup of a sequence comes after all of its rows, and its
//     H bonus workgroups come in order h = 0 .. H-1 (the last one collects
//     what the others publish).
// So a bonus workgroup waits only for workgroups of lower index, which the
// hardware normally starts first: its waits are short. Correctness and
// termination do not depend on that order: every wait is bounded, and a
// sequence whose bonus workgroup gives up is completed by the finisher
// launch, after the whole launch has drained.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define SPECV_HD __host__ __device__
#else
#define SPECV_HD
#endif

namespace specv {

// Split of a row into chunks so that small batches still fill the GPU:
// aim for ~2048 workgroups, never chunks shorter than 4096 elements.
inline void choose_split(int64_t row_tasks, int64_t V, int32_t* S, int64_t* chunk) {
    int64_t s = (2048 + row_tasks - 1) / row_tasks;
    const int64_t by_len = V / 4096 > 0 ? V / 4096 : 1;
    if (s > by_len) s = by_len;
    if (s > 64) s = 64;
    if (s < 1) s = 1;
    int64_t c = (V + s - 1) / s;
    c = (c + 7) / 8 * 8;
    s = (V + c - 1) / c;
    *S = int32_t(s);
    *chunk = c;
}

// Chunks per row of the fused verify + top-F kernel (its 2 * gamma + 2 rows
// per sequence), so that small batches still spread over the GPU. A draft-row
// chunk's top-K workgroup is bound by its chain of round trips more than by
// its bytes, so the split aims at ~1024 workgroups (not the ~2048 of
// choose_split) with chunks of at least 16384 elements (one chunk per row
// from ~57 sequences of gamma = 8 up), and at most kMaxTopfChunks so that a
// row's chunk keys (kTopfKeyWords each) fit the merging workgroup's LDS.
constexpr int kTopfKeyWords = 32;   // the largest F + 1
constexpr int kMaxTopfChunks = 31;
inline void small_split(int64_t rows, int64_t V, int32_t* S, int64_t* chunk) {
    int64_t s = (1024 + rows - 1) / rows;
    const int64_t by_len = V / 16384 > 0 ? V / 16384 : 1;
    if (s > by_len) s = by_len;
    if (s > kMaxTopfChunks) s = kMaxTopfChunks;
    if (s < 1) s = 1;
    int64_t c = (V + s - 1) / s;
    c = (c + 7) / 8 * 8;
    *chunk = c;
    *S = int32_t((V + c - 1) / c);
}

// How many sequences the bonus workgroups of a sequence trail its rows by in
// dispatch order: about one GPU-full of row workgroups (RS per sequence), so
// that when they start their rows are (nearly) done and they do not hold CU
// slots waiting.
inline SPECV_HD int32_t bonus_delay(int64_t B, int64_t RS) {
    const int64_t d = (1536 + RS - 1) / RS;
    return int32_t(d < B ? d : B);
}

// Chain launch: slots 0 .. nS-1 hold the T > 0 sequences, nS .. B-1 the
// greedy ones (nS = B: identity order). Unit u = the RS row workgroups of
// the sequence in slot u (u < B), then the H bonus workgroups of slot u - D
// (u >= D); units B .. B+D-1 hold the rest of the bonus workgroups: those of
// T > 0 slots in order, then the last one of each greedy slot (the only one
// with work), then the other greedy ones, which return at once. Maps workgroup g to its slot and its index w in the
// slot's tasks (w < RS: row chunk w; else bonus workgroup w - RS).
inline SPECV_HD void decode_chain(int64_t g, int64_t B, int64_t nS, int64_t RS, int64_t H, int64_t D, int& sidx,
                                  int64_t& w) {
    if (D > B) D = B;
    const int64_t a_end = D * RS;                      // units 0..D-1: rows only
    const int64_t b_end = a_end + (B - D) * (RS + H);  // units D..B-1: rows, then bonus of u - D
    if (g < a_end) {
        sidx = int(g / RS);
        w = g % RS;
    } else if (g < b_end) {
        const int64_t u = D + (g - a_end) / (RS + H);
        const int64_t o = (g - a_end) % (RS + H);
        sidx = int(o < RS ? u : u - D);
        w = o;
    } else {                                           // the bonus of slots B-D .. B-1
        const int64_t i = g - b_end;
        const int64_t s0 = B - D;
        const int64_t nT = nS > s0 ? nS - s0 : 0;      // T > 0 slots among them
        const int64_t g0 = s0 + nT;                    // the first greedy one
        const int64_t nG = B - g0;
        if (i < nT * H) {
            sidx = int(s0 + i / H);
            w = RS + i % H;
        } else if (i - nT * H < nG) {
            sidx = int(g0 + (i - nT * H));
            w = RS + H - 1;
        } else {
            const int64_t j = i - nT * H - nG;
            sidx = int(g0 + j % nG);
            w = RS + j / nG;
        }
    }
}

// Fused verify + top-F launch. Sequence slots 0 .. nS-1 hold the T > 0
// sequences and nS .. B-1 the greedy ones; each has `half` target rows
// (w = 0 .. half-1) and `half` draft rows (w = half .. 2*half-1), RS = 2*half
// rows in all. The rows come in B units of RS workgroups: first the T > 0
// sequences (unit u = sequence u), then the greedy sequences' rows as one
// list, all draft rows (top-K: the longest rows) before all target rows
// (argmax: the shortest); within a T > 0 unit the draft rows (softmax and
// top-K, the slowest) come before the target rows. The H bonus workgroups of
// T > 0 sequence v follow row unit v + D, so their draws (which re-read a
// row) overlap later rows, greedy ones included. The greedy sequences' bonus
// workgroups come last: first the last one (h = H-1, the only one with work:
// the greedy bonus is an argmax of published words) of each, then the
// others, which return at once. The launch thus ends on its shortest rows
// and cheapest tasks.
inline SPECV_HD void decode_fused(int64_t g, int64_t B, int64_t nS, int64_t half, int64_t H, int64_t D, int& sidx,
                                  int64_t& w) {
    const int64_t RS = 2 * half;
    const int64_t nG = B - nS;
    if (D > B) D = B;
    const int64_t u2 = D + nS < B ? D + nS : B;       // units D .. u2-1 carry a bonus unit
    const int64_t r1 = D * RS;                          // units 0 .. D-1: rows only
    const int64_t r2 = r1 + (u2 - D) * (RS + H);        // units D .. u2-1: rows, then bonus of u - D
    const int64_t r3 = r2 + (B - u2) * RS;              // units u2 .. B-1: rows only
    const int64_t r4 = r3 + (nS - (u2 - D)) * H;        // bonus of T > 0 sequences u2-D .. nS-1
    int64_t u, o;                                       // row unit and row within it
    if (g < r1) {
        u = g / RS;
        o = g % RS;
    } else if (g < r2) {
        u = D + (g - r1) / (RS + H);
        o = (g - r1) % (RS + H);
        if (o >= RS) {
            sidx = int(u - D);
            w = o;
            return;
        }
    } else if (g < r3) {
        u = u2 + (g - r2) / RS;
        o = (g - r2) % RS;
    } else if (g < r4) {
        sidx = int(u2 - D + (g - r3) / H);
        w = RS + (g - r3) % H;
        return;
    } else {                                            // greedy bonus workgroups: the last of each, then the rest
        const int64_t i = g - r4;
        if (i < nG) {
            sidx = int(nS + i);
            w = RS + H - 1;
        } else {
            sidx = int(nS + (i - nG) % nG);
            w = RS + (i - nG) / nG;
        }
        return;
    }
    if (u < nS) {
        sidx = int(u);
        w = o < half ? o + half : o - half;             // draft rows first
        return;
    }
    const int64_t k = (u - nS) * RS + o;                // index in the greedy row list
    if (k < nG * half) {                                // draft rows
        sidx = int(nS + k / half);
        w = half + k % half;
    } else {                                            // target rows
        sidx = int(nS + (k - nG * half) / half);
        w = (k - nG * half) % half;
    }
}

}  // namespace specv
