// Device building blocks shared by the verification kernels (gfx950, wave64).
//
// Rows are streamed once from HBM with 16-byte loads; each lane keeps running
// statistics in registers:
//  * SoftmaxAcc: online max and sum of 2^(z*c - mc) with c = log2(e)/T, the
//    normaliser of softmax(z/T) [Lecture 5: Speculative Decoding and
//    SpecInfer, sec. 2.1]. mc is the fp32 product m*c of the running max, and
//    every term is evaluated as exp2(fma(z, c, -mc)), so all terms of a lane
//    share one reference and rescaling is exact up to one rounding.
//  * ArgmaxAcc: the greedy (one-hot) token, lowest index on ties [sec. 2.7].
// (The top-K selection for the SSD bonus candidates is in specv_topk.hpp.)
// Lane results are merged within the wave by xor-shuffles and across the
// workgroup's waves through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace specv {

constexpr int kThreads = 256;               // one workgroup = 4 waves
constexpr int kWaveSize = 64;
constexpr int kWaves = kThreads / kWaveSize;
constexpr int kLaneElems = 8;               // elements per lane per step
constexpr int kTileElems = kWaveSize * kLaneElems;  // residual tile: 512
constexpr int kMaxTiles = 2048;             // vocab <= 2048 * 512
constexpr uint64_t kMaxWaitTicks = uint64_t(1) << 27;   // default wait bound: ~1.3 s at 100 MHz (WaitBound)
// Bound on a chain task's wait for another task's words before it defers
// its sequence to the finisher (~1.3 ms of the 100 MHz clock: far beyond a
// row's streaming time under full load).
constexpr uint64_t kRescueTicks = uint64_t(1) << 17;

enum { DT_F32 = 0, DT_BF16 = 1 };

// ---------------------------------------------------------------- elements

template <int DT> struct ElemT;
template <> struct ElemT<DT_F32> { static constexpr int kBytes = 4; };
template <> struct ElemT<DT_BF16> { static constexpr int kBytes = 2; };

// bf16 -> fp32 is exact (the 16 bits become the high half). It is written as
// a floating-point conversion rather than as bit operations so that the
// compiler knows the results are canonical floats: a max over them then
// needs no NaN-quieting instruction per operand, and chains of max fold into
// three-operand max instructions.
__device__ __forceinline__ float bf16_bits(uint16_t h) { return float(__builtin_bit_cast(__bf16, h)); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return bf16_bits(uint16_t(w)); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return bf16_bits(uint16_t(w >> 16)); }

template <int DT>
__device__ __forceinline__ float load_elem(const void* row, int64_t j) {
    if constexpr (DT == DT_F32) {
        return static_cast<const float*>(row)[j];
    } else {
        return bf16_bits(static_cast<const uint16_t*>(row)[j]);
    }
}

// Raw storage of kLaneElems consecutive elements: one 16-byte word for bf16,
// two for fp32.
template <int DT> struct Raw8 { uint4 w[ElemT<DT>::kBytes / 2]; };

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// Group loads outside the streaming loop (a bonus draw's pass over one or two
// rows, a tile re-read): ordinary loads, which hit when the row is still in
// the device's caches (see kPolicyCached).
template <int DT>
__device__ __forceinline__ void load_raw8(Raw8<DT>& r, const char* p) {
    const u32x4_t* q = reinterpret_cast<const u32x4_t*>(p);
#pragma unroll
    for (int i = 0; i < ElemT<DT>::kBytes / 2; ++i) {
        const u32x4_t x = q[i];
        r.w[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
}

// The streaming loop reads through buffer resources (base and size in scalar
// registers). A load whose offset lies at or past the resource's size returns
// zero without touching memory, so the loop needs no per-lane address
// arithmetic or clamping: each lane keeps one fixed offset, and the scalar
// unit moves the base. Only the per-lane offset is range checked (the scalar
// offset operand is not), hence the base, not that operand, advances.
constexpr int32_t kRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format

// Cache policy of the streaming loads. Most logit rows are read exactly once,
// so they carry the nontemporal hint: on gfx950 that streams at ~6.9 TB/s
// against ~6.0 TB/s for ordinary loads. The rows a bonus draw will probably
// read again (low positions of T > 0 sequences) are streamed with ordinary
// loads instead, so that the second read finds them in the caches.
constexpr int kPolicyStream = 2;             // cache-policy operand: nt
constexpr int kPolicyCached = 0;             // ordinary load

__device__ __forceinline__ __amdgpu_buffer_rsrc_t step_rsrc(const char* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, int32_t(bytes), kRsrcWord3);
}

template <int DT, int kPolicy>
__device__ __forceinline__ void buffer_raw8(Raw8<DT>& r, __amdgpu_buffer_rsrc_t rs, uint32_t voff) {
#pragma unroll
    for (int i = 0; i < ElemT<DT>::kBytes / 2; ++i) {
        const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(rs, int32_t(voff + 16u * i), 0, kPolicy);
        r.w[i] = make_uint4(x.x, x.y, x.z, x.w);
    }
}

// Values the caller guarantees equal across the workgroup, moved to scalar
// registers (the compiler cannot prove it for values read from LDS).
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
    return int64_t((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
    return reinterpret_cast<const char*>(uniform_i64(reinterpret_cast<int64_t>(p)));
}

template <int DT>
__device__ __forceinline__ void unpack8(const Raw8<DT>& r, float v[kLaneElems]) {
    if constexpr (DT == DT_F32) {
        v[0] = __uint_as_float(r.w[0].x); v[1] = __uint_as_float(r.w[0].y);
        v[2] = __uint_as_float(r.w[0].z); v[3] = __uint_as_float(r.w[0].w);
        v[4] = __uint_as_float(r.w[1].x); v[5] = __uint_as_float(r.w[1].y);
        v[6] = __uint_as_float(r.w[1].z); v[7] = __uint_as_float(r.w[1].w);
    } else {
        v[0] = bf16_lo(r.w[0].x); v[1] = bf16_hi(r.w[0].x);
        v[2] = bf16_lo(r.w[0].y); v[3] = bf16_hi(r.w[0].y);
        v[4] = bf16_lo(r.w[0].z); v[5] = bf16_hi(r.w[0].z);
        v[6] = bf16_lo(r.w[0].w); v[7] = bf16_hi(r.w[0].w);
    }
}

// Three-operand max as one instruction. Written out because the compiler,
// given a max over widened bf16 values whose only use is more max and
// compares, narrows it to bf16 and converts every intermediate back and forth
// (three instructions per max). Logits are never NaN (the interface requires
// it), so the IEEE-mode NaN rules of the instruction do not matter.
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ __forceinline__ float max8(const float v[kLaneElems]) {
    const float a = max3f(v[0], v[1], v[2]);
    const float b = max3f(v[3], v[4], v[5]);
    return max3f(max3f(a, v[6], v[7]), b, b);
}

// Maximum over U groups' maxima.
template <int U>
__device__ __forceinline__ float max_of(const float (&m)[U]) {
    float r = m[0];
    int u = 1;
#pragma unroll
    for (; u + 1 < U; u += 2) r = max3f(r, m[u], m[u + 1]);
    if (u < U) r = max3f(r, m[u], m[u]);
    return r;
}

// ------------------------------------------------------------- streaming
//
// Visits elements [lo, hi) of `row`. When the chunk start is 16-byte aligned
// the body is read in steps of kLaneElems elements per lane, U steps per lane
// per iteration (lane t takes steps t, t + kThreads, ...), and the remainder
// element by element; otherwise every element is read singly. Both loop
// bounds are uniform over the workgroup, so every lane calls the visitor's
// block() and one() on every iteration (visitors may use wave-wide
// operations); steps or elements past the end arrive as -inf with
// valid = false.
//
// Software pipelined through a ring of D buffers of U steps: while iteration
// i is processed, the loads of iterations i + 1 .. i + D - 1 are in flight,
// so D * U 16-byte loads per lane overlap the arithmetic while only U steps
// are unpacked at a time. Every load in the loop is issued unconditionally
// (a load under a per-lane or per-iteration branch makes the compiler wait
// for every outstanding load before the processing, which would serialise
// the ring); refills past the last iteration read zeros and are never visited.
// Per-lane validity is tested only in the last iteration.
template <int DT, int U, class Acc>
__device__ __forceinline__ void visit_steps(const Raw8<DT> (&r)[U], int64_t lo, int64_t s0, int64_t nstep,
                                            bool full, Acc& acc) {
    float v[U][kLaneElems];
    int64_t idx[U];
    bool valid[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t s = s0 + threadIdx.x + int64_t(u) * kThreads;
        valid[u] = full || s < nstep;
        idx[u] = lo + s * kLaneElems;
        unpack8<DT>(r[u], v[u]);
        if (!valid[u]) {
#pragma unroll
            for (int e = 0; e < kLaneElems; ++e) v[u][e] = -INFINITY;
        }
    }
    acc.template block<U>(v, idx, valid);
}

template <int DT, int U, int D, int kPolicy = kPolicyStream, class Acc>
__device__ __forceinline__ void stream_chunk(const void* row, int64_t lo, int64_t hi, Acc& acc) {
    static_assert(U >= 1 && D >= 0, "U >= 1 steps per iteration; D = 0 (prefetch) or a ring of D >= 1");
    constexpr int kB = ElemT<DT>::kBytes;
    constexpr int64_t kStride = int64_t(kThreads) * U;
    constexpr uint32_t kStepBytes = kLaneElems * kB;
    lo = uniform_i64(lo);
    hi = uniform_i64(hi);
    const char* base = uniform_ptr(static_cast<const char*>(row) + lo * kB);
    const int64_t n = hi - lo;
    const bool aligned = (reinterpret_cast<uintptr_t>(base) & 15u) == 0;
    const int64_t nstep = aligned ? n / kLaneElems : 0;
    const int64_t nit = (nstep + kStride - 1) / kStride;
    // Steps are read through a resource over the whole steps of the chunk
    // (fewer than 2^32 bytes: rows hold at most kMaxTiles * kTileElems
    // elements); steps past the end read as zero and are never visited.
    // (The remaining size is a signed max, which the scalar unit has; an
    // unsigned saturating subtract would be computed per lane and force a
    // loop over lanes around every load.)
    const int32_t total = int32_t(nstep) * int32_t(kStepBytes);
    const uint32_t voff = threadIdx.x * kStepBytes;
    auto load_it = [&](Raw8<DT> (&r)[U], int64_t it) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int32_t start = int32_t(it * kStride + int64_t(u) * kThreads) * int32_t(kStepBytes);
            buffer_raw8<DT, kPolicy>(r[u], step_rsrc(base + start, uint32_t(max(total - start, 0))), voff);
        }
    };

    if constexpr (D == 0) {
        // Prefetch form: one buffer in flight, issued before the current
        // iteration is processed and moved into place after it (fewer live
        // registers than a ring of two when the visitor is heavy).
        if (nstep > 0) {
            const int64_t nfull = nstep - nstep % kStride;
            Raw8<DT> cur[U];
            load_it(cur, 0);
            int64_t base0 = 0;
            for (; base0 < nfull; base0 += kStride) {
                Raw8<DT> nxt[U];
                load_it(nxt, base0 / kStride + 1);
                visit_steps<DT, U>(cur, lo, base0, nstep, true, acc);
#pragma unroll
                for (int u = 0; u < U; ++u) cur[u] = nxt[u];
            }
            if (base0 < nstep) visit_steps<DT, U>(cur, lo, base0, nstep, false, acc);
        }
    } else if (nstep > 0) {
        Raw8<DT> ring[D][U];
#pragma unroll
        for (int d = 0; d < D; ++d) load_it(ring[d], d);
        int64_t it0 = 0;
        for (; it0 + D <= nit; it0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                visit_steps<DT, U>(ring[d], lo, (it0 + d) * kStride, nstep, it0 + d + 1 < nit, acc);
                load_it(ring[d], it0 + D + d);
            }
        }
        // Drain: iterations it0 .. nit - 1 (fewer than D) are in the ring.
#pragma unroll
        for (int d = 0; d + 1 < D; ++d) {
            if (it0 + d < nit) visit_steps<DT, U>(ring[d], lo, (it0 + d) * kStride, nstep, false, acc);
        }
    }
    for (int64_t j0 = nstep * kLaneElems; j0 < n; j0 += kThreads) {
        const int64_t j = j0 + threadIdx.x;
        const bool ok = j < n;
        acc.one(ok ? load_elem<DT>(row, lo + j) : -INFINITY, lo + j, ok);
    }
}

// stream_chunk with the cache policy chosen at run time (cached: ordinary
// loads, for rows that will probably be read again).
template <int DT, int U, int D, class Acc>
__device__ __forceinline__ void stream_chunk_as(bool cached, const void* row, int64_t lo, int64_t hi, Acc& acc) {
    if (cached) stream_chunk<DT, U, D, kPolicyCached>(row, lo, hi, acc);
    else stream_chunk<DT, U, D, kPolicyStream>(row, lo, hi, acc);
}

// ------------------------------------------------------------------ Philox
//
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): ten rounds of two
// 32x32->64-bit products, key bumped by the Weyl constants between rounds.

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        if (r > 0) { k0 += 0x9E3779B9u; k1 += 0xBB67AE85u; }
        const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
        const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
    }
    return c;
}

// U(seed, offset, b, tag, j) in (0, 1]: word j & 3 of the block at counter
// (offset lo, offset hi, b, tag << 24 | j >> 2), top 24 bits plus one, / 2^24.
__device__ __forceinline__ float stream_uniform(uint64_t seed, uint64_t offset, uint32_t b,
                                                uint32_t tag, uint32_t j) {
    const uint4 o = philox4x32_10(
        make_uint4(uint32_t(offset), uint32_t(offset >> 32), b, (tag << 24) | (j >> 2)),
        uint32_t(seed), uint32_t(seed >> 32));
    const uint32_t w = (j & 3) == 0 ? o.x : (j & 3) == 1 ? o.y : (j & 3) == 2 ? o.z : o.w;
    return float((w >> 8) + 1u) * 5.9604644775390625e-08f;  // 2^-24
}

// ---------------------------------------------------------- reductions

// A chunk's statistics are one 64-bit value (published as a tagged pair,
// below); the reader recomputes mc = fp32(m * c):
//   softmax: hi = bits(max logit m), lo = ~bits(fp32 s), s = sum 2^(z*c - mc)
//            relative to mc;
//   greedy:  hi = bits(best logit),  lo = ~uint32(index), index >= 0;
//   skipped row (nothing read): hi = bits(-inf), lo = ~bits(0.0f).
__device__ __forceinline__ uint64_t pack_slot(float hi, uint32_t lo) {
    return (uint64_t(__float_as_uint(hi)) << 32) | uint64_t(lo);
}
__device__ __forceinline__ uint64_t pack_softmax(float m, double s) { return pack_slot(m, ~__float_as_uint(float(s))); }
__device__ __forceinline__ uint64_t pack_argmax(float v, int32_t idx) { return pack_slot(v, ~uint32_t(idx)); }
__device__ __forceinline__ uint64_t pack_skipped() { return pack_slot(-INFINITY, ~__float_as_uint(0.0f)); }
__device__ __forceinline__ float slot_hi(uint64_t w) { return __uint_as_float(uint32_t(w >> 32)); }
__device__ __forceinline__ float slot_s(uint64_t w) { return __uint_as_float(~uint32_t(w)); }
__device__ __forceinline__ int32_t slot_idx(uint64_t w) { return int32_t(~uint32_t(w)); }
__device__ __forceinline__ uint64_t pack_f64(double x) { return uint64_t(__double_as_longlong(x)); }
__device__ __forceinline__ double unpack_f64(uint64_t w) { return __longlong_as_double(int64_t(w)); }

// ------------------------------------------------------ published values
//
// Workgroups of one launch exchange 64-bit values through the workspace. A
// value is published as a pair of 64-bit words, each holding a 32-bit tag in
// its high half and one half of the value in its low half, written with
// agent-scope relaxed atomic stores: each word is single-copy atomic, so a
// reader that sees the tag in both words has the whole value, and no fence
// is needed (on gfx950 an agent-scope release fence is an L2 write-back).
// The tag is the call's epoch (nonzero, a new one for every call), or for the
// tree walkers' pass totals the epoch and the pass number, so a zero word or
// a word left by another call or pass never reads as published. Consumed
// words are returned to zero (the workspace's resting state).
__device__ __forceinline__ void publish_pair(uint64_t* p, uint64_t v, uint32_t tag) {
    const uint64_t t = uint64_t(tag) << 32;
    __hip_atomic_store(p, t | (v >> 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p + 1, t | (v & 0xffffffffull), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t peek(const uint64_t* w) {
    return __hip_atomic_load(const_cast<uint64_t*>(w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void clear_word(uint64_t* w) {
    __hip_atomic_store(w, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool pair_ok(uint64_t hi, uint64_t lo, uint32_t tag) {
    return uint32_t(hi >> 32) == tag && uint32_t(lo >> 32) == tag;
}
__device__ __forceinline__ uint64_t pair_value(uint64_t hi, uint64_t lo) { return (hi << 32) | (lo & 0xffffffffull); }
// The value of pair i (both words loaded now; the caller knows it is there).
__device__ __forceinline__ uint64_t read_pair(const uint64_t* p, int64_t i) {
    return pair_value(peek(p + 2 * i), peek(p + 2 * i + 1));
}

// a += b for softmax partials (both relative to their own mc).
__device__ __forceinline__ void merge_softmax(float& m, float& mc, double& s,
                                              float bm, float bmc, double bs) {
    if (bm == -INFINITY) return;
    if (m == -INFINITY) { m = bm; mc = bmc; s = bs; return; }
    if (bm > m) {
        s = s * exp2(double(mc) - double(bmc)) + bs;
        m = bm; mc = bmc;
    } else {
        s += bs * exp2(double(bmc) - double(mc));
    }
}

// Greedy order: larger value first, then lower index.
// (v, i) beats (bv, bi); an index < 0 marks "no element".
__device__ __forceinline__ bool argmax_better(float v, int32_t i, float bv, int32_t bi) {
    if (i < 0) return false;
    if (bi < 0) return true;
    return v > bv || (v == bv && i < bi);
}

__device__ __forceinline__ void wave_merge_softmax(float& m, float& mc, double& s) {
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
        const float om = __shfl_xor(m, o);
        const float omc = __shfl_xor(mc, o);
        const double os = __shfl_xor(s, o);
        merge_softmax(m, mc, s, om, omc, os);
    }
}

__device__ __forceinline__ void wave_merge_argmax(float& v, int32_t& i) {
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
        const float ov = __shfl_xor(v, o);
        const int32_t oi = __shfl_xor(i, o);
        if (argmax_better(ov, oi, v, i)) { v = ov; i = oi; }
    }
}

// Wave sums through DPP row moves (no LDS round trip per step): pairs within
// quads, then half-row and row mirrors give every lane its 16-lane row sum;
// two row broadcasts (lane 15 into rows 1 and 3, lane 31 into rows 2 and 3)
// leave the total in lane 63, which is returned to every lane. Disabled rows
// of a broadcast add 0.
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), kCtrl, kRowMask, 0xf, false));
}
constexpr int kDppQuadXor1 = 0xB1, kDppQuadXor2 = 0x4E, kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140,
              kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ float dpp_f32(float v) { return __uint_as_float(dpp_u32<kCtrl, kRowMask>(__float_as_uint(v))); }

template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t u = uint64_t(__double_as_longlong(v));
    const uint32_t lo = dpp_u32<kCtrl, kRowMask>(uint32_t(u));
    const uint32_t hi = dpp_u32<kCtrl, kRowMask>(uint32_t(u >> 32));
    return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}

__device__ __forceinline__ float wave_sum(float x) {
    x += dpp_f32<kDppQuadXor1>(x);
    x += dpp_f32<kDppQuadXor2>(x);
    x += dpp_f32<kDppRowHalfMirror>(x);
    x += dpp_f32<kDppRowMirror>(x);
    x += dpp_f32<kDppRowBcast15, 0xa>(x);
    x += dpp_f32<kDppRowBcast31, 0xc>(x);
    return __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(x)), kWaveSize - 1)));
}

__device__ __forceinline__ double wave_sum(double x) {
    x += dpp_f64<kDppQuadXor1>(x);
    x += dpp_f64<kDppQuadXor2>(x);
    x += dpp_f64<kDppRowHalfMirror>(x);
    x += dpp_f64<kDppRowMirror>(x);
    x += dpp_f64<kDppRowBcast15, 0xa>(x);
    x += dpp_f64<kDppRowBcast31, 0xc>(x);
    const uint64_t u = uint64_t(__double_as_longlong(x));
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u)), kWaveSize - 1));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(u >> 32)), kWaveSize - 1));
    return __longlong_as_double(int64_t((uint64_t(hi) << 32) | lo));
}

// Inclusive prefix sum across the wave (lane order).
__device__ __forceinline__ double wave_inclusive_scan(double x) {
    const int lane = threadIdx.x & (kWaveSize - 1);
#pragma unroll
    for (int o = 1; o < kWaveSize; o <<= 1) {
        const double y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    return x;
}

// Number of lanes below this one whose bit is set in m.
__device__ __forceinline__ int lanes_below(uint64_t m) {
    return int(__builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u)));
}

// Wave maximum of unsigned 64-bit values through the same DPP steps as
// wave_sum (disabled rows of a broadcast see 0, which never wins).
template <int kCtrl, int kRowMask = 0xf>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const uint32_t lo = dpp_u32<kCtrl, kRowMask>(uint32_t(v));
    const uint32_t hi = dpp_u32<kCtrl, kRowMask>(uint32_t(v >> 32));
    return (uint64_t(hi) << 32) | lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
    x = umax64(x, dpp_u64<kDppQuadXor1>(x));
    x = umax64(x, dpp_u64<kDppQuadXor2>(x));
    x = umax64(x, dpp_u64<kDppRowHalfMirror>(x));
    x = umax64(x, dpp_u64<kDppRowMirror>(x));
    x = umax64(x, dpp_u64<kDppRowBcast15, 0xa>(x));
    x = umax64(x, dpp_u64<kDppRowBcast31, 0xc>(x));
    const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x)), kWaveSize - 1));
    const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(x >> 32)), kWaveSize - 1));
    return (uint64_t(hi) << 32) | lo;
}

// ------------------------------------------------------------ accumulators

// Online softmax statistics of one lane. c = log2(e)/T as fp32.
struct SoftmaxAcc {
    float c;
    float m = -INFINITY;
    float mc = -INFINITY;
    double s = 0.0;

    __device__ explicit SoftmaxAcc(float c_) : c(c_) {}

    __device__ __forceinline__ void rebase(float cm) {
        if (cm > m) {
            const float mcn = cm * c;
            s = (m == -INFINITY) ? 0.0 : s * double(__builtin_amdgcn_exp2f(mc - mcn));
            m = cm;
            mc = mcn;
        }
    }

    template <int U>
    __device__ __forceinline__ void block(const float (&v)[U][kLaneElems], const int64_t*, const bool*) {
        float gm[U];
#pragma unroll
        for (int u = 0; u < U; ++u) gm[u] = max8(v[u]);
        const float cm = max_of<U>(gm);
        rebase(cm);
        const float nmc = (m == -INFINITY) ? 0.0f : -mc;
        float part[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float t[kLaneElems];
#pragma unroll
            for (int e = 0; e < kLaneElems; ++e) t[e] = __builtin_amdgcn_exp2f(fmaf(v[u][e], c, nmc));
            part[u] = ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
        }
        float tot = part[0];
#pragma unroll
        for (int u = 1; u < U; ++u) tot += part[u];
        s += double(tot);
    }

    __device__ __forceinline__ void one(float z, int64_t, bool ok) {
        if (!ok) return;
        rebase(z);
        if (m != -INFINITY) s += double(__builtin_amdgcn_exp2f(fmaf(z, c, -mc)));
    }
};

// Greedy argmax of one lane: lanes see their elements in increasing index
// order, so a strict comparison keeps the lowest index.
struct ArgmaxAcc {
    float best = -INFINITY;
    int32_t idx = -1;

    template <int U>
    __device__ __forceinline__ void block(const float (&v)[U][kLaneElems], const int64_t* base, const bool* valid) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float vm = max8(v[u]);
            if (valid[u] && (vm > best || idx < 0)) {
                int e = kLaneElems - 1;
#pragma unroll
                for (int k = kLaneElems - 2; k >= 0; --k) e = (v[u][k] == vm) ? k : e;
                best = vm;
                idx = int32_t(base[u] + e);
            }
        }
    }

    __device__ __forceinline__ void one(float z, int64_t j, bool ok) {
        if (ok && (z > best || idx < 0)) { best = z; idx = int32_t(j); }
    }
};

// Order-preserving 32-bit key of a logit (-0 mapped to +0): larger logit,
// larger key. Full 64-bit key = (logit key << 32) | ~index, so equal logits
// order by lower index first.
__device__ __forceinline__ uint32_t logit_key(float v) {
    uint32_t u = __float_as_uint(v);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint64_t full_key(float v, int64_t j) {
    return (uint64_t(logit_key(v)) << 32) | uint64_t(~uint32_t(j));
}

}  // namespace specv
