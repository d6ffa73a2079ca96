// Device helpers shared by the chunked kernels (int8-AdamW step, FP8
// copy-in): launch modes, the lane geometry of vector chunks, streaming
// loads and stores, workgroup reductions, the cooperative per-chunk slots
// of split blocks, and the quantiser's exact quotient.
#pragma once
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "tables.hpp"

namespace rs {
namespace kc {

enum { MODE_PARTIAL = 0, MODE_MAIN = 1, MODE_COOP = 2, MODE_ORDERED = 3 };

// When a one-launch split mode is safe, given the most chunks P of any block
// and the workgroups `capacity` of the kernel the device holds at once.
//
// MODE_ORDERED: chunks are taken from a counter in increasing order, so at
// most P - 1 workgroups can wait on chunks not yet taken (all in the block
// straddling the counter); a device holding more than P workgroups always
// has room for one more.  Asked here with a factor 2 margin, for kernels of
// other streams that may share the device.
inline bool ordered_ok(int64_t P, int64_t capacity) { return capacity >= 2 * P; }

// MODE_COOP: workgroup w takes chunk w.  gfx950 starts the workgroups of a
// launch on its 8 XCDs in turn and in index order on each XCD.  A wait can
// then only stall for good if every workgroup resident on one XCD waits for
// a chunk that XCD has not started; those have indices in (w - P, w) for
// the first such chunk w, at most ceil(P / 8) of them, so an XCD holding
// more than ceil(P / 8) workgroups cannot stall.  Asked here with a factor 2
// margin: capacity / 8 >= 2 ceil(P / 8).  (HIP does not promise this start
// order; RS_SPLIT_ORDERED needs no such promise.)
constexpr int kXcds = 8;
inline bool coop_ok(int64_t P, int64_t capacity) {
    return capacity >= 2 * kXcds * ((P + kXcds - 1) / kXcds) && capacity >= 2 * P;
}


// Bounded wait for the other chunks of a block (tens of ms of sleeps; a
// normal wait is microseconds).  After any timeout every later wait of the
// launch gives up at once, so a failed launch still ends quickly.
constexpr uint32_t kSpinLimit = 1u << 20;

// Reciprocal used by the quantiser: correctly rounded 1/a, 0 for a == 0.
__device__ __forceinline__ float quant_recip(float a) { return a == 0.0f ? 0.0f : 1.0f / a; }

// Blocks whose absmax is below 2^-60 (but not 0) take the plain division.
__device__ __forceinline__ bool quant_slow(float a) { return a < 0x1p-60f && a > 0.0f; }

// m / a by Markstein's correction from y = RN(1/a); correctly rounded for
// every quotient that can give a nonzero code when !quant_slow(a), and 0
// for a == 0 (y = 0, m = 0).
__device__ __forceinline__ float ratio_fast(float m, float a, float y) {
    const float q0 = m * y;
    const float r = __builtin_fmaf(-q0, a, m);
    return __builtin_fmaf(r, y, q0);
}

// OCP E4M3 encoding of the FP8 block rule (copy-in, and the step with FP8
// output): gfx950's conversion rounds to nearest even on the E4M3 grid
// (subnormals included).
// Saturation is explicit: a quotient beyond +-448 (possible only when s is
// a subnormal binary32) is clamped first.
__device__ __forceinline__ float e4m3_sat(float q) { return __builtin_amdgcn_fmed3f(q, -448.0f, 448.0f); }

// Codes of q0..q3 in bytes 0..3.
__device__ __forceinline__ uint32_t e4m3x4(float q0, float q1, float q2, float q3) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(q0), e4m3_sat(q1), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(q2), e4m3_sat(q3), w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint32_t e4m3_code(float q) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_sat(q), 0.0f, 0, false) & 0xffu;
}

// Quotient x / s of the block rule (correctly rounded), y = RN(1 / s).  The
// correction step of ratio_fast returns +0 for x = -0; the sign is x's.
__device__ __forceinline__ float fp8_ratio(float x, float s, float y) {
    return __builtin_copysignf(quant_slow(s) ? x / s : ratio_fast(x, s, y), x);
}

// Code of x in a block of scale s (s >= 0; s == 0 gives code 0).
__device__ __forceinline__ uint32_t fp8_of(float x, float s, float y) {
    return s == 0.0f ? 0u : e4m3_code(fp8_ratio(x, s, y));
}

// Codes of four elements of one block.
__device__ __forceinline__ uint32_t fp8x4_of(const float4& x, float s, float y) {
    if (s == 0.0f) return 0u;
    return e4m3x4(fp8_ratio(x.x, s, y), fp8_ratio(x.y, s, y), fp8_ratio(x.z, s, y),
                  fp8_ratio(x.w, s, y));
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Max over the workgroup of v[0 .. N); every thread gets the result.  red:
// N * (NT / 64) floats of LDS.
template <int NT, int N>
__device__ __forceinline__ void wg_maxn(float (&v)[N], float* red) {
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_max(v[i]);
    if (NT == 64) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) red[N * wave + i] = v[i];
    }
    __syncthreads();
    float x[N];
#pragma unroll
    for (int i = 0; i < N; ++i) x[i] = 0.0f;
#pragma unroll
    for (int w = 0; w < NT / 64; ++w) {
#pragma unroll
        for (int i = 0; i < N; ++i) x[i] = fmaxf(x[i], red[N * w + i]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = x[i];
}

// Max over the workgroup of (a, b); every thread gets the result.
template <int NT>
__device__ __forceinline__ void wg_max2(float& a, float& b, float* red) {
    a = wave_max(a);
    b = wave_max(b);
    if (NT == 64) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[2 * wave] = a;
        red[2 * wave + 1] = b;
    }
    __syncthreads();
    float x = 0.0f, y = 0.0f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) {
        x = fmaxf(x, red[2 * i]);
        y = fmaxf(y, red[2 * i + 1]);
    }
    __syncthreads();
    a = x;
    b = y;
}

__device__ __forceinline__ int64_t chunk_of(const Ranges& r, int64_t wg) {
    int i = 0;
    while (i + 1 < r.n && r.wg0[i + 1] <= wg) ++i;
    return r.lo[i] + (wg - r.wg0[i]);
}

// The chunks of a split block meet through per-chunk slots (PartSlot).  A
// chunk publishes its maxima with relaxed device-scope 64-bit stores, each
// carrying the sequence number of this call next to the value, so a reader
// that sees the new sequence also sees that chunk's value and no ordering
// between the stores or against other memory is needed (an acquire or
// release fence at device scope would write back or invalidate the XCD's
// whole L2).  Device-scope atomics bypass the per-XCD L2, so every XCD sees
// the same words.  One wave of a waiting workgroup polls the slots of all
// chunks of its block with relaxed loads, one chunk per lane, until all
// show the sequence, and reduces their maxima; the other waves wait at a
// barrier, so the polls stay a small share of the memory traffic.  Two
// values travel per chunk in `slots` (the step's m and v maxima; a
// single-value user publishes 0 as the second); a third one (T3: the new
// parameters' maximum of the step with FP8 output) travels in the .m words
// of a second slot array `tslots`.

__device__ __forceinline__ uint32_t coop_seq(const PartSlot* slots, int64_t c) {
    const uint64_t w = __hip_atomic_load(&slots[c].m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return (uint32_t)(w >> 32) + 1u;
}

__device__ __forceinline__ void coop_store(uint64_t* w, uint32_t seq, float x) {
    __hip_atomic_store(w, ((uint64_t)seq << 32) | __float_as_uint(x), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void coop_publish(PartSlot* slots, int64_t c, uint32_t seq, float am,
                                             float av) {
    coop_store(&slots[c].m, seq, am);
    coop_store(&slots[c].v, seq, av);
}

// Run by all lanes of one wave: waits (bounded) until every chunk of the
// block has published `seq`, and returns the block maxima in every lane
// (at only when T3).
template <bool T3>
__device__ __forceinline__ void coop_wait_t(const PartSlot* slots, const PartSlot* tslots,
                                            CoopCounters* counters, int64_t c0, int nparts,
                                            uint32_t seq, float& am, float& av, float& at) {
    const int lane = threadIdx.x & 63;
    uint32_t spins = 0;
    for (;;) {
        bool ok = true;
        float xm = 0.0f, xv = 0.0f, xt = 0.0f;
        for (int q = lane; q < nparts; q += 64) {
            const uint64_t wm =
                __hip_atomic_load(&slots[c0 + q].m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint64_t wv =
                __hip_atomic_load(&slots[c0 + q].v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            ok = ok && (uint32_t)(wm >> 32) == seq && (uint32_t)(wv >> 32) == seq;
            xm = fmaxf(xm, __uint_as_float((uint32_t)wm));
            xv = fmaxf(xv, __uint_as_float((uint32_t)wv));
            if (T3) {
                const uint64_t wt = __hip_atomic_load(&tslots[c0 + q].m, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                ok = ok && (uint32_t)(wt >> 32) == seq;
                xt = fmaxf(xt, __uint_as_float((uint32_t)wt));
            }
        }
        if (__all(ok)) {
            am = wave_max(xm);
            av = wave_max(xv);
            if (T3) at = wave_max(xt);
            return;
        }
        __builtin_amdgcn_s_sleep(1);
        ++spins;
        bool stop = spins > kSpinLimit;
        if (stop && lane == 0)
            __hip_atomic_fetch_or(&counters->timeout, 1u, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        if ((spins & 255u) == 0)
            stop = stop || __hip_atomic_load(&counters->timeout, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT) != 0;
        if (__any(stop)) {
            am = wave_max(xm);
            av = wave_max(xv);
            if (T3) at = wave_max(xt);
            return;
        }
    }
}

__device__ __forceinline__ void coop_wait(const PartSlot* slots, CoopCounters* counters,
                                          int64_t c0, int nparts, uint32_t seq, float& am,
                                          float& av) {
    float unused = 0.0f;
    coop_wait_t<false>(slots, nullptr, counters, c0, nparts, seq, am, av, unused);
}

// The whole workgroup's side of a wait: wave 0 polls, the maxima reach the
// other waves through LDS (bcast: three floats no other code uses
// meanwhile).
template <int NT, bool T3>
__device__ __forceinline__ void coop_wait_wg_t(const PartSlot* slots, const PartSlot* tslots,
                                               CoopCounters* counters, int64_t c0, int nparts,
                                               uint32_t seq, float* bcast, float& am, float& av,
                                               float& at) {
    if (NT == 64) {
        coop_wait_t<T3>(slots, tslots, counters, c0, nparts, seq, am, av, at);
        return;
    }
    if (threadIdx.x < 64) {
        coop_wait_t<T3>(slots, tslots, counters, c0, nparts, seq, am, av, at);
        if (threadIdx.x == 0) {
            bcast[0] = am;
            bcast[1] = av;
            if (T3) bcast[2] = at;
        }
    }
    __syncthreads();
    am = bcast[0];
    av = bcast[1];
    if (T3) at = bcast[2];
}

template <int NT>
__device__ __forceinline__ void coop_wait_wg(const PartSlot* slots, CoopCounters* counters,
                                             int64_t c0, int nparts, uint32_t seq, float* bcast,
                                             float& am, float& av) {
    float unused = 0.0f;
    coop_wait_wg_t<NT, false>(slots, nullptr, counters, c0, nparts, seq, bcast, am, av, unused);
}

// Lane element offsets of a vector chunk relative to d.pos: slice k of this
// lane starts at chunk element e = WSPAN * wave + 256 k + 4 lane, which is
// row e / cols, column e % cols of the chunk.
template <int KG>
__device__ __forceinline__ void lane_offsets(const ChunkDesc& d, uint32_t (&p)[KG],
                                             bool (&act)[KG]) {
    constexpr int WSPAN = 256 * KG;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int n = d.rows * d.cols;
    // row = e / cols via a multiply-high (exact for e, cols < 2^16)
    const uint32_t magic = d.rows > 1 ? (0xffffffffu / (uint32_t)d.cols) + 1u : 0u;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const int e = wave * WSPAN + 256 * k + 4 * lane;
        act[k] = e < n;
        if (d.rows == 1) {
            p[k] = (uint32_t)e;
        } else {
            const uint32_t row = __umulhi((uint32_t)e, magic);
            p[k] = row * (uint32_t)d.ld + ((uint32_t)e - row * (uint32_t)d.cols);
        }
    }
}

// Streaming accesses: every byte of the state is read once and written once
// per step, so loads and stores carry the non-temporal hint.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4 ld_f4(const float* p) {
    const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_float4(__uint_as_float(t.x), __uint_as_float(t.y), __uint_as_float(t.z),
                       __uint_as_float(t.w));
}
__device__ __forceinline__ uint2 ld_u2(const void* p) {
    const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ uint32_t ld_u1(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ void st_f4(float* p, float a, float b, float c, float d) {
    u32x4 t;
    t.x = __float_as_uint(a);
    t.y = __float_as_uint(b);
    t.z = __float_as_uint(c);
    t.w = __float_as_uint(d);
    __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}
__device__ __forceinline__ void st_u2(void* p, uint32_t a, uint32_t b) {
    u32x2 t;
    t.x = a;
    t.y = b;
    __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}
__device__ __forceinline__ void st_u1(void* p, uint32_t a) {
    __builtin_nontemporal_store(a, reinterpret_cast<uint32_t*>(p));
}

}  // namespace kc
}  // namespace rs
