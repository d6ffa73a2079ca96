// Fused blockwise-int8 AdamW over a rank's ragged local shard, for gfx950.
//
// veScale-FSDP page, section "Structure-aware training case study": 8-bit
// Adam with a per-parameter block granularity; RaggedShard keeps every
// block inside one rank, so each block is quantised locally and no metadata
// crosses blocks or ranks.  The quantiser (one fp32 absmax per block, m as
// int8 over 127 levels, v as uint8 over 255 levels) and the AdamW constants
// are this library's definition; the pages do not fix them.
//
// One workgroup of 1024 threads handles one chunk of <= 16384 elements;
// each lane owns 16 consecutive elements (four 16-byte fp32 loads, two for
// the bf16 gradient, one each for the int8/uint8 codes).  The new block
// absmax is a wave butterfly (DPP/permute) plus an LDS pass over the 16
// waves; the lane keeps its 16 m and v values in registers until the absmax
// is known, so every byte is read once and written once.  Blocks larger than
// one chunk are split over several workgroups and their absmax is combined
// either by a first launch that writes per-chunk partials (two-pass) or by
// device-scope counters inside one launch (cooperative).
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "raggedshard.h"

namespace rs {

namespace {

enum { MODE_PARTIAL = 0, MODE_MAIN = 1, MODE_COOP = 2 };

// Bounded wait for the other chunks of a block (about 50 ms of sleeps; a
// normal wait is microseconds).  After any timeout every later wait of the
// launch gives up at once, so a failed launch still ends quickly.
constexpr uint32_t kSpinLimit = 1u << 20;

struct StepArgs {
    Ranges r;  // chunk-index ranges; wg0 = prefix counts
    StepBuffers b;
    StepScalars sc;
    int64_t nwg;
};

__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t quant_m(float m, float a) {
    if (a == 0.0f) return 0u;
    float r = rintf((m / a) * 127.0f);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (uint32_t)(int32_t)r & 0xffu;
}

__device__ __forceinline__ uint32_t quant_v(float v, float a) {
    if (a == 0.0f) return 0u;
    float r = rintf((v / a) * 255.0f);
    r = fminf(fmaxf(r, 0.0f), 255.0f);
    return (uint32_t)r;
}

// The AdamW update of one element (binary32, fixed operation order; the
// build disables FMA contraction so products and sums round separately).
struct Elem {
    float m, v, th;
};

__device__ __forceinline__ Elem update(const StepScalars& sc, float theta, float g, float mh,
                                       float vh) {
    Elem e;
    e.m = (sc.beta1 * mh) + (sc.omega1 * g);
    e.v = (sc.beta2 * vh) + (sc.omega2 * (g * g));
    float t = theta * sc.c_decay;
    float den = (sqrtf(e.v) * sc.kappa) + sc.eps;
    e.th = t - (sc.step_size * (e.m / den));
    return e;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
    return x;
}

// Max over the workgroup of (a, b); every thread gets the result.
__device__ __forceinline__ void wg_max2(float& a, float& b, float* red) {
    a = wave_max(a);
    b = wave_max(b);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
        red[2 * wave] = a;
        red[2 * wave + 1] = b;
    }
    __syncthreads();
    float x = 0.0f, y = 0.0f;
    const int nw = blockDim.x >> 6;
    for (int i = 0; i < nw; ++i) {
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

// ------------------------------------------------------------ vector path

template <int MODE>
__device__ void vec_chunk(const ChunkDesc& d, int64_t c, const StepArgs& a, float s,
                          const float* dqm, const float* dqv, float* red) {
    const StepBuffers& B = a.b;
    const StepScalars& sc = a.sc;
    const bool split = d.nparts > 1;
    if (MODE == MODE_PARTIAL && !split) return;
    const int v = threadIdx.x;
    const int vpr = d.cols >> 4;
    const int nvec = d.rows * vpr;
    const bool act = v < nvec;
    int64_t p;
    if (d.rows == 1) {
        p = d.pos + int64_t(v) * kVec;
    } else {
        int row = v / vpr;
        p = d.pos + int64_t(row) * d.ld + int64_t(v - row * vpr) * kVec;
    }
    const bool multi = d.vpb_log2 >= 0;
    const int64_t blk = multi ? d.blk + (v >> d.vpb_log2) : d.blk;

    // old absmax of the block(s)
    float am_old = 0.0f, av_old = 0.0f;
    if (MODE == MODE_MAIN && split) {
        const ChunkPartial cp = B.cpart[c];
        am_old = cp.old_m;
        av_old = cp.old_v;
    } else if (act) {
        am_old = B.amax_m[blk];
        av_old = B.amax_v[blk];
    }

    // final absmax known up front in the second launch of the two-pass mode
    float fin_m = 0.0f, fin_v = 0.0f;
    if (MODE == MODE_MAIN && split) {
        const int64_t c0 = c - d.part;
        for (int q = 0; q < d.nparts; ++q) {
            const ChunkPartial cp = B.cpart[c0 + q];
            fin_m = fmaxf(fin_m, cp.pm);
            fin_v = fmaxf(fin_v, cp.pv);
        }
    }

    float M[kVec], V[kVec];
    float lam = 0.0f, lav = 0.0f;
    if (act) {
        const uint4 g0 = *reinterpret_cast<const uint4*>(B.grad + p);
        const uint4 g1 = *reinterpret_cast<const uint4*>(B.grad + p + 8);
        const uint4 qm = *reinterpret_cast<const uint4*>(B.qm + p);
        const uint4 qv = *reinterpret_cast<const uint4*>(B.qv + p);
        const uint32_t gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
        const uint32_t mw[4] = {qm.x, qm.y, qm.z, qm.w};
        const uint32_t vw[4] = {qv.x, qv.y, qv.z, qv.w};
        float th[kVec];
        if (MODE != MODE_PARTIAL) {
            const float4* tp = reinterpret_cast<const float4*>(B.theta + p);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float4 t = tp[i];
                th[4 * i] = t.x;
                th[4 * i + 1] = t.y;
                th[4 * i + 2] = t.z;
                th[4 * i + 3] = t.w;
            }
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) th[j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            const uint32_t w = gw[j >> 1];
            const float g = ((j & 1) ? bf16_hi(w) : bf16_lo(w)) * s;
            const uint32_t cm = (mw[j >> 2] >> (8 * (j & 3))) & 0xffu;
            const uint32_t cv = (vw[j >> 2] >> (8 * (j & 3))) & 0xffu;
            const float mh = dqm[cm] * am_old;
            const float vh = dqv[cv] * av_old;
            Elem e = update(sc, th[j], g, mh, vh);
            M[j] = e.m;
            V[j] = e.v;
            th[j] = e.th;
            lam = fmaxf(lam, fabsf(e.m));
            lav = fmaxf(lav, e.v);
        }
        if (MODE != MODE_PARTIAL) {
            float4* tp = reinterpret_cast<float4*>(B.theta + p);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                tp[i] = make_float4(th[4 * i], th[4 * i + 1], th[4 * i + 2], th[4 * i + 3]);
            if (B.out) {
                uint32_t o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    o[i] = (uint32_t)f32_to_bf16(th[2 * i]) | ((uint32_t)f32_to_bf16(th[2 * i + 1]) << 16);
                uint4* op = reinterpret_cast<uint4*>(B.out + p);
                op[0] = make_uint4(o[0], o[1], o[2], o[3]);
                op[1] = make_uint4(o[4], o[5], o[6], o[7]);
            }
        }
    }

    // new absmax
    float am, av;
    if (multi) {
        // blocks of (1 << vpb_log2) lanes inside one wave
        am = lam;
        av = lav;
        for (int off = 1; off < (1 << d.vpb_log2); off <<= 1) {
            am = fmaxf(am, __shfl_xor(am, off, 64));
            av = fmaxf(av, __shfl_xor(av, off, 64));
        }
    } else if (MODE == MODE_MAIN && split) {
        am = fin_m;
        av = fin_v;
    } else {
        am = lam;
        av = lav;
        wg_max2(am, av, red);
        if (split) {
            if (MODE == MODE_PARTIAL) {
                if (threadIdx.x == 0) B.cpart[c] = ChunkPartial{am, av, am_old, av_old};
                return;
            }
            // MODE_COOP: meet the other chunks of this block
            if (threadIdx.x == 0) {
                CoopSlot* cs = &B.coop[c - d.part];
                const uint64_t np = (uint64_t)d.nparts;
                const uint64_t a0 = __hip_atomic_load(&cs->arrive, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t gen = a0 / np;
                const int slot = (int)(gen & 1u);
                __hip_atomic_fetch_max(&cs->amax_m[slot], __float_as_uint(am), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_max(&cs->amax_v[slot], __float_as_uint(av), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&cs->amax_m[slot ^ 1], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&cs->amax_v[slot ^ 1], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_fetch_add(&cs->arrive, (uint64_t)1, __ATOMIC_RELEASE,
                                       __HIP_MEMORY_SCOPE_AGENT);
                const uint64_t target = (gen + 1) * np;
                uint32_t spins = 0;
                while (__hip_atomic_load(&cs->arrive, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT) <
                       target) {
                    __builtin_amdgcn_s_sleep(2);
                    ++spins;
                    if ((spins & 255u) == 0 &&
                        __hip_atomic_load(&B.counters->timeout, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT) != 0)
                        break;
                    if (spins > kSpinLimit) {
                        __hip_atomic_fetch_or(&B.counters->timeout, 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                }
                red[0] = __uint_as_float(__hip_atomic_load(&cs->amax_m[slot], __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT));
                red[1] = __uint_as_float(__hip_atomic_load(&cs->amax_v[slot], __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT));
            }
            __syncthreads();
            am = red[0];
            av = red[1];
        }
    }

    if (act) {
        uint32_t qmw[4] = {0, 0, 0, 0}, qvw[4] = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            qmw[j >> 2] |= quant_m(M[j], am) << (8 * (j & 3));
            qvw[j >> 2] |= quant_v(V[j], av) << (8 * (j & 3));
        }
        *reinterpret_cast<uint4*>(B.qm + p) = make_uint4(qmw[0], qmw[1], qmw[2], qmw[3]);
        *reinterpret_cast<uint4*>(B.qv + p) = make_uint4(qvw[0], qvw[1], qvw[2], qvw[3]);
        const bool writer = multi ? ((v & ((1 << d.vpb_log2) - 1)) == 0) : (v == 0 && d.part == 0);
        if (writer) {
            B.amax_m[blk] = am;
            B.amax_v[blk] = av;
        }
    }
}

// --------------------------------------------------- generic block paths

// One whole block of any shape or alignment, two sweeps.
__device__ void scalar_chunk(const ChunkDesc& d, const StepArgs& a, float s, const float* dqm,
                             const float* dqv, float* red) {
    const StepBuffers& B = a.b;
    const int64_t n = int64_t(d.rows) * d.cols;
    const float am_old = B.amax_m[d.blk], av_old = B.amax_v[d.blk];
    float lam = 0.0f, lav = 0.0f;
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const int64_t r = e / d.cols;
        const int64_t p = d.pos + r * d.ld + (e - r * d.cols);
        const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
        const float mh = dqm[uint8_t(B.qm[p])] * am_old;
        const float vh = dqv[B.qv[p]] * av_old;
        Elem el = update(a.sc, 0.0f, g, mh, vh);
        lam = fmaxf(lam, fabsf(el.m));
        lav = fmaxf(lav, el.v);
    }
    wg_max2(lam, lav, red);
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const int64_t r = e / d.cols;
        const int64_t p = d.pos + r * d.ld + (e - r * d.cols);
        const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
        const float mh = dqm[uint8_t(B.qm[p])] * am_old;
        const float vh = dqv[B.qv[p]] * av_old;
        Elem el = update(a.sc, B.theta[p], g, mh, vh);
        B.theta[p] = el.th;
        if (B.out) B.out[p] = f32_to_bf16(el.th);
        B.qm[p] = (int8_t)quant_m(el.m, lam);
        B.qv[p] = (uint8_t)quant_v(el.v, lav);
    }
    if (threadIdx.x == 0) {
        B.amax_m[d.blk] = lam;
        B.amax_v[d.blk] = lav;
    }
}

// A run of single-element blocks.
__device__ void elem_chunk(const ChunkDesc& d, const StepArgs& a, float s, const float* dqm,
                           const float* dqv) {
    const StepBuffers& B = a.b;
    for (int e = threadIdx.x; e < d.cols; e += blockDim.x) {
        const int64_t p = d.pos + e;
        const int64_t blk = d.blk + e;
        const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
        const float mh = dqm[uint8_t(B.qm[p])] * B.amax_m[blk];
        const float vh = dqv[B.qv[p]] * B.amax_v[blk];
        Elem el = update(a.sc, B.theta[p], g, mh, vh);
        B.theta[p] = el.th;
        if (B.out) B.out[p] = f32_to_bf16(el.th);
        const float am = fabsf(el.m), av = el.v;
        B.qm[p] = (int8_t)quant_m(el.m, am);
        B.qv[p] = (uint8_t)quant_v(el.v, av);
        B.amax_m[blk] = am;
        B.amax_v[blk] = av;
    }
}

template <int MODE>
__global__ __launch_bounds__(kStepThreads) void adam8_kernel(StepArgs a) {
    __shared__ float dqm[256], dqv[256];
    __shared__ float red[2 * (kStepThreads / 64)];
    __shared__ int64_t ticket_sh;
    // dequantisation tables: code -> code / 127 (int8), code / 255 (uint8)
    if (threadIdx.x < 256) {
        dqm[threadIdx.x] = (float)(int8_t)(uint8_t)threadIdx.x / 127.0f;
        dqv[threadIdx.x] = (float)threadIdx.x / 255.0f;
    }
    int64_t wg = blockIdx.x;
    if (MODE == MODE_COOP) {
        // chunks are claimed in table order by running workgroups, so a
        // block's missing chunks are always claimable (no wait cycle)
        if (threadIdx.x == 0)
            ticket_sh = (int64_t)__hip_atomic_fetch_add(&a.b.counters->ticket, 1u,
                                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        wg = ticket_sh;
    } else {
        __syncthreads();
    }
    if (wg < a.nwg) {
        const int64_t c = chunk_of(a.r, wg);
        const ChunkDesc d = a.b.chunks[c];
        const float s = a.b.gscale ? *a.b.gscale : 1.0f;
        if (d.kind == KIND_VEC) {
            vec_chunk<MODE>(d, c, a, s, dqm, dqv, red);
        } else if (MODE != MODE_PARTIAL) {
            if (d.kind == KIND_SCALAR)
                scalar_chunk(d, a, s, dqm, dqv, red);
            else
                elem_chunk(d, a, s, dqm, dqv);
        }
    }
    if (MODE == MODE_COOP) {
        __syncthreads();
        if (threadIdx.x == 0) {
            uint32_t prev = __hip_atomic_fetch_add(&a.b.counters->done, 1u, __ATOMIC_ACQ_REL,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            if (prev + 1 == (uint32_t)a.nwg) {
                // last workgroup of the launch: reset for the next one
                __hip_atomic_store(&a.b.counters->ticket, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.b.counters->done, 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

}  // namespace

hipError_t launch_adam8(const Ranges& chunk_ranges, const StepBuffers& b, const StepScalars& sc,
                        int32_t mode, hipStream_t s) {
    StepArgs a;
    a.r = chunk_ranges;
    int64_t total = 0;
    for (int i = 0; i < a.r.n; ++i) {
        a.r.wg0[i] = total;
        total += a.r.hi[i] - a.r.lo[i];
    }
    a.r.wg0[a.r.n] = total;
    a.b = b;
    a.sc = sc;
    a.nwg = total;
    if (total == 0) return hipSuccess;
    if (total > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)total), block(kStepThreads);
    if (mode == RS_SPLIT_COOPERATIVE) {
        hipLaunchKernelGGL(adam8_kernel<MODE_COOP>, grid, block, 0, s, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(adam8_kernel<MODE_PARTIAL>, grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(adam8_kernel<MODE_MAIN>, grid, block, 0, s, a);
    return hipGetLastError();
}

}  // namespace rs
