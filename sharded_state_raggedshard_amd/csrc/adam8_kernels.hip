// Fused blockwise-int8 AdamW over a rank's ragged local shard, for gfx950.
//
// veScale-FSDP page, section "Structure-aware training case study": 8-bit
// Adam with a per-parameter block granularity; RaggedShard keeps every
// block inside one rank, so each block is quantised locally and no metadata
// crosses blocks or ranks.  The quantiser (one fp32 absmax per block, m as
// int8 over 127 levels, v as uint8 over 255 levels) and the AdamW constants
// are this library's definition; the pages do not fix them.
//
// One workgroup handles one chunk.  A lane owns 4 KG elements (KG = 4):
// wave w of the workgroup covers chunk
// elements [256 KG w, 256 KG (w + 1)) as KG 256-element slices, and lane l
// owns elements 256 k + 4 l .. +3 of slice k, so each load and store
// instruction of a wave touches one contiguous span (1 KiB of fp32, 512 B of
// bf16, 256 B of codes).  The lane keeps its new m and v values in registers
// until the block absmax is known (wave butterfly, then LDS across waves), so
// every byte is read once and written once.
//
// Arithmetic: the moments m, v follow the fixed binary32 order of the
// definition with no FMA contraction, so they match a correctly rounded
// evaluation bit for bit.  The parameter update uses the hardware square
// root and reciprocal and falls back to correctly rounded operations where
// that could leave the parameter tolerance (see param_fast); the scalar and
// element paths use the correctly rounded operations throughout.
// The quantisation ratio m / absmax is the correctly rounded quotient too,
// formed from the block's correctly rounded reciprocal y and one residual
// step q = q0 + (m - q0*a)*y with q0 = m*y (Markstein's correction): exact
// for every quotient that can reach a nonzero code once absmax >= 2^-60;
// smaller absmax values take the plain division.
//
// Blocks larger than one chunk are split over several workgroups; their
// absmax is combined either by a first launch that writes per-chunk partials
// (two-pass) or inside one launch (cooperative): every chunk publishes its
// maxima into its own slot, tagged with a per-call sequence number, and every
// wave then polls the slots of its block (see adam8_kernel for why the waits
// end).  Each wait is bounded all the same and reports a timeout through the
// device status word if it ever gives up.
//
// FP8 output (the step followed by the FP8 copy-in of the new parameters,
// in one pass): the new parameters are formed before the block maxima are
// exchanged, their block absmax travels with those of m and v, and after
// the wait the lane encodes its parameters, still in registers, as E4M3
// codes of the block scale absmax / 448.  The copy-in's extra read of the
// parameters and its own wait disappear; one byte per element is added.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "raggedshard.h"

namespace rs {

namespace {

using namespace kc;

struct StepArgs {
    Ranges r;  // chunk-index ranges; wg0 = prefix counts
    StepBuffers b;
    StepScalars sc;
    int64_t nwg;  // chunks of the launch (linear indices 0 .. nwg - 1)
};

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Correctly rounded m / a (see the file comment); a >= 0, y = quant_recip(a).
__device__ __forceinline__ float ratio(float m, float a, float y) {
    if (quant_slow(a)) return m / a;
    return ratio_fast(m, a, y);
}

__device__ __forceinline__ uint32_t code_m(float m, float a, float y) {
    float c = rintf(ratio(m, a, y) * 127.0f);
    c = fminf(fmaxf(c, -127.0f), 127.0f);
    return (uint32_t)(int32_t)c & 0xffu;
}

__device__ __forceinline__ uint32_t code_v(float v, float a, float y) {
    float c = rintf(ratio(v, a, y) * 255.0f);
    c = fminf(fmaxf(c, 0.0f), 255.0f);
    return (uint32_t)c;
}

struct Elem {
    float m, v, th;
};

// One element of AdamW in the fixed binary32 order of the definition.
__device__ __forceinline__ Elem update(const StepScalars& sc, float theta, float g, float mh,
                                       float vh) {
    Elem e;
    e.m = (sc.beta1 * mh) + (sc.omega1 * g);
    e.v = (sc.beta2 * vh) + (sc.omega2 * (g * g));
    const float den = (sqrtf(e.v) * sc.kappa) + sc.eps;
    e.th = (theta * sc.c_decay) - (sc.step_size * (e.m / den));
    return e;
}

// Moments of one element (definition order, binary32).
__device__ __forceinline__ void moments(const StepScalars& sc, float g, float mh, float vh,
                                        float& m, float& v) {
    m = (sc.beta1 * mh) + (sc.omega1 * g);
    v = (sc.beta2 * vh) + (sc.omega2 * (g * g));
}

__device__ __forceinline__ float param(const StepScalars& sc, float theta, float m, float sq) {
    const float den = (sq * sc.kappa) + sc.eps;
    return (theta * sc.c_decay) - (sc.step_size * (m / den));
}

// The parameter update with the hardware square root and reciprocal (each
// within 1 ulp): the update u then carries a relative error below 8 ulp
// (4.8e-7) against the correctly rounded evaluation, so for |u| <= 0.02 the
// new parameter differs by at most 9.6e-9 plus one rounding of the result,
// inside |d| <= 1e-8 + 1e-6 |theta|.  Any other u (larger, infinite or NaN)
// sets `exact` and the caller recomputes with correctly rounded operations.
// No quantisation code depends on the parameter.
__device__ __forceinline__ float param_fast(const StepScalars& sc, float theta, float m, float v,
                                            bool& exact) {
    const float den = (__builtin_amdgcn_sqrtf(v) * sc.kappa) + sc.eps;
    const float u = sc.step_size * (m * __builtin_amdgcn_rcpf(den));
    exact = exact || !(fabsf(u) <= 0.02f);
    return (theta * sc.c_decay) - u;
}

// ------------------------------------------------------------ vector path

// What a lane reads of one vector chunk: master, gradient and codes of its
// 4 KG elements and the old absmax of the block(s) they belong to.
template <int KG>
struct VecIn {
    float4 TH[KG];
    uint2 GW[KG];
    uint32_t CM[KG], CV[KG];
    float amo[KG], avo[KG];
};

// Issues every load of a vector chunk.  Tile chunks keep rows * ld < 2^30,
// so a uniform chunk base plus 32-bit lane offsets addresses every element.
template <int MODE, int KG, bool F8>
__device__ __forceinline__ void vec_load(const ChunkDesc& d, int64_t c, const StepBuffers& B,
                                         VecIn<KG>& in) {
    constexpr int WSPAN = 256 * KG;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t p[KG];
    bool act[KG];
    lane_offsets<KG>(d, p, act);
    const bool split = d.nparts > 1;
    if (MODE == MODE_MAIN && split) {
        const ChunkPartial cp = B.cpart[c];
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            in.amo[k] = cp.old_m;
            in.avo[k] = cp.old_v;
        }
    } else if (d.run_log2 >= 0) {
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            const int64_t blk = d.blk + ((wave * WSPAN + 256 * k + 4 * lane) >> d.run_log2);
            in.amo[k] = act[k] ? B.amax_m[blk] : 0.0f;
            in.avo[k] = act[k] ? B.amax_v[blk] : 0.0f;
        }
    } else {
        const float x = B.amax_m[d.blk], y = B.amax_v[d.blk];
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            in.amo[k] = x;
            in.avo[k] = y;
        }
    }
    const float* th_b = B.theta + d.pos;
    const uint16_t* g_b = B.grad + d.pos;
    const int8_t* qm_b = B.qm + d.pos;
    const uint8_t* qv_b = B.qv + d.pos;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        uint2 gw = make_uint2(0u, 0u);
        uint32_t cm = 0u, cv = 0u;
        float4 th = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (act[k]) {
            gw = ld_u2(g_b + p[k]);
            cm = ld_u1(qm_b + p[k]);
            cv = ld_u1(qv_b + p[k]);
            if (MODE != MODE_PARTIAL || F8) th = ld_f4(th_b + p[k]);
        }
        in.GW[k] = gw;
        in.CM[k] = cm;
        in.CV[k] = cv;
        in.TH[k] = th;
    }
}

// What the phases of one vector chunk carry between them.
template <int KG>
struct VecState {
    float M[4 * KG], V[4 * KG];  // new moments of this lane's elements
    float T[4 * KG];             // new parameters (FP8 output only)
    float am[KG], av[KG];        // new absmax of the block(s) of each slice
    float at[KG];                // new parameters' absmax (FP8 output only)
    uint32_t seq;                // sequence number published (cooperative split)
    bool wait;                   // the block's other chunks must be waited for
};

// New parameters of four elements (one slice of a lane): the hardware square
// root and reciprocal, or correctly rounded operations where param_fast asks
// for them.
__device__ __forceinline__ void new_params(const StepScalars& sc, const float4& th,
                                           const float* M, const float* V, float (&t)[4]) {
    const float t0[4] = {th.x, th.y, th.z, th.w};
    bool exact = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) t[j] = param_fast(sc, t0[j], M[j], V[j], exact);
    if (__builtin_expect(exact, 0)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) t[j] = param(sc, t0[j], M[j], sqrtf(V[j]));
    }
}

// Front: moments and the new block maxima; a cooperative split chunk
// publishes its maxima.  With FP8 output (F8) the new parameters and their
// block maximum are formed here too, so they travel with the moments'
// maxima in the same wait.  Returns false when nothing is left to do (the
// partial pass of a split chunk).
template <int MODE, int NT, int KG, bool F8>
__device__ __forceinline__ bool vec_front(const ChunkDesc& d, int64_t c, const StepArgs& a,
                                          float s, const float* dqm, const float* dqv,
                                          float* red, const VecIn<KG>& in, VecState<KG>& st) {
    const StepBuffers& B = a.b;
    const StepScalars& sc = a.sc;
    const bool split = d.nparts > 1;
    // Sequence number this call publishes (cooperative split blocks): thread
    // 0 reads it before the workgroup max's barriers and every thread takes
    // it from LDS after them, so no thread can read the slot after thread 0
    // has published into it.
    uint32_t* seq_lds = reinterpret_cast<uint32_t*>(red + (F8 ? 3 : 2) * (NT / 64));
    if (MODE == MODE_COOP && split && d.run_log2 < 0 && threadIdx.x == 0)
        *seq_lds = coop_seq(B.coop, c);
    st.seq = 0u;
    st.wait = false;
    float lm[KG], lv[KG], lt[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) lm[k] = lv[k] = lt[k] = 0.0f;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        const float g[4] = {bf16_lo(in.GW[k].x) * s, bf16_hi(in.GW[k].x) * s,
                            bf16_lo(in.GW[k].y) * s, bf16_hi(in.GW[k].y) * s};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float mh = dqm[(in.CM[k] >> (8 * j)) & 0xffu] * in.amo[k];
            const float vh = dqv[(in.CV[k] >> (8 * j)) & 0xffu] * in.avo[k];
            moments(sc, g[j], mh, vh, st.M[4 * k + j], st.V[4 * k + j]);
            lm[k] = fmaxf(lm[k], fabsf(st.M[4 * k + j]));
            lv[k] = fmaxf(lv[k], st.V[4 * k + j]);
        }
    }
    if (F8) {
        uint32_t p[KG];
        bool act[KG];
        lane_offsets<KG>(d, p, act);
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            float t[4];
            new_params(sc, in.TH[k], st.M + 4 * k, st.V + 4 * k, t);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                st.T[4 * k + j] = t[j];
                if (act[k]) lt[k] = fmaxf(lt[k], fabsf(t[j]));
            }
        }
    }
    if (d.run_log2 >= 0) {
        // blocks of (1 << run_log2) elements = (1 << run_log2) / 4 lanes of one slice
        const int lanes = (1 << d.run_log2) >> 2;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            st.am[k] = lm[k];
            st.av[k] = lv[k];
            st.at[k] = lt[k];
            for (int off = 1; off < lanes; off <<= 1) {
                st.am[k] = fmaxf(st.am[k], __shfl_xor(st.am[k], off, 64));
                st.av[k] = fmaxf(st.av[k], __shfl_xor(st.av[k], off, 64));
                if (F8) st.at[k] = fmaxf(st.at[k], __shfl_xor(st.at[k], off, 64));
            }
        }
        return true;
    }
    float x, y, t = 0.0f;
    if (MODE == MODE_MAIN && split) {
        x = 0.0f;
        y = 0.0f;
        const int64_t c0 = c - d.part;
        for (int q = 0; q < d.nparts; ++q) {
            const ChunkPartial cp = B.cpart[c0 + q];
            x = fmaxf(x, cp.pm);
            y = fmaxf(y, cp.pv);
            if (F8) t = fmaxf(t, B.cpart_t[c0 + q]);
        }
    } else {
        x = lm[0];
        y = lv[0];
        t = lt[0];
#pragma unroll
        for (int k = 1; k < KG; ++k) {
            x = fmaxf(x, lm[k]);
            y = fmaxf(y, lv[k]);
            if (F8) t = fmaxf(t, lt[k]);
        }
        if (F8) {
            float v[3] = {x, y, t};
            wg_maxn<NT, 3>(v, red);
            x = v[0];
            y = v[1];
            t = v[2];
        } else {
            wg_max2<NT>(x, y, red);
        }
        if (split) {
            if (MODE == MODE_PARTIAL) {
                if (threadIdx.x == 0) {
                    B.cpart[c] = ChunkPartial{x, y, in.amo[0], in.avo[0]};
                    if (F8) B.cpart_t[c] = t;
                }
                return false;
            }
            st.seq = *seq_lds;  // written before the workgroup max's barriers
            st.wait = true;
            if (threadIdx.x == 0) {
                coop_publish(B.coop, c, st.seq, x, y);
                if (F8) coop_store(&B.coop_t[c].m, st.seq, t);
            }
        }
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        st.am[k] = x;
        st.av[k] = y;
        st.at[k] = t;
    }
    return true;
}

// Parameters: needs no absmax, so it runs before any wait (with FP8 output
// they were formed in the front).
template <int KG, bool F8>
__device__ __forceinline__ void vec_params(const ChunkDesc& d, const StepArgs& a,
                                           const VecIn<KG>& in, const VecState<KG>& st) {
    const StepScalars& sc = a.sc;
    uint32_t p[KG];
    bool act[KG];
    lane_offsets<KG>(d, p, act);
    float* th_b = a.b.theta + d.pos;
    uint16_t* out_b = a.b.out ? a.b.out + d.pos : nullptr;
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        if (!act[k]) continue;
        float t[4];
        if (F8) {
#pragma unroll
            for (int j = 0; j < 4; ++j) t[j] = st.T[4 * k + j];
        } else {
            new_params(sc, in.TH[k], st.M + 4 * k, st.V + 4 * k, t);
        }
        st_f4(th_b + p[k], t[0], t[1], t[2], t[3]);
        if (out_b)
            st_u2(out_b + p[k], f32_to_bf16(t[0]) | (f32_to_bf16(t[1]) << 16),
                  f32_to_bf16(t[2]) | (f32_to_bf16(t[3]) << 16));
    }
}

// Back: waits for the block's other chunks if needed (wave 0 polls, the
// others wait at a barrier), then quantises and stores codes and absmax
// (and, with FP8 output, the parameters' E4M3 codes and block scale).
template <int NT, int KG, bool F8>
__device__ __forceinline__ void vec_back(const ChunkDesc& d, int64_t c, const StepArgs& a,
                                         VecState<KG>& st, float* red) {
    constexpr int WSPAN = 256 * KG;
    const StepBuffers& B = a.b;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    uint32_t p[KG];
    bool act[KG];
    lane_offsets<KG>(d, p, act);
    int8_t* qm_b = B.qm + d.pos;
    uint8_t* qv_b = B.qv + d.pos;
    if (st.wait) {
        float x, y, t = 0.0f;
        // red[0..2] are free again after the workgroup max
        coop_wait_wg_t<NT, F8>(B.coop, B.coop_t, B.counters, c - d.part, d.nparts, st.seq, red,
                               x, y, t);
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            st.am[k] = x;
            st.av[k] = y;
            st.at[k] = t;
        }
    }
    uint8_t* f8_b = F8 ? B.fp8 + d.pos : nullptr;
    auto enc = [&](int k, float s8, float y8) {
        st_u1(f8_b + p[k], fp8x4_of(make_float4(st.T[4 * k], st.T[4 * k + 1], st.T[4 * k + 2],
                                                st.T[4 * k + 3]),
                                    s8, y8));
    };
    // |m| <= absmax bounds the codes: no clamp; int8 via a +128 offset
    auto quant = [&](int k, float a_m, float a_v, float ym, float yv) {
        uint32_t qmw = 0u, qvw = 0u;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            qmw = __builtin_amdgcn_cvt_pk_u8_f32(
                rintf(ratio_fast(st.M[4 * k + j], a_m, ym) * 127.0f) + 128.0f, j, qmw);
            qvw = __builtin_amdgcn_cvt_pk_u8_f32(
                rintf(ratio_fast(st.V[4 * k + j], a_v, yv) * 255.0f), j, qvw);
        }
        qmw ^= 0x80808080u;
        if (__builtin_expect(quant_slow(a_m) || quant_slow(a_v), 0)) {
            // absmax below 2^-60: plain division
            qmw = 0u;
            qvw = 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                qmw |= code_m(st.M[4 * k + j], a_m, ym) << (8 * j);
                qvw |= code_v(st.V[4 * k + j], a_v, yv) << (8 * j);
            }
        }
        st_u1(qm_b + p[k], qmw);
        st_u1(qv_b + p[k], qvw);
    };
    if (d.run_log2 >= 0) {
        const int lanes = (1 << d.run_log2) >> 2;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            if (!act[k]) continue;
            quant(k, st.am[k], st.av[k], quant_recip(st.am[k]), quant_recip(st.av[k]));
            const float s8 = F8 ? st.at[k] / 448.0f : 0.0f;
            if (F8) enc(k, s8, quant_recip(s8));
            if ((lane & (lanes - 1)) == 0) {
                const int64_t blk = d.blk + ((wave * WSPAN + 256 * k + 4 * lane) >> d.run_log2);
                B.amax_m[blk] = st.am[k];
                B.amax_v[blk] = st.av[k];
                if (F8) B.fp8_scale[blk] = s8;
            }
        }
    } else {
        // one block: one reciprocal per lane
        const float a_m = st.am[0], a_v = st.av[0];
        const float ym = quant_recip(a_m), yv = quant_recip(a_v);
#pragma unroll
        for (int k = 0; k < KG; ++k)
            if (act[k]) quant(k, a_m, a_v, ym, yv);
        const float s8 = F8 ? st.at[0] / 448.0f : 0.0f;
        if (F8) {
            const float y8 = quant_recip(s8);
#pragma unroll
            for (int k = 0; k < KG; ++k)
                if (act[k]) enc(k, s8, y8);
        }
        if (threadIdx.x == 0 && d.part == 0) {
            B.amax_m[d.blk] = a_m;
            B.amax_v[d.blk] = a_v;
            if (F8) B.fp8_scale[d.blk] = s8;
        }
    }
}

// The whole update of one vector chunk from its loaded inputs.
template <int MODE, int NT, int KG, bool F8>
__device__ __forceinline__ void vec_process(const ChunkDesc& d, int64_t c, const StepArgs& a,
                                            float s, const float* dqm, const float* dqv,
                                            float* red, const VecIn<KG>& in) {
    VecState<KG> st;
    if (!vec_front<MODE, NT, KG, F8>(d, c, a, s, dqm, dqv, red, in, st)) return;
    if (MODE != MODE_PARTIAL) vec_params<KG, F8>(d, a, in, st);
    vec_back<NT, KG, F8>(d, c, a, st, red);
}

// --------------------------------------------------- generic block paths

// One whole block, two sweeps (absmax, then update and codes), element by
// element over its pieces ds[0 .. nd): any shape, stride or alignment.
// With FP8 output the first sweep forms the new parameters too, for their
// absmax (the second forms them again, the same values).
template <int NT, bool F8>
__device__ void block_sweeps(const ChunkDesc* ds, int nd, int64_t blk, const StepArgs& a,
                             float s, const float* dqm, const float* dqv, float* red) {
    const StepBuffers& B = a.b;
    const float am_old = B.amax_m[blk], av_old = B.amax_v[blk];
    float lam = 0.0f, lav = 0.0f, lat = 0.0f;
    for (int q = 0; q < nd; ++q) {
        const ChunkDesc d = ds[q];
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols;
            const int64_t p = d.pos + r * d.ld + (e - r * d.cols);
            const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
            const float mh = dqm[uint8_t(B.qm[p])] * am_old;
            const float vh = dqv[B.qv[p]] * av_old;
            const Elem el = update(a.sc, F8 ? B.theta[p] : 0.0f, g, mh, vh);
            lam = fmaxf(lam, fabsf(el.m));
            lav = fmaxf(lav, el.v);
            if (F8) lat = fmaxf(lat, fabsf(el.th));
        }
    }
    if (F8) {
        float v[3] = {lam, lav, lat};
        wg_maxn<NT, 3>(v, red);
        lam = v[0];
        lav = v[1];
        lat = v[2];
    } else {
        wg_max2<NT>(lam, lav, red);
    }
    const float ym = quant_recip(lam), yv = quant_recip(lav);
    const float s8 = lat / 448.0f, y8 = quant_recip(s8);
    for (int q = 0; q < nd; ++q) {
        const ChunkDesc d = ds[q];
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols;
            const int64_t p = d.pos + r * d.ld + (e - r * d.cols);
            const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
            const float mh = dqm[uint8_t(B.qm[p])] * am_old;
            const float vh = dqv[B.qv[p]] * av_old;
            const Elem el = update(a.sc, B.theta[p], g, mh, vh);
            B.theta[p] = el.th;
            if (B.out) B.out[p] = (uint16_t)f32_to_bf16(el.th);
            if (F8) B.fp8[p] = (uint8_t)fp8_of(el.th, s8, y8);
            B.qm[p] = (int8_t)code_m(el.m, lam, ym);
            B.qv[p] = (uint8_t)code_v(el.v, lav, yv);
        }
    }
    if (threadIdx.x == 0) {
        B.amax_m[blk] = lam;
        B.amax_v[blk] = lav;
        if (F8) B.fp8_scale[blk] = s8;
    }
}

// A run of single-element blocks: the absmax is the element itself, so the
// codes are +-127 / 255 (or 0) and the state is lossless.
template <int NT, bool F8>
__device__ void elem_chunk(const ChunkDesc& d, const StepArgs& a, float s, const float* dqm,
                           const float* dqv) {
    const StepBuffers& B = a.b;
    for (int e = threadIdx.x; e < d.cols; e += NT) {
        const int64_t p = d.pos + e;
        const int64_t blk = d.blk + e;
        const float g = __uint_as_float(uint32_t(B.grad[p]) << 16) * s;
        const float mh = dqm[uint8_t(B.qm[p])] * B.amax_m[blk];
        const float vh = dqv[B.qv[p]] * B.amax_v[blk];
        const Elem el = update(a.sc, B.theta[p], g, mh, vh);
        B.theta[p] = el.th;
        if (B.out) B.out[p] = (uint16_t)f32_to_bf16(el.th);
        if (F8) {
            const float s8 = fabsf(el.th) / 448.0f;
            B.fp8[p] = (uint8_t)fp8_of(el.th, s8, quant_recip(s8));
            B.fp8_scale[blk] = s8;
        }
        const float am = fabsf(el.m), av = el.v;
        B.qm[p] = (int8_t)code_m(el.m, am, quant_recip(am));
        B.qv[p] = (uint8_t)code_v(el.v, av, quant_recip(av));
        B.amax_m[blk] = am;
        B.amax_v[blk] = av;
    }
}

// Dequantisation tables: code -> code / 127 (int8), code / 255 (uint8).
template <int NT>
__device__ __forceinline__ void fill_tables(float* dqm, float* dqv) {
    for (int i = threadIdx.x; i < 256; i += NT) {
        dqm[i] = (float)(int8_t)(uint8_t)i / 127.0f;
        dqv[i] = (float)i / 255.0f;
    }
    __syncthreads();
}

// One chunk, start to end.
template <int MODE, int NT, int KG, bool F8>
__device__ __forceinline__ void one_chunk(const ChunkDesc& d, int64_t c, const StepArgs& a, float s,
                                          const float* dqm, const float* dqv, float* red) {
    // the partial pass only visits chunks of split blocks
    if (MODE == MODE_PARTIAL && (d.kind != KIND_VEC || d.nparts == 1)) return;
    if (d.kind == KIND_VEC) {
        VecIn<KG> in;
        vec_load<MODE, KG, F8>(d, c, a.b, in);
        vec_process<MODE, NT, KG, F8>(d, c, a, s, dqm, dqv, red, in);
    } else if (MODE != MODE_PARTIAL) {
        if (d.kind == KIND_SCALAR)
            block_sweeps<NT, F8>(a.b.chunks + c, 1, d.blk, a, s, dqm, dqv, red);
        else
            elem_chunk<NT, F8>(d, a, s, dqm, dqv);
    }
}

// One workgroup per chunk; each lane owns 4 KG elements (KG 4-element
// groups).  MODE_PARTIAL and MODE_MAIN are the two launches of the two-pass
// split.  MODE_COOP and MODE_ORDERED combine split blocks inside one launch
// (cooperative slots, see the file comment): in MODE_COOP workgroup w takes
// chunk w; in MODE_ORDERED each workgroup takes the next chunk from a
// counter (kept by the launch: the workgroup that takes the last chunk
// zeroes it for the next launch), so chunks are taken in increasing order
// whatever order the hardware starts workgroups in.  Then a waiting
// workgroup can only lack chunks not yet taken, and those all belong to the
// one block that straddles the counter, whose fewer than P chunks already
// taken are all the waiting workgroups there can be (P = most chunks of a
// block); a device that holds more than P workgroups of the kernel always
// has room to start one more, which takes the next chunk.  MODE_COOP relies
// instead on workgroups starting in index order on each XCD (what the
// hardware does; see launch_nt).
//
// Both cooperative modes read the device status word at the start: if a
// wait gave up in an earlier launch (or the caller set the word), a split
// block takes no wait at all -- the workgroup of its first chunk updates the
// whole block in two sweeps and the block's other chunks do nothing.  A
// timeout thus costs time, not state, until rs_plan_check_device clears
// the word.
//
// F8: the step with FP8 output (the new parameters' E4M3 codes and block
// scales, the FP8 copy-in's rule); a separate instance of every mode.
template <int MODE, int NT, int KG, bool F8>
__global__ __launch_bounds__(NT) void adam8_kernel(StepArgs a) {
    constexpr bool kCoop = MODE == MODE_COOP || MODE == MODE_ORDERED;
    __shared__ float dqm[256], dqv[256];
    // the workgroup max (2 or 3 values per wave), then the sequence word
    __shared__ float red[(F8 ? 3 : 2) * (NT / 64) + 2];
    __shared__ uint32_t status;
    __shared__ int64_t taken;
    if (kCoop && threadIdx.x == 0) {
        CoopCounters* k = a.b.counters;
        status = __hip_atomic_load(&k->timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (MODE == MODE_ORDERED) {
            const uint32_t t = __hip_atomic_fetch_add(&k->claim[0], 1u, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT);
            if ((int64_t)t + 1 == a.nwg)
                __hip_atomic_store(&k->claim[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            taken = t;
        }
    }
    // the chunk descriptor is read before the barrier where the chunk is known
    // (its latency overlaps the status word's and the table fill)
    int64_t c = 0;
    ChunkDesc d;
    if (MODE != MODE_ORDERED) {
        c = chunk_of(a.r, blockIdx.x);
        d = a.b.chunks[c];
    }
    fill_tables<NT>(dqm, dqv);  // its barrier publishes `status` and `taken`
    if (MODE == MODE_ORDERED) {
        c = chunk_of(a.r, taken);
        d = a.b.chunks[c];
    }
    const float s = a.b.gscale ? *a.b.gscale : 1.0f;
    if (kCoop && status != 0u && d.kind == KIND_VEC && d.nparts > 1 && d.run_log2 < 0) {
        if (d.part == 0)
            block_sweeps<NT, F8>(a.b.chunks + c, d.nparts, d.blk, a, s, dqm, dqv, red);
        return;
    }
    one_chunk<kCoop ? MODE_COOP : MODE, NT, KG, F8>(d, c, a, s, dqm, dqv, red);
}

// Workgroups of a cooperative kernel the device holds at once.
template <int MODE, int NT, int KG, bool F8>
int coop_capacity() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int per_cu = 0, ncu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(adam8_kernel<MODE, NT, KG, F8>), NT, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached[dev] = per_cu * ncu;
    }
    return cached[dev];
}

template <int NT, int KG, bool F8>
hipError_t launch_mode(const StepArgs& a, int32_t mode, int32_t max_nparts, hipStream_t s) {
    const dim3 grid((unsigned)a.nwg), block(NT);
    if (max_nparts > 1 && mode == RS_SPLIT_COOPERATIVE &&
        coop_ok(max_nparts, coop_capacity<MODE_COOP, NT, KG, F8>())) {
        hipLaunchKernelGGL((adam8_kernel<MODE_COOP, NT, KG, F8>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (max_nparts > 1 && mode == RS_SPLIT_ORDERED &&
        ordered_ok(max_nparts, coop_capacity<MODE_ORDERED, NT, KG, F8>())) {
        hipLaunchKernelGGL((adam8_kernel<MODE_ORDERED, NT, KG, F8>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (max_nparts > 1) {
        hipLaunchKernelGGL((adam8_kernel<MODE_PARTIAL, NT, KG, F8>), grid, block, 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((adam8_kernel<MODE_MAIN, NT, KG, F8>), grid, block, 0, s, a);
    return hipGetLastError();
}

template <int NT, int KG>
hipError_t launch_nt(const StepArgs& a, int32_t mode, int32_t max_nparts, hipStream_t s) {
    if (a.b.fp8) return launch_mode<NT, KG, true>(a, mode, max_nparts, s);
    return launch_mode<NT, KG, false>(a, mode, max_nparts, s);
}

}  // namespace

// Lanes own 16 elements: fewer, larger workgroups amortise the per-chunk
// reduction and the cross-workgroup wait better than more waves with less
// work each.
constexpr int kStepKG = 4;

StepGeometry step_geometry(int64_t chunk_elems) {
    const int kg = kStepKG;
    const int64_t lanes = (chunk_elems + 4 * kg - 1) / (4 * kg);
    int nt = 64;
    while (nt < lanes && nt < kMaxStepThreads) nt *= 2;
    return StepGeometry{nt, kg};
}

hipError_t launch_adam8(const Ranges& chunk_ranges, const StepBuffers& b, const StepScalars& sc,
                        int32_t mode, int64_t chunk_elems, int32_t max_nparts, hipStream_t s) {
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
    const StepGeometry g = step_geometry(chunk_elems);
    switch (g.threads) {
    case 64:
        return launch_nt<64, kStepKG>(a, mode, max_nparts, s);
    case 128:
        return launch_nt<128, kStepKG>(a, mode, max_nparts, s);
    case 256:
        return launch_nt<256, kStepKG>(a, mode, max_nparts, s);
    case 512:
        return launch_nt<512, kStepKG>(a, mode, max_nparts, s);
    default:
        return launch_nt<1024, kStepKG>(a, mode, max_nparts, s);
    }
}

}  // namespace rs
