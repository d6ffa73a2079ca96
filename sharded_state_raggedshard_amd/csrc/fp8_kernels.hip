// FP8 copy-in and copy-out of the planned buffer for gfx950.
//
// veScale-FSDP page, section "Problem and motivation": structure-aware
// training quantises blocks, for instance 128 x 128 tiles in FP8; with
// RaggedShard every block lies inside one rank, so each rank can quantise
// its own blocks before the AllGather and the gathered buffer carries one
// byte per element instead of two.  The scaling rule is this library's:
// per quantisation block s = absmax / 448 (binary32), code = nearest OCP
// E4M3 value of x / s (correctly rounded binary32 quotient), ties to the even
// code, saturating at +-448; absmax 0 gives s = 0 and codes 0.  The copy-out
// writes bf16(e4m3(code) * s) to the bound bf16 views.
//
// The work table has chunks of at most 16384 elements, so a 128 x 128 tile
// (and any block of that size or less) is one workgroup's chunk and its
// absmax is a workgroup reduction; larger blocks are split and combined by
// the same cooperative slots as the step (or two launches).  Lane geometry:
// 16 elements per lane as four 4-element groups, as in the step.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "raggedshard.h"

namespace rs {

namespace {

using namespace kc;

constexpr int kKG = 4;  // 4-element groups per lane

struct Fp8Args {
    Ranges r;  // chunk-index ranges of the FP8 table; wg0 = prefix counts
    Fp8Buffers b;
    TensorTables tt;
    int64_t nwg;
};

// OCP E4M3 code of a finite or infinite q: round to nearest even on the
// E4M3 grid, |q| >= 448 saturates to 448, NaN -> 0x7f (sign kept).
// Normal range: keep the top 3 mantissa bits with a round-to-nearest-even
// carry (the carry may move into the exponent); below 2^-6 the grid step is
// 2^-9, so the code is rint(|q| * 512) (0..8, where 8 is the smallest normal).
__device__ __forceinline__ uint32_t e4m3_code(float q) {
    const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
    const float a = fabsf(q);
    uint32_t code;
    if (!(a < 448.0f)) {
        code = (a != a) ? 0x7fu : 0x7eu;
    } else if (a < 0x1p-6f) {
        code = (uint32_t)rintf(a * 512.0f);
    } else {
        const uint32_t b = __float_as_uint(a);
        code = ((b + 0x7ffffu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
        if (code > 0x7eu) code = 0x7eu;
    }
    return sign | code;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    if ((c & 0x7fu) == 0x7fu) return __uint_as_float(0x7fc00000u);
    const uint32_t e = (c >> 3) & 0xfu, m = c & 7u;
    const float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (c & 0x80u) ? -v : v;
}

__device__ __forceinline__ uint32_t f32_to_bf16(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Code of x in a block of scale s (s >= 0), y = RN(1 / s).
__device__ __forceinline__ uint32_t fp8_of(float x, float s, float y) {
    if (s == 0.0f) return 0u;
    const float q = quant_slow(s) ? x / s : ratio_fast(x, s, y);
    return e4m3_code(q);
}

// Tensor (buffer order) holding buffer position pos.
__device__ __forceinline__ int tensor_at(const TensorTables& tt, int64_t pos) {
    int j = tt.gidx[pos / kGranule];
    while (j < tt.n && tt.tend[j] <= pos) ++j;
    return j;
}

// Whole block of any shape, two sweeps (absmax, then codes).
template <int NT>
__device__ void fp8_scalar_chunk(const ChunkDesc& d, const float* src, uint8_t* buf, float* scale,
                                 float* red) {
    const int64_t n = int64_t(d.rows) * d.cols;
    float am = 0.0f, dummy = 0.0f;
    for (int64_t e = threadIdx.x; e < n; e += NT) {
        const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
        am = fmaxf(am, fabsf(src[off]));
    }
    wg_max2<NT>(am, dummy, red);
    const float s = am / 448.0f, y = quant_recip(s);
    for (int64_t e = threadIdx.x; e < n; e += NT) {
        const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
        buf[d.pos + off] = (uint8_t)fp8_of(src[off], s, y);
    }
    if (threadIdx.x == 0) scale[d.blk] = s;
}

// A run of single-element blocks: each element is its own block.
template <int NT>
__device__ void fp8_elem_chunk(const ChunkDesc& d, const float* src, uint8_t* buf, float* scale) {
    for (int e = threadIdx.x; e < d.cols; e += NT) {
        const float x = src[e];
        const float s = fabsf(x) / 448.0f;
        buf[d.pos + e] = (uint8_t)fp8_of(x, s, quant_recip(s));
        scale[d.blk + e] = s;
    }
}

template <int MODE, int NT>
__global__ __launch_bounds__(NT) void fp8_pack_kernel(Fp8Args a) {
    constexpr int KG = kKG, WSPAN = 256 * KG;
    __shared__ float red[2 * (NT / 64) + 2];
    const int64_t c = chunk_of(a.r, blockIdx.x);
    const ChunkDesc d = a.b.chunks[c];
    const bool split = d.nparts > 1;
    if (MODE == MODE_PARTIAL && (d.kind != KIND_VEC || !split)) return;
    const int j = tensor_at(a.tt, d.pos);
    const float* src = reinterpret_cast<const float*>(a.tt.views[j]) + (d.pos - a.tt.tstart[j]);
    if (d.kind == KIND_SCALAR) {
        if (MODE != MODE_PARTIAL) fp8_scalar_chunk<NT>(d, src, a.b.buf, a.b.scale, red);
        return;
    }
    if (d.kind == KIND_ELEM) {
        if (MODE != MODE_PARTIAL) fp8_elem_chunk<NT>(d, src, a.b.buf, a.b.scale);
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t p[KG];
    bool act[KG];
    lane_offsets<KG>(d, p, act);
    float4 X[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        X[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        if (act[k]) X[k] = ld_f4(src + p[k]);
    }
    float lm[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k)
        lm[k] = fmaxf(fmaxf(fabsf(X[k].x), fabsf(X[k].y)), fmaxf(fabsf(X[k].z), fabsf(X[k].w)));
    uint8_t* out = a.b.buf + d.pos;
    auto store = [&](int k, float s, float y) {
        const uint32_t w = fp8_of(X[k].x, s, y) | (fp8_of(X[k].y, s, y) << 8) |
                           (fp8_of(X[k].z, s, y) << 16) | (fp8_of(X[k].w, s, y) << 24);
        st_u1(out + p[k], w);
    };
    if (d.run_log2 >= 0) {
        // runs of blocks of (1 << run_log2) elements, (1 << run_log2) / 4 lanes each
        const int lanes = (1 << d.run_log2) >> 2;
#pragma unroll
        for (int k = 0; k < KG; ++k) {
            float am = lm[k];
            for (int off = 1; off < lanes; off <<= 1) am = fmaxf(am, __shfl_xor(am, off, 64));
            if (!act[k]) continue;
            const float s = am / 448.0f;
            store(k, s, quant_recip(s));
            if ((lane & (lanes - 1)) == 0)
                a.b.scale[d.blk + ((wave * WSPAN + 256 * k + 4 * lane) >> d.run_log2)] = s;
        }
        return;
    }
    float x = lm[0], dummy = 0.0f;
#pragma unroll
    for (int k = 1; k < KG; ++k) x = fmaxf(x, lm[k]);
    // sequence number of a cooperative split block: read by thread 0 before
    // the workgroup max's barriers, taken from LDS by every thread after
    // them (so none reads the slot after thread 0 has published into it)
    uint32_t* seq_lds = reinterpret_cast<uint32_t*>(red + 2 * (NT / 64));
    if (MODE == MODE_COOP && split && threadIdx.x == 0) *seq_lds = coop_seq(a.b.coop, c);
    if (MODE == MODE_MAIN && split) {
        x = 0.0f;
        for (int q = 0; q < d.nparts; ++q) x = fmaxf(x, a.b.cpart[c - d.part + q].pm);
    } else {
        wg_max2<NT>(x, dummy, red);
        if (split) {
            if (MODE == MODE_PARTIAL) {
                if (threadIdx.x == 0) a.b.cpart[c] = ChunkPartial{x, 0.0f, 0.0f, 0.0f};
                return;
            }
            const uint32_t seq = *seq_lds;  // written before wg_max2's barriers
            if (threadIdx.x == 0) coop_publish(a.b.coop, c, seq, x, 0.0f);
            coop_wait(a.b.coop, a.b.counters, c - d.part, d.nparts, seq, x, dummy);
        }
    }
    const float s = x / 448.0f, y = quant_recip(s);
#pragma unroll
    for (int k = 0; k < KG; ++k)
        if (act[k]) store(k, s, y);
    if (threadIdx.x == 0 && d.part == 0) a.b.scale[d.blk] = s;
}

// Copy-out: bf16(e4m3(code) * s) into the bound bf16 views.
template <int NT>
__global__ __launch_bounds__(NT) void fp8_unpack_kernel(Fp8Args a) {
    constexpr int KG = kKG, WSPAN = 256 * KG;
    const int64_t c = chunk_of(a.r, blockIdx.x);
    const ChunkDesc d = a.b.chunks[c];
    const int j = tensor_at(a.tt, d.pos);
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.tt.views[j]) + (d.pos - a.tt.tstart[j]);
    const uint8_t* in = a.b.buf + d.pos;
    const float* scale = a.b.scale;
    if (d.kind != KIND_VEC) {
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
            const float s = (d.kind == KIND_ELEM) ? scale[d.blk + e] : scale[d.blk];
            dst[off] = (uint16_t)f32_to_bf16(e4m3_value(in[off]) * s);
        }
        return;
    }
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t p[KG];
    bool act[KG];
    lane_offsets<KG>(d, p, act);
    uint32_t W[KG];
    float S[KG];
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        W[k] = 0u;
        S[k] = 0.0f;
        if (act[k]) {
            W[k] = ld_u1(in + p[k]);
            S[k] = scale[d.run_log2 >= 0
                             ? d.blk + ((wave * WSPAN + 256 * k + 4 * lane) >> d.run_log2)
                             : d.blk];
        }
    }
#pragma unroll
    for (int k = 0; k < KG; ++k) {
        if (!act[k]) continue;
        const float s = S[k];
        const uint32_t b0 = f32_to_bf16(e4m3_value(W[k] & 0xffu) * s);
        const uint32_t b1 = f32_to_bf16(e4m3_value((W[k] >> 8) & 0xffu) * s);
        const uint32_t b2 = f32_to_bf16(e4m3_value((W[k] >> 16) & 0xffu) * s);
        const uint32_t b3 = f32_to_bf16(e4m3_value(W[k] >> 24) * s);
        st_u2(dst + p[k], b0 | (b1 << 16), b2 | (b3 << 16));
    }
}

// Zero bytes in the padding of the selected slices (copy tiles, tensor walk).
__global__ __launch_bounds__(kCopyThreads) void fp8_pad_kernel(Ranges r, TensorTables tt,
                                                               uint8_t* buf) {
    int i = 0;
    while (i + 1 < r.n && r.wg0[i + 1] <= blockIdx.x) ++i;
    const int64_t tile = r.lo[i] / kCopyTile + (blockIdx.x - r.wg0[i]);
    const int64_t t0 = max(r.lo[i], tile * kCopyTile), t1 = min(r.hi[i], (tile + 1) * kCopyTile);
    int j = tt.gidx[t0 / kGranule];
    while (j < tt.n && tt.tend[j] <= t0) ++j;
    int64_t cur = t0;
    while (cur < t1) {
        const int64_t e = (j < tt.n) ? min(t1, max(cur, tt.tstart[j])) : t1;
        for (int64_t p = cur + threadIdx.x; p < e; p += kCopyThreads) buf[p] = 0;
        if (j >= tt.n || e >= t1) break;
        cur = min(t1, tt.tend[j]);
        ++j;
    }
}

template <int NT>
int fp8_coop_capacity() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int per_cu = 0, ncu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(fp8_pack_kernel<MODE_COOP, NT>), NT, 0) !=
                hipSuccess ||
            hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return 0;
        cached[dev] = per_cu * ncu;
    }
    return cached[dev];
}

Fp8Args make_args(const Ranges& chunk_ranges, const Fp8Buffers& b, const TensorTables& tt) {
    Fp8Args a;
    a.r = chunk_ranges;
    int64_t total = 0;
    for (int i = 0; i < a.r.n; ++i) {
        a.r.wg0[i] = total;
        total += a.r.hi[i] - a.r.lo[i];
    }
    a.r.wg0[a.r.n] = total;
    a.b = b;
    a.tt = tt;
    a.nwg = total;
    return a;
}

}  // namespace

hipError_t launch_pad_fp8(const Ranges& elem_ranges, const TensorTables& tt, uint8_t* buf,
                          hipStream_t s) {
    Ranges pr = elem_ranges;
    const int64_t ntiles = tile_ranges(pr);
    if (ntiles == 0) return hipSuccess;
    hipLaunchKernelGGL(fp8_pad_kernel, dim3((unsigned)ntiles), dim3(kCopyThreads), 0, s, pr, tt, buf);
    return hipGetLastError();
}

hipError_t launch_pack_fp8(const Ranges& chunk_ranges, const Fp8Buffers& b, const TensorTables& tt,
                           int32_t mode, int32_t max_nparts, hipStream_t s) {
    constexpr int NT = int(kFp8Chunk / 16);
    const Fp8Args a = make_args(chunk_ranges, b, tt);
    if (a.nwg == 0) return hipSuccess;
    if (a.nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.nwg), block(NT);
    // cooperative only with a 2x margin on residency, as in the step
    if (max_nparts > 1 && mode == RS_SPLIT_COOPERATIVE &&
        2 * (int64_t)max_nparts <= fp8_coop_capacity<NT>()) {
        hipLaunchKernelGGL((fp8_pack_kernel<MODE_COOP, NT>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (max_nparts > 1) {
        hipLaunchKernelGGL((fp8_pack_kernel<MODE_PARTIAL, NT>), grid, block, 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((fp8_pack_kernel<MODE_MAIN, NT>), grid, block, 0, s, a);
    return hipGetLastError();
}

hipError_t launch_unpack_fp8(const Ranges& chunk_ranges, const Fp8Buffers& b,
                             const TensorTables& tt, hipStream_t s) {
    constexpr int NT = int(kFp8Chunk / 16);
    const Fp8Args a = make_args(chunk_ranges, b, tt);
    if (a.nwg == 0) return hipSuccess;
    if (a.nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fp8_unpack_kernel<NT>), dim3((unsigned)a.nwg), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace rs
