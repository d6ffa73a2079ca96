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

#include <algorithm>
#include <mutex>

#include "kernel_common.hpp"
#include "launch.hpp"
#include "raggedshard.h"

namespace rs {

namespace {

using namespace kc;

// Lane geometry: KG 4-element groups per lane; a chunk is one pass of a
// workgroup (NT * 4 * KG == 16384 elements).
constexpr int kPackKG = 8;
constexpr int kUnpackKG = 4;
constexpr int kPackNT = int(kFp8Chunk / (4 * kPackKG));
constexpr int kUnpackNT = int(kFp8Chunk / (4 * kUnpackKG));
static_assert(kPackNT * 4 * kPackKG == kFp8Chunk && kUnpackNT * 4 * kUnpackKG == kFp8Chunk,
              "an FP8 chunk is one workgroup pass");

struct Fp8Args {
    Ranges r;  // chunk-index ranges of the FP8 table; wg0 = prefix counts
    Fp8Buffers b;
    TensorTables tt;
    int64_t nwg;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Exact decode of one E4M3 code (gfx950 conversion).
__device__ __forceinline__ float e4m3_value(uint32_t c) { return __builtin_amdgcn_cvt_f32_fp8((int)c, 0); }

// bf16 bits of (a, b), round to nearest even, a in the low half.
__device__ __forceinline__ uint32_t bf16x2_bits(float a, float b) {
    const f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// n zero bytes from p (p is any byte address of a 16-byte aligned buffer).
template <int NT>
__device__ void zero_bytes(uint8_t* p, int64_t n) {
    const int64_t head = min(n, int64_t((16 - (reinterpret_cast<uintptr_t>(p) & 15)) & 15));
    const int64_t nv = (n - head) >> 4;
    for (int64_t i = threadIdx.x; i < head; i += NT) p[i] = 0;
    uint4* q = reinterpret_cast<uint4*>(p + head);
    for (int64_t i = threadIdx.x; i < nv; i += NT) q[i] = make_uint4(0u, 0u, 0u, 0u);
    for (int64_t i = head + 16 * nv + threadIdx.x; i < n; i += NT) p[i] = 0;
}

// Whole block of any shape, two sweeps (absmax, then codes), element by
// element over its pieces ds[0 .. nd) (all in one tensor, whose bound view
// starts at buffer position tstart).
template <int NT>
__device__ void fp8_block_sweeps(const ChunkDesc* ds, int nd, const float* view, int64_t tstart,
                                 uint8_t* buf, float* scale, float* red) {
    float am = 0.0f, dummy = 0.0f;
    for (int q = 0; q < nd; ++q) {
        const ChunkDesc d = ds[q];
        const float* src = view + (d.pos - tstart);
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
            am = fmaxf(am, fabsf(src[off]));
        }
    }
    wg_max2<NT>(am, dummy, red);
    const float s = am / 448.0f, y = quant_recip(s);
    for (int q = 0; q < nd; ++q) {
        const ChunkDesc d = ds[q];
        const float* src = view + (d.pos - tstart);
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
            buf[d.pos + off] = (uint8_t)fp8_of(src[off], s, y);
        }
    }
    if (threadIdx.x == 0) scale[ds[0].blk] = s;
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

// Codes (and scale) of one chunk.
template <int MODE, int NT>
__device__ __forceinline__ void fp8_pack_chunk(const Fp8Args& a, int64_t c, const ChunkDesc& d,
                                               float* red) {
    constexpr int KG = kPackKG, WSPAN = 256 * KG;
    const bool split = d.nparts > 1;
    if (MODE == MODE_PARTIAL && (d.kind != KIND_VEC || !split)) return;
    if (d.kind == KIND_PAD) {
        zero_bytes<NT>(a.b.buf + d.pos, d.cols);
        return;
    }
    const int j = d.tensor;
    const float* src = reinterpret_cast<const float*>(a.tt.views[j]) + (d.pos - a.tt.tstart[j]);
    if (d.kind == KIND_SCALAR) {
        if (MODE != MODE_PARTIAL)
            fp8_block_sweeps<NT>(a.b.chunks + c, 1, reinterpret_cast<const float*>(a.tt.views[j]),
                                 a.tt.tstart[j], a.b.buf, a.b.scale, red);
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
    auto store = [&](int k, float s, float y) { st_u1(out + p[k], fp8x4_of(X[k], s, y)); };
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
            // red[0..1] are free again after the workgroup max
            coop_wait_wg<NT>(a.b.coop, a.b.counters, c - d.part, d.nparts, seq, red, x, dummy);
        }
    }
    const float s = x / 448.0f, y = quant_recip(s);
#pragma unroll
    for (int k = 0; k < KG; ++k)
        if (act[k]) store(k, s, y);
    if (threadIdx.x == 0 && d.part == 0) a.b.scale[d.blk] = s;
}

// One workgroup per chunk.  MODE_PARTIAL / MODE_MAIN: the two launches of
// the two-pass split; MODE_COOP / MODE_ORDERED: one launch, split blocks
// meeting on the cooperative slots, the chunk taken as in the step's kernel
// (workgroup index, or a counter), with the same wait-free whole-block path
// while the device status word is set.
template <int MODE, int NT>
__global__ __launch_bounds__(NT) void fp8_pack_kernel(Fp8Args a) {
    constexpr bool kCoop = MODE == MODE_COOP || MODE == MODE_ORDERED;
    __shared__ float red[2 * (NT / 64) + 2];
    __shared__ uint32_t status;
    __shared__ int64_t taken;
    // the chunk descriptor is read before the barrier where the chunk is known
    // (its latency overlaps the status word's)
    int64_t c = 0;
    ChunkDesc d;
    if (MODE != MODE_ORDERED) {
        c = chunk_of(a.r, blockIdx.x);
        d = a.b.chunks[c];
    }
    if (kCoop) {
        if (threadIdx.x == 0) {
            CoopCounters* k = a.b.counters;
            status = __hip_atomic_load(&k->timeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (MODE == MODE_ORDERED) {
                const uint32_t t = __hip_atomic_fetch_add(&k->claim[0], 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                if ((int64_t)t + 1 == a.nwg)
                    __hip_atomic_store(&k->claim[0], 0u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                taken = t;
            }
        }
        __syncthreads();
    }
    if (MODE == MODE_ORDERED) {
        c = chunk_of(a.r, taken);
        d = a.b.chunks[c];
    }
    if (kCoop && status != 0u && d.kind == KIND_VEC && d.nparts > 1 && d.run_log2 < 0) {
        if (d.part == 0) {
            const int j = d.tensor;
            fp8_block_sweeps<NT>(a.b.chunks + c, d.nparts,
                                 reinterpret_cast<const float*>(a.tt.views[j]), a.tt.tstart[j],
                                 a.b.buf, a.b.scale, red);
        }
        return;
    }
    fp8_pack_chunk<kCoop ? MODE_COOP : MODE, NT>(a, c, d, red);
}

// Copy-out: bf16(e4m3(code) * s) into the bound bf16 views.
template <int NT>
__global__ __launch_bounds__(NT) void fp8_unpack_kernel(Fp8Args a) {
    constexpr int KG = kUnpackKG, WSPAN = 256 * KG;
    const int64_t c = chunk_of(a.r, blockIdx.x);
    const ChunkDesc d = a.b.chunks[c];
    if (d.kind == KIND_PAD) return;
    const int j = d.tensor;
    uint16_t* dst = reinterpret_cast<uint16_t*>(a.tt.views[j]) + (d.pos - a.tt.tstart[j]);
    const uint8_t* in = a.b.buf + d.pos;
    const float* scale = a.b.scale;
    if (d.kind != KIND_VEC) {
        const int64_t n = int64_t(d.rows) * d.cols;
        for (int64_t e = threadIdx.x; e < n; e += NT) {
            const int64_t r = e / d.cols, off = r * d.ld + (e - r * d.cols);
            const float s = (d.kind == KIND_ELEM) ? scale[d.blk + e] : scale[d.blk];
            dst[off] = (uint16_t)bf16x2_bits(e4m3_value(in[off]) * s, 0.0f);
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
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)W[k], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)W[k], true);
        st_u2(dst + p[k], bf16x2_bits(lo.x * s, lo.y * s), bf16x2_bits(hi.x * s, hi.y * s));
    }
}

template <int MODE, int NT>
int fp8_coop_capacity() {
    static std::mutex mu;
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    std::lock_guard<std::mutex> lock(mu);
    if (cached[dev] == 0) {
        int per_cu = 0, ncu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(
                &per_cu, reinterpret_cast<const void*>(fp8_pack_kernel<MODE, NT>), NT, 0) !=
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

hipError_t launch_pack_fp8(const Ranges& chunk_ranges, const Fp8Buffers& b, const TensorTables& tt,
                           int32_t mode, int32_t max_nparts, hipStream_t s) {
    constexpr int NT = kPackNT;
    const Fp8Args a = make_args(chunk_ranges, b, tt);
    if (a.nwg == 0) return hipSuccess;
    if (a.nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 grid((unsigned)a.nwg), block(NT);
    if (max_nparts > 1 && mode == RS_SPLIT_COOPERATIVE &&
        coop_ok(max_nparts, fp8_coop_capacity<MODE_COOP, NT>())) {
        hipLaunchKernelGGL((fp8_pack_kernel<MODE_COOP, NT>), grid, block, 0, s, a);
        return hipGetLastError();
    }
    if (max_nparts > 1 && mode == RS_SPLIT_ORDERED &&
        ordered_ok(max_nparts, fp8_coop_capacity<MODE_ORDERED, NT>())) {
        hipLaunchKernelGGL((fp8_pack_kernel<MODE_ORDERED, NT>), grid, block, 0, s, a);
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
    constexpr int NT = kUnpackNT;
    const Fp8Args a = make_args(chunk_ranges, b, tt);
    if (a.nwg == 0) return hipSuccess;
    if (a.nwg > 0x7fffffffLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((fp8_unpack_kernel<NT>), dim3((unsigned)a.nwg), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace rs
