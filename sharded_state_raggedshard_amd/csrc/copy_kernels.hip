// DBuffer copy-in / copy-out and group ops for gfx950.
//
// veScale-FSDP page, section "Distributed Buffer (DBuffer)": the buffer
// offers fused group operations (scale, zero, copy) over all tensors of a
// bucket, and a persistent address map gives every parameter a fixed
// location inside the buffer.  Here each op is one launch over the selected
// slices; the copy kernels walk the planned tensor table so a tile of the
// buffer is a handful of straight segments (tensor data or padding), moved
// with 16-byte accesses.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"
#include "raggedshard.h"

namespace rs {

// Partial sums of the allocation-free L2 norm (rs_group_l2norm_static): two
// tagged 64-bit words per workgroup, at most kL2Blocks workgroups, then the
// epoch word (zero at load; each call advances it by one).  Every GPU the
// library runs on holds its own copy until the process ends, and every call
// on that GPU shares it.  In host code this name is only a stand-in for the
// symbol: the device address comes from hipGetSymbolAddress (l2_scratch).
static __device__ __align__(256) double scratch[kL2Words];

namespace {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Quiet NaN with the sign of x (the copy-in's NaN rule).
__device__ __forceinline__ uint32_t canonical_nan(float x) {
    return ((__float_as_uint(x) >> 16) & 0x8000u) | 0x7fc0u;
}

// bf16 bits of (a, b), a in the low half: gfx950's packed conversion, round
// to nearest even; a NaN becomes the quiet NaN with its sign (whatever
// payload the conversion would keep).
__device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 v = {a, b};
    uint32_t r = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
    r = a != a ? (r & 0xffff0000u) | canonical_nan(a) : r;
    r = b != b ? (r & 0x0000ffffu) | (canonical_nan(b) << 16) : r;
    return r;
}

__device__ __forceinline__ uint16_t f32_to_bf16(float x) { return (uint16_t)pack2(x, 0.0f); }

__device__ __forceinline__ float bf16_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint)
__device__ __forceinline__ uint4 load_stream(const void* p) {
    u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// Which range a workgroup belongs to (ranges are few; uniform scan).
__device__ __forceinline__ int find_range(const Ranges& r, int64_t wg) {
    int i = 0;
    while (i + 1 < r.n && r.wg0[i + 1] <= wg) ++i;
    return i;
}

// Tile [t0, t1) of workgroup wg under copy tiling.
__device__ __forceinline__ void tile_of(const Ranges& r, int64_t wg, int64_t& t0, int64_t& t1) {
    int i = find_range(r, wg);
    int64_t tile = r.lo[i] / kCopyTile + (wg - r.wg0[i]);
    t0 = max(r.lo[i], tile * kCopyTile);
    t1 = min(r.hi[i], (tile + 1) * kCopyTile);
}

// Tensor j of the buffer-order tables with its start, end and view, loaded
// together (j == n: none).
struct TensorRef {
    int j;
    int64_t start = 0, end = 0;
    uint64_t view = 0;
    __device__ TensorRef(const TensorTables& tt, int j0) : j(j0) { load(tt); }
    __device__ void load(const TensorTables& tt) {
        if (j < tt.n) {
            start = tt.tstart[j];
            end = tt.tend[j];
            view = tt.views[j];
        }
    }
    __device__ void next(const TensorTables& tt) {
        ++j;
        load(tt);
    }
};

// ---------------------------------------------------------------- pack

__device__ __forceinline__ void zero_seg16(uint16_t* buf, int64_t s, int64_t e) {
    const int tid = threadIdx.x;
    int64_t b0 = min(e, (s + 7) & ~int64_t(7));
    int64_t b1 = max(b0, e & ~int64_t(7));
    for (int64_t p = s + tid; p < b0; p += kCopyThreads) buf[p] = 0;
    for (int64_t p = b1 + tid; p < e; p += kCopyThreads) buf[p] = 0;
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (int64_t p = b0 + int64_t(tid) * 8; p < b1; p += int64_t(kCopyThreads) * 8)
        *reinterpret_cast<uint4*>(buf + p) = z;
}

__device__ __forceinline__ void pack_seg(uint16_t* buf, const float* src, int64_t tstart, int64_t s,
                                         int64_t e, bool vec) {
    const int tid = threadIdx.x;
    if (!vec) {
        for (int64_t p = s + tid; p < e; p += kCopyThreads) buf[p] = f32_to_bf16(src[p - tstart]);
        return;
    }
    int64_t b0 = min(e, (s + 7) & ~int64_t(7));
    int64_t b1 = max(b0, e & ~int64_t(7));
    for (int64_t p = s + tid; p < b0; p += kCopyThreads) buf[p] = f32_to_bf16(src[p - tstart]);
    for (int64_t p = b1 + tid; p < e; p += kCopyThreads) buf[p] = f32_to_bf16(src[p - tstart]);
    // 2048-element steps; in each, lane t converts elements 4 t .. 4 t + 3 of
    // the first and of the second 1024, so every load instruction of a wave
    // reads one contiguous 1 KiB span (and every store writes 512 B)
    constexpr int64_t STEP = int64_t(kCopyThreads) * 8, HALF = STEP / 2;
    int64_t p0 = b0 + int64_t(tid) * 4;
    for (; p0 + 3 * STEP + HALF < b1; p0 += 4 * STEP) {
        uint4 x[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) x[u] = load_stream(src + (p0 + u * HALF - tstart));
#pragma unroll
        for (int u = 0; u < 8; ++u)
            *reinterpret_cast<uint2*>(buf + p0 + u * HALF) =
                make_uint2(pack2(__uint_as_float(x[u].x), __uint_as_float(x[u].y)),
                           pack2(__uint_as_float(x[u].z), __uint_as_float(x[u].w)));
    }
    for (int64_t p = p0; p < b1; p += HALF) {
        const uint4 x = load_stream(src + (p - tstart));
        *reinterpret_cast<uint2*>(buf + p) = make_uint2(pack2(__uint_as_float(x.x), __uint_as_float(x.y)),
                                                        pack2(__uint_as_float(x.z), __uint_as_float(x.w)));
    }
}

__global__ __launch_bounds__(kCopyThreads) void pack_kernel(Ranges r, TensorTables tt,
                                                             uint16_t* __restrict__ buf) {
    int64_t t0, t1;
    tile_of(r, blockIdx.x, t0, t1);
    // the tile's first tensor from the granule index (one granule per tile),
    // then its start, end and view in one dependent step
    TensorRef t(tt, tt.gidx[t0 / kGranule]);
    while (t.j < tt.n && t.end <= t0) t.next(tt);
    int64_t cur = t0;
    while (cur < t1) {
        if (t.j < tt.n && t.start < t1) {
            const int64_t s = max(cur, t.start);
            if (s > cur) zero_seg16(buf, cur, s);
            const int64_t e = min(t1, t.end);
            pack_seg(buf, reinterpret_cast<const float*>(t.view), t.start, s, e, tt.vec_ok != 0);
            cur = e;
            t.next(tt);
        } else {
            zero_seg16(buf, cur, t1);
            cur = t1;
        }
    }
}

// -------------------------------------------------------------- unpack

__global__ __launch_bounds__(kCopyThreads) void unpack_kernel(Ranges r, TensorTables tt,
                                                               const uint16_t* __restrict__ buf) {
    int64_t t0, t1;
    tile_of(r, blockIdx.x, t0, t1);
    TensorRef t(tt, tt.gidx[t0 / kGranule]);
    while (t.j < tt.n && t.end <= t0) t.next(tt);
    const int tid = threadIdx.x;
    for (; t.j < tt.n && t.start < t1; t.next(tt)) {
        const int64_t ts = t.start;
        uint16_t* dst = reinterpret_cast<uint16_t*>(t.view);
        if (dst == buf + ts) continue;  // the view aliases the gathered buffer
        const int64_t s = max(t0, ts);
        const int64_t e = min(t1, t.end);
        if (!tt.vec_ok) {
            for (int64_t p = s + tid; p < e; p += kCopyThreads) dst[p - ts] = buf[p];
            continue;
        }
        int64_t b0 = min(e, (s + 7) & ~int64_t(7));
        int64_t b1 = max(b0, e & ~int64_t(7));
        for (int64_t p = s + tid; p < b0; p += kCopyThreads) dst[p - ts] = buf[p];
        for (int64_t p = b1 + tid; p < e; p += kCopyThreads) dst[p - ts] = buf[p];
        constexpr int64_t STEP = int64_t(kCopyThreads) * 8;
        int64_t p0 = b0 + int64_t(tid) * 8;
        for (; p0 + 3 * STEP < b1; p0 += 4 * STEP) {
            uint4 v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = load_stream(buf + p0 + u * STEP);
#pragma unroll
            for (int u = 0; u < 4; ++u) *reinterpret_cast<uint4*>(dst + (p0 + u * STEP - ts)) = v[u];
        }
        for (int64_t p = p0; p < b1; p += STEP) {
            uint4 v = load_stream(buf + p);
            *reinterpret_cast<uint4*>(dst + (p - ts)) = v;
        }
    }
}

// ----------------------------------------------------------- group ops

// Elements per 16-byte vector: 8 (bf16) or 4 (fp32).
template <typename T>
struct VecOf;
template <>
struct VecOf<uint16_t> {
    static constexpr int n = 8;
};
template <>
struct VecOf<float> {
    static constexpr int n = 4;
};

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void zero_kernel(Ranges r, T* __restrict__ buf) {
    constexpr int V = VecOf<T>::n;
    int64_t t0, t1;
    tile_of(r, blockIdx.x, t0, t1);
    const int tid = threadIdx.x;
    int64_t b0 = min(t1, (t0 + V - 1) & ~int64_t(V - 1));
    int64_t b1 = max(b0, t1 & ~int64_t(V - 1));
    for (int64_t p = t0 + tid; p < b0; p += kCopyThreads) buf[p] = T(0);
    for (int64_t p = b1 + tid; p < t1; p += kCopyThreads) buf[p] = T(0);
    const uint4 z = make_uint4(0, 0, 0, 0);
    for (int64_t p = b0 + int64_t(tid) * V; p < b1; p += int64_t(kCopyThreads) * V)
        *reinterpret_cast<uint4*>(buf + p) = z;
}

__device__ __forceinline__ float scale1(float x, float f) { return x * f; }
__device__ __forceinline__ uint16_t scale1(uint16_t x, float f) {
    return f32_to_bf16(bf16_to_f32(x) * f);
}
__device__ __forceinline__ uint4 scale_vec(uint4 v, float f, uint16_t*) {
    uint4 o;
    o.x = pack2(bf16_to_f32(v.x & 0xffffu) * f, bf16_to_f32(v.x >> 16) * f);
    o.y = pack2(bf16_to_f32(v.y & 0xffffu) * f, bf16_to_f32(v.y >> 16) * f);
    o.z = pack2(bf16_to_f32(v.z & 0xffffu) * f, bf16_to_f32(v.z >> 16) * f);
    o.w = pack2(bf16_to_f32(v.w & 0xffffu) * f, bf16_to_f32(v.w >> 16) * f);
    return o;
}
__device__ __forceinline__ uint4 scale_vec(uint4 v, float f, float*) {
    uint4 o;
    o.x = __float_as_uint(__uint_as_float(v.x) * f);
    o.y = __float_as_uint(__uint_as_float(v.y) * f);
    o.z = __float_as_uint(__uint_as_float(v.z) * f);
    o.w = __float_as_uint(__uint_as_float(v.w) * f);
    return o;
}

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void scale_kernel(Ranges r, T* __restrict__ buf, float f) {
    constexpr int V = VecOf<T>::n;
    int64_t t0, t1;
    tile_of(r, blockIdx.x, t0, t1);
    const int tid = threadIdx.x;
    int64_t b0 = min(t1, (t0 + V - 1) & ~int64_t(V - 1));
    int64_t b1 = max(b0, t1 & ~int64_t(V - 1));
    for (int64_t p = t0 + tid; p < b0; p += kCopyThreads) buf[p] = scale1(buf[p], f);
    for (int64_t p = b1 + tid; p < t1; p += kCopyThreads) buf[p] = scale1(buf[p], f);
    for (int64_t p = b0 + int64_t(tid) * V; p < b1; p += int64_t(kCopyThreads) * V) {
        uint4* q = reinterpret_cast<uint4*>(buf + p);
        *q = scale_vec(*q, f, (T*)nullptr);
    }
}

__device__ __forceinline__ double sq1(float x) { return (double)x * (double)x; }
__device__ __forceinline__ double sq1(uint16_t x) {
    double d = (double)bf16_to_f32(x);
    return d * d;
}
__device__ __forceinline__ double sq_vec(uint4 v, uint16_t*) {
    double a = 0.0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double lo = (double)bf16_to_f32(w[i] & 0xffffu);
        double hi = (double)bf16_to_f32(w[i] >> 16);
        a += lo * lo;
        a += hi * hi;
    }
    return a;
}
__device__ __forceinline__ double sq_vec(uint4 v, float*) {
    double a = 0.0;
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double x = (double)__uint_as_float(w[i]);
        a += x * x;
    }
    return a;
}

// Workgroup-wide sum in a fixed tree order; result valid in thread 0.
__device__ __forceinline__ double wg_sum(double v) {
    __shared__ double red[kCopyThreads / 64];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kCopyThreads / 64; ++i) s += red[i];
    return s;
}

// Clipping coefficient min(1, max_norm / (sqrt(sumsq) + 1e-6)), binary64,
// rounded once to binary32.
__device__ __forceinline__ float clip_of(double sumsq, double max_norm) {
    double c = max_norm / (sqrt(sumsq) + 1e-6);
    if (c > 1.0) c = 1.0;
    return (float)c;
}

// Fixed grid (nwg workgroups); workgroup w takes tiles w, w + nwg, ... and
// publishes its partial sum into slot w; the last workgroup of the grid then
// collects the nwg partials and adds them in index order, so the result
// does not depend on timing.  No read-modify-write is involved (2048 atomic
// additions on one word would serialise at the memory): every call has a
// sequence number, one more than the epoch word that the previous call left
// (read by every workgroup at its start: the collector advances it only
// once every partial of this call is in), and a slot holds the partial's two
// 32-bit halves, each beside that number in one 64-bit word, so the
// collector takes a slot only once both words show this call's number.
// All of it through device-scope atomics, which bypass the per-XCD L2, in
// relaxed order (a release or acquire at device scope would also write back
// or invalidate the XCD's whole L2).  The collector's wait is bounded; if it
// ever gives up (only calls that overlap on one scratch area can make it)
// the result is NaN.
constexpr uint32_t kL2SpinLimit = 1u << 22;

template <typename T>
__global__ __launch_bounds__(kCopyThreads) void sumsq_kernel(Ranges r, const T* __restrict__ buf,
                                                             int64_t ntiles, uint64_t* slots,
                                                             double* out, double max_norm,
                                                             float* scale) {
    constexpr int V = VecOf<T>::n;
    const int tid = threadIdx.x;
    uint64_t* epoch = slots + 2 * kL2Blocks;
    __shared__ uint32_t seq_lds;
    if (tid == 0)
        seq_lds = (uint32_t)__hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) + 1u;
    double acc = 0.0;
    for (int64_t wg = blockIdx.x; wg < ntiles; wg += gridDim.x) {
        int64_t t0, t1;
        tile_of(r, wg, t0, t1);
        int64_t b0 = min(t1, (t0 + V - 1) & ~int64_t(V - 1));
        int64_t b1 = max(b0, t1 & ~int64_t(V - 1));
        for (int64_t p = t0 + tid; p < b0; p += kCopyThreads) acc += sq1(buf[p]);
        for (int64_t p = b1 + tid; p < t1; p += kCopyThreads) acc += sq1(buf[p]);
        for (int64_t p = b0 + int64_t(tid) * V; p < b1; p += int64_t(kCopyThreads) * V)
            acc += sq_vec(load_stream(buf + p), (T*)nullptr);
    }
    const double s = wg_sum(acc);  // its barrier also publishes seq_lds
    const uint64_t seq = (uint64_t)seq_lds << 32;
    if (tid == 0) {
        const uint64_t bits = (uint64_t)__double_as_longlong(s);
        __hip_atomic_store(&slots[2 * blockIdx.x], seq | (bits & 0xffffffffu), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&slots[2 * blockIdx.x + 1], seq | (bits >> 32), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    }
    if (blockIdx.x != gridDim.x - 1) return;
    __syncthreads();  // thread 0 is done reading wg_sum's LDS before its next use
    // the collector: every thread takes slots tid, tid + 256, ... (issuing
    // all of a thread's loads at once measured no faster)
    const int n = (int)gridDim.x;
    const uint32_t want = (uint32_t)(seq >> 32);
    double tot = 0.0;
    uint32_t spins = 0;
    bool failed = false;
    for (int i = tid; i < n; i += kCopyThreads) {
        uint64_t lo, hi;
        for (;;) {
            lo = __hip_atomic_load(&slots[2 * i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            hi = __hip_atomic_load(&slots[2 * i + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if ((uint32_t)(lo >> 32) == want && (uint32_t)(hi >> 32) == want) break;
            if (++spins > kL2SpinLimit) {
                failed = true;
                break;
            }
            __builtin_amdgcn_s_sleep(1);
        }
        tot += __longlong_as_double((long long)((hi << 32) | (lo & 0xffffffffu)));
    }
    if (failed) tot = __longlong_as_double(0x7ff8000000000000ll);
    const double t = wg_sum(tot);  // a NaN from any thread reaches the sum
    if (tid == 0) {
        *out = t;
        if (scale) *scale = clip_of(t, max_norm);
        __hip_atomic_store(epoch, seq >> 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

__global__ void clip_kernel(const double* sumsq, double max_norm, float* scale) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *scale = clip_of(*sumsq, max_norm);
}

}  // namespace

int64_t tile_ranges(Ranges& r) {
    int64_t total = 0;
    for (int i = 0; i < r.n; ++i) {
        r.wg0[i] = total;
        if (r.hi[i] > r.lo[i]) total += (r.hi[i] - 1) / kCopyTile - r.lo[i] / kCopyTile + 1;
    }
    r.wg0[r.n] = total;
    return total;
}

hipError_t launch_pack(const Ranges& r, const TensorTables& tt, uint16_t* buf, hipStream_t s) {
    Ranges rr = r;
    int64_t nwg = tile_ranges(rr);
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s, rr, tt, buf);
    return hipGetLastError();
}

hipError_t launch_unpack(const Ranges& r, const TensorTables& tt, const uint16_t* buf,
                         hipStream_t s) {
    Ranges rr = r;
    int64_t nwg = tile_ranges(rr);
    if (nwg == 0) return hipSuccess;
    hipLaunchKernelGGL(unpack_kernel, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s, rr, tt, buf);
    return hipGetLastError();
}

hipError_t launch_zero(const Ranges& r, void* buf, int32_t dtype, hipStream_t s) {
    Ranges rr = r;
    int64_t nwg = tile_ranges(rr);
    if (nwg == 0) return hipSuccess;
    if (dtype == RS_BF16)
        hipLaunchKernelGGL(zero_kernel<uint16_t>, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s,
                           rr, (uint16_t*)buf);
    else
        hipLaunchKernelGGL(zero_kernel<float>, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s, rr,
                           (float*)buf);
    return hipGetLastError();
}

hipError_t launch_scale(const Ranges& r, void* buf, int32_t dtype, float f, hipStream_t s) {
    Ranges rr = r;
    int64_t nwg = tile_ranges(rr);
    if (nwg == 0) return hipSuccess;
    if (dtype == RS_BF16)
        hipLaunchKernelGGL(scale_kernel<uint16_t>, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s,
                           rr, (uint16_t*)buf, f);
    else
        hipLaunchKernelGGL(scale_kernel<float>, dim3((unsigned)nwg), dim3(kCopyThreads), 0, s, rr,
                           (float*)buf, f);
    return hipGetLastError();
}

hipError_t launch_l2norm(const Ranges& r, const void* buf, int32_t dtype, double* d_scratch,
                         double* d_out, double max_norm, float* d_scale, hipStream_t s) {
    Ranges rr = r;
    int64_t ntiles = tile_ranges(rr);
    int nwg = (int)std::min<int64_t>(std::max<int64_t>(ntiles, 1), kL2Blocks);
    uint64_t* slots = reinterpret_cast<uint64_t*>(d_scratch);
    if (dtype == RS_BF16)
        hipLaunchKernelGGL(sumsq_kernel<uint16_t>, dim3(nwg), dim3(kCopyThreads), 0, s, rr,
                           (const uint16_t*)buf, ntiles, slots, d_out, max_norm, d_scale);
    else
        hipLaunchKernelGGL(sumsq_kernel<float>, dim3(nwg), dim3(kCopyThreads), 0, s, rr,
                           (const float*)buf, ntiles, slots, d_out, max_norm, d_scale);
    return hipGetLastError();
}

hipError_t l2_scratch(double** out, int64_t* capacity) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static double* addr[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        // once per device, with that device current: its copy of the array
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        addr[dev] = static_cast<double*>(p);
    }
    *out = addr[dev];
    *capacity = kL2Blocks;
    return hipSuccess;
}

int64_t l2norm_partials(const Ranges& r) {
    Ranges rr = r;
    const int64_t ntiles = tile_ranges(rr);
    return std::min<int64_t>(std::max<int64_t>(ntiles, 1), kL2Blocks);
}

hipError_t launch_clip(const double* d_sumsq, double max_norm, float* d_scale, hipStream_t s) {
    hipLaunchKernelGGL(clip_kernel, dim3(1), dim3(64), 0, s, d_sumsq, max_norm, d_scale);
    return hipGetLastError();
}

}  // namespace rs
