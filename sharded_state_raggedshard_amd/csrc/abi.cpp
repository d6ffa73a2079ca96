// C-ABI entry points: argument checks, slice selection, table upload and
// kernel launches.  Every check happens before the first launch.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <utility>
#include <vector>

#include "launch.hpp"
#include "plan.hpp"
#include "raggedshard.h"

namespace {

thread_local std::string g_err;

rs_status fail(rs_status st, std::string msg) {
    g_err = std::move(msg);
    return st;
}

rs_status hip_fail(hipError_t e, const char* what) {
    return fail(RS_EHIP, std::string(what) + ": " + hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

rs_status ensure_tables(rs::Plan& p) {
    if (p.tables_built) return RS_OK;
    std::string e;
    rs_status st = rs::build_tables(p, e);
    return st == RS_OK ? RS_OK : fail(st, e);
}

using RangeVec = std::vector<std::pair<int64_t, int64_t>>;

rs_status check_sel(const rs::Plan& p, int32_t bucket, int32_t rank) {
    if (bucket != RS_ALL && (bucket < 0 || bucket >= (int32_t)p.b.size()))
        return fail(RS_EINVAL, "bucket out of range");
    if (rank != RS_ALL && (rank < 0 || rank >= p.m)) return fail(RS_EINVAL, "rank out of range");
    return RS_OK;
}

void push_merged(RangeVec& v, int64_t lo, int64_t hi) {
    if (hi <= lo) return;
    if (!v.empty() && v.back().second == lo)
        v.back().second = hi;
    else
        v.emplace_back(lo, hi);
}

// Buffer-element ranges of the selected slices.
RangeVec elem_ranges(const rs::Plan& p, int32_t bucket, int32_t rank) {
    RangeVec v;
    for (int32_t k = 0; k < (int32_t)p.b.size(); ++k) {
        if (bucket != RS_ALL && k != bucket) continue;
        const rs::BucketInfo& B = p.b[k];
        if (rank == RS_ALL)
            push_merged(v, B.base, B.base + (int64_t)p.m * B.S);
        else
            push_merged(v, B.base + (int64_t)rank * B.S, B.base + (int64_t)(rank + 1) * B.S);
    }
    return v;
}

// Chunk-index ranges of the selected slices.
RangeVec chunk_ranges(const rs::Plan& p, int32_t bucket, int32_t rank) {
    RangeVec v;
    for (int32_t k = 0; k < (int32_t)p.b.size(); ++k) {
        if (bucket != RS_ALL && k != bucket) continue;
        if (rank == RS_ALL)
            push_merged(v, p.cb(k, 0), p.cb(k, p.m));
        else
            push_merged(v, p.cb(k, rank), p.cb(k, rank + 1));
    }
    return v;
}

char* ws(const rs::Plan& p, size_t off);

// Chunk-index ranges of the selected slices in the FP8 work table.
RangeVec chunk_ranges8(const rs::Plan& p, int32_t bucket, int32_t rank) {
    RangeVec v;
    for (int32_t k = 0; k < (int32_t)p.b.size(); ++k) {
        if (bucket != RS_ALL && k != bucket) continue;
        if (rank == RS_ALL)
            push_merged(v, p.cb8(k, 0), p.cb8(k, p.m));
        else
            push_merged(v, p.cb8(k, rank), p.cb8(k, rank + 1));
    }
    return v;
}

rs::Fp8Buffers fp8_buffers(const rs::Plan& p, uint8_t* buf, float* scale) {
    rs::Fp8Buffers b;
    b.buf = buf;
    b.scale = scale;
    b.chunks = reinterpret_cast<const rs::ChunkDesc*>(ws(p, p.off_chunks8));
    b.cpart = reinterpret_cast<rs::ChunkPartial*>(ws(p, p.off_cpart8));
    b.coop = reinterpret_cast<rs::PartSlot*>(ws(p, p.off_coop8));
    b.counters = reinterpret_cast<rs::CoopCounters*>(ws(p, p.off_flag));
    return b;
}

// Splits a range list into launch-sized groups.
std::vector<rs::Ranges> groups(const RangeVec& v) {
    std::vector<rs::Ranges> out;
    for (size_t i = 0; i < v.size(); i += rs::kMaxRanges) {
        rs::Ranges r{};
        r.n = (int32_t)std::min<size_t>(rs::kMaxRanges, v.size() - i);
        for (int32_t j = 0; j < r.n; ++j) {
            r.lo[j] = v[i + j].first;
            r.hi[j] = v[i + j].second;
        }
        out.push_back(r);
    }
    return out;
}

char* ws(const rs::Plan& p, size_t off) { return static_cast<char*>(p.d_ws) + off; }

rs::TensorTables tables(const rs::Plan& p, bool src) {
    rs::TensorTables tt;
    tt.tstart = reinterpret_cast<const int64_t*>(ws(p, p.off_tstart));
    tt.tend = reinterpret_cast<const int64_t*>(ws(p, p.off_tend));
    tt.views = reinterpret_cast<const uint64_t*>(ws(p, src ? p.off_src : p.off_dst));
    tt.gidx = reinterpret_cast<const int32_t*>(ws(p, p.off_gidx));
    tt.n = (int32_t)p.t.size();
    tt.vec_ok = src ? p.src_vec : p.dst_vec;
    return tt;
}

rs_status check_dtype(int32_t dtype) {
    if (dtype != RS_F32 && dtype != RS_BF16) return fail(RS_EINVAL, "dtype must be RS_F32 or RS_BF16");
    return RS_OK;
}

}  // namespace

rs_status rs::set_error(rs_status st, std::string msg) { return fail(st, std::move(msg)); }

extern "C" {

const char* rs_last_error(void) { return g_err.c_str(); }

const char* rs_version(void) { return "raggedshard-gfx950 0.1"; }

rs_status rs_plan_layout(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t g_coll,
                         int32_t order, rs_plan** out) {
    if (!out) return fail(RS_EINVAL, "out is NULL");
    *out = nullptr;
    try {
        rs_plan* h = new rs_plan;
        std::string err;
        rs_status st = rs::plan_layout(specs, n, m, g_coll, order, h->p, err);
        if (st != RS_OK) {
            delete h;
            return fail(st, err);
        }
        *out = h;
        return RS_OK;
    } catch (const std::bad_alloc&) {
        return fail(RS_ENOMEM, "host allocation failed");
    }
}

void rs_plan_free(rs_plan* plan) { delete plan; }

rs_status rs_plan_info(const rs_plan* plan, int32_t* n_tensors, int32_t* n_buckets, int32_t* m,
                       int64_t* total_elems, int64_t* n_blocks) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    const rs::Plan& p = plan->p;
    if (n_tensors) *n_tensors = (int32_t)p.t.size();
    if (n_buckets) *n_buckets = (int32_t)p.b.size();
    if (m) *m = p.m;
    if (total_elems) *total_elems = p.total;
    if (n_blocks) *n_blocks = p.nblocks;
    return RS_OK;
}

rs_status rs_plan_bucket(const rs_plan* plan, int32_t bucket, int64_t* S, int64_t* base,
                         int64_t* padding, int64_t* n_blocks) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    const rs::Plan& p = plan->p;
    if (bucket < 0 || bucket >= (int32_t)p.b.size()) return fail(RS_EINVAL, "bucket out of range");
    const rs::BucketInfo& B = p.b[bucket];
    if (S) *S = B.S;
    if (base) *base = B.base;
    if (padding) *padding = B.padding;
    if (n_blocks) *n_blocks = B.nblk;
    return RS_OK;
}

rs_status rs_plan_offsets(const rs_plan* plan, int64_t* offsets, int64_t* blk0) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    const rs::Plan& p = plan->p;
    for (size_t i = 0; i < p.t.size(); ++i) {
        if (offsets) offsets[i] = p.t[i].off;
        if (blk0) blk0[i] = p.t[i].blk0;
    }
    return RS_OK;
}

rs_status rs_plan_rank_blocks(const rs_plan* plan, int32_t bucket, int32_t rank, int64_t* first,
                              int64_t* count) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    const rs::Plan& p = plan->p;
    if (bucket < 0 || bucket >= (int32_t)p.b.size() || rank < 0 || rank >= p.m)
        return fail(RS_EINVAL, "bucket or rank out of range");
    const int64_t a = p.rank_blk[size_t(bucket) * (p.m + 1) + rank];
    const int64_t b = p.rank_blk[size_t(bucket) * (p.m + 1) + rank + 1];
    if (first) *first = a;
    if (count) *count = b - a;
    return RS_OK;
}

rs_status rs_plan_set_chunk(rs_plan* plan, int64_t chunk_elems) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    if (chunk_elems < 64 || chunk_elems > rs::kMaxChunk || chunk_elems % rs::kChunkAlign != 0)
        return fail(RS_EINVAL, "chunk size must be a multiple of 16 in 64..16384");
    if (plan->p.uploaded) return fail(RS_ESTATE, "chunk size is fixed once the plan is uploaded");
    if (plan->p.chunk_elems != chunk_elems) {
        plan->p.chunk_elems = chunk_elems;
        plan->p.tables_built = false;
    }
    return RS_OK;
}

rs_status rs_plan_set_split_mode(rs_plan* plan, int32_t mode) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    if (mode != RS_SPLIT_TWO_PASS && mode != RS_SPLIT_COOPERATIVE && mode != RS_SPLIT_ORDERED)
        return fail(RS_EINVAL, "unknown split mode");
    plan->p.split_mode = mode;
    return RS_OK;
}

rs_status rs_plan_chunk_count(const rs_plan* plan, int64_t* n_chunks, int64_t* chunk_elems) {
    if (!plan) return fail(RS_EINVAL, "NULL argument");
    rs::Plan& p = const_cast<rs_plan*>(plan)->p;
    rs_status st = ensure_tables(p);
    if (st != RS_OK) return st;
    if (n_chunks) *n_chunks = (int64_t)p.chunks.size();
    if (chunk_elems) *chunk_elems = p.chunk_elems;
    return RS_OK;
}

size_t rs_plan_device_bytes(const rs_plan* plan) {
    if (!plan) {
        fail(RS_EINVAL, "plan is NULL");
        return 0;
    }
    rs::Plan& p = const_cast<rs_plan*>(plan)->p;
    if (ensure_tables(p) != RS_OK) return 0;
    return p.ws_bytes;
}

rs_status rs_plan_upload(rs_plan* plan, void* d_workspace, size_t bytes, void* stream) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    rs::Plan& p = plan->p;
    rs_status st = ensure_tables(p);
    if (st != RS_OK) return st;
    if (!d_workspace || !aligned(d_workspace, 256))
        return fail(RS_EINVAL, "workspace must be a non-NULL 256-byte aligned device pointer");
    if (bytes < p.ws_bytes)
        return fail(RS_ENOMEM, "workspace smaller than rs_plan_device_bytes()");
    hipStream_t s = as_stream(stream);
    char* w = static_cast<char*>(d_workspace);
    hipError_t e = hipMemsetAsync(w, 0, p.ws_bytes, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemsetAsync(workspace)");
    struct Copy {
        size_t off;
        const void* src;
        size_t bytes;
    };
    const Copy copies[] = {
        {p.off_tstart, p.tstart.data(), p.tstart.size() * 8},
        {p.off_tend, p.tend.data(), p.tend.size() * 8},
        {p.off_gidx, p.gidx.data(), p.gidx.size() * 4},
        {p.off_chunks, p.chunks.data(), p.chunks.size() * sizeof(rs::ChunkDesc)},
        {p.off_chunks8, p.chunks8.data(), p.chunks8.size() * sizeof(rs::ChunkDesc)},
    };
    for (const Copy& c : copies) {
        if (c.bytes == 0) continue;
        e = hipMemcpyAsync(w + c.off, c.src, c.bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(tables)");
    }
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(upload)");
    p.d_ws = d_workspace;
    p.uploaded = true;
    p.src_bound = p.dst_bound = false;
    return RS_OK;
}

rs_status rs_bind_views(rs_plan* plan, int32_t which, void* const* d_ptrs, void* stream) {
    if (!plan || !d_ptrs) return fail(RS_EINVAL, "NULL argument");
    rs::Plan& p = plan->p;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded");
    if (which != RS_VIEW_F32_SRC && which != RS_VIEW_BF16_DST)
        return fail(RS_EINVAL, "which must be RS_VIEW_F32_SRC or RS_VIEW_BF16_DST");
    const size_t n = p.t.size();
    std::vector<uint64_t> sorted(n);
    bool starts_ok = true;
    for (size_t j = 0; j < n; ++j) {
        const int32_t i = p.by_pos[j];
        void* v = d_ptrs[i];
        if (!v || !aligned(v, 16))
            return fail(RS_EINVAL, "view " + std::to_string(i) + " is NULL or not 16-byte aligned");
        sorted[j] = reinterpret_cast<uint64_t>(v);
        if (p.t[i].pos % 8 != 0) starts_ok = false;
    }
    const size_t off = which == RS_VIEW_F32_SRC ? p.off_src : p.off_dst;
    hipStream_t s = as_stream(stream);
    hipError_t e = hipMemcpyAsync(ws(p, off), sorted.data(), n * 8, hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(views)");
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize(views)");
    if (which == RS_VIEW_F32_SRC) {
        p.src_bound = true;
        p.src_vec = starts_ok;
    } else {
        p.dst_bound = true;
        p.dst_vec = starts_ok;
    }
    return RS_OK;
}

rs_status rs_pack_shard(const rs_plan* plan, int32_t bucket, int32_t rank, uint16_t* d_buf,
                        void* stream) {
    if (!plan || !d_buf) return fail(RS_EINVAL, "NULL argument");
    const rs::Plan& p = plan->p;
    if (!aligned(d_buf, 16)) return fail(RS_EINVAL, "buffer not 16-byte aligned");
    rs_status st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    if (!p.uploaded || !p.src_bound) return fail(RS_ESTATE, "plan not uploaded or fp32 views not bound");
    const rs::TensorTables tt = tables(p, true);
    for (const rs::Ranges& r : groups(elem_ranges(p, bucket, rank))) {
        hipError_t e = rs::launch_pack(r, tt, d_buf, as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "pack launch");
    }
    return RS_OK;
}

rs_status rs_unpack_full(const rs_plan* plan, int32_t bucket, const uint16_t* d_buf, void* stream) {
    if (!plan || !d_buf) return fail(RS_EINVAL, "NULL argument");
    const rs::Plan& p = plan->p;
    if (!aligned(d_buf, 16)) return fail(RS_EINVAL, "buffer not 16-byte aligned");
    rs_status st = check_sel(p, bucket, RS_ALL);
    if (st != RS_OK) return st;
    if (!p.uploaded || !p.dst_bound) return fail(RS_ESTATE, "plan not uploaded or bf16 views not bound");
    const rs::TensorTables tt = tables(p, false);
    for (const rs::Ranges& r : groups(elem_ranges(p, bucket, RS_ALL))) {
        hipError_t e = rs::launch_unpack(r, tt, d_buf, as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "unpack launch");
    }
    return RS_OK;
}

rs_status rs_pack_shard_fp8(const rs_plan* plan, int32_t bucket, int32_t rank, uint8_t* d_buf,
                            float* d_scale, void* stream) {
    if (!plan || !d_buf || !d_scale) return fail(RS_EINVAL, "NULL argument");
    const rs::Plan& p = plan->p;
    if (!aligned(d_buf, 16) || !aligned(d_scale, 4)) return fail(RS_EINVAL, "misaligned pointer");
    rs_status st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    if (!p.uploaded || !p.src_bound) return fail(RS_ESTATE, "plan not uploaded or fp32 views not bound");
    if (!p.src_vec) return fail(RS_EINVAL, "FP8 copy-in needs 16-byte aligned fp32 views");
    const rs::TensorTables tt = tables(p, true);
    const hipStream_t s = as_stream(stream);
    const rs::Fp8Buffers b = fp8_buffers(p, d_buf, d_scale);
    for (const rs::Ranges& r : groups(chunk_ranges8(p, bucket, rank))) {
        hipError_t e = rs::launch_pack_fp8(r, b, tt, p.split_mode, p.max_nparts8, s);
        if (e != hipSuccess) return hip_fail(e, "fp8 pack launch");
    }
    return RS_OK;
}

rs_status rs_unpack_full_fp8(const rs_plan* plan, int32_t bucket, const uint8_t* d_buf,
                             const float* d_scale, void* stream) {
    if (!plan || !d_buf || !d_scale) return fail(RS_EINVAL, "NULL argument");
    const rs::Plan& p = plan->p;
    if (!aligned(d_buf, 16) || !aligned(d_scale, 4)) return fail(RS_EINVAL, "misaligned pointer");
    rs_status st = check_sel(p, bucket, RS_ALL);
    if (st != RS_OK) return st;
    if (!p.uploaded || !p.dst_bound) return fail(RS_ESTATE, "plan not uploaded or bf16 views not bound");
    if (!p.dst_vec) return fail(RS_EINVAL, "FP8 copy-out needs 16-byte aligned bf16 views");
    const rs::TensorTables tt = tables(p, false);
    const rs::Fp8Buffers b =
        fp8_buffers(p, const_cast<uint8_t*>(d_buf), const_cast<float*>(d_scale));
    for (const rs::Ranges& r : groups(chunk_ranges8(p, bucket, RS_ALL))) {
        hipError_t e = rs::launch_unpack_fp8(r, b, tt, as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "fp8 unpack launch");
    }
    return RS_OK;
}

rs_status rs_group_zero(const rs_plan* plan, int32_t bucket, int32_t rank, void* d_buf,
                        int32_t dtype, void* stream) {
    if (!plan || !d_buf) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_buf, 16)) return fail(RS_EINVAL, "buffer not 16-byte aligned");
    rs_status st = check_dtype(dtype);
    if (st != RS_OK) return st;
    const rs::Plan& p = plan->p;
    st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    for (const rs::Ranges& r : groups(elem_ranges(p, bucket, rank))) {
        hipError_t e = rs::launch_zero(r, d_buf, dtype, as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "zero launch");
    }
    return RS_OK;
}

rs_status rs_group_scale(const rs_plan* plan, int32_t bucket, int32_t rank, void* d_buf,
                         int32_t dtype, float s, void* stream) {
    if (!plan || !d_buf) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_buf, 16)) return fail(RS_EINVAL, "buffer not 16-byte aligned");
    rs_status st = check_dtype(dtype);
    if (st != RS_OK) return st;
    const rs::Plan& p = plan->p;
    st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    for (const rs::Ranges& r : groups(elem_ranges(p, bucket, rank))) {
        hipError_t e = rs::launch_scale(r, d_buf, dtype, s, as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "scale launch");
    }
    return RS_OK;
}

rs_status rs_group_l2norm(const rs_plan* plan, int32_t bucket, int32_t rank, const void* d_buf,
                          int32_t dtype, double* d_sumsq, void* stream) {
    if (!plan || !d_buf || !d_sumsq) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_buf, 16) || !aligned(d_sumsq, 8)) return fail(RS_EINVAL, "misaligned pointer");
    rs_status st = check_dtype(dtype);
    if (st != RS_OK) return st;
    const rs::Plan& p = plan->p;
    st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded (the norm uses workspace scratch)");
    std::vector<rs::Ranges> g = groups(elem_ranges(p, bucket, rank));
    if (g.size() != 1) return fail(RS_EINVAL, "selection has more slices than one launch takes");
    hipError_t e = rs::launch_l2norm(g[0], d_buf, dtype, reinterpret_cast<double*>(ws(p, p.off_l2)),
                                     d_sumsq, 0.0, nullptr, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "l2norm launch");
    return RS_OK;
}

rs_status rs_group_l2norm_static(const rs_plan* plan, int32_t bucket, int32_t rank,
                                 const void* d_buf, int32_t dtype, double* d_sumsq, void* stream) {
    if (!plan || !d_buf || !d_sumsq) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_buf, 16) || !aligned(d_sumsq, 8)) return fail(RS_EINVAL, "misaligned pointer");
    rs_status st = check_dtype(dtype);
    if (st != RS_OK) return st;
    const rs::Plan& p = plan->p;
    st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    std::vector<rs::Ranges> g = groups(elem_ranges(p, bucket, rank));
    if (g.size() != 1) return fail(RS_EINVAL, "selection has more slices than one launch takes");
    double* partials = nullptr;
    int64_t capacity = 0;
    hipError_t e = rs::l2_scratch(&partials, &capacity);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    const int64_t need = rs::l2norm_partials(g[0]);
    if (need > capacity)
        return fail(RS_EINVAL, "the norm needs " + std::to_string(need) +
                                   " partial sums; the library's array holds " +
                                   std::to_string(capacity));
    e = rs::launch_l2norm(g[0], d_buf, dtype, partials, d_sumsq, 0.0, nullptr, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "l2norm launch");
    return RS_OK;
}

rs_status rs_group_l2norm_clip(const rs_plan* plan, int32_t bucket, int32_t rank, const void* d_buf,
                               int32_t dtype, double max_norm, double* d_sumsq, float* d_scale,
                               void* stream) {
    if (!plan || !d_buf || !d_sumsq || !d_scale) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_buf, 16) || !aligned(d_sumsq, 8) || !aligned(d_scale, 4))
        return fail(RS_EINVAL, "misaligned pointer");
    if (!(max_norm > 0.0) || !std::isfinite(max_norm)) return fail(RS_EINVAL, "max_norm must be finite and > 0");
    rs_status st = check_dtype(dtype);
    if (st != RS_OK) return st;
    const rs::Plan& p = plan->p;
    st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded (the norm uses workspace scratch)");
    std::vector<rs::Ranges> g = groups(elem_ranges(p, bucket, rank));
    if (g.size() != 1) return fail(RS_EINVAL, "selection has more slices than one launch takes");
    hipError_t e = rs::launch_l2norm(g[0], d_buf, dtype, reinterpret_cast<double*>(ws(p, p.off_l2)),
                                     d_sumsq, max_norm, d_scale, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "l2norm launch");
    return RS_OK;
}

rs_status rs_clip_coef(const double* d_sumsq, double max_norm, float* d_scale, void* stream) {
    if (!d_sumsq || !d_scale) return fail(RS_EINVAL, "NULL argument");
    if (!(max_norm > 0.0) || !std::isfinite(max_norm)) return fail(RS_EINVAL, "max_norm must be finite and > 0");
    hipError_t e = rs::launch_clip(d_sumsq, max_norm, d_scale, as_stream(stream));
    if (e != hipSuccess) return hip_fail(e, "clip launch");
    return RS_OK;
}

}  // extern "C"

namespace {

// The step with its optional outputs: bf16 (d_bf16_out) and FP8 (d_fp8 and
// d_fp8_scale, both or neither).
rs_status adam8_step(const rs_plan* plan, int32_t bucket, int32_t rank, float* d_master,
                     const uint16_t* d_grad, int8_t* d_qm, uint8_t* d_qv, float* d_amax_m,
                     float* d_amax_v, const rs_adam_hparams* hp, const float* d_grad_scale,
                     uint16_t* d_bf16_out, uint8_t* d_fp8, float* d_fp8_scale, void* stream) {
    if (!plan || !d_master || !d_grad || !d_qm || !d_qv || !d_amax_m || !d_amax_v || !hp)
        return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_master, 16) || !aligned(d_grad, 16) || !aligned(d_qm, 16) || !aligned(d_qv, 16) ||
        !aligned(d_amax_m, 4) || !aligned(d_amax_v, 4) || (d_grad_scale && !aligned(d_grad_scale, 4)) ||
        (d_bf16_out && !aligned(d_bf16_out, 16)) || (d_fp8 && !aligned(d_fp8, 16)) ||
        (d_fp8_scale && !aligned(d_fp8_scale, 4)))
        return fail(RS_EINVAL, "misaligned pointer");
    const rs::Plan& p = plan->p;
    rs_status st = check_sel(p, bucket, rank);
    if (st != RS_OK) return st;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded");
    if (hp->step < 1) return fail(RS_EINVAL, "step must be >= 1");
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0) || !(hp->beta2 >= 0.0 && hp->beta2 < 1.0) ||
        !std::isfinite(hp->lr) || !std::isfinite(hp->eps) || !std::isfinite(hp->weight_decay))
        return fail(RS_EINVAL, "hyper-parameters out of range");
    // step scalars: binary64 on the host, rounded once to binary32
    const double t = (double)hp->step;
    rs::StepScalars sc;
    sc.beta1 = (float)hp->beta1;
    sc.beta2 = (float)hp->beta2;
    sc.omega1 = (float)(1.0 - hp->beta1);
    sc.omega2 = (float)(1.0 - hp->beta2);
    sc.eps = (float)hp->eps;
    sc.c_decay = (float)(1.0 - hp->lr * hp->weight_decay);
    sc.step_size = (float)(hp->lr / (1.0 - std::pow(hp->beta1, t)));
    sc.kappa = (float)(1.0 / std::sqrt(1.0 - std::pow(hp->beta2, t)));
    rs::StepBuffers b;
    b.theta = d_master;
    b.grad = d_grad;
    b.qm = d_qm;
    b.qv = d_qv;
    b.amax_m = d_amax_m;
    b.amax_v = d_amax_v;
    b.gscale = d_grad_scale;
    b.out = d_bf16_out;
    b.chunks = reinterpret_cast<const rs::ChunkDesc*>(ws(p, p.off_chunks));
    b.cpart = reinterpret_cast<rs::ChunkPartial*>(ws(p, p.off_cpart));
    b.coop = reinterpret_cast<rs::PartSlot*>(ws(p, p.off_coop));
    b.counters = reinterpret_cast<rs::CoopCounters*>(ws(p, p.off_flag));
    b.fp8 = d_fp8;
    b.fp8_scale = d_fp8_scale;
    b.cpart_t = reinterpret_cast<float*>(ws(p, p.off_cpart_t));
    b.coop_t = reinterpret_cast<rs::PartSlot*>(ws(p, p.off_coop_t));
    for (const rs::Ranges& r : groups(chunk_ranges(p, bucket, rank))) {
        hipError_t e = rs::launch_adam8(r, b, sc, p.split_mode, p.chunk_elems, p.max_nparts,
                                        as_stream(stream));
        if (e != hipSuccess) return hip_fail(e, "adam8 launch");
    }
    return RS_OK;
}

}  // namespace

extern "C" {

rs_status rs_adam8_step(const rs_plan* plan, int32_t bucket, int32_t rank, float* d_master,
                        const uint16_t* d_grad, int8_t* d_qm, uint8_t* d_qv, float* d_amax_m,
                        float* d_amax_v, const rs_adam_hparams* hp, const float* d_grad_scale,
                        uint16_t* d_bf16_out, void* stream) {
    return adam8_step(plan, bucket, rank, d_master, d_grad, d_qm, d_qv, d_amax_m, d_amax_v, hp,
                      d_grad_scale, d_bf16_out, nullptr, nullptr, stream);
}

rs_status rs_adam8_step_fp8(const rs_plan* plan, int32_t bucket, int32_t rank, float* d_master,
                            const uint16_t* d_grad, int8_t* d_qm, uint8_t* d_qv,
                            float* d_amax_m, float* d_amax_v, const rs_adam_hparams* hp,
                            const float* d_grad_scale, uint16_t* d_bf16_out, uint8_t* d_fp8,
                            float* d_fp8_scale, void* stream) {
    if (!d_fp8 || !d_fp8_scale) return fail(RS_EINVAL, "NULL argument");
    return adam8_step(plan, bucket, rank, d_master, d_grad, d_qm, d_qv, d_amax_m, d_amax_v, hp,
                      d_grad_scale, d_bf16_out, d_fp8, d_fp8_scale, stream);
}

rs_status rs_plan_check_device(rs_plan* plan, void* stream) {
    if (!plan) return fail(RS_EINVAL, "plan is NULL");
    rs::Plan& p = plan->p;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded");
    hipStream_t s = as_stream(stream);
    rs::CoopCounters c{};
    hipError_t e = hipMemcpyAsync(&c, ws(p, p.off_flag), sizeof(c), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "reading device status");
    if (c.timeout != 0) {
        uint32_t zero = 0;
        e = hipMemcpyAsync(ws(p, p.off_flag + offsetof(rs::CoopCounters, timeout)), &zero, 4,
                           hipMemcpyHostToDevice, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) return hip_fail(e, "clearing device status");
        return fail(RS_EHIP, "the device status word was set: a cooperative block wait gave up "
                             "(or the caller set it); one-launch steps and FP8 copy-ins took the "
                             "wait-free whole-block path meanwhile");
    }
    return RS_OK;
}

rs_status rs_plan_status_offset(const rs_plan* plan, size_t* byte_offset) {
    if (!plan || !byte_offset) return fail(RS_EINVAL, "NULL argument");
    const rs::Plan& p = plan->p;
    if (!p.uploaded) return fail(RS_ESTATE, "plan not uploaded");
    *byte_offset = p.off_flag + offsetof(rs::CoopCounters, timeout);
    return RS_OK;
}

}  // extern "C"
