// Host-side plan: the RaggedShard layout of every bucket and the device
// work tables derived from it.
#pragma once
#include <cstdint>
#include <string>
#include <vector>

#include "raggedshard.h"
#include "tables.hpp"

namespace rs {

struct TensorInfo {
    int64_t N = 0, R = 0, C = 0;
    int64_t u = 0;     // cut unit: a rank boundary inside the tensor lies on a multiple of u
    int64_t b = 0;     // elements of one (clipped) block
    int64_t A = 0;     // offset alignment lcm(g_coll, b)
    int64_t nblk = 0;  // quantisation blocks
    int32_t gran = 0, br = 0, bc = 0, bucket = 0;
    int64_t off = 0;   // bucket-relative offset
    int64_t pos = 0;   // absolute offset in the concatenated buffer
    int64_t blk0 = 0;  // global id of the first block
};

struct BucketInfo {
    int64_t S = 0, base = 0, real = 0, padding = 0, nblk = 0, blk0 = 0;
    std::vector<int32_t> tensors;  // tensor indices, placement order
};

struct Plan {
    int32_t m = 0;
    int64_t g_coll = 0;
    std::vector<TensorInfo> t;       // caller's tensor order
    std::vector<BucketInfo> b;
    std::vector<int32_t> by_pos;     // tensor indices in buffer order
    int64_t total = 0, nblocks = 0;

    // step work table (built for one chunk size)
    int64_t chunk_elems = kDefaultChunk;
    bool tables_built = false;
    std::vector<ChunkDesc> chunks;
    int32_t max_nparts = 1;            // most chunks any block is split into
    std::vector<int64_t> chunk_begin;  // [nb * (m + 1)]
    // FP8 copy-in work table (chunk size kFp8Chunk)
    std::vector<ChunkDesc> chunks8;
    int32_t max_nparts8 = 1;
    std::vector<int64_t> chunk_begin8;
    std::vector<int64_t> rank_blk;     // [nb * (m + 1)] first global block id per rank
    std::vector<int32_t> gidx;         // first tensor (buffer order) ending after granule start
    std::vector<int64_t> tstart, tend; // buffer order

    // workspace layout (byte offsets)
    size_t off_tstart = 0, off_tend = 0, off_src = 0, off_dst = 0, off_gidx = 0;
    size_t off_chunks = 0, off_cpart = 0, off_coop = 0, off_l2 = 0, off_flag = 0;
    size_t off_cpart_t = 0, off_coop_t = 0;  // the step's third value (FP8 output)
    size_t off_chunks8 = 0, off_cpart8 = 0, off_coop8 = 0;
    size_t ws_bytes = 0;

    // device state
    void* d_ws = nullptr;
    bool uploaded = false, src_bound = false, dst_bound = false;
    bool src_vec = true, dst_vec = true;   // all views 16-byte aligned and starts % 8 == 0
    int32_t split_mode = RS_SPLIT_COOPERATIVE;

    int64_t cb(int32_t bucket, int32_t rank) const { return chunk_begin[size_t(bucket) * (m + 1) + rank]; }
    int64_t cb8(int32_t bucket, int32_t rank) const { return chunk_begin8[size_t(bucket) * (m + 1) + rank]; }
};

// Plans every bucket (options: an RS_ORDER_* value, optionally with
// RS_ALIGN_CUT_UNIT).  Returns RS_OK or an error with a message.
rs_status plan_layout(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t g_coll,
                      int32_t options, Plan& out, std::string& err);

// Builds the chunk table, rank boundaries, tensor tables and workspace
// layout for the plan's chunk size.
rs_status build_tables(Plan& p, std::string& err);

// Records the message rs_last_error() returns on this thread; returns st.
rs_status set_error(rs_status st, std::string msg);

// Earliest admissible offset of tensor t at or after e for a fixed S, or -1.
int64_t earliest_offset(const TensorInfo& t, int32_t m, int64_t S, int64_t e);

}  // namespace rs

// The ABI's opaque plan handle.
struct rs_plan {
    rs::Plan p;
};
