// Device-table formats shared by the host table builder (plan.cpp) and the
// kernels.  Plain structs only; no code.
#pragma once
#include <cstdint>

namespace rs {

// Work unit of the int8-AdamW kernel: what one workgroup updates.
//   KIND_VEC    rows x cols elements (cols % 16 == 0, rows of stride ld, pos %
//               16 == 0) handled as 16-element vectors, one per lane.
//               vpb_log2 < 0: the chunk is part `part` of `nparts` of one
//               block `blk`.  vpb_log2 >= 0: a contiguous run (rows == 1) of
//               whole blocks of (1 << vpb_log2) vectors each, first block blk.
//   KIND_SCALAR one whole block of any shape/alignment (rows x cols, stride
//               ld), element by element, two sweeps.
//   KIND_ELEM   `cols` contiguous elements, each its own block (blk + i).
enum ChunkKind : int32_t { KIND_VEC = 0, KIND_SCALAR = 1, KIND_ELEM = 2 };

struct alignas(16) ChunkDesc {
    int64_t pos;   // absolute buffer element of (row 0, col 0)
    int64_t blk;   // global block id (first block)
    int64_t ld;    // row stride in elements
    int32_t rows;
    int32_t cols;
    int32_t part;
    int32_t nparts;
    int32_t kind;
    int32_t vpb_log2;
};
static_assert(sizeof(ChunkDesc) == 48, "ChunkDesc layout");

// Per-chunk scratch of the two-pass split reduction: partial absmax of the
// chunk and the block's old absmax, saved before the block is rewritten.
struct alignas(16) ChunkPartial {
    float pm, pv, old_m, old_v;
};

// Per-split-block scratch of the cooperative reduction, at the index of the
// block's first chunk.  arrive counts part arrivals over all calls
// (generation g = arrive / nparts, since every call adds exactly nparts);
// amax_*[g & 1] holds the float bits of the running maxima of generation g,
// and generation g clears the other slot for generation g + 1.
struct alignas(16) CoopSlot {
    uint64_t arrive;
    uint32_t amax_m[2];
    uint32_t amax_v[2];
    uint32_t pad[2];
};

// Launch-wide counters of the cooperative step: chunk tickets handed out in
// order and finished workgroups (the last one resets both).
struct alignas(16) CoopCounters {
    uint32_t ticket;
    uint32_t done;
    uint32_t timeout;  // set when a bounded wait gave up
    uint32_t pad;
};
static_assert(sizeof(CoopSlot) == 32, "CoopSlot layout");

constexpr int kVec = 16;             // elements per lane in the step kernel
constexpr int kStepThreads = 1024;   // workgroup size of the step kernel
constexpr int64_t kMaxChunk = int64_t(kVec) * kStepThreads;  // 16384
constexpr int64_t kGranule = 65536;  // copy-kernel tensor-lookup granule
constexpr int kL2Blocks = 2048;      // max partial sums of the L2 norm

}  // namespace rs
