// Device-table formats shared by the host table builder (plan.cpp) and the
// kernels.  Plain structs only; no code.
#pragma once
#include <cstdint>

namespace rs {

// Work unit of the int8-AdamW kernel: what one workgroup updates.
//   KIND_VEC    rows x cols elements (cols % 4 == 0, rows of stride ld,
//               pos % 4 == 0, ld % 4 == 0) handled as 4-element vectors:
//               with KG 4-element groups per lane, wave w covers chunk
//               elements [256 KG w, 256 KG (w + 1)) as KG 256-element
//               slices, lane l holding elements 256 k + 4 l .. +3.
//               run_log2 < 0: the chunk is part `part` of `nparts` of one
//               block `blk`.  run_log2 >= 0: a contiguous run (rows == 1) of
//               whole blocks of (1 << run_log2) elements (4..256), first
//               block blk.
//   KIND_SCALAR one whole block of any shape/alignment (rows x cols, stride
//               ld), element by element, two sweeps.
//   KIND_ELEM   `cols` contiguous elements, each its own block (blk + i).
//   KIND_PAD    `cols` contiguous padding elements of one rank's slice (FP8
//               table only: the copy-in zeroes them, the copy-out skips them).
enum ChunkKind : int32_t { KIND_VEC = 0, KIND_SCALAR = 1, KIND_ELEM = 2, KIND_PAD = 3 };

struct alignas(16) ChunkDesc {
    int64_t pos;   // absolute buffer element of (row 0, col 0)
    int64_t blk;   // global block id (first block)
    int64_t ld;    // row stride in elements
    int32_t rows;
    int32_t cols;
    int32_t part;
    int32_t nparts;
    int16_t kind;
    int16_t run_log2;
    int32_t tensor;  // the chunk's tensor in buffer order (-1 for padding)
};
static_assert(sizeof(ChunkDesc) == 48, "ChunkDesc layout");

// Per-chunk scratch of the two-pass split reduction: partial absmax of the
// chunk and the block's old absmax, saved before the block is rewritten.
struct alignas(16) ChunkPartial {
    float pm, pv, old_m, old_v;
};

// Per-chunk slot of the cooperative reduction: the chunk's partial maxima,
// each as one 64-bit word (sequence << 32) | float bits.  Every call that
// touches a split block updates all of its chunks, so the chunks of a block
// always hold the same sequence; a call publishes sequence + 1 and waits
// until every chunk of the block shows it.  Zeroed by the upload.
struct alignas(16) PartSlot {
    uint64_t m;
    uint64_t v;
};

// Device words of the one-launch split modes: the status word, and the
// chunk counter of RS_SPLIT_ORDERED launches (claim[0]; the workgroup that
// takes a launch's last chunk zeroes it for the next launch; claim[1] is
// unused).  The counter sits on its own 128-byte line.
struct alignas(256) CoopCounters {
    uint32_t timeout;  // set when a bounded wait gave up
    uint32_t pad0[31];
    uint32_t claim[2];
    uint32_t pad1[30];
};
static_assert(sizeof(CoopCounters) == 256, "CoopCounters layout");
static_assert(sizeof(PartSlot) == 16, "PartSlot layout");

constexpr int kVecAlign = 4;         // vector width (elements) of the step kernel
constexpr int kChunkAlign = 16;      // chunk sizes are multiples of 16 elements
constexpr int kMaxStepThreads = 1024;
constexpr int64_t kMaxChunk = int64_t(16) * kMaxStepThreads;  // 16 elements per lane at most
constexpr int kMaxRunLog2 = 8;       // small-block runs: blocks of 4..256 elements
constexpr int64_t kDefaultChunk = 8192;
constexpr int64_t kFp8Chunk = 16384;  // FP8 copy-in: a 128 x 128 tile is one chunk
constexpr int64_t kGranule = 8192;   // copy-kernel tensor-lookup granule (one copy tile)
constexpr int kL2Blocks = 2048;      // max partial sums of the L2 norm
// L2-norm scratch in 64-bit words: two tagged words per partial sum, then
// the epoch word (a 256-byte line of its own)
constexpr int kL2Words = 2 * kL2Blocks + 32;

}  // namespace rs
