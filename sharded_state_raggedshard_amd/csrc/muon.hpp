// Distributed Muon: tables shared by the host plan (muon.cpp) and the
// kernels (muon_kernels.hip).  Plain structs and launcher declarations.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

namespace rs {
namespace mu {

// One Muon matrix: a tensor of the plan viewed as R x C (row-major), the
// whole of it on its root rank.  Newton-Schulz works on X (n x k, n <= k):
// X = U / s, or its transpose when R > C (tr); Y = X^T (k x n) is kept next
// to it, so every product of the iteration reads both operands along their
// rows.  Offsets are in elements (bf16) of the Newton-Schulz workspace.
struct alignas(8) MuonMat {
    int64_t R, C, n, k;
    int64_t pos;        // first element of the tensor in the DBuffers
    int64_t root_off;   // first element in the root buffer (the uneven RaggedShard)
    int64_t x, y0, y1;  // X (n x k); Y (k x n), two buffers used in turn
    int64_t a, b;       // A = X X^T and B (n x n)
    int64_t g0, gn;     // its chunks [g0, g0 + gn) of the gather / apply table
    double sqmax;       // sqrt(max(R, C)), binary64
    int32_t tr;         // R > C: X is U^T / s
    int32_t root;
};
static_assert(sizeof(MuonMat) == 120, "MuonMat layout");

// A run of `count` consecutive elements (from element e0) of matrix `mat`.
struct alignas(16) MuonChunk {
    int64_t e0;
    int32_t mat;
    int32_t count;
};

constexpr int64_t kChunk = 8192;   // elements of one gather / apply chunk
constexpr int kPrepTile = 64;      // prep kernel: 64 x 64 tiles of U
constexpr int kGemmTile = 128;     // Newton-Schulz products: 128 x 128 output tiles,
constexpr int kGemmTile2 = 256;    // or 256 x 256 when both dimensions are multiples of 64
constexpr int64_t kRootAlign = 64; // root-buffer offsets: multiples of 64 elements
// Newton-Schulz: the published quintic coefficients and five steps
constexpr float kNsA = 3.4445f, kNsB = -4.7750f, kNsC = 2.0315f;
constexpr int kNsSteps = 5;
constexpr double kNsEps = 1e-7;

enum { G_GRAM = 0, G_POLY = 1, G_UPDATE = 2 };

struct Tables {
    const MuonMat* mats;
    const MuonChunk* chunks;
    // prefix tile counts, 7 tables of nm + 1: prep (64 x 64 tiles of U); the
    // three products in 128 x 128 tiles; the three products in 256 x 256 tiles
    const int64_t* tiles;
    double* partials;      // one sum of squares per chunk
    double* norms;         // per matrix: sqrt(sum of its chunk sums) + 1e-7
    uint16_t* ws;          // Newton-Schulz buffers
    int32_t nm;
};

// Launchers over matrices [i0, i1) (sorted by root) and their chunks [c0, c1).
hipError_t launch_gather(const Tables& t, int64_t c0, int64_t c1, float* mom, const uint16_t* grad,
                         float mu, uint16_t* root, hipStream_t s);
// host_tiles: a host copy of t.tiles (grid sizes).  wide: every matrix of
// [i0, i1) has both dimensions multiples of 64, so the 256 x 256 kernel runs.
hipError_t launch_orthogonalize(const Tables& t, const int64_t* host_tiles, int32_t i0, int32_t i1,
                                int64_t c0, int64_t c1, bool wide, uint16_t* root, hipStream_t s);
hipError_t launch_apply(const Tables& t, int64_t c0, int64_t c1, float* theta,
                        const uint16_t* root, double lr02, float c_decay, hipStream_t s);

}  // namespace mu
}  // namespace rs
