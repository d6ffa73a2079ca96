// Kernel launchers (implemented in the .hip files).  Plain pointers only.
#pragma once
#include <hip/hip_runtime_api.h>

#include <cstdint>

#include "tables.hpp"

namespace rs {

constexpr int kMaxRanges = 64;

// Up to kMaxRanges half-open element ranges [lo, hi) of one launch, with the
// prefix count of workgroups assigned to each.
struct Ranges {
    int32_t n;
    int32_t pad;
    int64_t lo[kMaxRanges];
    int64_t hi[kMaxRanges];
    int64_t wg0[kMaxRanges + 1];
};

// Copy kernels work on tiles of kCopyTile elements aligned to absolute
// multiples of kCopyTile (a divisor of kGranule).
constexpr int64_t kCopyTile = 8192;
constexpr int kCopyThreads = 256;

// Tensor tables in buffer order (device).
struct TensorTables {
    const int64_t* tstart;
    const int64_t* tend;
    const uint64_t* views;  // fp32 sources (pack) or bf16 destinations (unpack)
    const int32_t* gidx;
    int32_t n;
    int32_t vec_ok;  // every start % 8 == 0 and every view 16-byte aligned
};

// Fills wg0 for copy-style tiling; returns the total workgroup count.
int64_t tile_ranges(Ranges& r);

hipError_t launch_pack(const Ranges& r, const TensorTables& tt, uint16_t* buf, hipStream_t s);
hipError_t launch_unpack(const Ranges& r, const TensorTables& tt, const uint16_t* buf,
                         hipStream_t s);
hipError_t launch_zero(const Ranges& r, void* buf, int32_t dtype, hipStream_t s);
hipError_t launch_scale(const Ranges& r, void* buf, int32_t dtype, float f, hipStream_t s);
// One launch; d_scratch: kL2Words 64-bit words (tagged partial sums, then
// an epoch word that each call advances; zero when first used).  With
// d_scale, the same launch also writes the clipping coefficient for
// max_norm.
hipError_t launch_l2norm(const Ranges& r, const void* buf, int32_t dtype, double* d_scratch,
                         double* d_out, double max_norm, float* d_scale, hipStream_t s);
hipError_t launch_clip(const double* d_sumsq, double max_norm, float* d_scale, hipStream_t s);

// Partial sums the L2 norm of ranges r writes (one per first-pass workgroup).
int64_t l2norm_partials(const Ranges& r);
// Device address (current device) and size in doubles of the library's own
// partial-sum array for the allocation-free L2 norm.
hipError_t l2_scratch(double** out, int64_t* capacity);

// fp32 step scalars derived on the host.
struct StepScalars {
    float beta1, beta2, omega1, omega2, eps, c_decay, step_size, kappa;
};

struct StepBuffers {
    float* theta;
    const uint16_t* grad;
    int8_t* qm;
    uint8_t* qv;
    float* amax_m;
    float* amax_v;
    const float* gscale;  // nullable
    uint16_t* out;        // nullable
    const ChunkDesc* chunks;
    ChunkPartial* cpart;
    PartSlot* coop;
    CoopCounters* counters;
    // FP8 output of the new parameters (nullable: no FP8 output): codes at
    // buffer positions and one scale per global block; with it, the split
    // reductions carry the parameters' maximum in cpart_t (two-pass) and in
    // the .m words of coop_t (one launch), one entry per chunk
    uint8_t* fp8;
    float* fp8_scale;
    float* cpart_t;
    PartSlot* coop_t;
};

// Chunk-index ranges [lo, hi) of the chunk table; mode RS_SPLIT_*.  A
// one-launch mode is used only when the device holds enough workgroups of
// the kernel for max_nparts (kc::coop_ok, kc::ordered_ok); otherwise the
// launch falls back to two-pass.
hipError_t launch_adam8(const Ranges& chunk_ranges, const StepBuffers& b, const StepScalars& sc,
                        int32_t mode, int64_t chunk_elems, int32_t max_nparts, hipStream_t s);

// FP8 copy-in / copy-out (chunk table of kFp8Chunk-element chunks).
struct Fp8Buffers {
    uint8_t* buf;          // one byte per buffer element
    float* scale;          // one per global block id
    const ChunkDesc* chunks;
    ChunkPartial* cpart;   // two-pass partial absmax per chunk
    PartSlot* coop;        // cooperative slots per chunk
    CoopCounters* counters;
};

// Codes and scales of the chunks in chunk_ranges (src views in tt); padding
// chunks are zeroed.
hipError_t launch_pack_fp8(const Ranges& chunk_ranges, const Fp8Buffers& b, const TensorTables& tt,
                           int32_t mode, int32_t max_nparts, hipStream_t s);
// bf16 copy-out of the chunks in chunk_ranges (dst views in tt).
hipError_t launch_unpack_fp8(const Ranges& chunk_ranges, const Fp8Buffers& b,
                             const TensorTables& tt, hipStream_t s);

// Workgroup size and 4-element groups per lane of the step kernel for a
// chunk size.
struct StepGeometry {
    int threads;
    int kg;
};
StepGeometry step_geometry(int64_t chunk_elems);

}  // namespace rs
