/*
 * Plain CPU oracle for the RaggedShard / Distributed Buffer shard-state path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this library.  It shares no
 * code, header, table or constant generator with the HIP library, and the
 * HIP library never calls it.
 *
 * Method source: "veScale-FSDP: Flexible and High-Performance FSDP at Scale
 * (MLSys 2026)", awesome-system-papers page, section "Core method":
 *   - "RaggedShard" (block-wise granularity: element, row, 2-D block; the
 *     LCM rule for sharding along a dimension > 0),
 *   - "Grouped communication: structure-aware planning (Algorithm 1)" (the
 *     layout problem: minimal uniform per-device size S under
 *     Non-Sharded Block, Contiguous Tensor Memory and Balanced Load;
 *     padding only between tensors; offsets aligned to LCM(g_coll, block)),
 *   - "Distributed Buffer (DBuffer)" (group ops scale / zero / copy over
 *     the buffer, persistent per-parameter addresses),
 *   - "Structure-aware training case study" (8-bit Adam with a per-parameter
 *     block granularity, each block quantised locally).
 * The pages do not define the 8-bit quantiser or the optimizer constants;
 * the step below is the explicit definition this project adopts (absmax
 * per block, int8 m with 127 levels, uint8 v with 255 levels, AdamW with
 * decoupled, lr-scaled weight decay and bias correction).
 *
 * Arithmetic: IEEE binary32 with round-to-nearest-even, correctly rounded
 * '/' and sqrtf, no FMA contraction (built with -ffp-contract=off), no
 * denormal flushing.  The L2 norm is accumulated in binary64.
 *
 * Parity status per function is listed in the oracle section of the design doc;
 * every function here is pinned by tests under tests/ (test_oracle_*.py).
 */
#ifndef RS_ORACLE_H
#define RS_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORC_ELEMENT = 0, ORC_ROWS = 1, ORC_TILE = 2 };

/* One RaggedShard tensor: row-major shape, granularity (ROWS: br = k rows;
 * TILE: br x bc).  align_unit selects the alignment reading: 0 aligns
 * offsets to lcm(g_coll, elements of one block), 1 to lcm(g_coll, cut unit)
 * (the alternative reading of "block size" in the planning rule of the
 * veScale-FSDP page, section "Grouped communication"). */
typedef struct {
    int32_t ndim;
    int64_t shape[4];
    int32_t gran;
    int32_t br, bc;
    int32_t align_unit;
} orc_tensor;

/* Quantities derived from a tensor for a given g_coll. */
typedef struct {
    int64_t N;     /* elements */
    int64_t R, C;  /* 2-D view: C = last dim, R = N / C (1-D: [d0, 1]) */
    int64_t u;     /* cut unit: rank boundaries inside the tensor fall on multiples of u */
    int64_t b;     /* elements in one (clipped) non-shardable block */
    int64_t A;     /* offset alignment lcm(g_coll, b), or lcm(g_coll, u) with align_unit */
    int64_t nblk;  /* number of quantisation blocks */
} orc_derived;

/* Returns 0 on success, -1 on an invalid spec. */
int orc_derive(const orc_tensor* t, int64_t g_coll, orc_derived* d);

/* Greedy earliest-feasible placement for one fixed S.  Returns 1 and fills
 * off[] if every tensor can be placed, 0 otherwise. */
int orc_place_fixed_S(const orc_derived* d, int n, int m, int64_t g_coll, int64_t S,
                      int64_t* off);

/* Minimal S (scan from the balanced lower bound in steps of g_coll) and the
 * lexicographically smallest offsets at that S.  Returns 0 on success. */
int orc_plan_bucket(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t* S_out,
                    int64_t* off_out);

/* Exhaustive search over every offset tuple (tiny inputs only).  Same
 * outputs as orc_plan_bucket.  Returns 0 on success, -1 if no S <= S_cap
 * works. */
int orc_plan_bruteforce(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S_cap,
                        int64_t* S_out, int64_t* off_out);

/* Exhaustive feasibility at one fixed S (tiny inputs only): 1 and the
 * lexicographically smallest offsets if some offset tuple satisfies every
 * constraint at S, else 0; -1 on invalid input. */
int orc_bruteforce_feasible_at(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S,
                               int64_t* off_out);

/* The scan's skip rule: 0 if some tensor is longer than 2S while S is not a
 * multiple of its cut unit (such an S is infeasible), else 1; -1 on invalid
 * input. */
int orc_wide_tensor_ok(const orc_tensor* ts, int n, int64_t g_coll, int64_t S);

/* Blocks with elements in two ranks (rank = position / S) when tensor t
 * starts at off[t]; offsets are taken as given (no order, alignment or
 * bound is checked), so naive layouts can be counted too.  Invariant I1 of
 * a plan is this count being zero.  -1 on invalid input. */
int64_t orc_count_cut_blocks(const orc_tensor* ts, int n, int64_t S, const int64_t* off);

/* Invariants I1..I5 of a bucket plan.  Returns 0 if all hold, otherwise the
 * number (1..5) of the first violated invariant. */
int orc_check_plan(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S,
                   const int64_t* off);

/* fp32 -> bf16 bits, round to nearest even; NaN -> quiet NaN with sign. */
uint16_t orc_bf16(float x);
float orc_bf16_to_f32(uint16_t h);
void orc_bf16_array(const float* x, uint16_t* y, int64_t n);

/* ---- buffer-level operations --------------------------------------------
 * A "layout" describes every tensor of every bucket in one concatenated
 * buffer: tensor i belongs to bucket bucket_of[i] and starts at absolute
 * element pos[i] (= base of its bucket + bucket-relative offset); its
 * first quantisation block has global id blk0[i].  Bucket k has per-rank
 * size S[k] and starts at base[k]; every bucket has m ranks.
 * Selections: bucket = -1 means every bucket, rank = -1 every rank. */
typedef struct {
    int n;                     /* tensors */
    int nb;                    /* buckets */
    int m;                     /* ranks */
    const orc_tensor* spec;    /* [n] */
    const int32_t* bucket_of;  /* [n] */
    const int64_t* pos;        /* [n] absolute start */
    const int64_t* blk0;       /* [n] first global block id */
    const int64_t* S;          /* [nb] */
    const int64_t* base;       /* [nb] */
    int64_t g_coll;
} orc_layout;

/* buf[p] = bf16(view_t[p - pos_t]) inside tensors, 0 in padding, for every
 * p of the selected slices. */
void orc_pack(const orc_layout* L, int bucket, int rank, const float* const* views,
              uint16_t* buf);
/* view_t[i] = buf[pos_t + i] for every tensor of the selected buckets. */
void orc_unpack(const orc_layout* L, int bucket, uint16_t* const* views, const uint16_t* buf);

/* ---- FP8 copy-in (E4M3 with one scale per quantisation block) ----------
 * The structure-aware case study of the veScale-FSDP page names
 * block-wise FP8 quantisation with 128x128 blocks (section "Problem and
 * motivation"); the scaling rule here is this library's reading: per
 * quantisation block, s = absmax / 448 (binary32, correctly rounded),
 * code = nearest OCP E4M3 value of x / s (correctly rounded binary32
 * quotient), ties to the even code, saturating at +-448; absmax 0 gives
 * s = 0 and codes 0.  The copy-out is bf16(e4m3(code) * s). */

/* OCP E4M3 (bias 7, no infinities, 0x7f / 0xff NaN): nearest value of x,
 * ties to the even code, |x| beyond 448 saturates to +-448; NaN -> 0x7f
 * with the sign of x. */
uint8_t orc_e4m3(float x);
float orc_e4m3_to_f32(uint8_t q);

/* One block: returns s and writes the n codes. */
float orc_fp8_block(int64_t n, const float* x, uint8_t* codes);

/* buf (one byte per buffer element) and scales (one float per global block
 * id) for the blocks of the selected slices; padding of the selected slices
 * receives 0. */
void orc_pack_fp8(const orc_layout* L, int bucket, int rank, const float* const* views,
                  uint8_t* buf, float* scales);
/* view_t[i] = bf16(e4m3(buf[pos_t + i]) * scale of its block). */
void orc_unpack_fp8(const orc_layout* L, int bucket, uint16_t* const* views, const uint8_t* buf,
                    const float* scales);

/* Group ops over the selected slices (padding included).
 * dtype: 0 = fp32, 1 = bf16. */
void orc_group_zero(const orc_layout* L, int bucket, int rank, void* buf, int dtype);
void orc_group_scale(const orc_layout* L, int bucket, int rank, void* buf, int dtype, float s);
/* Sum of squares in binary64, index order; returns the sum (norm = sqrt). */
double orc_group_sumsq(const orc_layout* L, int bucket, int rank, const void* buf, int dtype);
/* Clipping coefficient min(1, max_norm / (sqrt(sumsq) + 1e-6)) in binary64,
 * rounded once to binary32. */
float orc_clip_coef(double sumsq, double max_norm);

/* ---- blockwise-int8 AdamW ------------------------------------------------ */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step; /* t >= 1 */
} orc_hparams;

/* fp32 scalars derived once in binary64 and rounded to binary32. */
typedef struct {
    float beta1, beta2, omega1, omega2, eps, c_decay, step_size, kappa;
} orc_scalars;

void orc_scalars_from(const orc_hparams* h, orc_scalars* s);

/* One quantisation block whose n elements were gathered into contiguous
 * arrays (block element order).  am / av hold the old absmax on entry and
 * the new one on exit.  out (nullable) receives bf16 of the new params. */
void orc_adam8_block(int64_t n, float* theta, const uint16_t* grad, int8_t* qm, uint8_t* qv,
                     float* am, float* av, const orc_scalars* sc, float gscale,
                     uint16_t* out);

/* The step over every block of the selected slices, on whole buffers laid
 * out by L (state buffers share the layout of the parameter buffer; absmax
 * arrays are indexed by global block id). */
void orc_adam8_step(const orc_layout* L, int bucket, int rank, float* theta,
                    const uint16_t* grad, int8_t* qm, uint8_t* qv, float* amax_m,
                    float* amax_v, const orc_hparams* h, float gscale, uint16_t* out);

/* Element positions of block k of a tensor placed at absolute position p0;
 * writes up to cap positions and returns the block's element count. */
int64_t orc_block_positions(const orc_tensor* t, int64_t p0, int64_t k, int64_t* out,
                            int64_t cap);

#ifdef __cplusplus
}
#endif
#endif
