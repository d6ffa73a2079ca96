/*
 * raggedshard.h -- C-ABI of the MI355X (gfx950) RaggedShard / Distributed
 * Buffer shard-state library.
 *
 * The method is veScale-FSDP as described on the awesome-system-papers page
 * "veScale-FSDP: Flexible and High-Performance FSDP at Scale (MLSys 2026)",
 * section "Core method".  Each entry point below names the passage of that
 * section that defines the operation.
 *
 * Conventions
 *   - Element offsets and sizes are int64 element counts.
 *   - One "DBuffer" is a device array of m * S_b elements per bucket b, the
 *     buckets concatenated in bucket order (bucket b starts at base_b).
 *     Rank r's slice of bucket b is [base_b + r*S_b, base_b + (r+1)*S_b).
 *     On one GPU all m simulated ranks live in the same array; every device
 *     pointer argument named d_buf / d_master / d_grad / d_qm / d_qv is the
 *     base of such a full array and the library adds base_b + r*S_b itself.
 *   - Absmax arrays (one fp32 per quantisation block) are indexed by global
 *     block id: buckets in order, tensors in buffer order (the given order
 *     unless a planner order option reorders them), blocks in order (row
 *     blocks top to bottom, tiles row-major over the tile grid, elements in
 *     order).  A rank's blocks of one bucket form a contiguous id range.
 *   - bucket = RS_ALL selects every bucket, rank = RS_ALL every rank.
 *   - stream: a hipStream_t passed as void* (NULL = the null stream).  Every
 *     device call is asynchronous and stream-ordered; nothing synchronises
 *     the host except rs_plan_upload and rs_bind_views.
 *   - Ownership: the library owns the host-side plans, and a Muon plan also
 *     one stream and two events of its own (created by rs_muon_upload,
 *     released by rs_muon_free).  The caller owns every device allocation
 *     (DBuffers, absmax arrays, workspace, views) and the stream.  The
 *     library never allocates device memory.
 *   - Errors: every call returns an rs_status; all argument checks happen on
 *     the host before any launch, and a failed check launches nothing.
 *     rs_last_error() returns a thread-local message for the last non-OK
 *     status of the calling thread.
 *   - Device pointers must be 16-byte aligned.
 *   - Concurrency: calls on distinct plans are independent.  Device calls on
 *     one plan share that plan's workspace scratch and must be ordered on
 *     one stream (or synchronised by the caller); the one exception,
 *     rs_muon_orthogonalize for different roots, is stated there.
 */
#ifndef RAGGEDSHARD_H
#define RAGGEDSHARD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct rs_plan rs_plan; /* opaque, host-owned */

typedef enum {
    RS_OK = 0,
    RS_EINVAL = -1,    /* invalid argument (null pointer, bad spec, out-of-range index, misalignment) */
    RS_EOVERFLOW = -2, /* a size or offset does not fit in int64 / the device tables */
    RS_ESTATE = -3,    /* call out of order: plan not uploaded, views not bound */
    RS_EHIP = -4,      /* a HIP runtime call or kernel launch failed */
    RS_ENOMEM = -5     /* host allocation failed, or the workspace is too small */
} rs_status;

/* Quantisation / sharding granularity of a tensor (RaggedShard section:
 * the atomic block may be an element, a group of rows, or a 2-D block). */
enum { RS_ELEMENT = 0, RS_ROWS = 1, RS_TILE = 2 };
enum { RS_F32 = 0, RS_BF16 = 1 };
enum { RS_VIEW_F32_SRC = 0, RS_VIEW_BF16_DST = 1 };
/* Planner options (the `order` argument of rs_plan_layout): one tensor
 * order, optionally or-ed with RS_ALIGN_CUT_UNIT.  The planning rule of the
 * veScale-FSDP page (section "Grouped communication") names three tensor
 * orders: the default one, by block size and by shape; read here as the
 * given order, block size (elements of one block) descending, and element
 * count descending, ties keeping the given order.  RS_ALIGN_CUT_UNIT takes
 * the other reading of the "block size" in the alignment rule: offsets are
 * multiples of lcm(g_coll, cut unit) instead of lcm(g_coll, block
 * elements) (only tiles narrower than their tensor, and row blocks of
 * tensors shorter than one block, differ). */
enum {
    RS_ORDER_GIVEN = 0,
    RS_ORDER_BY_BLOCK = 1,
    RS_ORDER_BY_SIZE = 2,
    RS_ORDER_MASK = 0xff,
    RS_ALIGN_CUT_UNIT = 0x100
};
/* How a quantisation block larger than one chunk is reduced across the
 * workgroups that share it (int8-AdamW step and FP8 copy-in):
 *   RS_SPLIT_TWO_PASS:    two launches (per-chunk partial absmax, then the
 *                         update); re-reads the inputs of split blocks.
 *   RS_SPLIT_COOPERATIVE: one launch in which the chunks of a block meet on
 *                         device-scope slots; workgroup w takes chunk w, and
 *                         the waits end because gfx950 starts workgroups in
 *                         index order on each XCD (measured behaviour, not a
 *                         HIP promise).  The fastest mode; the default.
 *   RS_SPLIT_ORDERED:     the same single launch, but every workgroup takes
 *                         its chunk from a counter, so the waits end whatever
 *                         order workgroups start in (one device-scope atomic
 *                         per workgroup; slower). */
enum { RS_SPLIT_TWO_PASS = 0, RS_SPLIT_COOPERATIVE = 1, RS_SPLIT_ORDERED = 2 };

#define RS_ALL (-1)

/* One RaggedShard tensor.  Row-major shape[0..ndim) (ndim 1..4).  The
 * tensor is viewed as [R, C] with C = shape[ndim-1] (a 1-D tensor is
 * [d0, 1]; leading dimensions fold into R).
 *   RS_ELEMENT: every element is its own block.
 *   RS_ROWS:    blocks of br whole rows (the last block may be shorter).
 *   RS_TILE:    br x bc tiles (br >= 2), row-major over the tile grid; edge
 *               tiles are clipped.
 * bucket: communication bucket index (buckets 0..nb-1 all non-empty). */
typedef struct {
    int32_t ndim;
    int32_t gran;
    int32_t br;
    int32_t bc;
    int32_t bucket;
    int32_t reserved; /* must be 0 */
    int64_t shape[4];
} rs_tensor_spec;

/* AdamW hyper-parameters (binary64; the library rounds the derived step
 * scalars once to binary32).  step is t >= 1. */
typedef struct {
    double lr, beta1, beta2, eps, weight_decay;
    int64_t step;
} rs_adam_hparams;

/* ------------------------------------------------------------------ plan */

/* Plan a layout (page section "Grouped communication: structure-aware
 * planning (Algorithm 1)").  For each bucket independently: the minimal
 * per-rank size S_b (a multiple of g_coll) such that the bucket's tensors,
 * in the given order, sit in one buffer of m*S_b elements with
 *   - no block split across two ranks (Non-Sharded Block; a cut inside a
 *     tensor falls on a multiple of its cut unit: 1 element, br whole rows),
 *   - each tensor contiguous, padding only between tensors (Contiguous
 *     Tensor Memory), every offset a multiple of lcm(g_coll, elements of one
 *     block),
 *   - m equal slices (Balanced Load);
 * among placements with that S_b the lexicographically smallest offsets.
 * Tensors are placed in the order `order` selects (RS_ORDER_GIVEN: as
 * given); offsets are reported per tensor in the caller's order either way.
 * Host only, synchronous; a long scan over S runs on up to 16 host threads
 * (joined before the call returns; the result does not depend on them).
 * On success *out receives a new plan (free with rs_plan_free).
 * Errors: RS_EINVAL (n < 1, m < 1, g_coll < 1, bad spec, empty bucket,
 * unknown order or option bits),
 * RS_EOVERFLOW (sizes beyond 2^50 elements), RS_ENOMEM. */
rs_status rs_plan_layout(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t g_coll,
                         int32_t order, rs_plan** out);

/* Releases a plan (NULL is allowed).  Does not touch device memory. */
void rs_plan_free(rs_plan* plan);

/* Whole-plan sizes: tensor count, bucket count, ranks, total buffer
 * elements (sum of m*S_b) and total quantisation blocks.  Any output
 * pointer may be NULL. */
rs_status rs_plan_info(const rs_plan* plan, int32_t* n_tensors, int32_t* n_buckets, int32_t* m,
                       int64_t* total_elems, int64_t* n_blocks);

/* Per-bucket results: S_b, base_b, padding elements (m*S_b minus real
 * elements) and block count.  Any output pointer may be NULL. */
rs_status rs_plan_bucket(const rs_plan* plan, int32_t bucket, int64_t* S, int64_t* base,
                         int64_t* padding, int64_t* n_blocks);

/* offsets[i] = bucket-relative offset of tensor i; blk0[i] = global id of
 * its first block.  Arrays of n entries; either may be NULL. */
rs_status rs_plan_offsets(const rs_plan* plan, int64_t* offsets, int64_t* blk0);

/* Global block id range [first, first+count) of rank's blocks in bucket. */
rs_status rs_plan_rank_blocks(const rs_plan* plan, int32_t bucket, int32_t rank, int64_t* first,
                              int64_t* count);

/* Maximum elements one workgroup handles in the step (a multiple of 16 in
 * 64..16384).  Larger blocks are split into chunks.  The planner's default
 * is 4096, or 8192 for plans of more than 2^30 elements of which at most
 * half sit in tiles narrower than their tensor.  Must be called before
 * rs_plan_upload.  Errors: RS_EINVAL,
 * RS_ESTATE (uploaded). */
rs_status rs_plan_set_chunk(rs_plan* plan, int64_t chunk_elems);

/* RS_SPLIT_COOPERATIVE (default), RS_SPLIT_ORDERED or RS_SPLIT_TWO_PASS;
 * may change at any time between calls.  The one-launch modes fall back to
 * two launches when the device cannot hold twice the workgroups a block can
 * keep waiting (twice the most chunks of any block; for the cooperative
 * mode also twice that per XCD). */
rs_status rs_plan_set_split_mode(rs_plan* plan, int32_t mode);

/* Number of chunks of the step's work table and the chunk size in effect
 * (for sizing and reporting).  Either output pointer may be NULL. */
rs_status rs_plan_chunk_count(const rs_plan* plan, int64_t* n_chunks, int64_t* chunk_elems);

/* Device bytes the workspace must provide (tables + scratch). */
size_t rs_plan_device_bytes(const rs_plan* plan);

/* Persistent address mapping (DBuffer section): copies the plan's tables
 * into the caller's device workspace (>= rs_plan_device_bytes bytes,
 * 256-byte aligned) and zeroes its scratch.  The plan keeps d_workspace;
 * the caller keeps it alive until the plan is freed.  Synchronises the
 * stream.  Errors: RS_EINVAL, RS_ENOMEM (bytes too small), RS_EHIP. */
rs_status rs_plan_upload(rs_plan* plan, void* d_workspace, size_t bytes, void* stream);

/* Binds per-tensor device views (DBuffer section: zero-copy per-parameter
 * data pointers):
 *   RS_VIEW_F32_SRC:  d_ptrs[i] -> N_i fp32 values of tensor i (pack source)
 *   RS_VIEW_BF16_DST: d_ptrs[i] -> N_i bf16 values of tensor i (unpack
 *                     destination; a view equal to d_buf + pos_i aliases the
 *                     gathered buffer and is skipped by rs_unpack_full).
 * d_ptrs is a host array of n device pointers (16-byte aligned).
 * Synchronises the stream.  Errors: RS_EINVAL, RS_ESTATE (not uploaded). */
rs_status rs_bind_views(rs_plan* plan, int32_t which, void* const* d_ptrs, void* stream);

/* ------------------------------------------------------------ copy in/out */

/* Copy-in (DBuffer section; copy is one of the fused group ops): for every
 * position p of the selected slices, d_buf[p] = bf16_rne(view_t[p - pos_t])
 * when p lies in tensor t, and 0 in padding.  bf16_rne: round to nearest
 * even, NaN -> quiet NaN with its sign.  rank = RS_ALL packs all m slices
 * (on one GPU: the all-gathered buffer).  Needs RS_VIEW_F32_SRC views.
 * Errors: RS_EINVAL, RS_ESTATE, RS_EHIP. */
rs_status rs_pack_shard(const rs_plan* plan, int32_t bucket, int32_t rank, uint16_t* d_buf,
                        void* stream);

/* Copy-out: view_t[i] = d_buf[pos_t + i] for every tensor of the selected
 * bucket(s); views that alias d_buf are skipped (zero copy).  Needs
 * RS_VIEW_BF16_DST views.  Errors: RS_EINVAL, RS_ESTATE, RS_EHIP. */
rs_status rs_unpack_full(const rs_plan* plan, int32_t bucket, const uint16_t* d_buf,
                         void* stream);

/* ------------------------------------------------------- FP8 copy-in/out
 * Block-wise FP8 (page section "Problem and motivation": 128 x 128 FP8
 * blocks), made possible by RaggedShard keeping every quantisation block in
 * one rank.  Rule (this library's reading): per quantisation block of the
 * plan, s = absmax / 448 in binary32; code = nearest OCP E4M3 value of x / s
 * (correctly rounded binary32 quotient), ties to the even code, saturating
 * at +-448; absmax 0 gives s = 0 and codes 0.  One byte per buffer element
 * (the gathered buffer is half the bf16 one), one fp32 scale per block.
 * Non-finite inputs give undefined codes (the kernels do not fault). */

/* Codes of the selected slices' blocks into d_buf (one byte per buffer
 * element, full bucket-set array as for rs_pack_shard; padding of the
 * selected slices set to 0) and their scales into d_scale (one float per
 * global block id).  Reads the bound fp32 views, which must be 16-byte
 * aligned.  Split blocks use the plan's split mode.  d_buf 16-byte aligned.
 * Errors: RS_EINVAL, RS_ESTATE (not uploaded / views not bound). */
rs_status rs_pack_shard_fp8(const rs_plan* plan, int32_t bucket, int32_t rank, uint8_t* d_buf,
                            float* d_scale, void* stream);

/* view_t[i] = bf16(e4m3(d_buf[pos_t + i]) * d_scale[block of the element])
 * for every tensor of the selected bucket(s), into the bound bf16 views
 * (16-byte aligned).  Errors as rs_unpack_full. */
rs_status rs_unpack_full_fp8(const rs_plan* plan, int32_t bucket, const uint8_t* d_buf,
                             const float* d_scale, void* stream);

/* -------------------------------------------------------------- group ops
 * DBuffer section: one fused launch per op over all selected slices of a
 * DBuffer (padding included).  dtype RS_F32 or RS_BF16. */

/* d_buf[p] = +0. */
rs_status rs_group_zero(const rs_plan* plan, int32_t bucket, int32_t rank, void* d_buf,
                        int32_t dtype, void* stream);

/* fp32: x * s;  bf16: bf16_rne(float(x) * s). */
rs_status rs_group_scale(const rs_plan* plan, int32_t bucket, int32_t rank, void* d_buf,
                         int32_t dtype, float s, void* stream);

/* *d_sumsq = sum of float(x)^2 over the selection, squares and sum in
 * binary64 (the global L2 norm is its square root; per-rank values are the
 * partial sums an all-reduce would add).  Deterministic: a fixed two-level
 * reduction order (per-workgroup sums, then those sums in workgroup order,
 * added by the grid's last workgroup; one launch).  NaN / Inf propagate.
 * d_sumsq: one device double.  Uses the plan's workspace: calls on one plan
 * that overlap (several streams) race (the result may then be NaN). */
rs_status rs_group_l2norm(const rs_plan* plan, int32_t bucket, int32_t rank, const void* d_buf,
                          int32_t dtype, double* d_sumsq, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, allocation-free serving or training loops, harnesses that forbid
 * hipMalloc -- and so may not have uploaded the plan: rs_group_l2norm with
 * the same arguments and result (the same kernels, bit for bit), but its
 * partial sums live in the library's own device array (2048 partial sums
 * as tagged 64-bit word pairs and a call counter, 32.25 KiB per GPU, held
 * until the process ends) instead of the plan's workspace.  Allocates
 * nothing and needs no rs_plan_upload.  The array holds one partial per
 * workgroup, and the launch never uses more than 2048 workgroups; a launch
 * that would need more is rejected with RS_EINVAL.  Each call tags its
 * partials with the next value of the counter (zero when the library
 * loads), so what earlier calls left in the array is never taken and
 * nothing needs clearing between calls.  Every call on one GPU shares the array: calls that overlap on
 * one GPU (several streams, several threads) race and must be ordered by the
 * caller.  Errors as rs_group_l2norm, and RS_EHIP if the array's device
 * address cannot be obtained. */
rs_status rs_group_l2norm_static(const rs_plan* plan, int32_t bucket, int32_t rank,
                                 const void* d_buf, int32_t dtype, double* d_sumsq, void* stream);

/* Gradient-clipping coefficient on the device:
 * *d_scale = (float) min(1, max_norm / (sqrt(*d_sumsq) + 1e-6)), in binary64.
 * Separate from the norm because on m GPUs the per-rank sums of squares are
 * all-reduced between the two. */
rs_status rs_clip_coef(const double* d_sumsq, double max_norm, float* d_scale, void* stream);

/* rs_group_l2norm and rs_clip_coef in one launch, for a selection that is
 * the whole norm (every rank of the buckets on this device, or m = 1):
 * *d_sumsq as rs_group_l2norm, *d_scale as rs_clip_coef for max_norm, bit
 * for bit.  d_scale: one device float, 4-byte aligned.  Errors as
 * rs_group_l2norm, and RS_EINVAL for max_norm not finite and > 0. */
rs_status rs_group_l2norm_clip(const rs_plan* plan, int32_t bucket, int32_t rank, const void* d_buf,
                               int32_t dtype, double max_norm, double* d_sumsq, float* d_scale,
                               void* stream);

/* ----------------------------------------------------------- int8 AdamW */

/* Blockwise-int8 AdamW over the selected slices (page section
 * "Structure-aware training case study": 8-bit Adam with a per-parameter
 * block granularity, each block quantised on its own, no metadata
 * exchanged between blocks).  For every block B of the selection:
 *   g  = float(d_grad[i]) * s          (s = *d_grad_scale, or 1 if NULL)
 *   m^ = (q_m[i] / 127) * amax_m[B],   v^ = (q_v[i] / 255) * amax_v[B]
 *   m  = b1*m^ + (1-b1)*g,             v  = b2*v^ + (1-b2)*g*g
 *   theta = theta*(1 - lr*wd) - (lr/(1-b1^t)) * m / (sqrt(v)/sqrt(1-b2^t) + eps)
 *   amax_m[B] = max|m|, amax_v[B] = max v,
 *   q_m[i] = rne(m/amax_m*127) (0 if amax 0), q_v[i] = rne(v/amax_v*255).
 * All arithmetic binary32; the quantisation codes are exact (correctly
 * rounded division); theta may differ from a correctly rounded evaluation
 * by a few ulp.  d_master fp32, d_grad bf16, d_qm int8, d_qv uint8 are
 * full DBuffers; d_amax_m / d_amax_v hold one fp32 per global block.
 * d_bf16_out (nullable): bf16_rne(theta) written at the same positions
 * (fused copy-in).  Padding positions are never read or written.
 * Errors: RS_EINVAL, RS_ESTATE, RS_EHIP. */
rs_status rs_adam8_step(const rs_plan* plan, int32_t bucket, int32_t rank, float* d_master,
                        const uint16_t* d_grad, int8_t* d_qm, uint8_t* d_qv, float* d_amax_m,
                        float* d_amax_v, const rs_adam_hparams* hp, const float* d_grad_scale,
                        uint16_t* d_bf16_out, void* stream);

/* rs_adam8_step followed by the FP8 copy-in of the new parameters, in one
 * pass (page sections "Structure-aware training case study", 8-bit Adam, and
 * "Problem and motivation", block-wise FP8: both work on the same
 * quantisation blocks, which RaggedShard keeps inside one rank).  Every
 * output of rs_adam8_step as there (d_bf16_out nullable), and for every
 * block B of the selection the FP8 rule of rs_pack_shard_fp8 applied to the
 * new parameters theta' (the values written to d_master):
 *   d_fp8_scale[B] = max|theta'| / 448 (binary32),
 *   d_fp8[i] = E4M3 code of theta'[i] / d_fp8_scale[B] (correctly rounded
 *              quotient, ties to even, saturating; scale 0 gives code 0),
 * so the codes and scales are exactly those rs_pack_shard_fp8 gives for
 * views holding theta'.  d_fp8: one byte per buffer element (full
 * bucket-set array, 16-byte aligned); padding positions are not written
 * (rs_pack_shard_fp8 writes them 0; they stay so).  d_fp8_scale: one float
 * per global block id.  Saves the copy-in's separate read of the master
 * (4 bytes per element) and its own cross-chunk wait on split blocks.
 * Errors: as rs_adam8_step; RS_EINVAL if d_fp8 or d_fp8_scale is NULL. */
rs_status rs_adam8_step_fp8(const rs_plan* plan, int32_t bucket, int32_t rank, float* d_master,
                            const uint16_t* d_grad, int8_t* d_qm, uint8_t* d_qv,
                            float* d_amax_m, float* d_amax_v, const rs_adam_hparams* hp,
                            const float* d_grad_scale, uint16_t* d_bf16_out, uint8_t* d_fp8,
                            float* d_fp8_scale, void* stream);

/* ------------------------------------------------------- distributed Muon
 * veScale-FSDP page, section "Structure-aware training case study",
 * distributed Muon (Algorithm 2), with the uneven per-device distribution of
 * the "RaggedShard" section: SelectRoot picks one root rank per matrix for
 * load balance; the matrix's update is redistributed to RaggedShard(root),
 * the whole matrix on the root and nothing on the other ranks; the root runs
 * Newton-Schulz; the result is redistributed back and applies to the
 * parameters (the other ranks' Newton-Schulz is a no-op).  On one GPU every
 * rank's region of that uneven layout lives in one "root buffer" (bf16,
 * rs_muon_layout), next to the DBuffers of the plan.
 * This library's reading of the update (Muon with decoupled weight decay and
 * a per-matrix scale, as in large-scale Muon):
 *   M <- momentum * M + g                       (binary32, DBuffer layout)
 *   U = bf16(M)                                 (redistributed to the root)
 *   X = U / (||U||_F + 1e-7), its transpose when R > C; five times
 *   A = X X^T, B = b A + c A A, X = a X + B X   ((a, b, c) = (3.4445,
 *                                                -4.7750, 2.0315); bf16
 *                                                values, binary32 sums)
 *   O = X (transposed back)                     (redistributed back)
 *   theta <- theta (1 - lr wd) - (lr 0.2 sqrt(max(R, C))) O   (binary32)
 * SelectRoot: longest processing time first on the Newton-Schulz flops
 * 5 (4 n^2 k + 2 n^3), n = min(R, C), k = max(R, C); ties to the earlier
 * matrix and the lower rank.  Root layout: rank by rank, each rank's
 * matrices whole and back to back in the given order, every start a
 * multiple of 64 elements. */
typedef struct rs_muon rs_muon; /* opaque, host-owned */

typedef struct {
    double lr, momentum, weight_decay;
} rs_muon_hparams;

/* A Muon plan over n tensors of `plan` (indices into the plan's tensor
 * list): each is taken as its 2-D view R x C (R, C multiples of 8, buffer
 * offset a multiple of 8).  The plan is only read here; the Muon plan keeps
 * what it needs.  Host only.  Errors: RS_EINVAL (bad or repeated index, a
 * shape the kernels do not take), RS_EOVERFLOW, RS_ENOMEM. */
rs_status rs_muon_plan(const rs_plan* plan, const int32_t* tensors, int32_t n, rs_muon** out);

/* Releases a Muon plan (NULL is allowed). */
void rs_muon_free(rs_muon* muon);

/* roots[i], offsets[i]: root rank and root-buffer element offset of matrix
 * i (given order); regions[r], r = 0..m: start of rank r's region (rank r
 * holds [regions[r], regions[r + 1])); *root_elems: root-buffer length.
 * Any output pointer may be NULL. */
rs_status rs_muon_layout(const rs_muon* muon, int32_t* roots, int64_t* offsets, int64_t* regions,
                         int64_t* root_elems);

/* Device bytes of the Muon workspace: tables, per-chunk partial sums and
 * per-matrix norms, and the Newton-Schulz buffers (X, two Y, A, B per
 * matrix, bf16). */
size_t rs_muon_device_bytes(const rs_muon* muon);

/* Copies the tables into the caller's workspace (>= rs_muon_device_bytes,
 * 256-byte aligned); the Muon plan keeps the pointer.  On its first call it
 * also creates the plan's own stream and two events on the current device
 * (used by rs_muon_orthogonalize).  Synchronises the stream.  Errors:
 * RS_EINVAL, RS_ENOMEM (too small), RS_EHIP. */
rs_status rs_muon_upload(rs_muon* muon, void* d_workspace, size_t bytes, void* stream);

/* Momentum and redistribution to the roots, for the matrices of `root`
 * (RS_ALL: every root): M = momentum * M + float(g) over each matrix's
 * elements in the DBuffers d_mom (fp32) and d_grad (bf16), and
 * d_root[offset + e] = bf16(M[pos + e]).  Errors: RS_EINVAL, RS_ESTATE (not
 * uploaded), RS_EHIP. */
rs_status rs_muon_gather(const rs_muon* muon, int32_t root, float* d_mom, const uint16_t* d_grad,
                         const rs_muon_hparams* hp, uint16_t* d_root, void* stream);

/* Newton-Schulz of the matrices of `root` (RS_ALL: every root), in place in
 * the root buffer: reads U, leaves O (bf16).  Uses the workspace's buffers
 * of those matrices only: calls for different roots touch disjoint memory
 * and may run concurrently on different streams (one GPU standing in for
 * several roots); calls whose roots overlap (the same root, or RS_ALL)
 * must be stream-ordered.  With two or more matrices selected whose
 * X X^T products have fewer output tiles than two per compute unit, they run
 * as two groups of about equal cost, the second on the plan's own stream,
 * forked from `stream` and joined back to it with the plan's two events
 * (event record and wait only: the call stays capturable in a HIP graph);
 * calls on several streams at once share that stream, which orders their
 * second groups.  Errors as rs_muon_gather. */
rs_status rs_muon_orthogonalize(const rs_muon* muon, int32_t root, uint16_t* d_root, void* stream);

/* Redistribution back and the update, for the matrices of `root` (RS_ALL:
 * every root): theta[pos + e] = theta * (1 - lr wd) - (lr 0.2 sqrt(max(R,
 * C))) * float(d_root[offset + e]), in binary32 (the two scalars computed in
 * binary64 and rounded once).  d_master is the fp32 DBuffer.  Errors as
 * rs_muon_gather. */
rs_status rs_muon_apply(const rs_muon* muon, int32_t root, float* d_master, const uint16_t* d_root,
                        const rs_muon_hparams* hp, void* stream);

/* Synchronises the stream and reports a device-side failure of the
 * one-launch split modes: RS_EHIP if a bounded wait for the other chunks of
 * a block gave up since the last check, or if the caller set the status
 * word (rs_plan_status_offset); else RS_OK.  Clears the word.  While the
 * word is set, every one-launch step or FP8 copy-in updates each split block
 * whole in the workgroup of its first chunk, with no wait: results stay
 * exact, only slower.  The launch in which a wait gives up leaves the codes
 * (or FP8 codes and scale) of that wait's block unspecified. */
rs_status rs_plan_check_device(rs_plan* plan, void* stream);

/* Byte offset, inside the uploaded workspace, of the device status word (one
 * uint32, nonzero after a cooperative wait gave up).  A caller may read it
 * without synchronising, or store a nonzero value to force the wait-free
 * whole-block path of the cooperative launches.  Errors: RS_EINVAL,
 * RS_ESTATE (not uploaded). */
rs_status rs_plan_status_offset(const rs_plan* plan, size_t* byte_offset);

/* Thread-local message of the last non-OK status ("" if none). */
const char* rs_last_error(void);

/* Library version string. */
const char* rs_version(void);

#ifdef __cplusplus
}
#endif
#endif /* RAGGEDSHARD_H */
