/*
 * Plain CPU oracle for the RaggedShard / DBuffer shard-state path.
 * TEST INFRASTRUCTURE ONLY (see oracle.h).  Slow on purpose: every loop
 * follows the definition it implements, with no blocking or fusion.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared oracle.c -lm
 * (no -ffast-math, no -march: binary32 arithmetic stays IEEE RNE).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ util */

static int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        int64_t t = a % b;
        a = b;
        b = t;
    }
    return a;
}

static int64_t lcm64(int64_t a, int64_t b) { return a / gcd64(a, b) * b; }

static int64_t roundup64(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

static int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }

/* --------------------------------------------------------- tensor derive
 * RaggedShard section: the atomic (non-shardable) unit is an element, a
 * group of rows or a 2-D block.  A row-major tensor is viewed as [R, C] with
 * C its last dimension (a 1-D tensor is [d0, 1]; leading dimensions of a
 * 3-D fused-expert tensor fold into R).  Following the LCM rule for
 * sharding along a dimension > 0, a block that spans whole rows (ROWS) or a
 * band of rows (TILE, whose tiles of one band interleave in memory) can only
 * be cut between bands, so the cut unit is k*C (ROWS) or br*C (TILE).  The
 * planning section aligns each offset to lcm(g_coll, block size), with the
 * block size read as the element count of one clipped block. */
int orc_derive(const orc_tensor* t, int64_t g_coll, orc_derived* d) {
    if (!t || !d || g_coll < 1) return -1;
    if (t->ndim < 1 || t->ndim > 4) return -1;
    int64_t N = 1;
    for (int i = 0; i < t->ndim; ++i) {
        if (t->shape[i] < 1) return -1;
        if (N > (((int64_t)1) << 50) / t->shape[i]) return -1;
        N *= t->shape[i];
    }
    int64_t C = (t->ndim >= 2) ? t->shape[t->ndim - 1] : 1;
    int64_t R = N / C;
    d->N = N;
    d->R = R;
    d->C = C;
    switch (t->gran) {
    case ORC_ELEMENT:
        d->u = 1;
        d->b = 1;
        d->nblk = N;
        break;
    case ORC_ROWS:
        if (t->br < 1) return -1;
        d->u = (int64_t)t->br * C;
        d->b = min64(t->br, R) * C;
        d->nblk = (R + t->br - 1) / t->br;
        break;
    case ORC_TILE:
        if (t->br < 2 || t->bc < 1) return -1;
        d->u = (int64_t)t->br * C;
        d->b = min64(t->br, R) * min64(t->bc, C);
        d->nblk = ((R + t->br - 1) / t->br) * ((C + t->bc - 1) / t->bc);
        break;
    default:
        return -1;
    }
    d->A = lcm64(g_coll, t->align_unit ? d->u : d->b);
    return 0;
}

/* Non-Sharded Block for one tensor at offset o: every rank boundary j*S
 * (j = 1..m-1) strictly inside [o, o+N) lies a whole number of cut units
 * after the tensor start. */
static int no_split_at(const orc_derived* d, int m, int64_t S, int64_t o) {
    for (int j = 1; j < m; ++j) {
        int64_t cut = (int64_t)j * S;
        if (cut > o && cut < o + d->N && (cut - o) % d->u != 0) return 0;
    }
    return 1;
}

/* Greedy placement for a fixed S.  Tensors keep the given order (the
 * planning section: production uses the default order).  For a fixed S the
 * admissible offsets of a tensor depend only on the end e of the previous
 * tensor, and a smaller e never removes an admissible offset, so placing
 * every tensor at its earliest admissible offset finds a placement whenever
 * one exists, and that placement is the lexicographically smallest one. */
int orc_place_fixed_S(const orc_derived* d, int n, int m, int64_t g_coll, int64_t S,
                      int64_t* off) {
    (void)g_coll;
    int64_t cap = (int64_t)m * S;
    int64_t e = 0;
    for (int t = 0; t < n; ++t) {
        int64_t o = roundup64(e, d[t].A);
        for (;;) {
            if (o + d[t].N > cap) return 0;
            if (no_split_at(&d[t], m, S, o)) break;
            o += d[t].A;
        }
        off[t] = o;
        e = o + d[t].N;
    }
    return 1;
}

/* A tensor longer than 2S holds two consecutive rank boundaries j*S and
 * (j+1)*S wherever it sits inside [0, m*S]; both must fall on cut units, so
 * S itself must be a multiple of u.  An S that fails this for some tensor is
 * infeasible without running the greedy. */
static int passes_wide_tensor_test(const orc_derived* d, int n, int64_t S) {
    for (int t = 0; t < n; ++t)
        if (d[t].N > 2 * S && S % d[t].u != 0) return 0;
    return 1;
}

static int64_t balanced_lower_bound(const orc_derived* d, int n, int m, int64_t g_coll) {
    int64_t total = 0;
    for (int t = 0; t < n; ++t) total += d[t].N;
    return roundup64((total + m - 1) / m, g_coll);
}

/* S at which everything fits inside rank 0 (no boundary inside any tensor):
 * the greedy always succeeds there, so the scan below ends. */
static int64_t all_in_rank0_S(const orc_derived* d, int n, int64_t g_coll) {
    int64_t e = 0;
    for (int t = 0; t < n; ++t) e = roundup64(e, d[t].A) + d[t].N;
    return roundup64(e, g_coll);
}

/* The layout problem of the planning section: the minimal uniform per-rank
 * size S (a multiple of g_coll, since slices are collective units) for which
 * the tensors, in the given order, can be placed without a split block,
 * without padding inside a tensor, and inside m equal slices.  Scans S
 * upward from the balanced lower bound; feasibility is not monotone in S,
 * so the scan does not bisect. */
int orc_plan_bucket(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t* S_out,
                    int64_t* off_out) {
    if (n < 1 || m < 1 || g_coll < 1) return -1;
    orc_derived* d = (orc_derived*)calloc((size_t)n, sizeof(orc_derived));
    if (!d) return -1;
    for (int t = 0; t < n; ++t)
        if (orc_derive(&ts[t], g_coll, &d[t])) {
            free(d);
            return -1;
        }
    int64_t S0 = balanced_lower_bound(d, n, m, g_coll);
    int64_t Smax = all_in_rank0_S(d, n, g_coll);
    int rc = -1;
    for (int64_t S = S0; S <= Smax; S += g_coll) {
        if (!passes_wide_tensor_test(d, n, S)) continue;
        if (orc_place_fixed_S(d, n, m, g_coll, S, off_out)) {
            *S_out = S;
            rc = 0;
            break;
        }
    }
    free(d);
    return rc;
}

/* ------------------------------------------------------------ brute force */

typedef struct {
    const orc_derived* d;
    int n, m;
    int64_t S;
    int64_t* cur;
} bf_ctx;

/* Depth-first over every offset of tensor t (ascending, multiples of A_t,
 * after the previous tensor), checking the constraints of tensor t; the
 * first complete tuple found is the lexicographic minimum. */
static int bf_rec(bf_ctx* c, int t, int64_t e) {
    if (t == c->n) return 1;
    const orc_derived* d = &c->d[t];
    int64_t cap = (int64_t)c->m * c->S;
    for (int64_t o = 0; o + d->N <= cap; o += d->A) {
        if (o < e) continue;
        if (!no_split_at(d, c->m, c->S, o)) continue;
        c->cur[t] = o;
        if (bf_rec(c, t + 1, o + d->N)) return 1;
    }
    return 0;
}

int orc_plan_bruteforce(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S_cap,
                        int64_t* S_out, int64_t* off_out) {
    if (n < 1 || n > 16 || m < 1 || g_coll < 1) return -1;
    orc_derived d[16];
    for (int t = 0; t < n; ++t)
        if (orc_derive(&ts[t], g_coll, &d[t])) return -1;
    int64_t total = 0;
    for (int t = 0; t < n; ++t) total += d[t].N;
    /* every slice holds at most S elements: S >= ceil(total / m) */
    int64_t S0 = roundup64((total + m - 1) / m, g_coll);
    for (int64_t S = S0; S <= S_cap; S += g_coll) {
        bf_ctx c = {d, n, m, S, off_out};
        if (bf_rec(&c, 0, 0)) {
            *S_out = S;
            return 0;
        }
    }
    return -1;
}

int orc_bruteforce_feasible_at(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S,
                               int64_t* off_out) {
    if (n < 1 || n > 16 || m < 1 || g_coll < 1 || S < 1) return -1;
    orc_derived d[16];
    for (int t = 0; t < n; ++t)
        if (orc_derive(&ts[t], g_coll, &d[t])) return -1;
    bf_ctx c = {d, n, m, S, off_out};
    return bf_rec(&c, 0, 0);
}

int orc_wide_tensor_ok(const orc_tensor* ts, int n, int64_t g_coll, int64_t S) {
    if (n < 1 || g_coll < 1 || S < 1) return -1;
    orc_derived* d = (orc_derived*)calloc((size_t)n, sizeof(orc_derived));
    if (!d) return -1;
    int rc = 1;
    for (int t = 0; t < n; ++t)
        if (orc_derive(&ts[t], g_coll, &d[t])) rc = -1;
    if (rc == 1) rc = passes_wide_tensor_test(d, n, S);
    free(d);
    return rc;
}

/* ------------------------------------------------------------- invariants */

int64_t orc_block_positions(const orc_tensor* t, int64_t p0, int64_t k, int64_t* out,
                            int64_t cap) {
    orc_derived d;
    if (orc_derive(t, 1, &d)) return -1;
    int64_t cnt = 0;
    if (t->gran == ORC_ELEMENT) {
        if (cap > 0) out[0] = p0 + k;
        return 1;
    }
    if (t->gran == ORC_ROWS) {
        int64_t r0 = k * t->br, r1 = min64(r0 + t->br, d.R);
        for (int64_t p = p0 + r0 * d.C; p < p0 + r1 * d.C; ++p) {
            if (cnt < cap) out[cnt] = p;
            ++cnt;
        }
        return cnt;
    }
    int64_t nbc = (d.C + t->bc - 1) / t->bc;
    int64_t i = k / nbc, j = k % nbc;
    int64_t r0 = i * t->br, r1 = min64(r0 + t->br, d.R);
    int64_t c0 = j * t->bc, c1 = min64(c0 + t->bc, d.C);
    for (int64_t r = r0; r < r1; ++r)
        for (int64_t col = c0; col < c1; ++col) {
            if (cnt < cap) out[cnt] = p0 + r * d.C + col;
            ++cnt;
        }
    return cnt;
}

/* First and last buffer position of block k (positions grow with the
 * element order inside a block). */
static void block_extent(const orc_tensor* t, const orc_derived* d, int64_t p0, int64_t k,
                         int64_t* lo, int64_t* hi) {
    if (t->gran == ORC_ELEMENT) {
        *lo = *hi = p0 + k;
    } else if (t->gran == ORC_ROWS) {
        int64_t r0 = k * t->br, r1 = min64(r0 + t->br, d->R);
        *lo = p0 + r0 * d->C;
        *hi = p0 + r1 * d->C - 1;
    } else {
        int64_t nbc = (d->C + t->bc - 1) / t->bc;
        int64_t i = k / nbc, j = k % nbc;
        int64_t r0 = i * t->br, r1 = min64(r0 + t->br, d->R);
        int64_t c0 = j * t->bc, c1 = min64(c0 + t->bc, d->C);
        *lo = p0 + r0 * d->C + c0;
        *hi = p0 + (r1 - 1) * d->C + (c1 - 1);
    }
}

int64_t orc_count_cut_blocks(const orc_tensor* ts, int n, int64_t S, const int64_t* off) {
    if (!ts || !off || n < 0 || S <= 0) return -1;
    int64_t cut = 0;
    for (int t = 0; t < n; ++t) {
        orc_derived d;
        if (orc_derive(&ts[t], 1, &d)) return -1;
        if (ts[t].gran == ORC_ELEMENT) continue;
        for (int64_t k = 0; k < d.nblk; ++k) {
            int64_t lo, hi;
            block_extent(&ts[t], &d, off[t], k, &lo, &hi);
            if (lo / S != hi / S) ++cut;
        }
    }
    return cut;
}

int orc_check_plan(const orc_tensor* ts, int n, int m, int64_t g_coll, int64_t S,
                   const int64_t* off) {
    orc_derived* d = (orc_derived*)calloc((size_t)n, sizeof(orc_derived));
    if (!d) return -1;
    int bad = 0;
    for (int t = 0; t < n; ++t)
        if (orc_derive(&ts[t], g_coll, &d[t])) bad = -1;
    /* I4: alignment */
    if (!bad && (S <= 0 || S % g_coll != 0)) bad = 4;
    for (int t = 0; !bad && t < n; ++t)
        if (off[t] < 0 || off[t] % d[t].A != 0) bad = 4;
    /* I2: in order, disjoint, each tensor one contiguous range */
    for (int t = 0; !bad && t + 1 < n; ++t)
        if (off[t + 1] < off[t] + d[t].N) bad = 2;
    /* I3: everything inside the m equal slices */
    if (!bad && off[n - 1] + d[n - 1].N > (int64_t)m * S) bad = 3;
    /* I1: no block has elements in two ranks (rank = position / S grows
     * with position, so the block's two extreme positions decide) */
    for (int t = 0; !bad && t < n; ++t) {
        if (ts[t].gran == ORC_ELEMENT) continue;
        for (int64_t k = 0; k < d[t].nblk; ++k) {
            int64_t lo, hi;
            block_extent(&ts[t], &d[t], off[t], k, &lo, &hi);
            if (lo / S != hi / S) {
                bad = 1;
                break;
            }
        }
    }
    /* I5: minimality -- every smaller candidate S is infeasible */
    if (!bad) {
        int64_t* tmp = (int64_t*)calloc((size_t)n, sizeof(int64_t));
        int64_t S0 = balanced_lower_bound(d, n, m, g_coll);
        for (int64_t Sp = S0; Sp < S; Sp += g_coll) {
            if (passes_wide_tensor_test(d, n, Sp) &&
                orc_place_fixed_S(d, n, m, g_coll, Sp, tmp)) {
                bad = 5;
                break;
            }
        }
        free(tmp);
    }
    free(d);
    return bad;
}

/* ------------------------------------------------------------------ bf16 */

uint16_t orc_bf16(float x) {
    uint32_t bits;
    memcpy(&bits, &x, 4);
    if ((bits & 0x7fffffffu) > 0x7f800000u) return (uint16_t)(((bits >> 16) & 0x8000u) | 0x7fc0u);
    uint32_t lsb = (bits >> 16) & 1u;
    return (uint16_t)((bits + 0x7fffu + lsb) >> 16);
}

float orc_bf16_to_f32(uint16_t h) {
    uint32_t bits = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

void orc_bf16_array(const float* x, uint16_t* y, int64_t n) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_bf16(x[i]);
}

/* ------------------------------------------------------- slice selection */

/* Calls fn(lo, hi) for each selected slice range in bucket, rank order. */
typedef void (*range_fn)(int64_t lo, int64_t hi, void* ctx);

static void for_each_range(const orc_layout* L, int bucket, int rank, range_fn fn, void* ctx) {
    for (int k = 0; k < L->nb; ++k) {
        if (bucket >= 0 && k != bucket) continue;
        if (rank < 0) {
            fn(L->base[k], L->base[k] + (int64_t)L->m * L->S[k], ctx);
        } else {
            fn(L->base[k] + (int64_t)rank * L->S[k], L->base[k] + (int64_t)(rank + 1) * L->S[k], ctx);
        }
    }
}

/* ------------------------------------------------------------ pack/unpack */

typedef struct {
    uint16_t* buf;
} zero16_ctx;

static void zero16(int64_t lo, int64_t hi, void* vctx) {
    zero16_ctx* c = (zero16_ctx*)vctx;
    for (int64_t p = lo; p < hi; ++p) c->buf[p] = 0;
}

static int in_selection(const orc_layout* L, int bucket, int rank, int k, int64_t p) {
    if (bucket >= 0 && k != bucket) return 0;
    if (rank < 0) return 1;
    int64_t lo = L->base[k] + (int64_t)rank * L->S[k];
    return p >= lo && p < lo + L->S[k];
}

/* DBuffer copy-in: the selected slices of the bf16 buffer receive the
 * bf16-rounded fp32 values of the tensors placed there, and zeros in the
 * padding between tensors. */
void orc_pack(const orc_layout* L, int bucket, int rank, const float* const* views,
              uint16_t* buf) {
    zero16_ctx zc = {buf};
    for_each_range(L, bucket, rank, zero16, &zc);
    for (int t = 0; t < L->n; ++t) {
        int k = L->bucket_of[t];
        if (bucket >= 0 && k != bucket) continue;
        orc_derived d;
        orc_derive(&L->spec[t], L->g_coll, &d);
        for (int64_t i = 0; i < d.N; ++i) {
            int64_t p = L->pos[t] + i;
            if (in_selection(L, bucket, rank, k, p)) buf[p] = orc_bf16(views[t][i]);
        }
    }
}

/* DBuffer copy-out: every tensor of the selected buckets receives its
 * contiguous range of the gathered buffer. */
void orc_unpack(const orc_layout* L, int bucket, uint16_t* const* views, const uint16_t* buf) {
    for (int t = 0; t < L->n; ++t) {
        if (bucket >= 0 && L->bucket_of[t] != bucket) continue;
        orc_derived d;
        orc_derive(&L->spec[t], L->g_coll, &d);
        for (int64_t i = 0; i < d.N; ++i) views[t][i] = buf[L->pos[t] + i];
    }
}

/* -------------------------------------------------------------- group ops */

typedef struct {
    void* buf;
    int dtype;
    float s;
    double acc;
} group_ctx;

static void zero_range(int64_t lo, int64_t hi, void* vctx) {
    group_ctx* c = (group_ctx*)vctx;
    for (int64_t p = lo; p < hi; ++p) {
        if (c->dtype == 0)
            ((float*)c->buf)[p] = 0.0f;
        else
            ((uint16_t*)c->buf)[p] = 0;
    }
}

static void scale_range(int64_t lo, int64_t hi, void* vctx) {
    group_ctx* c = (group_ctx*)vctx;
    for (int64_t p = lo; p < hi; ++p) {
        if (c->dtype == 0) {
            float* f = (float*)c->buf;
            f[p] = f[p] * c->s;
        } else {
            uint16_t* h = (uint16_t*)c->buf;
            h[p] = orc_bf16(orc_bf16_to_f32(h[p]) * c->s);
        }
    }
}

static void sumsq_range(int64_t lo, int64_t hi, void* vctx) {
    group_ctx* c = (group_ctx*)vctx;
    for (int64_t p = lo; p < hi; ++p) {
        double x = (c->dtype == 0) ? (double)((const float*)c->buf)[p]
                                   : (double)orc_bf16_to_f32(((const uint16_t*)c->buf)[p]);
        c->acc += x * x;
    }
}

void orc_group_zero(const orc_layout* L, int bucket, int rank, void* buf, int dtype) {
    group_ctx c = {buf, dtype, 0.0f, 0.0};
    for_each_range(L, bucket, rank, zero_range, &c);
}

void orc_group_scale(const orc_layout* L, int bucket, int rank, void* buf, int dtype, float s) {
    group_ctx c = {buf, dtype, s, 0.0};
    for_each_range(L, bucket, rank, scale_range, &c);
}

double orc_group_sumsq(const orc_layout* L, int bucket, int rank, const void* buf, int dtype) {
    group_ctx c = {(void*)buf, dtype, 0.0f, 0.0};
    for_each_range(L, bucket, rank, sumsq_range, &c);
    return c.acc;
}

float orc_clip_coef(double sumsq, double max_norm) {
    double norm = sqrt(sumsq);
    double c = max_norm / (norm + 1e-6);
    if (c > 1.0) c = 1.0;
    return (float)c;
}

/* --------------------------------------------------------- int8 AdamW */

void orc_scalars_from(const orc_hparams* h, orc_scalars* s) {
    double t = (double)h->step;
    s->beta1 = (float)h->beta1;
    s->beta2 = (float)h->beta2;
    s->omega1 = (float)(1.0 - h->beta1);
    s->omega2 = (float)(1.0 - h->beta2);
    s->eps = (float)h->eps;
    s->c_decay = (float)(1.0 - h->lr * h->weight_decay);
    s->step_size = (float)(h->lr / (1.0 - pow(h->beta1, t)));
    s->kappa = (float)(1.0 / sqrt(1.0 - pow(h->beta2, t)));
}

static float dequant_m(int8_t q) { return (float)q / 127.0f; }
static float dequant_v(uint8_t q) { return (float)q / 255.0f; }

static int8_t quant_m(float x, float a) {
    if (a == 0.0f) return 0;
    float r = rintf((x / a) * 127.0f);
    if (!(r == r)) return 0;
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

static uint8_t quant_v(float x, float a) {
    if (a == 0.0f) return 0;
    float r = rintf((x / a) * 255.0f);
    if (!(r == r)) return 0;
    if (r > 255.0f) r = 255.0f;
    if (r < 0.0f) r = 0.0f;
    return (uint8_t)r;
}

/* The 8-bit Adam case study: one block, quantised on its own.
 *  1. dequantise the stored moments with the block's old absmax,
 *  2. AdamW in binary32 (fixed operation order below),
 *  3. new absmax = max |m|, max v over the block,
 *  4. requantise m to int8 (127 levels) and v to uint8 (255 levels). */
void orc_adam8_block(int64_t n, float* theta, const uint16_t* grad, int8_t* qm, uint8_t* qv,
                     float* am, float* av, const orc_scalars* sc, float gscale,
                     uint16_t* out) {
    float* M = (float*)malloc((size_t)n * sizeof(float));
    float* V = (float*)malloc((size_t)n * sizeof(float));
    float a_m = *am, a_v = *av;
    float new_am = 0.0f, new_av = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float g = orc_bf16_to_f32(grad[i]) * gscale;
        float mh = dequant_m(qm[i]) * a_m;
        float vh = dequant_v(qv[i]) * a_v;
        float m = (sc->beta1 * mh) + (sc->omega1 * g);
        float v = (sc->beta2 * vh) + (sc->omega2 * (g * g));
        float th = theta[i] * sc->c_decay;
        float den = (sqrtf(v) * sc->kappa) + sc->eps;
        th = th - (sc->step_size * (m / den));
        theta[i] = th;
        if (out) out[i] = orc_bf16(th);
        M[i] = m;
        V[i] = v;
        if (fabsf(m) > new_am) new_am = fabsf(m);
        if (v > new_av) new_av = v;
    }
    for (int64_t i = 0; i < n; ++i) {
        qm[i] = quant_m(M[i], new_am);
        qv[i] = quant_v(V[i], new_av);
    }
    *am = new_am;
    *av = new_av;
    free(M);
    free(V);
}

void orc_adam8_step(const orc_layout* L, int bucket, int rank, float* theta,
                    const uint16_t* grad, int8_t* qm, uint8_t* qv, float* amax_m,
                    float* amax_v, const orc_hparams* h, float gscale, uint16_t* out) {
    orc_scalars sc;
    orc_scalars_from(h, &sc);
    for (int t = 0; t < L->n; ++t) {
        int k = L->bucket_of[t];
        if (bucket >= 0 && k != bucket) continue;
        orc_derived d;
        orc_derive(&L->spec[t], L->g_coll, &d);
        int64_t cap = d.b;
        int64_t* P = (int64_t*)malloc((size_t)cap * sizeof(int64_t));
        float* th = (float*)malloc((size_t)cap * sizeof(float));
        uint16_t* g = (uint16_t*)malloc((size_t)cap * sizeof(uint16_t));
        int8_t* m = (int8_t*)malloc((size_t)cap);
        uint8_t* v = (uint8_t*)malloc((size_t)cap);
        uint16_t* o = (uint16_t*)malloc((size_t)cap * sizeof(uint16_t));
        for (int64_t blk = 0; blk < d.nblk; ++blk) {
            int64_t cnt = orc_block_positions(&L->spec[t], L->pos[t], blk, P, cap);
            /* a block lies inside one rank; its first element decides */
            if (!in_selection(L, bucket, rank, k, P[0])) continue;
            for (int64_t i = 0; i < cnt; ++i) {
                th[i] = theta[P[i]];
                g[i] = grad[P[i]];
                m[i] = qm[P[i]];
                v[i] = qv[P[i]];
            }
            int64_t id = L->blk0[t] + blk;
            orc_adam8_block(cnt, th, g, m, v, &amax_m[id], &amax_v[id], &sc, gscale,
                            out ? o : NULL);
            for (int64_t i = 0; i < cnt; ++i) {
                theta[P[i]] = th[i];
                qm[P[i]] = m[i];
                qv[P[i]] = v[i];
                if (out) out[P[i]] = o[i];
            }
        }
        free(P);
        free(th);
        free(g);
        free(m);
        free(v);
        free(o);
    }
}

/* ------------------------------------------------------------ FP8 copy-in */

/* Value of an OCP E4M3 code: exponent field e (bias 7), mantissa m (3
 * bits); e = 0 encodes m * 2^-9; 0x7f / 0xff are NaN. */
static double e4m3_value(int code) {
    int e = (code >> 3) & 0xf, m = code & 7;
    double v = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -v : v;
}

float orc_e4m3_to_f32(uint8_t q) {
    if ((q & 0x7f) == 0x7f) return NAN;
    return (float)e4m3_value(q);
}

/* Nearest code by search over the 127 finite non-negative values (codes
 * 0x00..0x7e, increasing with the code), ties to the even code. */
uint8_t orc_e4m3(float x) {
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    if (isnan(x)) return (uint8_t)(sign | 0x7f);
    double a = fabs((double)x);
    if (a >= 448.0) return (uint8_t)(sign | 0x7e);
    int lo = 0;
    while (lo + 1 <= 0x7e && e4m3_value(lo + 1) <= a) ++lo; /* largest code with value <= a */
    int best = lo;
    if (lo < 0x7e) {
        double dl = a - e4m3_value(lo), dh = e4m3_value(lo + 1) - a;
        if (dh < dl || (dh == dl && ((lo + 1) & 1) == 0)) best = lo + 1;
    }
    return (uint8_t)(sign | best);
}

/* The block rule: s = absmax / 448, codes of x / s (0 when s == 0). */
float orc_fp8_block(int64_t n, const float* x, uint8_t* codes) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float s = amax / 448.0f;
    for (int64_t i = 0; i < n; ++i) codes[i] = (s == 0.0f) ? 0 : orc_e4m3(x[i] / s);
    return s;
}

void orc_pack_fp8(const orc_layout* L, int bucket, int rank, const float* const* views,
                  uint8_t* buf, float* scales) {
    /* padding of the selected slices: 0 */
    for (int k = 0; k < L->nb; ++k) {
        if (bucket >= 0 && k != bucket) continue;
        for (int r = 0; r < L->m; ++r) {
            if (rank >= 0 && r != rank) continue;
            int64_t lo = L->base[k] + (int64_t)r * L->S[k];
            for (int64_t p = lo; p < lo + L->S[k]; ++p) buf[p] = 0;
        }
    }
    for (int t = 0; t < L->n; ++t) {
        int k = L->bucket_of[t];
        if (bucket >= 0 && k != bucket) continue;
        orc_derived d;
        orc_derive(&L->spec[t], L->g_coll, &d);
        int64_t* P = (int64_t*)malloc((size_t)d.b * sizeof(int64_t));
        for (int64_t blk = 0; blk < d.nblk; ++blk) {
            int64_t cnt = orc_block_positions(&L->spec[t], L->pos[t], blk, P, d.b);
            if (!in_selection(L, bucket, rank, k, P[0])) continue;
            float* x = (float*)malloc((size_t)cnt * sizeof(float));
            uint8_t* q = (uint8_t*)malloc((size_t)cnt);
            for (int64_t i = 0; i < cnt; ++i) x[i] = views[t][P[i] - L->pos[t]];
            scales[L->blk0[t] + blk] = orc_fp8_block(cnt, x, q);
            for (int64_t i = 0; i < cnt; ++i) buf[P[i]] = q[i];
            free(x);
            free(q);
        }
        free(P);
    }
}

void orc_unpack_fp8(const orc_layout* L, int bucket, uint16_t* const* views, const uint8_t* buf,
                    const float* scales) {
    for (int t = 0; t < L->n; ++t) {
        if (bucket >= 0 && L->bucket_of[t] != bucket) continue;
        orc_derived d;
        orc_derive(&L->spec[t], L->g_coll, &d);
        int64_t* P = (int64_t*)malloc((size_t)d.b * sizeof(int64_t));
        for (int64_t blk = 0; blk < d.nblk; ++blk) {
            int64_t cnt = orc_block_positions(&L->spec[t], L->pos[t], blk, P, d.b);
            float s = scales[L->blk0[t] + blk];
            for (int64_t i = 0; i < cnt; ++i)
                views[t][P[i] - L->pos[t]] = orc_bf16(orc_e4m3_to_f32(buf[P[i]]) * s);
        }
        free(P);
    }
}
