// Distributed Muon on one GPU, for gfx950.
//
// veScale-FSDP page, section "Structure-aware training case study",
// distributed Muon (Algorithm 2): a root rank is chosen per matrix for load
// balance, the matrix's update is redistributed so that the root holds all
// of it (an uneven RaggedShard: per-rank sizes differ), Newton-Schulz runs on
// the root, and the result goes back to the sharded layout to update the
// parameters.  On one GPU every rank's slices live in the DBuffers and every
// root's region in one root buffer:
//   gather:        M <- mu M + g (binary32, in the DBuffers) and
//                  root[off + e] = bf16(M[pos + e]);
//   orthogonalize: X = U / (||U||_F + 1e-7) (or its transpose), then five
//                  quintic Newton-Schulz steps A = X X^T, B = b A + c A A,
//                  X = a X + B X as bf16 MFMA products with binary32
//                  accumulation, every stored value bf16; the result goes
//                  back into the root buffer;
//   apply:         theta <- theta (1 - lr wd) - (lr 0.2 sqrt(max(R, C))) O.
// The products are dense contractions, so they run on the matrix cores
// (v_mfma_f32_32x32x16_bf16).  Every product is written as C = P Q^T with P
// and Q read along their rows: A = X X^T and B = c A A^T + b A directly (A
// is symmetric), and the update as Y' = a Y + Y B^T on Y = X^T (B is
// symmetric), whose tiles are also stored transposed as the next X.
#include <hip/hip_runtime.h>

#include "muon.hpp"

namespace rs {
namespace mu {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bits of x, round to nearest even; NaN -> quiet NaN with its sign.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float bf16_val(uint32_t h) { return __uint_as_float(h << 16); }

// Sum over the workgroup in a fixed order (result in thread 0).
template <int NT>
__device__ __forceinline__ double wg_sum(double v, double* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0)
        for (int w = 0; w < NT / 64; ++w) s += red[w];
    return s;
}

// Index i in [i0, i1) with pre[i] <= t < pre[i + 1] (pre ascending).
__device__ __forceinline__ int find_mat(const int64_t* pre, int i0, int i1, int64_t t) {
    int lo = i0, hi = i1 - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pre[mid] <= t)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// ------------------------------------------------------------ gather

constexpr int kVT = 256;  // threads of the gather / apply kernels: 8192 = 256 x 4 x 8

__global__ __launch_bounds__(kVT) void gather_kernel(Tables t, int64_t c0, float* __restrict__ mom,
                                                     const uint16_t* __restrict__ grad, float mu,
                                                     uint16_t* __restrict__ root) {
    const MuonChunk ch = t.chunks[c0 + blockIdx.x];
    const MuonMat& m = t.mats[ch.mat];
    const int64_t pos = m.pos + ch.e0, ro = m.root_off + ch.e0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int e = (v * kVT + (int)threadIdx.x) * 8;
        if (e < ch.count) {
            const uint4 gw = *reinterpret_cast<const uint4*>(grad + pos + e);
            float4* mp = reinterpret_cast<float4*>(mom + pos + e);
            const float4 a = mp[0], b = mp[1];
            const uint32_t g2[4] = {gw.x, gw.y, gw.z, gw.w};
            float mv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float g = bf16_val((g2[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                mv[j] = (mu * mv[j]) + g;
                h[j] = bf16_bits(mv[j]);
            }
            mp[0] = make_float4(mv[0], mv[1], mv[2], mv[3]);
            mp[1] = make_float4(mv[4], mv[5], mv[6], mv[7]);
            *reinterpret_cast<uint4*>(root + ro + e) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
        }
    }
}

// ----------------------------------------------------------------- norm

// Sum of squares of one chunk of U (binary64); the scale kernel adds a
// matrix's chunk sums in a fixed order.
__global__ __launch_bounds__(kVT) void norm_kernel(Tables t, int64_t c0,
                                                   const uint16_t* __restrict__ root) {
    __shared__ double red[kVT / 64];
    const MuonChunk ch = t.chunks[c0 + blockIdx.x];
    const MuonMat& m = t.mats[ch.mat];
    const int64_t ro = m.root_off + ch.e0;
    double acc = 0.0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int e = (v * kVT + (int)threadIdx.x) * 8;
        if (e < ch.count) {
            const uint4 w = *reinterpret_cast<const uint4*>(root + ro + e);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double u = (double)bf16_val((ww[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                acc += u * u;
            }
        }
    }
    const double s = wg_sum<kVT>(acc, red);
    if (threadIdx.x == 0) t.partials[c0 + blockIdx.x] = s;
}

// Each matrix's scale s = sqrt(sum of its chunk sums) + 1e-7, once per
// matrix (one workgroup each), for the prepare kernel's tiles.
__global__ __launch_bounds__(256) void scale_kernel(Tables t, int32_t i0) {
    __shared__ double red[4];
    const int i = i0 + (int)blockIdx.x;
    const MuonMat& m = t.mats[i];
    double part = 0.0;
    for (int64_t q = threadIdx.x; q < m.gn; q += 256) part += t.partials[m.g0 + q];
    const double tot = wg_sum<256>(part, red);
    if (threadIdx.x == 0) t.norms[i] = sqrt(tot) + kNsEps;
}

// ------------------------------------------------------------- prepare

// X0 = bf16(U / s) (U's transpose when R > C) and Y0 = X0^T, one 64 x 64
// tile of U per workgroup; s from the scale kernel.
// The quotient is the binary64 one, rounded to binary32 and then to bf16.
__global__ __launch_bounds__(256) void prep_kernel(Tables t, int32_t i0, int32_t i1,
                                                   const uint16_t* __restrict__ root) {
    constexpr int T = kPrepTile;
    __shared__ uint16_t tileT[T][T + 8];
    const int64_t* pre = t.tiles;
    const int64_t tg = pre[i0] + blockIdx.x;
    const int i = find_mat(pre, i0, i1, tg);
    const MuonMat& m = t.mats[i];
    const double s = t.norms[i];
    const int64_t local = tg - pre[i];
    const int64_t tcols = (m.C + T - 1) / T;
    const int64_t r0 = (local / tcols) * T, cc0 = (local % tcols) * T;
    // straight copy: rows of U -> rows of X (R <= C) or of Y (R > C)
    uint16_t* straight = t.ws + (m.tr ? m.y0 : m.x);
    uint16_t* trans = t.ws + (m.tr ? m.x : m.y0);
    const uint16_t* u = root + m.root_off;
    for (int v = 0; v < 2; ++v) {
        const int idx = v * 256 + (int)threadIdx.x;
        const int row = idx >> 3, cv = (idx & 7) * 8;
        const int64_t r = r0 + row, c = cc0 + cv;
        if (r < m.R && c < m.C) {
            const uint4 w = *reinterpret_cast<const uint4*>(u + r * m.C + c);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            uint32_t h[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const double x = (double)bf16_val((ww[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                h[j] = bf16_bits((float)(x / s));
                tileT[cv + j][row] = (uint16_t)h[j];
            }
            *reinterpret_cast<uint4*>(straight + r * m.C + c) =
                make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                           h[6] | (h[7] << 16));
        }
    }
    __syncthreads();
    // transposed copy: column c of the tile -> row c of the transposed buffer (row length R)
    for (int v = 0; v < 2; ++v) {
        const int idx = v * 256 + (int)threadIdx.x;
        const int col = idx >> 3, rv = (idx & 7) * 8;
        const int64_t c = cc0 + col, r = r0 + rv;
        if (c < m.C && r < m.R) {
            uint32_t w[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                w[j] = (uint32_t)tileT[col][rv + 2 * j] | ((uint32_t)tileT[col][rv + 2 * j + 1] << 16);
            *reinterpret_cast<uint4*>(trans + c * m.R + r) = make_uint4(w[0], w[1], w[2], w[3]);
        }
    }
}

// ------------------------------------------------------- the products

constexpr int BM = kGemmTile, BN = kGemmTile, BK = 64, GT = 256;
constexpr int LDSR = BK + 8;  // bf16 per LDS row: 16 bytes of padding against bank conflicts

struct GemmArgs {
    Tables t;
    int32_t i0, i1;
    int32_t kind;  // G_GRAM, G_POLY, G_UPDATE
    int32_t it;    // Newton-Schulz step (selects the Y buffers)
    int32_t last;  // last step: the result goes to the root buffer
    int32_t table; // which prefix tile table (tile size) the launch counts on
    uint16_t* root;
};

// One product of a Newton-Schulz step: C = alpha P Q^T + beta R, P: M x K and
// Q: N x K read along rows; R and C: M x N; Rt = R^T (N x M, row-major) for
// kernels that read the addend by columns; Cs / Ct: where C goes straight /
// transposed (either may be null).  All bf16, leading dimensions in elements.
struct Prod {
    const uint16_t *P, *Q, *Rr, *Rt;
    uint16_t *Cs, *Ct;
    int64_t M, N, K, ldp, ldq, ldr, ldrt, ldc, ldct;
    float alpha, beta;
};

__device__ __forceinline__ Prod product_of(const GemmArgs& g, const MuonMat& md) {
    uint16_t* ws = g.t.ws;
    const int64_t yin = (g.it & 1) ? md.y1 : md.y0;
    const int64_t yout = (g.it & 1) ? md.y0 : md.y1;
    Prod p;
    p.Rr = p.Rt = nullptr;
    p.Cs = p.Ct = nullptr;
    p.ldr = p.ldrt = p.ldc = p.ldct = 0;
    p.alpha = 1.0f;
    p.beta = 0.0f;
    if (g.kind == G_GRAM) {  // A = X X^T
        p.P = p.Q = ws + md.x;
        p.ldp = p.ldq = md.k;
        p.M = p.N = md.n;
        p.K = md.k;
        p.Cs = ws + md.a;
        p.ldc = md.n;
    } else if (g.kind == G_POLY) {  // B = c A A^T + b A  (A = A^T)
        p.P = p.Q = p.Rr = p.Rt = ws + md.a;
        p.ldp = p.ldq = p.ldr = p.ldrt = md.n;
        p.M = p.N = p.K = md.n;
        p.alpha = kNsC;
        p.beta = kNsB;
        p.Cs = ws + md.b;
        p.ldc = md.n;
    } else {  // Y' = Y B^T + a Y, stored as Y' and as X' = Y'^T  (Y^T = X)
        p.P = p.Rr = ws + yin;
        p.Rt = ws + md.x;
        p.Q = ws + md.b;
        p.ldp = p.ldq = p.ldr = md.n;
        p.ldrt = md.k;
        p.M = md.k;
        p.N = p.K = md.n;
        p.beta = kNsA;
        if (!g.last) {
            p.Cs = ws + yout;
            p.ldc = md.n;
            p.Ct = ws + md.x;
            p.ldct = md.k;
        } else if (md.tr) {  // the result is Y (R x C, C = n)
            p.Cs = g.root + md.root_off;
            p.ldc = md.n;
        } else {  // the result is X (R x C, C = k)
            p.Ct = g.root + md.root_off;
            p.ldct = md.k;
        }
    }
    return p;
}

// Output tile (tm, tn) of the launch's tile `local` of a product: every tile
// of the update; for the symmetric products only tm <= tn, each tile then
// also stored transposed into the same matrix (off the diagonal).
__device__ __forceinline__ void tile_of_product(const GemmArgs& g, Prod& p, int64_t local,
                                                int64_t tile, int64_t& tm, int64_t& tn) {
    const int64_t ntn = (p.N + tile - 1) / tile;
    if (g.kind == G_UPDATE) {
        tm = local / ntn;
        tn = local % ntn;
        return;
    }
    tm = 0;
    while (local >= ntn - tm) {
        local -= ntn - tm;
        ++tm;
    }
    tn = tm + local;
    if (tn != tm) {
        p.Ct = p.Cs;
        p.ldct = p.ldc;
    }
}

// One 128 x 128 tile of C = alpha P Q^T + beta R (P: M x K, Q: N x K, R and
// C: M x N, all row-major bf16), stored straight (Cs) and/or transposed
// (Ct).  Four waves, each a 64 x 64 quarter as 2 x 2 MFMA tiles of 32 x 32;
// K in steps of 64 through two LDS buffers, the next step's global loads in
// flight while the current one is multiplied.
__global__ __launch_bounds__(GT) void ns_gemm_kernel(GemmArgs g) {
    // K loop: two buffers of the P and Q tiles; epilogue: the bf16 result
    // tile, straight and transposed
    constexpr int kStage = BM * LDSR;
    constexpr int kOutR = BN + 8;  // bf16 per row of the staged result tiles
    static_assert(2 * BM * kOutR <= 4 * kStage, "result tiles fit the K-loop buffers");
    __shared__ __attribute__((aligned(16))) uint16_t lds[4 * kStage];
    uint16_t(*sP)[kStage] = reinterpret_cast<uint16_t(*)[kStage]>(lds);
    uint16_t(*sQ)[kStage] = reinterpret_cast<uint16_t(*)[kStage]>(lds + 2 * kStage);
    const int nm = g.t.nm;
    const int64_t* pre = g.t.tiles + (int64_t)g.table * (nm + 1);
    const int64_t tg = pre[g.i0] + blockIdx.x;
    const int mi = find_mat(pre, g.i0, g.i1, tg);
    Prod pr = product_of(g, g.t.mats[mi]);
    int64_t tm, tn;
    tile_of_product(g, pr, tg - pre[mi], BM, tm, tn);
    const uint16_t *P = pr.P, *Q = pr.Q, *Rr = pr.Rr;
    uint16_t *Cs = pr.Cs, *Ct = pr.Ct;
    const int64_t M = pr.M, N = pr.N, K = pr.K, ldp = pr.ldp, ldq = pr.ldq, ldr = pr.ldr,
                  ldc = pr.ldc, ldct = pr.ldct;
    const float alpha = pr.alpha, beta = pr.beta;
    const int64_t m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int lrow = tid >> 3, lk = (tid & 7) * 8;  // this thread's global-load slots
    uint4 rp[4], rq[4];
    auto gload = [&](int64_t k0) {
        const int64_t kk = k0 + lk;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t pr = m0 + lrow + 32 * v, qr = n0 + lrow + 32 * v;
            rp[v] = (pr < M && kk < K) ? *reinterpret_cast<const uint4*>(P + pr * ldp + kk)
                                       : make_uint4(0u, 0u, 0u, 0u);
            rq[v] = (qr < N && kk < K) ? *reinterpret_cast<const uint4*>(Q + qr * ldq + kk)
                                       : make_uint4(0u, 0u, 0u, 0u);
        }
    };
    auto sstore = [&](int b) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            *reinterpret_cast<uint4*>(&sP[b][(lrow + 32 * v) * LDSR + lk]) = rp[v];
            *reinterpret_cast<uint4*>(&sQ[b][(lrow + 32 * v) * LDSR + lk]) = rq[v];
        }
    };
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    gload(0);
    sstore(0);
    __syncthreads();
    int b = 0;
    const int frow = lane & 31, fk = 8 * (lane >> 5);
    for (int64_t k0 = 0; k0 < K; k0 += BK) {
        const bool more = k0 + BK < K;
        if (more) gload(k0 + BK);
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            bf16x8 fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i)
                fa[i] = *reinterpret_cast<const bf16x8*>(
                    &sP[b][(wm * 64 + i * 32 + frow) * LDSR + kk + fk]);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                fb[j] = *reinterpret_cast<const bf16x8*>(
                    &sQ[b][(wn * 64 + j * 32 + frow) * LDSR + kk + fk]);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j],
                                                                        0, 0, 0);
        }
        if (more) sstore(b ^ 1);
        __syncthreads();
        b ^= 1;
    }
    // epilogue: lane l holds column l % 32 of a 32 x 32 tile, register r its
    // row 8 (r / 4) + 4 (l / 32) + r % 4.  The bf16 results go to LDS, straight
    // (sS[row][col]) and transposed (sT[col][row]); then whole rows of both
    // leave as 16-byte stores.  (The K loop's last barrier has freed LDS.)
    uint16_t* sS = lds;
    uint16_t* sT = lds + BM * kOutR;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int col = wn * 64 + j * 32 + (lane & 31);
                const int row0 = wm * 64 + i * 32 + 8 * q + 4 * (lane >> 5);
                const int64_t gn = n0 + col;
                uint32_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int64_t gm = m0 + row0 + r;
                    float v = alpha * acc[i][j][4 * q + r];
                    if (Rr && gm < M && gn < N) v = v + beta * bf16_val(Rr[gm * ldr + gn]);
                    h[r] = bf16_bits(v);
                    if (Cs) sS[(row0 + r) * kOutR + col] = (uint16_t)h[r];
                }
                if (Ct)
                    *reinterpret_cast<uint2*>(&sT[col * kOutR + row0]) =
                        make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
    __syncthreads();
    // M, N and the leading dimensions are multiples of 8: a 16-byte vector is
    // wholly inside or wholly outside the matrix
#pragma unroll
    for (int v = 0; v < (BM * BN / 8) / GT; ++v) {
        const int idx = v * GT + tid;
        const int row = idx >> 4, c8 = (idx & 15) * 8;
        if (Cs && m0 + row < M && n0 + c8 < N)
            *reinterpret_cast<uint4*>(Cs + (m0 + row) * ldc + n0 + c8) =
                *reinterpret_cast<const uint4*>(&sS[row * kOutR + c8]);
        if (Ct && n0 + row < N && m0 + c8 < M)
            *reinterpret_cast<uint4*>(Ct + (n0 + row) * ldct + m0 + c8) =
                *reinterpret_cast<const uint4*>(&sT[row * kOutR + c8]);
    }
}

// ------------------------------------------------ 256 x 256 products

constexpr int T2 = 256, BK2 = 64, NSTAGE = 2;
constexpr int GT2 = 512;               // eight waves: two per SIMD
constexpr int kRowsPerWave2 = T2 / (GT2 / 64);
constexpr int kStage2 = T2 * BK2;      // bf16 of one operand tile in LDS (32 KiB)
constexpr int kOutR2 = T2 + 8;         // bf16 per row of the staged result tile
static_assert(T2 * kOutR2 >= 2 * NSTAGE * kStage2, "the staged result tile covers the stages");

// s_waitcnt immediate (gfx9 encoding) that waits until at most n vector
// memory operations of the wave are outstanding, leaving the other counters.
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }

// A T2 x 64 bf16 tile (rows r0 .., k0 .. k0 + 63 of a row-major matrix) into
// LDS, straight from global memory (gfx950's 16-byte loads to LDS, no VGPR
// staging).  One instruction covers eight whole 128-byte row pieces (lane l:
// row l / 8, physical chunk l % 8): measured on this part, 128-byte pieces
// move twice the bytes per cycle of 64-byte ones.  LDS rows are 128 bytes;
// the 16-byte chunk c of row r sits at chunk c ^ ((r >> 1) & 7), so the 16
// lanes of a fragment read meet 16 different bank groups.  Wave w fills rows
// [32 w, 32 w + 32).  Rows past rmax read row rmax - 1: they only feed
// results outside the matrix, which are never stored.
__device__ __forceinline__ void tile_to_lds(const uint16_t* A, int64_t ld, int64_t r0,
                                            int64_t rmax, int64_t k0, uint16_t* dst) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int j = 0; j < kRowsPerWave2 / 8; ++j) {
        const int row = wave * kRowsPerWave2 + j * 8 + (lane >> 3);
        const int lc = (lane & 7) ^ ((row >> 1) & 7);
        int64_t gr = r0 + row;
        gr = gr < rmax ? gr : rmax - 1;
        __builtin_amdgcn_global_load_lds(A + gr * ld + k0 + lc * 8,
                                         dst + (wave * kRowsPerWave2 + j * 8) * BK2, 16, 0, 0);
    }
}

__device__ __forceinline__ bf16x8 frag2(const uint16_t* src, int row, int lc) {
    return *reinterpret_cast<const bf16x8*>(src + row * BK2 + ((lc ^ ((row >> 1) & 7)) << 3));
}

// One 256 x 256 tile of a product whose K is a multiple of 64.  Eight waves
// (two per SIMD, so one wave's LDS reads and barrier overlap the other's
// MFMAs), each a 128 x 64 part as 4 x 2 MFMA tiles (128 accumulators per
// lane); both operand tiles go straight to LDS through two stages of 64
// K-columns, the next stage's loads in flight while the current one is
// multiplied (each stage in two halves: 12 fragment reads, then 16 MFMAs).
// One workgroup per compute unit (132 KiB of LDS).
__global__ __launch_bounds__(GT2) void ns_gemm256_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) uint16_t lds[T2 * kOutR2];
    const int nm = g.t.nm;
    const int64_t* pre = g.t.tiles + (int64_t)g.table * (nm + 1);
    const int64_t tg = pre[g.i0] + blockIdx.x;
    const int mi = find_mat(pre, g.i0, g.i1, tg);
    Prod p = product_of(g, g.t.mats[mi]);
    int64_t tm, tn;
    tile_of_product(g, p, tg - pre[mi], T2, tm, tn);
    const int64_t m0 = tm * T2, n0 = tn * T2;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int TI = 4, TJ = 2;  // MFMA tiles of a wave: 128 rows x 64 columns
    const int wm = wave >> 2, wn = wave & 3;

    const int frow = lane & 31, half = lane >> 5;
    // lane l holds column l % 32 of each 32 x 32 MFMA tile, register r its
    // row 8 (r / 4) + 4 (l / 32) + r % 4: four consecutive rows per register
    // group
    auto row_of = [&](int i, int q) { return wm * 128 + i * 32 + 8 * q + 4 * half; };
    auto col_of = [&](int j) { return wn * 64 + j * 32 + frow; };
    f32x16 acc[TI][TJ];
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
    const int KT = (int)(p.K / BK2);
    auto issue = [&](int kt) {
        uint16_t* st = lds + (kt % NSTAGE) * 2 * kStage2;
        tile_to_lds(p.P, p.ldp, m0, p.M, (int64_t)kt * BK2, st);
        tile_to_lds(p.Q, p.ldq, n0, p.N, (int64_t)kt * BK2, st + kStage2);
    };
    for (int s = 0; s < NSTAGE - 1; ++s)
        if (s < KT) issue(s);
    for (int kt = 0; kt < KT; ++kt) {
        // stage kt has landed once at most the later stages' loads (8 per
        // stage per wave) are outstanding; the barrier then also tells every
        // wave that all are done reading the stage the next issue overwrites
        constexpr int kPerStage = 2 * (kRowsPerWave2 / 8);
        const int later = min(NSTAGE - 2, KT - 1 - kt);
        if (later >= 2)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPerStage));
        else if (later == 1)
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kPerStage));
        else
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        // a bare barrier (also a compiler memory fence): __syncthreads would
        // first wait for every outstanding load, the stages still in flight
        // included
        asm volatile("s_barrier" ::: "memory");
        if (kt + NSTAGE - 1 < KT) issue(kt + NSTAGE - 1);
        const uint16_t* sp = lds + (kt % NSTAGE) * 2 * kStage2;
        const uint16_t* sq = sp + kStage2;
        // each half of the stage: its 12 fragments read up front, then its 16
        // MFMAs back to back
#pragma unroll
        for (int hh = 0; hh < BK2 / 32; ++hh) {
            bf16x8 fa[2][TI], fb[2][TJ];
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
                const int lc = 2 * (2 * hh + k2) + half;
#pragma unroll
                for (int i = 0; i < TI; ++i) fa[k2][i] = frag2(sp, wm * 128 + i * 32 + frow, lc);
#pragma unroll
                for (int j = 0; j < TJ; ++j) fb[k2][j] = frag2(sq, wn * 64 + j * 32 + frow, lc);
            }
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
                for (int i = 0; i < TI; ++i)
#pragma unroll
                    for (int j = 0; j < TJ; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[k2][i], fb[k2][j],
                                                                            acc[i][j], 0, 0, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * (TI + TJ), 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 2 * TI * TJ, 0);
        }
    }
    __syncthreads();  // every wave is done with the stages: LDS is free
    // results bf16(alpha acc + beta R), stored straight and/or transposed as
    // 16-byte row pieces through an LDS tile (M, N and the leading dimensions
    // are multiples of 8).  The addend's tile (rows m0 .., columns n0 .. of
    // the row-major R) first comes into that LDS tile with coalesced 16-byte
    // row loads; each lane then replaces its own elements by the results,
    // keeping them packed for the transposed store.
    uint16_t* so = lds;
    auto tile_rows = [&](auto&& body) {
        for (int v = tid; v < T2 * (T2 / 8); v += GT2) body(v / (T2 / 8), (v % (T2 / 8)) * 8);
    };
    if (p.Rr) {
        tile_rows([&](int rr, int c8) {
            uint4 w = make_uint4(0u, 0u, 0u, 0u);
            if (m0 + rr < p.M && n0 + c8 < p.N)
                w = *reinterpret_cast<const uint4*>(p.Rr + (m0 + rr) * p.ldr + n0 + c8);
            *reinterpret_cast<uint4*>(so + rr * kOutR2 + c8) = w;
        });
        __syncthreads();
    }
    uint32_t hp[TI][TJ][4][2];  // results, bf16 pairs of rows (r, r + 1)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = row_of(i, q), col = col_of(j);
                uint32_t h[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    uint16_t* e = so + (row + r) * kOutR2 + col;
                    const float rv = p.Rr ? bf16_val(*e) : 0.0f;
                    h[r] = bf16_bits(p.alpha * acc[i][j][4 * q + r] + p.beta * rv);
                    *e = (uint16_t)h[r];
                }
                hp[i][j][q][0] = h[0] | (h[1] << 16);
                hp[i][j][q][1] = h[2] | (h[3] << 16);
            }
    __syncthreads();
    auto store_tile = [&](uint16_t* out, int64_t ra, int64_t ca, int64_t rlim, int64_t clim,
                          int64_t ld) {
        tile_rows([&](int rr, int c8) {
            if (ra + rr < rlim && ca + c8 < clim)
                *reinterpret_cast<uint4*>(out + (ra + rr) * ld + ca + c8) =
                    *reinterpret_cast<const uint4*>(so + rr * kOutR2 + c8);
        });
    };
    if (p.Cs) store_tile(p.Cs, m0, n0, p.M, p.N, p.ldc);
    if (p.Ct) {
        if (p.Cs) __syncthreads();  // the straight tile is out of LDS
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    *reinterpret_cast<uint2*>(so + col_of(j) * kOutR2 + row_of(i, q)) =
                        make_uint2(hp[i][j][q][0], hp[i][j][q][1]);
        __syncthreads();
        store_tile(p.Ct, n0, m0, p.N, p.M, p.ldct);
    }
}

// ---------------------------------------------------------------- apply

__global__ __launch_bounds__(kVT) void apply_kernel(Tables t, int64_t c0, float* __restrict__ theta,
                                                    const uint16_t* __restrict__ root, double lr02,
                                                    float c_decay) {
    const MuonChunk ch = t.chunks[c0 + blockIdx.x];
    const MuonMat& m = t.mats[ch.mat];
    const float scale = (float)(lr02 * m.sqmax);
    const int64_t pos = m.pos + ch.e0, ro = m.root_off + ch.e0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int e = (v * kVT + (int)threadIdx.x) * 8;
        if (e < ch.count) {
            const uint4 w = *reinterpret_cast<const uint4*>(root + ro + e);
            float4* tp = reinterpret_cast<float4*>(theta + pos + e);
            const float4 a = tp[0], b = tp[1];
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
            float th[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float o = bf16_val((ww[j >> 1] >> (16 * (j & 1))) & 0xffffu);
                th[j] = (th[j] * c_decay) - (scale * o);
            }
            tp[0] = make_float4(th[0], th[1], th[2], th[3]);
            tp[1] = make_float4(th[4], th[5], th[6], th[7]);
        }
    }
}

}  // namespace

hipError_t launch_gather(const Tables& t, int64_t c0, int64_t c1, float* mom, const uint16_t* grad,
                         float mu, uint16_t* root, hipStream_t s) {
    if (c1 <= c0) return hipSuccess;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)(c1 - c0)), dim3(kVT), 0, s, t, c0, mom, grad,
                       mu, root);
    return hipGetLastError();
}

hipError_t launch_orthogonalize(const Tables& t, const int64_t* host_tiles, int32_t i0, int32_t i1,
                                int64_t c0, int64_t c1, bool wide, uint16_t* root, hipStream_t s) {
    if (i1 <= i0) return hipSuccess;
    const int64_t stride = t.nm + 1;
    auto count = [&](int which) {
        return host_tiles[which * stride + i1] - host_tiles[which * stride + i0];
    };
    hipLaunchKernelGGL(norm_kernel, dim3((unsigned)(c1 - c0)), dim3(kVT), 0, s, t, c0, root);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(scale_kernel, dim3((unsigned)(i1 - i0)), dim3(256), 0, s, t, i0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_kernel, dim3((unsigned)count(0)), dim3(256), 0, s, t, i0, i1, root);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    for (int it = 0; it < kNsSteps; ++it) {
        for (int kind = G_GRAM; kind <= G_UPDATE; ++kind) {
            GemmArgs a;
            a.t = t;
            a.i0 = i0;
            a.i1 = i1;
            a.kind = kind;
            a.it = it;
            a.last = it == kNsSteps - 1;
            a.root = root;
            if (wide) {
                a.table = 4 + kind;
                hipLaunchKernelGGL(ns_gemm256_kernel, dim3((unsigned)count(4 + kind)), dim3(GT2), 0,
                                   s, a);
            } else {
                a.table = 1 + kind;
                hipLaunchKernelGGL(ns_gemm_kernel, dim3((unsigned)count(1 + kind)), dim3(GT), 0,
                                   s, a);
            }
            e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

hipError_t launch_apply(const Tables& t, int64_t c0, int64_t c1, float* theta, const uint16_t* root,
                        double lr02, float c_decay, hipStream_t s) {
    if (c1 <= c0) return hipSuccess;
    hipLaunchKernelGGL(apply_kernel, dim3((unsigned)(c1 - c0)), dim3(kVT), 0, s, t, c0, theta, root,
                       lr02, c_decay);
    return hipGetLastError();
}

}  // namespace mu
}  // namespace rs
