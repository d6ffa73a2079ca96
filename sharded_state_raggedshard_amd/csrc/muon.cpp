// Distributed Muon on one GPU: the host plan (SelectRoot, the uneven root
// layout, work tables) and its C-ABI entry points.
//
// veScale-FSDP page, section "Structure-aware training case study",
// distributed Muon (Algorithm 2), and section "RaggedShard" (a device may
// hold any number of blocks, none included: the uneven distribution the root
// gather needs).  SelectRoot is read as longest-processing-time balancing of
// the Newton-Schulz cost, 5 (4 n^2 k + 2 n^3) flops for an n x k matrix
// (n <= k): matrices by decreasing cost (ties: given order), each to the rank
// with the least cost so far (ties: lowest rank).
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <new>
#include <string>
#include <vector>

#include "muon.hpp"
#include "plan.hpp"
#include "raggedshard.h"

struct rs_muon {
    int32_t m = 0;
    int32_t n_given = 0;
    std::vector<rs::mu::MuonMat> mats;  // sorted by (root, given order)
    std::vector<int32_t> slot_of;       // given index -> index in mats
    std::vector<rs::mu::MuonChunk> chunks;
    std::vector<int64_t> tiles;         // 7 prefix tile tables (see rs::mu::Tables)
    std::vector<int64_t> region;        // m + 1 region starts in the root buffer
    std::vector<int32_t> first;         // m + 1: matrices of root r are [first[r], first[r + 1])
    int64_t root_elems = 0;
    size_t off_mats = 0, off_chunks = 0, off_tiles = 0, off_partials = 0, off_ns = 0, ws_bytes = 0;
    void* d_ws = nullptr;
    bool uploaded = false;
    // a second stream for Newton-Schulz (two groups of matrices at once) and
    // the events that fork it from and join it back to the caller's stream
    hipStream_t aux = nullptr;
    hipEvent_t ev_fork = nullptr, ev_join = nullptr;
    int32_t n_cu = 0;  // compute units of the device (at upload)
    ~rs_muon() {
        if (ev_join) (void)hipEventDestroy(ev_join);
        if (ev_fork) (void)hipEventDestroy(ev_fork);
        if (aux) (void)hipStreamDestroy(aux);
    }
};

namespace {

rs_status fail(rs_status st, std::string msg) { return rs::set_error(st, std::move(msg)); }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

double ns_cost(int64_t R, int64_t C) {
    const double n = (double)std::min(R, C), k = (double)std::max(R, C);
    return 5.0 * (4.0 * n * n * k + 2.0 * n * n * n);
}

rs::mu::Tables device_tables(const rs_muon& M) {
    char* w = static_cast<char*>(M.d_ws);
    rs::mu::Tables t;
    t.mats = reinterpret_cast<const rs::mu::MuonMat*>(w + M.off_mats);
    t.chunks = reinterpret_cast<const rs::mu::MuonChunk*>(w + M.off_chunks);
    t.tiles = reinterpret_cast<const int64_t*>(w + M.off_tiles);
    t.partials = reinterpret_cast<double*>(w + M.off_partials);
    t.norms = t.partials + M.chunks.size();
    t.ws = reinterpret_cast<uint16_t*>(w + M.off_ns);
    t.nm = (int32_t)M.mats.size();
    return t;
}

// Matrices [i0, i1) and chunks [c0, c1) of one root (or of all).
rs_status select(const rs_muon& M, int32_t root, int32_t& i0, int32_t& i1, int64_t& c0,
                 int64_t& c1) {
    if (root != RS_ALL && (root < 0 || root >= M.m)) return fail(RS_EINVAL, "root out of range");
    i0 = root == RS_ALL ? 0 : M.first[root];
    i1 = root == RS_ALL ? (int32_t)M.mats.size() : M.first[root + 1];
    c0 = i1 > i0 ? M.mats[i0].g0 : 0;
    c1 = i1 > i0 ? M.mats[i1 - 1].g0 + M.mats[i1 - 1].gn : 0;
    return RS_OK;
}

}  // namespace

extern "C" {

rs_status rs_muon_plan(const rs_plan* plan, const int32_t* tensors, int32_t n, rs_muon** out) {
    using namespace rs::mu;
    if (!plan || !tensors || !out) return fail(RS_EINVAL, "NULL argument");
    *out = nullptr;
    const rs::Plan& p = plan->p;
    if (n < 1) return fail(RS_EINVAL, "no Muon matrices");
    try {
        rs_muon* M = new rs_muon;
        M->m = p.m;
        M->n_given = n;
        std::vector<char> seen(p.t.size(), 0);
        std::vector<MuonMat> given(static_cast<size_t>(n));
        for (int32_t i = 0; i < n; ++i) {
            const int32_t ti = tensors[i];
            if (ti < 0 || ti >= (int32_t)p.t.size() || seen[size_t(ti)]) {
                delete M;
                return fail(RS_EINVAL, "tensor index out of range or repeated");
            }
            seen[size_t(ti)] = 1;
            const rs::TensorInfo& t = p.t[size_t(ti)];
            if (t.R < 8 || t.C < 8 || t.R % 8 != 0 || t.C % 8 != 0 || t.pos % 8 != 0) {
                delete M;
                return fail(RS_EINVAL, "tensor " + std::to_string(ti) +
                                           ": a Muon matrix needs both dimensions of its 2-D view "
                                           "multiples of 8 and a buffer offset that is one too");
            }
            MuonMat& mm = given[size_t(i)];
            mm = MuonMat{};
            mm.R = t.R;
            mm.C = t.C;
            mm.n = std::min(t.R, t.C);
            mm.k = std::max(t.R, t.C);
            mm.pos = t.pos;
            mm.tr = t.R > t.C ? 1 : 0;
            mm.sqmax = std::sqrt((double)mm.k);
        }
        // SelectRoot: longest processing time first
        std::vector<int32_t> order(static_cast<size_t>(n));
        for (int32_t i = 0; i < n; ++i) order[size_t(i)] = i;
        std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) {
            return ns_cost(given[a].R, given[a].C) > ns_cost(given[b].R, given[b].C);
        });
        std::vector<double> load(size_t(p.m), 0.0);
        for (int32_t i : order) {
            int32_t r = 0;
            for (int32_t j = 1; j < p.m; ++j)
                if (load[size_t(j)] < load[size_t(r)]) r = j;
            given[size_t(i)].root = r;
            load[size_t(r)] += ns_cost(given[i].R, given[i].C);
        }
        // the uneven root layout: rank by rank, each rank's matrices in the given order
        M->slot_of.assign(size_t(n), 0);
        M->region.assign(size_t(p.m) + 1, 0);
        M->first.assign(size_t(p.m) + 1, 0);
        int64_t off = 0;
        for (int32_t r = 0; r < p.m; ++r) {
            M->region[size_t(r)] = off;
            M->first[size_t(r)] = (int32_t)M->mats.size();
            for (int32_t i = 0; i < n; ++i) {
                if (given[size_t(i)].root != r) continue;
                off = round_up(off, kRootAlign);
                given[size_t(i)].root_off = off;
                off += given[size_t(i)].R * given[size_t(i)].C;
                M->slot_of[size_t(i)] = (int32_t)M->mats.size();
                M->mats.push_back(given[size_t(i)]);
            }
            off = round_up(off, kRootAlign);
        }
        M->region[size_t(p.m)] = off;
        M->first[size_t(p.m)] = (int32_t)M->mats.size();
        M->root_elems = off;
        // Newton-Schulz buffers, chunks and tile counts
        const int64_t nm = (int64_t)M->mats.size();
        M->tiles.assign(size_t(7 * (nm + 1)), 0);
        int64_t ns = 0;
        auto take = [&](int64_t elems) {
            const int64_t o = ns;
            ns = round_up(ns + elems, 128);
            return o;
        };
        for (int64_t j = 0; j < nm; ++j) {
            MuonMat& mm = M->mats[size_t(j)];
            mm.x = take(mm.n * mm.k);
            mm.y0 = take(mm.n * mm.k);
            mm.y1 = take(mm.n * mm.k);
            mm.a = take(mm.n * mm.n);
            mm.b = take(mm.n * mm.n);
            const int64_t N = mm.R * mm.C;
            mm.g0 = (int64_t)M->chunks.size();
            mm.gn = ceil_div(N, kChunk);
            for (int64_t e = 0; e < N; e += kChunk)
                M->chunks.push_back(MuonChunk{e, (int32_t)j, (int32_t)std::min(kChunk, N - e)});
            // A and B are symmetric: their products compute the tiles on and
            // above the diagonal only
            const int64_t tn = ceil_div(mm.n, kGemmTile), tn2 = ceil_div(mm.n, kGemmTile2);
            const int64_t tcount[7] = {ceil_div(mm.R, kPrepTile) * ceil_div(mm.C, kPrepTile),
                                       tn * (tn + 1) / 2, tn * (tn + 1) / 2,
                                       ceil_div(mm.k, kGemmTile) * tn,
                                       tn2 * (tn2 + 1) / 2, tn2 * (tn2 + 1) / 2,
                                       ceil_div(mm.k, kGemmTile2) * tn2};
            for (int w = 0; w < 7; ++w)
                M->tiles[size_t(w * (nm + 1) + j + 1)] = M->tiles[size_t(w * (nm + 1) + j)] + tcount[w];
        }
        if (M->chunks.size() > 0x7fffffffu) {
            delete M;
            return fail(RS_EOVERFLOW, "too many chunks");
        }
        size_t o = 0;
        M->off_mats = o;
        o = align256(o + M->mats.size() * sizeof(MuonMat));
        M->off_chunks = o;
        o = align256(o + M->chunks.size() * sizeof(MuonChunk));
        M->off_tiles = o;
        o = align256(o + M->tiles.size() * sizeof(int64_t));
        M->off_partials = o;  // per-chunk sums, then one norm per matrix
        o = align256(o + (M->chunks.size() + M->mats.size()) * sizeof(double));
        M->off_ns = o;
        o = align256(o + size_t(ns) * 2);
        M->ws_bytes = o;
        *out = M;
        return RS_OK;
    } catch (const std::bad_alloc&) {
        return fail(RS_ENOMEM, "host allocation failed");
    }
}

void rs_muon_free(rs_muon* muon) { delete muon; }

rs_status rs_muon_layout(const rs_muon* muon, int32_t* roots, int64_t* offsets, int64_t* regions,
                         int64_t* root_elems) {
    if (!muon) return fail(RS_EINVAL, "muon plan is NULL");
    for (int32_t i = 0; i < muon->n_given; ++i) {
        const rs::mu::MuonMat& mm = muon->mats[size_t(muon->slot_of[size_t(i)])];
        if (roots) roots[i] = mm.root;
        if (offsets) offsets[i] = mm.root_off;
    }
    if (regions)
        for (int32_t r = 0; r <= muon->m; ++r) regions[r] = muon->region[size_t(r)];
    if (root_elems) *root_elems = muon->root_elems;
    return RS_OK;
}

size_t rs_muon_device_bytes(const rs_muon* muon) {
    if (!muon) {
        fail(RS_EINVAL, "muon plan is NULL");
        return 0;
    }
    return muon->ws_bytes;
}

rs_status rs_muon_upload(rs_muon* muon, void* d_workspace, size_t bytes, void* stream) {
    if (!muon) return fail(RS_EINVAL, "muon plan is NULL");
    if (!d_workspace || !aligned(d_workspace, 256))
        return fail(RS_EINVAL, "workspace must be a non-NULL 256-byte aligned device pointer");
    if (bytes < muon->ws_bytes)
        return fail(RS_ENOMEM, "workspace smaller than rs_muon_device_bytes()");
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    char* w = static_cast<char*>(d_workspace);
    struct Copy {
        size_t off;
        const void* src;
        size_t bytes;
    };
    const Copy copies[] = {
        {muon->off_mats, muon->mats.data(), muon->mats.size() * sizeof(rs::mu::MuonMat)},
        {muon->off_chunks, muon->chunks.data(), muon->chunks.size() * sizeof(rs::mu::MuonChunk)},
        {muon->off_tiles, muon->tiles.data(), muon->tiles.size() * sizeof(int64_t)},
    };
    for (const Copy& c : copies) {
        if (c.bytes == 0) continue;
        hipError_t e = hipMemcpyAsync(w + c.off, c.src, c.bytes, hipMemcpyHostToDevice, s);
        if (e != hipSuccess) return fail(RS_EHIP, std::string("hipMemcpyAsync: ") + hipGetErrorString(e));
    }
    hipError_t e = hipStreamSynchronize(s);
    if (e != hipSuccess) return fail(RS_EHIP, std::string("hipStreamSynchronize: ") + hipGetErrorString(e));
    if (!muon->aux) {
        e = hipStreamCreateWithFlags(&muon->aux, hipStreamNonBlocking);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&muon->ev_fork, hipEventDisableTiming);
        if (e == hipSuccess) e = hipEventCreateWithFlags(&muon->ev_join, hipEventDisableTiming);
        int dev = 0;
        if (e == hipSuccess) e = hipGetDevice(&dev);
        if (e == hipSuccess)
            e = hipDeviceGetAttribute(&muon->n_cu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return fail(RS_EHIP, std::string("stream / event: ") + hipGetErrorString(e));
    }
    muon->d_ws = d_workspace;
    muon->uploaded = true;
    return RS_OK;
}

rs_status rs_muon_gather(const rs_muon* muon, int32_t root, float* d_mom, const uint16_t* d_grad,
                         const rs_muon_hparams* hp, uint16_t* d_root, void* stream) {
    if (!muon || !d_mom || !d_grad || !hp || !d_root) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_mom, 16) || !aligned(d_grad, 16) || !aligned(d_root, 16))
        return fail(RS_EINVAL, "misaligned pointer");
    if (!muon->uploaded) return fail(RS_ESTATE, "muon plan not uploaded");
    if (!std::isfinite(hp->momentum)) return fail(RS_EINVAL, "momentum must be finite");
    int32_t i0, i1;
    int64_t c0, c1;
    rs_status st = select(*muon, root, i0, i1, c0, c1);
    if (st != RS_OK) return st;
    hipError_t e = rs::mu::launch_gather(device_tables(*muon), c0, c1, d_mom, d_grad,
                                         (float)hp->momentum, d_root,
                                         reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RS_EHIP, std::string("gather launch: ") + hipGetErrorString(e));
    return RS_OK;
}

rs_status rs_muon_orthogonalize(const rs_muon* muon, int32_t root, uint16_t* d_root, void* stream) {
    if (!muon || !d_root) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_root, 16)) return fail(RS_EINVAL, "misaligned pointer");
    if (!muon->uploaded) return fail(RS_ESTATE, "muon plan not uploaded");
    int32_t i0, i1;
    int64_t c0, c1;
    rs_status st = select(*muon, root, i0, i1, c0, c1);
    if (st != RS_OK) return st;
    const rs_muon& M = *muon;
    // matrices [a, b): the 256 x 256 product kernel when every dimension is a
    // multiple of 64 (both kernels give the same bits), and their chunks
    auto run = [&](int32_t a, int32_t b, hipStream_t st) {
        bool wide = true;
        for (int32_t i = a; i < b; ++i)
            wide = wide && M.mats[size_t(i)].n % 64 == 0 && M.mats[size_t(i)].k % 64 == 0;
        const int64_t x0 = M.mats[size_t(a)].g0;
        const int64_t x1 = M.mats[size_t(b - 1)].g0 + M.mats[size_t(b - 1)].gn;
        return rs::mu::launch_orthogonalize(device_tables(M), M.tiles.data(), a, b, x0, x1, wide,
                                            d_root, st);
    };
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    hipError_t e = hipSuccess;
    // the X X^T launch's tiles (256 x 256 when every dimension is a multiple
    // of 64, else 128 x 128): fewer than two per CU leaves CUs idle
    bool wide_all = true;
    for (int32_t i = i0; i < i1; ++i)
        wide_all = wide_all && M.mats[size_t(i)].n % 64 == 0 && M.mats[size_t(i)].k % 64 == 0;
    const int64_t* gram = M.tiles.data() + (wide_all ? 4 : 1) * (int64_t)(M.mats.size() + 1);
    const bool underfilled = gram[i1] - gram[i0] < 2 * (int64_t)M.n_cu;
    if (i1 - i0 < 2 || !underfilled) {
        if (i1 > i0) e = run(i0, i1, s);
    } else {
        // two groups of about equal Newton-Schulz cost (matrices stay in root
        // order), the second on the plan's own stream: each group's launches
        // then fill the CUs that the other's last round of tiles leaves idle
        // (on a full device the two only compete, so launches of two or more
        // tiles per CU stay on one stream).  The groups touch disjoint
        // workspace and root-buffer regions.
        double tot = 0.0, acc = 0.0, best = 0.0;
        for (int32_t i = i0; i < i1; ++i) tot += ns_cost(M.mats[size_t(i)].R, M.mats[size_t(i)].C);
        int32_t im = i0 + 1;
        for (int32_t i = i0 + 1; i < i1; ++i) {
            acc += ns_cost(M.mats[size_t(i - 1)].R, M.mats[size_t(i - 1)].C);
            const double d = std::fabs(acc - (tot - acc));
            if (i == i0 + 1 || d < best) {
                best = d;
                im = i;
            }
        }
        e = hipEventRecord(M.ev_fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(M.aux, M.ev_fork, 0);
        if (e == hipSuccess) {
            e = run(im, i1, M.aux);
            if (e == hipSuccess) e = run(i0, im, s);
            // joined even after a failed launch: the caller's stream never
            // runs ahead of work queued on the plan's stream
            hipError_t ej = hipEventRecord(M.ev_join, M.aux);
            if (ej == hipSuccess) ej = hipStreamWaitEvent(s, M.ev_join, 0);
            if (e == hipSuccess) e = ej;
        }
    }
    if (e != hipSuccess)
        return fail(RS_EHIP, std::string("Newton-Schulz launch: ") + hipGetErrorString(e));
    return RS_OK;
}

rs_status rs_muon_apply(const rs_muon* muon, int32_t root, float* d_master, const uint16_t* d_root,
                        const rs_muon_hparams* hp, void* stream) {
    if (!muon || !d_master || !d_root || !hp) return fail(RS_EINVAL, "NULL argument");
    if (!aligned(d_master, 16) || !aligned(d_root, 16)) return fail(RS_EINVAL, "misaligned pointer");
    if (!muon->uploaded) return fail(RS_ESTATE, "muon plan not uploaded");
    if (!std::isfinite(hp->lr) || !std::isfinite(hp->weight_decay))
        return fail(RS_EINVAL, "lr and weight_decay must be finite");
    int32_t i0, i1;
    int64_t c0, c1;
    rs_status st = select(*muon, root, i0, i1, c0, c1);
    if (st != RS_OK) return st;
    hipError_t e = rs::mu::launch_apply(device_tables(*muon), c0, c1, d_master, d_root,
                                        hp->lr * 0.2, (float)(1.0 - hp->lr * hp->weight_decay),
                                        reinterpret_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(RS_EHIP, std::string("apply launch: ") + hipGetErrorString(e));
    return RS_OK;
}

}  // extern "C"
