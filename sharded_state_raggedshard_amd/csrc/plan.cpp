// RaggedShard layout planner and device work-table builder (host C++).
//
// Layout problem: veScale-FSDP page, section "Grouped communication:
// structure-aware planning (Algorithm 1)".  Given the tensors of a bucket in
// their default order, find the smallest per-rank size S (a multiple of
// g_coll) admitting a placement with no block cut by a rank boundary, each
// tensor contiguous with padding only between tensors, offsets aligned to
// lcm(g_coll, block elements), inside m equal slices.
//
// For a fixed S the admissible offsets of a tensor depend only on where the
// previous tensor ends, and an earlier end never removes an admissible
// offset, so earliest-offset placement is exact for that S (the page's
// monotone dp(t, i) for a fixed order).  Feasibility is not monotone in S,
// so S is scanned upward; three devices keep the scan short:
//   - each long tensor rules out values of S by itself (SFilter below), and
//     the scan jumps over them;
//   - inside one S, the earliest offset jumps straight to the next offset
//     that repairs the first offending boundary (Chinese remaindering of the
//     alignment and the cut unit) instead of stepping by the alignment;
//   - a scan that is still going after a few thousand values of S continues
//     on several host threads, each taking the next range of S in
//     increasing order; the smallest feasible S is the same whatever the
//     threads' timing.
#include "plan.hpp"

#include <algorithm>
#include <atomic>
#include <limits>
#include <map>
#include <system_error>
#include <thread>

namespace rs {

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 50;
constexpr int64_t kInf = std::numeric_limits<int64_t>::max() / 4;

int64_t gcd64(int64_t a, int64_t b) {
    while (b) {
        int64_t r = a % b;
        a = b;
        b = r;
    }
    return a;
}

// lcm, saturating at kInf
int64_t lcm_sat(int64_t a, int64_t b) {
    __int128 l = (__int128)(a / gcd64(a, b)) * b;
    return l > kInf ? kInf : (int64_t)l;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// modular inverse of a mod n (gcd(a, n) == 1, n > 1)
int64_t mod_inverse(int64_t a, int64_t n) {
    __int128 t = 0, nt = 1, r = n, nr = a % n;
    while (nr != 0) {
        __int128 q = r / nr;
        __int128 tmp = t - q * nt;
        t = nt;
        nt = tmp;
        tmp = r - q * nr;
        r = nr;
        nr = tmp;
    }
    if (t < 0) t += n;
    return (int64_t)t;
}

rs_status derive(const rs_tensor_spec& s, int64_t g_coll, bool align_unit, TensorInfo& t,
                 std::string& err) {
    if (s.ndim < 1 || s.ndim > 4) {
        err = "ndim must be 1..4";
        return RS_EINVAL;
    }
    if (s.reserved != 0 || s.bucket < 0) {
        err = "bad bucket / reserved field";
        return RS_EINVAL;
    }
    int64_t N = 1;
    for (int i = 0; i < s.ndim; ++i) {
        if (s.shape[i] < 1) {
            err = "shape dimensions must be >= 1";
            return RS_EINVAL;
        }
        if ((__int128)N * s.shape[i] > kMaxElems) {
            err = "tensor larger than 2^50 elements";
            return RS_EOVERFLOW;
        }
        N *= s.shape[i];
    }
    t.N = N;
    t.C = s.ndim >= 2 ? s.shape[s.ndim - 1] : 1;
    t.R = N / t.C;
    t.gran = s.gran;
    t.br = s.br;
    t.bc = s.bc;
    t.bucket = s.bucket;
    switch (s.gran) {
    case RS_ELEMENT:
        t.u = 1;
        t.b = 1;
        t.nblk = N;
        break;
    case RS_ROWS:
        if (s.br < 1) {
            err = "ROWS granularity needs br >= 1";
            return RS_EINVAL;
        }
        t.u = (int64_t)s.br * t.C;
        t.b = std::min<int64_t>(s.br, t.R) * t.C;
        t.nblk = ceil_div(t.R, s.br);
        break;
    case RS_TILE:
        if (s.br < 2 || s.bc < 1) {
            err = "TILE granularity needs br >= 2 and bc >= 1";
            return RS_EINVAL;
        }
        if (t.C > (int64_t(1) << 31) - 1) {
            err = "TILE rows wider than 2^31 elements";
            return RS_EOVERFLOW;
        }
        t.u = (int64_t)s.br * t.C;
        t.b = std::min<int64_t>(s.br, t.R) * std::min<int64_t>(s.bc, t.C);
        t.nblk = ceil_div(t.R, s.br) * ceil_div(t.C, s.bc);
        break;
    default:
        err = "unknown granularity";
        return RS_EINVAL;
    }
    if (t.u > kMaxElems) {
        err = "cut unit larger than 2^50 elements";
        return RS_EOVERFLOW;
    }
    if (t.b > (int64_t(1) << 31) - 1) {
        err = "a quantisation block holds more than 2^31 elements";
        return RS_EOVERFLOW;
    }
    t.A = lcm_sat(g_coll, align_unit ? t.u : t.b);
    if (t.A > kMaxElems) {
        err = "offset alignment larger than 2^50";
        return RS_EOVERFLOW;
    }
    return RS_OK;
}

// Smallest x > o with x = 0 (mod A), x = cut (mod u), x < cut; kInf if none.
int64_t next_aligned_cut_match(const TensorInfo& t, int64_t o, int64_t cut) {
    int64_t g = gcd64(t.A, t.u);
    int64_t c = cut % t.u;
    if (c % g != 0) return kInf;
    int64_t M = t.u / g;
    int64_t k0 = 0;
    if (M > 1) {
        int64_t a = (t.A / g) % M;
        k0 = (int64_t)(((__int128)((c / g) % M) * mod_inverse(a, M)) % M);
    }
    __int128 L = (__int128)t.A * M;
    __int128 x0 = (__int128)t.A * k0;
    __int128 x;
    if (x0 > o)
        x = x0;
    else
        x = x0 + ((((__int128)o + 1 - x0) + L - 1) / L) * L;
    if (x >= cut) return kInf;
    return (int64_t)x;
}

}  // namespace

int64_t earliest_offset(const TensorInfo& t, int32_t m, int64_t S, int64_t e) {
    const int64_t cap = (int64_t)m * S;
    int64_t o = round_up(e, t.A);
    for (;;) {
        if (o + t.N > cap) return -1;
        int64_t j0 = o / S + 1;
        int64_t j1 = std::min<int64_t>(m - 1, (o + t.N - 1) / S);
        int64_t bad = -1;
        for (int64_t j = j0; j <= j1; ++j) {
            if ((j * S - o) % t.u != 0) {
                bad = j;
                break;
            }
        }
        if (bad < 0) return o;
        int64_t cut = bad * S;
        int64_t past = round_up(cut, t.A);
        int64_t match = next_aligned_cut_match(t, o, cut);
        o = std::min(past, match);
    }
}

namespace {

// rest[i]: elements of tensors i.. (a lower bound on what still has to fit).
bool place_all(const std::vector<TensorInfo*>& ts, const std::vector<int64_t>& rest, int32_t m,
               int64_t S, std::vector<int64_t>& off) {
    const int64_t cap = (int64_t)m * S;
    int64_t e = 0;
    for (size_t i = 0; i < ts.size(); ++i) {
        if (e + rest[i] > cap) return false;
        int64_t o = earliest_offset(*ts[i], m, S, e);
        if (o < 0) return false;
        off[i] = o;
        e = o + ts[i]->N;
    }
    return true;
}

// What one tensor alone says about S.  A tensor longer than S holds a rank
// boundary j S (0 < j < m) strictly inside it, which must lie on a cut:
// j S = o (mod u) for its offset o, a multiple of A, so j S is a multiple of
// h = gcd(A, u), and some j < m achieves that only when h / gcd(S, h) <=
// m - 1.  A tensor longer than 2S holds two consecutive boundaries, so u
// divides S.  Both are necessary conditions, so skipping the values of S
// they exclude never skips a feasible S.
struct SFilter {
    int64_t N;
    int64_t g;                   // S stays a multiple of g_coll
    int64_t su;                  // lcm(u, g)
    int64_t h;
    std::vector<int64_t> steps;  // lcm(h / d, g) for the divisors d <= m - 1 of h

    SFilter(const TensorInfo& t, int32_t m, int64_t g_) : N(t.N), g(g_) {
        su = lcm_sat(t.u, g);
        h = gcd64(t.A, t.u);
        for (int64_t d = 1; d <= std::min<int64_t>(m - 1, h); ++d)
            if (h % d == 0) steps.push_back(lcm_sat(h / d, g));
        // keep the steps no other step divides (their multiples cover the rest)
        std::sort(steps.begin(), steps.end());
        steps.erase(std::unique(steps.begin(), steps.end()), steps.end());
        if (steps.size() <= 512) {
            std::vector<int64_t> keep;
            for (int64_t st : steps) {
                bool covered = false;
                for (int64_t k : keep) covered = covered || st % k == 0;
                if (!covered) keep.push_back(st);
            }
            steps.swap(keep);
        }
    }

    // smallest S' >= S (a multiple of g) this tensor does not rule out
    int64_t next(int64_t S, int32_t m) const {
        if (N > 2 * S) {
            if (S % su == 0) return S;
            return std::min(su >= kInf ? kInf : round_up(S, su), round_up(ceil_div(N, 2), g));
        }
        if (N > S && h / gcd64(S, h) > m - 1) {
            int64_t nxt = round_up(N, g);  // from S >= N on, no boundary has to fall inside
            for (int64_t st : steps) nxt = std::min(nxt, st >= kInf ? kInf : round_up(S, st));
            return nxt;
        }
        return S;
    }
};

// Smallest S' >= S passing every tensor's filter.
int64_t next_candidate(const std::vector<SFilter>& fs, int32_t m, int64_t S) {
    for (;;) {
        int64_t nxt = S;
        for (const SFilter& f : fs) nxt = std::max(nxt, f.next(S, m));
        if (nxt == S || nxt >= kInf) return nxt;
        S = nxt;
    }
}

// Candidates tried on the calling thread before the scan goes parallel, and
// the width (in values of S) of one range of the parallel scan.
constexpr int kSerialTries = 4096;
constexpr int64_t kRangeTries = 2048;
constexpr unsigned kMaxPlanThreads = 16;

rs_status plan_one_bucket(std::vector<TensorInfo*>& ts, int32_t m, int64_t g, int64_t& S_out,
                          std::string& err) {
    int64_t end0 = 0;
    for (auto* t : ts) end0 = round_up(end0, t->A) + t->N;
    // Every placement ends at or after end0 (the cut-free earliest
    // placement), so m*S >= end0; this bound also covers ceil(total / m).
    const int64_t S_lo = round_up(ceil_div(end0, m), g);
    const int64_t S_hi = round_up(end0, g);  // everything inside rank 0: always feasible
    std::vector<int64_t> off(ts.size()), rest(ts.size() + 1, 0);
    for (size_t i = ts.size(); i-- > 0;) rest[i] = rest[i + 1] + ts[i]->N;
    std::vector<SFilter> fs;
    for (auto* t : ts)
        if (t->N > S_lo) fs.emplace_back(*t, m, g);  // S >= S_lo: shorter tensors never filter

    auto done = [&](int64_t S) {
        place_all(ts, rest, m, S, off);
        for (size_t i = 0; i < ts.size(); ++i) ts[i]->off = off[i];
        S_out = S;
        return RS_OK;
    };
    int64_t S = S_lo;
    for (int tries = 0; tries < kSerialTries; ++tries) {
        S = next_candidate(fs, m, S);
        if (S > S_hi) break;
        if (place_all(ts, rest, m, S, off)) return done(S);
        S += g;
    }
    if (S <= S_hi) {
        // the rest of [S, S_hi] in ranges handed out in increasing order; a
        // range starting past the best S found so far is not needed
        const int64_t width = kRangeTries * g;
        std::atomic<int64_t> next_start{S}, best{kInf};
        auto worker = [&]() {
            std::vector<int64_t> o(ts.size());
            for (;;) {
                const int64_t a = next_start.fetch_add(width);
                if (a > S_hi || a >= best.load()) return;
                const int64_t b = std::min(a + width, S_hi + 1);
                for (int64_t s = next_candidate(fs, m, a); s < b && s < best.load();
                     s = next_candidate(fs, m, s + g)) {
                    if (place_all(ts, rest, m, s, o)) {
                        int64_t cur = best.load();
                        while (s < cur && !best.compare_exchange_weak(cur, s)) {
                        }
                        break;
                    }
                }
            }
        };
        unsigned nt = std::thread::hardware_concurrency();
        nt = std::max(1u, std::min(nt, kMaxPlanThreads));
        std::vector<std::thread> pool;
        try {
            for (unsigned i = 1; i < nt; ++i) pool.emplace_back(worker);
        } catch (const std::system_error&) {
            // fewer threads than asked for: the ones running (and this one) finish the scan
        }
        worker();
        for (auto& th : pool) th.join();
        if (best.load() < kInf) return done(best.load());
    }
    err = "internal: planner scan ended without a placement";
    return RS_EINVAL;
}

// First block (global id) whose first element is at or after position P,
// scanning the bucket's tensors in buffer order.
int64_t first_block_at(const Plan& p, const BucketInfo& B, int64_t P) {
    for (int32_t i : B.tensors) {
        const TensorInfo& t = p.t[i];
        if (t.pos + t.N <= P) continue;
        int64_t k;
        if (P <= t.pos) {
            k = 0;
        } else if (t.gran == RS_ELEMENT) {
            k = P - t.pos;
        } else {
            int64_t band = ceil_div(P - t.pos, t.u);
            k = (t.gran == RS_TILE) ? band * ceil_div(t.C, t.bc) : band;
        }
        if (k < t.nblk) return t.blk0 + k;
    }
    return B.blk0 + B.nblk;
}

}  // namespace

rs_status plan_layout(const rs_tensor_spec* specs, int32_t n, int32_t m, int64_t g_coll,
                      int32_t options, Plan& p, std::string& err) {
    if (!specs || n < 1 || m < 1 || g_coll < 1) {
        err = "need specs != NULL, n >= 1, m >= 1, g_coll >= 1";
        return RS_EINVAL;
    }
    if (m > (1 << 20) || g_coll > kMaxElems) {
        err = "m or g_coll out of range";
        return RS_EINVAL;
    }
    const int32_t order = options & RS_ORDER_MASK;
    if (order != RS_ORDER_GIVEN && order != RS_ORDER_BY_BLOCK && order != RS_ORDER_BY_SIZE) {
        err = "unknown tensor order";
        return RS_EINVAL;
    }
    if ((options & ~(RS_ORDER_MASK | RS_ALIGN_CUT_UNIT)) != 0) {
        err = "unknown planner option bits";
        return RS_EINVAL;
    }
    p.m = m;
    p.g_coll = g_coll;
    p.t.assign(n, TensorInfo{});
    int32_t nb = 0;
    for (int32_t i = 0; i < n; ++i) {
        rs_status st = derive(specs[i], g_coll, (options & RS_ALIGN_CUT_UNIT) != 0, p.t[i], err);
        if (st != RS_OK) {
            err = "tensor " + std::to_string(i) + ": " + err;
            return st;
        }
        nb = std::max(nb, specs[i].bucket + 1);
    }
    p.b.assign(nb, BucketInfo{});
    for (int32_t i = 0; i < n; ++i) p.b[p.t[i].bucket].tensors.push_back(i);
    // placement order inside each bucket (stable: ties keep the given order)
    for (BucketInfo& B : p.b) {
        if (order == RS_ORDER_BY_BLOCK)
            std::stable_sort(B.tensors.begin(), B.tensors.end(),
                             [&](int32_t x, int32_t y) { return p.t[x].b > p.t[y].b; });
        else if (order == RS_ORDER_BY_SIZE)
            std::stable_sort(B.tensors.begin(), B.tensors.end(),
                             [&](int32_t x, int32_t y) { return p.t[x].N > p.t[y].N; });
    }
    int64_t base = 0, blk = 0;
    p.by_pos.clear();
    std::map<std::vector<int64_t>, std::pair<int64_t, std::vector<int64_t>>> memo;
    for (int32_t k = 0; k < nb; ++k) {
        BucketInfo& B = p.b[k];
        if (B.tensors.empty()) {
            err = "bucket " + std::to_string(k) + " is empty";
            return RS_EINVAL;
        }
        std::vector<TensorInfo*> ts;
        for (int32_t i : B.tensors) ts.push_back(&p.t[i]);
        // Buckets with the same tensor list (identical layers) get the same
        // plan: the planner is a function of that list alone.
        std::vector<int64_t> key;
        key.reserve(ts.size() * 5);
        for (const TensorInfo* t : ts) {
            key.push_back(t->N);
            key.push_back(t->C);
            key.push_back(t->u);
            key.push_back(t->b);
            key.push_back(t->A);
        }
        auto hit = memo.find(key);
        if (hit != memo.end()) {
            B.S = hit->second.first;
            for (size_t j = 0; j < ts.size(); ++j) ts[j]->off = hit->second.second[j];
        } else {
            rs_status st = plan_one_bucket(ts, m, g_coll, B.S, err);
            if (st != RS_OK) return st;
            std::vector<int64_t> offs(ts.size());
            for (size_t j = 0; j < ts.size(); ++j) offs[j] = ts[j]->off;
            memo.emplace(std::move(key), std::make_pair(B.S, std::move(offs)));
        }
        if ((__int128)B.S * m + base > kMaxElems * 8) {
            err = "buffer larger than 2^53 elements";
            return RS_EOVERFLOW;
        }
        B.base = base;
        B.blk0 = blk;
        B.real = 0;
        for (int32_t i : B.tensors) {
            TensorInfo& t = p.t[i];
            t.pos = base + t.off;
            t.blk0 = blk;
            blk += t.nblk;
            B.real += t.N;
            p.by_pos.push_back(i);
        }
        B.nblk = blk - B.blk0;
        B.padding = (int64_t)m * B.S - B.real;
        base += (int64_t)m * B.S;
    }
    p.total = base;
    p.nblocks = blk;
    p.rank_blk.assign(size_t(nb) * (m + 1), 0);
    for (int32_t k = 0; k < nb; ++k) {
        const BucketInfo& B = p.b[k];
        for (int32_t r = 0; r <= m; ++r)
            p.rank_blk[size_t(k) * (m + 1) + r] =
                (r == m) ? B.blk0 + B.nblk : first_block_at(p, B, B.base + (int64_t)r * B.S);
    }
    // Default step chunk, as measured on gfx950: 4096 elements (more, smaller
    // workgroups resident per CU; pays on launches of up to about 2^30
    // elements and on strided tile rows), or 8192 for larger plans that are
    // mostly contiguous (fewer, longer workgroups amortise the per-chunk
    // work once the launch is long).
    int64_t strided = 0, all = 0;
    for (const TensorInfo& ti : p.t) {
        all += ti.N;
        if (ti.gran == RS_TILE && ti.R > 1 && ti.bc < ti.C) strided += ti.N;
    }
    const bool large = all > (int64_t(1) << 30) && 2 * strided <= all;
    p.chunk_elems = large ? kDefaultChunk : kDefaultChunk / 2;
    p.tables_built = false;
    return RS_OK;
}

// ------------------------------------------------------------ work tables

namespace {

bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

struct ChunkBuilder {
    const Plan& p;
    const BucketInfo& B;
    int64_t CH;
    std::vector<ChunkDesc>& out;
    int32_t tj = -1;  // the current tensor's index in buffer order

    int32_t rank_of(int64_t pos) const { return (int32_t)((pos - B.base) / B.S); }

    void scalar(int64_t pos, int64_t blk, int64_t rows, int64_t cols, int64_t ld) {
        ChunkDesc c{};
        c.pos = pos;
        c.blk = blk;
        c.ld = ld;
        c.rows = (int32_t)rows;
        c.cols = (int32_t)cols;
        c.part = 0;
        c.nparts = 1;
        c.kind = KIND_SCALAR;
        c.run_log2 = -1;
        c.tensor = tj;
        out.push_back(c);
    }

    void vec(int64_t pos, int64_t blk, int64_t rows, int64_t cols, int64_t ld, int32_t part,
             int32_t nparts, int32_t run_log2) {
        ChunkDesc c{};
        c.pos = pos;
        c.blk = blk;
        c.ld = ld;
        c.rows = (int32_t)rows;
        c.cols = (int32_t)cols;
        c.part = part;
        c.nparts = nparts;
        c.kind = KIND_VEC;
        c.run_log2 = (int16_t)run_log2;
        c.tensor = tj;
        out.push_back(c);
    }

    // One contiguous block [s, s + n).
    void contiguous_block(int64_t s, int64_t n, int64_t blk) {
        if (s % kVecAlign != 0 || n % kVecAlign != 0) {
            scalar(s, blk, 1, n, n);
            return;
        }
        if (n <= CH) {
            vec(s, blk, 1, n, n, 0, 1, -1);
            return;
        }
        int32_t np = (int32_t)ceil_div(n, CH);
        for (int32_t q = 0; q < np; ++q)
            vec(s + q * CH, blk, 1, std::min(CH, n - q * CH), 0, q, np, -1);
    }

    void tensor(const TensorInfo& t) {
        if (t.gran == RS_ELEMENT) {
            // runs of single-element blocks, never across a rank boundary
            int64_t i = 0;
            while (i < t.N) {
                int64_t p0 = t.pos + i;
                int64_t rank_end = B.base + (rank_of(p0) + 1) * B.S;
                int64_t len = std::min({CH, t.N - i, rank_end - p0});
                ChunkDesc c{};
                c.pos = p0;
                c.blk = t.blk0 + i;
                c.ld = 0;
                c.rows = 1;
                c.cols = (int32_t)len;
                c.part = 0;
                c.nparts = 1;
                c.kind = KIND_ELEM;
                c.run_log2 = -1;
                c.tensor = tj;
                out.push_back(c);
                i += len;
            }
            return;
        }
        const bool contiguous_blocks = (t.gran == RS_ROWS) || (t.bc >= t.C);
        if (contiguous_blocks) {
            // block k covers rows [k*br, min((k+1)*br, R)) in full
            const int64_t full = t.u;  // elements of a full block
            int64_t k = 0;
            while (k < t.nblk) {
                int64_t s = t.pos + k * t.u;
                int64_t n = std::min(t.u, t.N - k * t.u);
                if (n == full && s % kVecAlign == 0 && pow2(n) && n >= kVecAlign &&
                    n <= (int64_t(1) << kMaxRunLog2) && n < CH) {
                    // run of whole small blocks of one rank, reduced in lane groups
                    int32_t r = rank_of(s);
                    int64_t k1 = k + 1;
                    while (k1 < t.nblk && (k1 - k + 1) * n <= CH) {
                        int64_t s1 = t.pos + k1 * t.u;
                        if (std::min(t.u, t.N - k1 * t.u) != n || rank_of(s1) != r) break;
                        ++k1;
                    }
                    vec(s, t.blk0 + k, 1, (k1 - k) * n, 0, 0, 1, ilog2(n));
                    k = k1;
                    continue;
                }
                contiguous_block(s, n, t.blk0 + k);
                ++k;
            }
            return;
        }
        // 2-D tiles narrower than a row: rows of bc elements with stride C
        const int64_t nbc = ceil_div(t.C, t.bc);
        for (int64_t k = 0; k < t.nblk; ++k) {
            int64_t bi = k / nbc, bj = k % nbc;
            int64_t r0 = bi * t.br, rows = std::min<int64_t>(t.br, t.R - r0);
            int64_t c0 = bj * t.bc, cols = std::min<int64_t>(t.bc, t.C - c0);
            int64_t s = t.pos + r0 * t.C + c0;
            // vector tiles address their elements with 32-bit offsets from the
            // chunk start: rows * C must stay below 2^30
            if (s % kVecAlign != 0 || cols % kVecAlign != 0 || t.C % kVecAlign != 0 || cols > CH ||
                std::min<int64_t>(rows, CH / std::max<int64_t>(cols, 1)) * t.C >= (int64_t(1) << 30)) {
                scalar(s, t.blk0 + k, rows, cols, t.C);
                continue;
            }
            if (rows * cols <= CH) {
                vec(s, t.blk0 + k, rows, cols, t.C, 0, 1, -1);
                continue;
            }
            int64_t rpp = CH / cols;
            int32_t np = (int32_t)ceil_div(rows, rpp);
            for (int32_t q = 0; q < np; ++q)
                vec(s + q * rpp * t.C, t.blk0 + k, std::min(rpp, rows - q * rpp), cols, t.C, q,
                    np, -1);
        }
    }
};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

}  // namespace

// One chunk table (chunks in buffer order, per-bucket-and-rank begin
// indices, the most chunks of one block) for a chunk size.  With pad, the
// padding of every slice is listed too, as KIND_PAD chunks of at most
// `chunk` elements that never cross a rank boundary.
static rs_status build_chunks(const Plan& p, int64_t chunk, bool pad, std::vector<ChunkDesc>& chunks,
                              std::vector<int64_t>& begin, int32_t& max_nparts, std::string& err) {
    const int32_t nb = (int32_t)p.b.size();
    const int32_t m = p.m;
    chunks.clear();
    begin.assign(size_t(nb) * (m + 1), 0);
    int32_t tj = 0;  // buffer-order index of the next tensor
    for (int32_t k = 0; k < nb; ++k) {
        const BucketInfo& B = p.b[k];
        size_t first = chunks.size();
        ChunkBuilder cbld{p, B, chunk, chunks};
        int64_t cur = B.base;  // end of what is listed so far
        auto pad_to = [&](int64_t end) {
            while (pad && cur < end) {
                const int64_t rank_end = B.base + ((cur - B.base) / B.S + 1) * B.S;
                const int64_t e = std::min({end, rank_end, cur + chunk});
                ChunkDesc c{};
                c.pos = cur;
                c.blk = -1;
                c.ld = 0;
                c.rows = 1;
                c.cols = (int32_t)(e - cur);
                c.part = 0;
                c.nparts = 1;
                c.kind = KIND_PAD;
                c.run_log2 = -1;
                c.tensor = -1;
                chunks.push_back(c);
                cur = e;
            }
        };
        // B.tensors is in buffer order
        for (int32_t i : B.tensors) {
            const TensorInfo& t = p.t[i];
            pad_to(t.pos);
            cbld.tj = tj++;
            cbld.tensor(t);
            cur = t.pos + t.N;
        }
        pad_to(B.base + (int64_t)m * B.S);
        // chunks come out in buffer order, so their ranks never decrease
        size_t c = first;
        for (int32_t r = 0; r <= m; ++r) {
            int64_t lim = B.base + (int64_t)r * B.S;
            while (c < chunks.size() && chunks[c].pos < lim) ++c;
            begin[size_t(k) * (m + 1) + r] = (int64_t)c;
        }
        begin[size_t(k) * (m + 1) + m] = (int64_t)chunks.size();
    }
    max_nparts = 1;
    for (const ChunkDesc& c : chunks) {
        if (c.nparts > 65535) {
            err = "a block needs more than 65535 chunks; raise the chunk size";
            return RS_EOVERFLOW;
        }
        max_nparts = std::max(max_nparts, c.nparts);
    }
    return RS_OK;
}

rs_status build_tables(Plan& p, std::string& err) {
    rs_status st = build_chunks(p, p.chunk_elems, false, p.chunks, p.chunk_begin, p.max_nparts, err);
    if (st != RS_OK) return st;
    st = build_chunks(p, kFp8Chunk, true, p.chunks8, p.chunk_begin8, p.max_nparts8, err);
    if (st != RS_OK) return st;
    // tensor tables in buffer order and the granule index
    const size_t n = p.t.size();
    p.tstart.resize(n);
    p.tend.resize(n);
    for (size_t j = 0; j < n; ++j) {
        const TensorInfo& t = p.t[p.by_pos[j]];
        p.tstart[j] = t.pos;
        p.tend[j] = t.pos + t.N;
    }
    const int64_t ngran = ceil_div(std::max<int64_t>(p.total, 1), kGranule);
    p.gidx.assign(size_t(ngran), (int32_t)n);
    {
        size_t j = 0;
        for (int64_t g = 0; g < ngran; ++g) {
            int64_t gs = g * kGranule;
            while (j < n && p.tend[j] <= gs) ++j;
            p.gidx[size_t(g)] = (int32_t)j;
        }
    }
    size_t off = 0;
    p.off_tstart = off;
    off = align256(off + n * 8);
    p.off_tend = off;
    off = align256(off + n * 8);
    p.off_src = off;
    off = align256(off + n * 8);
    p.off_dst = off;
    off = align256(off + n * 8);
    p.off_gidx = off;
    off = align256(off + size_t(ngran) * 4);
    p.off_chunks = off;
    off = align256(off + p.chunks.size() * sizeof(ChunkDesc));
    p.off_cpart = off;
    off = align256(off + p.chunks.size() * sizeof(ChunkPartial));
    p.off_coop = off;
    off = align256(off + p.chunks.size() * sizeof(PartSlot));
    p.off_cpart_t = off;
    off = align256(off + p.chunks.size() * sizeof(float));
    p.off_coop_t = off;
    off = align256(off + p.chunks.size() * sizeof(PartSlot));
    p.off_chunks8 = off;
    off = align256(off + p.chunks8.size() * sizeof(ChunkDesc));
    p.off_cpart8 = off;
    off = align256(off + p.chunks8.size() * sizeof(ChunkPartial));
    p.off_coop8 = off;
    off = align256(off + p.chunks8.size() * sizeof(PartSlot));
    p.off_l2 = off;
    off = align256(off + size_t(kL2Words) * 8);
    p.off_flag = off;
    off = align256(off + sizeof(CoopCounters));
    p.ws_bytes = off;
    p.tables_built = true;
    return RS_OK;
}

}  // namespace rs
