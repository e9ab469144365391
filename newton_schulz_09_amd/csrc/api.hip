// C ABI of libmuon.so: validation, workspace layout and the launch sequence
// of the Muon hot path (declared and documented in include/muon.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon.h"
#include "internal.hpp"

namespace muon {

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return status;
}

int ok() {
    g_last_error.clear();
    return MUON_OK;
}

int hip_fail(hipError_t e, const char* where) {
    return fail(MUON_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

int device_cus();

// X' bytes of one a X + B X launch from which it stores X' with streaming
// stores (set between the sizes measured either way: 34 MB and 170 MB)
constexpr int64_t kStreamOutBytes = int64_t{96} << 20;

// GEMM tile edge for the short side m of `count` m x n matrices.  Padding m
// and n to the tile keeps the GEMMs free of edge handling; the choice trades
// padded work against the larger tile's better operand reuse.
// MUON_NS5_TILE=64/128/256 in the environment forces one edge for every
// shape (read once, for tuning sweeps).
int choose_tile(int64_t m, int64_t n, int64_t count) {
    static const int forced = [] {
        const char* s = getenv("MUON_NS5_TILE");
        const int t = s ? atoi(s) : 0;
        return (t == 64 || t == 128 || t == 256) ? t : 0;
    }();
    if (forced) return forced;
    if (m <= 64) return 64;
    if (m >= 2048) return 256;
    // Below m = 2048 the 128 tile, whose extra workgroups fill the CUs
    // better; where its padded m is a multiple of 256, X X^T and a X + B X
    // still run on 256 x 256 tiles.  Where it is not, 256 tiles over m padded
    // to 256 are taken if that pads m by at most 8% more and the batch gives
    // a X + B X two rounds of the device's CUs or more: every product then
    // runs on the 256 engines, whose operand reuse outweighs the padding
    // (the GPT-2 1.5B set, m = 1600: 54.3 -> 51.5 ms per step).
    const int64_t mp128 = round_up(m, 128), mp256 = round_up(m, 256);
    if (mp128 % 256 != 0 && mp256 * 100 <= mp128 * 108) {
        const int64_t c = count < kMaxGroup ? count : kMaxGroup;
        if (c * (mp256 / 256) * (round_up(n, 256) / 256) >= 2 * static_cast<int64_t>(device_cus())) return 256;
    }
    return 128;
}

// Row skew (elements) added to every workspace row stride: 64 bf16 = 128
// bytes, one cache line (MUON_LD_SKEW=0/32/64/128 overrides it, for tuning).
int ld_skew() {
    static const int skew = [] {
        const char* s = getenv("MUON_LD_SKEW");
        const int v = s ? atoi(s) : 64;
        return (v == 0 || v == 32 || v == 64 || v == 128) ? v : 64;
    }();
    return skew;
}

// Tile rows per band of the full-grid product: all of them when there are
// at most 8 (each column panel of X^T is then read once), else 4
// (MUON_GEMM_BAND=n caps it at n, for tuning).
int band_rows(int tiles_m) {
    static const int cap = [] {
        const char* s = getenv("MUON_GEMM_BAND");
        const int v = s ? atoi(s) : 0;
        return v >= 1 ? v : 0;
    }();
    int b = tiles_m <= 8 ? tiles_m : 4;
    if (cap && b > cap) b = cap;
    return b;
}

// U V^T through an SVD: a block pair needs no rotation once the largest
// cosine between two of its rows is at most kSvdTol (float32 rows: a few
// units of float32 rounding, the orthogonality float32 storage holds); rows
// shorter than kSvdRankTol times the longest are taken as null space (the
// rows a zero singular value leaves are float32 rounding noise, about 1e-7
// of the longest).
constexpr double kSvdTol = 1e-6;
constexpr double kSvdRankTol = 1e-6;

// A dispatch's grid (workgroups x 256 work-items) must fit in 32 bits.
constexpr int64_t kMaxWorkgroups = (int64_t{1} << 32) / kThreads - 1;
// Cast workgroups per launch: beyond this each casts several tiles.
// MUON_CAST_WG_CAP=n lowers the cap (read once per process; tests of the
// several-tiles path, which only very large inputs reach otherwise, run in
// a process of their own with it set).
// 64 x 64 tiles per cast workgroup (MUON_CAST_TILES=n, for tuning sweeps):
// one norm reduction serves them all, and each next tile is loaded while
// the current one is converted.
int cast_tiles_per_wg() {
    static const int n = [] {
        const char* s = getenv("MUON_CAST_TILES");
        const int v = s ? atoi(s) : 4;
        return (v >= 1 && v <= 64) ? v : 4;
    }();
    return n;
}

int64_t max_cast_workgroups() {
    static const int64_t cap = [] {
        const char* s = getenv("MUON_CAST_WG_CAP");
        const long long v = s ? atoll(s) : 0;
        const int64_t limit = int64_t{1} << 20;
        return (v >= 1 && v < limit) ? static_cast<int64_t>(v) : limit;
    }();
    return cap;
}

// Compute units of the current device, queried once per device (256 on a
// whole MI355X; fewer on a partitioned one).  Without a usable device (the
// workspace queries run on hosts with none) the whole chip's 256.
constexpr int kDefaultCus = 256;
constexpr int kMaxDevices = 64;
int device_cus() {
    static std::atomic<int> cached[kMaxDevices];  // 0: not queried yet
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return kDefaultCus;
    }
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
        (void)hipGetLastError();
        n = kDefaultCus;
    }
    cached[dev].store(n, std::memory_order_relaxed);
    return n;
}

}  // namespace

// Tile of the symmetric products.  With 256 tiles (m >= 2048) a pass has
// n256 = cnt T (T + 1) / 2 upper tiles, one workgroup per CU each, so it takes
// ceil(n256 / CUs) rounds of the device's CUs (256 on MI355X): one 4096^2 matrix has 136 tiles, a
// single round that leaves almost half of them idle; two have 272, a second
// round of 16.  192 tiles on m rounded up to 192 give more, smaller tiles
// (253 per 4096^2 matrix), each round lasting about 0.5625 / 0.85 of a 256
// round (the smaller share of the work at the measured lower speed per
// flop).  192 is taken where that predicts at least 10% less time; measured:
// one 4096^2 1.68 -> 1.53 ms, two 3.17 -> 2.78 ms, while the 16 matrices of
// 2048 x 8192 (9.96 against 10.44 ms) and eight of them keep 256.  The
// padding stays zero, and every element is accumulated in the same K order
// under any tile.  MUON_SYM_TILE=256, 192 (where it covers mp) or 128 forces
// the choice for m >= 2048 (for tuning).
void choose_sym_tile(Ns5Plan* p) {
    p->sym_tile = p->tile;
    p->msym = p->mp;
    if (p->tile != 256) return;
    static const int forced = [] {
        const char* s = getenv("MUON_SYM_TILE");
        const int t = s ? atoi(s) : 0;
        return (t == 128 || t == 192 || t == 256) ? t : 0;
    }();
    if (forced == 128) {  // mp, a multiple of 256, is one of 128 too
        p->sym_tile = 128;
        return;
    }
    const int m192 = static_cast<int>(round_up(p->m, 192));
    if (forced == 256 || m192 < p->mp) return;  // the 192 padding must cover mp
    const double cus = device_cus();
    const double t256 = p->mp / 256, t192 = m192 / 192;
    const double rounds256 = ceil(p->cnt * t256 * (t256 + 1) / 2 / cus);
    const double rounds192 = ceil(p->cnt * t192 * (t192 + 1) / 2 / cus) * 0.5625 / 0.85;
    if (forced == 192 || rounds192 < 0.9 * rounds256) {
        p->sym_tile = 192;
        p->msym = m192;
    }
}

bool make_plan(int64_t rows, int64_t cols, int64_t count, Ns5Plan* p) {
    if (rows < 1 || cols < 1 || count < 1) return false;
    const int64_t m = rows < cols ? rows : cols;
    const int64_t n = rows < cols ? cols : rows;
    if (m > MUON_NS5_MAX_SHORT || n > MUON_NS5_MAX_LONG) return false;
    p->rows = rows;
    p->cols = cols;
    p->m = static_cast<int>(m);
    p->n = static_cast<int>(n);
    p->tall = rows > cols;
    p->tile = choose_tile(m, n, count);
    p->mp = static_cast<int>(round_up(m, p->tile));
    p->np = static_cast<int>(round_up(n, p->tile));
    int64_t nb = (rows * cols + 16383) / 16384;
    p->nb = static_cast<int>(nb < 1 ? 1 : (nb > kMaxNormBlocks ? kMaxNormBlocks : nb));
    const int64_t bx_tiles = static_cast<int64_t>(p->mp / p->tile) * (p->np / p->tile);
    int64_t cnt = count < kMaxGroup ? count : kMaxGroup;
    if (cnt * bx_tiles > kMaxWorkgroups) cnt = kMaxWorkgroups / bx_tiles;
    if (cnt < 1) return false;
    p->cnt = static_cast<int>(cnt);
    choose_sym_tile(p);
    p->ldx = p->np + ld_skew();
    p->lda = p->msym + ld_skew();
    p->x_elems = static_cast<size_t>(p->msym) * p->ldx;
    p->a_elems = static_cast<size_t>(p->msym) * p->lda;
    size_t off = 0;
    const size_t xb = align256(cnt * p->x_elems * sizeof(bf16_t));
    const size_t ab = align256(cnt * p->a_elems * sizeof(bf16_t));
    p->off_x[0] = off; off += xb;
    p->off_x[1] = off; off += xb;
    p->off_a = off; off += ab;
    p->off_b = off; off += ab;
    p->off_part = off; off += align256(cnt * p->nb * sizeof(double));
    p->bytes = off;
    return true;
}

namespace {

struct EventSink {
    void* const* events = nullptr;
    int pairs = 0;
    int recorded = 0;
};

// A set of same-shaped matrices of one call.
struct Segment {
    int64_t rows, cols, count;
    const float* const* G;
    float* const* out;
    float* const* buf;  // momentum buffers (fused Muon step), or null
};

// Up to kMaxGroup matrices of one segment, with its workspace layout at byte
// offset `base` of its launch group's workspace.
struct Chunk {
    const float* const* G;
    float* const* out;
    float* const* buf;
    Ns5Plan plan;
    size_t base;
};

// Chunks that share the tile size: each GEMM of each NS5 step is a single
// launch over all of them.  Groups run one after another, each reusing the
// workspace from its start.  A small group holds matrices of the small range
// (short side <= kSmallM, long side <= kSmallN): each of its chunks is one
// launch that runs the whole step in LDS (its workspace share is reserved
// but not used).
struct Group {
    std::vector<Chunk> chunks;
    bool small = false;
    int tile = 0;
    int mats = 0;
    int64_t bx_blocks = 0;  // workgroups of the largest launch (a X + B X)
    size_t bytes = 0;
};

int64_t bx_blocks(const Ns5Plan& p) {
    return static_cast<int64_t>(p.mp / p.tile) * (p.np / p.tile) * p.cnt;
}

// Splits validated segments into launch groups (deterministic in the shapes,
// so the workspace query and the call agree).  cap > 0 bounds every group's
// workspace to cap bytes (a fixed workspace): chunks are cut to fit, and a
// matrix that needs more on its own is an error.
int plan_groups(const Segment* segs, int nseg, std::vector<Group>* groups, size_t cap = 0) {
    groups->clear();
    for (int si = 0; si < nseg; ++si) {
        const Segment& sg = segs[si];
        for (int64_t start = 0; start < sg.count;) {
            Ns5Plan pl;
            if (!make_plan(sg.rows, sg.cols, sg.count - start, &pl))
                return fail(MUON_ERR_UNSUPPORTED, "shape %lld x %lld is beyond the supported limits",
                            (long long)sg.rows, (long long)sg.cols);
            while (cap > 0 && pl.bytes > cap) {
                if (pl.cnt == 1)
                    return fail(MUON_ERR_UNSUPPORTED,
                                "a %lld x %lld matrix needs %zu bytes of workspace, more than the %zu the "
                                "library holds", (long long)sg.rows, (long long)sg.cols, pl.bytes, cap);
                // bytes grow about linearly with the matrices of a chunk
                int64_t fit = static_cast<int64_t>(static_cast<double>(pl.cnt) * cap / pl.bytes);
                if (fit >= pl.cnt) fit = pl.cnt - 1;
                make_plan(sg.rows, sg.cols, fit < 1 ? 1 : fit, &pl);
            }
            const bool small = pl.m <= kSmallM && pl.n <= kSmallN;
            Group* g = groups->empty() ? nullptr : &groups->back();
            if (!g || g->small != small || g->tile != pl.tile || g->chunks[0].plan.sym_tile != pl.sym_tile ||
                g->mats + pl.cnt > kMaxGroup || (cap > 0 && g->bytes + pl.bytes > cap) ||
                static_cast<int>(g->chunks.size()) == kMaxSeg || g->bx_blocks + bx_blocks(pl) > kMaxWorkgroups) {
                groups->emplace_back();
                g = &groups->back();
                g->tile = pl.tile;
                g->small = small;
            }
            Chunk c;
            c.G = sg.G ? sg.G + start : nullptr;
            c.out = sg.out ? sg.out + start : nullptr;
            c.buf = sg.buf ? sg.buf + start : nullptr;
            c.plan = pl;
            c.base = g->bytes;
            g->chunks.push_back(c);
            g->mats += pl.cnt;
            g->bx_blocks += bx_blocks(pl);
            g->bytes += pl.bytes;
            start += pl.cnt;
        }
    }
    return MUON_OK;
}

size_t groups_bytes(const std::vector<Group>& groups) {
    size_t b = 0;
    for (const Group& g : groups) b = g.bytes > b ? g.bytes : b;
    return b;
}

int check_common(int steps, float eps) {
    if (steps < 0) return fail(MUON_ERR_INVALID_ARG, "steps must be >= 0 (got %d)", steps);
    if (!isfinite(eps)) return fail(MUON_ERR_INVALID_ARG, "eps must be finite");
    return MUON_OK;
}

int check_workspace(void* ws, size_t ws_bytes, size_t need) {
    if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is null");
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(MUON_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < need) return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
    return MUON_OK;
}

// Workspace pointers of one chunk.
struct ChunkBufs {
    bf16_t *X[2], *A, *B;
    double* part;
};

ChunkBufs bufs_of(char* ws, const Chunk& c) {
    char* b = ws + c.base;
    const Ns5Plan& p = c.plan;
    ChunkBufs r;
    r.X[0] = reinterpret_cast<bf16_t*>(b + p.off_x[0]);
    r.X[1] = reinterpret_cast<bf16_t*>(b + p.off_x[1]);
    r.A = reinterpret_cast<bf16_t*>(b + p.off_a);
    r.B = reinterpret_cast<bf16_t*>(b + p.off_b);
    r.part = reinterpret_cast<double*>(b + p.off_part);
    return r;
}

// The launch sequence: per chunk the norm and the bf16 cast, then per NS5
// step one launch per product over every chunk of the group.
// Coefficients (a, b, c) of one iteration step X <- a X + (b A + c A A) X.
struct Coeffs {
    float a, b, c;
};
constexpr Coeffs kQuintic{MUON_NS5_A, MUON_NS5_B, MUON_NS5_C};

// What the last step does with O: write it to the outputs, or (apply) update
// the parameters held there, p <- p - lr * O.
struct Update {
    bool apply = false;
    float lr = 0.0f;
    bool bf16_io = false;  // G and the outputs hold bfloat16 (the outputs get X as is)
};

int run_groups(const std::vector<Group>& groups, const Coeffs& k, const Update& up, float mu, int steps, float eps,
               char* ws, hipStream_t stream,
               EventSink* sink, hipEvent_t after_prologue = nullptr) {
    (void)hipGetLastError();  // start from a clean error state
    for (const Group& grp : groups) {
        if (grp.small) {  // one launch: a workgroup per matrix, every chunk a segment
            SmallArgs sa{};
            sa.nseg = static_cast<int>(grp.chunks.size());
            sa.steps = steps;
            sa.apply = up.apply ? 1 : 0;
            sa.mu = mu;
            sa.eps = eps;
            sa.a = k.a;
            sa.b = k.b;
            sa.c = k.c;
            sa.lr = up.lr;
            ConstPtrTable gt{};
            PtrTable ot{}, bt{};
            const bool fused = grp.chunks[0].buf != nullptr;  // the same for every chunk of a call
            int at = 0;
            for (int ci = 0; ci < sa.nseg; ++ci) {
                const Chunk& c = grp.chunks[ci];
                const Ns5Plan& pl = c.plan;
                SmallSeg& sg = sa.seg[ci];
                sg.first = at;
                sg.cnt = pl.cnt;
                sg.rows = static_cast<int>(pl.rows);
                sg.cols = static_cast<int>(pl.cols);
                sg.m = pl.m;
                sg.n = pl.n;
                sg.np = static_cast<int>(round_up(pl.n, 32));
                sg.tall = pl.tall ? 1 : 0;
                for (int i = 0; i < pl.cnt; ++i, ++at) {
                    gt.p[at] = c.G[i];
                    ot.p[at] = c.out[i];
                    if (fused) bt.p[at] = c.buf[i];
                }
            }
            hipError_t e = launch_ns5_small(sa, gt, ot, fused ? &bt : nullptr, up.bf16_io, stream);
            if (e != hipSuccess) return hip_fail(e, "small-matrix launch");
            if (after_prologue && &grp == &groups.front()) {
                hipError_t e = hipEventRecord(after_prologue, stream);
                if (e != hipSuccess) return hip_fail(e, "event record");
            }
            continue;
        }
        const int nseg = static_cast<int>(grp.chunks.size());
        PtrTable out_all{};
        int out_base[kMaxSeg];
        {
            int k = 0;
            for (int ci = 0; ci < nseg; ++ci) {
                out_base[ci] = k;
                for (int i = 0; i < grp.chunks[ci].plan.cnt; ++i) out_all.p[k++] = grp.chunks[ci].out[i];
            }
        }
        // the norm pass over every chunk (fused with the momentum in the Muon
        // step: bf16(u) is staged in X[1], which step 1 overwrites later),
        // then the bf16 cast into X[0], one launch each
        ConstPtrTable g_all{};
        PtrTable b_all{};
        const bool fused = grp.chunks[0].buf != nullptr;  // the same for every chunk of a call
        const bool in16 = up.bf16_io;
        NormLaunch nl{};
        CastLaunch cl{};
        nl.nseg = cl.nseg = nseg;
        int nb_norm = 0, nb_cast = 0;
        int64_t cast_tiles = 0;
        for (const Chunk& c : grp.chunks) {
            const int rows_pad = c.plan.tall ? c.plan.np : c.plan.msym;
            const int cols_pad = c.plan.tall ? c.plan.msym : c.plan.np;
            cast_tiles += static_cast<int64_t>(rows_pad / 64) * (cols_pad / 64) * c.plan.cnt;
        }
        // tiles per cast workgroup: cast_tiles_per_wg(), more if the grid
        // would be too large
        const int64_t cast_cap = max_cast_workgroups();
        int per_wg = static_cast<int>((cast_tiles + cast_cap - 1) / cast_cap);
        if (per_wg < cast_tiles_per_wg()) per_wg = cast_tiles_per_wg();
        for (int ci = 0; ci < nseg; ++ci) {
            const Chunk& c = grp.chunks[ci];
            const Ns5Plan& pl = c.plan;
            ChunkBufs b = bufs_of(ws, c);
            bool vec = (pl.rows * pl.cols) % (in16 ? 8 : 4) == 0;
            for (int i = 0; i < pl.cnt; ++i) {
                g_all.p[out_base[ci] + i] = c.G[i];
                if (fused) b_all.p[out_base[ci] + i] = c.buf[i];
                vec = vec && (reinterpret_cast<uintptr_t>(c.G[i]) & 15u) == 0 &&
                      (!fused || (reinterpret_cast<uintptr_t>(c.buf[i]) & 15u) == 0);
            }
            NormSeg& ns = nl.seg[ci];
            ns.first_block = nb_norm;
            ns.nb = pl.nb;
            ns.ptr_base = out_base[ci];
            ns.vec = vec ? 1 : 0;
            ns.numel = pl.rows * pl.cols;
            ns.chunk = (ns.numel + pl.nb - 1) / pl.nb;
            if (vec) ns.chunk = in16 ? (ns.chunk + 7) / 8 * 8 : (ns.chunk + 3) / 4 * 4;
            ns.ub = fused ? b.X[1] : nullptr;
            ns.ub_mat = static_cast<int64_t>(pl.x_elems);
            ns.partials = b.part;
            nb_norm += pl.nb * pl.cnt;
            CastSeg& cs = cl.seg[ci];
            const int rows_pad = pl.tall ? pl.np : pl.msym;
            const int cols_pad = pl.tall ? pl.msym : pl.np;
            cs.first_block = nb_cast;
            cs.tiles_c = cols_pad / 64;
            cs.tiles_per_mat = (rows_pad / 64) * cs.tiles_c;
            cs.per_wg = per_wg;
            cs.wg_per_mat = (cs.tiles_per_mat + per_wg - 1) / per_wg;
            cs.ptr_base = out_base[ci];
            cs.rows = static_cast<int>(pl.rows);
            cs.cols = static_cast<int>(pl.cols);
            cs.tall = pl.tall ? 1 : 0;
            cs.nb = pl.nb;
            cs.ldx = pl.ldx;
            cs.ub = fused ? b.X[1] : nullptr;
            cs.ub_mat = static_cast<int64_t>(pl.x_elems);
            cs.partials = b.part;
            cs.X = b.X[0];
            cs.x_mat = static_cast<int64_t>(pl.x_elems);
            nb_cast += cs.wg_per_mat * pl.cnt;
        }
        hipError_t e = launch_norm(nl, nb_norm, g_all, fused ? &b_all : nullptr, mu, stream, in16);
        if (e != hipSuccess) return hip_fail(e, fused ? "momentum + norm launch" : "norm (sum of squares) launch");
        e = launch_scale_cast(cl, nb_cast, g_all, fused || in16, eps, stream);
        if (e != hipSuccess) return hip_fail(e, "scale/cast launch");
        if (after_prologue && &grp == &groups.front()) {
            e = hipEventRecord(after_prologue, stream);
            if (e != hipSuccess) return hip_fail(e, "event record");
        }
        if (steps == 0) {
            for (int ci = 0; ci < nseg; ++ci) {
                const Chunk& c = grp.chunks[ci];
                PtrTable ot{};
                for (int i = 0; i < c.plan.cnt; ++i) ot.p[i] = c.out[i];
                e = launch_copy_out(c.plan, c.plan.cnt, bufs_of(ws, c).X[0], ot, stream, up.apply, up.lr,
                                    up.bf16_io);
                if (e != hipSuccess) return hip_fail(e, "copy-out launch");
            }
        }
        if (steps == 0) continue;

        // tile of the a X + B X product (rows x columns of the output).  With
        // 128-tiled groups a larger tile wherever every chunk's padded sizes
        // allow it: 256 x 256 (8 waves; half the operand bytes per flop of the
        // 128 tile, measured fastest on the 768-class shapes), else 256 x 128;
        // otherwise the group's square tile.  MUON_BX_TILE=128 keeps the square
        // tile and MUON_BX_TILE=256128 asks for 256 x 128 (for tuning sweeps).
        int bx_tm = grp.tile, bx_tn = grp.tile;
        if (grp.tile == 128) {
            static const int want = [] {
                const char* e = getenv("MUON_BX_TILE");
                return e ? atoi(e) : 0;
            }();
            bool rows256 = true, cols256 = true, rows192 = true;
            for (const Chunk& c : grp.chunks) {
                rows256 = rows256 && c.plan.mp % 256 == 0;
                cols256 = cols256 && c.plan.np % 256 == 0;
                rows192 = rows192 && c.plan.mp % 192 == 0;
            }
            if (want == 192256 && rows192 && cols256) {
                bx_tm = 192;
                bx_tn = 256;
            } else if (want != 128 && want != 256128 && rows256 && cols256) {
                bx_tm = bx_tn = 256;
            } else if (want != 128 && rows256) {
                bx_tm = 256;
                bx_tn = 128;
            }
        }
        // tile of X X^T: 256 (8 waves; half the operand bytes per flop of the
        // 128 tile) wherever every chunk's padded m allows it, else the
        // group's (MUON_SYRK_TILE=128 keeps the group's, for tuning sweeps).
        // Its K (= n) differs between segments, and 256 tiles are few, so
        // its segments go longest K first: the last workgroups to start are
        // the shortest.
        int syrk_tile = grp.tile;
        {
            static const int want = [] {
                const char* e = getenv("MUON_SYRK_TILE");
                return e ? atoi(e) : 0;
            }();
            bool rows256 = true;
            for (const Chunk& c : grp.chunks) rows256 = rows256 && c.plan.mp % 256 == 0;
            if (want != 128 && grp.tile == 128 && rows256) syrk_tile = 256;
            if (grp.chunks[0].plan.sym_tile == 192) syrk_tile = 192;  // the same for every chunk of a group
        }
        int syrk_order[kMaxSeg];
        for (int ci = 0; ci < nseg; ++ci) syrk_order[ci] = ci;
        for (int a = 1; a < nseg; ++a)  // insertion sort by n, descending (stable)
            for (int b = a; b > 0 && grp.chunks[syrk_order[b]].plan.n > grp.chunks[syrk_order[b - 1]].plan.n; --b) {
                const int t = syrk_order[b];
                syrk_order[b] = syrk_order[b - 1];
                syrk_order[b - 1] = t;
            }
        // X[1]'s rows past mp (the symmetric products' padding) are never
        // written by a X + B X: they start at zero (X[0]'s by the cast)
        for (const Chunk& c : grp.chunks) {
            if (c.plan.msym <= c.plan.mp) continue;
            e = launch_zero_rows(bufs_of(ws, c).X[1], static_cast<int64_t>(c.plan.x_elems), c.plan.cnt, c.plan.mp,
                                 c.plan.msym, c.plan.ldx, stream);
            if (e != hipSuccess) return hip_fail(e, "padding reset launch");
        }
        int cur = 0;
        for (int s = 0; s < steps; ++s) {
            const int nxt = cur ^ 1;
            const bool last = (s == steps - 1);
            GemmLaunch syrk{}, aab{}, bx{};
            syrk.nseg = aab.nseg = bx.nseg = nseg;
            int nb_syrk = 0, nb_sym = 0, nb_bx = 0;
            for (int k = 0; k < nseg; ++k) {  // A = X X^T, longest K first
                const Chunk& c = grp.chunks[syrk_order[k]];
                const Ns5Plan& pl = c.plan;
                ChunkBufs b = bufs_of(ws, c);
                const int tiles_m = pl.msym / syrk_tile;
                const int64_t xe = static_cast<int64_t>(pl.x_elems);
                GemmArgs& g1 = syrk.seg[k];
                g1.first_block = nb_syrk;
                g1.out_base = out_base[syrk_order[k]];
                g1.P = b.X[cur]; g1.p_mat = xe; g1.ldp = pl.ldx;
                g1.Q = b.X[cur]; g1.q_mat = xe; g1.ldq = pl.ldx;
                g1.kpad = static_cast<int>(round_up(pl.n, 64));
                g1.tiles = tiles_m; g1.tiles_n = tiles_m; g1.tiles_per_mat = tiles_m * (tiles_m + 1) / 2;
                g1.C = b.A; g1.c_mat = static_cast<int64_t>(pl.a_elems); g1.ldc = pl.lda;
                g1.m = pl.m; g1.n = pl.n; g1.tall = pl.tall ? 1 : 0;
                nb_syrk += g1.tiles_per_mat * pl.cnt;
            }
            for (int ci = 0; ci < nseg; ++ci) {
                const Chunk& c = grp.chunks[ci];
                const Ns5Plan& pl = c.plan;
                ChunkBufs b = bufs_of(ws, c);
                const int tiles_m = pl.msym / pl.sym_tile;
                const int64_t xe = static_cast<int64_t>(pl.x_elems);
                const int64_t ae = static_cast<int64_t>(pl.a_elems);
                // B = b A + c A A  (the upper triangle of tiles)
                GemmArgs& g2 = aab.seg[ci];
                g2.first_block = nb_sym;
                g2.out_base = out_base[ci];
                g2.tiles = tiles_m; g2.tiles_n = tiles_m; g2.tiles_per_mat = tiles_m * (tiles_m + 1) / 2;
                g2.m = pl.m; g2.n = pl.n; g2.tall = pl.tall ? 1 : 0;
                g2.P = b.A; g2.p_mat = ae; g2.ldp = pl.lda;
                g2.Q = b.A; g2.q_mat = ae; g2.ldq = pl.lda;
                g2.kpad = static_cast<int>(round_up(pl.m, 64));
                g2.C = b.B; g2.c_mat = ae; g2.ldc = pl.lda;
                g2.E = b.A; g2.e_mat = ae; g2.lde = pl.lda;
                g2.alpha = k.b; g2.beta = k.c;
                nb_sym += g2.tiles_per_mat * pl.cnt;
                // X' = a X + B X
                GemmArgs& g3 = bx.seg[ci];
                g3.first_block = nb_bx;
                g3.out_base = out_base[ci];
                g3.P = b.B; g3.p_mat = ae; g3.ldp = pl.lda;
                g3.Q = b.X[cur]; g3.q_mat = xe; g3.ldq = pl.ldx;  // NN: X read as is
                g3.kpad = static_cast<int>(round_up(pl.m, 64));
                const int btm = pl.mp / bx_tm, btn = pl.np / bx_tn;
                g3.tiles = btm; g3.tiles_n = btn; g3.tiles_per_mat = btm * btn;
                g3.band = band_rows(btm);
                g3.E = b.X[cur]; g3.e_mat = xe; g3.lde = pl.ldx;
                g3.alpha = k.a; g3.beta = 1.0f;
                g3.C = b.X[nxt]; g3.c_mat = xe; g3.ldc = pl.ldx;
                g3.m = pl.m; g3.n = pl.n; g3.tall = pl.tall ? 1 : 0;
                g3.apply = up.apply ? 1 : 0; g3.lr = up.lr; g3.out16 = up.bf16_io ? 1 : 0;
                nb_bx += g3.tiles_per_mat * pl.cnt;
            }
            // the symmetric products' K differs between segments (X X^T: n);
            // deal whole matrices over the XCDs when the tile counts agree
            for (GemmLaunch* L : {&syrk, &aab}) {
                int tpm = L->seg[0].tiles_per_mat;
                for (int ci = 1; ci < nseg; ++ci)
                    if (L->seg[ci].tiles_per_mat != tpm) tpm = 0;
                L->interleave_tpm = tpm;
            }
            // X' of a large launch goes out with streaming stores, so that it
            // does not displace the operands its tiles share in the caches;
            // a small one (that the next X X^T finds in the caches) does not:
            // measured on one box, the 124M set (170 MB of X') gained 13 us
            // per step, one 4096^2 matrix (34 MB) lost 2%
            int64_t x_bytes = 0;
            for (const Chunk& c : grp.chunks)
                x_bytes += static_cast<int64_t>(c.plan.x_elems) * c.plan.cnt * 2;
            bx.stream_out = x_bytes >= kStreamOutBytes ? 1 : 0;
            e = launch_gemm(GEMM_SYRK, syrk_tile, syrk_tile, syrk, nb_syrk, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "X X^T launch");
            const int aab_tile = grp.chunks[0].plan.sym_tile;
            e = launch_gemm(GEMM_AAB, aab_tile, aab_tile, aab, nb_sym, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "b A + c A A launch");
            const bool timed = sink && !last && sink->recorded < sink->pairs;
            if (timed) {
                e = hipEventRecord(static_cast<hipEvent_t>(sink->events[2 * sink->recorded]), stream);
                if (e != hipSuccess) return hip_fail(e, "event record");
            }
            e = launch_gemm(last ? GEMM_BX_FINAL : GEMM_BX, bx_tm, bx_tn, bx, nb_bx, last ? &out_all : nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "a X + B X launch");
            if (timed) {
                e = hipEventRecord(static_cast<hipEvent_t>(sink->events[2 * sink->recorded + 1]), stream);
                if (e != hipSuccess) return hip_fail(e, "event record");
                ++sink->recorded;
            }
            cur = nxt;
        }
    }
    return ok();
}

// Same-shape matrices of a grouped call, validated.
int grouped_segment(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                    Segment* seg) {
    if (!G || !out) return fail(MUON_ERR_INVALID_ARG, "null pointer array");
    if (count < 1) return fail(MUON_ERR_INVALID_ARG, "count must be >= 1 (got %lld)", (long long)count);
    if (rows < 1 || cols < 1)
        return fail(MUON_ERR_INVALID_ARG, "rows and cols must be >= 1 (got %lld x %lld)", (long long)rows,
                    (long long)cols);
    for (int64_t i = 0; i < count; ++i)
        if (!G[i] || !out[i]) return fail(MUON_ERR_INVALID_ARG, "null matrix pointer at index %lld", (long long)i);
    seg->rows = rows;
    seg->cols = cols;
    seg->count = count;
    seg->G = G;
    seg->out = out;
    seg->buf = nullptr;
    return MUON_OK;
}

// A mixed-shape batch bucketed into segments by shape (in order of first
// appearance), with per-segment pointer arrays held in `gs` / `os`.
int batched_segments(const float* const* G, float* const* out, float* const* buf, const int64_t* rows,
                     const int64_t* cols, int64_t count, bool need_ptrs, std::vector<Segment>* segs,
                     std::vector<std::vector<const float*>>* gs, std::vector<std::vector<float*>>* os,
                     std::vector<std::vector<float*>>* bs) {
    if (!rows || !cols) return fail(MUON_ERR_INVALID_ARG, "null shape array");
    if (need_ptrs && (!G || !out)) return fail(MUON_ERR_INVALID_ARG, "null pointer array");
    if (count < 1) return fail(MUON_ERR_INVALID_ARG, "count must be >= 1 (got %lld)", (long long)count);
    std::vector<int64_t> key_r, key_c;
    std::vector<int> which(static_cast<size_t>(count));
    for (int64_t i = 0; i < count; ++i) {
        if (rows[i] < 1 || cols[i] < 1)
            return fail(MUON_ERR_INVALID_ARG, "matrix %lld: rows and cols must be >= 1 (got %lld x %lld)",
                        (long long)i, (long long)rows[i], (long long)cols[i]);
        if (need_ptrs && (!G[i] || !out[i]))
            return fail(MUON_ERR_INVALID_ARG, "null matrix pointer at index %lld", (long long)i);
        if (need_ptrs && buf && !buf[i])
            return fail(MUON_ERR_INVALID_ARG, "null momentum buffer at index %lld", (long long)i);
        if (need_ptrs && buf && buf[i] == out[i])
            return fail(MUON_ERR_INVALID_ARG, "out must not alias the momentum buffer (index %lld)", (long long)i);
        int k = 0;
        while (k < static_cast<int>(key_r.size()) && !(key_r[k] == rows[i] && key_c[k] == cols[i])) ++k;
        if (k == static_cast<int>(key_r.size())) {
            key_r.push_back(rows[i]);
            key_c.push_back(cols[i]);
        }
        which[static_cast<size_t>(i)] = k;
    }
    const size_t nk = key_r.size();
    gs->assign(nk, {});
    os->assign(nk, {});
    bs->assign(nk, {});
    std::vector<int64_t> cnt(nk, 0);
    for (int64_t i = 0; i < count; ++i) {
        const int k = which[static_cast<size_t>(i)];
        ++cnt[k];
        if (need_ptrs) {
            (*gs)[k].push_back(G[i]);
            (*os)[k].push_back(out[i]);
            if (buf) (*bs)[k].push_back(buf[i]);
        }
    }
    segs->clear();
    for (size_t k = 0; k < nk; ++k) {
        Segment sg;
        sg.rows = key_r[k];
        sg.cols = key_c[k];
        sg.count = cnt[k];
        sg.G = need_ptrs ? (*gs)[k].data() : nullptr;
        sg.out = need_ptrs ? (*os)[k].data() : nullptr;
        sg.buf = (need_ptrs && buf) ? (*bs)[k].data() : nullptr;
        segs->push_back(sg);
    }
    return MUON_OK;
}

// Multi-stream schedule of a large batch.  The step's prologue (momentum and
// the norm, then the cast) streams HBM while the products keep the matrix
// cores busy, so a batch runs as K parts: the first on the caller's stream,
// part p on side stream p of the library (kept per device), started once part
// p - 1's prologue is done, so that each part's prologue overlaps the other
// parts' products.  Every segment's matrices are dealt round-robin to the
// parts (all get the same mix of shapes).  Each part is an ordinary batch, so
// every matrix gets bitwise what it gets alone.  Measured on one box, two
// runs each, 1 / 2 / 3 / 4 parts: the GPT-2 124M step 1.789-1.795 /
// 1.732-1.752 / 1.695-1.698 / 1.734-1.741 ms; the 16 extreme-aspect matrices
// 9.54-9.58 / 9.17-9.19 / 10.58-10.59 / 10.55-10.60 ms.  More parts pay where
// the prologue is a larger share of the work: its cost grows with the
// elements, the products' with the elements times the short side m, so K = 3
// where the batch holds at least 4e-5 elements per nominal flop (m up to about
// 1000; the 124M set, 5.6e-5), else 2 (the extreme-aspect set, 2.2e-5): then
// 1.685-1.693 and 9.08-9.13 ms in three runs.  Taken for a batch of one launch
// group with at least 2 K matrices and 5e11 nominal flops.  MUON_SPLIT=0 turns
// it off, MUON_SPLIT=2..4 forces K (for tuning).
constexpr double kSplitMinFlops = 5e11;  // nominal NS5 flops of a batch worth splitting
constexpr double kThreePartsRatio = 4e-5;  // elements per nominal flop from which K = 3
constexpr int kMaxParts = 4;
// K forced from the environment (0: not forced; 1: no split)
int split_parts_forced() {
    static const int k = [] {
        const char* e = getenv("MUON_SPLIT");
        if (!e) return 0;
        const int v = atoi(e);
        return v <= 1 ? 1 : (v > kMaxParts ? kMaxParts : v);
    }();
    return k;
}
struct Parts {
    int k = 1;
    std::vector<Segment> segs[kMaxParts];
    std::vector<std::vector<const float*>> gs[kMaxParts];
    std::vector<std::vector<float*>> os[kMaxParts], bs[kMaxParts];
};
// Parts for a batch (1: no split).
int split_parts(const std::vector<Segment>& segs) {
    const int forced = split_parts_forced();
    if (forced == 1) return 1;
    double flops = 0.0, elems = 0.0;
    int64_t mats = 0;
    for (const Segment& sg : segs) {
        const double m = static_cast<double>(sg.rows < sg.cols ? sg.rows : sg.cols);
        const double n = static_cast<double>(sg.rows < sg.cols ? sg.cols : sg.rows);
        flops += static_cast<double>(sg.count) * 5.0 * (4.0 * m * m * n + 2.0 * m * m * m);
        elems += static_cast<double>(sg.count) * m * n;
        mats += sg.count;
    }
    const int k = forced ? forced : (elems >= kThreePartsRatio * flops ? 3 : 2);
    return (mats >= 2 * k && flops >= kSplitMinFlops) ? k : 1;
}
// Deals the matrices to the k parts round-robin, in segment order and
// without restarting at each segment: matrix i of a segment goes to part
// (s + i) mod k, s being the number of matrices in the segments before it
// (mod k).  Each segment is shared as evenly as it can be, and every part
// gets at least floor(count / k) matrices.
void split_parts_of(const std::vector<Segment>& segs, bool ptrs, int k, Parts* pt) {
    pt->k = k;
    for (int part = 0; part < k; ++part) {
        pt->segs[part].clear();
        pt->gs[part].assign(segs.size(), {});
        pt->os[part].assign(segs.size(), {});
        pt->bs[part].assign(segs.size(), {});
    }
    int start = 0;  // the part that takes the segment's first matrix
    for (size_t q = 0; q < segs.size(); ++q) {
        const Segment& sg = segs[q];
        for (int part = 0; part < k; ++part) {
            const int64_t first = (part - start + k) % k;  // the segment's first matrix in this part
            const int64_t cnt = sg.count > first ? (sg.count - first + k - 1) / k : 0;
            if (cnt == 0) continue;
            if (ptrs) {
                for (int64_t i = first; i < sg.count; i += k) {
                    pt->gs[part][q].push_back(sg.G[i]);
                    pt->os[part][q].push_back(sg.out[i]);
                    if (sg.buf) pt->bs[part][q].push_back(sg.buf[i]);
                }
            }
            Segment ps = sg;
            ps.count = cnt;
            ps.G = ptrs ? pt->gs[part][q].data() : nullptr;
            ps.out = ptrs ? pt->os[part][q].data() : nullptr;
            ps.buf = (ptrs && sg.buf) ? pt->bs[part][q].data() : nullptr;
            pt->segs[part].push_back(ps);
        }
        start = static_cast<int>((start + sg.count) % k);
    }
}
// The plan of a batch: its launch groups, or those of its parts (each part's
// workspace after the previous one's).  Returns a status.
struct BatchPlan {
    int parts = 1;
    Parts split;
    std::vector<Group> groups[kMaxParts];
    size_t off[kMaxParts] = {};
    size_t bytes = 0;
};
int plan_batch(const std::vector<Segment>& segs, bool ptrs, bool allow_split, BatchPlan* bp) {
    int st = plan_groups(segs.data(), static_cast<int>(segs.size()), &bp->groups[0]);
    if (st) return st;
    bp->bytes = groups_bytes(bp->groups[0]);
    bp->parts = 1;
    // (a batch of several launch groups already runs them one after another;
    // measured, the 1.5B set's two groups lost 0.9% as two halves and 1.3%
    // as its two groups on two streams)
    const int k = allow_split && bp->groups[0].size() == 1 ? split_parts(segs) : 1;
    if (k < 2) return MUON_OK;
    bp->parts = k;
    split_parts_of(segs, ptrs, k, &bp->split);
    size_t off = 0;
    for (int part = 0; part < k; ++part) {
        st = plan_groups(bp->split.segs[part].data(), static_cast<int>(bp->split.segs[part].size()),
                         &bp->groups[part]);
        if (st) return st;
        bp->off[part] = off;
        off = align256(off + groups_bytes(bp->groups[part]));
    }
    bp->bytes = off;
    return MUON_OK;
}

// The side streams and events of the multi-stream schedule, per device, made
// on first use (default priority; the streams do not synchronise with the
// null stream).  Calls that use them enqueue under one lock, since the events
// are shared.
struct SideStreams {
    std::once_flag once;
    bool ok = false;
    hipStream_t stream[kMaxParts] = {};                     // [0] unused (the caller's)
    hipEvent_t fork = nullptr, prologue[kMaxParts] = {}, join[kMaxParts] = {};
};
SideStreams g_side[kMaxDevices];
std::mutex g_side_lock;
SideStreams* side_streams() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return nullptr;
    }
    SideStreams* s = &g_side[dev];
    std::call_once(s->once, [s] {
        bool ok = hipEventCreateWithFlags(&s->fork, hipEventDisableTiming) == hipSuccess;
        for (int p = 0; p < kMaxParts && ok; ++p) {
            if (p > 0) ok = hipStreamCreateWithFlags(&s->stream[p], hipStreamNonBlocking) == hipSuccess;
            ok = ok && hipEventCreateWithFlags(&s->prologue[p], hipEventDisableTiming) == hipSuccess &&
                 hipEventCreateWithFlags(&s->join[p], hipEventDisableTiming) == hipSuccess;
        }
        s->ok = ok;
        if (!ok) (void)hipGetLastError();
    });
    return s->ok ? s : nullptr;
}

int run_batched(const float* const* G, float* const* out, float* const* buf, float mu, const int64_t* rows,
                const int64_t* cols, int64_t count, int steps, float eps, void* ws, size_t ws_bytes,
                hipStream_t stream, EventSink* sink, const Coeffs& k = kQuintic, const Update& up = Update{}) {
    int st = check_common(steps, eps);
    if (st) return st;
    std::vector<Segment> segs;
    std::vector<std::vector<const float*>> gs;
    std::vector<std::vector<float*>> os, bs;
    st = batched_segments(G, out, buf, rows, cols, count, true, &segs, &gs, &os, &bs);
    if (st) return st;
    // (the measurement hook times whole launches: never split)
    BatchPlan bp;
    st = plan_batch(segs, true, sink == nullptr, &bp);
    if (st) return st;
    st = check_workspace(ws, ws_bytes, bp.bytes);
    if (st) return st;
    char* w = static_cast<char*>(ws);
    SideStreams* side = bp.parts > 1 ? side_streams() : nullptr;
    if (!side) {
        // one stream: the parts (when planned) one after the other
        for (int part = 0; part < bp.parts; ++part) {
            st = run_groups(bp.groups[part], k, up, mu, steps, eps, w + bp.off[part], stream,
                            part == 0 ? sink : nullptr);
            if (st) return st;
        }
        return ok();
    }
    std::lock_guard<std::mutex> lock(g_side_lock);
    hipError_t e = hipEventRecord(side->fork, stream);
    if (e != hipSuccess) return hip_fail(e, "side stream fork");
    for (int part = 0; part < bp.parts; ++part) {
        hipStream_t s = part == 0 ? stream : side->stream[part];
        if (part > 0) {
            // after everything before the call, and after the previous
            // part's prologue
            e = hipStreamWaitEvent(s, side->fork, 0);
            if (e == hipSuccess) e = hipStreamWaitEvent(s, side->prologue[part - 1], 0);
            if (e != hipSuccess) return hip_fail(e, "side stream wait");
        }
        st = run_groups(bp.groups[part], k, up, mu, steps, eps, w + bp.off[part], s, nullptr,
                        part + 1 < bp.parts ? side->prologue[part] : nullptr);
        if (st) return st;
    }
    for (int part = 1; part < bp.parts; ++part) {
        e = hipEventRecord(side->join[part], side->stream[part]);
        if (e == hipSuccess) e = hipStreamWaitEvent(stream, side->join[part], 0);
        if (e != hipSuccess) return hip_fail(e, "side stream join");
    }
    return ok();
}

// ---- the iteration carried in float32 (f32_iter.hip)
//
// Per pass of up to kMaxGroup same-shaped matrices the workspace holds float32
// X[2] (mp x ldx), A and B (mp x lda) and the float64 norm partials; m and n
// are padded to the 128 tile, rows carry a 32-float skew.  Passes run one
// after another, each reusing the workspace from its start.
constexpr int kF32Tile = 128;

struct F32Plan {
    int64_t rows, cols;
    int m, n, mp, np, ldx, lda, nb, cnt;
    bool tall;
    size_t off_x[2], off_a, off_b, off_part, bytes;
};

bool plan_f32(int64_t rows, int64_t cols, int64_t count, F32Plan* p) {
    if (rows < 1 || cols < 1 || count < 1) return false;
    const int64_t m = rows < cols ? rows : cols;
    const int64_t n = rows < cols ? cols : rows;
    if (m > MUON_NS5_MAX_SHORT || n > MUON_NS5_MAX_LONG) return false;
    p->rows = rows;
    p->cols = cols;
    p->m = static_cast<int>(m);
    p->n = static_cast<int>(n);
    p->tall = rows > cols;
    p->mp = static_cast<int>(round_up(m, kF32Tile));
    p->np = static_cast<int>(round_up(n, kF32Tile));
    p->ldx = p->np + 32;
    p->lda = p->mp + 32;
    int64_t nb = (rows * cols + 16383) / 16384;
    p->nb = static_cast<int>(nb < 1 ? 1 : (nb > kMaxNormBlocks ? kMaxNormBlocks : nb));
    const int64_t tiles = static_cast<int64_t>(p->mp / kF32Tile) * (p->np / kF32Tile);
    int64_t cnt = count < kMaxGroup ? count : kMaxGroup;
    if (cnt * tiles > kMaxWorkgroups) cnt = kMaxWorkgroups / tiles;
    if (cnt < 1) return false;
    p->cnt = static_cast<int>(cnt);
    const size_t xb = align256(static_cast<size_t>(cnt) * p->mp * p->ldx * sizeof(float));
    const size_t ab = align256(static_cast<size_t>(cnt) * p->mp * p->lda * sizeof(float));
    size_t off = 0;
    p->off_x[0] = off; off += xb;
    p->off_x[1] = off; off += xb;
    p->off_a = off; off += ab;
    p->off_b = off; off += ab;
    p->off_part = off; off += align256(static_cast<size_t>(cnt) * p->nb * sizeof(double));
    p->bytes = off;
    return true;
}

// Workspace bytes of a validated batch: the largest pass.
int f32_bytes(const std::vector<Segment>& segs, size_t* bytes) {
    *bytes = 0;
    for (const Segment& sg : segs) {
        F32Plan pl;
        if (!plan_f32(sg.rows, sg.cols, sg.count, &pl))
            return fail(MUON_ERR_UNSUPPORTED, "shape %lld x %lld is beyond the supported limits", (long long)sg.rows,
                        (long long)sg.cols);
        if (pl.bytes > *bytes) *bytes = pl.bytes;
    }
    return MUON_OK;
}

int run_f32(const float* const* G, float* const* out, const int64_t* rows, const int64_t* cols, int64_t count,
            int steps, const Coeffs& k, float eps, void* ws, size_t ws_bytes, hipStream_t stream) {
    int st = check_common(steps, eps);
    if (st) return st;
    std::vector<Segment> segs;
    std::vector<std::vector<const float*>> gs;
    std::vector<std::vector<float*>> os, bs;
    st = batched_segments(G, out, nullptr, rows, cols, count, true, &segs, &gs, &os, &bs);
    if (st) return st;
    size_t need = 0;
    st = f32_bytes(segs, &need);
    if (st) return st;
    st = check_workspace(ws, ws_bytes, need);
    if (st) return st;
    (void)hipGetLastError();  // start from a clean error state
    char* base = static_cast<char*>(ws);
    for (const Segment& sg : segs) {
        for (int64_t start = 0; start < sg.count;) {
            F32Plan pl;
            plan_f32(sg.rows, sg.cols, sg.count - start, &pl);
            const int cnt = pl.cnt;
            ConstPtrTable gt{};
            PtrTable ot{};
            bool vec = (pl.rows * pl.cols) % 4 == 0;
            for (int i = 0; i < cnt; ++i) {
                gt.p[i] = sg.G[start + i];
                ot.p[i] = sg.out[start + i];
                vec = vec && (reinterpret_cast<uintptr_t>(gt.p[i]) & 15u) == 0;
            }
            float* X[2] = {reinterpret_cast<float*>(base + pl.off_x[0]), reinterpret_cast<float*>(base + pl.off_x[1])};
            float* A = reinterpret_cast<float*>(base + pl.off_a);
            float* B = reinterpret_cast<float*>(base + pl.off_b);
            double* part = reinterpret_cast<double*>(base + pl.off_part);
            // the norm's float64 partial sums (the pass the bf16 iteration uses)
            NormLaunch nl{};
            nl.nseg = 1;
            NormSeg& ns = nl.seg[0];
            ns.first_block = 0;
            ns.nb = pl.nb;
            ns.ptr_base = 0;
            ns.vec = vec ? 1 : 0;
            ns.numel = pl.rows * pl.cols;
            ns.chunk = (ns.numel + pl.nb - 1) / pl.nb;
            if (vec) ns.chunk = (ns.chunk + 3) / 4 * 4;
            ns.ub = nullptr;
            ns.ub_mat = 0;
            ns.partials = part;
            hipError_t e = launch_norm(nl, pl.nb * cnt, gt, nullptr, 0.0f, stream);
            if (e != hipSuccess) return hip_fail(e, "norm (sum of squares) launch");
            F32Scale sc{};
            sc.partials = part;
            sc.nb = pl.nb;
            sc.rows = static_cast<int>(pl.rows);
            sc.cols = static_cast<int>(pl.cols);
            sc.tall = pl.tall ? 1 : 0;
            sc.eps = eps;
            sc.cnt = cnt;
            if (steps == 0) {  // X0 itself, in G's orientation
                sc.to_out = 1;
                sc.tiles_c = static_cast<int>((pl.cols + 31) / 32);
                sc.tiles_per_mat = static_cast<int>((pl.rows + 31) / 32) * sc.tiles_c;
                e = launch_f32_scale(sc, gt, &ot, stream);
                if (e != hipSuccess) return hip_fail(e, "float32 scale launch");
                start += cnt;
                continue;
            }
            sc.to_out = 0;
            sc.X = X[0];
            sc.x_mat = static_cast<int64_t>(pl.mp) * pl.ldx;
            sc.ldx = pl.ldx;
            sc.tiles_c = pl.np / 32;
            sc.tiles_per_mat = (pl.mp / 32) * sc.tiles_c;
            e = launch_f32_scale(sc, gt, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "float32 scale launch");
            const int tm = pl.mp / kF32Tile, tn = pl.np / kF32Tile;
            const int64_t xe = static_cast<int64_t>(pl.mp) * pl.ldx, ae = static_cast<int64_t>(pl.mp) * pl.lda;
            int cur = 0;
            for (int s = 0; s < steps; ++s) {
                const int nxt = cur ^ 1;
                const bool last = s == steps - 1;
                F32Gemm g1{};  // A = X X^T
                g1.P = X[cur]; g1.p_mat = xe; g1.ldp = pl.ldx;
                g1.Q = X[cur]; g1.q_mat = xe; g1.ldq = pl.ldx;
                g1.C = A; g1.c_mat = ae; g1.ldc = pl.lda;
                g1.K = pl.np;
                g1.tiles = tm; g1.tiles_n = tm; g1.tiles_per_mat = tm * (tm + 1) / 2;
                e = launch_f32_gemm(GEMM_SYRK, g1, g1.tiles_per_mat * cnt, nullptr, stream);
                if (e != hipSuccess) return hip_fail(e, "float32 X X^T launch");
                F32Gemm g2{};  // B = b A + c A A
                g2.P = A; g2.p_mat = ae; g2.ldp = pl.lda;
                g2.Q = A; g2.q_mat = ae; g2.ldq = pl.lda;
                g2.C = B; g2.c_mat = ae; g2.ldc = pl.lda;
                g2.E = A; g2.e_mat = ae; g2.lde = pl.lda;
                g2.alpha = k.b; g2.beta = k.c;
                g2.K = pl.mp;
                g2.tiles = tm; g2.tiles_n = tm; g2.tiles_per_mat = tm * (tm + 1) / 2;
                e = launch_f32_gemm(GEMM_AAB, g2, g2.tiles_per_mat * cnt, nullptr, stream);
                if (e != hipSuccess) return hip_fail(e, "float32 b A + c A A launch");
                F32Gemm g3{};  // X' = a X + B X
                g3.P = B; g3.p_mat = ae; g3.ldp = pl.lda;
                g3.Q = X[cur]; g3.q_mat = xe; g3.ldq = pl.ldx;
                g3.C = X[nxt]; g3.c_mat = xe; g3.ldc = pl.ldx;
                g3.E = X[cur]; g3.e_mat = xe; g3.lde = pl.ldx;
                g3.alpha = k.a;
                g3.K = pl.mp;
                g3.tiles = tm; g3.tiles_n = tn; g3.tiles_per_mat = tm * tn;
                g3.m = pl.m; g3.n = pl.n; g3.tall = pl.tall ? 1 : 0;
                e = launch_f32_gemm(last ? GEMM_BX_FINAL : GEMM_BX, g3, g3.tiles_per_mat * cnt, last ? &ot : nullptr,
                                    stream);
                if (e != hipSuccess) return hip_fail(e, "float32 a X + B X launch");
                cur = nxt;
            }
            start += cnt;
        }
    }
    return ok();
}

// ---- U V^T through an SVD on the GPU (polar_svd.hip)
//
// Per pass of up to kMaxGroup same-shaped matrices: [W | J] (m_pad rows of
// ld floats each), then per matrix two unsigned counters and m_pad float64
// row lengths.  m is padded to whole pairs of 32-row blocks (a multiple of
// 64, at least 64), n to a multiple of 64.
struct SvdPlan {
    int m, n, m_pad, n_pad, ld, cnt;
    bool tall;
    size_t off_wj, off_state, off_len, bytes;
};

bool plan_svd(int64_t rows, int64_t cols, int64_t count, SvdPlan* p) {
    if (rows < 1 || cols < 1 || count < 1) return false;
    const int64_t m = rows < cols ? rows : cols;
    const int64_t n = rows < cols ? cols : rows;
    if (m > MUON_POLAR_MAX_SHORT || n > MUON_NS5_MAX_LONG) return false;
    p->m = static_cast<int>(m);
    p->n = static_cast<int>(n);
    p->tall = rows > cols;
    p->m_pad = static_cast<int>(round_up(m < 64 ? 64 : m, 64));
    p->n_pad = static_cast<int>(round_up(n, 64));
    p->ld = p->n_pad + p->m_pad;
    p->cnt = static_cast<int>(count < kMaxGroup ? count : kMaxGroup);
    const size_t wj = align256(static_cast<size_t>(p->cnt) * p->m_pad * p->ld * sizeof(float));
    p->off_wj = 0;
    p->off_state = wj;
    p->off_len = p->off_state + align256(static_cast<size_t>(p->cnt) * 2 * sizeof(unsigned int));
    p->bytes = p->off_len + align256(static_cast<size_t>(p->cnt) * p->m_pad * sizeof(double));
    return true;
}

int run_polar_svd(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                  int max_sweeps, void* ws, size_t ws_bytes, hipStream_t stream) {
    Segment sg;
    int st = grouped_segment(G, out, count, rows, cols, &sg);
    if (st) return st;
    if (max_sweeps < 1 || max_sweeps > 64)
        return fail(MUON_ERR_INVALID_ARG, "max_sweeps must be in 1 .. 64 (got %d)", max_sweeps);
    SvdPlan pl;
    if (!plan_svd(rows, cols, count, &pl))
        return fail(MUON_ERR_UNSUPPORTED, "shape %lld x %lld is beyond the supported limits", (long long)rows,
                    (long long)cols);
    st = check_workspace(ws, ws_bytes, pl.bytes);
    if (st) return st;
    (void)hipGetLastError();
    char* base = static_cast<char*>(ws);
    for (int64_t start = 0; start < count; start += pl.cnt) {
        const int cnt = static_cast<int>(count - start < pl.cnt ? count - start : pl.cnt);
        ConstPtrTable gt{};
        PtrTable ot{};
        for (int i = 0; i < cnt; ++i) {
            gt.p[i] = G[start + i];
            ot.p[i] = out[start + i];
        }
        SvdArgs a{};
        a.wj = reinterpret_cast<float*>(base + pl.off_wj);
        a.mat_elems = static_cast<int64_t>(pl.m_pad) * pl.ld;
        a.ld = pl.ld;
        a.m = pl.m;
        a.n = pl.n;
        a.m_pad = pl.m_pad;
        a.n_pad = pl.n_pad;
        a.blocks = pl.m_pad / 32;
        a.count = cnt;
        a.tall = pl.tall ? 1 : 0;
        a.tol = kSvdTol;
        a.rank_tol = kSvdRankTol;
        a.state = reinterpret_cast<unsigned int*>(base + pl.off_state);
        a.inv_len = reinterpret_cast<double*>(base + pl.off_len);
        hipError_t e = launch_svd_init(a, gt, stream);
        if (e != hipSuccess) return hip_fail(e, "SVD set-up launch");
        for (int sw = 0; sw < max_sweeps; ++sw) {
            e = launch_svd_sweep(a, sw == max_sweeps - 1, stream);
            if (e != hipSuccess) return hip_fail(e, "SVD sweep launch");
        }
        e = launch_svd_finish(a, ot, stream);
        if (e != hipSuccess) return hip_fail(e, "U V^T launch");
    }
    return ok();
}

}  // namespace

// The Muon step (momentum + NS5) on a workspace of fixed size ws_bytes:
// launch groups are cut so that each fits, and a matrix that does not fit on
// its own is an error (nothing enqueued).  `workspace` supplies the address
// once the arguments have been validated.  Results are bitwise those of
// muon_momentum_ns5_batched, whose matrices do not depend on their batch.
int run_momentum_ns5_fixed_workspace(const float* const* g, float* const* buf, float* const* out,
                                     const int64_t* rows, const int64_t* cols, int64_t count, float mu, int steps,
                                     float eps, size_t ws_bytes, int (*workspace)(void**), hipStream_t stream) {
    if (!buf) return fail(MUON_ERR_INVALID_ARG, "null momentum buffer array");
    int st = check_common(steps, eps);
    if (st) return st;
    std::vector<Segment> segs;
    std::vector<std::vector<const float*>> gs;
    std::vector<std::vector<float*>> os, bs;
    st = batched_segments(g, out, buf, rows, cols, count, true, &segs, &gs, &os, &bs);
    if (st) return st;
    std::vector<Group> groups;
    st = plan_groups(segs.data(), static_cast<int>(segs.size()), &groups, ws_bytes);
    if (st) return st;
    void* ws = nullptr;  // only once the arguments are known to be valid
    st = workspace(&ws);
    if (st) return st;
    st = check_workspace(ws, ws_bytes, groups_bytes(groups));
    if (st) return st;
    return run_groups(groups, kQuintic, Update{}, mu, steps, eps, static_cast<char*>(ws), stream, nullptr);
}

int fail_status(int status, const char* msg) { return fail(status, "%s", msg); }

}  // namespace muon

extern "C" {

int muon_momentum_nesterov(const float* g, float* buf, float* u, int64_t numel, float mu, void* stream) {
    using namespace muon;
    if (numel < 0) return fail(MUON_ERR_INVALID_ARG, "numel must be >= 0 (got %lld)", (long long)numel);
    if (numel == 0) return ok();
    if (!g || !buf || !u) return fail(MUON_ERR_INVALID_ARG, "null pointer argument");
    if (u == buf) return fail(MUON_ERR_INVALID_ARG, "u must not alias buf");
    (void)hipGetLastError();
    hipError_t e = launch_momentum(g, buf, u, numel, mu, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "momentum launch");
    return ok();
}

static_assert(muon::kMaxMomentumGroup == MUON_NESTEROV_MAX_GROUP, "grouped momentum pass size");

int muon_momentum_nesterov_grouped(const float* const* g, float* const* buf, float* const* u, const int64_t* numel,
                                   int64_t count, float mu, void* stream) {
    using namespace muon;
    if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count must be >= 0 (got %lld)", (long long)count);
    if (count == 0) return ok();
    if (!g || !buf || !u || !numel) return fail(MUON_ERR_INVALID_ARG, "null array argument");
    for (int64_t i = 0; i < count; ++i) {
        if (numel[i] < 0)
            return fail(MUON_ERR_INVALID_ARG, "numel[%lld] must be >= 0 (got %lld)", (long long)i,
                        (long long)numel[i]);
        if (numel[i] > 0 && (!g[i] || !buf[i] || !u[i]))
            return fail(MUON_ERR_INVALID_ARG, "null pointer at index %lld", (long long)i);
        if (numel[i] > 0 && u[i] == buf[i])
            return fail(MUON_ERR_INVALID_ARG, "u must not alias buf (index %lld)", (long long)i);
    }
    (void)hipGetLastError();
    // passes of up to kMaxMomentumGroup non-empty matrices, one launch each
    MomentumGroup t{};
    int n = 0;
    int64_t longest = 0;
    for (int64_t i = 0; i <= count; ++i) {
        if (i < count && numel[i] > 0) {
            t.g[n] = g[i];
            t.buf[n] = buf[i];
            t.u[n] = u[i];
            t.numel[n] = numel[i];
            longest = numel[i] > longest ? numel[i] : longest;
            ++n;
        }
        if (n > 0 && (n == kMaxMomentumGroup || i == count)) {
            hipError_t e = launch_momentum_grouped(t, n, longest, mu, static_cast<hipStream_t>(stream));
            if (e != hipSuccess) return hip_fail(e, "grouped momentum launch");
            n = 0;
            longest = 0;
        }
    }
    return ok();
}

size_t muon_ns5_workspace_size(int64_t rows, int64_t cols, int64_t count) {
    using namespace muon;
    if (rows < 1 || cols < 1 || count < 1) return 0;
    Segment sg{rows, cols, count, nullptr, nullptr, nullptr};
    std::vector<Group> groups;
    const std::string saved = g_last_error;
    const int st = plan_groups(&sg, 1, &groups);
    g_last_error = saved;
    return st ? 0 : groups_bytes(groups);
}

size_t muon_ns5_batched_workspace_size(const int64_t* rows, const int64_t* cols, int64_t count) {
    using namespace muon;
    const std::string saved = g_last_error;
    std::vector<Segment> segs;
    std::vector<std::vector<const float*>> gs;
    std::vector<std::vector<float*>> os, bs;
    BatchPlan bp;
    int st = batched_segments(nullptr, nullptr, nullptr, rows, cols, count, false, &segs, &gs, &os, &bs);
    if (!st) st = plan_batch(segs, false, true, &bp);
    g_last_error = saved;
    return st ? 0 : bp.bytes;
}

int muon_ns5(const void* G, void* out, int64_t rows, int64_t cols, muon_dtype dtype, int steps, float eps,
             void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!G || !out) return fail(MUON_ERR_INVALID_ARG, "null G or out");
    return muon_ns5_grouped(&G, &out, 1, rows, cols, dtype, steps, eps, workspace, workspace_bytes, stream);
}

int muon_ns5_grouped(const void* const* G, void* const* out, int64_t count, int64_t rows, int64_t cols,
                     muon_dtype dtype, int steps, float eps, void* workspace, size_t workspace_bytes,
                     void* stream) {
    using namespace muon;
    if (dtype != MUON_F32 && dtype != MUON_BF16)
        return fail(MUON_ERR_INVALID_ARG, "unknown dtype %d", static_cast<int>(dtype));
    // the pointer tables carry addresses only; the kernels read and write
    // the element type the update names
    Segment sg;
    int st = grouped_segment(reinterpret_cast<const float* const*>(G), reinterpret_cast<float* const*>(out), count,
                             rows, cols, &sg);
    if (st) return st;
    st = check_common(steps, eps);
    if (st) return st;
    std::vector<Group> groups;
    st = plan_groups(&sg, 1, &groups);
    if (st) return st;
    st = check_workspace(workspace, workspace_bytes, groups_bytes(groups));
    if (st) return st;
    Update up;
    up.bf16_io = dtype == MUON_BF16;
    return run_groups(groups, kQuintic, up, 0.0f, steps, eps, static_cast<char*>(workspace),
                      static_cast<hipStream_t>(stream), nullptr);
}

int muon_ns5_batched(const float* const* G, float* const* out, const int64_t* rows, const int64_t* cols,
                     int64_t count, int steps, float eps, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    return run_batched(G, out, nullptr, 0.0f, rows, cols, count, steps, eps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), nullptr);
}

int muon_newton_schulz_batched(const float* const* G, float* const* out, const int64_t* rows, const int64_t* cols,
                               int64_t count, int steps, const float* coeffs, float eps, void* workspace,
                               size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!coeffs) return fail(MUON_ERR_INVALID_ARG, "null coefficient array");
    for (int i = 0; i < 3; ++i)
        if (!isfinite(coeffs[i])) return fail(MUON_ERR_INVALID_ARG, "coefficient %d is not finite", i);
    return run_batched(G, out, nullptr, 0.0f, rows, cols, count, steps, eps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), nullptr, Coeffs{coeffs[0], coeffs[1], coeffs[2]});
}

int muon_momentum_ns5_batched(const float* const* g, float* const* buf, float* const* out, const int64_t* rows,
                              const int64_t* cols, int64_t count, float mu, int steps, float eps, void* workspace,
                              size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!buf) return fail(MUON_ERR_INVALID_ARG, "null momentum buffer array");
    return run_batched(g, out, buf, mu, rows, cols, count, steps, eps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), nullptr);
}

int muon_ns5_batched_bf16(const uint16_t* const* G, uint16_t* const* out, const int64_t* rows, const int64_t* cols,
                          int64_t count, int steps, float eps, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    Update up;
    up.bf16_io = true;
    // the pointer tables carry addresses only; the kernels read and write bf16
    return run_batched(reinterpret_cast<const float* const*>(G), reinterpret_cast<float* const*>(out), nullptr,
                       0.0f, rows, cols, count, steps, eps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), nullptr, kQuintic, up);
}

int muon_momentum_ns5_apply_batched(const float* const* g, float* const* buf, float* const* p, const int64_t* rows,
                                    const int64_t* cols, int64_t count, float mu, float lr, int steps, float eps,
                                    void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!buf) return fail(MUON_ERR_INVALID_ARG, "null momentum buffer array");
    if (!p) return fail(MUON_ERR_INVALID_ARG, "null parameter array");
    if (!isfinite(lr)) return fail(MUON_ERR_INVALID_ARG, "lr must be finite");
    if (g && count > 0)
        for (int64_t i = 0; i < count; ++i)
            if (p[i] && p[i] == g[i])
                return fail(MUON_ERR_INVALID_ARG, "parameters must not alias the gradient (index %lld)", (long long)i);
    Update up;
    up.apply = true;
    up.lr = lr;
    return run_batched(g, p, buf, mu, rows, cols, count, steps, eps, workspace, workspace_bytes,
                       static_cast<hipStream_t>(stream), nullptr, kQuintic, up);
}

size_t muon_newton_schulz_f32_workspace_size(const int64_t* rows, const int64_t* cols, int64_t count) {
    using namespace muon;
    const std::string saved = g_last_error;
    std::vector<Segment> segs;
    std::vector<std::vector<const float*>> gs;
    std::vector<std::vector<float*>> os, bs;
    size_t bytes = 0;
    int st = batched_segments(nullptr, nullptr, nullptr, rows, cols, count, false, &segs, &gs, &os, &bs);
    if (!st) st = f32_bytes(segs, &bytes);
    g_last_error = saved;
    return st ? 0 : bytes;
}

int muon_newton_schulz_f32_batched(const float* const* G, float* const* out, const int64_t* rows,
                                   const int64_t* cols, int64_t count, int steps, const float* coeffs, float eps,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    Coeffs k = kQuintic;
    if (coeffs) {
        for (int i = 0; i < 3; ++i)
            if (!isfinite(coeffs[i])) return fail(MUON_ERR_INVALID_ARG, "coefficient %d is not finite", i);
        k = Coeffs{coeffs[0], coeffs[1], coeffs[2]};
    }
    return run_f32(G, out, rows, cols, count, steps, k, eps, workspace, workspace_bytes,
                   static_cast<hipStream_t>(stream));
}

int muon_ns5_batched_timed(const float* const* G, float* const* out, float* const* buf, float mu,
                           const int64_t* rows, const int64_t* cols, int64_t count, int steps, float eps,
                           void* workspace, size_t workspace_bytes, void* stream, void* const* events,
                           int n_event_pairs, int* recorded) {
    using namespace muon;
    if (recorded) *recorded = 0;
    if (n_event_pairs < 0 || (!events && n_event_pairs > 0))
        return fail(MUON_ERR_INVALID_ARG, "bad event array");
    EventSink sink;
    sink.events = events;
    sink.pairs = events ? n_event_pairs : 0;
    const int st = run_batched(G, out, buf, mu, rows, cols, count, steps, eps, workspace, workspace_bytes,
                               static_cast<hipStream_t>(stream), &sink);
    if (recorded) *recorded = sink.recorded;
    return st;
}

size_t muon_polar_svd_workspace_size(int64_t rows, int64_t cols, int64_t count) {
    using namespace muon;
    SvdPlan pl;
    return plan_svd(rows, cols, count, &pl) ? pl.bytes : 0;
}

int muon_polar_svd_grouped(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                           int max_sweeps, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    return run_polar_svd(G, out, count, rows, cols, max_sweeps, workspace, workspace_bytes,
                         static_cast<hipStream_t>(stream));
}

const char* muon_status_string(int status) {
    switch (status) {
        case MUON_OK: return "ok";
        case MUON_ERR_INVALID_ARG: return "invalid argument";
        case MUON_ERR_UNSUPPORTED: return "unsupported size";
        case MUON_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
        case MUON_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* muon_last_error(void) { return muon::g_last_error.c_str(); }

}  // extern "C"
