// C ABI of libmuon.so: validation, workspace layout and the launch sequence
// of the Muon hot path (declared and documented in include/muon.h).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include <string>

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

// GEMM tile edge for the short side m.  Padding m and n to the tile keeps the
// GEMMs free of edge handling; the choice trades padded work against the
// larger tile's better operand reuse.  MUON_NS5_TILE=64/128/256 in the
// environment forces one edge for every shape (read once, for tuning sweeps).
int choose_tile(int64_t m) {
    static const int forced = [] {
        const char* s = getenv("MUON_NS5_TILE");
        const int t = s ? atoi(s) : 0;
        return (t == 64 || t == 128 || t == 256) ? t : 0;
    }();
    if (forced) return forced;
    if (m <= 64) return 64;
    // 256-wide tiles reuse each operand panel twice as much but give a
    // quarter of the workgroups: below m = 2048 the 128 tile fills the 256
    // CUs better (measured on the 768- and 1600-class shapes)
    if (m < 2048) return 128;
    return 256;
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

// A dispatch's grid (workgroups x 256 work-items) must fit in 32 bits.
constexpr int64_t kMaxWorkgroups = (int64_t{1} << 32) / kThreads - 1;

}  // namespace

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
    p->tile = choose_tile(m);
    p->mp = static_cast<int>(round_up(m, p->tile));
    p->np = static_cast<int>(round_up(n, p->tile));
    int64_t nb = (rows * cols + 16383) / 16384;
    p->nb = static_cast<int>(nb < 1 ? 1 : (nb > kMaxNormBlocks ? kMaxNormBlocks : nb));
    const int64_t bx_tiles = static_cast<int64_t>(p->mp / p->tile) * (p->np / p->tile);
    int64_t cnt = count < kMaxGroup ? count : kMaxGroup;
    if (cnt * bx_tiles > kMaxWorkgroups) cnt = kMaxWorkgroups / bx_tiles;
    if (cnt < 1) return false;
    p->cnt = static_cast<int>(cnt);
    p->ldx = p->np + ld_skew();
    p->ldxt = p->mp + ld_skew();
    p->lda = p->mp + ld_skew();
    p->x_elems = static_cast<size_t>(p->mp) * p->ldx;
    p->xt_elems = static_cast<size_t>(p->np) * p->ldxt;
    p->a_elems = static_cast<size_t>(p->mp) * p->lda;
    size_t off = 0;
    const size_t xb = align256(cnt * p->x_elems * sizeof(bf16_t));
    const size_t xtb = align256(cnt * p->xt_elems * sizeof(bf16_t));
    const size_t ab = align256(cnt * p->a_elems * sizeof(bf16_t));
    p->off_x[0] = off; off += xb;
    p->off_x[1] = off; off += xb;
    p->off_xt[0] = off; off += xtb;
    p->off_xt[1] = off; off += xtb;
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

int run_ns5(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols, int steps,
            float eps, void* ws, size_t ws_bytes, hipStream_t stream, EventSink* sink) {
    if (rows < 1 || cols < 1) return fail(MUON_ERR_INVALID_ARG, "rows and cols must be >= 1 (got %lld x %lld)",
                                          (long long)rows, (long long)cols);
    if (steps < 0) return fail(MUON_ERR_INVALID_ARG, "steps must be >= 0 (got %d)", steps);
    if (!isfinite(eps)) return fail(MUON_ERR_INVALID_ARG, "eps must be finite");
    for (int64_t i = 0; i < count; ++i) {
        if (!G[i] || !out[i]) return fail(MUON_ERR_INVALID_ARG, "null matrix pointer at index %lld", (long long)i);
    }
    Ns5Plan plan;
    if (!make_plan(rows, cols, count, &plan))
        return fail(MUON_ERR_UNSUPPORTED, "shape %lld x %lld is beyond the supported limits", (long long)rows,
                    (long long)cols);
    if (!ws) return fail(MUON_ERR_WORKSPACE, "workspace is null");
    if (reinterpret_cast<uintptr_t>(ws) & 255u) return fail(MUON_ERR_WORKSPACE, "workspace is not 256-byte aligned");
    if (ws_bytes < plan.bytes)
        return fail(MUON_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, plan.bytes);

    (void)hipGetLastError();  // start from a clean error state
    char* base = static_cast<char*>(ws);
    bf16_t* X[2] = {reinterpret_cast<bf16_t*>(base + plan.off_x[0]), reinterpret_cast<bf16_t*>(base + plan.off_x[1])};
    bf16_t* XT[2] = {reinterpret_cast<bf16_t*>(base + plan.off_xt[0]),
                     reinterpret_cast<bf16_t*>(base + plan.off_xt[1])};
    bf16_t* A = reinterpret_cast<bf16_t*>(base + plan.off_a);
    bf16_t* B = reinterpret_cast<bf16_t*>(base + plan.off_b);
    double* part = reinterpret_cast<double*>(base + plan.off_part);
    const int T = plan.tile;
    const int tiles_m = plan.mp / T, tiles_n = plan.np / T;
    const int64_t xe = static_cast<int64_t>(plan.x_elems), xte = static_cast<int64_t>(plan.xt_elems);
    const int64_t ae = static_cast<int64_t>(plan.a_elems);

    for (int64_t start = 0; start < count; start += plan.cnt) {
        const int cnt = static_cast<int>(count - start < plan.cnt ? count - start : plan.cnt);
        ConstPtrTable gt{};
        PtrTable ot{};
        for (int i = 0; i < cnt; ++i) {
            gt.p[i] = G[start + i];
            ot.p[i] = out[start + i];
        }
        hipError_t e = launch_sumsq(gt, cnt, rows * cols, plan.nb, part, stream);
        if (e != hipSuccess) return hip_fail(e, "norm (sum of squares) launch");
        bf16_t* nat = plan.tall ? XT[0] : X[0];
        bf16_t* tr = plan.tall ? X[0] : XT[0];
        e = launch_scale_cast(gt, cnt, plan, part, eps, nat, tr, stream);
        if (e != hipSuccess) return hip_fail(e, "scale/cast launch");
        if (steps == 0) {
            e = launch_copy_out(plan, cnt, nat, ot, stream);
            if (e != hipSuccess) return hip_fail(e, "copy-out launch");
            continue;
        }
        int cur = 0;
        for (int s = 0; s < steps; ++s) {
            const int nxt = cur ^ 1;
            const bool last = (s == steps - 1);
            GemmArgs g{};
            // A = X X^T
            g.P = X[cur]; g.p_mat = xe; g.ldp = plan.ldx;
            g.Q = X[cur]; g.q_mat = xe; g.ldq = plan.ldx;
            g.kpad = static_cast<int>(round_up(plan.n, 64));
            g.tiles = tiles_m; g.tiles_n = tiles_m; g.tiles_per_mat = tiles_m * (tiles_m + 1) / 2;
            g.C = A; g.c_mat = ae; g.ldc = plan.lda;
            e = launch_gemm(GEMM_SYRK, T, g, cnt, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "X X^T launch");
            // B = b A + c A A
            g.P = A; g.p_mat = ae; g.ldp = plan.lda;
            g.Q = A; g.q_mat = ae; g.ldq = plan.lda;
            g.kpad = static_cast<int>(round_up(plan.m, 64));
            g.C = B; g.c_mat = ae; g.ldc = plan.lda;
            g.E = A; g.e_mat = ae; g.lde = plan.lda;
            g.alpha = MUON_NS5_B; g.beta = MUON_NS5_C;
            e = launch_gemm(GEMM_AAB, T, g, cnt, nullptr, stream);
            if (e != hipSuccess) return hip_fail(e, "b A + c A A launch");
            // X' = a X + B X
            g.P = B; g.p_mat = ae; g.ldp = plan.lda;
            g.Q = XT[cur]; g.q_mat = xte; g.ldq = plan.ldxt;
            g.kpad = static_cast<int>(round_up(plan.m, 64));
            g.tiles = tiles_m; g.tiles_n = tiles_n; g.tiles_per_mat = tiles_m * tiles_n;
            g.E = XT[cur]; g.e_mat = xte; g.lde = plan.ldxt;
            g.alpha = MUON_NS5_A; g.beta = 1.0f;
            g.C = X[nxt]; g.c_mat = xe; g.ldc = plan.ldx;
            g.CT = XT[nxt]; g.ct_mat = xte; g.ldct = plan.ldxt;
            g.m = plan.m; g.n = plan.n; g.tall = plan.tall ? 1 : 0;
            const bool timed = sink && !last && sink->recorded < sink->pairs;
            if (timed) {
                e = hipEventRecord(static_cast<hipEvent_t>(sink->events[2 * sink->recorded]), stream);
                if (e != hipSuccess) return hip_fail(e, "event record");
            }
            e = launch_gemm(last ? GEMM_BX_FINAL : GEMM_BX, T, g, cnt, last ? &ot : nullptr, stream);
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

}  // namespace

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

size_t muon_ns5_workspace_size(int64_t rows, int64_t cols, int64_t count) {
    muon::Ns5Plan plan;
    if (!muon::make_plan(rows, cols, count, &plan)) return 0;
    return plan.bytes;
}

int muon_ns5(const float* G, float* out, int64_t rows, int64_t cols, int steps, float eps, void* workspace,
             size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!G || !out) return fail(MUON_ERR_INVALID_ARG, "null G or out");
    return run_ns5(&G, &out, 1, rows, cols, steps, eps, workspace, workspace_bytes,
                   static_cast<hipStream_t>(stream), nullptr);
}

int muon_ns5_grouped(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                     int steps, float eps, void* workspace, size_t workspace_bytes, void* stream) {
    using namespace muon;
    if (!G || !out) return fail(MUON_ERR_INVALID_ARG, "null pointer array");
    if (count < 1) return fail(MUON_ERR_INVALID_ARG, "count must be >= 1 (got %lld)", (long long)count);
    return run_ns5(G, out, count, rows, cols, steps, eps, workspace, workspace_bytes,
                   static_cast<hipStream_t>(stream), nullptr);
}

int muon_ns5_grouped_timed(const float* const* G, float* const* out, int64_t count, int64_t rows, int64_t cols,
                           int steps, float eps, void* workspace, size_t workspace_bytes, void* stream,
                           void* const* events, int n_event_pairs, int* recorded) {
    using namespace muon;
    if (recorded) *recorded = 0;
    if (!G || !out) return fail(MUON_ERR_INVALID_ARG, "null pointer array");
    if (count < 1) return fail(MUON_ERR_INVALID_ARG, "count must be >= 1 (got %lld)", (long long)count);
    if (n_event_pairs < 0 || (!events && n_event_pairs > 0))
        return fail(MUON_ERR_INVALID_ARG, "bad event array");
    EventSink sink;
    sink.events = events;
    sink.pairs = events ? n_event_pairs : 0;
    const int st = run_ns5(G, out, count, rows, cols, steps, eps, workspace, workspace_bytes,
                           static_cast<hipStream_t>(stream), &sink);
    if (recorded) *recorded = sink.recorded;
    return st;
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
