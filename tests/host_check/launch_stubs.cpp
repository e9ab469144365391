// Host-only stand-ins for the library's kernel launchers, linked with the
// real host code of api.hip and static_ws.hip into a CPU program built with
// AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_host_sanitizers.py).
// Instead of launching, each stub checks, in 64-bit arithmetic, that every
// workspace range the kernel would address lies inside the workspace the
// driver registered, that its grid is consistent with its segment tables,
// and that its pointer-table indices stay below MUON_NS5_MAX_GROUP.  A
// failed check prints the launch and aborts.
#include <stdio.h>
#include <stdlib.h>

#include "../../newton_schulz_09_amd/csrc/internal.hpp"

namespace hostcheck {
uintptr_t ws_lo = 0, ws_hi = 0;   // the workspace of the call being checked
long launches = 0;
}  // namespace hostcheck

namespace muon {

namespace {

[[noreturn]] void die(const char* what, long long a, long long b) {
    fprintf(stderr, "host check failed: %s (%lld, %lld)\n", what, a, b);
    abort();
}

// [p, p + bytes) inside the registered workspace
void in_ws(const void* p, long long bytes, const char* what) {
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    if (bytes <= 0) die(what, bytes, 0);
    if (lo < hostcheck::ws_lo || lo + static_cast<uintptr_t>(bytes) > hostcheck::ws_hi)
        die(what, static_cast<long long>(lo - hostcheck::ws_lo), bytes);
}

// matrices [0, cnt) of `mat` elements each, rows x cols used with leading
// dimension ld, element size es
void region(const void* base, long long mat, int cnt, long long rows, long long cols, long long ld, int es,
            const char* what) {
    if (cols > ld) die(what, cols, ld);
    const long long last = (cnt - 1) * mat + (rows - 1) * ld + cols;  // one past the last element
    if ((cnt - 1) * mat < 0 || last <= 0) die(what, cnt, mat);
    if (cnt > 1 && mat < rows * ld) die("matrices overlap", mat, rows * ld);
    in_ws(base, last * es, what);
}

int seg_count(int si, int nseg, int first_block, int next_first, int blocks, int per_mat, const char* what) {
    const int end = si + 1 < nseg ? next_first : blocks;
    const int n = end - first_block;
    if (per_mat <= 0 || n <= 0 || n % per_mat != 0) die(what, n, per_mat);
    return n / per_mat;
}

}  // namespace

hipError_t launch_momentum(const float*, float*, float*, int64_t numel, float, hipStream_t) {
    if (numel <= 0) die("momentum numel", numel, 0);
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_momentum_grouped(const MomentumGroup& t, int count, int64_t max_numel, float, hipStream_t) {
    if (count < 1 || count > kMaxMomentumGroup) die("grouped momentum count", count, 0);
    for (int i = 0; i < count; ++i)
        if (t.numel[i] <= 0 || t.numel[i] > max_numel || !t.g[i] || !t.buf[i] || !t.u[i])
            die("grouped momentum entry", i, t.numel[i]);
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_norm(const NormLaunch& L, int blocks, const ConstPtrTable& G, const PtrTable* BUF, float,
                       hipStream_t, bool) {
    if (L.nseg < 1 || L.nseg > kMaxSeg) die("norm segments", L.nseg, 0);
    for (int si = 0; si < L.nseg; ++si) {
        const NormSeg& s = L.seg[si];
        const int cnt = seg_count(si, L.nseg, s.first_block, si + 1 < L.nseg ? L.seg[si + 1].first_block : 0,
                                  blocks, s.nb, "norm grid");
        if (s.ptr_base < 0 || s.ptr_base + cnt > kMaxGroup) die("norm pointer table", s.ptr_base, cnt);
        for (int i = 0; i < cnt; ++i)
            if (!G.p[s.ptr_base + i] || (BUF && !BUF->p[s.ptr_base + i])) die("norm null pointer", i, 0);
        if (s.chunk * s.nb < s.numel || (s.vec && s.chunk % 4)) die("norm chunking", s.chunk, s.numel);
        in_ws(s.partials, static_cast<long long>(cnt) * s.nb * 8, "norm partials");
        if (s.ub) region(s.ub, s.ub_mat, cnt, 1, s.numel, s.numel, 2, "norm staging copy");
    }
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_scale_cast(const CastLaunch& L, int blocks, const ConstPtrTable& G, bool, float, hipStream_t) {
    if (L.nseg < 1 || L.nseg > kMaxSeg) die("cast segments", L.nseg, 0);
    for (int si = 0; si < L.nseg; ++si) {
        const CastSeg& s = L.seg[si];
        const int cnt = seg_count(si, L.nseg, s.first_block, si + 1 < L.nseg ? L.seg[si + 1].first_block : 0,
                                  blocks, s.wg_per_mat, "cast grid");
        if (static_cast<long long>(s.wg_per_mat) * s.per_wg < s.tiles_per_mat) die("cast tiles", s.wg_per_mat, s.per_wg);
        if (s.ptr_base < 0 || s.ptr_base + cnt > kMaxGroup) die("cast pointer table", s.ptr_base, cnt);
        for (int i = 0; i < cnt; ++i)
            if (!G.p[s.ptr_base + i]) die("cast null pointer", i, 0);
        // X: the padded extent in the iteration's orientation
        const long long rows_pad = static_cast<long long>(s.tiles_per_mat / s.tiles_c) * 64;
        const long long cols_pad = static_cast<long long>(s.tiles_c) * 64;
        const long long xr = s.tall ? cols_pad : rows_pad, xc = s.tall ? rows_pad : cols_pad;
        if (xr < (s.tall ? s.cols : s.rows) || xc < (s.tall ? s.rows : s.cols)) die("cast covers G", xr, xc);
        region(s.X, s.x_mat, cnt, xr, xc, s.ldx, 2, "cast X");
        in_ws(s.partials, static_cast<long long>(cnt) * s.nb * 8, "cast partials");
        if (s.ub) region(s.ub, s.ub_mat, cnt, 1, static_cast<long long>(s.rows) * s.cols, s.ub_mat, 2, "cast staging");
    }
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_zero_rows(bf16_t* X, int64_t x_mat, int cnt, int first_row, int rows, int ld, hipStream_t) {
    if (first_row >= rows || cnt < 1) return hipSuccess;
    region(X, x_mat, cnt, rows, ld, ld, 2, "zeroed rows");
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_copy_out(const Ns5Plan& plan, int cnt, const bf16_t* X, const PtrTable& out, hipStream_t, bool,
                           float, bool) {
    if (cnt < 1 || cnt > kMaxGroup) die("copy-out count", cnt, 0);
    for (int i = 0; i < cnt; ++i)
        if (!out.p[i]) die("copy-out null pointer", i, 0);
    region(X, static_cast<long long>(plan.x_elems), cnt, plan.m, plan.n, plan.ldx, 2, "copy-out X");
    ++hostcheck::launches;
    return hipSuccess;
}

// The small-matrix launch reads G, writes out (and buf) only: every
// segment's shape must fit the kernel's LDS tiles, the segments must tile
// the pointer tables in order, and every pointer used must be set.
hipError_t launch_ns5_small(const SmallArgs& s, const ConstPtrTable& G, const PtrTable& out, const PtrTable* buf,
                            bool io16, hipStream_t) {
    if (s.nseg < 1 || s.nseg > kMaxSeg) die("small segments", s.nseg, 0);
    if (io16 && (buf || s.apply)) die("small bf16 with momentum or update", 0, 0);
    int total = 0;
    for (int q = 0; q < s.nseg; ++q) {
        const SmallSeg& sg = s.seg[q];
        if (sg.first != total || sg.cnt < 1) die("small segment table", sg.first, total);
        if (sg.m < 1 || sg.m > kSmallM || sg.n < sg.m || sg.n > kSmallN) die("small shape", sg.m, sg.n);
        if (sg.np % 32 != 0 || sg.np < sg.n || sg.np > kSmallN) die("small padded width", sg.np, sg.n);
        if (static_cast<long long>(sg.rows) * sg.cols != static_cast<long long>(sg.m) * sg.n)
            die("small extent", sg.rows, sg.cols);
        if ((sg.rows > sg.cols) != (sg.tall != 0)) die("small orientation", sg.rows, sg.cols);
        total += sg.cnt;
    }
    if (total > kMaxGroup) die("small pointer table", total, kMaxGroup);
    for (int i = 0; i < total; ++i) {
        if (!G.p[i] || !out.p[i]) die("small null pointer", i, 0);
        if (buf && !buf->p[i]) die("small null buffer", i, 0);
    }
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_gemm(GemmKind kind, int tile, int tile_n, const GemmLaunch& L, int blocks, const PtrTable* out,
                       hipStream_t) {
    const bool sym = kind == GEMM_SYRK || kind == GEMM_AAB;
    if (L.nseg < 1 || L.nseg > kMaxSeg) die("gemm segments", L.nseg, 0);
    if (blocks < 1 || static_cast<long long>(blocks) * 512 >= (1ll << 32)) die("gemm grid", blocks, 0);
    if (sym && tile != tile_n) die("symmetric tile", tile, tile_n);
    if (kind == GEMM_BX_FINAL && !out) die("final step without outputs", 0, 0);
    if (L.interleave_tpm > 0)
        for (int si = 0; si < L.nseg; ++si)
            if (L.seg[si].tiles_per_mat != L.interleave_tpm) die("interleave", si, L.interleave_tpm);
    for (int si = 0; si < L.nseg; ++si) {
        const GemmArgs& a = L.seg[si];
        const int cnt = seg_count(si, L.nseg, a.first_block, si + 1 < L.nseg ? L.seg[si + 1].first_block : 0,
                                  blocks, a.tiles_per_mat, "gemm grid");
        if (a.kpad % 64 || a.kpad < 64) die("K padding", a.kpad, 0);
        const long long rows = static_cast<long long>(a.tiles) * tile, cols = static_cast<long long>(a.tiles_n) * tile_n;
        if (a.tiles_per_mat != (sym ? a.tiles * (a.tiles + 1) / 2 : a.tiles * a.tiles_n)) die("tiles", a.tiles, a.tiles_n);
        if (sym) {   // NT: P and Q are rows x kpad, C (and E) rows x rows
            if (a.tiles != a.tiles_n) die("symmetric grid", a.tiles, a.tiles_n);
            region(a.P, a.p_mat, cnt, rows, a.kpad, a.ldp, 2, "P");
            region(a.Q, a.q_mat, cnt, rows, a.kpad, a.ldq, 2, "Q");
            region(a.C, a.c_mat, cnt, rows, rows, a.ldc, 2, "C");
            if (kind == GEMM_AAB) region(a.E, a.e_mat, cnt, rows, rows, a.lde, 2, "E");
        } else {     // NN: P rows x kpad, Q kpad x cols, E and C rows x cols
            if (a.band < 1 || a.band > a.tiles) die("band", a.band, a.tiles);
            region(a.P, a.p_mat, cnt, rows, a.kpad, a.ldp, 2, "P");
            region(a.Q, a.q_mat, cnt, a.kpad, cols, a.ldq, 2, "Q");
            region(a.E, a.e_mat, cnt, rows, cols, a.lde, 2, "E");
            if (kind == GEMM_BX) region(a.C, a.c_mat, cnt, rows, cols, a.ldc, 2, "C");
            if (rows < a.m || cols < a.n) die("output covered", rows, cols);
            if (kind == GEMM_BX_FINAL) {
                if (a.out_base < 0 || a.out_base + cnt > kMaxGroup) die("output table", a.out_base, cnt);
                for (int i = 0; i < cnt; ++i)
                    if (!out->p[a.out_base + i]) die("final null output", i, 0);
            }
        }
    }
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_f32_gemm(GemmKind kind, const F32Gemm& g, int blocks, const PtrTable* out, hipStream_t) {
    const bool sym = kind == GEMM_SYRK || kind == GEMM_AAB;
    if (g.tiles_per_mat < 1 || blocks % g.tiles_per_mat) die("float32 grid", blocks, g.tiles_per_mat);
    const int cnt = blocks / g.tiles_per_mat;
    if (g.K % 16) die("float32 K", g.K, 0);
    const long long rows = g.tiles * 128ll, cols = g.tiles_n * 128ll;
    region(g.P, g.p_mat, cnt, rows, g.K, g.ldp, 4, "float32 P");
    if (kind == GEMM_SYRK) region(g.Q, g.q_mat, cnt, cols, g.K, g.ldq, 4, "float32 Q");
    else region(g.Q, g.q_mat, cnt, g.K, cols, g.ldq, 4, "float32 Q");
    if (kind != GEMM_BX_FINAL) region(g.C, g.c_mat, cnt, rows, cols, g.ldc, 4, "float32 C");
    if (kind != GEMM_SYRK) region(g.E, g.e_mat, cnt, rows, cols, g.lde, 4, "float32 E");
    if (kind == GEMM_BX_FINAL) {
        if (!out || cnt > kMaxGroup) die("float32 outputs", cnt, 0);
        for (int i = 0; i < cnt; ++i)
            if (!out->p[i]) die("float32 null output", i, 0);
    }
    if (sym && g.tiles != g.tiles_n) die("float32 symmetric grid", g.tiles, g.tiles_n);
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_f32_scale(const F32Scale& s, const ConstPtrTable& G, const PtrTable* out, hipStream_t) {
    if (s.cnt < 1 || s.cnt > kMaxGroup) die("float32 scale count", s.cnt, 0);
    for (int i = 0; i < s.cnt; ++i)
        if (!G.p[i] || (s.to_out && !out->p[i])) die("float32 scale pointer", i, 0);
    in_ws(s.partials, static_cast<long long>(s.cnt) * s.nb * 8, "float32 partials");
    if (!s.to_out) {
        const long long xr = static_cast<long long>(s.tiles_per_mat / s.tiles_c) * 32, xc = s.tiles_c * 32ll;
        region(s.X, s.x_mat, s.cnt, xr, xc, s.ldx, 4, "float32 X");
    }
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_svd_init(const SvdArgs& a, const ConstPtrTable& G, hipStream_t) {
    if (a.count < 1 || a.count > kMaxGroup) die("SVD count", a.count, 0);
    for (int i = 0; i < a.count; ++i)
        if (!G.p[i]) die("SVD null input", i, 0);
    if (a.m_pad % 64 || a.n_pad % 64 || a.ld != a.m_pad + a.n_pad || a.blocks * 32 != a.m_pad)
        die("SVD layout", a.m_pad, a.n_pad);
    if (a.m > a.m_pad || a.n > a.n_pad || a.mat_elems != static_cast<long long>(a.m_pad) * a.ld)
        die("SVD padding", a.m, a.n);
    region(a.wj, a.mat_elems, a.count, a.m_pad, a.ld, a.ld, 4, "SVD [W | J]");
    in_ws(a.state, a.count * 8ll, "SVD state");
    in_ws(a.inv_len, static_cast<long long>(a.count) * a.m_pad * 8, "SVD row lengths");
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_svd_sweep(const SvdArgs& a, bool, hipStream_t) {
    region(a.wj, a.mat_elems, a.count, a.m_pad, a.ld, a.ld, 4, "SVD [W | J]");
    if (a.blocks < 2 || a.blocks % 2) die("SVD blocks", a.blocks, 0);
    ++hostcheck::launches;
    return hipSuccess;
}

hipError_t launch_svd_finish(const SvdArgs& a, const PtrTable& out, hipStream_t) {
    for (int i = 0; i < a.count; ++i)
        if (!out.p[i]) die("SVD null output", i, 0);
    in_ws(a.inv_len, static_cast<long long>(a.count) * a.m_pad * 8, "SVD row lengths");
    ++hostcheck::launches;
    return hipSuccess;
}

}  // namespace muon
