// CPU driver of the library's host code (api.hip) with the launch stubs of
// launch_stubs.cpp: every entry point that plans and enqueues work is called
// on the workloads and at the largest accepted shapes, with a fake
// workspace address range registered for the stubs to check against.
// Nothing is dereferenced on the device side: the stubs never launch.
// Built with AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py; prints "host check ok: N launches".
#include <stdio.h>
#include <stdlib.h>

#include <vector>

#include "../../include/muon.h"
#include "../../newton_schulz_09_amd/csrc/internal.hpp"

namespace hostcheck {
extern uintptr_t ws_lo, ws_hi;
extern long launches;
}  // namespace hostcheck

namespace {

constexpr uintptr_t kWs = uintptr_t{1} << 44;   // fake, 256-byte aligned, never dereferenced
int failures = 0;

void expect_ok(int st, const char* what) {
    if (st != MUON_OK) {
        printf("FAILED: %s: status %d (%s)\n", what, st, muon_last_error());
        ++failures;
    }
}

struct Batch {
    std::vector<int64_t> rows, cols;
    std::vector<const float*> g;
    std::vector<float*> out, buf;
    void add(int64_t r, int64_t c, int n = 1) {
        for (int i = 0; i < n; ++i) {
            rows.push_back(r);
            cols.push_back(c);
            const uintptr_t k = rows.size();
            g.push_back(reinterpret_cast<const float*>(uintptr_t{1} << 40 | k << 12));
            out.push_back(reinterpret_cast<float*>(uintptr_t{2} << 40 | k << 12));
            buf.push_back(reinterpret_cast<float*>(uintptr_t{3} << 40 | k << 12));
        }
    }
    int64_t n() const { return static_cast<int64_t>(rows.size()); }
};

// "shrink" mode registers every workspace 256 bytes short of the size the
// library asked for, so that the stubs must catch the last region
size_t g_shrink = 0;

void* set_ws(size_t bytes) {
    hostcheck::ws_lo = kWs;
    hostcheck::ws_hi = kWs + bytes - g_shrink;
    return reinterpret_cast<void*>(kWs);
}

int fake_static_ws(void** p) {
    *p = reinterpret_cast<void*>(kWs);
    return MUON_OK;
}

void run_all(const Batch& b, const char* name) {
    const size_t need = muon_ns5_batched_workspace_size(b.rows.data(), b.cols.data(), b.n());
    if (need == 0) {
        printf("FAILED: %s: no workspace size\n", name);
        ++failures;
        return;
    }
    void* ws = set_ws(need);
    const float cubic[3] = {1.5f, -0.5f, 0.0f};
    expect_ok(muon_ns5_batched(b.g.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(), 5, 1e-7f, ws, need,
                               nullptr), name);
    expect_ok(muon_ns5_batched(b.g.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(), 0, 1e-7f, ws, need,
                               nullptr), name);
    expect_ok(muon_newton_schulz_batched(b.g.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(), 2, cubic,
                                         1e-7f, ws, need, nullptr), name);
    expect_ok(muon_momentum_ns5_batched(b.g.data(), b.buf.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(),
                                        0.95f, 5, 1e-7f, ws, need, nullptr), name);
    expect_ok(muon_momentum_ns5_apply_batched(b.g.data(), b.buf.data(), b.out.data(), b.rows.data(), b.cols.data(),
                                              b.n(), 0.95f, 0.02f, 5, 1e-7f, ws, need, nullptr), name);
    expect_ok(muon_ns5_batched_bf16(reinterpret_cast<const uint16_t* const*>(b.g.data()),
                                    reinterpret_cast<uint16_t* const*>(b.out.data()), b.rows.data(), b.cols.data(),
                                    b.n(), 5, 1e-7f, ws, need, nullptr), name);
    expect_ok(muon_ns5_batched_timed(b.g.data(), b.out.data(), b.buf.data(), 0.95f, b.rows.data(), b.cols.data(),
                                     b.n(), 5, 1e-7f, ws, need, nullptr, nullptr, 0, nullptr), name);
    // the fixed-workspace planning of the static entry point, on a 256 MiB range
    set_ws(MUON_STATIC_WORKSPACE_BYTES);
    bool fits = true;
    for (int64_t i = 0; i < b.n(); ++i)
        fits = fits && muon_ns5_workspace_size(b.rows[i], b.cols[i], 1) <= MUON_STATIC_WORKSPACE_BYTES;
    const int st = muon::run_momentum_ns5_fixed_workspace(b.g.data(), b.buf.data(), b.out.data(), b.rows.data(),
                                                          b.cols.data(), b.n(), 0.95f, 5, 1e-7f,
                                                          MUON_STATIC_WORKSPACE_BYTES, fake_static_ws, nullptr);
    if (fits) expect_ok(st, name);
    else if (st != MUON_ERR_UNSUPPORTED) {
        printf("FAILED: %s: too large for the static workspace, status %d\n", name, st);
        ++failures;
    }
    // the iteration carried in float32
    const size_t need32 = muon_newton_schulz_f32_workspace_size(b.rows.data(), b.cols.data(), b.n());
    void* ws32 = set_ws(need32);
    expect_ok(muon_newton_schulz_f32_batched(b.g.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(), 5,
                                             nullptr, 1e-7f, ws32, need32, nullptr), name);
    expect_ok(muon_newton_schulz_f32_batched(b.g.data(), b.out.data(), b.rows.data(), b.cols.data(), b.n(), 0,
                                             cubic, 1e-7f, ws32, need32, nullptr), name);
}

}  // namespace

int main(int argc, char** argv) {
    if (argc > 1 && argv[1][0] == 's') g_shrink = 256;
    {
        Batch b;
        b.add(1, 1);
        run_all(b, "1 x 1");
    }
    {
        Batch b;
        b.add(64, 128);
        b.add(128, 64);
        run_all(b, "64 x 128 and its transpose");
    }
    {
        Batch b;
        for (int l = 0; l < 12; ++l) {
            b.add(768, 2304);
            b.add(768, 768);
            b.add(768, 3072);
            b.add(3072, 768);
        }
        run_all(b, "GPT-2 124M set");
    }
    {
        Batch b;
        for (int l = 0; l < 48; ++l) {
            b.add(1600, 4800);
            b.add(1600, 1600);
            b.add(1600, 6400);
            b.add(6400, 1600);
        }
        run_all(b, "GPT-2 1.5B set");
    }
    {
        Batch b;
        b.add(2048, 8192, 8);
        b.add(8192, 2048, 8);
        run_all(b, "extreme aspect set");
    }
    {
        Batch b;
        b.add(4096, 4096, 2);
        run_all(b, "two 4096 x 4096");
    }
    {
        Batch b;
        b.add(16, 1 << 20);
        b.add(1 << 20, 16);
        run_all(b, "longest sides");
    }
    {
        Batch b;
        b.add(MUON_NS5_MAX_SHORT, MUON_NS5_MAX_SHORT);
        run_all(b, "16384 x 16384");
    }
    {
        Batch b;
        b.add(5632, 5632);
        b.add(5648, 5648);
        run_all(b, "around the static workspace limit");
    }
    {
        Batch b;
        for (int r = 0; r < 13; ++r)
            for (int i = 0; i < 11; ++i) b.add(40 + 3 * i, 90 + 5 * i);
        b.add(257, 90, 3);
        b.add(200, 900, 130);
        run_all(b, "many shapes and passes");
    }
    {
        std::vector<const float*> g;
        std::vector<float*> buf, u;
        std::vector<int64_t> numel;
        for (int i = 0; i < 150; ++i) {
            g.push_back(reinterpret_cast<const float*>(uintptr_t{1} << 40 | uintptr_t(i + 1) << 12));
            buf.push_back(reinterpret_cast<float*>(uintptr_t{3} << 40 | uintptr_t(i + 1) << 12));
            u.push_back(reinterpret_cast<float*>(uintptr_t{2} << 40 | uintptr_t(i + 1) << 12));
            numel.push_back(i % 7 == 3 ? 0 : int64_t{1} << (i % 31));
        }
        expect_ok(muon_momentum_nesterov_grouped(g.data(), buf.data(), u.data(), numel.data(), 150, 0.95f, nullptr),
                  "grouped momentum");
        expect_ok(muon_momentum_nesterov(g[0], buf[0], u[0], int64_t{1} << 33, 0.95f, nullptr), "momentum 2^33");
    }
    {
        // U V^T through the GPU SVD, same-shaped groups (more than one pass
        // for 130 matrices)
        const int64_t shapes[][2] = {{3, 5}, {768, 3072}, {3072, 768}, {4096, 4096}, {16, 1 << 20}};
        for (const auto& sh : shapes) {
            Batch b;
            b.add(sh[0], sh[1], sh[0] == 3 ? 130 : 2);
            const size_t need = muon_polar_svd_workspace_size(sh[0], sh[1], b.n());
            void* ws = set_ws(need);
            expect_ok(muon_polar_svd_grouped(b.g.data(), b.out.data(), b.n(), sh[0], sh[1], 12, ws, need, nullptr),
                      "polar SVD");
        }
    }
    if (failures) return 1;
    printf("host check ok: %ld launches\n", hostcheck::launches);
    return 0;
}
