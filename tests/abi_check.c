/* A plain C client of the boundary: compiled with a C compiler against
 * include/muon.h and linked to libmuon.so, it exercises the calls that need no
 * GPU (workspace queries, argument validation, status strings) and prints
 * "ok" when every check holds.  Driven by tests/test_abi_c.py. */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "muon.h"

static int failures = 0;

static void expect(int cond, const char* what) {
    if (!cond) {
        printf("FAILED: %s (last error: %s)\n", what, muon_last_error());
        ++failures;
    }
}

int main(void) {
    /* never dereferenced: every call below fails validation or enqueues nothing */
    void* fake = (void*)0x100000;
    const int64_t rows[2] = {64, 130}, cols[2] = {128, 65};
    const float* g2[2] = {(const float*)0x100000, (const float*)0x100100};
    float* o2[2] = {(float*)0x300000, (float*)0x300100};
    float* b2[2] = {(float*)0x500000, (float*)0x500100};
    const float cubic[3] = {1.5f, -0.5f, 0.0f};
    size_t need;

    expect(muon_ns5_workspace_size(64, 128, 1) > 0, "workspace for one 64 x 128");
    expect(muon_ns5_workspace_size(64, 128, 1) == muon_ns5_workspace_size(128, 64, 1), "orientation-free");
    expect(muon_ns5_workspace_size(0, 5, 1) == 0, "zero rows rejected");
    need = muon_ns5_batched_workspace_size(rows, cols, 2);
    expect(need > 0, "batched workspace");
    expect(muon_newton_schulz_f32_workspace_size(rows, cols, 2) > 0, "float32 workspace");

    expect(muon_momentum_nesterov(NULL, NULL, NULL, 0, 0.95f, NULL) == MUON_OK, "empty momentum");
    expect(muon_momentum_nesterov(NULL, (float*)fake, (float*)fake, 4, 0.95f, NULL) == MUON_ERR_INVALID_ARG,
           "null gradient");
    expect(muon_momentum_nesterov_grouped(NULL, NULL, NULL, NULL, 0, 0.95f, NULL) == MUON_OK, "empty group");
    expect(muon_ns5(NULL, fake, 64, 128, MUON_F32, 5, 1e-7f, fake, 1 << 20, NULL) == MUON_ERR_INVALID_ARG, "null G");
    expect(muon_ns5(fake, fake, 64, 128, (muon_dtype)7, 5, 1e-7f, fake, 1 << 20, NULL) == MUON_ERR_INVALID_ARG,
           "unknown dtype");
    {
        const void* gv[2] = {g2[0], g2[1]};
        void* ov[2] = {o2[0], o2[1]};
        expect(muon_ns5_grouped(gv, ov, 2, 64, 128, MUON_BF16, 5, 1e-7f, (void*)0x200000, 256, NULL) ==
                   MUON_ERR_WORKSPACE,
               "bf16 group with a small workspace");
        expect(muon_ns5_grouped(gv, ov, 0, 64, 128, MUON_BF16, 5, 1e-7f, (void*)0x200000, 1 << 20, NULL) ==
                   MUON_ERR_INVALID_ARG,
               "empty group");
    }
    expect(muon_ns5_batched(g2, o2, rows, cols, 2, 5, 1e-7f, (void*)0x200000, need - 256, NULL) == MUON_ERR_WORKSPACE,
           "small workspace");
    expect(muon_ns5_batched(g2, o2, rows, cols, 2, -1, 1e-7f, (void*)0x200000, need, NULL) == MUON_ERR_INVALID_ARG,
           "negative steps");
    expect(muon_newton_schulz_batched(g2, o2, rows, cols, 2, 5, NULL, 1e-7f, (void*)0x200000, need, NULL) ==
               MUON_ERR_INVALID_ARG,
           "null coefficients");
    expect(muon_newton_schulz_batched(g2, o2, rows, cols, 2, 5, cubic, 1e-7f, (void*)0x200010, need, NULL) ==
               MUON_ERR_WORKSPACE,
           "misaligned workspace");
    expect(muon_momentum_ns5_batched(g2, NULL, o2, rows, cols, 2, 0.95f, 5, 1e-7f, (void*)0x200000, need, NULL) ==
               MUON_ERR_INVALID_ARG,
           "null momentum buffers");
    expect(muon_momentum_ns5_batched_static(g2, NULL, o2, rows, cols, 2, 0.95f, 5, 1e-7f, NULL) ==
               MUON_ERR_INVALID_ARG,
           "static-workspace step without buffers");
    expect(MUON_STATIC_WORKSPACE_BYTES == (256u << 20), "static workspace size");
    expect(muon_momentum_ns5_apply_batched(g2, b2, o2, rows, cols, 2, 0.95f, INFINITY, 5, 1e-7f, (void*)0x200000,
                                           need, NULL) == MUON_ERR_INVALID_ARG,
           "infinite learning rate");
    expect(strlen(muon_last_error()) > 0, "a message for the last failure");
    expect(strcmp(muon_status_string(MUON_OK), "ok") == 0, "status string");
    if (failures == 0) printf("ok\n");
    return failures == 0 ? 0 : 1;
}
