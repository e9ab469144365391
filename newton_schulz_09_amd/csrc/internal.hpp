// Internal interfaces between the C-ABI layer (api.hip) and the kernels.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "common.hpp"

namespace muon {

// Layout of one NS5 pass over `cnt` same-shaped matrices.
//
// G is rows x cols; the iteration runs on X (m x n, m = min, n = max).  Every
// dimension is padded to a multiple of the GEMM tile T; the padding is written
// as zeros by the cast kernel and stays exactly zero through the iteration
// (zero rows/columns of X give zero rows/columns of A, B and the next X), so
// the GEMMs run on whole tiles with no edge predication.
//
// Per matrix the workspace holds, all bf16:
//   X[2]  (mp x np, row-major)  and  XT[2] (np x mp): the iterate in both
//         orientations, ping-ponged between steps, so that every product is
//         a "both operands contiguous along K" (NT) product:
//             A  = X  . X^T   -> NT(X,  X)     K = n
//             AA = A  . A^T   -> NT(A,  A)     K = m   (A is symmetric)
//             BX = B  . X     -> NT(B,  XT)    K = m
//   A, B  (mp x mp)
// plus float64 partial sums of squares for the Frobenius norm.
struct Ns5Plan {
    int64_t rows, cols;
    int m, n;
    bool tall;
    int tile;
    int mp, np;
    int nb;    // norm partials per matrix
    int cnt;   // matrices per pass
    // row strides (elements) of X (mp rows), X^T (np rows) and A, B (mp rows):
    // the padded widths plus a skew that keeps rows of power-of-two widths
    // from all starting on the same memory channel
    int ldx, ldxt, lda;
    size_t x_elems, xt_elems, a_elems;  // per-matrix element counts
    size_t off_x[2], off_xt[2], off_a, off_b, off_part;  // byte offsets
    size_t bytes;
};

bool make_plan(int64_t rows, int64_t cols, int64_t count, Ns5Plan* plan);

enum GemmKind { GEMM_SYRK = 0, GEMM_AAB = 1, GEMM_BX = 2, GEMM_BX_FINAL = 3 };

// One segment of a GEMM launch: `cnt` same-shaped matrices laid out as in
// an Ns5Plan.  A launch covers up to kMaxSeg segments that share the tile
// size; workgroups [first_block, first_block + cnt * tiles_per_mat) of the
// launch's logical grid belong to this segment.
constexpr int kMaxSeg = 8;

struct GemmArgs {
    int first_block;
    int out_base;       // index of the segment's first matrix in the output table
    const bf16_t* P;
    int64_t p_mat;
    int ldp;
    const bf16_t* Q;
    int64_t q_mat;
    int ldq;
    int kpad;
    int tiles;          // tiles per side of the output grid (rows)
    int tiles_n;        // tiles along the output columns
    int tiles_per_mat;
    int band;           // full grid: tiles are ordered in bands of this many tile rows
    bf16_t* C;
    int64_t c_mat;
    int ldc;
    bf16_t* CT;
    int64_t ct_mat;
    int ldct;
    const bf16_t* E;
    int64_t e_mat;
    int lde;
    float alpha, beta;
    int m, n, tall;
};

struct GemmLaunch {
    GemmArgs seg[kMaxSeg];
    int nseg;
};

hipError_t launch_momentum(const float* g, float* buf, float* u, int64_t numel, float mu,
                           hipStream_t stream);

hipError_t launch_sumsq(const ConstPtrTable& G, int cnt, int64_t numel, int nb, double* partials,
                        hipStream_t stream);

// ub (if non-null): dense bf16 copies of the inputs (stride ub_mat per
// matrix) to cast from instead of the float32 G.
hipError_t launch_scale_cast(const ConstPtrTable& G, const bf16_t* ub, int64_t ub_mat, int cnt, const Ns5Plan& plan,
                             const double* partials, float eps, bf16_t* nat, bf16_t* tr, hipStream_t stream);

hipError_t launch_momentum_norm(const ConstPtrTable& G, const PtrTable& BUF, int cnt, int64_t numel, int nb,
                                float mu, bf16_t* ub, int64_t ub_mat, double* partials, hipStream_t stream);

hipError_t launch_copy_out(const Ns5Plan& plan, int cnt, const bf16_t* nat, const PtrTable& out,
                           hipStream_t stream);

hipError_t launch_gemm(GemmKind kind, int tile, const GemmLaunch& launch, int blocks, const PtrTable* out,
                       hipStream_t stream);

}  // namespace muon
