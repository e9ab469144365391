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
// Per matrix the workspace holds:
//   X[2]  (mp x ldx, bf16, row-major): the iterate, ping-ponged between
//         steps.  A = X X^T is an NT product (both operands contiguous along
//         n); B X reads X as is (NN, through transposing LDS reads), so X is
//         never stored transposed.  X[1] also stages bf16(u) in the fused
//         Muon step until step 1 overwrites it.
//   A, B  (mp x lda, bf16)
//   float64 partial sums of squares for the Frobenius norm.
struct Ns5Plan {
    int64_t rows, cols;
    int m, n;
    bool tall;
    int tile;
    int mp, np;
    // tile of the symmetric products (X X^T, b A + c A A) and the padded
    // size they run on: the group tile and mp, or for m >= 2048 possibly 192
    // and m rounded up to 192 (>= mp), where that gives the CUs a fuller round
    // of tiles.  X has msym rows (the rows past mp stay zero) and A, B are
    // msym x msym.
    int sym_tile, msym;
    int nb;    // norm partials per matrix
    int cnt;   // matrices per pass
    // row strides (elements) of X (msym rows) and A, B (msym rows): the padded
    // widths plus a skew that keeps rows of power-of-two widths from all
    // starting on the same memory channel
    int ldx, lda;
    size_t x_elems, a_elems;  // per-matrix element counts
    size_t off_x[2], off_a, off_b, off_part;  // byte offsets
    size_t bytes;
};

bool make_plan(int64_t rows, int64_t cols, int64_t count, Ns5Plan* plan);

// muon_momentum_ns5_batched on a workspace of fixed size (api.hip): the batch
// runs in launch groups that each fit in ws_bytes; `workspace` is asked for
// the workspace's address (returning 0 or a MUON status) once the arguments
// have been validated.
int run_momentum_ns5_fixed_workspace(const float* const* g, float* const* buf, float* const* out,
                                     const int64_t* rows, const int64_t* cols, int64_t count, float mu, int steps,
                                     float eps, size_t ws_bytes, int (*workspace)(void**), hipStream_t stream);
// Records `msg` as the calling thread's last error and returns `status`.
int fail_status(int status, const char* msg);

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
    const bf16_t* E;
    int64_t e_mat;
    int lde;
    float alpha, beta;
    int m, n, tall;
    // final step: 0 writes O to the output table; 1 updates the parameters
    // there instead, p <- p - lr * O (one float32 rounding)
    int apply;
    float lr;
    int out16;  // final step: the output table holds bfloat16 (X as is)
};

struct GemmLaunch {
    GemmArgs seg[kMaxSeg];
    int nseg;
    // > 0: every segment has this many tiles per matrix, and whole matrices
    // are dealt round-robin over the XCDs (balances segments whose K
    // differs); 0: each XCD takes one contiguous range of the grid
    int interleave_tpm;
    // a X + B X only: 1 stores X' with streaming (non-temporal) stores
    int stream_out;
};

hipError_t launch_momentum(const float* g, float* buf, float* u, int64_t numel, float mu,
                           hipStream_t stream);

// Grouped momentum: up to kMaxMomentumGroup matrices per launch (one grid row
// each), passed by value in the kernel arguments.
constexpr int kMaxMomentumGroup = 64;
struct MomentumGroup {
    const float* g[kMaxMomentumGroup];
    float* buf[kMaxMomentumGroup];
    float* u[kMaxMomentumGroup];
    int64_t numel[kMaxMomentumGroup];
};
hipError_t launch_momentum_grouped(const MomentumGroup& t, int count, int64_t max_numel, float mu,
                                   hipStream_t stream);

// One chunk of a batched norm pass: workgroups [first_block, first_block +
// cnt * nb) of the launch; matrix i of the chunk is entry ptr_base + i of the
// launch's pointer tables.
struct NormSeg {
    int first_block;
    int nb;        // workgroups (float64 partial sums) per matrix
    int ptr_base;
    int vec;       // 16-byte accesses: pointers aligned, numel and chunk multiples of 4
    int64_t numel; // elements per matrix
    int64_t chunk; // elements per workgroup
    bf16_t* ub;    // momentum pass: bf16(u) staging copy, ub_mat elements per matrix
    int64_t ub_mat;
    double* partials;
};
struct NormLaunch {
    NormSeg seg[kMaxSeg];
    int nseg;
};

// Sum of squares of G (BUF null), or Nesterov momentum fused with it (buf
// updated, bf16(u) staged in ub): one launch over every chunk.
// in16: G holds bfloat16 values (sum of squares only).
hipError_t launch_norm(const NormLaunch& L, int blocks, const ConstPtrTable& G, const PtrTable* BUF, float mu,
                       hipStream_t stream, bool in16 = false);

// One chunk of a batched cast: X0 = bf16(bf16(G) / (||G|| + eps)) into X (the
// transpose of G when G is tall), over X's padded extent.  Each workgroup
// casts `per_wg` consecutive 64 x 64 tiles of one matrix.
struct CastSeg {
    int first_block;
    int tiles_c;        // tile columns of G's padded extent
    int tiles_per_mat;
    int wg_per_mat;     // ceil(tiles_per_mat / per_wg)
    int per_wg;
    int ptr_base;
    int rows, cols, tall, nb, ldx;
    const bf16_t* ub;   // bf16(G) staging copy (bf16 input; null: G itself is bf16), ub_mat elements per matrix
    int64_t ub_mat;
    const double* partials;
    bf16_t* X;
    int64_t x_mat;
};
struct CastLaunch {
    CastSeg seg[kMaxSeg];
    int nseg;
};

// bf16_in: cast from the staging copies (every chunk has one); else from the
// float32 G of the pointer table.
hipError_t launch_scale_cast(const CastLaunch& L, int blocks, const ConstPtrTable& G, bool bf16_in, float eps,
                             hipStream_t stream);

// out[i] = float32 of X (transposed back when G is tall): the steps = 0 result.
// apply: out[i] <- out[i] - lr * X (the parameter update) instead; out16:
// out[i] holds bfloat16 and receives X as is.
// Zeroes rows [first_row, rows) of each of cnt row-major bf16 matrices (ld
// elements per row, x_mat elements apart).
hipError_t launch_zero_rows(bf16_t* X, int64_t x_mat, int cnt, int first_row, int rows, int ld, hipStream_t stream);

hipError_t launch_copy_out(const Ns5Plan& plan, int cnt, const bf16_t* X, const PtrTable& out, hipStream_t stream,
                           bool apply = false, float lr = 0.0f, bool out16 = false);

// The whole NS5 (or Muon step) of small matrices, short side up to kSmallM
// and long side up to kSmallN, one workgroup per matrix with everything in
// LDS (small.hip), one launch over up to kMaxSeg segments of same-shaped
// matrices: segment q covers entries [first, first + cnt) of the pointer
// tables.  np is n rounded up to 32.  buf: the fused Muon step (float32
// only); io16: G and the outputs hold bfloat16 (pure NS5); apply: p <- p - lr
// * O into out.
constexpr int kSmallM = 64;
constexpr int kSmallN = 256;
struct SmallSeg {
    int first, cnt;
    int rows, cols, m, n, np, tall;
};
struct SmallArgs {
    SmallSeg seg[kMaxSeg];
    int nseg, steps, apply;
    float mu, eps, a, b, c, lr;
};
hipError_t launch_ns5_small(const SmallArgs& s, const ConstPtrTable& G, const PtrTable& out, const PtrTable* buf,
                            bool io16, hipStream_t stream);

// One GEMM launch of `blocks` workgroups with tile x tile_n output tiles:
// square tiles of 64, 128 or 256 for every kind, and 256 x 128 or 192 x 256
// for a X + B X.
hipError_t launch_gemm(GemmKind kind, int tile, int tile_n, const GemmLaunch& launch, int blocks,
                       const PtrTable* out, hipStream_t stream);

// The iteration carried in float32 (f32_iter.hip): one launch per product
// over `cnt` same-shaped matrices, 128 x 128 output tiles, float32 operands
// padded to whole tiles (the padding stays zero, as in the bf16 iteration).
// C = P Q with P M x K row-major; Q N x K row-major (X X^T) or K x N
// row-major (A A, B X); E is the fused update's second operand.
struct F32Gemm {
    const float* P;
    int64_t p_mat;
    int ldp;
    const float* Q;
    int64_t q_mat;
    int ldq;
    float* C;
    int64_t c_mat;
    int ldc;
    const float* E;
    int64_t e_mat;
    int lde;
    float alpha, beta;  // b A + c A A: alpha = b, beta = c; a X + B X: alpha = a
    int K;              // a multiple of 16
    int tiles, tiles_n, tiles_per_mat;
    int m, n, tall;     // last step: the output is m x n (or its transpose when tall)
};
hipError_t launch_f32_gemm(GemmKind kind, const F32Gemm& g, int blocks, const PtrTable* out, hipStream_t stream);

// X0 = G / (||G|| + eps) in float32 from the float64 norm partials (nb per
// matrix), into X (padded, transposed when G is tall) or (to_out) into the
// outputs in G's orientation.  32 x 32 tiles: tiles_c per row of tiles.
struct F32Scale {
    const double* partials;
    int nb;
    int rows, cols, tall;
    float* X;
    int64_t x_mat;
    int ldx;
    int tiles_c, tiles_per_mat;
    int cnt;  // matrices
    int to_out;
    float eps;
};
hipError_t launch_f32_scale(const F32Scale& s, const ConstPtrTable& G, const PtrTable* out, hipStream_t stream);

// U V^T through a block one-sided Jacobi SVD (polar_svd.hip), over `count`
// same-shaped matrices.  [W | J] per matrix: m_pad rows of ld floats, W in
// columns [0, n_pad) and the accumulated rotation J in [n_pad, ld).
struct SvdArgs {
    float* wj;
    int64_t mat_elems;   // floats per matrix (m_pad * ld)
    int ld;              // n_pad + m_pad
    int m, n, m_pad, n_pad;
    int blocks;          // row blocks of 32: m_pad / 32 (even)
    int count;
    int tall;            // G is tall: W = G^T, Q written back transposed
    double tol;          // largest cosine between two rows that needs no rotation
    double rank_tol;     // rows shorter than this times the longest are null space
    unsigned int* state; // per matrix: rotations in the current sweep, converged flag
    double* inv_len;     // per matrix: m_pad row lengths, then their inverses
};
hipError_t launch_svd_init(const SvdArgs& a, const ConstPtrTable& G, hipStream_t stream);
hipError_t launch_svd_sweep(const SvdArgs& a, bool last, hipStream_t stream);
hipError_t launch_svd_finish(const SvdArgs& a, const PtrTable& out, hipStream_t stream);

}  // namespace muon
