// The Newton-Schulz iteration carried in float32: the steps of the printed
// zeroth_power_via_newtonschulz5 (Muon section, Synced report on
// Modded-NanoGPT) with float32 in place of bfloat16, the precision the
// section's summary paragraph contrasts with the bf16 iteration.
//
//   X0 = G / (||G||_F + eps)      one float32 rounding of the float64 quotient
//                                 (transposed when G is tall)
//   A  = X X^T                    upper 128 x 128 tiles, mirrored
//   B  = b A + c A A              upper tiles, mirrored, fused update
//   X' = a X + B X                full tile grid, fused update; the last step
//                                 writes G's orientation, clipped to rows x cols
//
// gfx950 has no reduced-precision float32 matrix path, so the products run
// on v_mfma_f32_32x32x2_f32 (float32 operands, float32 accumulation), whose
// dense peak is 157.3 TFLOP/s, 1/16 of the bf16 one.  At that rate one MFMA
// (4096 flops) occupies a SIMD for 64 cycles, far longer than the LDS reads
// and global loads that feed it, so the engine is a plain one: 128 x 128
// tiles, 4 waves of 64 x 64 (2 x 2 fragments of 32 x 32), K steps of 16
// staged k-major in LDS through registers (the next step's global loads are
// in flight while the current one is multiplied), several workgroups per CU.
#include <stdlib.h>

#include "internal.hpp"

namespace muon {

namespace {

constexpr int FT = 128;        // output tile
constexpr int FK = 16;         // K step
constexpr int FLD = FT + 4;    // LDS row length (floats): k-major rows of 128 plus 4
constexpr int FT_THREADS = 256;
constexpr int kFKBlock = 64;   // K steps (of FK) per block of the two-level sum: 1024 K values
constexpr int kSplitK = 4096;  // longest K summed in one level
constexpr int64_t kMaxF32ScaleBlocks = int64_t{1} << 20;  // scale workgroups per launch

// MFMA v_mfma_f32_32x32x2_f32 operand layout: lane l supplies A[l % 32][l / 32]
// of the 32 x 2 left operand and B[l / 32][l % 32] of the 2 x 32 right one;
// accumulator register r of lane l holds row 8 (r / 4) + 4 (l / 32) + r % 4,
// column l % 32 of the 32 x 32 result.
template <int KIND, bool SPLIT>
__global__ __launch_bounds__(FT_THREADS) void k_f32_gemm(F32Gemm g, PtrTable out) {
    constexpr bool SYM = (KIND == GEMM_SYRK || KIND == GEMM_AAB);
    constexpr bool QT = (KIND == GEMM_SYRK);  // Q given as N x K rows (X X^T)
    __shared__ __attribute__((aligned(16))) float sP[2][FK][FLD];
    __shared__ __attribute__((aligned(16))) float sQ[2][FK][FLD];

    const int b = static_cast<int>(blockIdx.x);
    const int mat = b / g.tiles_per_mat;
    int t = b - mat * g.tiles_per_mat;
    int ti, tj;
    if constexpr (SYM) {  // upper triangle of tiles, row by row
        ti = 0;
        int rowlen = g.tiles;
        while (t >= rowlen) {
            t -= rowlen;
            ++ti;
            --rowlen;
        }
        tj = ti + t;
    } else {
        ti = t / g.tiles_n;
        tj = t - ti * g.tiles_n;
    }
    const int i0 = ti * FT, j0 = tj * FT;
    // P: rows i0.. of an M x K row-major matrix.  Q: rows j0.. of an N x K
    // matrix (QT), or columns j0.. of a K x N one.
    const float* P = g.P + static_cast<int64_t>(mat) * g.p_mat + static_cast<int64_t>(i0) * g.ldp;
    const float* Q = QT ? g.Q + static_cast<int64_t>(mat) * g.q_mat + static_cast<int64_t>(j0) * g.ldq
                        : g.Q + static_cast<int64_t>(mat) * g.q_mat + j0;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // Each thread moves two 16-byte pieces of each operand per K step.
    // Row-major M x K (and N x K) tiles: piece q covers row idx / 4, K
    // columns 4 (idx % 4) .. +3, stored transposed (k-major) in LDS.  K x N
    // tiles: row idx / 32, columns 4 (idx % 32) .. +3, stored as is.
    f32x4 rp[2], rq[2];
    auto gload = [&](int k0) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + FT_THREADS * q;
            const int r = idx >> 2, c = idx & 3;
            rp[q] = *reinterpret_cast<const f32x4*>(P + static_cast<int64_t>(r) * g.ldp + k0 + 4 * c);
            if constexpr (QT) {
                rq[q] = *reinterpret_cast<const f32x4*>(Q + static_cast<int64_t>(r) * g.ldq + k0 + 4 * c);
            } else {
                const int rr = idx >> 5, cc = idx & 31;
                rq[q] = *reinterpret_cast<const f32x4*>(Q + static_cast<int64_t>(k0 + rr) * g.ldq + 4 * cc);
            }
        }
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int idx = tid + FT_THREADS * q;
            const int r = idx >> 2, c = idx & 3;
#pragma unroll
            for (int e = 0; e < 4; ++e) sP[buf][4 * c + e][r] = rp[q][e];
            if constexpr (QT) {
#pragma unroll
                for (int e = 0; e < 4; ++e) sQ[buf][4 * c + e][r] = rq[q][e];
            } else {
                const int rr = idx >> 5, cc = idx & 31;
                *reinterpret_cast<f32x4*>(&sQ[buf][rr][4 * cc]) = rq[q];
            }
        }
    };

    // SPLIT (long K): a two-level sum.  The matrix cores accumulate one block
    // of kFKBlock K steps (1024 K values) at a time into `acc`, and each
    // block's sum is added to `tot` with one float32 rounding, block after
    // block.  The matrix cores' accumulator drifts from a round-to-nearest
    // sum by an amount that grows with the number of terms it carries, so
    // capping that number keeps a long K as close to the float64 sum as a
    // short one.  The second set of accumulators costs registers (two waves
    // per SIMD instead of four), so sums of up to kSplitK terms keep the one
    // level.
    f32x16 acc[2][2], tot[2][2];
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = tot[fm][fn][r] = 0.0f;

    const int nk = g.K / FK;
    gload(0);
    lstore(0);
    __syncthreads();
    const int fr = lane & 31, fk = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * FK);
#pragma unroll
        for (int kk = 0; kk < FK; kk += 2) {
            float a[2], bq[2];
#pragma unroll
            for (int f = 0; f < 2; ++f) {
                a[f] = sP[cur][kk + fk][wm * 64 + f * 32 + fr];
                bq[f] = sQ[cur][kk + fk][wn * 64 + f * 32 + fr];
            }
#pragma unroll
            for (int fm = 0; fm < 2; ++fm)
#pragma unroll
                for (int fn = 0; fn < 2; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[fm], bq[fn], acc[fm][fn], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        if (SPLIT && ((kt + 1) % kFKBlock == 0 || kt + 1 == nk)) {  // close the block
#pragma unroll
            for (int fm = 0; fm < 2; ++fm)
#pragma unroll
                for (int fn = 0; fn < 2; ++fn)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        tot[fm][fn][r] += acc[fm][fn][r];
                        acc[fm][fn][r] = 0.0f;
                    }
        }
        __syncthreads();
    }

    // ---- epilogue: element (i, j) of the tile from register r of fragment
    // (fm, fn); the fused update in float32, one rounding each
    float* C = SYM || KIND == GEMM_BX ? g.C + static_cast<int64_t>(mat) * g.c_mat : nullptr;
    const float* E = g.E ? g.E + static_cast<int64_t>(mat) * g.e_mat : nullptr;
    float* o = KIND == GEMM_BX_FINAL ? out.p[mat] : nullptr;
#pragma unroll
    for (int fm = 0; fm < 2; ++fm)
#pragma unroll
        for (int fn = 0; fn < 2; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int i = i0 + wm * 64 + fm * 32 + 8 * (r >> 2) + 4 * fk + (r & 3);
                const int j = j0 + wn * 64 + fn * 32 + fr;
                float v = SPLIT ? tot[fm][fn][r] : acc[fm][fn][r];
                if constexpr (KIND == GEMM_SYRK) {
                    // upper tiles hold (i, j) and its mirror; a diagonal tile
                    // writes i <= j only, so A is exactly symmetric
                    if (ti < tj || i <= j) {
                        C[static_cast<int64_t>(i) * g.ldc + j] = v;
                        C[static_cast<int64_t>(j) * g.ldc + i] = v;
                    }
                } else if constexpr (KIND == GEMM_AAB) {  // b A + c (A A)
                    if (ti < tj || i <= j) {
                        v = fmaf(g.beta, v, g.alpha * E[static_cast<int64_t>(i) * g.lde + j]);
                        C[static_cast<int64_t>(i) * g.ldc + j] = v;
                        C[static_cast<int64_t>(j) * g.ldc + i] = v;
                    }
                } else {  // a X + (B X)
                    v = fmaf(g.alpha, E[static_cast<int64_t>(i) * g.lde + j], v);
                    if constexpr (KIND == GEMM_BX) {
                        C[static_cast<int64_t>(i) * g.ldc + j] = v;
                    } else if (i < g.m && j < g.n) {  // G's orientation, rows x cols
                        if (g.tall)
                            o[static_cast<int64_t>(j) * g.m + i] = v;
                        else
                            o[static_cast<int64_t>(i) * g.n + j] = v;
                    }
                }
            }
}

// X0 = fl32(G / d) with d = sqrt(sum of the matrix's float64 partials) + eps,
// the quotient formed in float64.  32 x 32 tiles of 32 x 8 threads, taken
// grid-stride (the grid is capped so that the largest shapes fit a launch).
// Into the workspace (X's padded extent, zeros outside G, transposed through
// LDS when G is tall), or (to_out) straight into the outputs in G's
// orientation.
__global__ __launch_bounds__(FT_THREADS) void k_f32_scale(F32Scale s, ConstPtrTable G, PtrTable out) {
    const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
    __shared__ double dsh;
    __shared__ float tl[32][33];
    const int64_t total = static_cast<int64_t>(s.tiles_per_mat) * s.cnt;
    for (int64_t b = blockIdx.x; b < total; b += gridDim.x) {
        const int mat = static_cast<int>(b / s.tiles_per_mat);
        const int t = static_cast<int>(b - static_cast<int64_t>(mat) * s.tiles_per_mat);
        const int ti = t / s.tiles_c, tj = t - ti * s.tiles_c;
        __syncthreads();  // the previous tile is done with dsh and tl
        if (threadIdx.x == 0) {  // fixed order: every tile of a matrix gets the same d
            const double* pp = s.partials + static_cast<int64_t>(mat) * s.nb;
            double acc = 0.0;
            for (int p = 0; p < s.nb; ++p) acc += pp[p];
            dsh = sqrt(acc) + static_cast<double>(s.eps);
        }
        __syncthreads();
        const double d = dsh;
        const float* g = G.p[mat];
        const int i0 = ti * 32, j0 = tj * 32;
        if (s.to_out) {  // rows x cols, no padding, no transpose
            float* o = out.p[mat];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = i0 + ty + 8 * rr, j = j0 + tx;
                if (i < s.rows && j < s.cols)
                    o[static_cast<int64_t>(i) * s.cols + j] =
                        static_cast<float>(static_cast<double>(g[static_cast<int64_t>(i) * s.cols + j]) / d);
            }
            continue;
        }
        float* X = s.X + static_cast<int64_t>(mat) * s.x_mat;
        const int m = s.tall ? s.cols : s.rows, n = s.tall ? s.rows : s.cols;
        if (!s.tall) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = i0 + ty + 8 * rr, j = j0 + tx;
                const float v =
                    (i < m && j < n) ? static_cast<float>(static_cast<double>(g[static_cast<int64_t>(i) * s.cols + j]) / d)
                                     : 0.0f;
                X[static_cast<int64_t>(i) * s.ldx + j] = v;
            }
        } else {
            // X[i][j] = G[j][i]: read the G tile along its rows, write X along
            // its rows
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int jj = j0 + ty + 8 * rr, ii = i0 + tx;
                tl[ty + 8 * rr][tx] = (jj < n && ii < m) ? g[static_cast<int64_t>(jj) * s.cols + ii] : 0.0f;
            }
            __syncthreads();
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = i0 + ty + 8 * rr, j = j0 + tx;
                X[static_cast<int64_t>(i) * s.ldx + j] = static_cast<float>(static_cast<double>(tl[tx][ty + 8 * rr]) / d);
            }
        }
    }
}

}  // namespace

hipError_t launch_f32_gemm(GemmKind kind, const F32Gemm& g, int blocks, const PtrTable* out, hipStream_t stream) {
    PtrTable o{};
    if (out) o = *out;
    const bool split = g.K > kSplitK;
    switch (kind * 2 + (split ? 1 : 0)) {
        case GEMM_SYRK * 2: k_f32_gemm<GEMM_SYRK, false><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_SYRK * 2 + 1: k_f32_gemm<GEMM_SYRK, true><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_AAB * 2: k_f32_gemm<GEMM_AAB, false><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_AAB * 2 + 1: k_f32_gemm<GEMM_AAB, true><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_BX * 2: k_f32_gemm<GEMM_BX, false><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_BX * 2 + 1: k_f32_gemm<GEMM_BX, true><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_BX_FINAL * 2: k_f32_gemm<GEMM_BX_FINAL, false><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        case GEMM_BX_FINAL * 2 + 1: k_f32_gemm<GEMM_BX_FINAL, true><<<blocks, FT_THREADS, 0, stream>>>(g, o); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_f32_scale(const F32Scale& s, const ConstPtrTable& G, const PtrTable* out, hipStream_t stream) {
    PtrTable o{};
    if (out) o = *out;
    // the kernel walks s.tiles_per_mat * s.cnt tiles grid-stride
    // MUON_F32_SCALE_WG_CAP=n lowers the cap (read once per process; tests of
    // the several-tiles path, which only very large inputs reach otherwise,
    // run in a process of their own with it set)
    static const int64_t cap = [] {
        const char* e = getenv("MUON_F32_SCALE_WG_CAP");
        const long long v = e ? atoll(e) : 0;
        return (v >= 1 && v < kMaxF32ScaleBlocks) ? static_cast<int64_t>(v) : kMaxF32ScaleBlocks;
    }();
    const int64_t total = static_cast<int64_t>(s.tiles_per_mat) * s.cnt;
    const int64_t grid = total < cap ? total : cap;
    k_f32_scale<<<static_cast<unsigned>(grid), FT_THREADS, 0, stream>>>(s, G, o);
    return hipGetLastError();
}

}  // namespace muon
