// U V^T of G = U S V^T through an SVD on the GPU: the orthogonalisation that
// the Muon section of the Synced report on Modded-NanoGPT says NS5
// approximates, and that it calls too slow to use in the optimizer.  Built
// as a second workload to measure that claim against NS5 on the same
// matrices.
//
// Method: block one-sided Jacobi (Hestenes) on the rows of W (m x n, m <= n,
// G itself or its transpose), float32 storage, float64 arithmetic.
//   * [W | J] holds W and the accumulated rotation J (m x m, starting at I).
//   * The rows are split into blocks of kRowsPerBlock; one sweep pairs every
//     block with every other once (round-robin: P - 1 rounds of P / 2
//     disjoint pairs for P blocks, one launch per round over all matrices).
//   * A pair of blocks (64 rows): its Gram matrix M = W_pair W_pair^T in
//     float64; if some pair of its rows is not yet orthogonal to the
//     tolerance, M is diagonalised by cyclic Jacobi in LDS, R M R^T = D, and R
//     is applied to the pair's rows of [W | J].  The rows of W then become
//     mutually orthogonal: J W = D^(1/2) N with N orthonormal, so G's SVD is
//     W = J^T D^(1/2) N and U V^T = J^T N.
//   * After each sweep a matrix whose pairs all met the tolerance is marked
//     converged, and later launches skip it; sweeps stop at max_sweeps.
//   * Finally N = rows of W scaled to unit length (rows whose length is below
//     a rank tolerance, the null space of a rank-deficient G, become 0, so
//     the result is U_r V_r^T over the nonzero singular values) and
//     Q = J^T N is written in G's orientation.
// No step waits on another workgroup: launches are ordered on the stream.
#include "internal.hpp"

namespace muon {

namespace {

constexpr int kRowsPerBlock = 32;
constexpr int kPairRows = 2 * kRowsPerBlock;  // rows of one block pair: 64
constexpr int kChunk = 64;                     // columns per LDS chunk
constexpr int kEigSweeps = 16;                 // cap on the cyclic Jacobi sweeps of one 64 x 64 problem

// Global row index of row r (0..63) of the pair (bi, bj).
__device__ __forceinline__ int pair_row(int r, int bi, int bj) {
    return r < kRowsPerBlock ? bi * kRowsPerBlock + r : bj * kRowsPerBlock + (r - kRowsPerBlock);
}

// Round-robin (circle method) on P players: in round r (0 .. P-2), pair k
// (0 .. P/2 - 1) is (P-1, r) for k = 0 and ((r + k) mod (P-1),
// (r - k) mod (P-1)) otherwise; over P - 1 rounds every two players meet once.
__device__ __forceinline__ void round_pair(int P, int r, int k, int* bi, int* bj) {
    if (k == 0) {
        *bi = r;
        *bj = P - 1;
    } else {
        const int a = (r + k) % (P - 1), b = (r - k + (P - 1)) % (P - 1);
        *bi = a < b ? a : b;
        *bj = a < b ? b : a;
    }
}

// One round: every block pair of every non-converged matrix.
__global__ __launch_bounds__(kThreads) void k_svd_round(SvdArgs a, int round) {
    const int pairs = a.blocks / 2;
    const int mat = static_cast<int>(blockIdx.x) / pairs, k = static_cast<int>(blockIdx.x) % pairs;
    if (a.state[2 * mat + 1]) return;  // converged (uniform over the workgroup)
    int bi, bj;
    round_pair(a.blocks, round, k, &bi, &bj);
    float* WJ = a.wj + static_cast<int64_t>(mat) * a.mat_elems;

    __shared__ double M[kPairRows][kPairRows + 1];
    __shared__ double R[kPairRows][kPairRows + 1];
    __shared__ float C[kPairRows][kChunk + 1];
    __shared__ double cs[kPairRows / 2], sn[kPairRows / 2];
    __shared__ int pp[kPairRows / 2], qq[kPairRows / 2];
    __shared__ double red[kThreads / 64];
    __shared__ int flag;

    const int t = threadIdx.x;
    const int ti = 4 * (t / 16), tj = 4 * (t % 16);  // this thread's 4 x 4 block of a 64 x 64 result

    // ---- Gram matrix of the pair's 64 rows of W, float64
    double g[4][4] = {};
    for (int c0 = 0; c0 < a.n_pad; c0 += kChunk) {
        __syncthreads();
        for (int e = t; e < kPairRows * kChunk / 4; e += kThreads) {
            const int r = e / (kChunk / 4), q = e % (kChunk / 4);
            const f32x4 v = *reinterpret_cast<const f32x4*>(
                WJ + static_cast<int64_t>(pair_row(r, bi, bj)) * a.ld + c0 + 4 * q);
            C[r][4 * q + 0] = v[0];
            C[r][4 * q + 1] = v[1];
            C[r][4 * q + 2] = v[2];
            C[r][4 * q + 3] = v[3];
        }
        __syncthreads();
        for (int kk = 0; kk < kChunk; ++kk) {
            double x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = C[ti + u][kk];
                y[u] = C[tj + u][kk];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) g[u][v] = fma(x[u], y[v], g[u][v]);
        }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            M[ti + u][tj + v] = g[u][v];
            R[ti + u][tj + v] = (ti + u == tj + v) ? 1.0 : 0.0;
        }
    __syncthreads();

    // ---- largest cosine between two of the pair's rows; below the tolerance
    // the pair is left as it is
    double worst = 0.0;
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = ti + u, j = tj + v;
            const double d = M[i][i] * M[j][j];
            if (i < j && d > 0.0) worst = fmax(worst, fabs(M[i][j]) / sqrt(d));
        }
    for (int off = 32; off >= 1; off >>= 1) worst = fmax(worst, __shfl_xor(worst, off, 64));
    if ((t & 63) == 0) red[t >> 6] = worst;
    __syncthreads();
    worst = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    if (worst <= a.tol) return;
    if (t == 0) atomicAdd(reinterpret_cast<unsigned int*>(&a.state[2 * mat]), 1u);

    // ---- diagonalise M: cyclic Jacobi, 63 rounds of 32 disjoint rotations
    // per sweep (the same circle method on 64 indices); each rotation acts on
    // rows p, q (then columns p, q) as row_p <- c row_p - s row_q,
    // row_q <- s row_p + c row_q, with tan of its angle chosen to zero M_pq
    for (int sweep = 0; sweep < kEigSweeps; ++sweep) {
        for (int r = 0; r < kPairRows - 1; ++r) {
            if (t < kPairRows / 2) {
                int p, q;
                round_pair(kPairRows, r, t, &p, &q);
                const double mpq = M[p][q], mpp = M[p][p], mqq = M[q][q];
                double c = 1.0, s = 0.0;
                if (fabs(mpq) > 1e-300 && fabs(mpq) > 1e-17 * sqrt(fabs(mpp * mqq))) {
                    const double tau = (mqq - mpp) / (2.0 * mpq);
                    const double tn = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
                    c = 1.0 / sqrt(1.0 + tn * tn);
                    s = tn * c;
                }
                cs[t] = c;
                sn[t] = s;
                pp[t] = p;
                qq[t] = q;
            }
            __syncthreads();
            // rows of M and of R: 32 pairs x 64 columns, 8 per thread
            for (int e = t; e < (kPairRows / 2) * kPairRows; e += kThreads) {
                const int w = e / kPairRows, j = e % kPairRows;
                const int p = pp[w], q = qq[w];
                const double c = cs[w], s = sn[w];
                const double mp = M[p][j], mq = M[q][j];
                M[p][j] = c * mp - s * mq;
                M[q][j] = s * mp + c * mq;
                const double rp = R[p][j], rq = R[q][j];
                R[p][j] = c * rp - s * rq;
                R[q][j] = s * rp + c * rq;
            }
            __syncthreads();
            // columns of M
            for (int e = t; e < (kPairRows / 2) * kPairRows; e += kThreads) {
                const int w = e / kPairRows, i = e % kPairRows;
                const int p = pp[w], q = qq[w];
                const double c = cs[w], s = sn[w];
                const double mp = M[i][p], mq = M[i][q];
                M[i][p] = c * mp - s * mq;
                M[i][q] = s * mp + c * mq;
            }
            __syncthreads();
        }
        // converged when every off-diagonal entry is negligible against its
        // diagonal pair
        double off = 0.0;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = ti + u, j = tj + v;
                const double d = fabs(M[i][i] * M[j][j]);
                if (i < j && fabs(M[i][j]) > 1e-300) off = fmax(off, d > 0.0 ? fabs(M[i][j]) / sqrt(d) : 1.0);
            }
        for (int o = 32; o >= 1; o >>= 1) off = fmax(off, __shfl_xor(off, o, 64));
        if ((t & 63) == 0) red[t >> 6] = off;
        __syncthreads();
        if (t == 0) flag = fmax(fmax(red[0], red[1]), fmax(red[2], red[3])) <= 1e-15;
        __syncthreads();
        if (flag) break;
    }

    // ---- [W | J] rows of the pair <- R x those rows, chunk by chunk
    for (int c0 = 0; c0 < a.ld; c0 += kChunk) {
        __syncthreads();
        for (int e = t; e < kPairRows * kChunk / 4; e += kThreads) {
            const int r = e / (kChunk / 4), q = e % (kChunk / 4);
            const f32x4 v = *reinterpret_cast<const f32x4*>(
                WJ + static_cast<int64_t>(pair_row(r, bi, bj)) * a.ld + c0 + 4 * q);
            C[r][4 * q + 0] = v[0];
            C[r][4 * q + 1] = v[1];
            C[r][4 * q + 2] = v[2];
            C[r][4 * q + 3] = v[3];
        }
        __syncthreads();
        double o[4][4] = {};
        for (int kk = 0; kk < kPairRows; ++kk) {
            double x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = R[ti + u][kk];
                y[u] = C[kk][tj + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) o[u][v] = fma(x[u], y[v], o[u][v]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4 v{static_cast<float>(o[u][0]), static_cast<float>(o[u][1]), static_cast<float>(o[u][2]),
                          static_cast<float>(o[u][3])};
            *reinterpret_cast<f32x4*>(WJ + static_cast<int64_t>(pair_row(ti + u, bi, bj)) * a.ld + c0 + tj) = v;
        }
    }
}

// After a sweep: a matrix none of whose pairs rotated is converged; the
// rotation counters start again from zero.
__global__ void k_svd_sweep_end(SvdArgs a, int last) {
    const int mat = static_cast<int>(blockIdx.x * blockDim.x + threadIdx.x);
    if (mat >= a.count) return;
    if (a.state[2 * mat] == 0u || last) a.state[2 * mat + 1] = 1u;
    a.state[2 * mat] = 0u;
}

// [W | J] <- W^T or W (G's values, zero padded) and the identity.
__global__ void k_svd_init(SvdArgs a, ConstPtrTable G) {
    const int mat = blockIdx.y;
    float* WJ = a.wj + static_cast<int64_t>(mat) * a.mat_elems;
    const float* g = G.p[mat];
    const int64_t total = static_cast<int64_t>(a.m_pad) * a.ld;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < total;
         e += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        const int i = static_cast<int>(e / a.ld), j = static_cast<int>(e % a.ld);
        float v = 0.0f;
        if (j < a.n_pad) {
            if (i < a.m && j < a.n) v = a.tall ? g[static_cast<int64_t>(j) * a.m + i] : g[static_cast<int64_t>(i) * a.n + j];
        } else if (j - a.n_pad == i) {
            v = 1.0f;
        }
        WJ[e] = v;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.state[2 * mat] = 0u;
        a.state[2 * mat + 1] = 0u;
    }
}

// Length of every row of W (float64), one wave per row.
__global__ __launch_bounds__(kThreads) void k_svd_row_len(SvdArgs a) {
    const int mat = blockIdx.y, row = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (row >= a.m_pad) return;  // whole waves
    const float* w = a.wj + static_cast<int64_t>(mat) * a.mat_elems + static_cast<int64_t>(row) * a.ld;
    double s = 0.0;
    for (int j = lane; j < a.n_pad; j += 64) {
        const double v = w[j];
        s = fma(v, v, s);
    }
    for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
    if (lane == 0) a.inv_len[static_cast<int64_t>(mat) * a.m_pad + row] = sqrt(s);
}

// 1 / (row length), or 0 for rows below the rank tolerance (rank_tol times
// the longest row of the matrix: the null space of a rank-deficient G).  One
// workgroup per matrix.
__global__ __launch_bounds__(kThreads) void k_svd_row_scale(SvdArgs a) {
    double* inv = a.inv_len + static_cast<int64_t>(blockIdx.x) * a.m_pad;
    __shared__ double red[kThreads / 64];
    double longest = 0.0;
    for (int i = threadIdx.x; i < a.m_pad; i += kThreads) longest = fmax(longest, inv[i]);
    for (int off = 32; off >= 1; off >>= 1) longest = fmax(longest, __shfl_xor(longest, off, 64));
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = longest;
    __syncthreads();
    longest = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    for (int i = threadIdx.x; i < a.m_pad; i += kThreads) {
        const double len = inv[i];
        inv[i] = (len > 0.0 && len > a.rank_tol * longest) ? 1.0 / len : 0.0;
    }
}

// Q = J^T diag(inv_len) W, written in G's orientation: 64 x 64 output tiles,
// K (the m rows) in chunks of 64 through LDS, float64 sums.
__global__ __launch_bounds__(kThreads) void k_svd_polar(SvdArgs a, PtrTable out) {
    const int mat = blockIdx.z;
    const int i0 = blockIdx.y * 64, j0 = blockIdx.x * 64;  // rows (of m) and columns (of n) of Q
    const float* WJ = a.wj + static_cast<int64_t>(mat) * a.mat_elems;
    const double* inv = a.inv_len + static_cast<int64_t>(mat) * a.m_pad;
    __shared__ float Jt[64][65];  // Jt[k][i] = J[k0 + k][i0 + i]
    __shared__ float Nt[64][65];  // Nt[k][j] = inv[k0 + k] W[k0 + k][j0 + j]
    const int t = threadIdx.x, ti = 4 * (t / 16), tj = 4 * (t % 16);
    double o[4][4] = {};
    for (int k0 = 0; k0 < a.m_pad; k0 += 64) {
        __syncthreads();
        for (int e = t; e < 64 * 64; e += kThreads) {
            const int k = e / 64, c = e % 64;
            const int64_t row = static_cast<int64_t>(k0 + k) * a.ld;
            Jt[k][c] = WJ[row + a.n_pad + i0 + c];
            Nt[k][c] = static_cast<float>(inv[k0 + k] * WJ[row + j0 + c]);
        }
        __syncthreads();
        for (int k = 0; k < 64; ++k) {
            double x[4], y[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                x[u] = Jt[k][ti + u];
                y[u] = Nt[k][tj + u];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int v = 0; v < 4; ++v) o[u][v] = fma(x[u], y[v], o[u][v]);
        }
    }
    float* q = out.p[mat];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int i = i0 + ti + u, j = j0 + tj + v;
            if (i < a.m && j < a.n) {
                if (a.tall)
                    q[static_cast<int64_t>(j) * a.m + i] = static_cast<float>(o[u][v]);
                else
                    q[static_cast<int64_t>(i) * a.n + j] = static_cast<float>(o[u][v]);
            }
        }
}

}  // namespace

hipError_t launch_svd_init(const SvdArgs& a, const ConstPtrTable& G, hipStream_t stream) {
    const int64_t total = static_cast<int64_t>(a.m_pad) * a.ld;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 4096) blocks = 4096;
    k_svd_init<<<dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(a.count)), kThreads, 0, stream>>>(a, G);
    return hipGetLastError();
}

hipError_t launch_svd_sweep(const SvdArgs& a, bool last, hipStream_t stream) {
    const int rounds = a.blocks - 1;
    for (int r = 0; r < rounds; ++r) {
        k_svd_round<<<a.count * (a.blocks / 2), kThreads, 0, stream>>>(a, r);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    k_svd_sweep_end<<<(a.count + 63) / 64, 64, 0, stream>>>(a, last ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_svd_finish(const SvdArgs& a, const PtrTable& out, hipStream_t stream) {
    k_svd_row_len<<<dim3(static_cast<unsigned>(a.m_pad / (kThreads / 64)), static_cast<unsigned>(a.count)), kThreads,
                    0, stream>>>(a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    k_svd_row_scale<<<a.count, kThreads, 0, stream>>>(a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 grid(static_cast<unsigned>((a.n + 63) / 64), static_cast<unsigned>((a.m + 63) / 64),
                    static_cast<unsigned>(a.count));
    k_svd_polar<<<grid, kThreads, 0, stream>>>(a, out);
    return hipGetLastError();
}

}  // namespace muon
