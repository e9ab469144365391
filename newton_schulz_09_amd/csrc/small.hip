// The whole Muon step of a small matrix (short side up to 64, long side up to
// 256) in one workgroup: the Nesterov momentum, the Frobenius norm and bf16
// cast, every quintic Newton-Schulz step and the output (the printed
// zeroth_power_via_newtonschulz5 of the Muon section, Synced report on
// Modded-NanoGPT), with X, its transpose, A and B resident in LDS.
//
// Such a matrix leaves nearly all of the GPU idle in the tiled path, which
// spends its time in the 17 launches of a step (momentum + norm, cast, three
// products per NS5 step); here the call is one launch of one workgroup per
// matrix, of 8 waves (two per SIMD, so that one hides the other's
// latencies).  The arithmetic and its rounding points are those of the tiled
// path: momentum as two float32 fused multiply-adds, the sum of squares of u
// in float64, X0 = bf16(bf16(u) / (||u|| + eps)) with the quotient in
// float64, products on the 32 x 32 x 16 bf16 matrix cores with float32
// accumulation in K order, A = bf16(X X^T) and B = bf16(c (A A) + b A) from
// their upper blocks (diagonal blocks symmetrised), X' = bf16(B X + a X).
// Every matrix in the small range takes this path in every entry point, so a
// matrix gets bitwise the same result alone or in any batch.
#include "internal.hpp"

namespace muon {

namespace {

constexpr int kST = 512;  // threads per workgroup: 8 waves, two per SIMD
constexpr int kLdx = kSmallN + 8;  // X row stride (elements): 16-byte aligned rows
constexpr int kLdt = kSmallM + 8;  // X^T, A and B row stride

typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 ld8(const bf16_t* p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4s*>(p));
}

__device__ __forceinline__ double wave_sum_small(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Walks the elements e = e0, e0 + stride, ... of a row-major extent with
// `width` columns as (row, col) pairs, carrying instead of dividing.
struct RowCol {
    int r, c, dr, dc, width;
    __device__ __forceinline__ RowCol(int e0, int stride, int w)
        : r(e0 / w), c(e0 - (e0 / w) * w), dr(stride / w), dc(stride - (stride / w) * w), width(w) {}
    __device__ __forceinline__ void next() {
        r += dr;
        c += dc;
        if (c >= width) {
            c -= width;
            ++r;
        }
    }
};

// Row and column of accumulator register r of a 32 x 32 fragment in lane l.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// One symmetric 64 x 64 product C = bf16(beta * (P P^T) + alpha * E) of a
// 64-row operand P (K columns, a multiple of 16, row stride ldp), over its
// upper 32 x 32 blocks on waves 0..2; with beta = 1 and alpha = 0 (no E) it is
// A = bf16(X X^T).  Block (0, 1) is also stored transposed, a diagonal block
// keeps its upper triangle and mirrors it, so C is exactly symmetric.
template <bool HAS_E>
__device__ __forceinline__ void sym_product(const bf16_t* P, int ldp, int K, const bf16_t* E, float alpha,
                                            float beta, bf16_t* C, int wave, int lane) {
    if (wave >= 3) return;
    const int bi = wave == 2 ? 1 : 0, bj = wave == 0 ? 0 : 1;
    const bf16_t* pa = P + (32 * bi + (lane & 31)) * ldp + 8 * (lane >> 5);
    const bf16_t* pb = P + (32 * bj + (lane & 31)) * ldp + 8 * (lane >> 5);
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
    for (int k0 = 0; k0 < K; k0 += 16)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(pa + k0), ld8(pb + k0), acc, 0, 0, 0);
    const int col = lane & 31;
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
        v[r] = acc[r];
        if constexpr (HAS_E)
            v[r] = fmaf(beta, v[r], alpha * bf16_to_f32(E[(32 * bi + acc_row(r, lane)) * kLdt + 32 * bj + col]));
    }
    if (bi != bj) {  // (wave-uniform) the block and its transpose
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int gi = 32 * bi + acc_row(r, lane), gj = 32 * bj + col;
            const bf16_t h = f32_to_bf16(v[r]);
            C[gi * kLdt + gj] = h;
            C[gj * kLdt + gi] = h;
        }
    } else {  // a diagonal block: its upper triangle, mirrored
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int row = acc_row(r, lane);
            const int gi = 32 * bi + row, gj = 32 * bj + col;
            const bf16_t h = f32_to_bf16(v[r]);
            if (row <= col) {
                C[gi * kLdt + gj] = h;
                C[gj * kLdt + gi] = h;
            }
        }
    }
}

template <bool MOM, bool IO16>
__global__ __launch_bounds__(kST) void k_ns5_small(SmallArgs s, ConstPtrTable G, PtrTable OUT, PtrTable BUF) {
    __shared__ __attribute__((aligned(16))) bf16_t X[kSmallM * kLdx];   // m x n (64 x np used)
    __shared__ __attribute__((aligned(16))) bf16_t XT[kSmallN * kLdt];  // n x m
    __shared__ __attribute__((aligned(16))) bf16_t A[kSmallM * kLdt];
    __shared__ __attribute__((aligned(16))) bf16_t B[kSmallM * kLdt];
    __shared__ double red[kST / 64];
    const int mat = static_cast<int>(blockIdx.x), tid = static_cast<int>(threadIdx.x);
    // (the wave index read as uniform, so that branches on it stay scalar)
    const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int si = 0;
#pragma unroll
    for (int q = 1; q < kMaxSeg; ++q)
        if (q < s.nseg && mat >= s.seg[q].first) si = q;
    const SmallSeg& sg = s.seg[si];
    const int rows = sg.rows, cols = sg.cols, m = sg.m, n = sg.n, np = sg.np;
    const bool tall = sg.tall != 0;

    // padding rows and columns are zero and stay zero through the iteration
    for (int i = tid; i < kSmallM * kLdx / 8; i += kST) reinterpret_cast<u32x4s*>(X)[i] = u32x4s{0, 0, 0, 0};
    for (int i = tid; i < kSmallN * kLdt / 8; i += kST) reinterpret_cast<u32x4s*>(XT)[i] = u32x4s{0, 0, 0, 0};
    __syncthreads();

    // momentum (fused step), bf16(u) staged in X in the iteration's
    // orientation, float64 sum of squares of u; each thread issues the loads
    // of 8 elements before it uses any, so their latencies overlap
    const int numel = rows * cols;
    const float* g = G.p[mat];
    float* buf = MOM ? BUF.p[mat] : nullptr;
    double ss = 0.0;
    constexpr int kU = 8;
    // 16-byte accesses where every row holds whole runs of 4 and the
    // pointers are aligned (float32 only)
    const bool vec = !IO16 && (cols & 3) == 0 && (reinterpret_cast<uintptr_t>(g) & 15u) == 0 &&
                     (!MOM || (reinterpret_cast<uintptr_t>(buf) & 15u) == 0);
    if (vec) {
        const int n4 = numel / 4;
        RowCol rc(4 * tid, 4 * kST, cols);
        for (int v0 = tid; v0 < n4; v0 += kU * kST) {
            f32x4 gv[kU], bv[kU];
#pragma unroll
            for (int q = 0; q < kU; ++q) {
                const int i4 = v0 + q * kST;
                if (i4 < n4) {
                    gv[q] = reinterpret_cast<const f32x4*>(g)[i4];
                    if constexpr (MOM) bv[q] = reinterpret_cast<const f32x4*>(buf)[i4];
                }
            }
#pragma unroll
            for (int q = 0; q < kU; ++q) {
                const int i4 = v0 + q * kST;
                if (i4 < n4) {
                    f32x4 bn;
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float u = gv[q][t];
                        if constexpr (MOM) {
                            bn[t] = fmaf(s.mu, bv[q][t], gv[q][t]);
                            u = fmaf(s.mu, bn[t], gv[q][t]);
                        }
                        ss += static_cast<double>(u) * static_cast<double>(u);
                        X[(tall ? rc.c + t : rc.r) * kLdx + (tall ? rc.r : rc.c + t)] = f32_to_bf16(u);
                    }
                    if constexpr (MOM) reinterpret_cast<f32x4*>(buf)[i4] = bn;
                }
                rc.next();
            }
        }
    }
    RowCol rc(tid, kST, cols);
    for (int e0 = vec ? numel : tid; e0 < numel; e0 += kU * kST) {
        float gv[kU], bv[kU];
#pragma unroll
        for (int q = 0; q < kU; ++q) {
            const int e = e0 + q * kST;
            gv[q] = 0.0f;
            bv[q] = 0.0f;
            if (e < numel) {
                if constexpr (IO16) {
                    gv[q] = bf16_to_f32(reinterpret_cast<const bf16_t*>(g)[e]);
                } else {
                    gv[q] = g[e];
                    if constexpr (MOM) bv[q] = buf[e];
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kU; ++q) {
            const int e = e0 + q * kST;
            if (e < numel) {
                float u = gv[q];
                if constexpr (MOM) {
                    const float b = fmaf(s.mu, bv[q], gv[q]);
                    buf[e] = b;
                    u = fmaf(s.mu, b, gv[q]);
                }
                ss += static_cast<double>(u) * static_cast<double>(u);
                X[(tall ? rc.c : rc.r) * kLdx + (tall ? rc.r : rc.c)] = f32_to_bf16(u);
            }
            rc.next();
        }
    }
    ss = wave_sum_small(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int w = 0; w < kST / 64; ++w) total += red[w];
    const double d = sqrt(total) + static_cast<double>(s.eps);
    const float r32 = static_cast<float>(1.0 / d);
    const bool fast_ok = r32 >= 0x1p-126f && r32 <= 0x1.fffffep127f;
    // X0 = bf16(bf16(u) / d), the quotient in float64 and rounded once;
    // four elements per pass, so that their divisions overlap
    {
        RowCol ij(tid, kST, n);
        for (int e0 = tid; e0 < m * n; e0 += 4 * kST) {
            int ii[4], jj[4];
            double q[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                ii[t] = ij.r;
                jj[t] = ij.c;
                ij.next();
                q[t] = e0 + t * kST < m * n ? static_cast<double>(bf16_to_f32(X[ii[t] * kLdx + jj[t]])) : 0.0;
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (e0 + t * kST < m * n) {
                    // q = v fl32(1/d) rounds like v / d unless it lies near a
                    // bf16 rounding midpoint (the cast kernel's criterion)
                    const float q32 = static_cast<float>(q[t]) * r32;
                    const bf16_t x0 = fast_ok && !cast_needs_f64(q32) ? f32_to_bf16(q32) : f64_to_bf16(q[t] / d);
                    X[ii[t] * kLdx + jj[t]] = x0;
                    XT[jj[t] * kLdt + ii[t]] = x0;
                }
            }
        }
    }
    __syncthreads();

    const int nbj = np / 32, nblk = 2 * nbj;  // 32 x 32 blocks of X (at most 16)
    for (int step = 0; step < s.steps; ++step) {
        sym_product<false>(X, kLdx, np, nullptr, 0.0f, 1.0f, A, wave, lane);  // A = X X^T
        __syncthreads();
        sym_product<true>(A, kLdt, kSmallM, A, s.b, s.c, B, wave, lane);  // B = c A A + b A
        __syncthreads();
        // X' = B X + a X: block q of X' on wave q mod 4, K = 64 (B's rows and
        // columns past m are zero)
        f32x16 acc[16 / (kST / 64)];
#pragma unroll
        for (int t = 0; t < 16 / (kST / 64); ++t) {
            const int q = wave + (kST / 64) * t;
            if (q < nblk) {
                const int bi = q / nbj, bj = q - bi * nbj;
                const bf16_t* pa = B + (32 * bi + (lane & 31)) * kLdt + 8 * (lane >> 5);
                const bf16_t* pb = XT + (32 * bj + (lane & 31)) * kLdt + 8 * (lane >> 5);
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[t][r] = 0.0f;
#pragma unroll
                for (int k0 = 0; k0 < kSmallM; k0 += 16)
                    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ld8(pa + k0), ld8(pb + k0), acc[t], 0, 0, 0);
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi = 32 * bi + acc_row(r, lane), gj = 32 * bj + (lane & 31);
                    acc[t][r] = fmaf(s.a, bf16_to_f32(X[gi * kLdx + gj]), acc[t][r]);
                }
            }
        }
        __syncthreads();  // every wave is done reading X, X^T and B
#pragma unroll
        for (int t = 0; t < 16 / (kST / 64); ++t) {
            const int q = wave + (kST / 64) * t;
            if (q < nblk) {
                const int bi = q / nbj, bj = q - bi * nbj;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int gi = 32 * bi + acc_row(r, lane), gj = 32 * bj + (lane & 31);
                    const bf16_t h = f32_to_bf16(acc[t][r]);
                    X[gi * kLdx + gj] = h;
                    XT[gj * kLdt + gi] = h;
                }
            }
        }
        __syncthreads();
    }

    // the result in G's orientation (rows x cols): X, or X^T when G is tall
    float* o = OUT.p[mat];
    const bool ovec = !IO16 && (cols & 3) == 0 && (reinterpret_cast<uintptr_t>(o) & 15u) == 0;
    if (ovec) {
        RowCol oc4(4 * tid, 4 * kST, cols);
        for (int v0 = tid; v0 < numel / 4; v0 += kST, oc4.next()) {
            f32x4 w;
#pragma unroll
            for (int t = 0; t < 4; ++t)
                w[t] = bf16_to_f32(tall ? XT[(oc4.r) * kLdt + oc4.c + t] : X[oc4.r * kLdx + oc4.c + t]);
            f32x4* dst = reinterpret_cast<f32x4*>(o) + v0;
            if (s.apply) {
                const f32x4 p = *dst;
#pragma unroll
                for (int t = 0; t < 4; ++t) w[t] = fmaf(-s.lr, w[t], p[t]);
            }
            *dst = w;
        }
    }
    RowCol oc(tid, kST, cols);
    for (int e = ovec ? numel : tid; e < numel; e += kST, oc.next()) {
        const int r = oc.r, c = oc.c;
        const bf16_t h = tall ? XT[r * kLdt + c] : X[r * kLdx + c];
        if constexpr (IO16) {
            reinterpret_cast<bf16_t*>(o)[e] = h;
        } else {
            const float v = bf16_to_f32(h);
            o[e] = s.apply ? fmaf(-s.lr, v, o[e]) : v;
        }
    }
}

}  // namespace

hipError_t launch_ns5_small(const SmallArgs& s, const ConstPtrTable& G, const PtrTable& out, const PtrTable* buf,
                            bool io16, hipStream_t stream) {
    if (s.nseg < 1 || s.nseg > kMaxSeg || (io16 && (buf || s.apply))) return hipErrorInvalidValue;
    int total = 0;
    for (int q = 0; q < s.nseg; ++q) {
        const SmallSeg& sg = s.seg[q];
        if (sg.first != total || sg.cnt < 1 || sg.m < 1 || sg.m > kSmallM || sg.n < sg.m || sg.n > kSmallN ||
            sg.np % 32 != 0 || sg.np < sg.n || sg.np > kSmallN)
            return hipErrorInvalidValue;
        total += sg.cnt;
    }
    if (total > kMaxGroup) return hipErrorInvalidValue;
    const dim3 grid(static_cast<unsigned>(total));
    if (buf)
        k_ns5_small<true, false><<<grid, kST, 0, stream>>>(s, G, out, *buf);
    else if (io16)
        k_ns5_small<false, true><<<grid, kST, 0, stream>>>(s, G, out, PtrTable{});
    else
        k_ns5_small<false, false><<<grid, kST, 0, stream>>>(s, G, out, PtrTable{});
    return hipGetLastError();
}

}  // namespace muon
