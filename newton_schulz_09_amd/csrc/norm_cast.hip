// Frobenius norm and bf16 cast of the NS5 input (the printed
// zeroth_power_via_newtonschulz5 of the Muon section, Synced report on
// Modded-NanoGPT: X = G.bfloat16() / (G.norm() + eps), transposed when G has
// more rows than columns).
//
// Two passes, both HBM-bound (in the fused Muon step the first is
// k_momentum_norm, which also applies the momentum and stages bf16(u)):
//   k_sumsq      reads G once (4 B/elem) and writes one float64 partial sum
//                of squares per workgroup: per-lane float64 accumulation,
//                wavefront butterfly shuffles, then LDS across the 4 waves.
//                The split of G into workgroups is fixed, so the result is
//                deterministic (no atomics).
//   k_scale_cast reduces a matrix's partials in a fixed order (every
//                workgroup gets the same float64 norm), then reads G again
//                (or its bf16 staging copy) and writes
//                X0 = bf16( bf16(G) / (||G|| + eps) ) in the iteration's
//                orientation: directly, or transposed through an LDS tile
//                when G is tall.  The quotient is formed in float64 and
//                rounded once to bf16.  Padding to the GEMM tile is written
//                as zeros.
#include "internal.hpp"

namespace muon {

namespace {

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

__global__ __launch_bounds__(kThreads) void k_sumsq(ConstPtrTable G, int64_t numel, int nb,
                                                    int64_t chunk, double* partials) {
    const int mat = blockIdx.y;
    const float* g = G.p[mat];
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t end = begin + chunk < numel ? begin + chunk : numel;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    int64_t i = begin + threadIdx.x;
    for (; i + 3 * kThreads < end; i += 4 * kThreads) {
        const float x0 = g[i], x1 = g[i + kThreads], x2 = g[i + 2 * kThreads], x3 = g[i + 3 * kThreads];
        s0 = fma(static_cast<double>(x0), static_cast<double>(x0), s0);
        s1 = fma(static_cast<double>(x1), static_cast<double>(x1), s1);
        s2 = fma(static_cast<double>(x2), static_cast<double>(x2), s2);
        s3 = fma(static_cast<double>(x3), static_cast<double>(x3), s3);
    }
    for (; i < end; i += kThreads) {
        const float x = g[i];
        s0 = fma(static_cast<double>(x), static_cast<double>(x), s0);
    }
    double s = wave_sum((s0 + s1) + (s2 + s3));
    __shared__ double red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        partials[static_cast<int64_t>(mat) * nb + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

// Nesterov momentum fused with the first pass of the norm: one workgroup per
// contiguous chunk of one matrix reads g and buf, writes the new buf, writes
// u rounded to bf16 (the bf16(G) of the cast) into a dense staging copy, and
// leaves one float64 partial sum of squares of the float32 u.  u itself is
// never stored in float32.  VEC: 16-byte accesses (pointers 16-byte aligned,
// numel and chunk multiples of 4).
template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_momentum_norm(ConstPtrTable G, PtrTable BUF, int64_t numel, int nb,
                                                            int64_t chunk, float mu, bf16_t* ub, int64_t ub_mat,
                                                            double* partials) {
    const int mat = blockIdx.y;
    const float* g = G.p[mat];
    float* buf = BUF.p[mat];
    bf16_t* u16 = ub + static_cast<int64_t>(mat) * ub_mat;
    const int64_t begin = static_cast<int64_t>(blockIdx.x) * chunk;
    const int64_t end = begin + chunk < numel ? begin + chunk : numel;
    double s0 = 0.0, s1 = 0.0;
    if constexpr (VEC) {
        for (int64_t i = begin + 4 * static_cast<int64_t>(threadIdx.x); i < end; i += 4 * kThreads) {
            const f32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + i));
            f32x4 bv = *reinterpret_cast<const f32x4*>(buf + i);
            float u[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                bv[q] = fmaf(mu, bv[q], gv[q]);
                u[q] = fmaf(mu, bv[q], gv[q]);
            }
            *reinterpret_cast<f32x4*>(buf + i) = bv;
            typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2v*>(u16 + i) = u32x2v{f32x2_to_bf16x2(u[0], u[1]), f32x2_to_bf16x2(u[2], u[3])};
            s0 = fma(static_cast<double>(u[0]), static_cast<double>(u[0]), s0);
            s1 = fma(static_cast<double>(u[1]), static_cast<double>(u[1]), s1);
            s0 = fma(static_cast<double>(u[2]), static_cast<double>(u[2]), s0);
            s1 = fma(static_cast<double>(u[3]), static_cast<double>(u[3]), s1);
        }
    } else {
        for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
            const float b = fmaf(mu, buf[i], g[i]);
            const float u = fmaf(mu, b, g[i]);
            buf[i] = b;
            u16[i] = f32_to_bf16(u);
            s0 = fma(static_cast<double>(u), static_cast<double>(u), s0);
        }
    }
    double s = wave_sum(s0 + s1);
    __shared__ double red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        partials[static_cast<int64_t>(mat) * nb + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
    }
}

constexpr int kCastTile = 64;

// BF16IN: the input is the dense bf16 staging copy written by
// k_momentum_norm (already bf16(G)); otherwise the float32 G of the table.
// One workgroup per 64x64 tile of G: each thread handles runs of 8
// consecutive columns (16-byte accesses where the shape allows), and a tall
// G's tile is transposed through LDS so that X rows are also written 16
// bytes at a time.
template <bool BF16IN>
__global__ __launch_bounds__(kThreads) void k_scale_cast(ConstPtrTable G, const bf16_t* ub, int64_t ub_mat, int rows,
                                                         int cols, int tiles_c, const double* partials, int nb,
                                                         float eps, bf16_t* X, int ldx, int64_t x_mat, int tall) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const int mat = blockIdx.y;
    const int tr_i = blockIdx.x / tiles_c, tc_i = blockIdx.x % tiles_c;
    const int r0 = tr_i * kCastTile, c0 = tc_i * kCastTile;
    const float* g = BF16IN ? nullptr : G.p[mat];
    const bf16_t* u16 = BF16IN ? ub + static_cast<int64_t>(mat) * ub_mat : nullptr;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

    __shared__ double s_norm;
    __shared__ __attribute__((aligned(16))) bf16_t tile_t[kCastTile][kCastTile + 8];  // [col][row]

    if (wave == 0) {
        const double* part = partials + static_cast<int64_t>(mat) * nb;
        double s = 0.0;
        for (int k = lane; k < nb; k += 64) s += part[k];
        s = wave_sum(s);
        if (lane == 0) s_norm = sqrt(s) + static_cast<double>(eps);
    }
    __syncthreads();
    const double d = s_norm;
    bf16_t* Xm = X + static_cast<int64_t>(mat) * x_mat;
    // 16-byte loads need every row start aligned: cols a multiple of 8 (bf16)
    // or 4 (float32), and the base aligned
    const bool vec = BF16IN ? ((cols & 7) == 0 && (reinterpret_cast<uintptr_t>(u16) & 15u) == 0)
                            : ((cols & 3) == 0 && (reinterpret_cast<uintptr_t>(g) & 15u) == 0);

#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = threadIdx.x + h * kThreads;  // 0 .. 511
        const int r = idx >> 3, cg = (idx & 7) * 8;  // tile row, first of 8 columns
        const int gr = r0 + r, gc = c0 + cg;
        float v[8];
        if (gr < rows && vec && gc + 8 <= cols) {
            if constexpr (BF16IN) {
                const u32x4v w = *reinterpret_cast<const u32x4v*>(u16 + static_cast<int64_t>(gr) * cols + gc);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[2 * e] = bf16_to_f32(static_cast<bf16_t>(w[e] & 0xffffu));
                    v[2 * e + 1] = bf16_to_f32(static_cast<bf16_t>(w[e] >> 16));
                }
            } else {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(g + static_cast<int64_t>(gr) * cols + gc);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(g + static_cast<int64_t>(gr) * cols + gc + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[e] = bf16_to_f32(f32_to_bf16(lo[e]));
                    v[4 + e] = bf16_to_f32(f32_to_bf16(hi[e]));
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[e] = 0.0f;
                if (gr < rows && gc + e < cols) {
                    if constexpr (BF16IN)
                        v[e] = bf16_to_f32(u16[static_cast<int64_t>(gr) * cols + gc + e]);
                    else
                        v[e] = bf16_to_f32(f32_to_bf16(g[static_cast<int64_t>(gr) * cols + gc + e]));
                }
            }
        }
        // X0 = bf16(bf16(G) / d): the quotient in float64, one rounding;
        // padding stays zero (0 / d = 0)
        bf16_t hx[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) hx[e] = f64_to_bf16(static_cast<double>(v[e]) / d);
        if (!tall) {
            u32x4v w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                w[e] = static_cast<uint32_t>(hx[2 * e]) | (static_cast<uint32_t>(hx[2 * e + 1]) << 16);
            *reinterpret_cast<u32x4v*>(Xm + static_cast<int64_t>(gr) * ldx + gc) = w;
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) tile_t[cg + e][r] = hx[e];
        }
    }
    if (!tall) return;  // uniform across the workgroup
    __syncthreads();
    // X = G^T: X row c0 + c holds G column c0 + c; 8 consecutive G rows per thread
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = threadIdx.x + h * kThreads;
        const int c = idx >> 3, rg = (idx & 7) * 8;
        const u32x4v w = *reinterpret_cast<const u32x4v*>(&tile_t[c][rg]);
        *reinterpret_cast<u32x4v*>(Xm + static_cast<int64_t>(c0 + c) * ldx + r0 + rg) = w;
    }
}

__global__ __launch_bounds__(kThreads) void k_copy_out(PtrTable out, int rows, int cols, int tall, int ldx,
                                                       const bf16_t* X, int64_t x_mat) {
    const int mat = blockIdx.y;
    const int64_t total = static_cast<int64_t>(rows) * cols;
    const bf16_t* src = X + static_cast<int64_t>(mat) * x_mat;
    float* dst = out.p[mat];
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t r = i / cols, c = i - r * cols;  // position in G's orientation
        dst[i] = bf16_to_f32(tall ? src[c * ldx + r] : src[r * ldx + c]);
    }
}

}  // namespace

hipError_t launch_sumsq(const ConstPtrTable& G, int cnt, int64_t numel, int nb, double* partials,
                        hipStream_t stream) {
    const int64_t chunk = (numel + nb - 1) / nb;
    k_sumsq<<<dim3(nb, cnt), kThreads, 0, stream>>>(G, numel, nb, chunk, partials);
    return hipGetLastError();
}

hipError_t launch_scale_cast(const ConstPtrTable& G, const bf16_t* ub, int64_t ub_mat, int cnt, const Ns5Plan& plan,
                             const double* partials, float eps, bf16_t* X, hipStream_t stream) {
    // X is G's orientation unless G is tall (then it is G^T), written over its
    // padded extent (padding as zeros)
    const int rows_pad = plan.tall ? plan.np : plan.mp;
    const int cols_pad = plan.tall ? plan.mp : plan.np;
    const int tiles_r = rows_pad / kCastTile, tiles_c = cols_pad / kCastTile;
    const dim3 grid(tiles_r * tiles_c, cnt);
    if (ub)
        k_scale_cast<true><<<grid, kThreads, 0, stream>>>(G, ub, ub_mat, static_cast<int>(plan.rows),
                                                          static_cast<int>(plan.cols), tiles_c, partials, plan.nb,
                                                          eps, X, plan.ldx, static_cast<int64_t>(plan.x_elems),
                                                          plan.tall ? 1 : 0);
    else
        k_scale_cast<false><<<grid, kThreads, 0, stream>>>(G, nullptr, 0, static_cast<int>(plan.rows),
                                                           static_cast<int>(plan.cols), tiles_c, partials, plan.nb,
                                                           eps, X, plan.ldx, static_cast<int64_t>(plan.x_elems),
                                                           plan.tall ? 1 : 0);
    return hipGetLastError();
}

hipError_t launch_momentum_norm(const ConstPtrTable& G, const PtrTable& BUF, int cnt, int64_t numel, int nb,
                                float mu, bf16_t* ub, int64_t ub_mat, double* partials, hipStream_t stream) {
    bool vec = (numel % 4) == 0;
    for (int i = 0; i < cnt && vec; ++i)
        vec = ((reinterpret_cast<uintptr_t>(G.p[i]) | reinterpret_cast<uintptr_t>(BUF.p[i])) & 15u) == 0;
    int64_t chunk = (numel + nb - 1) / nb;
    if (vec) chunk = (chunk + 3) / 4 * 4;
    if (vec)
        k_momentum_norm<true><<<dim3(nb, cnt), kThreads, 0, stream>>>(G, BUF, numel, nb, chunk, mu, ub, ub_mat,
                                                                       partials);
    else
        k_momentum_norm<false><<<dim3(nb, cnt), kThreads, 0, stream>>>(G, BUF, numel, nb, chunk, mu, ub, ub_mat,
                                                                        partials);
    return hipGetLastError();
}

hipError_t launch_copy_out(const Ns5Plan& plan, int cnt, const bf16_t* X, const PtrTable& out, hipStream_t stream) {
    const int64_t total = plan.rows * plan.cols;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 2048) blocks = 2048;
    k_copy_out<<<dim3(static_cast<unsigned>(blocks), cnt), kThreads, 0, stream>>>(
        out, static_cast<int>(plan.rows), static_cast<int>(plan.cols), plan.tall ? 1 : 0, plan.ldx, X,
        static_cast<int64_t>(plan.x_elems));
    return hipGetLastError();
}

}  // namespace muon
