// Frobenius norm and bf16 cast of the NS5 input (the printed
// zeroth_power_via_newtonschulz5 of the Muon section, Synced report on
// Modded-NanoGPT: X = G.bfloat16() / (G.norm() + eps), transposed when G has
// more rows than columns), and the Nesterov momentum that precedes it in the
// Muon step.
//
// Two passes, both HBM-bound, each one launch over every chunk of a launch
// group (segment tables in the kernel arguments, like the GEMMs):
//   k_norm       reads G once (4 B/elem) and writes one float64 partial sum
//                of squares per workgroup: per-lane float64 accumulation,
//                wavefront butterfly shuffles, then LDS across the 4 waves.
//                The split of G into workgroups is fixed, so the result is
//                deterministic (no atomics).  In the fused Muon step it also
//                applies the momentum and stages bf16(u) (14 B/elem).
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

// Workgroup b of a batched launch -> its segment (the last one whose first
// workgroup is at or before b).
template <typename Launch>
__device__ __forceinline__ int segment_of(const Launch& L, int b) {
    int si = 0;
#pragma unroll
    for (int q = 1; q < kMaxSeg; ++q)
        if (q < L.nseg && b >= L.seg[q].first_block) si = q;
    return si;
}

// MOM = false: sum of squares of G.  MOM = true: Nesterov momentum fused with
// the first pass of the norm: buf <- mu buf + g, u = g + mu buf; buf is
// written back, u rounded to bf16 (the bf16(G) of the cast) goes to a dense
// staging copy, and only u's float64 sum of squares is kept (u itself is
// never stored in float32).  One workgroup per contiguous chunk of one
// matrix, one float64 partial per workgroup: the split is fixed, so the norm
// is deterministic (no atomics).
// IN16: G holds bfloat16 values (the bf16-input NS5; no momentum), read 8
// at a time where aligned.
template <bool MOM, bool IN16 = false>
__global__ __launch_bounds__(kThreads) void k_norm(NormLaunch L, ConstPtrTable G, PtrTable BUF, float mu) {
    static_assert(!(MOM && IN16), "the momentum pass reads float32 gradients");
    const NormSeg& sg = L.seg[segment_of(L, static_cast<int>(blockIdx.x))];
    const int local = static_cast<int>(blockIdx.x) - sg.first_block;
    const int mat = local / sg.nb, part = local - mat * sg.nb;
    const float* g = G.p[sg.ptr_base + mat];
    if constexpr (IN16) {
        const bf16_t* h = reinterpret_cast<const bf16_t*>(g);
        const int64_t begin = static_cast<int64_t>(part) * sg.chunk;
        const int64_t end = begin + sg.chunk < sg.numel ? begin + sg.chunk : sg.numel;
        double s0 = 0.0, s1 = 0.0;
        if (sg.vec) {  // 16-byte aligned, numel and chunk multiples of 8
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            for (int64_t i = begin + 8 * static_cast<int64_t>(threadIdx.x); i < end; i += 8 * kThreads) {
                const u32x4v w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(h + i));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const double lo = bf16_to_f32(static_cast<bf16_t>(w[q] & 0xffffu));
                    const double hi = bf16_to_f32(static_cast<bf16_t>(w[q] >> 16));
                    s0 = fma(lo, lo, s0);
                    s1 = fma(hi, hi, s1);
                }
            }
        } else {
            for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
                const double v = bf16_to_f32(h[i]);
                s0 = fma(v, v, s0);
            }
        }
        double s = wave_sum(s0 + s1);
        __shared__ double red16[kThreads / 64];
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        if (lane == 0) red16[wave] = s;
        __syncthreads();
        if (threadIdx.x == 0)
            sg.partials[static_cast<int64_t>(mat) * sg.nb + part] = (red16[0] + red16[1]) + (red16[2] + red16[3]);
        return;
    }
    float* buf = MOM ? BUF.p[sg.ptr_base + mat] : nullptr;
    bf16_t* u16 = MOM ? sg.ub + static_cast<int64_t>(mat) * sg.ub_mat : nullptr;
    const int64_t begin = static_cast<int64_t>(part) * sg.chunk;
    const int64_t end = begin + sg.chunk < sg.numel ? begin + sg.chunk : sg.numel;
    double s0 = 0.0, s1 = 0.0;
    if (sg.vec) {
        // four consecutive elements at i: momentum, staging, sum of squares
        auto step4 = [&](int64_t i, const f32x4& gv, f32x4 bv) {
            float u[4];
            if constexpr (MOM) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    bv[q] = fmaf(mu, bv[q], gv[q]);
                    u[q] = fmaf(mu, bv[q], gv[q]);
                }
                __builtin_nontemporal_store(bv, reinterpret_cast<f32x4*>(buf + i));
                typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                *reinterpret_cast<u32x2v*>(u16 + i) =
                    u32x2v{f32x2_to_bf16x2(u[0], u[1]), f32x2_to_bf16x2(u[2], u[3])};
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) u[q] = gv[q];
            }
            s0 = fma(static_cast<double>(u[0]), static_cast<double>(u[0]), s0);
            s1 = fma(static_cast<double>(u[1]), static_cast<double>(u[1]), s1);
            s0 = fma(static_cast<double>(u[2]), static_cast<double>(u[2]), s0);
            s1 = fma(static_cast<double>(u[3]), static_cast<double>(u[3]), s1);
        };
        // two groups per iteration (all their loads in flight together), in
        // the same per-thread order as one group at a time
        for (int64_t i = begin + 4 * static_cast<int64_t>(threadIdx.x); i < end; i += 8 * kThreads) {
            const int64_t i2 = i + 4 * kThreads;
            const bool two = i2 < end;
            // g and buf are touched once per step: they stream past the caches
            // (non-temporal), which then keep the staging copy written here
            // and the X the cast writes from it for the first X X^T
            const f32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + i));
            f32x4 bv{}, gv2{}, bv2{};
            if constexpr (MOM) bv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(buf + i));
            if (two) {
                gv2 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + i2));
                if constexpr (MOM) bv2 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(buf + i2));
            }
            step4(i, gv, bv);
            if (two) step4(i2, gv2, bv2);
        }
    } else {
        for (int64_t i = begin + threadIdx.x; i < end; i += kThreads) {
            float u = g[i];
            if constexpr (MOM) {
                const float b = fmaf(mu, buf[i], u);
                u = fmaf(mu, b, u);
                buf[i] = b;
                u16[i] = f32_to_bf16(u);
            }
            s0 = fma(static_cast<double>(u), static_cast<double>(u), s0);
        }
    }
    double s = wave_sum(s0 + s1);
    __shared__ double red[kThreads / 64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) sg.partials[static_cast<int64_t>(mat) * sg.nb + part] = (red[0] + red[1]) + (red[2] + red[3]);
}

constexpr int kCastTile = 64;


// One 64 x 64 tile of the cast: this thread's two runs of 8 consecutive
// columns (rows idx / 8 for idx = tid and tid + 256), as bf16(G) in float.
template <bool BF16IN>
__device__ __forceinline__ void cast_load(const float* g, const bf16_t* u16, int rows, int cols, bool vec, int r0,
                                          int c0, float (&v)[2][8]) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int idx = threadIdx.x + h * kThreads;
        const int gr = r0 + (idx >> 3), gc = c0 + (idx & 7) * 8;
        if (gr < rows && vec && gc + 8 <= cols) {
            if constexpr (BF16IN) {  // read once: streamed
                const u32x4v w = __builtin_nontemporal_load(reinterpret_cast<const u32x4v*>(u16 + static_cast<int64_t>(gr) * cols + gc));
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[h][2 * e] = bf16_to_f32(static_cast<bf16_t>(w[e] & 0xffffu));
                    v[h][2 * e + 1] = bf16_to_f32(static_cast<bf16_t>(w[e] >> 16));
                }
            } else {
                const f32x4 lo = *reinterpret_cast<const f32x4*>(g + static_cast<int64_t>(gr) * cols + gc);
                const f32x4 hi = *reinterpret_cast<const f32x4*>(g + static_cast<int64_t>(gr) * cols + gc + 4);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    v[h][e] = bf16_to_f32(f32_to_bf16(lo[e]));
                    v[h][4 + e] = bf16_to_f32(f32_to_bf16(hi[e]));
                }
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                v[h][e] = 0.0f;
                if (gr < rows && gc + e < cols) {
                    if constexpr (BF16IN)
                        v[h][e] = bf16_to_f32(u16[static_cast<int64_t>(gr) * cols + gc + e]);
                    else
                        v[h][e] = bf16_to_f32(f32_to_bf16(g[static_cast<int64_t>(gr) * cols + gc + e]));
                }
            }
        }
    }
}

// BF16IN: the input is the dense bf16 staging copy written by the momentum
// pass (already bf16(G)); otherwise the float32 G of the table.  Each
// workgroup casts per_wg consecutive 64 x 64 tiles of one matrix of G's
// padded extent: it reduces the norm from the partials once (every
// workgroup of a matrix sums them in the same order, so all get the same
// float64 norm), then loads each next tile while converting the current one.
// Each thread handles runs of 8 consecutive columns (16-byte accesses where
// the shape allows); a tall G's tile is transposed through LDS so that X rows
// are also written 16 bytes at a time.
template <bool BF16IN>
__global__ __launch_bounds__(kThreads) void k_scale_cast(CastLaunch L, ConstPtrTable G, float eps) {
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    const CastSeg& sg = L.seg[segment_of(L, static_cast<int>(blockIdx.x))];
    const int local = static_cast<int>(blockIdx.x) - sg.first_block;
    const int mat = local / sg.wg_per_mat;
    const int t_begin = (local - mat * sg.wg_per_mat) * sg.per_wg;
    const int t_end = t_begin + sg.per_wg < sg.tiles_per_mat ? t_begin + sg.per_wg : sg.tiles_per_mat;
    const float* g = BF16IN ? nullptr : G.p[sg.ptr_base + mat];
    // bf16 input: the staging copy, or (bf16-input NS5) G itself
    const bf16_t* u16 = !BF16IN ? nullptr
                        : sg.ub ? sg.ub + static_cast<int64_t>(mat) * sg.ub_mat
                                : reinterpret_cast<const bf16_t*>(G.p[sg.ptr_base + mat]);
    const int rows = sg.rows, cols = sg.cols;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // 16-byte loads need every row start aligned: cols a multiple of 8 (bf16)
    // or 4 (float32), and the base aligned
    const bool vec = BF16IN ? ((cols & 7) == 0 && (reinterpret_cast<uintptr_t>(u16) & 15u) == 0)
                            : ((cols & 3) == 0 && (reinterpret_cast<uintptr_t>(g) & 15u) == 0);
    bf16_t* Xm = sg.X + static_cast<int64_t>(mat) * sg.x_mat;

    __shared__ double s_norm;
    __shared__ __attribute__((aligned(16))) bf16_t tile_t[kCastTile][kCastTile + 8];  // [col][row]

    // the first tile's loads go out before the norm reduction, which they do
    // not depend on
    float v[2][8], vn[2][8];
    cast_load<BF16IN>(g, u16, rows, cols, vec, (t_begin / sg.tiles_c) * kCastTile,
                      (t_begin % sg.tiles_c) * kCastTile, v);
    if (wave == 0) {
        const double* part = sg.partials + static_cast<int64_t>(mat) * sg.nb;
        double s = 0.0;
        for (int k = lane; k < sg.nb; k += 64) s += part[k];
        s = wave_sum(s);
        if (lane == 0) s_norm = sqrt(s) + static_cast<double>(eps);
    }
    __syncthreads();
    const double d = s_norm;
    // X0 = bf16(fl64(v / d)) for each bf16 value v.  Fast path: q = v *
    // fl32(1/d) in float32 is within ~2 float32 ulps of v / d, so its
    // hardware round to bf16 is the same unless q lies within a few ulps of a
    // bf16 rounding midpoint (low 16 bits near 0x8000); those elements, and
    // any q that is not a normal float32, take the float64 quotient instead.
    const float r32 = static_cast<float>(1.0 / d);
    const bool fast_ok = r32 >= 0x1p-126f && r32 <= 0x1.fffffep127f;

    for (int t = t_begin; t < t_end; ++t) {
        const int r0 = (t / sg.tiles_c) * kCastTile, c0 = (t % sg.tiles_c) * kCastTile;
        if (t + 1 < t_end)
            cast_load<BF16IN>(g, u16, rows, cols, vec, ((t + 1) / sg.tiles_c) * kCastTile,
                              ((t + 1) % sg.tiles_c) * kCastTile, vn);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int idx = threadIdx.x + h * kThreads;
            const int r = idx >> 3, cg = (idx & 7) * 8;
            // X0 = bf16(bf16(G) / d) (padding stays zero: 0 / d = 0)
            u32x4v w;
            uint32_t slow = fast_ok ? 0u : 0xffu;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float q0 = v[h][2 * e] * r32, q1 = v[h][2 * e + 1] * r32;
                w[e] = f32x2_to_bf16x2(q0, q1);
                slow |= (cast_needs_f64(q0) ? 1u : 0u) << (2 * e);
                slow |= (cast_needs_f64(q1) ? 1u : 0u) << (2 * e + 1);
            }
            if (slow) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    if (slow & (1u << e)) {
                        const uint32_t hx = f64_to_bf16(static_cast<double>(v[h][e]) / d);
                        const int sh = 16 * (e & 1);
                        w[e >> 1] = (w[e >> 1] & ~(0xffffu << sh)) | (hx << sh);
                    }
                }
            }
            if (!sg.tall) {
                *reinterpret_cast<u32x4v*>(Xm + static_cast<int64_t>(r0 + r) * sg.ldx + c0 + cg) = w;
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) tile_t[cg + e][r] = static_cast<bf16_t>((w[e >> 1] >> (16 * (e & 1))) & 0xffffu);
            }
        }
        if (sg.tall) {  // uniform across the workgroup
            __syncthreads();
            // X = G^T: X row c0 + c holds G column c0 + c; 8 consecutive G rows per thread
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int idx = threadIdx.x + h * kThreads;
                const int c = idx >> 3, rg = (idx & 7) * 8;
                const u32x4v w = *reinterpret_cast<const u32x4v*>(&tile_t[c][rg]);
                *reinterpret_cast<u32x4v*>(Xm + static_cast<int64_t>(c0 + c) * sg.ldx + r0 + rg) = w;
            }
            __syncthreads();  // tile_t is refilled by the next tile
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[h][e] = vn[h][e];
    }
}

// Zeroes n elements from `offset` of matrix blockIdx.y (x_mat apart).
__global__ __launch_bounds__(kThreads) void k_zero_rows(bf16_t* X, int64_t x_mat, int64_t offset, int64_t n) {
    bf16_t* p = X + static_cast<int64_t>(blockIdx.y) * x_mat + offset;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
        p[i] = 0;
}

// out[i] = float32 of X in G's orientation (the steps = 0 result), with
// `apply` the parameter update out[i] <- out[i] - lr * X instead, or with
// `out16` X itself as bfloat16.
__global__ __launch_bounds__(kThreads) void k_copy_out(PtrTable out, int rows, int cols, int tall, int ldx,
                                                       const bf16_t* X, int64_t x_mat, int apply, float lr,
                                                       int out16) {
    const int mat = blockIdx.y;
    const int64_t total = static_cast<int64_t>(rows) * cols;
    const bf16_t* src = X + static_cast<int64_t>(mat) * x_mat;
    float* dst = out.p[mat];
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < total;
         i += static_cast<int64_t>(gridDim.x) * kThreads) {
        const int64_t r = i / cols, c = i - r * cols;  // position in G's orientation
        const bf16_t x = tall ? src[c * ldx + r] : src[r * ldx + c];
        if (out16) {
            reinterpret_cast<bf16_t*>(dst)[i] = x;
        } else {
            const float o = bf16_to_f32(x);
            dst[i] = apply ? fmaf(-lr, o, dst[i]) : o;
        }
    }
}

}  // namespace

hipError_t launch_norm(const NormLaunch& L, int blocks, const ConstPtrTable& G, const PtrTable* BUF, float mu,
                       hipStream_t stream, bool in16) {
    if (in16)
        k_norm<false, true><<<blocks, kThreads, 0, stream>>>(L, G, PtrTable{}, mu);
    else if (BUF)
        k_norm<true><<<blocks, kThreads, 0, stream>>>(L, G, *BUF, mu);
    else
        k_norm<false><<<blocks, kThreads, 0, stream>>>(L, G, PtrTable{}, mu);
    return hipGetLastError();
}

hipError_t launch_scale_cast(const CastLaunch& L, int blocks, const ConstPtrTable& G, bool bf16_in, float eps,
                             hipStream_t stream) {
    if (bf16_in)
        k_scale_cast<true><<<blocks, kThreads, 0, stream>>>(L, G, eps);
    else
        k_scale_cast<false><<<blocks, kThreads, 0, stream>>>(L, G, eps);
    return hipGetLastError();
}

hipError_t launch_zero_rows(bf16_t* X, int64_t x_mat, int cnt, int first_row, int rows, int ld, hipStream_t stream) {
    const int64_t n = static_cast<int64_t>(rows - first_row) * ld;
    if (n <= 0 || cnt <= 0) return hipSuccess;
    int64_t blocks = (n + kThreads - 1) / kThreads;
    if (blocks > 1024) blocks = 1024;
    k_zero_rows<<<dim3(static_cast<unsigned>(blocks), static_cast<unsigned>(cnt)), kThreads, 0, stream>>>(
        X, x_mat, static_cast<int64_t>(first_row) * ld, n);
    return hipGetLastError();
}

hipError_t launch_copy_out(const Ns5Plan& plan, int cnt, const bf16_t* X, const PtrTable& out, hipStream_t stream,
                           bool apply, float lr, bool out16) {
    const int64_t total = plan.rows * plan.cols;
    int64_t blocks = (total + kThreads - 1) / kThreads;
    if (blocks > 2048) blocks = 2048;
    k_copy_out<<<dim3(static_cast<unsigned>(blocks), cnt), kThreads, 0, stream>>>(
        out, static_cast<int>(plan.rows), static_cast<int>(plan.cols), plan.tall ? 1 : 0, plan.ldx, X,
        static_cast<int64_t>(plan.x_elems), apply ? 1 : 0, lr, out16 ? 1 : 0);
    return hipGetLastError();
}

}  // namespace muon
