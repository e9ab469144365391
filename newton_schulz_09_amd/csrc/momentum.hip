// Nesterov momentum (summary paragraph of the Muon section in the Synced
// report on Modded-NanoGPT: the gradient first passes through Nesterov
// momentum, and the resulting direction is what gets orthogonalised).  Reading of the lost formula: buf <- mu*buf + g ;
// u <- g + mu*buf, each a single float32 fused multiply-add.
//
// HBM-bound streaming kernel: 16 bytes per element (read g and buf, write buf
// and u).  Each thread moves kUnroll float4 groups per trip, issuing all loads
// before any store so several 16-byte requests are in flight per lane.
#include "internal.hpp"

namespace muon {

namespace {

constexpr int kUnroll = 4;

__device__ __forceinline__ void nesterov1(float g, float& b, float& u, float mu) {
    b = fmaf(mu, b, g);
    u = fmaf(mu, b, g);
}

__global__ __launch_bounds__(kThreads) void k_momentum_vec4(const f32x4* g, f32x4* buf, f32x4* u,
                                                            int64_t n4, float mu) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads * kUnroll;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kThreads * kUnroll + threadIdx.x; base < n4;
         base += stride) {
        f32x4 gv[kUnroll], bv[kUnroll];
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) {
            const int64_t i = base + static_cast<int64_t>(r) * kThreads;
            if (i < n4) {
                gv[r] = __builtin_nontemporal_load(&g[i]);
                bv[r] = buf[i];
            }
        }
#pragma unroll
        for (int r = 0; r < kUnroll; ++r) {
            const int64_t i = base + static_cast<int64_t>(r) * kThreads;
            if (i < n4) {
                f32x4 uv;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float b = bv[r][q], w;
                    nesterov1(gv[r][q], b, w, mu);
                    bv[r][q] = b;
                    uv[q] = w;
                }
                buf[i] = bv[r];
                __builtin_nontemporal_store(uv, &u[i]);
            }
        }
    }
}

__global__ __launch_bounds__(kThreads) void k_momentum_scalar(const float* g, float* buf, float* u,
                                                              int64_t begin, int64_t numel, float mu) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    for (int64_t i = begin + static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < numel;
         i += stride) {
        float b = buf[i], uv;
        nesterov1(g[i], b, uv, mu);
        buf[i] = b;
        u[i] = uv;
    }
}

// Grouped form: matrix blockIdx.y of the table, the same update; 16-byte
// groups where its three pointers are aligned, then a scalar tail.
__global__ __launch_bounds__(kThreads) void k_momentum_grouped(MomentumGroup t, float mu) {
    const int k = blockIdx.y;
    const float* g = t.g[k];
    float* buf = t.buf[k];
    float* u = t.u[k];
    const int64_t numel = t.numel[k];
    const bool aligned = ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(buf) |
                           reinterpret_cast<uintptr_t>(u)) & 15u) == 0;
    const int64_t n4 = aligned ? numel / 4 : 0;
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kThreads;
    const int64_t first = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t i = first; i < n4; i += stride) {
        const f32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g) + i);
        f32x4 bv = reinterpret_cast<const f32x4*>(buf)[i], uv;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float b = bv[q], w;
            nesterov1(gv[q], b, w, mu);
            bv[q] = b;
            uv[q] = w;
        }
        reinterpret_cast<f32x4*>(buf)[i] = bv;
        __builtin_nontemporal_store(uv, reinterpret_cast<f32x4*>(u) + i);
    }
    for (int64_t i = 4 * n4 + first; i < numel; i += stride) {
        float b = buf[i], uv;
        nesterov1(g[i], b, uv, mu);
        buf[i] = b;
        u[i] = uv;
    }
}

inline int grid_for(int64_t work_items, int per_block) {
    int64_t blocks = (work_items + per_block - 1) / per_block;
    if (blocks > 4096) blocks = 4096;
    if (blocks < 1) blocks = 1;
    return static_cast<int>(blocks);
}

}  // namespace

hipError_t launch_momentum(const float* g, float* buf, float* u, int64_t numel, float mu,
                           hipStream_t stream) {
    const bool aligned = ((reinterpret_cast<uintptr_t>(g) | reinterpret_cast<uintptr_t>(buf) |
                           reinterpret_cast<uintptr_t>(u)) & 15u) == 0;
    int64_t done = 0;
    if (aligned) {
        const int64_t n4 = numel / 4;
        if (n4 > 0) {
            k_momentum_vec4<<<grid_for(n4, kThreads * kUnroll), kThreads, 0, stream>>>(
                reinterpret_cast<const f32x4*>(g), reinterpret_cast<f32x4*>(buf),
                reinterpret_cast<f32x4*>(u), n4, mu);
        }
        done = n4 * 4;
    }
    if (done < numel) {
        k_momentum_scalar<<<grid_for(numel - done, kThreads), kThreads, 0, stream>>>(g, buf, u, done,
                                                                                    numel, mu);
    }
    return hipGetLastError();
}

hipError_t launch_momentum_grouped(const MomentumGroup& t, int count, int64_t max_numel, float mu,
                                  hipStream_t stream) {
    // about 4 float4 groups per thread for the largest matrix, at most 2048
    // workgroups per matrix
    const int bx = grid_for((max_numel + 15) / 16, kThreads) < 2048 ? grid_for((max_numel + 15) / 16, kThreads)
                                                                   : 2048;
    k_momentum_grouped<<<dim3(static_cast<unsigned>(bx), static_cast<unsigned>(count)), kThreads, 0, stream>>>(t,
                                                                                                             mu);
    return hipGetLastError();
}

}  // namespace muon
