// The three products of every NS5 step (the printed
// zeroth_power_via_newtonschulz5 of the Muon section, Synced report on
// Modded-NanoGPT):
//     A = X X^T              (SYRK: upper-triangle tiles only, mirrored)
//     B = b A + c A A        (A is symmetric, so A A = A A^T; upper tiles,
//                             mirrored; the b A + c (.) update is fused)
//     X' = a X + B X         (full tile grid; a X + (.) fused; X' is stored
//                             in both orientations for the next step, or as
//                             float32 in G's orientation after the last step)
//
// All three are "NT" products  C[i][j] = sum_k P[i][k] Q[j][k]  with both
// operands contiguous along k, which is the operand layout of the CDNA
// matrix cores.  Engine: 256 threads = 4 wavefronts of 64 lanes in a 2x2
// arrangement, each wave owning a (T/2)x(T/2) sub-tile built from 32x32 MFMA
// fragments (v_mfma_f32_32x32x16_bf16, fp32 accumulation); K advances 64 at a
// time through double-buffered LDS tiles (one barrier per K step, the next
// tile's global loads in flight while the current one is multiplied).  LDS
// rows are 128 bytes; the 16-byte chunk index is XOR-swizzled with the row so
// that both the row-wise stores and the fragment loads are bank-conflict
// free.  Matrices of a group are batched into one launch (blockIdx.x encodes
// matrix and tile).
#include "internal.hpp"

namespace muon {

namespace {

constexpr int BK = 64;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

template <int T, int KIND>
__global__ __launch_bounds__(kThreads, 1) void k_gemm_nt(GemmArgs args, PtrTable out) {
    constexpr bool SYM = (KIND == GEMM_SYRK || KIND == GEMM_AAB);
    constexpr int BM = T, BN = T;
    constexpr int WTM = BM / 2, WTN = BN / 2;  // wave sub-tile
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr int CH_P = BM * (BK / 8) / kThreads;  // 16-byte chunks per thread per operand
    constexpr int CH_Q = BN * (BK / 8) / kThreads;
    static_assert(CH_P >= 1 && CH_Q >= 1, "tile too small for the loader");

    __shared__ __attribute__((aligned(16))) bf16_t lds[2][(BM + BN) * BK];

    // ---- which matrix and which output tile
    const int mat = blockIdx.x / args.tiles_per_mat;
    int t = blockIdx.x - mat * args.tiles_per_mat;
    int ti, tj;
    if constexpr (SYM) {
        ti = 0;
        int rowlen = args.tiles;
        while (t >= rowlen) {
            t -= rowlen;
            ++ti;
            --rowlen;
        }
        tj = ti + t;
    } else {
        ti = t / args.tiles_n;
        tj = t - ti * args.tiles_n;
    }
    const int i0 = ti * BM, j0 = tj * BN;
    const bf16_t* P = args.P + mat * args.p_mat + static_cast<int64_t>(i0) * args.ldp;
    const bf16_t* Q = args.Q + mat * args.q_mat + static_cast<int64_t>(j0) * args.ldq;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    uint4 regP[CH_P], regQ[CH_Q];
    auto gload = [&](int k0) {
#pragma unroll
        for (int c = 0; c < CH_P; ++c) {
            const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
            regP[c] = *reinterpret_cast<const uint4*>(P + static_cast<int64_t>(row) * args.ldp + k0 + ch * 8);
        }
#pragma unroll
        for (int c = 0; c < CH_Q; ++c) {
            const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
            regQ[c] = *reinterpret_cast<const uint4*>(Q + static_cast<int64_t>(row) * args.ldq + k0 + ch * 8);
        }
    };
    auto lstore = [&](int b) {
        bf16_t* sP = lds[b];
        bf16_t* sQ = lds[b] + BM * BK;
#pragma unroll
        for (int c = 0; c < CH_P; ++c) {
            const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<uint4*>(sP + row * BK + ((ch ^ (row & 7)) << 3)) = regP[c];
        }
#pragma unroll
        for (int c = 0; c < CH_Q; ++c) {
            const int idx = tid + c * kThreads, row = idx >> 3, ch = idx & 7;
            *reinterpret_cast<uint4*>(sQ + row * BK + ((ch ^ (row & 7)) << 3)) = regQ[c];
        }
    };

    f32x16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

    const int nk = args.kpad / BK;
    gload(0);
    lstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const bf16_t* sP = lds[cur];
        const bf16_t* sQ = lds[cur] + BM * BK;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + (lane >> 5);
            bf16x8 a[FM], b[FN];
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int row = wm * WTM + fm * 32 + (lane & 31);
                a[fm] = as_bf16x8(*reinterpret_cast<const uint4*>(sP + row * BK + ((ch ^ (row & 7)) << 3)));
            }
#pragma unroll
            for (int fn = 0; fn < FN; ++fn) {
                const int row = wn * WTN + fn * 32 + (lane & 31);
                b[fn] = as_bf16x8(*reinterpret_cast<const uint4*>(sQ + row * BK + ((ch ^ (row & 7)) << 3)));
            }
#pragma unroll
            for (int fm = 0; fm < FM; ++fm)
#pragma unroll
                for (int fn = 0; fn < FN; ++fn)
                    acc[fm][fn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[fm], b[fn], acc[fm][fn], 0, 0, 0);
        }
        if (kt + 1 < nk) lstore(cur ^ 1);
        __syncthreads();
    }

    // ---- epilogue.  Accumulator register r of a 32x32 fragment holds, in
    // lane l, row 8*(r/4) + 4*(l/32) + r%4 and column l%32: each lane owns
    // runs of 4 consecutive rows in one column.
    const bool diag = SYM && (ti == tj);
    const int64_t cm = static_cast<int64_t>(mat);
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            const int j = j0 + wn * WTN + fn * 32 + (lane & 31);
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int ib = i0 + wm * WTM + fm * 32 + 8 * g4 + 4 * (lane >> 5);
                float v[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) v[q] = acc[fm][fn][4 * g4 + q];
                if constexpr (KIND == GEMM_AAB) {
                    // A is symmetric: A[i][j] = A[j][i], read along the contiguous run
                    const bf16_t* e = args.E + cm * args.e_mat + static_cast<int64_t>(j) * args.lde + ib;
                    const uint2 ev = *reinterpret_cast<const uint2*>(e);
                    const bf16_t eh[4] = {static_cast<bf16_t>(ev.x & 0xffff), static_cast<bf16_t>(ev.x >> 16),
                                          static_cast<bf16_t>(ev.y & 0xffff), static_cast<bf16_t>(ev.y >> 16)};
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = fmaf(args.beta, v[q], args.alpha * bf16_to_f32(eh[q]));
                } else if constexpr (KIND == GEMM_BX || KIND == GEMM_BX_FINAL) {
                    // old X[i][j] read from X^T[j][i], which is the Q operand
                    const bf16_t* e = args.E + cm * args.e_mat + static_cast<int64_t>(j) * args.lde + ib;
                    const uint2 ev = *reinterpret_cast<const uint2*>(e);
                    const bf16_t eh[4] = {static_cast<bf16_t>(ev.x & 0xffff), static_cast<bf16_t>(ev.x >> 16),
                                          static_cast<bf16_t>(ev.y & 0xffff), static_cast<bf16_t>(ev.y >> 16)};
#pragma unroll
                    for (int q = 0; q < 4; ++q) v[q] = fmaf(args.alpha, bf16_to_f32(eh[q]), v[q]);
                }
                bf16_t h[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) h[q] = f32_to_bf16(v[q]);

                if constexpr (SYM) {
                    bf16_t* C = args.C + cm * args.c_mat;
                    if (!diag || ib + 3 <= j) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) C[static_cast<int64_t>(ib + q) * args.ldc + j] = h[q];
                        uint2 pk;
                        pk.x = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
                        pk.y = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
                        *reinterpret_cast<uint2*>(C + static_cast<int64_t>(j) * args.ldc + ib) = pk;
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            if (ib + q <= j) {
                                C[static_cast<int64_t>(ib + q) * args.ldc + j] = h[q];
                                C[static_cast<int64_t>(j) * args.ldc + ib + q] = h[q];
                            }
                        }
                    }
                } else if constexpr (KIND == GEMM_BX) {
                    bf16_t* C = args.C + cm * args.c_mat;
                    bf16_t* CT = args.CT + cm * args.ct_mat;
#pragma unroll
                    for (int q = 0; q < 4; ++q) C[static_cast<int64_t>(ib + q) * args.ldc + j] = h[q];
                    uint2 pk;
                    pk.x = static_cast<uint32_t>(h[0]) | (static_cast<uint32_t>(h[1]) << 16);
                    pk.y = static_cast<uint32_t>(h[2]) | (static_cast<uint32_t>(h[3]) << 16);
                    *reinterpret_cast<uint2*>(CT + static_cast<int64_t>(j) * args.ldct + ib) = pk;
                } else {  // GEMM_BX_FINAL: float32 output in G's orientation
                    float* o = out.p[mat];
                    if (j < args.n) {
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int i = ib + q;
                            if (i < args.m) {
                                const float f = bf16_to_f32(h[q]);
                                if (args.tall)
                                    o[static_cast<int64_t>(j) * args.m + i] = f;
                                else
                                    o[static_cast<int64_t>(i) * args.n + j] = f;
                            }
                        }
                    }
                }
            }
        }
    }
}

template <int T>
hipError_t launch_t(GemmKind kind, const GemmArgs& args, int cnt, const PtrTable* out, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(args.tiles_per_mat) * cnt);
    PtrTable o{};
    if (out) o = *out;
    switch (kind) {
        case GEMM_SYRK: k_gemm_nt<T, GEMM_SYRK><<<grid, kThreads, 0, stream>>>(args, o); break;
        case GEMM_AAB: k_gemm_nt<T, GEMM_AAB><<<grid, kThreads, 0, stream>>>(args, o); break;
        case GEMM_BX: k_gemm_nt<T, GEMM_BX><<<grid, kThreads, 0, stream>>>(args, o); break;
        case GEMM_BX_FINAL: k_gemm_nt<T, GEMM_BX_FINAL><<<grid, kThreads, 0, stream>>>(args, o); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, int tile, const GemmArgs& args, int cnt, const PtrTable* out,
                       hipStream_t stream) {
    switch (tile) {
        case 64: return launch_t<64>(kind, args, cnt, out, stream);
        case 128: return launch_t<128>(kind, args, cnt, out, stream);
        case 256: return launch_t<256>(kind, args, cnt, out, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace muon
