// The three products of every NS5 step (the printed
// zeroth_power_via_newtonschulz5 of the Muon section, Synced report on
// Modded-NanoGPT):
//     A = X X^T              (SYRK: upper-triangle tiles only, mirrored)
//     B = b A + c A A        (A is symmetric, so A A = A A^T; upper tiles,
//                             mirrored; the b A + c (.) update is fused)
//     X' = a X + B X         (full tile grid; a X is added inside the K loop
//                             from the X rows staged there; X' is stored
//                             row-major for the next step, or as float32 in
//                             G's orientation after the last step)
//
// The symmetric two are "NT" products  C[i][j] = sum_k P[i][k] Q[j][k]  with
// both operands contiguous along k, the operand layout of the CDNA matrix
// cores.  a X + B X is "NN": its second operand X is row-major (contiguous
// along n, not k); its tiles are stored row-major in LDS and the MFMA
// fragments are formed with gfx950's transposing LDS reads
// (ds_read_b64_tr_b16), so X is never stored transposed.
//
// Engine (gfx950): WGM x WGN wavefronts of 64 lanes, each owning a
// (BM/WGM)x(BN/WGN) sub-tile built from 32x32 MFMA fragments
// (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  The 256x256 tiles of
// a X + B X and of X X^T run on 2x4 waves (two per SIMD; a symmetric
// product's diagonal tiles then go in 64x64 blocks), the other square tiles
// on 2x2, the 256x128 tile of a X + B X on 4x2.  K advances
// BK at a time through a ring of STAGES LDS buffers filled by direct
// global->LDS loads (global_load_lds_dwordx4: each lane supplies a global
// address, the 64 lanes' 16-byte pieces land contiguously in LDS), so the
// loads of the next STAGES-1 K steps are in flight while one is multiplied,
// without passing through registers.  One barrier per K step; the waits are
// issued explicitly so that only the loads of the step about to be used are
// waited for.  Inside a K step the MFMAs, the LDS fragment reads and the
// global->LDS loads are issued interleaved in a fixed order.
//
// LDS layout: row-major tiles of BK bf16 per row.  The 16-byte chunk c of
// row r is stored at slot c ^ f(r); the loads place it there by choosing
// which global chunk each lane fetches.  f spreads the fragment reads (32
// consecutive rows, one chunk each, 16 bytes per lane) over all banks whether
// the LDS serves 8 or 16 lanes of a 16-byte read per cycle.
//
// Work distribution: one workgroup per output tile, every matrix of every
// segment (a set of same-shaped matrices; up to kMaxSeg shapes that share the
// tile size) in the same launch.  Consecutive workgroups are dispatched
// round-robin over the 8 XCDs (each with its own L2), so the workgroup index
// is remapped: for the full grid (a X + B X) every XCD takes a contiguous
// range of tiles, and within a matrix tiles are ordered in bands of `band`
// tile rows, column by column inside a band, so that the tiles resident on
// one XCD share operand panels (with all tile rows in one band, each column
// panel of the second operand is read from memory once); for the symmetric
// products, whose K differs between segments, whole matrices are dealt to
// the XCDs in turn.  The mapping only places work: every output element is
// accumulated in the same K order under any tile shape or mapping (and a X
// enters the sum at the same K), so a matrix gets bitwise the same result in
// any batch.
#include <stdlib.h>

#include <type_traits>

#include "internal.hpp"

namespace muon {

namespace {

constexpr int kXcds = 8;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const void* global_cptr;
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Workgroup b of G -> logical index, so that XCD x (which receives the
// workgroups b = x, x + 8, ...) processes one contiguous logical range.
__device__ __forceinline__ int xcd_remap(int b, int G) {
    const int q = G / kXcds, r = G % kXcds, x = b % kXcds;
    return x * q + (x < r ? x : r) + b / kXcds;
}

// Workgroup b of G -> logical index when every matrix has tpm tiles: XCD x
// takes whole matrices x, x + 8, x + 16, ... (its tiles of one matrix in
// order), so segments of different K are spread evenly over the XCDs.  The
// matrices past the last multiple of 8 keep the dispatch order.
__device__ __forceinline__ int xcd_interleave(int b, int G, int tpm) {
    const int full = (G / tpm) / kXcds * kXcds * tpm;  // workgroups of whole rounds of 8 matrices
    if (b >= full) return b;
    const int x = b % kXcds, i = b / kXcds;
    return ((i / tpm) * kXcds + x) * tpm + i % tpm;
}

// Slot permutation of row r for CPR 16-byte chunks per row (8 or 4).
template <int CPR>
__device__ __forceinline__ int swz(int r) {
    if constexpr (CPR == 8) return ((r >> 1) ^ (r << 2)) & 7;
    else return ((r >> 1) ^ (r >> 3)) & 3;
}

// Slot permutation of row r of a row-major K x N tile (CPRQ chunks per row)
// read with transposing reads: the 8 rows one read touches (two runs of 4,
// 8 apart) get distinct offsets within one 256-byte bank cycle (rows of 256
// bytes or more all start on the same bank, so the offsets step by 32 bytes;
// 128-byte rows alternate halves and step by 16).
template <int CPRQ>
__device__ __forceinline__ int swq(int r) {
    return ((((r & 3) << 1) | ((r >> 3) & 1)) * (CPRQ >= 16 ? 2 : 1)) & (CPRQ - 1);
}


// Slot of 16-byte chunk c in a row of N chunks of an epilogue staging tile,
// keyed on the row: XOR for power-of-two N, a rotation otherwise (both
// permute the row's chunks).
template <int N>
__device__ __forceinline__ int eslot(int c, int key) {
    if constexpr ((N & (N - 1)) == 0) return c ^ (key & (N - 1));
    else return (c + key) % N;
}

// ds_read_b64_tr_b16: in every group of 16 lanes, lane r supplies the LDS
// address of 4 consecutive 16-bit values (row r of a 16 x 4 block R); lane i
// receives R[4e + i/4][i%4] for e = 0..3.  With lane r pointing at
// (k + r/4, c + 4 (r%4)) of a row-major tile, lane i receives the four values
// (k .. k+3, c + i): four consecutive K of one column.
//
// Issued as inline asm: the compiler's wait insertion cannot tell that these
// reads do not overlap the global->LDS loads in flight and would otherwise
// wait for all of them first.  The asm is invisible to that pass, so every
// consumer waits explicitly (lgkm_wait_tie) before using the result.
__device__ __forceinline__ u32x2 lds_read_tr4(const bf16_t* p) {
    const uint32_t a = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16_t*)(p)));
    uint64_t v;
    asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(a));
    return __builtin_bit_cast(u32x2, v);
}

// 8-byte LDS read, as inline asm for the same reason (used while
// global->LDS loads are in flight).
__device__ __forceinline__ u32x2 lds_read8(const bf16_t* p) {
    const uint32_t a = static_cast<uint32_t>(
        reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const bf16_t*)(p)));
    uint64_t v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(a));
    return __builtin_bit_cast(u32x2, v);
}

// Wait for this wave's LDS reads, with `x` passing through the wait so that
// no use of it can be scheduled before it.
template <typename T>
__device__ __forceinline__ void lgkm_wait_tie(T& x) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(x));
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding and its LDS operations are done, then barrier.  Written as one
// asm statement with a memory clobber so the compiler keeps LDS accesses on
// their side of it.
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Waves per SIMD the register allocation must leave room for.  4-wave
// a X + B X workgroups whose LDS lets two of them share a CU ask for two:
// within that budget the MFMA accumulators live in ordinary VGPRs, which the
// a X update inside the K loop writes directly (with a budget of one wave per
// SIMD they go to AGPRs, and every K step copies them out and back).
template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int KIND>
constexpr int min_waves_per_simd() {
    constexpr bool two_fit = 2 * STAGES * (BM + BN) * BK * 2 <= 160 * 1024;  // two workgroups' LDS per CU
    return (WGM * WGN == 4 && two_fit && (KIND == GEMM_BX || KIND == GEMM_BX_FINAL)) ? 2 : 1;
}

template <int BM, int BN, int BK, int STAGES, int WGM, int WGN, int KIND>
__global__ __launch_bounds__(64 * WGM * WGN, (min_waves_per_simd<BM, BN, BK, STAGES, WGM, WGN, KIND>())) void k_gemm_nt(
    GemmLaunch launch, PtrTable out) {
    constexpr bool SYM = (KIND == GEMM_SYRK || KIND == GEMM_AAB);
    static_assert(!SYM || BM == BN, "symmetric products use square tiles");
    static_assert(BK == 64 || BK == 32, "BK is 32 or 64");
    static_assert(STAGES >= 2 && STAGES <= 4, "2..4 stages");
    constexpr int NW = WGM * WGN;              // wavefronts per workgroup
    constexpr int WTM = BM / WGM, WTN = BN / WGN;  // wave sub-tile
    static_assert(!SYM || WGM == WGN || (WTN == 64 && WTM % 64 == 0),
                  "a non-square wave grid of a symmetric product handles diagonal tiles in 64 x 64 blocks");
    constexpr int FM = WTM / 32, FN = WTN / 32;
    // a X + B X reads its second operand, X, in its own row-major layout ("NN"):
    // the Q tile is BK rows of K by BN columns, and the MFMA fragments (8
    // consecutive K of one column per lane) come from transposing LDS reads
    constexpr bool NN = (KIND == GEMM_BX || KIND == GEMM_BX_FINAL);
    constexpr int CPR = BK / 8;            // 16-byte chunks per LDS row (NT tiles)
    constexpr int RPI = 64 / CPR;          // rows filled by one wave-wide 1 KB load
    constexpr int CPRQ = NN ? BN / 8 : CPR;  // the same for the Q tile
    constexpr int RPIQ = 64 / CPRQ;
    constexpr int IP = BM / RPI / NW;      // loads per wave per stage, P operand
    constexpr int IQ = NN ? BK / RPIQ / NW : BN / RPI / NW;  // and Q operand
    constexpr int NLOAD = IP + IQ;
    constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per stage
    static_assert(IP >= 1 && IQ >= 1 && RPIQ >= 1 && IP * RPI * NW == BM &&
                      IQ * NW * (NN ? RPIQ : RPI) == (NN ? BK : BN),
                  "tile shape not supported by the loader");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave sub-tiles are made of 32 x 32 fragments");
    static_assert(BM * BN <= STAGES * STAGE, "the epilogue reuses the stages as four wave sub-tiles");

    __shared__ __attribute__((aligned(1024))) bf16_t lds[STAGES * STAGE];

    // ---- which segment, which matrix and which output tile
    const int lid = launch.interleave_tpm > 0
                        ? xcd_interleave(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x),
                                         launch.interleave_tpm)
                        : xcd_remap(static_cast<int>(blockIdx.x), static_cast<int>(gridDim.x));
    int si = 0;
#pragma unroll
    for (int q = 1; q < kMaxSeg; ++q)
        if (q < launch.nseg && lid >= launch.seg[q].first_block) si = q;
    const GemmArgs& args = launch.seg[si];
    const int local = lid - args.first_block;
    const int mat = local / args.tiles_per_mat;
    int t = local - mat * args.tiles_per_mat;
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
        const int per_band = args.band * args.tiles_n;
        const int band = t / per_band;
        const int first = band * args.band;
        const int rows_in_band = args.tiles - first < args.band ? args.tiles - first : args.band;
        const int w = t - band * per_band;
        ti = first + w % rows_in_band;
        tj = w / rows_in_band;
    }
    const int i0 = ti * BM, j0 = tj * BN;

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS targets stay scalar
    const int wm = wave / WGN, wn = wave % WGN;

    // ---- loader: load i of this wave fills rows r0 = (wave*IP + i)*RPI ..
    // r0 + RPI - 1 of its operand; lane l covers row r0 + l / CPR and LDS slot
    // l % CPR, so it fetches global chunk (l % CPR) ^ f(row).
    const bf16_t* gp[IP];
    const bf16_t* gq[IQ];
    {
        const bf16_t* P = args.P + mat * args.p_mat + static_cast<int64_t>(i0) * args.ldp;
        const int lr = lane / CPR, ls = lane % CPR;
#pragma unroll
        for (int i = 0; i < IP; ++i) {
            const int row = (wave * IP + i) * RPI + lr;
            gp[i] = P + static_cast<int64_t>(row) * args.ldp + ((ls ^ swz<CPR>(row)) << 3);
        }
        if constexpr (NN) {
            // Q rows are K rows of X; the tile's columns start at j0
            const bf16_t* Q = args.Q + mat * args.q_mat + j0;
            const int lrq = lane / CPRQ, lsq = lane % CPRQ;
#pragma unroll
            for (int i = 0; i < IQ; ++i) {
                const int row = (wave * IQ + i) * RPIQ + lrq;
                gq[i] = Q + static_cast<int64_t>(row) * args.ldq + ((lsq ^ swq<CPRQ>(row)) << 3);
            }
        } else {
            const bf16_t* Q = args.Q + mat * args.q_mat + static_cast<int64_t>(j0) * args.ldq;
#pragma unroll
            for (int i = 0; i < IQ; ++i) {
                const int row = (wave * IQ + i) * RPI + lr;
                gq[i] = Q + static_cast<int64_t>(row) * args.ldq + ((ls ^ swz<CPR>(row)) << 3);
            }
        }
    }
    // the Q operand's row stride, read once: inside the K loop a reload from
    // the kernel arguments would wait on the scalar memory counter, which LDS
    // reads share
    const int64_t ldq = __builtin_amdgcn_readfirstlane(args.ldq);
    // A diagonal tile of a symmetric product (ti == tj) reads the same rows
    // as P and as Q: on 256 x 256 tiles with two stages its Q loads are
    // skipped and its Q fragments come from the P tile.  (The waits of deeper
    // pipelines count NLOAD loads per step; on smaller tiles the branch
    // around each load cost more than the loads it saved: X X^T of the
    // 1600-class matrices on 128 tiles took 3% longer.)
    constexpr bool Q_SHARE = SYM && STAGES == 2 && BM == 256;
    const bool q_is_p = Q_SHARE && ti == tj;
    const int qoff = q_is_p ? 0 : BM * BK;  // where a stage's Q tile starts
    // load L (< IP: P rows, else Q rows) of K step kt into LDS stage `stage`
    auto issue_one = [&](int L, int kt, int stage) {
        if (Q_SHARE && L >= IP && q_is_p) return;
        bf16_t* sP = lds + stage * STAGE;
        const int k0 = kt * BK;
        if (L < IP)
            __builtin_amdgcn_global_load_lds((global_cptr)(gp[L] + k0),
                                             (lds_ptr)(sP + (wave * IP + L) * RPI * BK), 16, 0, 0);
        else if constexpr (NN)
            __builtin_amdgcn_global_load_lds((global_cptr)(gq[L - IP] + static_cast<int64_t>(k0) * ldq),
                                             (lds_ptr)(sP + BM * BK + (wave * IQ + L - IP) * RPIQ * BN), 16, 0,
                                             0);
        else
            __builtin_amdgcn_global_load_lds((global_cptr)(gq[L - IP] + k0),
                                             (lds_ptr)(sP + BM * BK + (wave * IQ + L - IP) * RPI * BK), 16, 0,
                                             0);
    };

    // NN Q fragments: lane l (group g = l/16, r = l%16) points at K row
    // 16 kk + 8 (g/2) + r/4 (+4 for the second half) and column
    // 16 (g%2) + 4 (r%4) of the 32-column fragment; the row's slot
    // permutation is the same for every kk and both halves.
    const int tq_g = lane >> 4, tq_r = lane & 15;
    const int tq_row = 8 * (tq_g >> 1) + (tq_r >> 2);                // + 16 kk (+ 4)
    const int tq_col = 16 * (tq_g & 1) + 4 * (tq_r & 3);             // + column of the fragment
    const int tq_sw = swq<CPRQ>(tq_row);
    auto q_frag_nn = [&](const bf16_t* sQs, int kk, int col0) -> bf16x8 {
        const int col = col0 + tq_col;
        const bf16_t* p0 = sQs + (16 * kk + tq_row) * BN + ((((col >> 3) ^ tq_sw)) << 3) + (col & 7);
        const u32x2 lo = lds_read_tr4(p0);
        const u32x2 hi = lds_read_tr4(p0 + 4 * BN);
        return __builtin_bit_cast(bf16x8, u32x4{lo.x, lo.y, hi.x, hi.y});
    };

    // ---- fragment reads: lane l reads row (l % 32) of a 32-row fragment,
    // logical chunk 2 kk + l / 32, i.e. slot (2 kk + l / 32) ^ f(l % 32)
    // (f depends on the row modulo 16 only, and fragments start at multiples
    // of 32).
    int soff[BK / 16];
    {
        const int r = lane & 31, hi = lane >> 5;
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) soff[kk] = r * BK + (((2 * kk + hi) ^ swz<CPR>(r)) << 3);
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[fm][fn][r] = 0.0f;

    // The second operand of the fused update (AAB: A[j][i] = A[i][j]; BX:
    // old X[i][j]) is the K slice [i0, i0 + BM) of the Q operand, which passes
    // through LDS during the K loop, so it is never read from memory again.
    // a X + B X adds a X[i][j] to the accumulator inside the K loop, as soon
    // as the K values below 64 (floor(i / 64) + 1) are summed: the same point
    // under every tile shape and K step, so a matrix's result does not depend
    // on its batch.  Wave sub-tiles of up to 4 fragments copy the values out
    // of the stage of the K step that holds them (with BK = 32 that is one
    // step before the sum reaches the point, for rows in the first half of a
    // 64 block); larger ones (BK = 64 only) read and add them in that step.
    // b A + c A A scales the whole sum by c, so its operand is added in the
    // epilogue: copied out the same way for sub-tiles up to 64 x 64, staged
    // through LDS after the loop for larger ones (their copies would not fit
    // in registers).  K steps past kpad hold only padding, whose values are
    // zero.
    constexpr bool CAPTURE_E = (NN || KIND == GEMM_AAB) && FM * FN <= 4;
    constexpr bool APPLY_NOW = NN && !CAPTURE_E;
    static_assert(!APPLY_NOW || BK == 64, "sub-tiles of more than 4 fragments add a X on BK = 64 only");
    u32x2 ev[CAPTURE_E ? FM : 1][CAPTURE_E ? FN : 1][4];
    if constexpr (CAPTURE_E) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) ev[fm][fn][g4] = u32x2{0u, 0u};
    }

    // b A + c A A's operand for sub-tiles too large to capture: the BM x BN
    // tile of A at (i0, j0), row-major (A is symmetric, so it stands in for
    // its transpose), is loaded after the K loop from the base of the LDS with
    // 16-byte global->LDS loads, in two halves of EH rows; each lane then
    // reads its runs of 4 rows of one column with transposing reads.
    constexpr bool STAGE_E = KIND == GEMM_AAB && !CAPTURE_E;
    constexpr int CPRE = BN / 8, RPIE = 64 / CPRE, EH = BM / 2;
    constexpr int NEH = EH / (RPIE > 0 ? RPIE : 1) / NW;  // loads per wave per half
    static_assert(!STAGE_E || (RPIE >= 1 && NEH >= 1 && NEH * RPIE * NW == EH),
                  "E tile shape not supported by the loader");
    // chunk permutation of the staged rows: the transposing reads read runs
    // of 4 rows (the Q-tile permutation)
    auto swe = [](int row) { return swq<CPRE>(row); };
    const bf16_t* Et = args.E + static_cast<int64_t>(mat) * args.e_mat + static_cast<int64_t>(i0) * args.lde + j0;
    // load i of half h of this wave's share of the E tile to `dst` (the
    // half's first row)
    auto issue_e = [&](int i, int h, bf16_t* dst) {
        const int lre = lane / CPRE, lse = lane % CPRE;
        const int rl = (wave * NEH + i) * RPIE + lre;  // row within the half
        const int row = h * EH + rl;
        __builtin_amdgcn_global_load_lds(
            (global_cptr)(Et + static_cast<int64_t>(row) * args.lde + ((lse ^ swe(row)) << 3)),
            (lds_ptr)(dst + (wave * NEH + i) * RPIE * BN), 16, 0, 0);
    };

    const int nk = args.kpad / BK;
    // Every iteration issues the NLOAD loads of one K step (STAGES-1 steps
    // ahead), so the number of loads outstanding behind step kt is always
    // (STAGES-2)*NLOAD.  Steps past the end are clamped to the last one: they
    // refill a stage that no later iteration reads.
#pragma unroll
    for (int s = 0; s < STAGES - 1; ++s) {
        const int ks = s < nk ? s : nk - 1;
#pragma unroll
        for (int L = 0; L < NLOAD; ++L) issue_one(L, ks, s);
    }

    // Per K step: the MFMAs of slice kk (NMF of them) are interleaved with
    // the LDS reads of slice kk+1's fragments and with this step's global->LDS
    // loads, one instruction after another (full scheduling barriers keep the
    // order), so the wave never stops issuing MFMAs for a burst of memory
    // instructions.
    constexpr int NKK = BK / 16;
    constexpr int NMF = FM * FN;
    constexpr int NR = FM + FN;                                  // fragment reads per slice
    constexpr int RWIN = NMF * 3 / 4 > 0 ? NMF * 3 / 4 : 1;      // reads follow MFMAs 0 .. RWIN-1
    constexpr int TOT = NKK * NMF;
    constexpr int LWIN = STAGES == 2 ? (TOT / 2 > 0 ? TOT / 2 : 1) : (TOT * 3 / 4 > 0 ? TOT * 3 / 4 : 1);

    for (int kt = 0; kt < nk; ++kt) {
        wait_vm_barrier<(STAGES - 2) * NLOAD>();
        // every wave is past step kt-1, so its stage can be refilled
        const int kl = kt + STAGES - 1 < nk ? kt + STAGES - 1 : nk - 1;
        const int sl = (kt + STAGES - 1) % STAGES;

        const bf16_t* sP = lds + (kt % STAGES) * STAGE + wm * WTM * BK;
        const bf16_t* sQ = lds + (kt % STAGES) * STAGE + qoff + wn * WTN * BK;
        const bf16_t* sQs_nn = lds + (kt % STAGES) * STAGE + BM * BK;  // NN: the whole Q tile
        bf16x8 a[2][FM], b[2][FN];
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
            a[0][fm] = as_bf16x8(*reinterpret_cast<const u32x4*>(sP + fm * 32 * BK + soff[0]));
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            if constexpr (NN)
                b[0][fn] = q_frag_nn(sQs_nn, 0, wn * WTN + fn * 32);
            else
                b[0][fn] = as_bf16x8(*reinterpret_cast<const u32x4*>(sQ + fn * 32 * BK + soff[0]));
        }
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
            const int c = kk & 1, n = c ^ 1;
            if constexpr (NN) {
                // the transposing reads of this slice's Q fragments are asm
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int fn = 0; fn < FN; ++fn) lgkm_wait_tie(b[c][fn]);
            }
#pragma unroll
            for (int q = 0; q < NMF; ++q) {
                __builtin_amdgcn_sched_barrier(0);
                // NN: Q as the MFMA's first operand, so that the accumulator
                // is the fragment transposed: each lane holds 4 consecutive
                // columns of one output row (contiguous in X)
                if constexpr (NN)
                    acc[q / FN][q % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b[c][q % FN], a[c][q / FN],
                                                                                  acc[q / FN][q % FN], 0, 0, 0);
                else
                    acc[q / FN][q % FN] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[c][q / FN], b[c][q % FN],
                                                                                  acc[q / FN][q % FN], 0, 0, 0);
                __builtin_amdgcn_sched_barrier(0);
                if (kk + 1 < NKK) {
#pragma unroll
                    for (int r = 0; r < NR; ++r) {
                        if ((r * RWIN) / NR == q) {
                            if (r < FM)
                                a[n][r] = as_bf16x8(
                                    *reinterpret_cast<const u32x4*>(sP + r * 32 * BK + soff[kk + 1]));
                            else if constexpr (NN)
                                b[n][r - FM] = q_frag_nn(sQs_nn, kk + 1, wn * WTN + (r - FM) * 32);
                            else
                                b[n][r - FM] = as_bf16x8(
                                    *reinterpret_cast<const u32x4*>(sQ + (r - FM) * 32 * BK + soff[kk + 1]));
                        }
                    }
                }
                const int g = kk * NMF + q;
                // (with two stages, the last step's loads would only refill a
                // stage no later step reads, and are skipped)
                if (STAGES > 2 || kt + 1 < nk) {
#pragma unroll
                    for (int L = 0; L < NLOAD; ++L)
                        if ((L * LWIN) / NLOAD == g) issue_one(L, kl, sl);
                }
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        // a X[i][j] for the rows whose 64 block of K ends with this step
        auto add_ax = [&](int fm, int fn, int g4, u32x2 e4) {
            const float e0 = bf16_to_f32(static_cast<bf16_t>(e4.x & 0xffffu));
            const float e1 = bf16_to_f32(static_cast<bf16_t>(e4.x >> 16));
            const float e2 = bf16_to_f32(static_cast<bf16_t>(e4.y & 0xffffu));
            const float e3 = bf16_to_f32(static_cast<bf16_t>(e4.y >> 16));
            acc[fm][fn][4 * g4 + 0] = fmaf(args.alpha, e0, acc[fm][fn][4 * g4 + 0]);
            acc[fm][fn][4 * g4 + 1] = fmaf(args.alpha, e1, acc[fm][fn][4 * g4 + 1]);
            acc[fm][fn][4 * g4 + 2] = fmaf(args.alpha, e2, acc[fm][fn][4 * g4 + 2]);
            acc[fm][fn][4 * g4 + 3] = fmaf(args.alpha, e3, acc[fm][fn][4 * g4 + 3]);
        };
        if constexpr (APPLY_NOW) {
            const bf16_t* sQs = lds + (kt % STAGES) * STAGE + BM * BK;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int ik = i0 + wm * WTM + fm * 32;  // first row of this fragment row block
                if (kt == ik / BK) {
                    const int krow = ik - kt * BK + (lane & 31);
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        u32x2 e4[4];
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int col = wn * WTN + fn * 32 + 8 * g4 + 4 * (lane >> 5);
                            e4[g4] = lds_read8(sQs + krow * BN + (((col >> 3) ^ swq<CPRQ>(krow)) << 3) + (col & 7));
                        }
                        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(e4[0]), "+v"(e4[1]), "+v"(e4[2]), "+v"(e4[3]));
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) add_ax(fm, fn, g4, e4[g4]);
                    }
                }
            }
        }
        if constexpr (CAPTURE_E) {
            const bf16_t* sQs = lds + (kt % STAGES) * STAGE + qoff;
#pragma unroll
            for (int fm = 0; fm < FM; ++fm) {
                const int ik = i0 + wm * WTM + fm * 32;  // first K index of this fragment row block
                if (kt == ik / BK) {
                    const int kin = ik - kt * BK;
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn) {
                        if constexpr (NN) {
                            // X row kin + (l % 32), columns 8 g4 + 4 (l/32) .. +3 of
                            // this fragment: one 8-byte read per g4
                            const int krow = kin + (lane & 31);
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                const int col = wn * WTN + fn * 32 + 8 * g4 + 4 * (lane >> 5);
                                ev[fm][fn][g4] = lds_read8(
                                    sQs + krow * BN + (((col >> 3) ^ swq<CPRQ>(krow)) << 3) + (col & 7));
                            }
                        } else {
                            const int jrow = wn * WTN + fn * 32 + (lane & 31);
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                const int kk = kin + 8 * g4 + 4 * (lane >> 5);
                                ev[fm][fn][g4] = *reinterpret_cast<const u32x2*>(
                                    sQs + jrow * BK + (((kk >> 3) ^ swz<CPR>(jrow)) << 3) + (kk & 7));
                            }
                        }
                    }
                }
            }
            if constexpr (NN) {
#pragma unroll
                for (int fm = 0; fm < FM; ++fm) {
                    const int ik = i0 + wm * WTM + fm * 32;
                    if (kt == (ik / 64 + 1) * (64 / BK) - 1) {
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn) {
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                lgkm_wait_tie(ev[fm][fn][g4]);  // captured by asm reads
                                add_ax(fm, fn, g4, ev[fm][fn][g4]);
                            }
                        }
                    }
                }
            }
        }
    }
    // drain the loads of the clamped tail steps before the epilogue
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (STAGE_E) {
        // the epilogue operand's tile, from the LDS base, once every wave is
        // done reading the stages
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
        for (int i = 0; i < NEH; ++i) {
            issue_e(i, 0, lds);
            issue_e(i, 1, lds + EH * BN);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
    }

    // ---- epilogue.  Accumulator register r of a 32x32 fragment holds, in
    // lane l, row 8*(r/4) + 4*(l/32) + r%4 and column l%32: each lane owns
    // runs of 4 consecutive rows in one column.  For NN (operands swapped in
    // the MFMA) rows and columns trade places: each lane owns runs of 4
    // consecutive columns of one row.  The fused update is applied in
    // registers and rounded once to bf16; then every wave passes its
    // (WTM x WTN) sub-tile through its own LDS region to store whole rows with
    // 16-byte stores: as is, and for the symmetric products also transposed
    // into the mirror block.
    const int64_t cm = static_cast<int64_t>(mat);
    const int i0w = i0 + wm * WTM, j0w = j0 + wn * WTN;  // this wave's sub-tile origin
    // 4 bf16: rows ib..ib+3 of column j (NN: columns of row i)
    u32x2 hv[FM][FN][4];
    // (a X + B X added its a X inside the K loop)
    constexpr bool HAS_E = KIND == GEMM_AAB;
    static_assert(!HAS_E || CAPTURE_E || STAGE_E, "the epilogue operand is captured or staged");
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) {
            u32x2 es[4];
            if constexpr (STAGE_E) {
                // rows of the staged tile: runs of 4 rows of one column
                const int ec = wn * WTN + fn * 32 + tq_col;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int er = wm * WTM + fm * 32 + 8 * g4 + 4 * (tq_g >> 1) + (tq_r >> 2);
                    es[g4] = lds_read_tr4(lds + er * BN + (((ec >> 3) ^ swe(er)) << 3) + (ec & 7));
                }
                asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(es[0]), "+v"(es[1]), "+v"(es[2]), "+v"(es[3]));
            }
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float v0 = acc[fm][fn][4 * g4 + 0], v1 = acc[fm][fn][4 * g4 + 1];
                float v2 = acc[fm][fn][4 * g4 + 2], v3 = acc[fm][fn][4 * g4 + 3];
                if constexpr (HAS_E) {
                    // b A + c (A A): A[i..i+3][j] = A[j][i..i+3] (symmetric),
                    // the run of 4 this lane owns
                    const u32x2 e4 = CAPTURE_E ? ev[fm][fn][g4] : es[g4];
                    const float e0 = bf16_to_f32(static_cast<bf16_t>(e4.x & 0xffffu));
                    const float e1 = bf16_to_f32(static_cast<bf16_t>(e4.x >> 16));
                    const float e2 = bf16_to_f32(static_cast<bf16_t>(e4.y & 0xffffu));
                    const float e3 = bf16_to_f32(static_cast<bf16_t>(e4.y >> 16));
                    v0 = fmaf(args.beta, v0, args.alpha * e0);
                    v1 = fmaf(args.beta, v1, args.alpha * e1);
                    v2 = fmaf(args.beta, v2, args.alpha * e2);
                    v3 = fmaf(args.beta, v3, args.alpha * e3);
                }
                hv[fm][fn][g4].x = f32x2_to_bf16x2(v0, v1);
                hv[fm][fn][g4].y = f32x2_to_bf16x2(v2, v3);
            }
        }
    }

    // every wave is done with the K loop's LDS stages before any reuses them
    __syncthreads();
    bf16_t* W = lds + wave * (WTM * WTN);
    constexpr int CT_ = WTM / 8;  // 16-byte chunks per row of the transposed sub-tile (WTN rows)
    constexpr int CN_ = WTN / 8;  // and of the direct one (WTM rows)

    // (a) write the transposed sub-tile [jj][ii]: 8-byte pieces, chunk index
    // XOR-swizzled with the row so the 32 rows a store touches spread over
    // the banks
    auto put_t = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int jj = fn * 32 + (lane & 31);
                    const int ii = fm * 32 + 8 * g4 + 4 * (lane >> 5);
                    *reinterpret_cast<u32x2*>(W + jj * WTM + (eslot<CT_>(ii >> 3, jj) << 3) + (ii & 7)) =
                        hv[fm][fn][g4];
                }
    };
    // (b) write the direct sub-tile [ii][jj] (2-byte pieces).  Its chunk
    // swizzle is keyed on ii / 4, so a lane's run of 4 rows shares one
    // address computation (the rows are immediate offsets).  `sym` keeps only
    // ii <= jj and mirrors it, which makes a diagonal sub-tile exactly
    // symmetric.
    auto put_n = [&](bool sym) {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int jj = fn * 32 + (lane & 31);
                    const int ib = fm * 32 + 8 * g4 + 4 * (lane >> 5);
                    const uint32_t w2[2] = {hv[fm][fn][g4].x, hv[fm][fn][g4].y};
                    bf16_t* row0 = W + ib * WTN + (eslot<CN_>(jj >> 3, ib >> 2) << 3) + (jj & 7);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int ii = ib + q;
                        const bf16_t h = static_cast<bf16_t>((w2[q >> 1] >> (16 * (q & 1))) & 0xffffu);
                        if (!sym || ii <= jj) {
                            row0[q * WTN] = h;
                            if (sym) W[jj * WTN + (eslot<CN_>(ii >> 3, jj >> 2) << 3) + (ii & 7)] = h;
                        }
                    }
                }
    };
    // NN layout (each lane owns row ii, columns jj .. jj+3):
    // (d) the direct sub-tile [ii][jj], one 8-byte piece per run, chunk
    // swizzle keyed on ii / 2 (rows pair up in a 256-byte bank cycle, so 16
    // consecutive rows land on distinct banks)
    auto put_rn = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ii = fm * 32 + (lane & 31);
                    const int jj = fn * 32 + 8 * g4 + 4 * (lane >> 5);
                    *reinterpret_cast<u32x2*>(W + ii * WTN + (eslot<CN_>(jj >> 3, ii >> 1) << 3) + (jj & 7)) =
                        hv[fm][fn][g4];
                }
    };
    // (e) the transposed sub-tile [jj][ii] (2-byte pieces), swizzle keyed on
    // the row jj as in (a)
    auto put_tn = [&]() {
#pragma unroll
        for (int fm = 0; fm < FM; ++fm)
#pragma unroll
            for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int ii = fm * 32 + (lane & 31);
                    const int jj = fn * 32 + 8 * g4 + 4 * (lane >> 5);
                    const uint32_t w2[2] = {hv[fm][fn][g4].x, hv[fm][fn][g4].y};
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        W[(jj + q) * WTM + (eslot<CT_>(ii >> 3, jj + q) << 3) + (ii & 7)] =
                            static_cast<bf16_t>((w2[q >> 1] >> (16 * (q & 1))) & 0xffffu);
                }
    };
    auto lds_fence = [&]() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); };
    // (c) store the LDS sub-tile (ROWS rows of CPR chunks) as bf16 rows of
    // dst with leading dimension ld
    // (`shift` selects the layout's swizzle key: row (transposed), row / 4
    // (direct) or row / 2 (NN direct))
    auto store_bf16 = [&](auto cpr_c, int rows, int shift, bf16_t* dst, int ld) {
        constexpr int cpr = decltype(cpr_c)::value;
        for (int q = lane; q < rows * cpr; q += 64) {
            const int row = q / cpr, c = q % cpr;
            const u32x4 v =
                *reinterpret_cast<const u32x4*>(W + row * cpr * 8 + (eslot<cpr>(c, row >> shift) << 3));
            u32x4* d = reinterpret_cast<u32x4*>(dst + static_cast<int64_t>(row) * ld + c * 8);
            if (KIND == GEMM_BX && launch.stream_out)
                __builtin_nontemporal_store(v, d);
            else
                *d = v;
        }
    };

    if constexpr (SYM && WGM != WGN) {
        // non-square wave grid (sub-tiles of WTM x 64): off-diagonal tiles as
        // below; on a diagonal tile each 64 x 64 block of the wave's sub-tile
        // lies wholly above the diagonal (stored with its mirror), on it
        // (symmetrised, stored once) or wholly below (the mirror of another)
        bf16_t* C = args.C + cm * args.c_mat;
        if (ti != tj) {
            put_t();
            lds_fence();
            store_bf16(std::integral_constant<int, CT_>{}, WTN, 0, C + static_cast<int64_t>(j0w) * args.ldc + i0w,
                       args.ldc);
            lds_fence();
            put_n(false);
            lds_fence();
            store_bf16(std::integral_constant<int, CN_>{}, WTM, 2, C + static_cast<int64_t>(i0w) * args.ldc + j0w,
                       args.ldc);
        } else {
#pragma unroll
            for (int b = 0; b < WTM / 64; ++b) {
                const int rb = wm * WTM + 64 * b, cb = wn * 64;  // tile-local origin of the block
                if (rb > cb) continue;
                const int gi = i0 + rb, gj = j0 + cb;
                // the block's two fragment rows, staged as a 64 x 64 tile
#pragma unroll
                for (int f = 0; f < 2; ++f)
#pragma unroll
                    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                        for (int g4 = 0; g4 < 4; ++g4) {
                            const int fm = 2 * b + f;
                            const int jj = fn * 32 + (lane & 31);
                            const int ib = f * 32 + 8 * g4 + 4 * (lane >> 5);
                            const uint32_t w2[2] = {hv[fm][fn][g4].x, hv[fm][fn][g4].y};
                            if (rb < cb) {  // above: the mirror [jj][ii] first (8-byte pieces)
                                *reinterpret_cast<u32x2*>(W + jj * 64 + (eslot<8>(ib >> 3, jj) << 3) + (ib & 7)) =
                                    hv[fm][fn][g4];
                            } else {  // on the diagonal: keep ii <= jj and mirror it
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const int ii = ib + q;
                                    if (ii <= jj) {
                                        const bf16_t h = static_cast<bf16_t>((w2[q >> 1] >> (16 * (q & 1))) & 0xffffu);
                                        W[ii * 64 + (eslot<8>(jj >> 3, ii >> 2) << 3) + (jj & 7)] = h;
                                        W[jj * 64 + (eslot<8>(ii >> 3, jj >> 2) << 3) + (ii & 7)] = h;
                                    }
                                }
                            }
                        }
                lds_fence();
                if (rb < cb) {
                    store_bf16(std::integral_constant<int, 8>{}, 64, 0, C + static_cast<int64_t>(gj) * args.ldc + gi,
                               args.ldc);
                    lds_fence();
                    // then the block itself [ii][jj] (2-byte pieces)
#pragma unroll
                    for (int f = 0; f < 2; ++f)
#pragma unroll
                        for (int fn = 0; fn < FN; ++fn)
#pragma unroll
                            for (int g4 = 0; g4 < 4; ++g4) {
                                const int fm = 2 * b + f;
                                const int jj = fn * 32 + (lane & 31);
                                const int ib = f * 32 + 8 * g4 + 4 * (lane >> 5);
                                const uint32_t w2[2] = {hv[fm][fn][g4].x, hv[fm][fn][g4].y};
#pragma unroll
                                for (int q = 0; q < 4; ++q)
                                    W[(ib + q) * 64 + (eslot<8>(jj >> 3, ib >> 2) << 3) + (jj & 7)] =
                                        static_cast<bf16_t>((w2[q >> 1] >> (16 * (q & 1))) & 0xffffu);
                            }
                    lds_fence();
                }
                store_bf16(std::integral_constant<int, 8>{}, 64, 2, C + static_cast<int64_t>(gi) * args.ldc + gj,
                           args.ldc);
                lds_fence();
            }
        }
    } else if constexpr (SYM) {
        bf16_t* C = args.C + cm * args.c_mat;
        if (ti != tj || wm < wn) {
            // off-diagonal block: the block itself and its mirror
            put_t();
            lds_fence();
            store_bf16(std::integral_constant<int, CT_>{}, WTN, 0, C + static_cast<int64_t>(j0w) * args.ldc + i0w, args.ldc);
            lds_fence();
            put_n(false);
            lds_fence();
            store_bf16(std::integral_constant<int, CN_>{}, WTM, 2, C + static_cast<int64_t>(i0w) * args.ldc + j0w, args.ldc);
        } else if (wm == wn) {
            // diagonal block: symmetrised once, stored once
            put_n(true);
            lds_fence();
            store_bf16(std::integral_constant<int, CN_>{}, WTM, 2, C + static_cast<int64_t>(i0w) * args.ldc + j0w, args.ldc);
        }
        // (wm > wn on a diagonal tile: the mirror of the wm < wn block)
    } else if constexpr (KIND == GEMM_BX) {
        put_rn();
        lds_fence();
        store_bf16(std::integral_constant<int, CN_>{}, WTM, 1,
                   args.C + cm * args.c_mat + static_cast<int64_t>(i0w) * args.ldc + j0w, args.ldc);
    } else {  // GEMM_BX_FINAL: float32 output in G's orientation, clipped to m x n
        float* o = out.p[args.out_base + mat];
        const bool tall = args.tall != 0;
        const int rows = tall ? WTN : WTM, cpr = tall ? CT_ : CN_;
        const int r0 = tall ? j0w : i0w, c0 = tall ? i0w : j0w;   // origin in the output
        const int rlim = tall ? args.n : args.m, clim = tall ? args.m : args.n;  // output rows x cols
        if (tall) put_tn(); else put_rn();  // keyed on the row / on the row / 2
        lds_fence();
        const bool vec_ok = (clim & 3) == 0 && (reinterpret_cast<uintptr_t>(o) & 15u) == 0;
        const bool vec16 = (clim & 7) == 0 && (reinterpret_cast<uintptr_t>(o) & 15u) == 0;
        for (int q = lane; q < rows * cpr; q += 64) {
            const int row = q / cpr, c = q % cpr;
            const int gr = r0 + row, gc = c0 + c * 8;
            if (gr >= rlim || gc >= clim) continue;
            const int slot = tall ? eslot<CT_>(c, row) : eslot<CN_>(c, row >> 1);
            const u32x4 v = *reinterpret_cast<const u32x4*>(W + row * cpr * 8 + (slot << 3));
            if (args.out16) {  // bfloat16 output: X as is
                bf16_t* d16 = reinterpret_cast<bf16_t*>(o) + static_cast<int64_t>(gr) * clim + gc;
                if (vec16 && gc + 8 <= clim) {
                    *reinterpret_cast<u32x4*>(d16) = v;
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (gc + e < clim) d16[e] = static_cast<bf16_t>((v[e >> 1] >> (16 * (e & 1))) & 0xffffu);
                }
                continue;
            }
            float f[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                f[2 * e] = bf16_to_f32(static_cast<bf16_t>(v[e] & 0xffffu));
                f[2 * e + 1] = bf16_to_f32(static_cast<bf16_t>(v[e] >> 16));
            }
            float* dst = o + static_cast<int64_t>(gr) * clim + gc;
            if (vec_ok && gc + 8 <= clim) {
                f32x4 lo = f32x4{f[0], f[1], f[2], f[3]}, hi = f32x4{f[4], f[5], f[6], f[7]};
                if (args.apply) {  // p - lr * O, one rounding
                    const f32x4 plo = *reinterpret_cast<const f32x4*>(dst);
                    const f32x4 phi = *reinterpret_cast<const f32x4*>(dst + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        lo[e] = fmaf(-args.lr, lo[e], plo[e]);
                        hi[e] = fmaf(-args.lr, hi[e], phi[e]);
                    }
                }
                // streaming stores: the output is never read again by this
                // launch, and must not evict the operands its tiles share in L2
                __builtin_nontemporal_store(lo, reinterpret_cast<f32x4*>(dst));
                __builtin_nontemporal_store(hi, reinterpret_cast<f32x4*>(dst + 4));
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    if (gc + e < clim) dst[e] = args.apply ? fmaf(-args.lr, f[e], dst[e]) : f[e];
            }
        }
    }
}

template <int BM, int BN, int BK, int STAGES, int WGM = 2, int WGN = 2>
hipError_t launch_t(GemmKind kind, const GemmLaunch& L, int blocks, const PtrTable* out, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(blocks));
    constexpr int NT = 64 * WGM * WGN;
    PtrTable o{};
    if (out) o = *out;
    if constexpr (BM == BN) {
        switch (kind) {
            case GEMM_SYRK:
                k_gemm_nt<BM, BN, BK, STAGES, WGM, WGN, GEMM_SYRK><<<grid, NT, 0, stream>>>(L, o);
                return hipGetLastError();
            case GEMM_AAB:
                k_gemm_nt<BM, BN, BK, STAGES, WGM, WGN, GEMM_AAB><<<grid, NT, 0, stream>>>(L, o);
                return hipGetLastError();
            default: break;
        }
    }
    // (sub-tiles of more than 4 fragments run a X + B X on BK = 64 only)
    if constexpr (BK != 64 && (BM / WGM / 32) * (BN / WGN / 32) > 4) {
        return hipErrorInvalidValue;
    } else {
        switch (kind) {
            case GEMM_BX: k_gemm_nt<BM, BN, BK, STAGES, WGM, WGN, GEMM_BX><<<grid, NT, 0, stream>>>(L, o); break;
            case GEMM_BX_FINAL:
                k_gemm_nt<BM, BN, BK, STAGES, WGM, WGN, GEMM_BX_FINAL><<<grid, NT, 0, stream>>>(L, o);
                break;
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
}

// The symmetric products only (tiles and engines a X + B X does not use).
template <int BM, int BK, int STAGES>
hipError_t launch_sym_t(GemmKind kind, const GemmLaunch& L, int blocks, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(blocks));
    switch (kind) {
        case GEMM_SYRK: k_gemm_nt<BM, BM, BK, STAGES, 2, 2, GEMM_SYRK><<<grid, 256, 0, stream>>>(L, PtrTable{}); break;
        case GEMM_AAB: k_gemm_nt<BM, BM, BK, STAGES, 2, 2, GEMM_AAB><<<grid, 256, 0, stream>>>(L, PtrTable{}); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(GemmKind kind, int tile, int tile_n, const GemmLaunch& launch, int blocks,
                       const PtrTable* out, hipStream_t stream) {
    // 256 x 128 tiles of a X + B X: 8 waves (4 x 2, each 64 x 64), BK 64,
    // three stages (144 KB of LDS, one workgroup per CU)
    if (tile == 256 && tile_n == 128) {
        if (kind != GEMM_BX && kind != GEMM_BX_FINAL) return hipErrorInvalidValue;
        return launch_t<256, 128, 64, 3, 4, 2>(kind, launch, blocks, out, stream);
    }
    // 192 x 256 tiles of a X + B X: 8 waves (2 x 4, each 96 x 64), BK 64,
    // two stages (112 KB of LDS)
    if (tile == 192 && tile_n == 256) {
        if (kind != GEMM_BX && kind != GEMM_BX_FINAL) return hipErrorInvalidValue;
        return launch_t<192, 256, 64, 2, 2, 4>(kind, launch, blocks, out, stream);
    }
    if (tile_n != tile) return hipErrorInvalidValue;
    // 192 x 192 tiles of the symmetric products (2 x 2 waves of 96 x 96):
    // 4224 = 22 x 192 gives 253 upper tiles where 4096 = 16 x 256 gives 136
    if (tile == 192) return launch_sym_t<192, 64, 2>(kind, launch, blocks, stream);
    // 256 x 256 tiles of a X + B X: 8 waves (2 x 4, each 128 x 64), two per SIMD
    if (tile == 256 && (kind == GEMM_BX || kind == GEMM_BX_FINAL))
        return launch_t<256, 256, 64, 2, 2, 4>(kind, launch, blocks, out, stream);
    // 256 x 256 tiles of X X^T: 8 waves (2 x 4, each 128 x 64; diagonal tiles
    // in 64 x 64 blocks); MUON_SYRK_WAVES=4 selects the 4-wave engine
    static const int syrk_waves = [] {
        const char* s = getenv("MUON_SYRK_WAVES");
        return (s && atoi(s) == 4) ? 4 : 8;
    }();
    if (tile == 256 && syrk_waves == 8 && kind == GEMM_SYRK)
        return launch_t<256, 256, 64, 2, 2, 4>(kind, launch, blocks, out, stream);
    // K pipeline: 0 = BK 64 with 2 stages, 1 = BK 32 with 4 stages,
    // 2 = BK 32 with 2 stages for tiles up to 128 (half the LDS, so more
    // workgroups per CU) (MUON_GEMM_PIPE in the environment, for tuning)
    static const int pipe = [] {
        const char* s = getenv("MUON_GEMM_PIPE");
        const int v = s ? atoi(s) : 0;
        return (v >= 0 && v <= 4) ? v : 0;
    }();
    if (pipe >= 3) {
        switch (tile * 8 + pipe) {
            case 128 * 8 + 3: return launch_t<128, 128, 64, 3>(kind, launch, blocks, out, stream);
            case 128 * 8 + 4: return launch_t<128, 128, 64, 4>(kind, launch, blocks, out, stream);
            default: break;
        }
    }
    switch (tile * 4 + (pipe >= 3 ? 0 : pipe)) {
        case 64 * 4 + 0: return launch_t<64, 64, 64, 2>(kind, launch, blocks, out, stream);
        case 64 * 4 + 1: return launch_t<64, 64, 32, 4>(kind, launch, blocks, out, stream);
        case 128 * 4 + 0: return launch_t<128, 128, 64, 2>(kind, launch, blocks, out, stream);
        case 128 * 4 + 1: return launch_t<128, 128, 32, 4>(kind, launch, blocks, out, stream);
        case 128 * 4 + 2: return launch_t<128, 128, 32, 2>(kind, launch, blocks, out, stream);
        case 64 * 4 + 2: return launch_t<64, 64, 32, 2>(kind, launch, blocks, out, stream);
        case 256 * 4 + 2: return launch_sym_t<256, 64, 2>(kind, launch, blocks, stream);
        case 256 * 4 + 0: return launch_sym_t<256, 64, 2>(kind, launch, blocks, stream);
        case 256 * 4 + 1: return launch_sym_t<256, 32, 4>(kind, launch, blocks, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace muon
