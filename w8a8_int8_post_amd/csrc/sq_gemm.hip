// sq_gemm.hip -- INT8 x INT8 -> INT32 GEMM with fused scale back, gfx950.
//
// P1 = abeam.tech explainer of "SmoothQuant: Accurate and Efficient
// Post-Training Quantization for Large Language Models": 用語解説 "INT8 GEMM"
// and 推論方法 (the heavy linear layers run as INT8 GEMMs after the offline
// transform).  P4 = blogs.itmedia.co.jp 量子化 blog, section 3 (multiply the
// scale factor back at inference).
//
//   acc[m, n] = sum_k xq[m, k] * wq[n, k]          (exact int32)
//   y[m, n]   = out( (fp32(acc) * x_scale[m]) * w_scale[n] )
//
// Both operands are K-contiguous ("TN"), the natural feed of the MFMA
// matrix cores: every lane's 16-byte fragment is one contiguous load.
//
// Kernels, chosen by the shape (M <= 64 tokens go to the few-token kernels of
// sq_decode.hip, except 17-64 tokens on layers at least 12288 channels wide):
//  * dma (M > 64, K % 128 == 0): workgroup tile BM x BN; 128-byte K slices go
//    from global memory straight into LDS (global_load_lds_dwordx4, no
//    register staging), double-buffered, as XOR-swizzled 16-byte chunks
//    (conflict-free ds_read_b128 fragment reads); v_mfma_i32_32x32x32_i8 with
//    the weight tile as the row operand, so each lane ends with four
//    consecutive output channels; the scaled 16-bit tile is staged through
//    LDS and written as coalesced 16-byte row pieces; XCD-aware tile order so
//    that tiles sharing operand panels run on the same XCD's L2.
//  * tiled (M > 64, other K): the same tiling with register-staged loads and
//    byte-granular masking of the K tail.
//  * the packed variant of dma reads the weights in the fragment-packed
//    layout (see pack_weight_kernel), which the few-token kernels need: there
//    every wave load of weights is one contiguous kilobyte, independent of K.
//
// The MFMA sums over K inside one instruction in whatever order the hardware
// takes; the A and B fragments give each lane the same K positions, so any
// order yields the same integer sum.
#include "sq_gemm_common.h"

#include <mutex>

namespace sq {
namespace {

// ---------------------------------------------------------------------------
// Tiled kernel.
template <int BM, int BN, int BK, int WM, int WN, int SWS, Out O, bool KVEC, bool EXT>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64, 1) void gemm_tiled_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    constexpr int WAVES_N = BN / WN;
    constexpr int NT = (BM / WM) * WAVES_N * 64;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int CPR = BK / 16;  // 16-byte chunks per tile row
    constexpr int A_PER_T = BM * CPR / NT;
    constexpr int B_PER_T = BN * CPR / NT;
    static_assert(BM * CPR % NT == 0 && BN * CPR % NT == 0, "tile/thread mismatch");
    static_assert(BK % 32 == 0, "BK must be a multiple of the MFMA K (32)");
    constexpr int STAGE = (BM + BN) * BK;
    __shared__ __attribute__((aligned(16))) int8_t smem[2 * STAGE];
    batch_entry<O>(A, B, sx, sw, Y, M, N, K, (int64_t)N * K);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;

    // Workgroup -> tile.  Hardware places workgroup b on XCD b % 8; give each
    // XCD a contiguous range of the logical order, and walk the logical order
    // in groups of GM tile rows so that concurrently running tiles share A
    // rows and B columns.
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN;
    const int total = nbm * nbn;
    const int bid = blockIdx.x;
    const int q = total >> 3, rr = total & 7, xcd = bid & 7, idx = bid >> 3;
    const int logical = (xcd < rr ? xcd * (q + 1) : rr * (q + 1) + (xcd - rr) * q) + idx;
    constexpr int GM = 8;
    const int group_size = GM * nbn;
    const int group = logical / group_size;
    const int first_m = group * GM;
    const int gsz = (nbm - first_m) < GM ? (nbm - first_m) : GM;
    const int in_group = logical - group * group_size;
    const int m0 = (first_m + in_group % gsz) * BM;
    const int n0 = (in_group / gsz) * BN;

    v4i ra[A_PER_T], rb[B_PER_T];

    auto gload = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * NT;
            ra[i] = load_chunk<KVEC>(A, m0 + c / CPR, M, k0 + (c % CPR) * 16, K);
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int c = tid + i * NT;
            rb[i] = load_chunk<KVEC>(B, n0 + c / CPR, N, k0 + (c % CPR) * 16, K);
        }
    };
    auto lds_off = [](int row, int chunk) {
        return row * BK + ((chunk ^ ((row >> SWS) & (CPR - 1))) << 4);
    };
    auto sstore = [&](int buf) {
        int8_t* sA = smem + buf * STAGE;
        int8_t* sB = sA + BM * BK;
#pragma unroll
        for (int i = 0; i < A_PER_T; ++i) {
            const int c = tid + i * NT;
            *reinterpret_cast<v4i*>(sA + lds_off(c / CPR, c % CPR)) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_PER_T; ++i) {
            const int c = tid + i * NT;
            *reinterpret_cast<v4i*>(sB + lds_off(c / CPR, c % CPR)) = rb[i];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    const int nk = (K + BK - 1) / BK;
    gload(0);
    sstore(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) gload((kt + 1) * BK);
        const int8_t* sA = smem + cur * STAGE;
        const int8_t* sB = sA + BM * BK;
#pragma unroll
        for (int s = 0; s < BK / 32; ++s) {
            const int chunk = s * 2 + (lane >> 5);
            v4i af[TM], bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int row = wm0 + i * 32 + (lane & 31);
                af[i] = *reinterpret_cast<const v4i*>(sA + lds_off(row, chunk));
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int row = wn0 + j * 32 + (lane & 31);
                bf[j] = *reinterpret_cast<const v4i*>(sB + lds_off(row, chunk));
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < nk) sstore(cur ^ 1);
        __syncthreads();
    }

    // Epilogue.  32 x 32 accumulator layout: lane l, element r holds row
    // 8*(r/4) + 4*(l/32) + r%4 and column l%32 of the sub-tile.
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn0 + j * 32 + (lane & 31);
        const bool nok = n < N;
        const float swn = (O != Out::I32 && nok) ? sw[n] : 0.0f;
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (nok && m < M) {
                    const float sxm = (O != Out::I32) ? sx[m] : 0.0f;
                    store_out_ext<O, EXT>(Y, (int64_t)m * N + n, acc[i][j][r], sxm, swn, epi, n);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// DMA kernel (K % BK == 0).  Out-of-range rows of a tile are clamped to the
// last valid row: they only feed output rows/columns that are never stored.
template <Out O> struct Half;
template <> struct Half<Out::F16> {
    typedef _Float16 T;
    __device__ static T cvt(float f) { return (_Float16)f; }
};
template <> struct Half<Out::BF16> {
    typedef uint16_t T;
    __device__ static T cvt(float f) { return BF16::from_f32(f); }
};

// Wait until at most N vector-memory loads of this wave are outstanding.
template <int N>
__device__ inline void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <int BM, int BN, int BK, int WM, int WN, Out O, bool PACKED_B, int MINB = 1,
          int NSTAGE = 2, bool EXT = false, bool NTS = false /* non-temporal output stores */,
          bool SPLITK = false, int KGR = 1 /* wave groups splitting K inside the workgroup */>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64 * KGR, MINB) void gemm_dma_kernel(
    const int8_t* __restrict__ A, const int8_t* __restrict__ B, const float* __restrict__ sx,
    const float* __restrict__ sw, void* __restrict__ Y, int M, int N, int K, Epi epi) {
    // XOR swizzle of the 16-byte chunks: chunk c of row r sits at c ^ ((r >>
    // SWS) & (CPR - 1)).  A fragment read takes 16 consecutive rows, one chunk,
    // in each 256-byte LDS cycle; with 128-byte rows the bank base repeats every
    // 2 rows (shift 1), with 64-byte rows every 4 (shift 2), so that the 16 rows
    // land on 16 distinct bank groups.
    constexpr int SWS = BK == 64 ? 2 : 1, GM = 8;
    constexpr int KGT = BK / 64;  // packed k-groups per K tile
    static_assert(BK == 64 || BK == 128, "BK is 64 or 128");
    // KGR > 1: KGR groups of NW waves, each multiplying the whole tile over
    // its own contiguous K range K / KGR (a multiple of BK) through its own
    // ring of stages; groups 1 .. KGR-1 hand their accumulators to group 0
    // through LDS after the loop, and all threads share the output stores.
    // KGR times the loads in flight per CU for a layer whose tiles number at
    // most one per CU.
    static_assert(KGR == 1 || KGR == 2 || KGR == 4, "one, two or four wave groups along K");
    constexpr int WAVES_N = BN / WN, NW = (BM / WM) * WAVES_N, NTG = NW * 64, NT = NTG * KGR;
    constexpr int TM = WM / 32, TN = WN / 32, CPR = BK / 16, S = BK / 32;
    constexpr int A_INS = BM * CPR / NTG, B_INS = BN * CPR / NTG;  // 1 KB wave loads per thread
    static_assert(BM * CPR % NTG == 0 && BN * CPR % NTG == 0, "tile/thread mismatch");
    constexpr int STAGE = (BM + BN) * BK;
    constexpr bool HALF_OUT = (O == Out::F16 || O == Out::BF16);
    constexpr int EPI_LD = BN * 2 + 16;  // staged output row pitch (bytes): padded, 16-byte aligned
    constexpr int EPI = HALF_OUT ? BM * EPI_LD : 0;
    constexpr int RED_G = NW * TN * TM * 16 * 64;  // accumulator words of one group
    constexpr int RED = (KGR - 1) * RED_G * 4;     // groups 1 .. KGR-1
    constexpr int RING = KGR * NSTAGE * STAGE > RED ? KGR * NSTAGE * STAGE : RED;
    constexpr int SMEM = RING > EPI ? RING : EPI;
    constexpr int INS = A_INS + B_INS;  // loads per thread per K tile
    static_assert(NSTAGE >= 1 && NSTAGE <= 4, "1 to 4 operand stages");
    __shared__ __attribute__((aligned(16))) int8_t smem[SMEM];
    const int tid = threadIdx.x, lane = tid & 63;
    // wave group and wave within it
    const int grp = KGR > 1 ? (tid >> 6) / NW : 0, wave = KGR > 1 ? (tid >> 6) % NW : tid >> 6;
    // SPLITK: blockIdx.y is the split (a contiguous range of K / epi.splits,
    // KGR multiples of BK); otherwise it is the batch entry.  Wave group grp
    // takes the grp-th of KGR equal parts of the workgroup's K range.
    int koff = grp * (K / KGR);
    if constexpr (SPLITK)
        koff = (int)blockIdx.y * (K / epi.splits) + grp * (K / epi.splits / KGR);
    else
        batch_entry<O>(A, B, sx, sw, Y, M, N, K,
                       PACKED_B ? (int64_t)((N + 15) / 16) * 16 * K : (int64_t)N * K);

    const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
    const int nbm = (M + BM - 1) / BM, nbn = (N + BN - 1) / BN, total = nbm * nbn;
    const int bid = blockIdx.x;
    const int q = total >> 3, rr = total & 7, xcd = bid & 7, idx = bid >> 3;
    const int logical = (xcd < rr ? xcd * (q + 1) : rr * (q + 1) + (xcd - rr) * q) + idx;
    const int group_size = GM * nbn, group = logical / group_size, first_m = group * GM;
    const int gsz = (nbm - first_m) < GM ? (nbm - first_m) : GM;
    const int in_group = logical - group * group_size;
    const int m0 = (first_m + in_group % gsz) * BM, n0 = (in_group / gsz) * BN;

    auto swz = [](int row) { return (row >> SWS) & (CPR - 1); };
    auto off = [&](int row, int chunk) { return row * BK + ((chunk ^ swz(row)) << 4); };
    // Packed B stage: 1 KB blocks (row block, k-group); inside a block the
    // 16-byte piece of row r, k-subgroup g sits at (g * 16 + r) * 16.
    auto boff = [&](int row, int chunk) {
        if constexpr (PACKED_B)
            return ((row >> 4) * KGT + (chunk >> 2)) * 1024 + (((chunk & 3) << 4) + (row & 15)) * 16;
        else
            return off(row, chunk);
    };
    // Each wave load fills 64 consecutive 16-byte LDS slots; slot p of a
    // stage holds row p / CPR, logical chunk (p % CPR) ^ swz(row).
    const int8_t* asrc[A_INS];
    const int8_t* bsrc[B_INS];
#pragma unroll
    for (int i = 0; i < A_INS; ++i) {
        const int p = (i * NW + wave) * 64 + lane, row = p / CPR, c = (p % CPR) ^ swz(row);
        const int gm = m0 + row < M ? m0 + row : M - 1;
        asrc[i] = A + (int64_t)gm * K + koff + c * 16;
    }
    const int KG = K / 64;  // 64-byte k-groups per packed row block
#pragma unroll
    for (int i = 0; i < B_INS; ++i) {
        if constexpr (PACKED_B) {
            // one contiguous 1 KB block per wave load: row block q / KGT, k-group q % KGT
            const int q = i * NW + wave;
            const int nb = (N + 15) / 16;
            const int rb = n0 / 16 + q / KGT < nb ? n0 / 16 + q / KGT : nb - 1;
            bsrc[i] = B + ((int64_t)rb * KG + koff / 64 + (q % KGT)) * 1024 + lane * 16;
        } else {
            const int p = (i * NW + wave) * 64 + lane, row = p / CPR, c = (p % CPR) ^ swz(row);
            const int gn = n0 + row < N ? n0 + row : N - 1;
            bsrc[i] = B + (int64_t)gn * K + koff + c * 16;
        }
    }
    auto issue = [&](int buf, int k0) {
        int8_t* sA = smem + (grp * NSTAGE + buf) * STAGE;
        int8_t* sB = sA + BM * BK;
#pragma unroll
        for (int i = 0; i < A_INS; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(asrc[i] + k0),
                (__attribute__((address_space(3))) void*)(sA + (i * NW + wave) * 1024), 16, 0, 0);
#pragma unroll
        for (int i = 0; i < B_INS; ++i)
            __builtin_amdgcn_global_load_lds(
                (const __attribute__((address_space(1))) void*)(bsrc[i] + (PACKED_B ? k0 * 16 : k0)),
                (__attribute__((address_space(3))) void*)(sB + (i * NW + wave) * 1024), 16, 0, 0);
    };

    v16i acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

    // NSTAGE operand stages in a ring: tiles kt+1 .. kt+NSTAGE-2 stay in
    // flight while tile kt is multiplied, and tile kt+NSTAGE-1 is issued into
    // the stage that tile kt-1 used.  One stage (short K, where a small LDS
    // footprint lets more workgroups share a CU): tile kt+1 is issued once
    // every wave is done with tile kt.
    const int nk = (SPLITK ? K / epi.splits : K) / KGR / BK;
    if constexpr (NSTAGE == 1) {
        if (nk > 0) issue(0, 0);
    } else {
#pragma unroll
        for (int p = 0; p < NSTAGE - 1; ++p)
            if (p < nk) issue(p, p * BK);
    }
    int cur = 0;  // stage of tile kt
    for (int kt = 0; kt < nk; ++kt) {
        // This wave's loads of tile kt have landed (loads complete in order,
        // so only the later tiles' may be outstanding); after the barrier
        // every wave's have, and every wave is done reading tile kt-1.
        const int ahead = nk - 1 - kt;  // tiles issued after tile kt, capped below
        if (NSTAGE >= 4 && ahead >= 2)
            wait_vm<2 * INS>();
        else if (NSTAGE >= 3 && ahead >= 1)
            wait_vm<INS>();
        else
            wait_vm<0>();
        asm volatile("s_barrier" ::: "memory");
        const int8_t* sA = smem + (grp * NSTAGE + cur) * STAGE;
        const int8_t* sB = sA + BM * BK;
        v4i af[2][TM], bf[2][TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
            af[0][i] = *reinterpret_cast<const v4i*>(sA + off(wm0 + i * 32 + (lane & 31), lane >> 5));
#pragma unroll
        for (int j = 0; j < TN; ++j)
            bf[0][j] = *reinterpret_cast<const v4i*>(sB + boff(wn0 + j * 32 + (lane & 31), lane >> 5));
        if constexpr (NSTAGE > 1) {
            const int nxt = kt + NSTAGE - 1;
            int nbuf = cur + NSTAGE - 1;
            nbuf = nbuf >= NSTAGE ? nbuf - NSTAGE : nbuf;
            if (nxt < nk) issue(nbuf, nxt * BK);
        }
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int cb = s & 1, nb = cb ^ 1;
            if (s + 1 < S) {
                const int ch = (s + 1) * 2 + (lane >> 5);
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    af[nb][i] = *reinterpret_cast<const v4i*>(sA + off(wm0 + i * 32 + (lane & 31), ch));
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bf[nb][j] = *reinterpret_cast<const v4i*>(sB + boff(wn0 + j * 32 + (lane & 31), ch));
            }
            // D = W_tile * X_tile^T: D's rows are output channels, its columns tokens.
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
                    acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[cb][j], af[cb][i], acc[j][i], 0, 0, 0);
        }
        __builtin_amdgcn_iglp_opt(0);  // interleave the LDS reads with the MFMAs
        if constexpr (NSTAGE == 1) {
            if (kt + 1 < nk) {
                __syncthreads();  // every wave's fragment reads of tile kt are done
                issue(0, (kt + 1) * BK);
            }
        }
        cur = cur + 1 == NSTAGE ? 0 : cur + 1;
    }

    if constexpr (KGR > 1) {
        // Every wave is past its last tile (its loads landed, its fragment
        // reads are in registers): groups 1 .. KGR-1 store their accumulators
        // over the operand stages, each in its own slice, and group 0 adds
        // them (integer sums, exact in any order).  Lane-major layout: a
        // wave's 64 lanes write 64 consecutive words.
        int32_t* red = reinterpret_cast<int32_t*>(smem);
        __syncthreads();
        if (grp != 0) {
            int32_t* mine = red + (grp - 1) * RED_G;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int i = 0; i < TM; ++i)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mine[(((wave * TN + j) * TM + i) * 16 + r) * 64 + lane] = acc[j][i][r];
        }
        __syncthreads();
        if (grp == 0) {
#pragma unroll
            for (int g = 0; g < KGR - 1; ++g)
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int i = 0; i < TM; ++i)
#pragma unroll
                        for (int r = 0; r < 16; ++r)
                            acc[j][i][r] += red[g * RED_G + (((wave * TN + j) * TM + i) * 16 + r) * 64 + lane];
        }
    }

    if constexpr (SPLITK) {
        // Split-K: every split stores its int32 partial tile in its own slice
        // [M x N] of the workspace (after kSplitkCounters tile counters), then
        // counts itself in the tile's counter; the split that arrives last
        // adds the other slices to its accumulators (integer sums: exact in
        // any order), resets the counter to zero for the next call and runs
        // the scale back.  No split waits for another.  N % 4 == 0 (one
        // 16-byte access per lane).  The slices are written and read with the
        // sc0 sc1 cache policy, i.e. through to and from the device's
        // coherence point (the XCDs' L2 caches are not coherent with one
        // another): a split's stores have completed there (vmcnt 0) before it
        // counts itself, and the last split reads only after its count
        // returned, so it sees every other slice without flushing any cache.
        constexpr int kCoherent = 1 | 16;  // sc0 | sc1
        __shared__ int sk_last;
        const int split = blockIdx.y, S = epi.splits;
        int32_t* slices = epi.ws + kSplitkCounters;
        const int64_t MN = (int64_t)M * N;
        auto slice = [&](int o) {
            return __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(slices + o * MN), (short)0,
                                                     (int)(MN * 4), 0x00020000);
        };
        if (KGR == 1 || grp == 0) {  // with wave groups, group 0 holds the sums
            const __amdgpu_buffer_rsrc_t mine = slice(split);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = m0 + wm0 + i * 32 + (lane & 31);
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + wn0 + j * 32 + 8 * g + 4 * (lane >> 5);
                        if (n < N)
                            __builtin_amdgcn_raw_buffer_store_b128(
                                __builtin_bit_cast(v4u, v4i{acc[j][i][4 * g], acc[j][i][4 * g + 1],
                                                            acc[j][i][4 * g + 2], acc[j][i][4 * g + 3]}),
                                mine, (m * N + n) * 4, 0, kCoherent);
                    }
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's slice stores are done
        __syncthreads();
        int* cnt = reinterpret_cast<int*>(epi.ws) + (m0 / BM) * nbn + n0 / BN;
        if (tid == 0) sk_last = atomicAdd(cnt, 1) == S - 1;
        __syncthreads();
        if (!sk_last) return;
        for (int o = 0; o < S && (KGR == 1 || grp == 0); ++o) {
            if (o == split) continue;
            const __amdgpu_buffer_rsrc_t theirs = slice(o);
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int m = m0 + wm0 + i * 32 + (lane & 31);
                if (m >= M) continue;
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int n = n0 + wn0 + j * 32 + 8 * g + 4 * (lane >> 5);
                        if (n < N) {
                            const v4i p = __builtin_bit_cast(
                                v4i, __builtin_amdgcn_raw_buffer_load_b128(theirs, (m * N + n) * 4, 0,
                                                                           kCoherent));
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[j][i][4 * g + e] += p[e];
                        }
                    }
            }
        }
        if (tid == 0) atomicExch(cnt, 0);
    }

    // Epilogue.  Sub-tile (j, i), lane l: token m = i*32 + l%32; elements
    // 4g..4g+3 are output channels 8g + 4*(l/32) + 0..3.
    if constexpr (!HALF_OUT) {
        // 32-bit outputs: a lane's four consecutive channels as one 16-byte
        // store where the row allows it (N % 4 == 0, Y 16-byte aligned)
        if (KGR > 1 && grp != 0) return;  // group 0 holds the sums (no barrier follows)
        const bool vec = (N % 4 == 0) && ((reinterpret_cast<uintptr_t>(Y) & 15) == 0);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm0 + i * 32 + (lane & 31);
            if (m >= M) continue;
            const float sxm = (O == Out::F32) ? sx[m] : 0.0f;
#pragma unroll
            for (int j = 0; j < TN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int n = n0 + wn0 + j * 32 + 8 * g + 4 * (lane >> 5);
                    if (vec && n + 3 < N) {
                        v4i v;
                        if constexpr (O == Out::I32) {
                            v = v4i{acc[j][i][4 * g], acc[j][i][4 * g + 1], acc[j][i][4 * g + 2],
                                    acc[j][i][4 * g + 3]};
                        } else {
#pragma unroll
                            for (int e = 0; e < 4; ++e) {
                                float f;
                                if constexpr (EXT)
                                    f = dequant_ext(acc[j][i][4 * g + e], sxm, sw[n + e],
                                                    epi.bias ? epi.bias[n + e] : 0.0f, epi.relu);
                                else
                                    f = dequant(acc[j][i][4 * g + e], sxm, sw[n + e]);
                                v[e] = __float_as_int(f);
                            }
                        }
                        v4i* dst = reinterpret_cast<v4i*>(static_cast<int*>(Y) + (int64_t)m * N + n);
                        if constexpr (NTS)
                            __builtin_nontemporal_store(v, dst);
                        else
                            *dst = v;
                        continue;
                    }
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (n + e < N) {
                            const float swn = (O == Out::F32) ? sw[n + e] : 0.0f;
                            store_out_ext<O, EXT>(Y, (int64_t)m * N + n + e, acc[j][i][4 * g + e],
                                                  sxm, swn, epi, n + e);
                        }
                }
        }
    } else {
        typedef typename Half<O>::T T;
        float sxv[TM];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
            const int m = m0 + wm0 + i * 32 + (lane & 31);
            sxv[i] = m < M ? sx[m] : 0.0f;
        }
        asm volatile("s_barrier" ::: "memory");  // all waves are done with the operand stages
        // float4 scale loads need a 16-byte aligned row of scales (a batch
        // entry of a product whose N is not a multiple of 4 is not)
        const bool sw_al = (reinterpret_cast<uintptr_t>(sw) & 15) == 0;
        // One 32-channel column block at a time, so that only its scales
        // (four float4) are live next to the accumulators.  With wave groups
        // only group 0 holds sums; every thread takes part in the write-out.
        if (KGR == 1 || grp == 0)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
            float4 swv[4], bv[4];
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int n = n0 + wn0 + j * 32 + 8 * g + 4 * (lane >> 5);
                if (n + 3 < N && sw_al)
                    swv[g] = *reinterpret_cast<const float4*>(sw + n);  // n % 4 == 0
                else
                    swv[g] = make_float4(n < N ? sw[n] : 0.f, n + 1 < N ? sw[n + 1] : 0.f,
                                         n + 2 < N ? sw[n + 2] : 0.f, n + 3 < N ? sw[n + 3] : 0.f);
                if constexpr (EXT) {
                    const float* bb = epi.bias;
                    if (!bb)
                        bv[g] = make_float4(0.f, 0.f, 0.f, 0.f);
                    else if (n + 3 < N)
                        bv[g] = *reinterpret_cast<const float4*>(bb + n);
                    else
                        bv[g] = make_float4(n < N ? bb[n] : 0.f, n + 1 < N ? bb[n + 1] : 0.f,
                                            n + 2 < N ? bb[n + 2] : 0.f, 0.f);
                }
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int ml = wm0 + i * 32 + (lane & 31);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int nl = wn0 + j * 32 + 8 * g + 4 * (lane >> 5);
                    const float4 w4 = swv[g];
                    T o[4];
                    if constexpr (EXT) {
                        const float4 b4 = bv[g];
                        const int rl = epi.relu;
                        o[0] = Half<O>::cvt(dequant_ext(acc[j][i][4 * g + 0], sxv[i], w4.x, b4.x, rl));
                        o[1] = Half<O>::cvt(dequant_ext(acc[j][i][4 * g + 1], sxv[i], w4.y, b4.y, rl));
                        o[2] = Half<O>::cvt(dequant_ext(acc[j][i][4 * g + 2], sxv[i], w4.z, b4.z, rl));
                        o[3] = Half<O>::cvt(dequant_ext(acc[j][i][4 * g + 3], sxv[i], w4.w, b4.w, rl));
                    } else {
                        o[0] = Half<O>::cvt(dequant(acc[j][i][4 * g + 0], sxv[i], w4.x));
                        o[1] = Half<O>::cvt(dequant(acc[j][i][4 * g + 1], sxv[i], w4.y));
                        o[2] = Half<O>::cvt(dequant(acc[j][i][4 * g + 2], sxv[i], w4.z));
                        o[3] = Half<O>::cvt(dequant(acc[j][i][4 * g + 3], sxv[i], w4.w));
                    }
                    *reinterpret_cast<uint2*>(smem + ml * EPI_LD + nl * 2) =
                        *reinterpret_cast<const uint2*>(o);
                }
            }
        }
        __syncthreads();
        // Write-out: 16 bytes (8 outputs) of one row per thread per step.
        constexpr int CH_ROW = BN / 8;
        const bool full_n = (n0 + BN <= N) && (N % 8 == 0);
        for (int c = tid; c < BM * CH_ROW; c += NT) {
            const int row = c / CH_ROW, col = (c % CH_ROW) * 8;
            const int m = m0 + row;
            if (m >= M) continue;
            T* y = static_cast<T*>(Y) + (int64_t)m * N + n0 + col;
            const int8_t* src = smem + row * EPI_LD + col * 2;
            if (full_n) {
                const v4i v = *reinterpret_cast<const v4i*>(src);
                if constexpr (NTS)
                    __builtin_nontemporal_store(v, reinterpret_cast<v4i*>(y));
                else
                    *reinterpret_cast<v4i*>(y) = v;
            } else {
                const T* s16 = reinterpret_cast<const T*>(src);
                for (int e = 0; e < 8; ++e)
                    if (n0 + col + e < N) y[e] = s16[e];
            }
        }
    }
}

// Tile shape for the DMA kernel.  A launch runs in rounds of (CUs x
// workgroups per CU) tiles; a partial last round leaves CUs idle, so the
// shape is chosen to minimise
//     rounds * (tile area * workgroups per CU) / efficiency,
// the time of the rounds in units of one CU's work on a 256 x 256 tile.
// Candidates: 256 x 256 (eight waves, two per SIMD, each a 64-token x
// 128-channel register tile: while one wave of a SIMD waits at its k-tile's
// barrier or for its fragments, the other keeps the matrix core busy; four
// waves of 128 x 128, a third fewer LDS fragment bytes per MFMA but one wave
// per SIMD, measured 3-10% slower: 8192 x 12288 x 49152 4654 -> 4239 us,
// 8192 x 49152 x 12288 4418 -> 4243 us, 2048 x 16384 x 4096 141 -> 132 us),
// 256 x 192 (eight waves of 64 x 96; 512 tiles make exactly two rounds of
// the 2048 x 12288 QKV shape that 256 x 256 covers in one and a half),
// 128 x 128 (two per CU), 256 x 128 (eight waves of 64 x 64) and 128 x 192
// (four waves of 64 x 96), the last two for shapes of about one round, where
// a tile per CU with fewer operand bytes per tile beats two 128 x 128 tiles
// (same-box sweep, 512 tokens: 512 x 12288 x 4096 38.1 -> 35.1 us with
// 128 x 192, 512 x 16384 x 4096 44.3 -> 41.2 us with 256 x 128; 2048 x 4096 x
// 16384 150.4 -> 138.8 us with 256 x 128).  All use BK 128 and two operand
// stages.  The efficiencies are relative throughputs per unit of tile area
// fitted to those measurements.  (K <= 128 bypasses the model: see
// launch_dma.)
struct TileCfg {
    int bm, bn, per_cu;
    double eff;
};
constexpr int kNumTiles = 5;
constexpr TileCfg kTiles[kNumTiles] = {{256, 256, 1, 1.0}, {256, 192, 1, 0.81}, {128, 128, 2, 0.78},
                                       {256, 128, 1, 0.80}, {128, 192, 1, 0.70}};

int cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

int pick_tile(int M, int N, int batch) {
    const int cus = cu_count();
    int best = 0;
    double best_cost = 0.0;
    for (int c = 0; c < kNumTiles; ++c) {
        const TileCfg& t = kTiles[c];
        const int64_t tiles = (int64_t)((M + t.bm - 1) / t.bm) * ((N + t.bn - 1) / t.bn) * batch;
        const int64_t slots = (int64_t)cus * t.per_cu;
        const int64_t rounds = (tiles + slots - 1) / slots;
        const double cost = (double)rounds * t.bm * t.bn * t.per_cu / t.eff;
        if (c == 0 || cost < best_cost) {
            best = c;
            best_cost = cost;
        }
    }
    return best;
}

template <Out O, bool PACKED, bool EXT>
hipError_t launch_dma(const int8_t* xq, const float* sx, const int8_t* w, const float* sw, int M,
                      int N, int K, void* y, Epi epi, hipStream_t s, int batch = 1) {
    auto tiles = [&](int bm, int bn) { return ((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (K <= 128) {
        // One k-tile (attention scores Q K^T over head_dim 128): the launch is
        // bound by writing the outputs; one operand stage keeps the LDS at
        // 34 KB, so four workgroups share a CU and one's loads overlap
        // another's output stores (measured 29% faster than two per CU), and
        // the outputs are stored non-temporally (another 20%: they are far
        // larger than the caches and are not read again by this launch).
        hipLaunchKernelGGL((gemm_dma_kernel<128, 128, 128, 64, 64, O, PACKED, 4, 1, EXT, true>),
                           dim3(tiles(128, 128), batch), dim3(256), 0, s, xq, w, sx, sw, y, M, N, K,
                           epi);
        return hipGetLastError();
    }
    {
        // Tiles numbering at most one per CU: each workgroup runs its whole K
        // loop alone on its CU, bound by the latency of its operand loads, so
        // 64-deep k-tiles go in a four-stage ring (twice the bytes in flight
        // per workgroup); 128 x 64 tiles while they are few enough, else 128
        // x 128.  Measured (packed weights, weights streamed from HBM):
        // 12288 x 4096 at 65 tokens 23.7 -> 19.1 us, at 200 tokens 27.2 ->
        // 24.0; 4096 x 8192 at 200 tokens 49.2 -> 33.8; 5120 x 5120 at 256
        // tokens 32.7 -> 25.6; 4096 x 16384 at 65 tokens 82.5 -> 62.1, at 768
        // tokens 106 -> 85; 8192 x 28672 at 384 tokens 190 -> 152; 12288 x
        // 49152 at 200 tokens 299 -> 253.  With more tiles than CUs the
        // deeper ring loses (8192 x 28672 at 768 tokens 233 -> 274 us).
        // From K = 2048 the workgroup holds two groups of four waves, each
        // with its own ring over half of K (twice the loads in flight per CU,
        // no partial sums leave the workgroup).  Same-box sweeps (packed
        // weights): 4096 x 16384 at 512 / 256 / 65 tokens 70.2 / 64.3 / 64.3 ->
        // 61.7 / 57.9 / 59.1 us; 4096 x 8192 at 512 tokens 35.1 -> 29.4; 8192 x
        // 28672 at 130 tokens 112.0 -> 101.9; 12288 x 49152 at 65 tokens 194.2
        // -> 165.7; 12288 x 4096 at 65 tokens 18.2 -> 14.7; 4096 x 4096 at 512
        // tokens 19.5 -> 16.9; 4096 x 2048 at 100 tokens 10.1 -> 8.7; 128 x 128
        // tiles: 8192 x 8192 at 512 tokens 50.7 -> 46.7, 8192 x 4096 29.1 ->
        // 27.4 us.
        // In the 128 x 64 form, 128-deep k-tiles in three stages per group
        // (144 KB of LDS) where K % 256 == 0: whole 128-byte activation row
        // pieces per load instead of halves, and more bytes in flight (same
        // box, packed weights, 64-deep four-stage -> 128-deep three-stage
        // rings): 4096 x 16384 at 512 / 256 / 65 tokens 62.9 / 58.0 / 45.4 ->
        // 53.1 / 44.9 / 41.8 us; 12288 x 49152 at 65 tokens 167.6 -> 145.2;
        // 4096 x 4096 at 512 tokens 17.3 -> 16.1; 12288 x 4096 at 65 tokens
        // 14.8 -> 14.6.  Four groups of 64-deep rings measured no better than
        // two (4096 x 16384 at 512 tokens 63.9 against 63.5 us).
        const int64_t cus = cu_count();
        if ((int64_t)tiles(128, 64) * batch <= cus) {
            if (K >= 2048 && K % 256 == 0)
                hipLaunchKernelGGL(
                    (gemm_dma_kernel<128, 64, 128, 64, 32, O, PACKED, 1, 3, EXT, false, false, 2>),
                    dim3(tiles(128, 64), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K, epi);
            else if (K >= 2048)
                hipLaunchKernelGGL(
                    (gemm_dma_kernel<128, 64, 64, 64, 32, O, PACKED, 1, 4, EXT, false, false, 2>),
                    dim3(tiles(128, 64), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K, epi);
            else
                hipLaunchKernelGGL((gemm_dma_kernel<128, 64, 64, 64, 32, O, PACKED, 3, 4, EXT>),
                                   dim3(tiles(128, 64), batch), dim3(256), 0, s, xq, w, sx, sw, y,
                                   M, N, K, epi);
            return hipGetLastError();
        }
        if ((int64_t)tiles(128, 128) * batch <= cus) {
            if (K >= 2048)
                hipLaunchKernelGGL(
                    (gemm_dma_kernel<128, 128, 64, 64, 64, O, PACKED, 1, 4, EXT, false, false, 2>),
                    dim3(tiles(128, 128), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K, epi);
            else
                hipLaunchKernelGGL((gemm_dma_kernel<128, 128, 64, 64, 64, O, PACKED, 2, 4, EXT>),
                                   dim3(tiles(128, 128), batch), dim3(256), 0, s, xq, w, sx, sw, y,
                                   M, N, K, epi);
            return hipGetLastError();
        }
        // 129-256 rows on wide, deep layers (K >= 8192, more 128-row tiles
        // than CUs): one row of 256 x 128 tiles when they number at most one
        // per CU -- up to 191 rows in the four-stage ring, from 192 rows as
        // eight waves of 64 x 64 with BK 128 in two stages -- else 128 x 192
        // tiles (four waves of 64 x 96, BK 128, two stages).  Same-box sweep
        // (packed weights): 28672 x 8192 at 130 / 200 / 256 tokens 72.5 /
        // 79.3 / 80.4 us (the ring 72.5 / 80.8 / 87.2); 49152 x 12288 at 130
        // / 200 / 256 tokens 153.8 / 164.8 / 166.5 us and 36864 x 12288 at
        // 256 tokens 148.9 us with 128 x 192, where a row of 256 x 256 tiles
        // in the ring took 175.3 / 191.6 / 204.7 and 188.6 us.  Not for more
        // rows or K = 4096 (12288 x 4096 at 512 tokens: the ring 39 -> 43 us).
        if (K >= 8192 && M > 128 && M <= 256) {
            if ((int64_t)tiles(256, 128) * batch <= cus) {
                if (M >= 192)
                    hipLaunchKernelGGL((gemm_dma_kernel<256, 128, 128, 64, 64, O, PACKED, 1, 2, EXT>),
                                       dim3(tiles(256, 128), batch), dim3(512), 0, s, xq, w, sx, sw,
                                       y, M, N, K, epi);
                else
                    hipLaunchKernelGGL((gemm_dma_kernel<256, 128, 64, 128, 64, O, PACKED, 1, 4, EXT>),
                                       dim3(tiles(256, 128), batch), dim3(256), 0, s, xq, w, sx, sw,
                                       y, M, N, K, epi);
                return hipGetLastError();
            }
            hipLaunchKernelGGL((gemm_dma_kernel<128, 192, 128, 64, 96, O, PACKED, 1, 2, EXT>),
                               dim3(tiles(128, 192), batch), dim3(256), 0, s, xq, w, sx, sw, y, M, N,
                               K, epi);
            return hipGetLastError();
        }
    }
    if (M <= 256) {
        // Few token rows and more tiles than CUs: 128-row tiles still leave
        // CUs idle on all but the widest layers, so the tiles are narrower
        // (128 x 64, four per CU).
        // Up to 128 rows: 64-deep k-tiles in a three-stage ring (measured
        // 12288 x 4096 at 65 tokens 23.1 -> 18.3 us, 4096 x 16384 98 -> 77);
        // up to 256 rows: 128-deep, two stages (25.3 -> 22.7 us).
        if (M <= 128)
            hipLaunchKernelGGL((gemm_dma_kernel<128, 64, 64, 64, 32, O, PACKED, 4, 3, EXT>),
                               dim3(tiles(128, 64), batch), dim3(256), 0, s, xq, w, sx, sw, y, M, N,
                               K, epi);
        else
            hipLaunchKernelGGL((gemm_dma_kernel<128, 64, 128, 64, 32, O, PACKED, 4, 2, EXT>),
                               dim3(tiles(128, 64), batch), dim3(256), 0, s, xq, w, sx, sw, y, M, N,
                               K, epi);
        return hipGetLastError();
    }
    switch (pick_tile(M, N, batch)) {
        case 0:
            hipLaunchKernelGGL((gemm_dma_kernel<256, 256, 128, 64, 128, O, PACKED, 1, 2, EXT>),
                               dim3(tiles(256, 256), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K,
                               epi);
            break;
        case 1:
            hipLaunchKernelGGL((gemm_dma_kernel<256, 192, 128, 64, 96, O, PACKED, 1, 2, EXT>),
                               dim3(tiles(256, 192), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K,
                               epi);
            break;
        case 2:
            hipLaunchKernelGGL((gemm_dma_kernel<128, 128, 128, 64, 64, O, PACKED, 2, 2, EXT>),
                               dim3(tiles(128, 128), batch), dim3(256), 0, s, xq, w, sx, sw, y, M, N, K,
                               epi);
            break;
        case 3:
            // 256 x 128 tiles in one round (at most one per CU): a third
            // 128-deep stage (144 KB of LDS) keeps more bytes in flight
            // (16384 x 4096 at 512 tokens 40.0 -> 38.8 us in a same-box
            // sweep); with more rounds the two-stage form
            if ((int64_t)tiles(256, 128) * batch <= cu_count())
                hipLaunchKernelGGL((gemm_dma_kernel<256, 128, 128, 64, 64, O, PACKED, 1, 3, EXT>),
                                   dim3(tiles(256, 128), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N,
                                   K, epi);
            else
                hipLaunchKernelGGL((gemm_dma_kernel<256, 128, 128, 64, 64, O, PACKED, 1, 2, EXT>),
                                   dim3(tiles(256, 128), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N,
                                   K, epi);
            break;
        default:
            // 128 x 192 tiles in one round (at most one per CU) from K = 2048:
            // two groups of four waves over the two halves of K, all 160 KB
            // of LDS (12288 x 4096 at 512 / 400 tokens 35.8 / 33.8 -> 34.0 /
            // 32.5 us in a same-box sweep; with more tiles, or for 256 x 128
            // tiles, the groups lose)
            if (K >= 2048 && (int64_t)tiles(128, 192) * batch <= cu_count())
                hipLaunchKernelGGL(
                    (gemm_dma_kernel<128, 192, 128, 64, 96, O, PACKED, 1, 2, EXT, false, false, 2>),
                    dim3(tiles(128, 192), batch), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K, epi);
            else
                hipLaunchKernelGGL((gemm_dma_kernel<128, 192, 128, 64, 96, O, PACKED, 1, 2, EXT>),
                                   dim3(tiles(128, 192), batch), dim3(256), 0, s, xq, w, sx, sw, y,
                                   M, N, K, epi);
            break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Fragment-packed weights.  Row block b (16 output channels) and 64-byte
// k-group c form one 1 KB block at ((b * KG) + c) * 1024 whose 16-byte piece l
// holds channel b*16 + l%16, bytes c*64 + (l/16)*16 .. +16 -- exactly the
// 16 x 64 operand of v_mfma_i32_16x16x64_i8, so a wave reads one fragment as
// one contiguous kilobyte.  KG = K / 64; rows past N are zero.
__global__ __launch_bounds__(256) void pack_weight_kernel(const int8_t* __restrict__ wq, int N, int K,
                                                          int8_t* __restrict__ wp) {
    const int KG = K / 64, NB = (N + 15) / 16;
    const int64_t pieces = (int64_t)NB * KG * 64;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pieces;
         i += (int64_t)gridDim.x * 256) {
        const int l = (int)(i & 63);
        const int64_t blk = i >> 6;
        const int c = (int)(blk % KG), b = (int)(blk / KG);
        const int n = b * 16 + (l & 15);
        v4i v = {0, 0, 0, 0};
        if (n < N) v = *reinterpret_cast<const v4i*>(wq + (int64_t)n * K + c * 64 + (l >> 4) * 16);
        *reinterpret_cast<v4i*>(wp + i * 16) = v;
    }
}

// 17-64 tokens: the few-token kernels read every activation fragment once per
// 16-channel block, so on wide layers (N >= 12288) the activation traffic
// outgrows the weights; there the 128 x 64 tiles win from about M * N >=
// 32 x 12288 (measured: 12288 x 4096 at 32 tokens 20.1 -> 18.5 us, at 64
// tokens 32.7 -> 18.5 us; 16384 x 4096 at 64 tokens 42.7 -> 23.0 us; 28672 x
// 8192 at 32 tokens 76.4 -> 56.1 us; narrow, deep layers such as 4096 x 16384
// keep the few-token kernels at every M <= 64).
bool few_tokens_to_tiles(int M, int N) {
    return M > 16 && N >= 12288 && (int64_t)M * N >= 32 * 12288;
}

template <Out O, bool EXT>
hipError_t gemm_packed_dispatch(const int8_t* xq, const float* sx, const int8_t* wp,
                                const float* sw, int M, int N, int K, void* y, Epi epi,
                                hipStream_t s) {
    if (M <= 64 && !few_tokens_to_tiles(M, N))
        return launch_skinny(xq, sx, wp, sw, M, N, K, y, O, true, s, epi);
    return launch_dma<O, true, EXT>(xq, sx, wp, sw, M, N, K, y, epi, s);
}

template <Out O, bool KVEC, bool EXT>
hipError_t gemm_dispatch(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw,
                         int M, int N, int K, void* y, Epi epi, hipStream_t s, int batch) {
    if (M <= 64 && !(KVEC && K % 128 == 0 && few_tokens_to_tiles(M, N))) {
        return launch_skinny(xq, sx, wq, sw, M, N, K, y, O, false, s, epi, batch);
    } else if (KVEC && K % 128 == 0) {
        return launch_dma<O, false, EXT>(xq, sx, wq, sw, M, N, K, y, epi, s, batch);
    } else {
        constexpr int BM = 256, BN = 256, BK = 64, WM = 128, WN = 64, SWS = 1;
        const int tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
        hipLaunchKernelGGL((gemm_tiled_kernel<BM, BN, BK, WM, WN, SWS, O, KVEC, EXT>), dim3(tiles, batch),
                           dim3((BM / WM) * (BN / WN) * 64), 0, s, xq, wq, sx, sw, y, M, N, K, epi);
    }
    return hipGetLastError();
}

template <Out O, bool EXT>
hipError_t gemm_out(const int8_t* xq, const float* sx, const int8_t* wq, const float* sw, int M,
                    int N, int K, void* y, Epi epi, hipStream_t s, int batch) {
    if (K % 16 == 0) return gemm_dispatch<O, true, EXT>(xq, sx, wq, sw, M, N, K, y, epi, s, batch);
    return gemm_dispatch<O, false, EXT>(xq, sx, wq, sw, M, N, K, y, epi, s, batch);
}

}  // namespace

int device_cu_count() { return cu_count(); }

int64_t packed_weight_bytes(int64_t N, int64_t K) { return ((N + 15) / 16) * (K / 64) * 1024; }

hipError_t launch_pack_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* wp, hipStream_t s) {
    const int64_t pieces = packed_weight_bytes(N, K) / 16;
    int64_t blocks = (pieces + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(pack_weight_kernel, dim3((unsigned)blocks), dim3(256), 0, s, wq, (int)N,
                       (int)K, wp);
    return hipGetLastError();
}

hipError_t launch_gemm_packed(const int8_t* xq, const float* x_scale, const int8_t* wp,
                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                              Out out, hipStream_t s, Epi epi) {
    const int m = (int)M, n = (int)N, k = (int)K;
#define SQ_PK(O, E) return gemm_packed_dispatch<O, E>(xq, x_scale, wp, w_scale, m, n, k, y, epi, s)
    const bool ext = epi.on();
    switch (out) {
        case Out::I32: SQ_PK(Out::I32, false);
        case Out::F16: if (ext) SQ_PK(Out::F16, true); SQ_PK(Out::F16, false);
        case Out::BF16: if (ext) SQ_PK(Out::BF16, true); SQ_PK(Out::BF16, false);
        case Out::F32: if (ext) SQ_PK(Out::F32, true); SQ_PK(Out::F32, false);
    }
#undef SQ_PK
    return hipErrorInvalidValue;
}

// Split-K: 128 x 64 tiles, one workgroup of two wave groups per CU (each
// group over half of its split's K range, 128-deep k-tiles in three stages,
// as the plain few-tile form).  Workspace layout: a fixed block of
// kSplitkCounters tile counters (only ever zero between calls, whatever the
// shape), then the splits' int32 slices [S][M][N].  K is split for deep
// layers (K >= 8192, K % 256 == 0) whose 128 x 64 output tiles number at
// most half the CUs, in 2, 4 or 8 ranges of at least 2048, so that tiles x
// splits fills at most one workgroup per CU.  Measured against the plain
// entry point (packed weights, the 128 x 64 few-tile form; same box): 4096 x
// 16384 (N x K) at 65 / 128 tokens 41.6 / 44.7 -> 28.8 / 32.7 us; 4096 x
// 12288 at 128 tokens 32.8 -> 25.0; 4096 x 8192 at 100 tokens 22.7 -> 19.6;
// 8192 x 28672 at 65 tokens 78.8 -> 78.4 us.  Layers with more tiles lose
// (4096 x 16384 at 512 tokens, one tile per CU: 55.0 plain, 93.3 in two
// splits) and are not split; the earlier split form (128 x 128 tiles, two
// workgroups of four waves per CU) took 49.0 / 50.7 / 42.3 / 23.9 / 78.3 us
// on the shapes above.
int64_t splitk_tiles(int64_t M, int64_t N) { return ((M + 127) / 128) * ((N + 63) / 64); }

int splitk_splits(int64_t M, int64_t N, int64_t K) {
    if (M <= 64 || N % 4 != 0 || K % 256 != 0 || K < 8192) return 1;
    const int64_t tiles = splitk_tiles(M, N), cus = cu_count();
    if (tiles > kSplitkCounters || 2 * tiles > cus) return 1;
    int S = 1;
    while (S < 8 && tiles * (2 * S) <= cus && K % (2 * S * 256) == 0 && K / (2 * S) >= 2048) S *= 2;
    return S;
}

int64_t splitk_workspace_bytes(int64_t M, int64_t N, int64_t K) {
    const int S = splitk_splits(M, N, K);
    if (S == 1) return 0;
    return 4 * (int64_t)kSplitkCounters + (4 * S * M * N + 255) / 256 * 256;
}

namespace {
template <Out O, bool PACKED>
hipError_t splitk_out(const int8_t* xq, const float* sx, const int8_t* w, const float* sw, int M,
                      int N, int K, void* y, int S, int32_t* ws, hipStream_t s) {
    Epi epi;
    epi.ws = ws;
    epi.splits = S;
    const int tiles = (int)splitk_tiles(M, N);
    hipLaunchKernelGGL((gemm_dma_kernel<128, 64, 128, 64, 32, O, PACKED, 1, 3, false, false, true, 2>),
                       dim3(tiles, S), dim3(512), 0, s, xq, w, sx, sw, y, M, N, K, epi);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm_splitk(const int8_t* xq, const float* x_scale, const int8_t* w,
                              const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                              Out out, bool packed, int32_t* ws, hipStream_t s) {
    const int S = splitk_splits(M, N, K);
    if (S == 1)
        return packed ? launch_gemm_packed(xq, x_scale, w, w_scale, M, N, K, y, out, s)
                      : launch_gemm(xq, x_scale, w, w_scale, M, N, K, y, out, s);
    const int m = (int)M, n = (int)N, k = (int)K;
#define SQ_SK(O) return packed ? splitk_out<O, true>(xq, x_scale, w, w_scale, m, n, k, y, S, ws, s) \
                               : splitk_out<O, false>(xq, x_scale, w, w_scale, m, n, k, y, S, ws, s)
    switch (out) {
        case Out::F16: SQ_SK(Out::F16);
        case Out::BF16: SQ_SK(Out::BF16);
        case Out::F32: SQ_SK(Out::F32);
        default: break;
    }
#undef SQ_SK
    return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// Split-K with the library's own scratch, for callers that cannot allocate a
// workspace (graph capture, serving loops).  The scratch is one static device
// array per GPU, sized for every split the library takes on a 256-CU device:
// the tiles x splits of a split launch number at most the CUs (tiles * S <=
// CUs), and a tile holds 128 x 64 int32 sums, so the slices take at most
// 256 * 8192 * 4 bytes = 8 MiB there.  The array's name is only a host-side
// stand-in: its device address comes from hipGetSymbolAddress, once per
// device.
constexpr int64_t kNoallocSlices = 8 << 20;
constexpr int64_t kNoallocBytes = 4 * (int64_t)kSplitkCounters + kNoallocSlices;
static __device__ __align__(256) int32_t scratch[kNoallocBytes / 4];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
int32_t* g_scratch_ptr[kMaxDevices] = {nullptr};

__global__ __launch_bounds__(256) void zero_counters_kernel(int32_t* c, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) c[i] = 0;
}
}  // namespace

int64_t noalloc_scratch_bytes() { return kNoallocBytes; }

hipError_t launch_gemm_splitk_noalloc(const int8_t* xq, const float* x_scale, const int8_t* wp,
                                      const float* w_scale, int64_t M, int64_t N, int64_t K,
                                      void* y, Out out, hipStream_t s) {
    const int S = splitk_splits(M, N, K);
    if (S == 1) return launch_gemm_packed(xq, x_scale, wp, w_scale, M, N, K, y, out, s);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int32_t* ws = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mu);
        if (!g_scratch_ptr[dev]) {
            void* p = nullptr;
            e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
            if (e != hipSuccess) return e;
            g_scratch_ptr[dev] = static_cast<int32_t*>(p);
        }
        ws = g_scratch_ptr[dev];
    }
    // the tile counters must start at zero: every split launch leaves them so,
    // but the array keeps whatever the last call on this GPU left, so they are
    // cleared by a small kernel (not a memset node, which graph capture would
    // record) ahead of every split launch
    const int tiles = (int)splitk_tiles(M, N);
    hipLaunchKernelGGL(zero_counters_kernel, dim3((tiles + 255) / 256), dim3(256), 0, s, ws, tiles);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_gemm_splitk(xq, x_scale, wp, w_scale, M, N, K, y, out, true, ws, s);
}

hipError_t launch_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq,
                       const float* w_scale, int64_t M, int64_t N, int64_t K, void* y, Out out,
                       hipStream_t s, Epi epi, int batch) {
    const int m = (int)M, n = (int)N, k = (int)K;
#define SQ_G(O, E) return gemm_out<O, E>(xq, x_scale, wq, w_scale, m, n, k, y, epi, s, batch)
    const bool ext = epi.on();
    switch (out) {
        case Out::I32: SQ_G(Out::I32, false);
        case Out::F16: if (ext) SQ_G(Out::F16, true); SQ_G(Out::F16, false);
        case Out::BF16: if (ext) SQ_G(Out::BF16, true); SQ_G(Out::BF16, false);
        case Out::F32: if (ext) SQ_G(Out::F32, true); SQ_G(Out::F32, false);
    }
#undef SQ_G
    return hipErrorInvalidValue;
}

}  // namespace sq
