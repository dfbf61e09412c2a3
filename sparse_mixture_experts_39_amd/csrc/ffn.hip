// Expert FFN stage for gfx950: ragged grouped GEMMs on the matrix cores.
//
// Every expert e owns the row range [off[e], off[e+1]) of the permuted
// activations; the layer merges the per-expert token groups into large matrix
// products instead of running one small product per token (CS336 lecture 4
// notes, section 10: tokens of several experts on one device become one big
// matrix multiply; Lecture29, "Batch size and throughput": bigger expert
// batches raise arithmetic intensity).  The experts are
//   SwiGLU: h = SiLU(a W1^T) * (a W3^T), y = h W2^T (Lecture29, "Dense baseline")
//   ReLU:   h = relu(a W1^T),            y = h W2^T (Shazeer notes, section 2.2)
// with fp32 accumulation and h, y stored in the activation dtype.
//
// Kernel design (one kernel template, k_grouped_gemm):
//   * 256 threads = 4 waves in a 2x2 grid; a block computes a BM x BN tile,
//     each wave a (BM/2) x (BN/2) tile of MFMA blocks.
//   * MFMA operand order: the weights are source 0 and the activations
//     source 1, so the accumulator lanes hold 4 consecutive output columns of
//     one row and the epilogue stores 8 (bf16) or 16 (fp32) bytes per lane.
//   * 16x16 MFMA blocks for both dtypes: bf16 uses v_mfma_f32_16x16x32_bf16
//     (one 16-byte fragment per lane = 8 k values, a half slice is one
//     k-step), fp32 four v_mfma_f32_16x16x4_f32 per 16-byte fragment.  With
//     twice as many, half as long MFMAs as the 32x32x16 form the same fenced
//     schedule (below) keeps the matrix unit busier (4-5 % on the Mixtral
//     GEMMs).  The k positions inside a fragment are the same for both
//     operands, so the product is exact whatever order the unit visits them.
//   * K is staged through LDS in slices of 128-byte rows (64 bf16 / 32 fp32
//     values): one direct-to-LDS buffer load (buffer_load_dwordx4 ... lds)
//     of a wave moves 8 rows x 128 bytes, i.e. whole 128-byte lines, with no
//     VGPR staging.  A and B slices live in two rings of NA and NB slots that
//     fill the 160 KB of LDS; one barrier per slice; the loads of later
//     slices are in flight while the MFMAs consume the current one.
//     16-byte chunks are XOR swizzled by (r >> 1) & 7 so the fragment reads of
//     16 consecutive rows at one logical chunk hit distinct banks.
//   * Ragged M: the tile plan holds prefix sums of ceil(M_e / BM); a block
//     finds its expert by binary search, so no host synchronisation is
//     needed.  Rows past the expert's end are loaded from its last row and
//     never stored.
//   * Tile order: block ids are dealt round-robin to the 8 XCDs, so the
//     linear tile index is remapped to give each XCD a contiguous range;
//     inside an expert, tiles go in groups of 8 N-tiles with M fastest, so
//     blocks running together on one XCD share weight panels and activation
//     panels in that XCD's L2.
//   * SwiGLU is fused: a BN-row weight tile interleaves 16-row blocks of W1
//     and W3 for the same BN/2 hidden units, so a wave holds the gate and up
//     accumulators of the same (row, unit) in one lane and writes h directly.
//   * Split-K tail: a mostly empty last round of tiles is cut into K ranges
//     (second launch, fp32 partials) and reduced in order by k_split_fixup.
//   * Remainder tiles: with 256-row tiles, an expert's last <= 128 rows go to
//     a further launch of 64-row tiles (kRemBM), so a row count just past a
//     multiple of 256 does not pay for a whole padded tile.
#include <algorithm>
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace moe {

// Epilogues.  The _SAVE forms also store the pre-activations (a, and u for
// SwiGLU) to C2 (row stride ldc2; u at column offset N), which a training
// forward keeps for the backward.
enum { EPI_STORE = 0, EPI_RELU = 1, EPI_SWIGLU = 2, EPI_SWIGLU_SAVE = 3, EPI_RELU_SAVE = 4 };

constexpr bool epi_swiglu(int e) { return e == EPI_SWIGLU || e == EPI_SWIGLU_SAVE; }
constexpr bool epi_relu(int e) { return e == EPI_RELU || e == EPI_RELU_SAVE; }
constexpr bool epi_save(int e) { return e == EPI_SWIGLU_SAVE || e == EPI_RELU_SAVE; }

struct GemmParams {
    const void* A;
    int64_t lda;
    const void* B0;
    const void* B1;
    int64_t bstride;        // elements between experts in B0 / B1
    void* C;
    int64_t ldc;
    int N;                  // output columns
    int K;
    int E;
    int NT;                 // N tiles
    int nk;                 // K slices of 128-byte rows
    const int32_t* offsets; // [E+1]
    const int32_t* plan;    // [E+1] tile prefix over experts, then full, split, tail
    float* partial;         // split-K partial accumulators
    void* C2;               // pre-activations (_SAVE epilogues)
    int64_t ldc2;
    int rem_bm;             // > 0: row tiles start after the expert's first
                            // floor(M_e / rem_bm) * rem_bm rows (remainder launch)
};

// First row of row tile mt of expert e.  The remainder launch covers the rows
// left after the expert's whole tiles of the main launch (rem_bm rows each).
__device__ __forceinline__ int tile_row0(const GemmParams& p, int e, int mt, int BM) {
    int base = p.offsets[e];
    if (p.rem_bm > 0) base += (p.offsets[e + 1] - base) / p.rem_bm * p.rem_bm;
    return base + mt * BM;
}

// Work decomposition.  The plan lists ceil(M_e / BM) row tiles per expert,
// each with NT column tiles, T tiles in all.  When the last round of tiles
// would leave the chip mostly idle (T mod kSplitUnits <= kSplitUnits / 2),
// those `tail` tiles are cut into `split` K ranges each, one block per range:
// every block writes its fp32 partial accumulators, and k_split_fixup adds
// the ranges of a tile in a fixed order and applies the epilogue, so results
// do not depend on timing.  kSplitUnits is the CU count of the target chip.
constexpr int kSplitUnits = 256;
constexpr int kMaxSplit = 16;

// Remainder tiles.  With 256-row tiles an expert whose row count lies just
// past a multiple of 256 pays a whole tile of padding rows for a few real
// ones.  When at most kRemThr rows are left after an expert's whole tiles,
// they go to a second launch of kRemBM-row tiles (ceil(r / kRemBM) of them,
// a quarter of the MFMA work of a 256-row tile each) instead.  Each launch
// has its own plan, and its own split-K tail.
#ifndef MOE_GEMM_REM
#define MOE_GEMM_REM 1
#endif
constexpr int kRemBM = 64;
constexpr int kRemThr = 128;

// Tile L of the natural order: experts in order; inside an expert, groups of
// NG column tiles, row tiles fastest inside a group.
__device__ __forceinline__ void decode_tile(const GemmParams& p, int L, int& e, int& mt, int& nt) {
    const int NT = p.NT;
    int lo = 0, hi = p.E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.plan[mid] * NT <= L) lo = mid; else hi = mid;
    }
    e = lo;
    const int tiles_e = p.plan[e + 1] - p.plan[e];
    const int local = L - p.plan[e] * NT;
    constexpr int NG = 8;
    const int grp = local / (tiles_e * NG);
    const int inside = local - grp * tiles_e * NG;
    mt = inside % tiles_e;
    nt = grp * NG + inside / tiles_e;
}

// XOR swizzle of the eight 16-byte chunks of a 128-byte LDS row.  LDS serves
// 16 lanes of a 16-byte read per pass: rows r .. r+15 at one logical chunk
// then cover every (row parity, physical chunk) pair, i.e. 16 distinct
// 16-byte bank groups.  Depends on r mod 16 only.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Ring depths of the A and B slices.  Batch j (issued after the barrier of
// slice j) loads A slice j + NA and B slice j + NB, in that order; before that
// barrier a wave waits until slice j + 1 has landed, which leaves `wait`
// of its own loads in flight (`wait0` before the first slice).  NB is NA or
// NA + 1; the depths maximise `wait` within 160 KB of LDS.
struct RingDepth {
    int na, nb, wait, wait0, bytes;
};
constexpr RingDepth ring_depth(int BM, int BN) {
    const int SA = BM * 128, SB = BN * 128, ga = BM / 32, gb = BN / 32;
    RingDepth best{2, 2, 0, ga + gb, 2 * (SA + SB)};
    for (int na = 2; na <= 16; ++na)
        for (int nb = na; nb <= na + 1; ++nb) {
            const int bytes = na * SA + nb * SB;
            if (bytes > 160 * 1024) continue;
            const int w = (nb == na ? 0 : gb) + (na - 2) * (ga + gb);
            if (w > best.wait || (w == best.wait && bytes < best.bytes)) best = {na, nb, w, w + ga + gb, bytes};
        }
    return best;
}

// s_waitcnt vmcnt(n) for a compile-time n (other counters left alone).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier that does not drain outstanding global loads (unlike
// __syncthreads, whose fence waits for every load): LDS reads are drained
// first, the compiler may not move memory operations across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Epilogue of one wave's accumulators (shared by the GEMM and the split-K
// fixup).
template <bool BF16, int BM, int BN, int EPI>
struct GemmEpilogue {
    static constexpr int WM = BM / 2, WN = BN / 2;
    static constexpr int MB = 16;              // 16x16 MFMA blocks
    static constexpr int FM = WM / MB, FN = WN / MB;
    static constexpr int RA = 4;               // accumulator registers per MFMA block
    typedef floatx4_t acc_t;

    // float4 index of partial element (i, j, 4*r4 .. 4*r4+3) of wave w, unit u
    __device__ static int64_t partial_index(int u, int w, int i, int j, int r4, int lane) {
        return (((((int64_t)u * 4 + w) * FN + i) * FM + j) * (RA / 4) + r4) * 64 + lane;
    }

    __device__ static void store_partial(const GemmParams& p, const acc_t (&acc)[FN][FM], int u, int w, int lane) {
        float4* dst = (float4*)p.partial;
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r4 = 0; r4 < RA / 4; ++r4)
                    dst[partial_index(u, w, i, j, r4, lane)] =
                        make_float4(acc[i][j][4 * r4], acc[i][j][4 * r4 + 1], acc[i][j][4 * r4 + 2], acc[i][j][4 * r4 + 3]);
    }

    // Column groups of the epilogue: the 16-row blocks i of the wave's B tile
    // are independent, except that SwiGLU pairs block 2p (gate) with block
    // 2p+1 (up).
    static constexpr int IG = epi_swiglu(EPI) ? 2 : 1;

    // Output of blocks i0 .. i0+IG-1 (acc[0 .. IG-1]).  In a 16x16 block,
    // lane l, element t holds D[n = 4(l/16) + t][m = l % 16]: a lane owns 4
    // consecutive output columns of one row and stores them at once.
    __device__ static void store_cols(const GemmParams& p, const acc_t (*acc)[FM], int i0, int row0, int rows, int nt,
                                      int wm, int wn, int lane) {
        auto store4_to = [&](void* dst, int64_t ld, int m, int64_t col, const float* v) {
            const int64_t o = (int64_t)(row0 + m) * ld + col;
            if constexpr (BF16) {
                uint2 w;
                w.x = pack_bf16x2(v[0], v[1]);
                w.y = pack_bf16x2(v[2], v[3]);
                *(uint2*)((uint16_t*)dst + o) = w;
            } else {
                *(float4*)((float*)dst + o) = make_float4(v[0], v[1], v[2], v[3]);
            }
        };
        auto store4 = [&](int m, int64_t col, const float* v) { store4_to(p.C, p.ldc, m, col, v); };
        auto silu_mul = [](float gt, float up) { return gt * __builtin_amdgcn_rcpf(1.0f + __expf(-gt)) * up; };
        {
            const int lg = lane >> 4;
#pragma unroll
            for (int j = 0; j < FM; ++j) {
                const int m = wm * WM + j * 16 + (lane & 15);
                if (m >= rows) continue;
                if constexpr (epi_swiglu(EPI)) {
                    const int fblock = (wn * FN + i0) >> 1;        // 16-row blocks alternate gate / up
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) v[t] = silu_mul(acc[0][j][t], acc[1][j][t]);
                    const int64_t col = (int64_t)nt * (BN / 2) + fblock * 16 + 4 * lg;
                    store4(m, col, v);
                    if constexpr (epi_save(EPI)) {
                        float a[4], u[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            a[t] = acc[0][j][t];
                            u[t] = acc[1][j][t];
                        }
                        store4_to(p.C2, p.ldc2, m, col, a);
                        store4_to(p.C2, p.ldc2, m, p.N + col, u);
                    }
                } else {
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        float x = acc[0][j][t];
                        if constexpr (epi_relu(EPI)) x = fmaxf(x, 0.0f);
                        v[t] = x;
                    }
                    const int64_t col = (int64_t)nt * BN + wn * WN + i0 * 16 + 4 * lg;
                    store4(m, col, v);
                    if constexpr (epi_save(EPI)) {
                        float a[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) a[t] = acc[0][j][t];
                        store4_to(p.C2, p.ldc2, m, col, a);
                    }
                }
            }
        }
    }

    __device__ static void store(const GemmParams& p, const acc_t (&acc)[FN][FM], int row0, int rows, int nt, int wm,
                                 int wn, int lane) {
#pragma unroll
        for (int i0 = 0; i0 < FN; i0 += IG) store_cols(p, acc + i0, i0, row0, rows, nt, wm, wn, lane);
    }
};

template <bool BF16, int BM, int BN, int EPI, bool SPLIT>
__global__ __launch_bounds__(256) void k_grouped_gemm(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the launch stub
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int MB = 16;                    // MFMA block edge (16x16x32 bf16, 16x16x4 fp32)
    constexpr int FM = WM / MB, FN = WN / MB;
    constexpr int ES = BF16 ? 2 : 4;
    constexpr int KS = 1;                     // k-steps per half slice
    constexpr int SA = BM * 128, SB = BN * 128;
    constexpr RingDepth RD = ring_depth(BM, BN);
    constexpr int NA = RD.na, NB = RD.nb;
    constexpr int GA = BM / 8, GB = BN / 8;   // 1 KB load groups: 8 rows x 128 bytes
    constexpr int ga = GA / 4, gb = GB / 4;   // groups per wave
    typedef GemmEpilogue<BF16, BM, BN, EPI> Epi;
    typedef typename Epi::acc_t acc_t;
    static_assert(FM >= 1 && FN >= 1, "tile smaller than one MFMA block");
    static_assert(!epi_swiglu(EPI) || (FN % 2) == 0, "SwiGLU pairs 16-row blocks");
    static_assert(RD.wait0 < 64 && RD.bytes <= 160 * 1024, "ring exceeds vmcnt or LDS");
    __shared__ __align__(16) uint8_t lds[RD.bytes];

    // ---- work unit.  Whole tiles (SPLIT = false): block ids are dealt
    // round-robin to the 8 XCDs, so tiles are remapped to give each XCD a
    // contiguous range (its blocks share weight and activation panels in its
    // L2).  Split units (SPLIT = true, a launch of its own): block u is unit
    // u, range u % split of tail tile u / split.
    const int total = p.plan[p.E] * p.NT;
    const int full = p.plan[p.E + 1], split = p.plan[p.E + 2], tail = p.plan[p.E + 3];
    int L, k0 = 0, k1 = p.nk, unit = -1;
    if constexpr (!SPLIT) {
        const int xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
        const int per_xcd = split > 1 ? full / 8 : (total + 7) / 8;
        if (slot >= per_xcd) return;
        L = xcd * per_xcd + slot;
        if (L >= total) return;
    } else {
        if (split <= 1) return;
        unit = blockIdx.x;
        if (unit >= tail * split) return;
        L = full + unit / split;
        const int c = unit % split;
        k0 = c * p.nk / split;
        k1 = (c + 1) * p.nk / split;
    }
    int e, mt, nt;
    decode_tile(p, L, e, mt, nt);
    const int row0 = tile_row0(p, e, mt, BM);
    const int rows = min(BM, p.offsets[e + 1] - row0);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
    const int wm = wave >> 1, wn = wave & 1;

    // ---- direct-to-LDS loads.  Slot layout: NA A slots of BM rows, then NB B
    // slots of BN rows, 128 bytes per row.  One buffer_load_dwordx4 ... lds of
    // a wave fills a 1 KB group: lane l lands at byte 16*l, i.e. row
    // 8*g + l/8, physical chunk l%8, and fetches logical chunk (l%8) ^ swz(row)
    // (the swizzle is applied on the global side).  Each wave loads ga A
    // groups and gb B groups of every slice.  Addresses are buffer descriptors
    // (SGPRs) holding the tile's base and extent, a 32-bit lane offset, and
    // the K offset in an SGPR.
    constexpr int kRsrcWord3 = 0x00020000;
    const int64_t brow_base = epi_swiglu(EPI) ? (int64_t)nt * (BN / 2) : (int64_t)nt * BN;
    const int b_rows = epi_swiglu(EPI) ? BN / 2 : BN;
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.A + (int64_t)row0 * p.lda * ES), (short)0,
        (int)(((int64_t)(rows - 1) * p.lda + p.K) * ES), kRsrcWord3);
    const int64_t boff = ((int64_t)e * p.bstride + brow_base * p.K) * ES;
    const __amdgpu_buffer_rsrc_t rsB0 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)p.B0 + boff), (short)0, (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rsB1 = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const uint8_t*)(epi_swiglu(EPI) ? p.B1 : p.B0) + boff), (short)0,
        (int)((int64_t)b_rows * p.K * ES), kRsrcWord3);
    uint32_t voffA[ga], voffB[gb];
#pragma unroll
    for (int q = 0; q < ga; ++q) {
        const int r = 8 * (wave * ga + q) + (lane >> 3);
        voffA[q] = (uint32_t)(min(r, rows - 1) * (int)p.lda * ES + (((lane & 7) ^ swz(r)) << 4));
    }
#pragma unroll
    for (int q = 0; q < gb; ++q) {
        const int g = wave * gb + q;
        const int r = 8 * g + (lane >> 3);
        // SwiGLU: 16-row block j of the tile is rows (j/2)*16 .. +15 of W1 (j
        // even) or W3 (j odd)
        const int rr = epi_swiglu(EPI) ? ((g >> 2) * 16 + (r & 15)) : r;
        voffB[q] = (uint32_t)(rr * p.K * ES + (((lane & 7) ^ swz(r)) << 4));
    }
    typedef __attribute__((address_space(3))) void* lds_ptr_t;
    const int nk = k1 - k0;
    // virtual slice v goes to slot v % N; slices past the end reload the last
    // one into a free slot (nobody reads it), which keeps the per-wave load
    // count of every batch the same
    auto issueA1 = [&](int v, int q) {      // group q of this wave's part of A slice v
        uint8_t* dst = &lds[(v % NA) * SA + wave * ga * 1024];
        const int koff = (k0 + min(v, nk - 1)) * 128;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_ptr_t)(dst + q * 1024), 16, voffA[q], koff, 0, 0);
    };
    auto issueB1 = [&](int v, int q) {
        uint8_t* dst = &lds[NA * SA + (v % NB) * SB + wave * gb * 1024];
        const int koff = (k0 + min(v, nk - 1)) * 128;
        const bool up = epi_swiglu(EPI) && (((wave * gb + q) >> 1) & 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(up ? rsB1 : rsB0, (lds_ptr_t)(dst + q * 1024), 16, voffB[q], koff,
                                                 0, 0);
    };
    auto issueA = [&](int v) {
#pragma unroll
        for (int q = 0; q < ga; ++q) issueA1(v, q);
    };
    auto issueB = [&](int v) {
#pragma unroll
        for (int q = 0; q < gb; ++q) issueB1(v, q);
    };

    acc_t acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[i][j][r] = 0.0f;

    // Fragment reads, per half slice h (64 bytes of K): lane l takes row
    // l % 16 of a 16-row block at logical chunk 4h + l/16 (8 bf16 k values,
    // one 16x16x32 MFMA; or 4 fp32 k values, four 16x16x4 MFMAs).
    // Weights are MFMA source 0 (rows = output columns n), activations
    // source 1 (columns = token rows m).  The swizzle depends on the row mod
    // 16 only, so blocks i of one operand differ by the constant i*MB*128.
    constexpr int NF = KS * (FM + FN);       // fragments per half slice
    int fo[2][KS][2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) {
            const int lr = lane & (MB - 1);
            const int ch = 4 * h + (lane >> 4);
            fo[h][s2][0] = (wm * WM + lr) * 128 + ((ch ^ swz(lr)) << 4);
            fo[h][s2][1] = NA * SA + (wn * WN + lr) * 128 + ((ch ^ swz(lr)) << 4);
        }
    // fragment r of half slice h: k-step r / (FM + FN), then FM A blocks and
    // FN B blocks
    auto read1 = [&](int ks, int h, u32x4_t* f, int r) {
        const int s2 = r / (FM + FN), q = r % (FM + FN);
        if (q < FM) f[r] = *(const u32x4_t*)(&lds[(ks % NA) * SA] + fo[h][s2][0] + q * MB * 128);
        else f[r] = *(const u32x4_t*)(&lds[(ks % NB) * SB] + fo[h][s2][1] + (q - FM) * MB * 128);
    };
    auto read_frags = [&](int ks, int h, u32x4_t* f) {
#pragma unroll
        for (int r = 0; r < NF; ++r) read1(ks, h, f, r);
    };
    auto mma = [&](const u32x4_t* f) {
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2)
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j) {
                    const u32x4_t fa = f[s2 * (FM + FN) + j], fb = f[s2 * (FM + FN) + FM + i];
                    if constexpr (BF16) {
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, fb), __builtin_bit_cast(bf16x8_t, fa), acc[i][j], 0, 0, 0);
                    } else {
                        const floatx4_t b4 = __builtin_bit_cast(floatx4_t, fb);
                        const floatx4_t a4 = __builtin_bit_cast(floatx4_t, fa);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[0], a4[0], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[1], a4[1], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[2], a4[2], acc[i][j], 0, 0, 0);
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(b4[3], a4[3], acc[i][j], 0, 0, 0);
                    }
                }
    };
    // MFMA m of a bf16 half slice: k-step m / (FN FM), B block (m / FM) % FN,
    // A block m % FM
    auto mma1 = [&](const u32x4_t* f, int m) {
        if constexpr (BF16) {
            const int s2 = m / (FN * FM), i = (m / FM) % FN, j = m % FM;
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, f[s2 * (FM + FN) + FM + i]),
                                                                __builtin_bit_cast(bf16x8_t, f[s2 * (FM + FN) + j]),
                                                                acc[i][j], 0, 0, 0);
        }
    };
    // Pipeline over slices ks = 0 .. nk-1 (two half slices each).  Between
    // two barriers runs one region: the second half of slice ks (fragments
    // in f1) and the first half of slice ks+1 (f0).  Region ks:
    //   wait until this wave's loads of slice ks+1 have landed; barrier
    //   (slice ks+1 is visible to all waves, and every wave has read both
    //   halves of slice ks, so its A and B slots are free); issue batch ks
    //   into those slots; read slice ks+1's first half into f0; MFMAs on f1;
    //   read slice ks+1's second half into f1; MFMAs on f0.
    // The prologue issues the batches j = -NB .. -1 (parts with a negative
    // slice index are skipped) in the same order, so the wait counts hold
    // from the first slice on.
    // bf16 schedule, pinned with scheduling fences: each half of a region is
    // CH chunks of MFMAs on one fragment set; the half's slice loads (A in
    // the first half, B in the second) are dealt one per chunk or so, and the
    // fragment reads of the other set go into the first CH/2 chunks, so they
    // land well before use and before the next barrier drains them.  A wave
    // then never queues a burst of loads behind the address unit while its
    // MFMAs wait (bursts stalled the matrix unit measurably).  fp32 keeps
    // scheduling hints only.
    constexpr int NMMA = KS * FM * FN * (BF16 ? 1 : 4);   // MFMAs per half slice
    constexpr int NV = ga + gb;                             // loads per batch
    u32x4_t f0[NF], f1[NF];
#pragma unroll
    for (int j = -NB; j < 0; ++j) {
        if (j + NA >= 0) issueA(j + NA);
        issueB(j + NB);
    }
    wait_vmcnt<RD.wait0>();
    lds_barrier();
    read_frags(0, 0, f0);
    read_frags(0, 1, f1);
    mma(f0);
    __builtin_amdgcn_sched_barrier(0);
    int ks = 0;
    if constexpr (BF16) {
        constexpr int CH = NMMA < 8 ? NMMA : 8;            // chunks per half region
        auto half = [&](bool loads, bool is_a, int v, int rks, int h, u32x4_t* fr, const u32x4_t* fm) {
#pragma unroll
            for (int c = 0; c < CH; ++c) {
                if (loads) {
                    const int nv = is_a ? ga : gb;
#pragma unroll
                    for (int q = 0; q < (ga > gb ? ga : gb); ++q)
                        if (q < nv && q * CH / nv == c) {
                            if (is_a) issueA1(v, q);
                            else issueB1(v, q);
                        }
                }
#pragma unroll
                for (int r = 0; r < NF; ++r)
                    if (r * (CH / 2 > 0 ? CH / 2 : 1) / NF == c) read1(rks, h, fr, r);
#pragma unroll
                for (int m = c * (NMMA / CH); m < (c + 1) * (NMMA / CH); ++m) mma1(fm, m);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        static_assert(NMMA % CH == 0, "chunks of whole MFMAs");
        for (; ks + 2 < nk; ++ks) {
            wait_vmcnt<RD.wait>();
            lds_barrier();
            half(true, true, ks + NA, ks + 1, 0, f0, f1);
            half(true, false, ks + NB, ks + 1, 1, f1, f0);
        }
        for (; ks + 1 < nk; ++ks) {      // last region with a next slice: no batch left to issue
            wait_vmcnt<RD.wait>();
            lds_barrier();
            half(false, true, 0, ks + 1, 0, f0, f1);
            half(false, false, 0, ks + 1, 1, f1, f0);
        }
    } else {
        for (; ks + 2 < nk; ++ks) {
            wait_vmcnt<RD.wait>();
            lds_barrier();
            issueA(ks + NA);
            issueB(ks + NB);
            read_frags(ks + 1, 0, f0);
            mma(f1);
            read_frags(ks + 1, 1, f1);
            mma(f0);
#pragma unroll
            for (int i = 0; i < NV; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 2 * NMMA / NV > 0 ? 2 * NMMA / NV : 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2 * NF / NV > 0 ? 2 * NF / NV : 1, 0);       // LDS read
                __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);                                        // load
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        for (; ks + 1 < nk; ++ks) {      // last region with a next slice: no batch left to issue
            wait_vmcnt<RD.wait>();
            lds_barrier();
            read_frags(ks + 1, 0, f0);
            mma(f1);
            read_frags(ks + 1, 1, f1);
            mma(f0);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    mma(f1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<0>();   // reloads of the last slice may still be landing

    if constexpr (SPLIT) Epi::store_partial(p, acc, unit, wave, lane);
    else Epi::store(p, acc, row0, rows, nt, wm, wn, lane);
#endif
}

// Split-K fixup: block (t, w, g) adds, in range order, the `split` partial
// accumulators of column group g of wave w of tail tile t, and applies the
// epilogue to them.
template <bool BF16, int BM, int BN, int EPI>
__global__ __launch_bounds__(64) void k_split_fixup(GemmParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef GemmEpilogue<BF16, BM, BN, EPI> Epi;
    constexpr int FM = Epi::FM, FN = Epi::FN, RA = Epi::RA, IG = Epi::IG, NGRP = FN / IG;
    const int full = p.plan[p.E + 1], split = p.plan[p.E + 2], tail = p.plan[p.E + 3];
    const int t = blockIdx.x / (4 * NGRP), w = (blockIdx.x / NGRP) % 4, i0 = (blockIdx.x % NGRP) * IG;
    const int lane = threadIdx.x;
    if (split <= 1 || t >= tail) return;
    typename Epi::acc_t acc[IG][FM];
    const float4* src = (const float4*)p.partial;
#pragma unroll
    for (int i = 0; i < IG; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int r = 0; r < RA; ++r) acc[i][j][r] = 0.0f;
    for (int c = 0; c < split; ++c) {
        const int u = t * split + c;
#pragma unroll
        for (int i = 0; i < IG; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
#pragma unroll
                for (int r4 = 0; r4 < RA / 4; ++r4) {
                    const float4 v = src[Epi::partial_index(u, w, i0 + i, j, r4, lane)];
                    acc[i][j][4 * r4] += v.x;
                    acc[i][j][4 * r4 + 1] += v.y;
                    acc[i][j][4 * r4 + 2] += v.z;
                    acc[i][j][4 * r4 + 3] += v.w;
                }
    }
    int e, mt, nt;
    decode_tile(p, full + t, e, mt, nt);
    const int row0 = tile_row0(p, e, mt, BM);
    const int rows = min(BM, p.offsets[e + 1] - row0);
    Epi::store_cols(p, acc, i0, row0, rows, nt, w >> 1, w & 1, lane);
#endif
}

// Tile plan: prefix[e+1] = sum_{e' <= e} (row tiles of expert e'), then the
// split-K decision {full, split, tail} (see kSplitUnits).  Expert e has
// ceil(M_e / BM) row tiles, or, with rem_bm > 0 and a remainder
// r = M_e mod BM in 1 .. kRemThr, floor(M_e / BM) tiles here and
// ceil(r / rem_bm) tiles in the remainder plan, which follows at
// prefix[E + 4] in the same layout.  With offsets == NULL the plan describes
// one group of uniform_rows rows and offsets_copy receives {0, uniform_rows}.
// One block of 1024 threads (E <= 1024).
// With prefix2 != NULL the same block also writes the plan of a second GEMM
// over the same groups (BM2, rem_bm2, NT2, nk2), so two GEMMs share a launch.
__global__ __launch_bounds__(1024) void k_tile_plan(const int32_t* __restrict__ offsets, int E, int uniform_rows,
                                                    int BM, int rem_bm, int NT, int nk,
                                                    int32_t* __restrict__ prefix, int32_t* __restrict__ offsets_copy,
                                                    int BM2, int rem_bm2, int NT2, int nk2,
                                                    int32_t* __restrict__ prefix2) {
    __shared__ int32_t scan[2][1024];
    const int e = threadIdx.x;
    int32_t M = 0;
    if (offsets == nullptr) {
        if (e == 0) {
            offsets_copy[0] = 0;
            offsets_copy[1] = uniform_rows;
            M = uniform_rows;
        }
        E = 1;
    } else if (e < E) {
        M = offsets[e + 1] - offsets[e];
    }
    auto plan = [&](int bm, int rbm, int nt, int nkk, int32_t* pre) {
        int32_t n = (M + bm - 1) / bm, n2 = 0;
        if (rbm > 0) {
            const int32_t r = M % bm;
            if (r > 0 && r <= kRemThr) {
                n = M / bm;
                n2 = (r + rbm - 1) / rbm;
            }
        }
        __syncthreads();   // a previous plan's reads of scan are done
        scan[0][e] = n;
        scan[1][e] = n2;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int32_t v0 = e >= off ? scan[0][e - off] : 0;
            const int32_t v1 = e >= off ? scan[1][e - off] : 0;
            __syncthreads();
            scan[0][e] += v0;
            scan[1][e] += v1;
            __syncthreads();
        }
        const int plans = rbm > 0 ? 2 : 1;
        for (int h = 0; h < plans; ++h) {
            int32_t* pr = pre + h * (E + 4);
            if (e == 0) pr[0] = 0;
            if (e < E) pr[e + 1] = scan[h][e];
            if (e == 0) {
                const int total = scan[h][E - 1] * nt;
                const int rem = total % kSplitUnits;
                int split = 1, tail = 0;
                if (rem > 0 && rem <= kSplitUnits / 2) {
                    int sp = kSplitUnits / rem;
                    sp = min(sp, kMaxSplit);
                    sp = min(sp, nkk / 4);                 // at least 4 slices per range
                    if (sp >= 2) {
                        split = sp;
                        tail = rem;
                    }
                }
                pr[E + 1] = total - tail;
                pr[E + 2] = split;
                pr[E + 3] = tail;
            }
        }
    };
    plan(BM, rem_bm, NT, nk, prefix);
    if (prefix2) plan(BM2, rem_bm2, NT2, nk2, prefix2);
}

size_t ffn_tile_plan_ints(int E) { return 2 * ((size_t)E + 4); }

// Tile counts and K slices of a grouped GEMM as launch_grouped_gemm sets them.
static void gemm_geometry(bool bf16, int epi, int N, int K, int BM, int BN, int& NT, int& nk, int& rem_bm) {
    NT = epi_swiglu(epi) ? N / (BN / 2) : N / BN;
    nk = K * (bf16 ? 2 : 4) / 128;
    rem_bm = (MOE_GEMM_REM && bf16 && BM == 256) ? kRemBM : 0;
}

hipError_t launch_tile_plans(bool bf16, const int32_t* offsets, int E, int64_t max_rows, int epi1, int N1, int K1,
                             int BM1, int BN1, int32_t* plan1, int epi2, int N2, int K2, int BM2, int BN2,
                             int32_t* plan2, hipStream_t s) {
    if (max_rows <= 0) return hipSuccess;
    if (!offsets) return hipErrorInvalidValue;
    int nt1, nk1, r1, nt2, nk2, r2;
    gemm_geometry(bf16, epi1, N1, K1, BM1, BN1, nt1, nk1, r1);
    gemm_geometry(bf16, epi2, N2, K2, BM2, BN2, nt2, nk2, r2);
    hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, E, (int)max_rows, BM1, r1, nt1, nk1, plan1,
                       (int32_t*)nullptr, BM2, r2, nt2, nk2, plan2);
    return hipGetLastError();
}

size_t gemm_partial_bytes(int BM, int BN) { return (size_t)kSplitUnits * BM * BN * sizeof(float); }

GemmShape pick_gemm_shape(bool bf16, int epi, int64_t rows, int E, int N) {
    const int64_t avg = E > 0 ? rows / E : rows;
    GemmShape g;
    g.BM = avg >= 384 ? 256 : (avg >= 96 ? 128 : 64);
    // fp32 tiles stop at 128 rows: 256 x 256 fp32 accumulators leave no
    // registers for the epilogue
    if (!bf16 && g.BM > 128) g.BM = 128;
    // output columns per tile for BN = 256 / 128 / 64 (SwiGLU tiles hold gate
    // and up rows, so they produce half as many columns)
    const int div = epi_swiglu(epi) ? 2 : 1;
    g.BN = (N % (256 / div) == 0) ? 256 : (N % (128 / div) == 0 ? 128 : 64);
    return g;
}

// Whole tiles, split units (exit at once when the plan has no split), fixup;
// the last two only when the plan may have a split.
template <bool BF16, int BM, int BN, int EPI>
static void launch_pair(const GemmParams& p, int grid, bool may_split, hipStream_t s) {
    hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI, false>), dim3(grid), dim3(256), 0, s, p);
    if (!may_split) return;
    hipLaunchKernelGGL((k_grouped_gemm<BF16, BM, BN, EPI, true>), dim3(kSplitUnits), dim3(256), 0, s, p);
    constexpr int groups = GemmEpilogue<BF16, BM, BN, EPI>::FN / GemmEpilogue<BF16, BM, BN, EPI>::IG;
    hipLaunchKernelGGL((k_split_fixup<BF16, BM, BN, EPI>), dim3(kSplitUnits / 2 * 4 * groups), dim3(64), 0, s, p);
}

template <bool BF16, int BM, int BN>
static void launch_bmbn(int epi, const GemmParams& p, int grid, bool ms, hipStream_t s) {
    switch (epi) {
        case EPI_STORE: launch_pair<BF16, BM, BN, EPI_STORE>(p, grid, ms, s); break;
        case EPI_RELU: launch_pair<BF16, BM, BN, EPI_RELU>(p, grid, ms, s); break;
        case EPI_RELU_SAVE: launch_pair<BF16, BM, BN, EPI_RELU_SAVE>(p, grid, ms, s); break;
        case EPI_SWIGLU_SAVE: launch_pair<BF16, BM, BN, EPI_SWIGLU_SAVE>(p, grid, ms, s); break;
        default: launch_pair<BF16, BM, BN, EPI_SWIGLU>(p, grid, ms, s); break;
    }
}

template <bool BF16>
static void launch_t(int epi, const GemmParams& p, int BM, int BN, int grid, bool ms, hipStream_t s) {
    if constexpr (BF16) {
        if (BM == 256) {
            if (BN == 256) return launch_bmbn<BF16, 256, 256>(epi, p, grid, ms, s);
            if (BN == 128) return launch_bmbn<BF16, 256, 128>(epi, p, grid, ms, s);
            return launch_bmbn<BF16, 256, 64>(epi, p, grid, ms, s);
        }
    }
    if (BN == 256) {
        if (BM == 128) return launch_bmbn<BF16, 128, 256>(epi, p, grid, ms, s);
        return launch_bmbn<BF16, 64, 256>(epi, p, grid, ms, s);
    }
    if (BN == 128) {
        if (BM == 128) return launch_bmbn<BF16, 128, 128>(epi, p, grid, ms, s);
        return launch_bmbn<BF16, 64, 128>(epi, p, grid, ms, s);
    }
    if (BM == 128) return launch_bmbn<BF16, 128, 64>(epi, p, grid, ms, s);
    return launch_bmbn<BF16, 64, 64>(epi, p, grid, ms, s);
}

// Whether a plan of `total` tiles takes the split-K tail (the rule of
// k_tile_plan, for launches whose row counts the host knows).
static bool plan_may_split(int64_t total, int nk) {
    const int64_t rem = total % kSplitUnits;
    if (rem <= 0 || rem > kSplitUnits / 2) return false;
    int64_t sp = kSplitUnits / rem;
    sp = std::min<int64_t>(sp, kMaxSplit);
    sp = std::min<int64_t>(sp, nk / 4);
    return sp >= 2;
}

hipError_t launch_grouped_gemm(bool bf16, int epi, const void* A, int64_t lda, const void* B0, const void* B1,
                               int64_t b_expert_stride, void* C, int64_t ldc, int N, int K, int E, int64_t max_rows,
                               const int32_t* offsets, int32_t* plan, int32_t* plan_copy, float* partial, int BM,
                               int BN, hipStream_t s, void* C2, int64_t ldc2, bool plan_ready) {
    if (max_rows <= 0) return hipSuccess;
    GemmParams p;
    p.A = A; p.lda = lda; p.B0 = B0; p.B1 = B1; p.bstride = b_expert_stride;
    p.C = C; p.ldc = ldc; p.N = N; p.K = K; p.E = offsets ? E : 1;
    p.NT = epi_swiglu(epi) ? N / (BN / 2) : N / BN;
    p.nk = K * (bf16 ? 2 : 4) / 128;
    p.offsets = offsets ? offsets : plan_copy;
    p.plan = plan;
    p.partial = partial;
    p.C2 = C2;
    p.ldc2 = ldc2;
    p.rem_bm = 0;
    const bool rem = MOE_GEMM_REM && bf16 && BM == 256;
    if (!plan_ready)
        hipLaunchKernelGGL(k_tile_plan, dim3(1), dim3(1024), 0, s, offsets, E, (int)max_rows, BM, rem ? kRemBM : 0,
                           p.NT, p.nk, plan, plan_copy, 0, 0, 0, 0, (int32_t*)nullptr);
    const int64_t m_tiles_ub = (max_rows + BM - 1) / BM + (p.E > 1 ? p.E : 0);
    int64_t grid = (m_tiles_ub * p.NT + 7) / 8 * 8;
    if (grid > 0x7fffffff) return hipErrorInvalidValue;
    if (!bf16 && BM > 128) return hipErrorInvalidValue;
    // With offsets == NULL the host knows the row count and launches only
    // the parts of the plan that have work; routed counts live on the device.
    bool main_split = true, rem_launch = rem, rem_split = true;
    if (offsets == nullptr) {
        const int64_t r = max_rows % BM;
        const bool rem_active = rem && r > 0 && r <= kRemThr;
        const int64_t n_main = rem_active ? max_rows / BM : (max_rows + BM - 1) / BM;
        main_split = plan_may_split(n_main * p.NT, p.nk);
        rem_launch = rem_active;
        rem_split = rem_active && plan_may_split((r + kRemBM - 1) / kRemBM * p.NT, p.nk);
    }
    if (bf16) launch_t<true>(epi, p, BM, BN, (int)grid, main_split, s);
    else launch_t<false>(epi, p, BM, BN, (int)grid, main_split, s);
    if (rem_launch) {
        GemmParams q = p;
        q.plan = plan + (p.E + 4);
        q.rem_bm = BM;
        const int64_t grid2 = ((int64_t)p.E * ((kRemThr + kRemBM - 1) / kRemBM) * p.NT + 7) / 8 * 8;
        if (grid2 > 0x7fffffff) return hipErrorInvalidValue;
        launch_t<true>(epi, q, kRemBM, BN, (int)grid2, rem_split, s);
    }
    return hipGetLastError();
}

}  // namespace moe
